// Host check of the attention kernels' workgroup -> (batch, query head, query tile) map
// (map_block with the launcher's schedule_tiles), built host-only by test_tile_map_host.py.
// For each shape, precision and LSE mode it walks every workgroup of the launch and checks:
//  * every (batch, head, query tile) is produced exactly once, within range;
//  * when B*Hkv is a multiple of 8, each XCD (workgroup id mod 8) runs only KV groups of
//    its pair of XCDs, and an even XCD runs its odd partner's items only in the first
//    places of its list (the heavy ones) while an odd XCD runs its partner's items only at
//    the places just before j (list places: launch places rotated within groups of 4 when
//    the engine rotation is on);
//  * with an exchange planned, the even XCDs' key tiles exceed the odd ones' by about twice
//    the planned shift (within the half-target tolerance the plan accepts).
// Prints one line per case and "cases <n> exchange <m> rotate <k> failures <f>".
#include "../bf16_causal_prefill_amd/csrc/attn_fwd.h"

#include <cmath>
#include <cstdio>
#include <vector>

using namespace attn;

static int failures = 0;

#define CHECK(cond, ...)                    \
  do {                                      \
    if (!(cond)) {                          \
      std::printf("FAIL: " __VA_ARGS__);    \
      std::printf("\n");                    \
      ++failures;                           \
      return;                               \
    }                                       \
  } while (0)

template <bool FP8, int BN>
static void check_case(int B, int Hq, int Hkv, int Nq, int Nk, int q_off, int lse_mode,
                       int& n_swap, int& n_rot) {
  constexpr int BM = 256;
  FwdParams p{};
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
  p.q_off = q_off < Nk ? q_off : Nk;
  p.lse = lse_mode == 0 ? nullptr : reinterpret_cast<float*>(16);
  p.lse_rounded = lse_mode == 2;
  p.n_qtiles = (Nq + BM - 1) / BM;
  schedule_tiles<FP8, BM, BN>(p);
  const long long grid = (long long)p.n_qtiles * B * Hq;
  std::vector<int> seen((size_t)grid, 0);
  const int G = Hq / Hkv;
  const bool xcd_path = (B * Hkv) % 8 == 0;
  std::vector<long long> xcd_work(8, 0);
  for (long long bid = 0; bid < grid; ++bid) {
    int b = -1, h = -1, qt = -1;
    map_block((int)bid, p, b, h, qt);
    CHECK(b >= 0 && b < B && h >= 0 && h < Hq && qt >= 0 && qt < p.n_qtiles,
          "out of range: bid %lld -> (%d, %d, %d)", bid, b, h, qt);
    const long long item = ((long long)b * Hq + h) * p.n_qtiles + qt;
    CHECK(seen[(size_t)item]++ == 0, "item (%d, %d, %d) twice", b, h, qt);
    // key tiles of the item, as the kernel counts them
    const long long wg_end = std::min<long long>((long long)qt * BM + BM, Nq);
    const long long keys = std::min<long long>(wg_end + p.q_off, Nk);
    xcd_work[bid & 7] += (keys + BN - 1) / BN;
    if (xcd_path) {
      const int x = (int)(bid & 7), kv = (b * Hkv + h / G) & 7;
      CHECK(kv == x || kv == (x ^ 1), "bid %lld on XCD %d runs KV group %d", bid, x, kv);
      // the place in the XCD's list: the launch place, rotated within full groups of 4
      // when the engine rotation is on (the exchange works on list places)
      long long local = bid >> 3;
      const long long grp = local >> 2, per = (long long)(B * Hkv / 8) * G;
      if (p.se_rotate && 4 * grp + 4 <= (long long)p.n_qtiles * per)
        local = 4 * grp + (((local & 3) + grp) & 3);
      if (kv != x) {
        if ((x & 1) == 0)
          CHECK(local < p.xcd_swap, "even XCD %d runs a partner item at place %lld", x, local);
        else
          CHECK(local >= p.xcd_swap_at - p.xcd_swap && local < p.xcd_swap_at,
                "odd XCD %d runs a partner item at place %lld", x, local);
      }
    }
  }
  for (long long i = 0; i < grid; ++i) CHECK(seen[(size_t)i] == 1, "item %lld missing", i);
  if (p.xcd_swap > 0) {
    long long even = 0, odd = 0;
    for (int x = 0; x < 8; x += 2) { even += xcd_work[x]; odd += xcd_work[x + 1]; }
    const double per_xcd = (even + odd) / 8.0, shift = (even - odd) / 8.0;   // per pair
    const double target = XCD_SHIFT * per_xcd;
    CHECK(std::fabs(shift - target) <= 0.5 * target + 1e-9,
          "shift %.1f key tiles per XCD against target %.1f", shift, target);
    CHECK(p.xcd_swap_at >= p.xcd_swap, "swap block at %d before the %d traded items",
          p.xcd_swap_at, p.xcd_swap);
    ++n_swap;
  }
  n_rot += p.se_rotate;
  std::printf("ok %s B=%d Hq=%d Hkv=%d Nq=%d Nk=%d off=%d lse=%d grid=%lld swap=%d at=%d "
              "rotate=%d\n", FP8 ? "fp8" : "bf16", B, Hq, Hkv, Nq, Nk, p.q_off, lse_mode, grid,
              p.xcd_swap, p.xcd_swap_at, p.se_rotate);
}

int main() {
  struct Shape { int B, Hq, Hkv, Nq, Nk, q_off; };
  const Shape shapes[] = {
      {1, 32, 8, 32768, 32768, 0}, {1, 16, 16, 32768, 32768, 0}, {1, 32, 8, 16384, 16384, 0},
      {1, 16, 16, 16384, 16384, 0}, {1, 32, 8, 4096, 4096, 0},   {8, 32, 8, 4096, 4096, 0},
      {2, 8, 8, 24576, 24576, 0},   {8, 16, 16, 4096, 4096, 0},  {16, 32, 8, 2048, 2048, 0},
      {1, 24, 8, 32768, 32768, 0},  {2, 12, 4, 20000, 20000, 0}, {1, 8, 8, 50000, 50000, 0},
      {3, 8, 8, 9000, 9000, 0},     {1, 6, 2, 1000, 1000, 0},    {1, 2, 2, 1, 1, 0},
      {8, 32, 8, 4096, 16384, 12288}, {1, 32, 8, 257, 40000, 39743}, {4, 16, 8, 3000, 2000, 5},
      {2, 64, 8, 12345, 12345, 0},  {1, 32, 8, 32768, 32768, 32768},
  };
  int cases = 0, n_swap = 0, n_rot = 0;
  for (const Shape& s : shapes) {
    for (int lse = 0; lse < 3; ++lse) {
      check_case<true, 128>(s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.q_off, lse, n_swap, n_rot);
      ++cases;
    }
    for (int lse = 0; lse < 2; ++lse) {
      check_case<false, 64>(s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.q_off, lse, n_swap, n_rot);
      ++cases;
    }
  }
  std::printf("cases %d exchange %d rotate %d failures %d\n", cases, n_swap, n_rot, failures);
  return failures == 0 ? 0 : 1;
}
