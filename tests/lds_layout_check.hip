// Host-side enumeration of the LDS addresses that the pipelined backward
// kernels read and write for a bf16 tile (no GPU needed).
//
// LDS serves a read 256 bytes (64 four-byte banks) at a time.  For every
// operand read the lanes that may be served together must cover 64 distinct
// banks, or the read is replayed.  The grouping of lanes is checked under all
// the candidate partitions below, so the layout does not depend on which one
// the hardware uses:
//   128-bit row reads (one 16-byte chunk per lane): lanes 16 apart in blocks
//     of 16, and blocks of 8 lanes paired with the other half-wave;
//   64-bit transposing reads (8 bytes per lane): 32 consecutive lanes, and
//   16-lane blocks paired with the other half-wave.
// The asynchronous copy writes lane l of a wave instruction at byte 16 l of
// its 1 KB destination; the check also confirms that every logical chunk
// lands where the reads look for it.
//
// Prints one line per failure and "ok" at the end when there is none.
#include <cstdio>
#include <set>
#include <vector>

#include "common.h"

using namespace attn;

static int failures = 0;

static void expect_banks(const std::vector<unsigned>& byte_addrs, int bytes_per_lane,
                         const char* what, int D, int a, int b) {
  std::set<unsigned> banks;
  for (unsigned x : byte_addrs)
    for (int w = 0; w < bytes_per_lane / 4; ++w) banks.insert((x / 4 + w) % 64);
  if (banks.size() != 64) {
    std::printf("conflict: %s D=%d (%d, %d): %zu distinct banks\n", what, D, a, b, banks.size());
    ++failures;
  }
}

template <int D> static void check() {
  std::vector<LanePlan<D>> plan;
  for (int lane = 0; lane < 64; ++lane) plan.emplace_back(lane);
  const std::vector<std::vector<int>> groups128 = [] {
    std::vector<std::vector<int>> g;
    for (int b = 0; b < 4; ++b) {             // lanes 16b .. 16b+15
      g.emplace_back();
      for (int i = 0; i < 16; ++i) g.back().push_back(16 * b + i);
    }
    for (int b = 0; b < 4; ++b) {             // lanes 8b .. 8b+7 and 32 + (8b .. 8b+7)
      g.emplace_back();
      for (int i = 0; i < 8; ++i) { g.back().push_back(8 * b + i); g.back().push_back(32 + 8 * b + i); }
    }
    return g;
  }();
  const std::vector<std::vector<int>> groups_tr = [] {
    std::vector<std::vector<int>> g(4);
    for (int i = 0; i < 32; ++i) { g[0].push_back(i); g[1].push_back(32 + i); }
    for (int i = 0; i < 16; ++i) {
      g[2].push_back(i); g[2].push_back(32 + i);
      g[3].push_back(16 + i); g[3].push_back(48 + i);
    }
    return g;
  }();
  for (int r0 = 0; r0 < 64; r0 += 16) {
    for (int n = 0; n < D / 16; ++n)
      for (size_t gi = 0; gi < groups128.size(); ++gi) {
        std::vector<unsigned> a;
        for (int lane : groups128[gi]) a.push_back(2u * (plan[lane].col[n] + r0 * D));
        expect_banks(a, 16, "row read", D, n, (int)gi);
      }
    for (int mt = 0; mt < D / 32; ++mt)
      for (int e = 0; e < 2; ++e)
        for (size_t gi = 0; gi < groups_tr.size(); ++gi) {
          std::vector<unsigned> a;
          for (int lane : groups_tr[gi]) a.push_back(2u * (plan[lane].tr[mt][e] + r0 * D));
          expect_banks(a, 8, "transposing read", D, mt * 2 + e, (int)gi);
        }
  }
  // copy placement: a dense 64-row tile (row stride D) copied by 4 waves
  using S = AsyncFillShape<64, D, 4>;
  using TT = Tile<bf16, 64, D>;
  std::vector<int> seen(64 * D / 8, 0);
  for (int wave = 0; wave < 4; ++wave)
    for (int lane = 0; lane < 64; ++lane) {
      unsigned off[S::PER];
      async_fill_plan<64, D, 4>(off, D, wave, lane);
      for (int i = 0; i < S::PER; ++i) {
        const int elem = (int)(off[i] / 2);
        const int row = elem / D, chunk = (elem % D) / 8;
        const int lds_elem = ((wave * S::PER + i) * 1024 + 16 * lane) / 2;
        if (elem % 8 != 0 || lds_elem != TT::off(row, chunk)) {
          std::printf("copy: D=%d wave %d lane %d instr %d puts (%d, %d) at %d, reads expect %d\n",
                      D, wave, lane, i, row, chunk, lds_elem, TT::off(row, chunk));
          ++failures;
        }
        ++seen[lds_elem / 8];
      }
    }
  for (int v : seen)
    if (v != 1) { std::printf("copy: D=%d a chunk slot written %d times\n", D, v); ++failures; break; }
}

int main() {
  check<64>();
  check<128>();
  check<256>();   // the generic kernels' 256 bucket reads the same addresses
  if (failures == 0) std::printf("ok\n");
  return failures == 0 ? 0 : 1;
}
