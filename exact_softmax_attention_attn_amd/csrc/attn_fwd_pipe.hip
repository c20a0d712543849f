// Forward (bf16, head dim 64 or 128) with the saved row scalar L = m + log z,
// pipelined so that the online softmax of one key sub-tile runs beside the
// matrix products of its neighbours.
//
// What it computes is the attention of ddx issue #217's loss (scores, weights
// normalised per row, weighted sum of values) and the one number per row that
// ddx issue #243 (item 2) keeps for the backward: L = m + log z, natural log of
// the row's normaliser of the scaled scores.
//
// Workgroup = 256 query rows of one (b, h): NW = 4 waves of 64 rows (two
// halves of 32, NH = 2) or 8 waves of 32 rows (NH = 1, two waves per SIMD).
// Q is the B operand of S^T = K Q^T and stays in AGPRs, so each lane owns one
// query row of each half, and the O^T accumulators stay in AGPRs.  With two
// halves each K and V operand read from LDS feeds both.
//
// Online softmax in log2 units, kept per query: m (running max of c s, c =
// scale log2 e) and l (running sum of exp2(c s - m)); the scale is applied in
// float32 by the FMA that feeds each exp2, so the backward kernels rebuild
// these scores to float32 rounding.  m moves only when a row's new max
// exceeds it by more than 8 (P stays below 2^8); the accumulators are then
// rescaled, which is rare once the max has settled.
//
// Per key sub-tile j of 32 rows, two chains of products:
//   A: S_{j+1}^T = K Q^T                    | exps of S_j half 1, pack P_j,
//                                             row sums of P_j
//   B: O^T_c += V^T P_j^T (c = 0, 1)        | mask, row max, rescale decision
//                                             and half-0 exps of S_{j+1}
// so every VALU stage reads a chain that finished one chain earlier (with one
// half, chain A only packs and sums, and the other wave on the SIMD fills the
// gaps).  Row sums
// are taken on the bf16 P that enters the products (pairs summed by
// v_dot2_f32_bf16), so O and l are normalised consistently.  The two lanes
// that share a query exchange their halves of a key sub-tile with
// v_permlane32_swap.
//
// Key tiles of 64 rows (K, V) rotate through three LDS buffers; the copy of
// tile t + 2 goes out right after the barrier that publishes tile t + 1.  Tiles
// whose next sub-tiles need no mask and whose tile two ahead is whole run
// without any of the edge checks.  SPARSE: the walk visits the key tiles kept
// by either mask row of the block's query rows; a wave whose own mask row
// drops a tile gives its scores -inf.  A row that keeps no key ends with
// l = 0: its output is 0 and its L is -inf.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

namespace {

template <bool B> using bool_c = std::integral_constant<bool, B>;

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// max / sum of a value with the lane 32 positions away (the lane that holds
// the other half of the same query's keys)
__device__ __forceinline__ float max_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of the 8 bf16 values of a packed fragment, accumulated onto acc
__device__ __forceinline__ float frag_sum(const bf16x8& f, float acc) {
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {f[2 * i], f[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
  return acc;
}

}  // namespace

template <int D, bool CAUSAL, bool SPARSE, int NH, int NW>
__global__ __launch_bounds__(NW * 64, 1) void fwd_bf16_pipe_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ Lout, int H, int N, int d, float scale_log2,
    const unsigned char* __restrict__ mask, int mask_heads) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int WQ = 32 * NH, BQ = NW * WQ, BKV = 64;
  static_assert(BQ == 256, "256 query rows per workgroup");
  constexpr int KS = D / 16, MT = D / 32, L = KS, AH = 4, NT = NW * 64;
  static_assert(L == 2 * MT, "chain length");
  using KT = Tile<bf16, BKV, D>;
  struct __align__(16) Buf {
    bf16 k[KT::ELEMS];
    bf16 v[KT::ELEMS];
  };
  __shared__ Buf buf0, buf1, buf2;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int nqb = gridDim.x;
  const BlockOrder bo = block_order();
  const int ib = CAUSAL ? (nqb - 1 - bo.rank) : bo.rank;   // longest first
  const int head = bo.head, b = bo.b;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;

  const int qb = ib * BQ;
  const int qw = qb + wave * WQ;               // this wave's first query row
  const LanePlan<D> plan(lane);
  frag qf[NH][KS];                             // read from LDS in the prologue
  f32x16 acc[NH][MT];
#pragma unroll
  for (int c = 0; c < NH; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) { acc[c][i] = zero16(); pin_agpr(acc[c][i]); }

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int ntiles_all = (kv_end + BKV - 1) / BKV;
  // block-sparse: the key tiles kept by either mask row of the block's query
  // rows, in order (entry = tile | which mask rows keep it << 14)
  __shared__ unsigned short vis[SPARSE ? kMaxVisit : 1];
  __shared__ int nvis;
  static_assert(!SPARSE || (BQ == 2 * kMaskBlock && kMaskBlock % WQ == 0),
                "mask rows per block and per wave");
  const int nb = (N + kMaskBlock - 1) / kMaskBlock;
  const int ntiles = !SPARSE ? ntiles_all : build_visits(vis, &nvis, ntiles_all,
      [&](int t) ATTN_INLINE -> unsigned {
        const unsigned char* mk = head_mask(mask, mask_heads, b, head, H, nb);
        const int r0 = qb / kMaskBlock, c = t * BKV / kMaskBlock;
        const unsigned code = (mk[r0 * nb + c] ? 1u : 0u) |
                              (r0 + 1 < nb && mk[(r0 + 1) * nb + c] ? 2u : 0u);
        return code ? (code << 14) | (unsigned)t : 0u;
      });
  // tile at walk position p (read where no LDS operation is in flight), and
  // whether this wave's mask row drops it
  auto tile_at = [&](int p) ATTN_INLINE -> int {
    if constexpr (SPARSE) return (int)(visit_entry(vis, p) & kVisitTile);
    else return p;
  };
  auto kill_at = [&](int p) ATTN_INLINE -> bool {
    if constexpr (SPARSE) return ((visit_entry(vis, p) >> (14 + wave * WQ / kMaskBlock)) & 1u) == 0u;
    else return false;
  };

  using FS = AsyncFillShape<BKV, D, NW>;
  unsigned copy_off[FS::PER];
  async_fill_plan<BKV, D, NW>(copy_off, rs, wave, lane);
  // a key tile into LDS: whole tiles by direct copies (2 PER instructions per
  // wave), the sequence's ragged last tile by the register path, zero padded
  auto fill = [&](Buf& B, int t) ATTN_INLINE {
    const int k0 = t * BKV;
    if (k0 + BKV <= N) {
      async_fill_untracked<BKV, D, NW>(KT{B.k}, K + base + k0 * rs, copy_off, wave);
      async_fill_untracked<BKV, D, NW>(KT{B.v}, V + base + k0 * rs, copy_off, wave);
    } else {
      fill_sync<bf16, BKV, D, NT>(KT{B.k}, K + base, rs, k0, N, d, tid);
      fill_sync<bf16, BKV, D, NT>(KT{B.v}, V + base, rs, k0, N, d, tid);
    }
  };

  float m[NH], lsum[NH];                       // per lane: its query of half c
  f32x16 sc[NH];                               // S_j, then P_j (fp32)
  frag bp[NH][2];                              // P_j packed (B operand of O^T += V^T P^T)

  // S^T of sub-tile j (rows 32 (j % 2) of tile buffer B) for both halves;
  // valu(i) runs after product pair i
  auto s_chain = [&](const Buf& B, int j, f32x16 (&s)[NH], auto&& valu) ATTN_INLINE {
    const int r0 = (j & 1) * 32;
    frag ring[AH];
#pragma unroll
    for (int n = 0; n < AH; ++n) ring[n] = plan.cols(B.k, r0, n);
#pragma unroll
    for (int c = 0; c < NH; ++c) s[c] = zero16();
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const frag a = ring[i % AH];
#pragma unroll
      for (int c = 0; c < NH; ++c) s[c] = M::mma(a, qf[c][i], s[c]);
      if (i + AH < L) ring[i % AH] = plan.cols(B.k, r0, i + AH);
      valu(i);
      fence();
    }
  };
  // O^T_c += V^T P_j^T for sub-tile j of tile buffer B
  auto pv_chain = [&](const Buf& B, int j, auto&& valu) ATTN_INLINE {
    const int r0 = (j & 1) * 32;
    frag ring[AH];
#pragma unroll
    for (int n = 0; n < AH; ++n) ring[n] = plan.rows(B.v, r0, n / MT, n % MT);
    fence();
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const frag t = ring[i % AH];
#pragma unroll
      for (int c = 0; c < NH; ++c) mma_acc_agpr(acc[c][i % MT], t, bp[c][i / MT]);
      if (i + AH < L) ring[i % AH] = plan.rows(B.v, r0, (i + AH) / MT, (i + AH) % MT);
      valu(i);
      fence();
    }
  };
  // keys of the sub-tile at key row ka above the query (causal) or past N get
  // -inf, every key when the wave's mask row drops the tile (kill)
  auto mask_sub = [&](f32x16 (&s)[NH], int ka, bool kill) ATTN_INLINE {
#pragma unroll
    for (int c = 0; c < NH; ++c) {
      const int q = qw + 32 * c + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = ka + acc_row(r, h);
        if (kill || (CAUSAL && kv > q) || kv >= N) s[c][r] = -__builtin_inff();
      }
    }
  };
  auto needs_mask = [&](int ka, bool kill) ATTN_INLINE {
    return kill || (CAUSAL && ka + 31 > qw) || ka + 32 > N;
  };
  // row max of c s (log2 units) per half, taken on the raw scores (c > 0
  // keeps their order)
  auto row_max = [&](const f32x16 (&s)[NH], float (&mx)[NH]) ATTN_INLINE {
#pragma unroll
    for (int c = 0; c < NH; ++c) {
      float x = s[c][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, s[c][r]);
      mx[c] = max_pair(x) * scale_log2;
    }
  };
  // P = exp2(c s - m) for elements [e0, e1) of half c
  auto exps = [&](f32x16 (&s)[NH], int c, int e0, int e1) ATTN_INLINE {
#pragma unroll
    for (int r = e0; r < e1; ++r) s[c][r] = fast_exp2(__builtin_fmaf(s[c][r], scale_log2, -m[c]));
  };
  auto pack_and_sum = [&](int c) ATTN_INLINE {
    bp[c][0] = M::pack(sc[c], 0);
    bp[c][1] = M::pack(sc[c], 1);
    pin_operand(bp[c][0]);
    pin_operand(bp[c][1]);
    lsum[c] += sum_pair(frag_sum(bp[c][1], frag_sum(bp[c][0], 0.f)));
  };

  // ---- prologue.  The block's 256 Q rows reach the waves' registers
  // through LDS by whole-row copies (a lane loading its own row would touch
  // 32 rows per instruction): rows 0..127 into buf1, 128..255 into buf2 (each
  // buffer's k and v tiles hold 64 rows), beside tile 0 into buf0; tile 1
  // goes to buf1 once the waves have read their rows.  Then S_0, m = its row
  // max (at least -1e30, so a row whose first keys are all masked stays
  // finite).
#pragma unroll
  for (int c = 0; c < NH; ++c) { m[c] = -1e30f; lsum[c] = 0.f; }
  {
    auto fill_rows = [&](bf16* t, int r0) ATTN_INLINE {
      if (r0 + BKV <= N) async_fill_untracked<BKV, D, NW>(KT{t}, Q + base + r0 * rs, copy_off, wave);
      else fill_sync<bf16, BKV, D, NT>(KT{t}, Q + base, rs, r0, N, d, tid);
    };
    fill_rows(buf1.k, qb);
    fill_rows(buf1.v, qb + 64);
    fill_rows(buf2.k, qb + 128);
    fill_rows(buf2.v, qb + 192);
    if (ntiles > 0) fill(buf0, tile_at(0));     // a sparse walk may visit nothing
    wait_async_fills();
    lds_barrier();
#pragma unroll
    for (int c = 0; c < NH; ++c) {
      const int r = wave * WQ + 32 * c;         // the half's first row in the block
      const Buf& qbuf = r < 128 ? buf1 : buf2;
      const bf16* qt = (r & 64) ? qbuf.v : qbuf.k;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qf[c][kk] = plan.cols(qt, r & 63, kk);
    }
#pragma unroll
    for (int c = 0; c < NH; ++c)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) pin_agpr(qf[c][kk]);
    lds_barrier();                              // buf1 and buf2 free again
  }
  if (ntiles > 0) {
    const int t0 = tile_at(0);
    if (ntiles > 1) fill(buf1, tile_at(1));     // lands during sub-tile 0
    s_chain(buf0, 0, sc, [&](int) ATTN_INLINE {});
    const bool kill0 = kill_at(0);
    if (needs_mask(t0 * BKV, kill0)) mask_sub(sc, t0 * BKV, kill0);
    float mx[NH];
    row_max(sc, mx);
#pragma unroll
    for (int c = 0; c < NH; ++c) m[c] = fmaxf(mx[c], -1e30f);
    exps(sc, 0, 0, 16);
  }

  // ---- one iteration: sub-tile j in buffer Bj; sub-tile j + 1 in buffer Bn,
  // at key row ka_next, dropped for this wave when kill_next.
  // MASKABLE = false: the next sub-tile needs no mask (checked by the caller).
  float alpha[NH];
  auto iteration = [&](auto maskable, int j, const Buf& Bj, const Buf& Bn,
                       bool has_next, int ka_next, bool kill_next) ATTN_INLINE {
    constexpr bool MASKABLE = decltype(maskable)::value;
    f32x16 sn[NH];
    // A: S_{j+1} | exps of S_j half 1, pack P_j and its row sums
    constexpr int EH = 16 / (L / 2);             // half-1 exps per product pair
    auto valu_a = [&](int i) ATTN_INLINE {
      if constexpr (NH > 1) {
        if (i < L / 2) exps(sc, 1, i * EH, (i + 1) * EH);
      }
      if (i == L / 2) pack_and_sum(0);
      if constexpr (NH > 1) {
        if (i == L / 2 + 1) pack_and_sum(1);
      }
    };
    if (has_next) {
      s_chain(Bn, j + 1, sn, valu_a);
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i) valu_a(i);
    }
    fence();
    // B: O^T += V^T P_j^T | mask, max, rescale decision, half-0 exps of S_{j+1}
    bool resc = false;
    auto valu_b = [&](int i) ATTN_INLINE {
      if (!has_next) return;
      if (MASKABLE && i == 0 && needs_mask(ka_next, kill_next)) mask_sub(sn, ka_next, kill_next);
      if (i == 1) {
        // the new max, alpha and the rescaled sum by selects, not a branch:
        // the exps below read m, and a branch here would hold them back
        // until the products of the chain had all been issued
        float mx[NH];
        row_max(sn, mx);
        bool any = false;
#pragma unroll
        for (int c = 0; c < NH; ++c) {
          const bool upd = mx[c] > m[c] + 8.f;
          any = any || upd;
          const float mnew = upd ? mx[c] : m[c];
          alpha[c] = upd ? fast_exp2(m[c] - mnew) : 1.f;
          lsum[c] = upd ? lsum[c] * alpha[c] : lsum[c];
          m[c] = mnew;
        }
        resc = __builtin_amdgcn_ballot_w64(any) != 0;
      }
      if (i >= 2) exps(sn, 0, (i - 2) * 16 / (L - 2), (i - 1) * 16 / (L - 2));
      // keep the exps beside the chain: without a use here the compiler
      // sinks them past the rare rescale branch that follows the chain (the
      // checked form, whose mask branch opens the chain, is left as it is:
      // there the pin cost 1.6% on a sparse walk)
      if (!MASKABLE && i == L - 1) pin_operand(sn[0]);
    };
    pv_chain(Bj, j, valu_b);
    if (resc) {
      // rare: scale the accumulators once P_j's products have landed, one
      // tile at a time so at most 16 values pass through VGPRs
      mma_acc_drain(acc);
#pragma unroll
      for (int c = 0; c < NH; ++c)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[c][i][r] *= alpha[c];
          pin_agpr(acc[c][i]);
          fence();
        }
    }
    if (has_next) {
#pragma unroll
      for (int c = 0; c < NH; ++c) sc[c] = sn[c];
    }
    fence();
  };
  // tile t: sub-tiles 2t, 2t + 1 (buffer cur); the next tile in nxt, the tile
  // two ahead goes to ahead.  The barrier before sub-tile 2t + 1's iteration
  // publishes tile t + 1 (its S chain reads it) and frees tile t - 1's buffer.
  auto tile = [&](int t, const Buf& cur, const Buf& nxt, Buf& ahead) ATTN_INLINE {
    const int tt = tile_at(t);
    const bool kt_ = kill_at(t);
    iteration(bool_c<true>{}, 2 * t, cur, cur, true, tt * BKV + 32, kt_);
    const bool more = t + 1 < ntiles;
    int tn = 0;
    bool kn = false;
    if (more) {
      wait_async_fills();
      lds_barrier();
      if (t + 2 < ntiles) fill(ahead, tile_at(t + 2));
      tn = tile_at(t + 1);
      kn = kill_at(t + 1);
    }
    iteration(bool_c<true>{}, 2 * t + 1, cur, nxt, more, tn * BKV, kn);
  };
  // tiles whose next sub-tiles (2t + 1, 2t + 2) need no mask for any wave and
  // whose tile two ahead is whole
  auto tile_inner = [&](int t, const Buf& cur, const Buf& nxt, Buf& ahead) ATTN_INLINE {
    iteration(bool_c<false>{}, 2 * t, cur, cur, true, 0, false);
    wait_async_fills();
    lds_barrier();
    const int k2 = (t + 2) * BKV;
    async_fill_untracked<BKV, D, NW>(KT{ahead.k}, K + base + k2 * rs, copy_off, wave);
    async_fill_untracked<BKV, D, NW>(KT{ahead.v}, V + base + k2 * rs, copy_off, wave);
    iteration(bool_c<false>{}, 2 * t + 1, cur, nxt, true, 0, false);
  };
  // inner: 64 t + 95 <= qb (causal: keys of sub-tiles up to 2t + 2 are at or
  // below every query of the block), t + 2 < ntiles, tile t + 2 whole
  // (a sparse walk takes every tile through the checked form)
  int inner_end = SPARSE ? 0 : min(ntiles - 2, N / BKV - 2);
  if (CAUSAL && !SPARSE) inner_end = min(inner_end, (qb - 95) / BKV + 1);
  int t = 0;
  for (; t + 3 <= inner_end; t += 3) {
    tile_inner(t, buf0, buf1, buf2);
    tile_inner(t + 1, buf1, buf2, buf0);
    tile_inner(t + 2, buf2, buf0, buf1);
  }
  for (; t + 3 <= ntiles; t += 3) {
    tile(t, buf0, buf1, buf2);
    tile(t + 1, buf1, buf2, buf0);
    tile(t + 2, buf2, buf0, buf1);
  }
  if (t < ntiles) tile(t, buf0, buf1, buf2);
  if (t + 1 < ntiles) tile(t + 1, buf1, buf2, buf0);

  mma_acc_drain(acc);
  // every wave is done with the key tiles: O leaves through LDS, whole rows
  // per store, three waves' staging areas per buffer
  static_assert(3 * RowStage<D>::BYTES <= sizeof(Buf) && NW <= 9, "staging area");
  lds_barrier();
  bf16* stage = reinterpret_cast<bf16*>(wave < 3 ? &buf0 : wave < 6 ? &buf1 : &buf2) +
                (wave % 3) * (RowStage<D>::BYTES / 2);
#pragma unroll
  for (int c = 0; c < NH; ++c) {
    const float inv = lsum[c] > 0.f ? 1.f / lsum[c] : 0.f;   // no kept key: O = 0
    store_rows_via_lds<D>(acc[c], O + base, rs, qw + 32 * c, N, inv, stage, lane);
    const int q = qw + 32 * c + l32;
    if (h == 0 && q < N)
      Lout[((long)b * H + head) * N + q] =
          lsum[c] > 0.f ? (m[c] + log2f(lsum[c])) * 0.69314718055994531f : -__builtin_inff();
  }
}

// Waves per workgroup: 8 of 32 query rows each (two waves per SIMD, which
// hide each other's softmax work at the price of twice the LDS operand reads
// per product), where a wave fits in 256 registers; otherwise 4 of 64 rows
// (the non-causal d = 128 form, whose edge checks need more registers).
template <int D, bool C, bool S>
static hipError_t fwd_pipe_run(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = (D == 128 && !C) ? 4 : 8, NH = 8 / NW;
  dim3 grid((a.N + 255) / 256, a.H, a.B);
  hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, C, S, NH, NW>), grid, dim3(NW * 64), 0, stream,
                     static_cast<const bf16*>(a.Q), static_cast<const bf16*>(a.K),
                     static_cast<const bf16*>(a.V), static_cast<bf16*>(a.O), a.L, a.H, a.N,
                     a.d, a.scale * kLog2e, a.mask, a.mask_heads);
  return hipGetLastError();
}
template <int D, bool C>
static hipError_t fwd_pipe_go(const FwdArgs& a, hipStream_t stream) {
  return a.mask ? fwd_pipe_run<D, C, true>(a, stream) : fwd_pipe_run<D, C, false>(a, stream);
}

hipError_t launch_fwd_lse_bf16_pipe(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? fwd_pipe_go<128, true>(a, stream)
                                  : fwd_pipe_go<128, false>(a, stream);
  return a.causal ? fwd_pipe_go<64, true>(a, stream) : fwd_pipe_go<64, false>(a, stream);
}

}  // namespace attn
