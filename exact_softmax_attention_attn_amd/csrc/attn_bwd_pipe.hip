// Software-pipelined bf16 backward kernels (dK/dV and dQ) for gfx950.
//
// Same method as the generic kernels (scores rebuilt per tile from Q, K and
// the saved row scalar, ddx issue #243 item 2; dS = P o (dP - D) with no
// row-max term, issue #243 item 1; PR #162's plan p = w/z then p @ v), with
// one wave per SIMD and the work of consecutive 32-row sub-tiles overlapped
// by hand:
//
//   step k:  stage A of sub-tile k      (the two products over the head dim)
//            stage B of sub-tile k - 1  (softmax-backward VALU work and the
//                                        products over positions)
//
// The two stages share no registers, so the matrix cores run stage A's
// chains while the VALU rebuilds P and dS for stage B, and the LDS reads for
// later products are issued a few instructions ahead of their use.  The
// instruction order inside a step is fixed with scheduling fences.  Tiles of
// 64 rows are triple-buffered in LDS and copied global->LDS two sub-steps
// before they are read.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

namespace {

template <bool B> using bool_c = std::integral_constant<bool, B>;

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ f32x4 lds_f32x4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

}  // namespace

// ---------------------------------------------------------------------------
// dK, dV (bf16).  Workgroup = 4 waves = 128 key rows of one (b, h); wave w
// owns key rows kv0 + [0, 32).  Its K rows (pre-multiplied by scale log2e)
// and V rows sit in AGPRs as the B operands of S = Q K^T and dP = dO V^T
// (column n = key row), so the results hold query rows along the registers:
// the row scalars -L log2e and -D then enter as the MFMA's C input, read from
// LDS straight into the accumulator registers, and
//   S' = Q (c K)^T - L2 = log2 of P,   dP' = dO V^T - D
// leave one exp2 and one multiply per element:  P = exp2(S'), dS = P o dP'.
// dV^T += dO^T P and dK^T += Q^T dS accumulate in AGPRs (asm MFMA).  Query
// tiles of 64 rows ping-pong between two separately named LDS buffers; the
// operand reads (Q, dO along the head dim; dO, Q across positions) run AH
// fragments ahead through a whole tile.  Causal: the walk starts at the
// diagonal; only its first two tiles carry the element mask.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ nL2, const float* __restrict__ nD,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int H, int N, int d, float scale_log2,
    float scale) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int BKV = 128, BQ = 64, KS = D / 16, MT = D / 32, AH = 4;
  constexpr int OPS = 2 * KS + 4 * MT;         // operand reads per 32-row sub-tile
  using QT = Tile<bf16, BQ, D>;
  struct __align__(16) Buf {
    bf16 q[QT::ELEMS];
    bf16 o[QT::ELEMS];
    float l[BQ];      // -L * log2(e)
    float dd[BQ];     // -D
  };
  __shared__ Buf buf0, buf1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int jb = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const float* Lh = nL2 + ((long)b * H + head) * N;
  const float* Dh = nD + ((long)b * H + head) * N;

  const int kvb = jb * BKV;
  const int kv0 = kvb + wave * 32;
  const int kv = kv0 + l32;
  const LanePlan<D> plan(lane);
  frag kf[KS], vf[KS];
  load_row_frags<bf16, D>(kf, K + base, rs, kv, N, d, h);
  load_row_frags<bf16, D>(vf, V + base, rs, kv, N, d, h);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int t = 0; t < 8; ++t) kf[ks][t] = (bf16)((float)kf[ks][t] * scale_log2);
    pin_agpr(kf[ks]);
    pin_agpr(vf[ks]);
  }

  f32x16 dv_acc[MT], dk_acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    dv_acc[i] = zero16(); pin_agpr(dv_acc[i]);
    dk_acc[i] = zero16(); pin_agpr(dk_acc[i]);
  }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kvb / BQ : 0;
  const int ntiles = nqt - qt0;

  auto fill = [&](Buf& B, int t) ATTN_INLINE {
    const int q0 = (qt0 + t) * BQ;
    if (q0 + BQ <= N && d == D) {
      fill_async(QT{B.q}, Q + base, rs, q0, wave, lane);
      fill_async(QT{B.o}, dO + base, rs, q0, wave, lane);
      if (wave == 0) fill_async_row64(B.l, Lh + q0);
      if (wave == 1) fill_async_row64(B.dd, Dh + q0);
    } else {
      fill_sync(QT{B.q}, Q + base, rs, q0, N, d, tid);
      fill_sync(QT{B.o}, dO + base, rs, q0, N, d, tid);
      if (tid < BQ) {
        const int q = q0 + tid;
        B.l[tid] = q < N ? Lh[q] : -__builtin_inff();   // padded rows: P = 0
        B.dd[tid] = q < N ? Dh[q] : 0.f;
      }
    }
  };

  auto tile_body = [&](int t, const Buf& B, auto masked_c) ATTN_INLINE {
    constexpr bool MASKED = decltype(masked_c)::value;
    // operand n of the tile: sub-tile n / OPS; within it Q cols, dO cols,
    // dO rows (dV), Q rows (dK)
    auto opnd = [&](int n) ATTN_INLINE -> frag {
      const int r0 = (n / OPS) * 32, m = n % OPS;
      if (m < KS) return plan.cols(B.q, r0, m);
      if (m < 2 * KS) return plan.cols(B.o, r0, m - KS);
      if (m < 2 * KS + 2 * MT) {
        const int i = m - 2 * KS;
        return plan.rows(B.o, r0, i / MT, i % MT);
      }
      const int i = m - 2 * KS - 2 * MT;
      return plan.rows(B.q, r0, i / MT, i % MT);
    };
    frag ring[AH];
#pragma unroll
    for (int n = 0; n < AH; ++n) ring[n] = opnd(n);
    fence();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int r0 = st * 32;
      const int qa = (qt0 + t) * BQ + r0;        // absolute first query row of the sub-tile
      const int n0 = st * OPS;
      // C inputs: -L2 and -D of the sub-tile's rows, in accumulator order
      f32x16 sc, pc;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&B.l[r0 + 8 * g + 4 * h]);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(&B.dd[r0 + 8 * g + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) { sc[4 * g + i] = lv[i]; pc[4 * g + i] = dv[i]; }
      }
      // S' = Q (c K)^T - L2
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int n = n0 + ks;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
        sc = M::mma(a, kf[ks], sc);
        fence();
      }
      // dP' = dO V^T - D  |  P = exp2(S') on the VALU
      constexpr int PER = 16 / KS;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int n = n0 + KS + ks;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
        pc = M::mma(a, vf[ks], pc);
#pragma unroll
        for (int e = 0; e < PER; ++e) sc[ks * PER + e] = fast_exp2(sc[ks * PER + e]);
        fence();
      }
      if constexpr (CAUSAL && MASKED) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kv > qa + acc_row(r, h)) sc[r] = 0.f;
      }
      frag bp[2];
      bp[0] = M::pack(sc, 0);
      bp[1] = M::pack(sc, 1);
      fence();
      // dV^T += dO^T P  |  dS = P o dP' on the VALU
      constexpr int PER2 = 16 / (2 * MT);
      frag bds[2];
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) {
        const int n = n0 + 2 * KS + i;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
        mma_acc_agpr(dv_acc[i % MT], a, bp[i / MT]);
#pragma unroll
        for (int e = 0; e < PER2; ++e) pc[i * PER2 + e] = sc[i * PER2 + e] * pc[i * PER2 + e];
        fence();
      }
      bds[0] = M::pack(pc, 0);
      bds[1] = M::pack(pc, 1);
      fence();
      // dK^T += Q^T dS
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) {
        const int n = n0 + 2 * KS + 2 * MT + i;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
        mma_acc_agpr(dk_acc[i % MT], a, bds[i / MT]);
        fence();
      }
    }
  };

  // Walk the query tiles from the last one back to the diagonal: every block
  // of a head starts on the same tiles at the same time, so they are shared
  // in L2 instead of each block streaming its own stretch.  Step k visits
  // tile ntiles - 1 - k, in buffer k % 2; the two diagonal tiles (BKV = 2 BQ)
  // come last and carry the causal mask.
  const int nmask = CAUSAL ? min(2, ntiles) : 0;
  const int kend = ntiles - nmask;
  auto tile_of = [&](int k) ATTN_INLINE { return ntiles - 1 - k; };
  auto step = [&](int k, const Buf& cur, Buf& nxt, auto masked_c) ATTN_INLINE {
    wait_async_fills();
    __syncthreads();
    if (k + 1 < ntiles) fill(nxt, tile_of(k + 1));
    tile_body(tile_of(k), cur, masked_c);
  };
  // Buffers are picked statically on every path (a runtime choice between
  // them makes the compiler shuffle the accumulators between registers, which
  // it cannot time against the in-flight products): an odd number of unmasked
  // steps starts in buf1, so the unmasked loop and the masked tail both start
  // in buf0.
  int k = 0;
  if (kend & 1) {
    fill(buf1, tile_of(0));
    step(0, buf1, buf0, bool_c<false>{});
    mma_acc_drain();                         // the join below may copy accumulators
    k = 1;
  } else {
    fill(buf0, tile_of(0));
  }
  for (; k < kend; k += 2) {
    step(k, buf0, buf1, bool_c<false>{});
    step(k + 1, buf1, buf0, bool_c<false>{});
  }
  if (nmask > 0) step(kend, buf0, buf1, bool_c<true>{});
  if (nmask > 1) step(kend + 1, buf1, buf0, bool_c<true>{});

  mma_acc_drain();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    store_acc_transposed<bf16>(dv_acc[mt], dV + base, rs, kv0, mt * 32, N, d, 1.f, lane);
    store_acc_transposed<bf16>(dk_acc[mt], dK + base, rs, kv0, mt * 32, N, d, scale, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ (bf16).  Workgroup = NW waves = 256 query rows of one (b, h); wave w owns
// query rows qw + [0, WQ) as WQ / 32 halves of 32 rows.  Q and dO of the
// wave's rows and its dQ^T accumulators live in AGPRs for the whole kernel;
// L2 and D are one scalar per lane and half.  With two halves each LDS
// operand fragment feeds two matrix instructions; with 8 waves (two per
// SIMD) one wave's softmax VALU work and LDS reads overlap the other's
// matrix instructions.  Per key sub-tile of 32 rows:
//   S^T = K Q^T, dP^T = V dO^T (with P = exp2(S scale log2e - L2) on the
//   VALU under the dP^T chain), dS = P o (dP - D), dQ^T += K^T dS^T.
// Operand reads run AH fragments ahead through a whole 64-row key tile.  Key
// tiles ping-pong between two separately named LDS buffers (so the
// transposing reads provably do not overlap the copy in flight).  No atomics.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int WQ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ nL2, const float* __restrict__ nD,
    bf16* __restrict__ dQ, int H, int N, int d, float scale_log2, float scale) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int NH = WQ / 32;                  // 32-row halves per wave
  constexpr int BQ = NW * WQ, BKV = 64, KS = D / 16, MT = D / 32, AH = 4;
  constexpr int NT = NW * 64;
  constexpr int PER = 16 / KS;                 // elements per half handled per dP step
  static_assert(NH == 1 || NH == 2, "32 or 64 query rows per wave");
  using KT = Tile<bf16, BKV, D>;
  struct __align__(16) Buf {
    bf16 k[KT::ELEMS];
    bf16 v[KT::ELEMS];
  };
  // Two separately named buffers, each always addressed through its own
  // name: the transposing LDS reads then provably do not overlap the copy in
  // flight into the other buffer, and need not wait for it.
  __shared__ Buf buf0, buf1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nqb = gridDim.x;
  const int ib = CAUSAL ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;  // longest first
  const int head = blockIdx.y, b = blockIdx.z;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const float* Lh = nL2 + ((long)b * H + head) * N;   // -L * log2(e)
  const float* Dh = nD + ((long)b * H + head) * N;    // -D

  const int qb = ib * BQ;
  const int qw = qb + wave * WQ;               // this wave's first query row
  const LanePlan<D> plan(lane);
  frag qf[NH][KS], of[NH][KS];
  float Lq[NH], Dq[NH];
#pragma unroll
  for (int c = 0; c < NH; ++c) {
    const int q = qw + 32 * c + l32;
    load_row_frags<bf16, D>(qf[c], Q + base, rs, q, N, d, h);
    load_row_frags<bf16, D>(of[c], dO + base, rs, q, N, d, h);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) { pin_agpr(qf[c][kk]); pin_agpr(of[c][kk]); }
    Lq[c] = q < N ? Lh[q] : -__builtin_inff();        // padded rows: P = 0
    Dq[c] = q < N ? Dh[q] : 0.f;
  }

  f32x16 acc[NH][MT];
#pragma unroll
  for (int c = 0; c < NH; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) { acc[c][i] = zero16(); pin_agpr(acc[c][i]); }

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  // first tile holding key rows above some of the block's query rows
  const int diag0 = CAUSAL ? max(0, min(ntiles, qb / BKV)) : ntiles;

  auto fill = [&](Buf& B, int kt) ATTN_INLINE {
    const int k0 = kt * BKV;
    if (k0 + BKV <= N && d == D) {
      fill_async<BKV, D, NW>(KT{B.k}, K + base, rs, k0, wave, lane);
      fill_async<BKV, D, NW>(KT{B.v}, V + base, rs, k0, wave, lane);
    } else {
      fill_sync<bf16, BKV, D, NT>(KT{B.k}, K + base, rs, k0, N, d, tid);
      fill_sync<bf16, BKV, D, NT>(KT{B.v}, V + base, rs, k0, N, d, tid);
    }
  };

  // One key tile (two sub-tiles of 32 rows).  The operand stream of a
  // sub-tile is K (head dim), V (head dim), K^T (positions); reads run AH
  // operands ahead through the whole tile.
  constexpr int OPS = 2 * KS + 2 * MT;          // operands per sub-tile
  auto tile_body = [&](int kt, const Buf& B, auto masked_c) ATTN_INLINE {
    constexpr bool MASKED = decltype(masked_c)::value;
    auto opnd = [&](int n) ATTN_INLINE -> frag {
      const int r0 = (n / OPS) * 32, m = n % OPS;
      if (m < KS) return plan.cols(B.k, r0, m);
      if (m < 2 * KS) return plan.cols(B.v, r0, m - KS);
      const int i = m - 2 * KS;                   // (ss, mt) = (i / MT, i % MT)
      return plan.rows(B.k, r0, i / MT, i % MT);
    };
    frag ring[AH];
#pragma unroll
    for (int n = 0; n < AH; ++n) ring[n] = opnd(n);
    fence();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int ka = kt * BKV + st * 32;          // absolute first key row of the sub-tile
      const int n0 = st * OPS;
      f32x16 sc[NH], pc[NH];
      // S^T = K Q^T
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int n = n0 + kk;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
#pragma unroll
        for (int c = 0; c < NH; ++c)
          sc[c] = kk == 0 ? M::mma(a, qf[c][0], zero16()) : M::mma(a, qf[c][kk], sc[c]);
        fence();
      }
      // dP^T = V dO^T | P = exp2(S scale log2e - L2) on the VALU
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int n = n0 + KS + kk;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
#pragma unroll
        for (int c = 0; c < NH; ++c)
          pc[c] = kk == 0 ? M::mma(a, of[c][0], zero16()) : M::mma(a, of[c][kk], pc[c]);
#pragma unroll
        for (int c = 0; c < NH; ++c)
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int r = kk * PER + e;
            sc[c][r] = fast_exp2(__builtin_fmaf(sc[c][r], scale_log2, Lq[c]));
          }
        fence();
      }
      // causal element mask, only on tiles that cross the diagonal
      if constexpr (CAUSAL && MASKED) {
#pragma unroll
        for (int c = 0; c < NH; ++c) {
          const int q = qw + 32 * c + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (ka + acc_row(r, h) > q) sc[c][r] = 0.f;
        }
      }
      fence();
      // dS = P o (dP - D): half 0 now, half 1 (if any) under half 0's dQ products
      frag bds[NH][2];
#pragma unroll
      for (int r = 0; r < 16; ++r) pc[0][r] = sc[0][r] * (pc[0][r] + Dq[0]);
      bds[0][0] = M::pack(pc[0], 0);
      bds[0][1] = M::pack(pc[0], 1);
      fence();
      frag t[2 * MT];
      constexpr int PER3 = 16 / (2 * MT);
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) {
        const int n = n0 + 2 * KS + i;
        t[i] = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
        mma_acc_agpr(acc[0][i % MT], t[i], bds[0][i / MT]);
        if constexpr (NH == 2) {
#pragma unroll
          for (int e = 0; e < PER3; ++e) {
            const int r = i * PER3 + e;
            pc[NH - 1][r] = sc[NH - 1][r] * (pc[NH - 1][r] + Dq[NH - 1]);
          }
        }
        fence();
      }
      if constexpr (NH == 2) {
        bds[1][0] = M::pack(pc[1], 0);
        bds[1][1] = M::pack(pc[1], 1);
        fence();
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) mma_acc_agpr(acc[1][i % MT], t[i], bds[1][i / MT]);
        fence();
      }
    }
  };

  // tile kt + 1 is copied into the other buffer while tile kt is consumed
  auto run_tile = [&](int kt, const Buf& cur, Buf& nxt, auto masked_c) ATTN_INLINE {
    wait_async_fills();
    __syncthreads();
    if (kt + 1 < ntiles) fill(nxt, kt + 1);
    tile_body(kt, cur, masked_c);
  };

  // even tiles use buf0, odd tiles buf1; the masked walk starts at an even
  // tile (a tile or so before the diagonal also takes the mask: harmless)
  const int split = diag0 & ~1;
  fill(buf0, 0);
  int kt = 0;
  for (; kt < split; kt += 2) {
    run_tile(kt, buf0, buf1, bool_c<false>{});
    run_tile(kt + 1, buf1, buf0, bool_c<false>{});
  }
  for (; kt < ntiles; kt += 2) {
    run_tile(kt, buf0, buf1, bool_c<true>{});
    if (kt + 1 < ntiles) run_tile(kt + 1, buf1, buf0, bool_c<true>{});
  }

  mma_acc_drain();
#pragma unroll
  for (int c = 0; c < NH; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      store_acc_transposed<bf16>(acc[c][mt], dQ + base, rs, qw + 32 * c, mt * 32, N, d, scale,
                                 lane);
}

// ---------------------------------------------------------------------------
// Launchers (bf16 only; the generic kernels serve f32)
// ---------------------------------------------------------------------------
static inline long rows_of(const BwdArgs& a) { return (long)a.B * a.H * a.N; }

template <int D, bool C>
static hipError_t dkdv_pipe_go(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, C>), grid, dim3(256), 0, stream,
                     static_cast<const bf16*>(a.Q), static_cast<const bf16*>(a.K),
                     static_cast<const bf16*>(a.V), static_cast<const bf16*>(a.dO),
                     a.Dws + rows_of(a), a.Dws, static_cast<bf16*>(a.dK),
                     static_cast<bf16*>(a.dV), a.H, a.N, a.d, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

// 256 query rows per workgroup as DQ_NW waves of 256 / DQ_NW rows
#ifndef ATTN_DQ_NW
#define ATTN_DQ_NW 4
#endif
template <int D, bool C>
static hipError_t dq_pipe_go(const BwdArgs& a, hipStream_t stream) {
  constexpr int NW = ATTN_DQ_NW, WQ = 256 / NW;
  dim3 grid((a.N + 255) / 256, a.H, a.B);
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, C, WQ, NW>), grid, dim3(NW * 64), 0, stream,
                     static_cast<const bf16*>(a.Q), static_cast<const bf16*>(a.K),
                     static_cast<const bf16*>(a.V), static_cast<const bf16*>(a.dO),
                     a.Dws + rows_of(a), a.Dws, static_cast<bf16*>(a.dQ), a.H, a.N, a.d,
                     a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

#define ATTN_PIPE_DISPATCH(FN, a, stream)                                  \
  do {                                                                     \
    const int bucket = head_dim_bucket((a).d);                             \
    if ((a).causal) {                                                      \
      if (bucket == 64) return FN<64, true>(a, stream);                    \
      return FN<128, true>(a, stream);                                     \
    }                                                                      \
    if (bucket == 64) return FN<64, false>(a, stream);                     \
    return FN<128, false>(a, stream);                                      \
  } while (0)

hipError_t launch_bwd_dkdv_bf16_pipe(const BwdArgs& a, hipStream_t stream) {
  ATTN_PIPE_DISPATCH(dkdv_pipe_go, a, stream);
}
hipError_t launch_bwd_dq_bf16_pipe(const BwdArgs& a, hipStream_t stream) {
  ATTN_PIPE_DISPATCH(dq_pipe_go, a, stream);
}

}  // namespace attn
