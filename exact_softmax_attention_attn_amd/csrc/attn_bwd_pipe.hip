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
// owns key rows kv0 + [0, 32) (K, V in registers; dV^T, dK^T accumulators).
// Stage A(k): S = Q K^T and dP = dO V^T for the 32 query rows of sub-tile k.
// Stage B(k): P = exp2(S scale log2e - L2) (masked on diagonal sub-tiles),
//             dV^T += dO^T P, dS = P o (dP - D), dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dws,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int H, int N, int d, float scale_log2,
    float scale) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int BKV = 128, BQ = 64, KS = D / 16, MT = D / 32, NB = 3;
  static_assert(KS == 2 * MT, "one product over positions per product over the head dim");
  using QT = Tile<bf16, BQ, D>;
  struct __align__(16) Buf {
    bf16 q[QT::ELEMS];
    bf16 o[QT::ELEMS];
    float l[BQ];
    float dd[BQ];
  };
  __shared__ Buf buf[NB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int jb = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const float* Lh = L2 + ((long)b * H + head) * N;
  const float* Dh = Dws + ((long)b * H + head) * N;

  const int kvb = jb * BKV;
  const int kv0 = kvb + wave * 32;
  const int kv = kv0 + l32;
  frag kf[KS], vf[KS];
  load_row_frags<bf16, D>(kf, K + base, rs, kv, N, d, h);
  load_row_frags<bf16, D>(vf, V + base, rs, kv, N, d, h);

  f32x16 dv_acc[MT], dk_acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) { dv_acc[i] = zero16(); dk_acc[i] = zero16(); }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kvb / BQ : 0;
  const int ntiles = nqt - qt0;
  const int nsub = 2 * ntiles;

  auto fill = [&](Buf& B, int qt) ATTN_INLINE {
    const int q0 = qt * BQ;
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
        B.l[tid] = q < N ? Lh[q] : __builtin_inff();   // padded rows: P = 0
        B.dd[tid] = q < N ? Dh[q] : 0.f;
      }
    }
  };

  // S / dP accumulators of two consecutive sub-tiles; the roles (stage A
  // output, stage B input) alternate from step to step.
  f32x16 s0, p0, s1, p1;

  // One step.  HAS_A / HAS_B select the stages; MASK_B applies the causal
  // element mask to stage B's sub-tile (k - 1).  sa/pa receive stage A's
  // products; sb/pb hold stage B's (overwritten with P and dS).
  auto step = [&](int k, f32x16& sa, f32x16& pa, f32x16& sb, f32x16& pb, auto has_a_c,
                  auto has_b_c, auto mask_b_c) ATTN_INLINE {
    constexpr bool HAS_A = decltype(has_a_c)::value;
    constexpr bool HAS_B = decltype(has_b_c)::value;
    constexpr bool MASK_B = decltype(mask_b_c)::value;
    const int kb = k > 0 ? k - 1 : 0;
    const Buf& BA = buf[(k >> 1) % NB];
    const Buf& BB = buf[(kb >> 1) % NB];
    const QT tqa{const_cast<bf16*>(BA.q)}, toa{const_cast<bf16*>(BA.o)};
    const QT tqb{const_cast<bf16*>(BB.q)}, tob{const_cast<bf16*>(BB.o)};
    const int ra = (k & 1) * 32;              // sub-tile k's first row in its tile
    const int rb = (kb & 1) * 32;             // sub-tile k-1's first row in its tile
    const int qab = (qt0 + (kb >> 1)) * BQ + rb;   // absolute first query row, stage B

    frag aq[KS], ao[KS], tv[KS], tk[KS];
    frag bp[2], bds[2];
    constexpr int AHEAD = 2;                  // operand reads issued this many products ahead
    constexpr int PER = 16 / KS;              // P / dS registers handled per product

    // ---- preamble: first operands of both stages
    if constexpr (HAS_A) {
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) aq[i] = tqa.along_cols(ra + l32, i, h);
    }
    if constexpr (HAS_B) {
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) tv[i] = tob.along_rows((i % MT) * 32 + l32, rb, i / MT, h);
    }
    fence();
    // ---- phase 1: S(k) chain | P(k-1) on the VALU
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (HAS_A) {
        if (ks == 0) sa = M::mma(aq[0], kf[0], zero16());
        else sa = M::mma(aq[ks], kf[ks], sa);
        if (ks + AHEAD < KS) aq[ks + AHEAD] = tqa.along_cols(ra + l32, ks + AHEAD, h);
      }
      if constexpr (HAS_B) {
        // registers 4g .. 4g+3 share one 16-byte read of L2 (rows 8g + 4h + 0..3)
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int r = ks * PER + j;
          const f32x4 lg = lds_f32x4(&BB.l[rb + 8 * (r >> 2) + 4 * h]);
          float p = fast_exp2(__builtin_fmaf(sb[r], scale_log2, -lg[r & 3]));
          if (MASK_B && kv > qab + acc_row(r, h)) p = 0.f;
          sb[r] = p;
        }
      }
      fence();
    }
    if constexpr (HAS_B) {
      bp[0] = M::pack(sb, 0);
      bp[1] = M::pack(sb, 1);
    }
    if constexpr (HAS_A) {
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) ao[i] = toa.along_cols(ra + l32, i, h);
    }
    fence();
    // ---- phase 2: dV(k-1) chain | dS(k-1) on the VALU
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if constexpr (HAS_B) {
        const int ss = i / MT, mt = i % MT;
        dv_acc[mt] = M::mma(tv[i], bp[ss], dv_acc[mt]);
        if (i + AHEAD < KS) {
          const int n = i + AHEAD;
          tv[n] = tob.along_rows((n % MT) * 32 + l32, rb, n / MT, h);
        } else {
          const int n = i + AHEAD - KS;       // first dK operands
          tk[n] = tqb.along_rows((n % MT) * 32 + l32, rb, n / MT, h);
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int r = i * PER + j;
          const f32x4 dg = lds_f32x4(&BB.dd[rb + 8 * (r >> 2) + 4 * h]);
          pb[r] = sb[r] * (pb[r] - dg[r & 3]);
        }
      }
      fence();
    }
    if constexpr (HAS_B) {
      bds[0] = M::pack(pb, 0);
      bds[1] = M::pack(pb, 1);
    }
    fence();
    // ---- phase 3: dP(k) chain | dK(k-1) chain, interleaved
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if constexpr (HAS_A) {
        if (i == 0) pa = M::mma(ao[0], vf[0], zero16());
        else pa = M::mma(ao[i], vf[i], pa);
        if (i + AHEAD < KS) ao[i + AHEAD] = toa.along_cols(ra + l32, i + AHEAD, h);
      }
      if constexpr (HAS_B) {
        const int ss = i / MT, mt = i % MT;
        dk_acc[mt] = M::mma(tk[i], bds[ss], dk_acc[mt]);
        if (i + AHEAD < KS) {
          const int n = i + AHEAD;
          tk[n] = tqb.along_rows((n % MT) * 32 + l32, rb, n / MT, h);
        }
      }
      fence();
    }
  };

  const bool_c<true> Y{};
  const bool_c<false> F{};
  // entering tile t: its copy was issued two sub-steps ago; start tile t + 1's
  auto boundary = [&](int t) ATTN_INLINE {
    wait_async_fills();
    __syncthreads();
    if (t + 1 < ntiles) fill(buf[(t + 1) % NB], qt0 + t + 1);
  };
  // tile t = steps 2t (stage B on sub-tile 2t - 1) and 2t + 1 (on sub-tile 2t)
  auto tile = [&](int t, auto mask_first, auto mask_second) ATTN_INLINE {
    boundary(t);
    step(2 * t, s0, p0, s1, p1, Y, Y, mask_first);
    step(2 * t + 1, s1, p1, s0, p0, Y, Y, mask_second);
  };

  // ---- prologue: two tiles in flight, stage A of sub-tile 0
  fill(buf[0], qt0);
  if (ntiles > 1) fill(buf[1], qt0 + 1);
  wait_async_fills();
  __syncthreads();
  step(0, s0, p0, s1, p1, Y, F, F);
  // Causal: stage B of sub-tiles 0..3 (steps 1..4) crosses the diagonal and is
  // peeled off; the loop that follows carries no mask and no branch.
  int t0 = 1;
  step(1, s1, p1, s0, p0, Y, Y, bool_c<CAUSAL>{});
  if constexpr (CAUSAL) {
    if (ntiles > 1) tile(1, Y, Y);
    if (ntiles > 2) tile(2, Y, F);
    t0 = 3;
  }
  for (int t = t0; t < ntiles; ++t) tile(t, F, F);
  // drain: stage B of the last sub-tile (held in s1, p1)
  if (CAUSAL && ntiles <= 2)
    step(nsub, s0, p0, s1, p1, F, Y, Y);
  else
    step(nsub, s0, p0, s1, p1, F, Y, F);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    store_acc_transposed<bf16>(dv_acc[mt], dV + base, rs, kv0, mt * 32, N, d, 1.f, lane);
    store_acc_transposed<bf16>(dk_acc[mt], dK + base, rs, kv0, mt * 32, N, d, scale, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ (bf16).  Workgroup = 4 waves = 256 query rows of one (b, h); wave w owns
// query rows qw + [0, 64) as two 32-row halves c = 0, 1.  Q and dO of both
// halves and the dQ^T accumulators live in AGPRs for the whole kernel; L2 and
// D are two scalars per lane.  Each LDS operand fragment feeds one product
// per half (two matrix instructions per read).
//
// Key sub-tiles of 32 rows are software-pipelined, step j:
//   phase 1: S^T(j) = K Q^T          | VALU: P(j-1) = exp2(S scale log2e - L2)
//   phase 2: dP^T(j) = V dO^T        | VALU: dS(j-1) = P o (dP - D), packed
//   phase 3: dQ^T += K^T dS^T (j-1)
// Operand reads run AH fragments ahead and across phase boundaries.  Key
// tiles of 64 rows rotate through four LDS buffers, copied two tiles ahead,
// so the tile of sub-tile j-1 is still resident while step j reads it.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dws,
    bf16* __restrict__ dQ, int H, int N, int d, float scale_log2, float scale) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int BQ = 256, WQ = 64, BKV = 64, KS = D / 16, MT = D / 32, AH = 4;
  constexpr int PER = 16 / KS;      // elements per half handled per phase iteration
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
  const float* Lh = L2 + ((long)b * H + head) * N;
  const float* Dh = Dws + ((long)b * H + head) * N;

  const int qb = ib * BQ;
  const int qw = qb + wave * WQ;               // this wave's first query row
  const LanePlan<D> plan(lane);
  frag qf[2][KS], of[2][KS];
  float Lq[2], Dq[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = qw + 32 * c + l32;
    load_row_frags<bf16, D>(qf[c], Q + base, rs, q, N, d, h);
    load_row_frags<bf16, D>(of[c], dO + base, rs, q, N, d, h);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) { pin_agpr(qf[c][kk]); pin_agpr(of[c][kk]); }
    Lq[c] = q < N ? Lh[q] : __builtin_inff();
    Dq[c] = q < N ? Dh[q] : 0.f;
  }

  f32x16 acc[2][MT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) { acc[c][i] = zero16(); pin_agpr(acc[c][i]); }

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  // first tile holding key rows above some of the block's query rows
  const int diag0 = CAUSAL ? max(0, min(ntiles, qb / BKV)) : ntiles;

  auto fill = [&](Buf& B, int kt) ATTN_INLINE {
    const int k0 = kt * BKV;
    if (k0 + BKV <= N && d == D) {
      fill_async(KT{B.k}, K + base, rs, k0, wave, lane);
      fill_async(KT{B.v}, V + base, rs, k0, wave, lane);
    } else {
      fill_sync(KT{B.k}, K + base, rs, k0, N, d, tid);
      fill_sync(KT{B.v}, V + base, rs, k0, N, d, tid);
    }
  };

  // One key tile (two sub-tiles of 32 rows).  The operand stream of a
  // sub-tile is K (head dim), V (head dim), K^T (positions); reads run AH
  // operands ahead through the whole tile.
  constexpr int OPS = 2 * KS + 2 * MT;          // operands per sub-tile
  auto tile_body = [&](int kt, const Buf& B, bool masked) ATTN_INLINE {
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
      f32x16 sc[2], pc[2];
      // S^T = K Q^T (both halves)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int n = n0 + kk;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          sc[c] = kk == 0 ? M::mma(a, qf[c][0], zero16()) : M::mma(a, qf[c][kk], sc[c]);
        fence();
      }
      // dP^T = V dO^T (both halves) | P = exp2(S scale log2e - L2) on the VALU
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int n = n0 + KS + kk;
        const frag a = ring[n % AH];
        if (n + AH < 2 * OPS) ring[n % AH] = opnd(n + AH);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          pc[c] = kk == 0 ? M::mma(a, of[c][0], zero16()) : M::mma(a, of[c][kk], pc[c]);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int r = kk * PER + e;
            sc[c][r] = fast_exp2(__builtin_fmaf(sc[c][r], scale_log2, -Lq[c]));
          }
        fence();
      }
      // causal element mask, only on tiles that cross the diagonal
      if (masked) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int q = qw + 32 * c + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (ka + acc_row(r, h) > q) sc[c][r] = 0.f;
        }
      }
      fence();
      // dS = P o (dP - D): half 0 now, half 1 under half 0's dQ products
      frag bds[2][2];
#pragma unroll
      for (int r = 0; r < 16; ++r) pc[0][r] = sc[0][r] * (pc[0][r] - Dq[0]);
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
#pragma unroll
        for (int e = 0; e < PER3; ++e) {
          const int r = i * PER3 + e;
          pc[1][r] = sc[1][r] * (pc[1][r] - Dq[1]);
        }
        fence();
      }
      bds[1][0] = M::pack(pc[1], 0);
      bds[1][1] = M::pack(pc[1], 1);
      fence();
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) mma_acc_agpr(acc[1][i % MT], t[i], bds[1][i / MT]);
      fence();
    }
  };

  // tile kt + 1 is copied into the other buffer while tile kt is consumed
  auto run_tile = [&](int kt, const Buf& cur, Buf& nxt) ATTN_INLINE {
    wait_async_fills();
    __syncthreads();
    if (kt + 1 < ntiles) fill(nxt, kt + 1);
    tile_body(kt, cur, kt >= diag0);
  };

  fill(buf0, 0);
  for (int kt = 0; kt < ntiles; kt += 2) {
    run_tile(kt, buf0, buf1);
    if (kt + 1 < ntiles) run_tile(kt + 1, buf1, buf0);
  }

  mma_acc_drain();
#pragma unroll
  for (int c = 0; c < 2; ++c)
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

template <int D, bool C>
static hipError_t dq_pipe_go(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 255) / 256, a.H, a.B);
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, C>), grid, dim3(256), 0, stream,
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
