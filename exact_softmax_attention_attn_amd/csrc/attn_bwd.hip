// Backward kernels: preprocess (D), key-block-outer dK/dV, query-block-outer dQ.
//
// Method: exact attention backward with the scores rebuilt per tile from Q,
// K and the saved row scalar L = m + log z (ddx issue #243, "Attention's
// gradient: a softmax shift's backward computed twice, and recomputing scores
// instead of saving them", item 2), in the plan of ddx PR #162 ("perf(ddx-ad):
// transpose causal attention's contractions without their joins", section
// "What changed": transpose p = w/z per score, then p @ v).  The row-max
// shift contributes nothing (issue #243, item 1), so dS = P o (dP - D).
#include "common.h"
#include "launch.h"

namespace attn {

// ---------------------------------------------------------------------------
// D[b, h, n] = sum_c dO[b, n, h, c] * O[b, n, h, c], float32.
// 16 lanes per row, 16 rows per 256-thread block; 16-lane shuffle reduction.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const T* __restrict__ O,
                                                             const T* __restrict__ dO,
                                                             float* __restrict__ Dout, int B, int H,
                                                             int N, int d) {
  constexpr int VEC = Mma<T>::VEC;
  const int sub = threadIdx.x & 15;
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);  // row = (b * N + n) * H + h
  const long rows = (long)B * N * H;
  float acc = 0.f;
  if (row < rows) {
    const T* o = O + row * d;
    const T* g = dO + row * d;
    for (int c = sub * VEC; c < d; c += 16 * VEC) {
      if constexpr (sizeof(T) == 2) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(o + c);
        bf16x8 b = *reinterpret_cast<const bf16x8*>(g + c);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc += (float)a[t] * (float)b[t];
      } else {
        f32x4 a = *reinterpret_cast<const f32x4*>(o + c);
        f32x4 b = *reinterpret_cast<const f32x4*>(g + c);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc += a[t] * b[t];
      }
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) {
    const int h = (int)(row % H);
    const long bn = row / H;
    const int n = (int)(bn % N);
    const int b = (int)(bn / N);
    Dout[((long)b * H + h) * N + n] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 4 waves = one block of 128 key rows of one (b, h);
// wave w owns key rows kv0 + [0, 32).  K and V of those rows live in
// registers as B operands of S = Q K^T and dP = dO V^T (column n = key row).
// The accumulators hold dV^T and dK^T (rows = head dim, columns = key rows).
// Query blocks of 64 rows are staged in LDS (row-major for the contractions
// over the head dim, transposed for the contractions over positions).
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dws,
    T* __restrict__ dK, T* __restrict__ dV, int H, int N, int d, float scale_log2, float scale) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BKV = 128, BQ = 64, KS = D / M::K, MT = D / 32, RS = 32 / M::K;
  using QTile = Tile<T, BQ, D, sizeof(T) == 2>;

  __shared__ __align__(16) unsigned char smem[2 * QTile::BYTES + 2 * BQ * sizeof(float)];
  T* sbase = reinterpret_cast<T*>(smem);
  const QTile qs{sbase, sbase + QTile::RM_ELEMS};
  const QTile dos{sbase + QTile::RM_ELEMS + QTile::TR_ELEMS,
                  sbase + 2 * QTile::RM_ELEMS + QTile::TR_ELEMS};
  float* sL = reinterpret_cast<float*>(smem + 2 * QTile::BYTES);
  float* sD = sL + BQ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int jb = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int H_ = H;
  const long rs = (long)H_ * d;                       // elements between positions
  const long base = ((long)b * N * H_ + head) * d;    // (b, 0, head, 0)
  const float* Lh = L + ((long)b * H_ + head) * N;
  const float* Dh = Dws + ((long)b * H_ + head) * N;

  const int kvb = jb * BKV;
  const int kv0 = kvb + wave * 32;
  frag kf[KS], vf[KS];
  load_row_frags<T, D>(kf, K + base, rs, kv0 + l32, N, d, h);
  load_row_frags<T, D>(vf, V + base, rs, kv0 + l32, N, d, h);

  f32x16 dv_acc[MT], dk_acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) { dv_acc[i] = zero16(); dk_acc[i] = zero16(); }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kvb / BQ : 0;
  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * BQ;
    __syncthreads();
    qs.template stage<256>(Q + base, rs, q0, N, d, tid);
    dos.template stage<256>(dO + base, rs, q0, N, d, tid);
    if (tid < BQ) {
      const int q = q0 + tid;
      sL[tid] = q < N ? Lh[q] * kLog2e : __builtin_inff();
      sD[tid] = q < N ? Dh[q] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < BQ / 32; ++st) {
      const int qa = q0 + st * 32;                       // first query row of the sub-tile
      if (CAUSAL && qa + 31 < kv0) continue;             // every pair above the diagonal
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = M::mma(qs.along_cols(st * 32 + l32, ks, h), kf[ks], s);
        dp = M::mma(dos.along_cols(st * 32 + l32, ks, h), vf[ks], dp);
      }
      // s, dp: register r = query row qa + acc_row(r, h), column = key row kv0 + l32
      const bool diag = CAUSAL && (qa < kv0 + 32);
      const int kv = kv0 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = st * 32 + acc_row(r, h);
        float p = fast_exp2(s[r] * scale_log2 - sL[qi]);
        if (diag && kv > q0 + qi) p = 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - sD[qi]);
      }
#pragma unroll
      for (int ss = 0; ss < RS; ++ss) {
        const frag bp = M::pack(s, ss);
        const frag bds = M::pack(dp, ss);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          dv_acc[mt] = M::mma(dos.along_rows(mt * 32 + l32, st * 32, ss, h), bp, dv_acc[mt]);
          dk_acc[mt] = M::mma(qs.along_rows(mt * 32 + l32, st * 32, ss, h), bds, dk_acc[mt]);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    store_acc_transposed<T>(dv_acc[mt], dV + base, rs, kv0, mt * 32, N, d, 1.f, lane);
    store_acc_transposed<T>(dk_acc[mt], dK + base, rs, kv0, mt * 32, N, d, scale, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 waves = one block of 128 query rows of one (b, h); wave
// w owns query rows q0 + [0, 32), whose Q and dO sit in registers as B
// operands of S^T = K Q^T and dP^T = V dO^T (column n = query row), so L and
// D are one scalar per lane.  Key blocks of 64 rows are staged in LDS.  The
// accumulator holds dQ^T; every dQ element is written once, no atomics.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dws,
    T* __restrict__ dQ, int H, int N, int d, float scale_log2, float scale) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BQ = 128, BKV = 64, KS = D / M::K, MT = D / 32, RS = 32 / M::K;
  using KTile = Tile<T, BKV, D, sizeof(T) == 2>;
  using VTile = Tile<T, BKV, D, false>;

  __shared__ __align__(16) unsigned char smem[KTile::BYTES + VTile::BYTES];
  T* sbase = reinterpret_cast<T*>(smem);
  const KTile ks_{sbase, sbase + KTile::RM_ELEMS};
  const VTile vs_{sbase + KTile::RM_ELEMS + KTile::TR_ELEMS, nullptr};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nqb = gridDim.x;
  const int ib = CAUSAL ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;  // longest first
  const int head = blockIdx.y, b = blockIdx.z;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const float* Lh = L + ((long)b * H + head) * N;
  const float* Dh = Dws + ((long)b * H + head) * N;

  const int qb = ib * BQ;
  const int qw = qb + wave * 32;      // this wave's first query row
  const int q = qw + l32;             // this lane's query row (column of S^T)
  frag qf[KS], of[KS];
  load_row_frags<T, D>(qf, Q + base, rs, q, N, d, h);
  load_row_frags<T, D>(of, dO + base, rs, q, N, d, h);
  const float Lq = q < N ? Lh[q] * kLog2e : __builtin_inff();
  const float Dq = q < N ? Dh[q] : 0.f;

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = zero16();

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int nkt = (kv_end + BKV - 1) / BKV;
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BKV;
    __syncthreads();
    ks_.template stage<256>(K + base, rs, k0, N, d, tid);
    vs_.template stage<256>(V + base, rs, k0, N, d, tid);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < BKV / 32; ++st) {
      const int ka = k0 + st * 32;
      if (CAUSAL && ka > qw + 31) continue;
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        s = M::mma(ks_.along_cols(st * 32 + l32, kk, h), qf[kk], s);
        dp = M::mma(vs_.along_cols(st * 32 + l32, kk, h), of[kk], dp);
      }
      // register r = key row ka + acc_row(r, h), column = query row q
      const bool diag = CAUSAL && (ka + 31 > qw);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(s[r] * scale_log2 - Lq);
        if (diag && ka + acc_row(r, h) > q) p = 0.f;
        dp[r] = p * (dp[r] - Dq);
      }
#pragma unroll
      for (int ss = 0; ss < RS; ++ss) {
        const frag bds = M::pack(dp, ss);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = M::mma(ks_.along_rows(mt * 32 + l32, st * 32, ss, h), bds, acc[mt]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    store_acc_transposed<T>(acc[mt], dQ + base, rs, qw, mt * 32, N, d, scale, lane);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_bwd_preprocess_t(const void* O, const void* dO, float* Dws, int B, int H, int N,
                                   int d, hipStream_t stream) {
  const long rows = (long)B * N * H;
  const unsigned grid = (unsigned)((rows + 15) / 16);
  hipLaunchKernelGGL(bwd_preprocess_kernel<T>, dim3(grid), dim3(256), 0, stream,
                     static_cast<const T*>(O), static_cast<const T*>(dO), Dws, B, H, N, d);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const void* O, const void* dO, float* Dws, int B, int H, int N,
                                 int d, int dtype, hipStream_t stream) {
  if (dtype == 1) return launch_bwd_preprocess_t<bf16>(O, dO, Dws, B, H, N, d, stream);
  return launch_bwd_preprocess_t<float>(O, dO, Dws, B, H, N, d, stream);
}

template <typename T, int D, bool C>
static hipError_t dkdv_go(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, C>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.L, a.Dws,
                     static_cast<T*>(a.dK), static_cast<T*>(a.dV), a.H, a.N, a.d,
                     a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

template <typename T, int D, bool C>
static hipError_t dq_go(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, C>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.L, a.Dws,
                     static_cast<T*>(a.dQ), a.H, a.N, a.d, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

#define ATTN_DISPATCH(FN, a, stream)                                                  \
  do {                                                                                \
    const int bucket = head_dim_bucket((a).d);                                        \
    if ((a).dtype == 1) {                                                             \
      if ((a).causal) {                                                               \
        if (bucket == 32) return FN<bf16, 32, true>(a, stream);                       \
        if (bucket == 64) return FN<bf16, 64, true>(a, stream);                       \
        return FN<bf16, 128, true>(a, stream);                                        \
      }                                                                               \
      if (bucket == 32) return FN<bf16, 32, false>(a, stream);                        \
      if (bucket == 64) return FN<bf16, 64, false>(a, stream);                        \
      return FN<bf16, 128, false>(a, stream);                                         \
    }                                                                                 \
    if ((a).causal) {                                                                 \
      if (bucket == 32) return FN<float, 32, true>(a, stream);                        \
      if (bucket == 64) return FN<float, 64, true>(a, stream);                        \
      return FN<float, 128, true>(a, stream);                                         \
    }                                                                                 \
    if (bucket == 32) return FN<float, 32, false>(a, stream);                         \
    if (bucket == 64) return FN<float, 64, false>(a, stream);                         \
    return FN<float, 128, false>(a, stream);                                          \
  } while (0)

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) { ATTN_DISPATCH(dkdv_go, a, stream); }
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) { ATTN_DISPATCH(dq_go, a, stream); }

}  // namespace attn
