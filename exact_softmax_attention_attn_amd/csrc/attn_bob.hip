// Backward of the backward: gradients of l2 = <gQ, dQ> + <gK, dK> + <gV, dV>
// with respect to Q, K, V and dO, with no N x N intermediate in memory.
//
// The FlashBoB paper's abstract ("FlashBoB: exact, I/O-efficient backward-
// over-backward for softmax attention") states the structure used here: two
// row-wise scalars fix every output through affine maps, which gives a
// two-pass schedule over recomputed tiles.  Written out from the chain rule,
// with P, dP = dO V^T, D and dS = P o (dP - D) as in the first backward:
//   G = scale (gQ K^T + Q gK^T)    (cotangent of dS)
//   A = dO gV^T                    (cotangent of P through dV)
//   r_i = sum_j P_ij G_ij,         E_i = sum_j (P_ij A_ij + dS_ij G_ij)
//   W   = P o (G - r)              (cotangent of dP)
//   dS2 = P o (A + (dP - D) o (G - r) - E)   (cotangent of S)
//   hQ  = scale (dS2 K + dS gK),   hK = scale (dS2^T Q + dS^T gQ)
//   hV  = W^T dO,                  hdO = P gV + W V
// (E uses sum_j dS_ij = 0, so it needs no r.)  Pass 1 (query-block outer)
// rebuilds S, dP, G, A per tile and reduces r and E per row; pass 2 walks the
// tiles again, key-block outer for hK, hV and query-block outer for hQ, hdO.
//
// The kernels follow the generic forward / backward kernels' tiling: 4 waves,
// 32 rows per wave, 64-row streamed tiles double-buffered in LDS, the wave's
// own rows as the B operands of 32x32 matrix products.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

namespace {
template <bool B> using bool_c = std::integral_constant<bool, B>;
}

// ---------------------------------------------------------------------------
// Query-block outer (PASS 1: r, E; PASS 2: hQ, hdO).  Workgroup = 128 query
// rows of one (b, h); wave w owns rows qw + [0, 32), whose Q, dO and gQ sit in
// registers as B operands, so S^T, dP^T, G^T, A^T come out with key rows along
// the registers and one query per lane (two lanes, l and l + 32, per query).
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, int PASS>
__global__ __launch_bounds__(256, 1) void bob_q_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const T* __restrict__ gQ, const T* __restrict__ gK,
    const T* __restrict__ gV, float* __restrict__ ws, T* __restrict__ hQ, T* __restrict__ hdO,
    int H, int N, int d, float scale_log2, float scale) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BQ = 128, BKV = 64, KS = D / M::K, MT = D / 32, RS = 32 / M::K;
  using KT = Tile<T, BKV, D>;
  struct __align__(16) Buf {
    T k[KT::ELEMS];
    T v[KT::ELEMS];
    T gk[KT::ELEMS];
    T gv[KT::ELEMS];
  };
  __shared__ Buf bufA, bufB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nqb = gridDim.x;
  const BlockOrder bo = block_order();
  const int ib = CAUSAL ? (nqb - 1 - bo.rank) : bo.rank;   // longest first
  const int head = bo.head, b = bo.b;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const long rows = (long)gridDim.z * H * N;             // B * H * N
  const long rbase = ((long)b * H + head) * N;
  // workspace: -D, -L log2(e), r, E, each [B, H, N]
  const float* nD = ws;
  const float* nL2 = ws + rows;
  float* R = ws + 2 * rows;
  float* E = ws + 3 * rows;

  const int qb = ib * BQ;
  const int qw = qb + wave * 32;
  const int q = qw + l32;                   // this lane's query row (column of the products)
  frag qf[KS], of[KS], gqf[KS];
  load_row_frags<T, D>(qf, Q + base, rs, q, N, d, h);
  load_row_frags<T, D>(of, dO + base, rs, q, N, d, h);
  load_row_frags<T, D>(gqf, gQ + base, rs, q, N, d, h);
  const float Lq = q < N ? nL2[rbase + q] : -__builtin_inff();   // padded rows: P = 0
  const float Dq = q < N ? nD[rbase + q] : 0.f;
  const float rq = (PASS == 2 && q < N) ? R[rbase + q] : 0.f;
  const float eq = (PASS == 2 && q < N) ? E[rbase + q] : 0.f;

  float racc = 0.f, eacc = 0.f;             // PASS 1: this lane's share of r and E
  f32x16 acc_q[PASS == 2 ? MT : 1], acc_o[PASS == 2 ? MT : 1];
#pragma unroll
  for (int i = 0; i < (PASS == 2 ? MT : 1); ++i) { acc_q[i] = zero16(); acc_o[i] = zero16(); }

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int nkt = (kv_end + BKV - 1) / BKV;

  auto fill = [&](Buf& B, int kt) ATTN_INLINE {
    const int k0 = kt * BKV;
    if constexpr (sizeof(T) == 2) {
      if (k0 + BKV <= N && d == D) {
        fill_async(KT{B.k}, K + base, rs, k0, wave, lane);
        fill_async(KT{B.v}, V + base, rs, k0, wave, lane);
        fill_async(KT{B.gk}, gK + base, rs, k0, wave, lane);
        fill_async(KT{B.gv}, gV + base, rs, k0, wave, lane);
        return;
      }
    }
    fill_sync(KT{B.k}, K + base, rs, k0, N, d, tid);
    fill_sync(KT{B.v}, V + base, rs, k0, N, d, tid);
    fill_sync(KT{B.gk}, gK + base, rs, k0, N, d, tid);
    fill_sync(KT{B.gv}, gV + base, rs, k0, N, d, tid);
  };

  auto body = [&](const Buf& B, int k0, bool masked) ATTN_INLINE {
    const KT kt_{const_cast<T*>(B.k)}, vt_{const_cast<T*>(B.v)};
    const KT gkt_{const_cast<T*>(B.gk)}, gvt_{const_cast<T*>(B.gv)};
#pragma unroll 1
    for (int st = 0; st < BKV / 32; ++st) {
      const int ka = k0 + st * 32;
      if (masked && ka > qw + 31) continue;          // every pair above the diagonal
      f32x16 s = zero16(), dp = zero16(), g = zero16(), a = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const frag kc = kt_.along_cols(st * 32 + l32, kk, h);
        s = M::mma(kc, qf[kk], s);
        g = M::mma(kc, gqf[kk], g);
      }
      // register r = key row ka + acc_row(r, h), column = query row q.  S is
      // complete here: P = exp2(S scale log2 e - L2) is formed beside the G,
      // dP and A products (scheduling fences keep the interleave).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        g = M::mma(gkt_.along_cols(st * 32 + l32, kk, h), qf[kk], g);
        const frag vc = vt_.along_cols(st * 32 + l32, kk, h);
        dp = M::mma(vc, of[kk], dp);
        a = M::mma(gvt_.along_cols(st * 32 + l32, kk, h), of[kk], a);
#pragma unroll
        for (int r = 16 * kk / KS; r < 16 * (kk + 1) / KS; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, Lq));
          if (masked && ka + acc_row(r, h) > q) p = 0.f;
          s[r] = p;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      auto elem = [&](int r) ATTN_INLINE {
        const float p = s[r];
        const float dpd = dp[r] + Dq;                 // dP - D
        const float gg = g[r] * scale;                // G
        if constexpr (PASS == 1) {
          racc += p * gg;
          eacc += p * a[r] + p * dpd * gg;
        } else {
          const float w = p * (gg - rq);
          s[r] = p;                                     // P
          dp[r] = p * dpd;                              // dS
          g[r] = p * (a[r] + dpd * (gg - rq) - eq);     // dS2
          a[r] = w;                                     // W
        }
      };
      if constexpr (PASS == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) elem(r);
      } else {
        // The first half of the registers (K steps 0 .. RS/2 - 1) is packed
        // first; its products run while the VALU works on the second half.
        constexpr int HS = RS / 2, NG = HS * MT;
        frag bp[RS], bds[RS], bds2[RS], bw[RS];
        auto pack = [&](int ss) ATTN_INLINE {
          bp[ss] = M::pack(s, ss);
          bds[ss] = M::pack(dp, ss);
          bds2[ss] = M::pack(g, ss);
          bw[ss] = M::pack(a, ss);
        };
        // hQ^T += K^T dS2^T + gK^T dS^T;  hdO^T += gV^T P^T + V^T W^T
        auto prods = [&](int ss, int mt) ATTN_INLINE {
          acc_q[mt] = M::mma(kt_.along_rows(mt * 32 + l32, st * 32, ss, h), bds2[ss], acc_q[mt]);
          acc_q[mt] = M::mma(gkt_.along_rows(mt * 32 + l32, st * 32, ss, h), bds[ss], acc_q[mt]);
          acc_o[mt] = M::mma(gvt_.along_rows(mt * 32 + l32, st * 32, ss, h), bp[ss], acc_o[mt]);
          acc_o[mt] = M::mma(vt_.along_rows(mt * 32 + l32, st * 32, ss, h), bw[ss], acc_o[mt]);
        };
#pragma unroll
        for (int r = 0; r < 8; ++r) elem(r);
#pragma unroll
        for (int ss = 0; ss < HS; ++ss) pack(ss);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          prods(i / MT, i % MT);
#pragma unroll
          for (int r = 8 + 8 * i / NG; r < 8 + 8 * (i + 1) / NG; ++r) elem(r);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ss = HS; ss < RS; ++ss) pack(ss);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NG; ++i) prods(HS + i / MT, i % MT);
      }
    }
  };

  auto step = [&](const Buf& cur, Buf& nxt, int kt) ATTN_INLINE {
    if (kt + 1 < nkt) fill(nxt, kt + 1);
    const int k0 = kt * BKV;
    body(cur, k0, CAUSAL && k0 + BKV - 1 > qb);
    wait_async_fills();
    __syncthreads();
  };

  fill(bufA, 0);
  wait_async_fills();
  __syncthreads();
  for (int kt = 0; kt < nkt; kt += 2) {
    step(bufA, bufB, kt);
    if (kt + 1 < nkt) step(bufB, bufA, kt + 1);
  }

  if constexpr (PASS == 1) {
    // the lane holds half of the query's keys; its partner 32 lanes away the rest
    racc += __shfl_xor(racc, 32);
    eacc += __shfl_xor(eacc, 32);
    if (h == 0 && q < N) {
      R[rbase + q] = racc;
      E[rbase + q] = eacc;
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      store_acc_transposed<T>(acc_q[mt], hQ + base, rs, qw, mt * 32, N, d, scale, lane);
      store_acc_transposed<T>(acc_o[mt], hdO + base, rs, qw, mt * 32, N, d, 1.f, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Key-block outer (pass 2: hK, hV).  Workgroup = 128 key rows of one (b, h);
// wave w owns key rows kv0 + [0, 32), whose K, V, gK, gV sit in registers as
// B operands, so S, dP, G, A come out with query rows along the registers;
// the query tiles (Q, dO, gQ and the four row scalars) stream through LDS.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bob_kv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const T* __restrict__ gQ, const T* __restrict__ gK,
    const T* __restrict__ gV, const float* __restrict__ ws, T* __restrict__ hK,
    T* __restrict__ hV, int H, int N, int d, float scale_log2, float scale) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BKV = 128, BQ = 64, KS = D / M::K, MT = D / 32, RS = 32 / M::K;
  using QT = Tile<T, BQ, D>;
  struct __align__(16) Buf {
    T q[QT::ELEMS];
    T o[QT::ELEMS];
    T gq[QT::ELEMS];
    float l[BQ];     // -L log2(e)
    float dd[BQ];    // -D
    float r[BQ];
    float e[BQ];
  };
  __shared__ Buf bufA, bufB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const BlockOrder bo = block_order();
  const int jb = bo.rank, head = bo.head, b = bo.b;      // rank 0 = longest walk
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const long rows = (long)gridDim.z * H * N;
  const long rbase = ((long)b * H + head) * N;
  const float* nD = ws + rbase;
  const float* nL2 = ws + rows + rbase;
  const float* R = ws + 2 * rows + rbase;
  const float* E = ws + 3 * rows + rbase;

  const int kvb = jb * BKV;
  const int kv0 = kvb + wave * 32;
  const int kv = kv0 + l32;
  frag kf[KS], vf[KS], gkf[KS], gvf[KS];
  load_row_frags<T, D>(kf, K + base, rs, kv, N, d, h);
  load_row_frags<T, D>(vf, V + base, rs, kv, N, d, h);
  load_row_frags<T, D>(gkf, gK + base, rs, kv, N, d, h);
  load_row_frags<T, D>(gvf, gV + base, rs, kv, N, d, h);

  f32x16 acc_k[MT], acc_v[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) { acc_k[i] = zero16(); acc_v[i] = zero16(); }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kvb / BQ : 0;

  auto fill = [&](Buf& B, int qt) ATTN_INLINE {
    const int q0 = qt * BQ;
    if constexpr (sizeof(T) == 2) {
      if (q0 + BQ <= N && d == D) {
        fill_async(QT{B.q}, Q + base, rs, q0, wave, lane);
        fill_async(QT{B.o}, dO + base, rs, q0, wave, lane);
        fill_async(QT{B.gq}, gQ + base, rs, q0, wave, lane);
        if (wave == 0) fill_async_row64(B.l, nL2 + q0);
        if (wave == 1) fill_async_row64(B.dd, nD + q0);
        if (wave == 2) fill_async_row64(B.r, R + q0);
        if (wave == 3) fill_async_row64(B.e, E + q0);
        return;
      }
    }
    fill_sync(QT{B.q}, Q + base, rs, q0, N, d, tid);
    fill_sync(QT{B.o}, dO + base, rs, q0, N, d, tid);
    fill_sync(QT{B.gq}, gQ + base, rs, q0, N, d, tid);
    if (tid < BQ) {
      const int qq = q0 + tid;
      B.l[tid] = qq < N ? nL2[qq] : -__builtin_inff();   // padded rows: P = 0
      B.dd[tid] = qq < N ? nD[qq] : 0.f;
      B.r[tid] = qq < N ? R[qq] : 0.f;
      B.e[tid] = qq < N ? E[qq] : 0.f;
    }
  };

  auto body = [&](const Buf& B, int q0, bool masked) ATTN_INLINE {
    const QT qt_{const_cast<T*>(B.q)}, ot_{const_cast<T*>(B.o)}, gqt_{const_cast<T*>(B.gq)};
#pragma unroll 1
    for (int st = 0; st < BQ / 32; ++st) {
      const int qa = q0 + st * 32;
      if (masked && qa + 31 < kv0) continue;       // every pair above the diagonal
      f32x16 s = zero16(), dp = zero16(), g = zero16(), a = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const frag qc = qt_.along_cols(st * 32 + l32, ks, h);
        s = M::mma(qc, kf[ks], s);
        g = M::mma(qc, gkf[ks], g);
      }
      // register r = query row qa + acc_row(r, h), column = key row kv; the
      // row scalars of registers 4 gi .. 4 gi + 3
      f32x4 lg[4], dg[4], rg[4], eg[4];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int i0 = st * 32 + 8 * gi + 4 * h;
        lg[gi] = *reinterpret_cast<const f32x4*>(&B.l[i0]);
        dg[gi] = *reinterpret_cast<const f32x4*>(&B.dd[i0]);
        rg[gi] = *reinterpret_cast<const f32x4*>(&B.r[i0]);
        eg[gi] = *reinterpret_cast<const f32x4*>(&B.e[i0]);
      }
      // S is complete here: P is formed beside the G, dP and A products
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        g = M::mma(gqt_.along_cols(st * 32 + l32, ks, h), kf[ks], g);
        const frag oc = ot_.along_cols(st * 32 + l32, ks, h);
        dp = M::mma(oc, vf[ks], dp);
        a = M::mma(oc, gvf[ks], a);
#pragma unroll
        for (int r = 16 * ks / KS; r < 16 * (ks + 1) / KS; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, lg[r / 4][r % 4]));
          if (masked && kv > qa + acc_row(r, h)) p = 0.f;
          s[r] = p;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      auto elem = [&](int r) ATTN_INLINE {
        const int gi = r / 4, i = r % 4;
        const float p = s[r];
        const float dpd = dp[r] + dg[gi][i];        // dP - D
        const float gg = g[r] * scale;              // G
        dp[r] = p * dpd;                            // dS
        s[r] = p * (a[r] + dpd * (gg - rg[gi][i]) - eg[gi][i]);   // dS2
        a[r] = p * (gg - rg[gi][i]);                // W
      };
      // The first half of the registers (K steps 0 .. RS/2 - 1) is packed
      // first; its products run while the VALU works on the second half.
      constexpr int HS = RS / 2, NG = HS * MT;
      frag bds[RS], bds2[RS], bw[RS];
      auto pack = [&](int ss) ATTN_INLINE {
        bds[ss] = M::pack(dp, ss);
        bds2[ss] = M::pack(s, ss);
        bw[ss] = M::pack(a, ss);
      };
      // hV^T += dO^T W;  hK^T += Q^T dS2 + gQ^T dS
      auto prods = [&](int ss, int mt) ATTN_INLINE {
        acc_v[mt] = M::mma(ot_.along_rows(mt * 32 + l32, st * 32, ss, h), bw[ss], acc_v[mt]);
        acc_k[mt] = M::mma(qt_.along_rows(mt * 32 + l32, st * 32, ss, h), bds2[ss], acc_k[mt]);
        acc_k[mt] = M::mma(gqt_.along_rows(mt * 32 + l32, st * 32, ss, h), bds[ss], acc_k[mt]);
      };
#pragma unroll
      for (int r = 0; r < 8; ++r) elem(r);
#pragma unroll
      for (int ss = 0; ss < HS; ++ss) pack(ss);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        prods(i / MT, i % MT);
#pragma unroll
        for (int r = 8 + 8 * i / NG; r < 8 + 8 * (i + 1) / NG; ++r) elem(r);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ss = HS; ss < RS; ++ss) pack(ss);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NG; ++i) prods(HS + i / MT, i % MT);
    }
  };

  auto step = [&](const Buf& cur, Buf& nxt, int qt) ATTN_INLINE {
    if (qt + 1 < nqt) fill(nxt, qt + 1);
    const int q0 = qt * BQ;
    body(cur, q0, CAUSAL && q0 < kvb + BKV);
    wait_async_fills();
    __syncthreads();
  };

  fill(bufA, qt0);
  wait_async_fills();
  __syncthreads();
  for (int qt = qt0; qt < nqt; qt += 2) {
    step(bufA, bufB, qt);
    if (qt + 1 < nqt) step(bufB, bufA, qt + 1);
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    store_acc_transposed<T>(acc_v[mt], hV + base, rs, kv0, mt * 32, N, d, 1.f, lane);
    store_acc_transposed<T>(acc_k[mt], hK + base, rs, kv0, mt * 32, N, d, scale, lane);
  }
}

// ---------------------------------------------------------------------------
// Launchers: preprocess (-D, -L log2 e), pass 1 (r, E), then both halves of
// pass 2, all on one stream.
// ---------------------------------------------------------------------------
template <typename T, int D, bool C>
static hipError_t bob_go(const BobArgs& a, hipStream_t stream) {
  const dim3 gq((a.N + 127) / 128, a.H, a.B);
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((bob_q_kernel<T, D, C, 1>), gq, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO),
                     static_cast<const T*>(a.gQ), static_cast<const T*>(a.gK),
                     static_cast<const T*>(a.gV), a.ws, static_cast<T*>(a.hQ),
                     static_cast<T*>(a.hdO), a.H, a.N, a.d, sl2, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_kv_kernel<T, D, C>), gq, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO),
                     static_cast<const T*>(a.gQ), static_cast<const T*>(a.gK),
                     static_cast<const T*>(a.gV), a.ws, static_cast<T*>(a.hK),
                     static_cast<T*>(a.hV), a.H, a.N, a.d, sl2, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_q_kernel<T, D, C, 2>), gq, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO),
                     static_cast<const T*>(a.gQ), static_cast<const T*>(a.gK),
                     static_cast<const T*>(a.gV), a.ws, static_cast<T*>(a.hQ),
                     static_cast<T*>(a.hdO), a.H, a.N, a.d, sl2, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_bwd(const BobArgs& a, hipStream_t stream) {
  hipError_t e = launch_bwd_preprocess(a.O, a.dO, a.L, a.ws, a.B, a.H, a.N, a.d, a.dtype, stream);
  if (e != hipSuccess) return e;
  const int bucket = head_dim_bucket(a.d);
  if (a.dtype == 1) {
    if (a.causal) {
      if (bucket == 32) return bob_go<bf16, 32, true>(a, stream);
      if (bucket == 64) return bob_go<bf16, 64, true>(a, stream);
      return bob_go<bf16, 128, true>(a, stream);
    }
    if (bucket == 32) return bob_go<bf16, 32, false>(a, stream);
    if (bucket == 64) return bob_go<bf16, 64, false>(a, stream);
    return bob_go<bf16, 128, false>(a, stream);
  }
  if (a.causal) {
    if (bucket == 32) return bob_go<float, 32, true>(a, stream);
    return bob_go<float, 64, true>(a, stream);
  }
  if (bucket == 32) return bob_go<float, 32, false>(a, stream);
  return bob_go<float, 64, false>(a, stream);
}

}  // namespace attn
