// Backward of the backward: gradients of l2 = <gQ, dQ> + <gK, dK> + <gV, dV>
// with respect to Q, K, V and dO, with no N x N intermediate in memory.
//
// Source: the page headed "Approaching I/O-optimality for Approximate
// Attention", its first abstract (FlashBoB), which sets the goal -- the exact
// gradient of the backward pass, with no N x N array in memory -- and says
// that a pair of per-row quantities is all such a pass needs beyond the
// recomputed tiles.  The formulas below are derived here from the chain rule,
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
// own rows as the B operands of 32x32 matrix products.  With a block mask
// (optional) each workgroup, whose 128 rows are one mask row or column,
// walks a visit list of the kept tiles instead of the whole range.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

namespace {
template <bool B> using bool_c = std::integral_constant<bool, B>;

__device__ __forceinline__ f32x16 splat16(float v) {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = v;
  return z;
}
}

// ---------------------------------------------------------------------------
// Query-block outer (PASS 1: r, E; PASS 2: hQ, hdO).  Workgroup = 128 query
// rows of one (b, h); wave w owns rows qw + [0, 32), whose Q, dO and gQ sit in
// registers as B operands, so S^T, dP^T, G^T, A^T come out with key rows along
// the registers and one query per lane (two lanes, l and l + 32, per query).
// ---------------------------------------------------------------------------
// Key rows per streamed tile: pass 1 at D = 128 (bf16) takes 32, so that its
// two 4-operand buffers (64 KB) leave LDS for a second workgroup on the CU,
// whose products and VALU work overlap this one's (pass 1 reduces into two
// scalars per row and fits two waves per SIMD); elsewhere 64.
template <typename T, int D, int PASS> constexpr int bob_q_tile_rows() {
  return (PASS == 1 && D == 128 && sizeof(T) == 2) ? 32 : 64;
}
template <typename T, int D, int PASS> constexpr int bob_q_min_blocks() {
  return bob_q_tile_rows<T, D, PASS>() == 32 ? 2 : 1;
}

template <typename T, int D, bool CAUSAL, int PASS>
__global__ __launch_bounds__(256, (bob_q_min_blocks<T, D, PASS>())) void bob_q_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const T* __restrict__ gQ, const T* __restrict__ gK,
    const T* __restrict__ gV, float* __restrict__ ws, T* __restrict__ hQ, T* __restrict__ hdO,
    int H, int N, int d, float scale_log2, float scale, const unsigned char* __restrict__ mask,
    int mask_heads) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BQ = 128, BKV = bob_q_tile_rows<T, D, PASS>(), KS = D / M::K, MT = D / 32,
                RS = 32 / M::K;
  constexpr int VT = 64, SUB = VT / BKV;     // visit-list tiles: 64 rows, SUB walk tiles each
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
  // the walk: key tiles 0 .. ceil(kv_end / BKV) - 1, or (block mask) those in
  // the kept 64-row tiles, a 64-row tile being kept when its mask block (row
  // ib: the workgroup's 128 query rows are one mask row) is
  static_assert(BQ == kMaskBlock, "one mask row per workgroup");
  __shared__ unsigned short vis[kMaxVisit];
  __shared__ int nvis;
  int ntiles = (kv_end + BKV - 1) / BKV;
  if (mask) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mk = head_mask(mask, mask_heads, b, head, H, nb);
    const int nvt = (kv_end + VT - 1) / VT;
    ntiles = SUB * build_visits(vis, &nvis, nvt, [&](int t) ATTN_INLINE -> unsigned {
      return mk[ib * nb + t * VT / kMaskBlock] ? (1u << 14) | (unsigned)t : 0u;
    });
  }
  // (masked, SUB = 2: the second half of a kept tile may lie past kv_end; its
  // rows read as zeros and every pair in it is masked, so it adds nothing)
  auto tile_at = [&](int p) ATTN_INLINE -> int {
    return mask ? SUB * (int)(visit_entry(vis, p / SUB) & kVisitTile) + p % SUB : p;
  };

  // bf16 whole tiles: direct copies by a plan built once (the tile base in
  // scalar registers, a 32-bit offset per lane and copy), waited for at the
  // end of each step
  using FS = AsyncFillShape<BKV, D>;
  unsigned copy_off[FS::PER];
  const int wu = wave_uniform(wave);
  if constexpr (sizeof(T) == 2) async_fill_plan<BKV, D>(copy_off, rs, wu, lane);
  auto fill = [&](Buf& B, int kt) ATTN_INLINE {
    const int k0 = kt * BKV;
    if constexpr (sizeof(T) == 2) {
      if (k0 + BKV <= N && d == D) {
        const long at = base + (long)k0 * rs;
        async_fill_untracked<BKV, D>(KT{B.k}, K + at, copy_off, wu);
        async_fill_untracked<BKV, D>(KT{B.v}, V + at, copy_off, wu);
        async_fill_untracked<BKV, D>(KT{B.gk}, gK + at, copy_off, wu);
        async_fill_untracked<BKV, D>(KT{B.gv}, gV + at, copy_off, wu);
        return;
      }
    }
    fill_sync(KT{B.k}, K + base, rs, k0, N, d, tid);
    fill_sync(KT{B.v}, V + base, rs, k0, N, d, tid);
    fill_sync(KT{B.gk}, gK + base, rs, k0, N, d, tid);
    fill_sync(KT{B.gv}, gV + base, rs, k0, N, d, tid);
  };

  // masked tiles keep key rows up to the lane's query (causal) and below N:
  // the zero rows padding the sequence's ragged last tile give S = 0, so
  // P = exp(-L), which overflows for L below about -88 and must not reach the
  // products (0 * inf)
  const int klim = CAUSAL ? q : N - 1;              // last kept key of the lane's query
  const int wlim = CAUSAL ? qw + 31 : N - 1;        // ... of any query of the wave
  // LDS operands are read ahead of the products that take them: two K steps
  // ahead in the first chain, one fenced group ahead after it, so each
  // group's reads are in flight while the previous group's products run.
  auto body = [&](const Buf& B, int k0, bool masked) ATTN_INLINE {
    const KT kt_{const_cast<T*>(B.k)}, vt_{const_cast<T*>(B.v)};
    const KT gkt_{const_cast<T*>(B.gk)}, gvt_{const_cast<T*>(B.gv)};
#pragma unroll 1
    for (int st = 0; st < BKV / 32; ++st) {
      const int ka = k0 + st * 32;
      if (masked && ka > wlim) continue;             // every pair masked
      const int rr = st * 32 + l32;
      // the hQ / hdO products of group i = (K step i / MT, columns i % MT)
      struct Ops { frag k, gk, gv, v; };
      auto rd = [&](int i) ATTN_INLINE -> Ops {
        const int ss = i / MT, c = (i % MT) * 32 + l32;
        return {kt_.along_rows(c, st * 32, ss, h), gkt_.along_rows(c, st * 32, ss, h),
                gvt_.along_rows(c, st * 32, ss, h), vt_.along_rows(c, st * 32, ss, h)};
      };
      Ops nx;
      // every register of a lane holds the lane's query, so its row scalars
      // start the accumulators: dP - D, and (pass 2) A - E
      f32x16 s = zero16(), g = zero16();
      f32x16 dp = PASS == 2 ? splat16(Dq) : zero16(), a = PASS == 2 ? splat16(-eq) : zero16();
      frag kc[KS], ngk, nv, ngv;
      kc[0] = kt_.along_cols(rr, 0, h);
      if constexpr (KS > 1) kc[1] = kt_.along_cols(rr, 1, h);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 2 < KS) kc[kk + 2] = kt_.along_cols(rr, kk + 2, h);
        if (kk == KS - 1) {
          ngk = gkt_.along_cols(rr, 0, h);
          nv = vt_.along_cols(rr, 0, h);
          ngv = gvt_.along_cols(rr, 0, h);
        }
        s = M::mma(kc[kk], qf[kk], s);
        g = M::mma(kc[kk], gqf[kk], g);
        __builtin_amdgcn_sched_barrier(0);
      }
      // register r = key row ka + acc_row(r, h), column = query row q.  S is
      // complete here: P = exp2(S scale log2 e - L2) is formed beside the G,
      // dP and A products (scheduling fences keep the interleave).
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const frag cgk = ngk, cv = nv, cgv = ngv;
        if (kk + 1 < KS) {
          ngk = gkt_.along_cols(rr, kk + 1, h);
          nv = vt_.along_cols(rr, kk + 1, h);
          ngv = gvt_.along_cols(rr, kk + 1, h);
        } else if constexpr (PASS == 2) {
          nx = rd(0);
        }
        g = M::mma(cgk, qf[kk], g);
        dp = M::mma(cv, of[kk], dp);
        a = M::mma(cgv, of[kk], a);
#pragma unroll
        for (int r = 16 * kk / KS; r < 16 * (kk + 1) / KS; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, Lq));
          if (masked && ka + acc_row(r, h) > klim) p = 0.f;
          s[r] = p;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      auto elem = [&](int r) ATTN_INLINE {
        const float p = s[r];
        const float dpd = PASS == 2 ? dp[r] : dp[r] + Dq;   // dP - D
        if constexpr (PASS == 1) {
          const float gg = g[r] * scale;              // G
          racc = __builtin_fmaf(p, gg, racc);
          eacc = __builtin_fmaf(p, __builtin_fmaf(dpd, gg, a[r]), eacc);
        } else {
          const float t = __builtin_fmaf(g[r], scale, -rq);   // G - r
          s[r] = p;                                           // P
          dp[r] = p * dpd;                                    // dS
          g[r] = p * __builtin_fmaf(dpd, t, a[r]);            // dS2 (a = A - E)
          a[r] = p * t;                                       // W
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
        auto prods = [&](int i) ATTN_INLINE {
          const Ops o = nx;
          if (i + 1 < 2 * NG) nx = rd(i + 1);
          const int ss = i / MT, mt = i % MT;
          acc_q[mt] = M::mma(o.k, bds2[ss], acc_q[mt]);
          acc_q[mt] = M::mma(o.gk, bds[ss], acc_q[mt]);
          acc_o[mt] = M::mma(o.gv, bp[ss], acc_o[mt]);
          acc_o[mt] = M::mma(o.v, bw[ss], acc_o[mt]);
        };
#pragma unroll
        for (int r = 0; r < 8; ++r) elem(r);
#pragma unroll
        for (int ss = 0; ss < HS; ++ss) pack(ss);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          prods(i);
#pragma unroll
          for (int r = 8 + 8 * i / NG; r < 8 + 8 * (i + 1) / NG; ++r) elem(r);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ss = HS; ss < RS; ++ss) pack(ss);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = NG; i < 2 * NG; ++i) {
          prods(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // step p: tile tile_at(p) in cur while tile tile_at(p + 1) is copied to nxt
  auto step = [&](const Buf& cur, Buf& nxt, int p) ATTN_INLINE {
    const int k0 = tile_at(p) * BKV;
    if (p + 1 < ntiles) fill(nxt, tile_at(p + 1));
    body(cur, k0, (CAUSAL && k0 + BKV - 1 > qb) || k0 + BKV > N);
    wait_async_fills();
    __syncthreads();
  };

  if (ntiles > 0) {                               // a masked walk may visit nothing
    fill(bufA, tile_at(0));
    wait_async_fills();
    __syncthreads();
  }
  for (int p = 0; p < ntiles; p += 2) {
    step(bufA, bufB, p);
    if (p + 1 < ntiles) step(bufB, bufA, p + 1);
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
    T* __restrict__ hV, int H, int N, int d, float scale_log2, float scale,
    const unsigned char* __restrict__ mask, int mask_heads) {
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
  // the walk: query tiles qt0 .. nqt - 1, or (block mask) the ones whose mask
  // block (row of the tile, column jb: the workgroup's 128 keys are one mask
  // column) is kept
  static_assert(BKV == kMaskBlock, "one mask column per workgroup");
  __shared__ unsigned short vis[kMaxVisit];
  __shared__ int nvis;
  int ntiles = nqt - qt0;
  if (mask) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mk = head_mask(mask, mask_heads, b, head, H, nb);
    ntiles = build_visits(vis, &nvis, ntiles, [&](int i) ATTN_INLINE -> unsigned {
      const int t = qt0 + i;
      return mk[(t * BQ / kMaskBlock) * nb + jb] ? (1u << 14) | (unsigned)t : 0u;
    });
  }
  auto tile_at = [&](int p) ATTN_INLINE -> int {
    return mask ? (int)(visit_entry(vis, p) & kVisitTile) : qt0 + p;
  };

  // bf16 whole tiles: direct copies by a plan built once, as in the
  // query-block outer kernel; each wave copies one of the four row scalars
  using FS = AsyncFillShape<BQ, D>;
  unsigned copy_off[FS::PER];
  const int wu = wave_uniform(wave);
  if constexpr (sizeof(T) == 2) async_fill_plan<BQ, D>(copy_off, rs, wu, lane);
  auto fill = [&](Buf& B, int qt) ATTN_INLINE {
    const int q0 = qt * BQ;
    if constexpr (sizeof(T) == 2) {
      if (q0 + BQ <= N && d == D) {
        const long at = base + (long)q0 * rs;
        async_fill_untracked<BQ, D>(QT{B.q}, Q + at, copy_off, wu);
        async_fill_untracked<BQ, D>(QT{B.o}, dO + at, copy_off, wu);
        async_fill_untracked<BQ, D>(QT{B.gq}, gQ + at, copy_off, wu);
        float* const dst[4] = {B.l, B.dd, B.r, B.e};
        const float* const src[4] = {nL2, nD, R, E};
        fill_row64_untracked(dst[wu], src[wu] + q0, lane);
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
      f32x16 s = zero16(), g = zero16(), a = zero16();
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
      f32x16 dp;                                    // starts at -D: dP - D
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = dg[r / 4][r % 4];
      // S is complete here: P is formed beside the G, dP and A products.
      // Their gQ and dO fragments are read one K step ahead of use.
      frag gqn = gqt_.along_cols(st * 32 + l32, 0, h), ocn = ot_.along_cols(st * 32 + l32, 0, h);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const frag gqc = gqn, oc = ocn;
        if (ks + 1 < KS) {
          gqn = gqt_.along_cols(st * 32 + l32, ks + 1, h);
          ocn = ot_.along_cols(st * 32 + l32, ks + 1, h);
        }
        g = M::mma(gqc, kf[ks], g);
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
        const float dpd = dp[r];                                  // dP - D
        const float t = __builtin_fmaf(g[r], scale, -rg[gi][i]);  // G - r
        dp[r] = p * dpd;                                          // dS
        s[r] = p * (__builtin_fmaf(dpd, t, a[r]) - eg[gi][i]);    // dS2
        a[r] = p * t;                                             // W
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
      // hV^T += dO^T W;  hK^T += Q^T dS2 + gQ^T dS.  Group i = (ss, mt) of
      // the NG * 2 groups; its three fragments are read one group ahead.
      frag ro[3];
      auto read_group = [&](int i) ATTN_INLINE {
        const int ss = i / MT, mt = i % MT;
        ro[0] = ot_.along_rows(mt * 32 + l32, st * 32, ss, h);
        ro[1] = qt_.along_rows(mt * 32 + l32, st * 32, ss, h);
        ro[2] = gqt_.along_rows(mt * 32 + l32, st * 32, ss, h);
      };
      auto prods = [&](int ss, int mt) ATTN_INLINE {
        const frag o0 = ro[0], o1 = ro[1], o2 = ro[2];
        const int i = ss * MT + mt;
        if (i + 1 < RS * MT) read_group(i + 1);
        acc_v[mt] = M::mma(o0, bw[ss], acc_v[mt]);
        acc_k[mt] = M::mma(o1, bds2[ss], acc_k[mt]);
        acc_k[mt] = M::mma(o2, bds[ss], acc_k[mt]);
      };
      read_group(0);
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

  // step p: tile tile_at(p) in cur while tile tile_at(p + 1) is copied to nxt
  auto step = [&](const Buf& cur, Buf& nxt, int p) ATTN_INLINE {
    const int q0 = tile_at(p) * BQ;
    if (p + 1 < ntiles) fill(nxt, tile_at(p + 1));
    body(cur, q0, CAUSAL && q0 < kvb + BKV);
    wait_async_fills();
    __syncthreads();
  };

  if (ntiles > 0) {                               // a masked walk may visit nothing
    fill(bufA, tile_at(0));
    wait_async_fills();
    __syncthreads();
  }
  for (int p = 0; p < ntiles; p += 2) {
    step(bufA, bufB, p);
    if (p + 1 < ntiles) step(bufB, bufA, p + 1);
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
                     static_cast<T*>(a.hdO), a.H, a.N, a.d, sl2, a.scale, a.mask,
                     a.mask_heads);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_kv_kernel<T, D, C>), gq, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO),
                     static_cast<const T*>(a.gQ), static_cast<const T*>(a.gK),
                     static_cast<const T*>(a.gV), a.ws, static_cast<T*>(a.hK),
                     static_cast<T*>(a.hV), a.H, a.N, a.d, sl2, a.scale, a.mask,
                     a.mask_heads);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bob_q2_pipe_serves(a)) return launch_bob_q2_pipe(a, stream);
  hipLaunchKernelGGL((bob_q_kernel<T, D, C, 2>), gq, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO),
                     static_cast<const T*>(a.gQ), static_cast<const T*>(a.gK),
                     static_cast<const T*>(a.gV), a.ws, static_cast<T*>(a.hQ),
                     static_cast<T*>(a.hdO), a.H, a.N, a.d, sl2, a.scale, a.mask,
                     a.mask_heads);
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
