// Backward kernels: preprocess (D), key-block-outer dK/dV, query-block-outer dQ.
//
// Method: exact attention backward with the scores rebuilt per tile from Q,
// K and the saved row scalar L = m + log z (ddx issue #243, "Attention's
// gradient: a softmax shift's backward computed twice, and recomputing scores
// instead of saving them", item 2), in the plan of ddx PR #162 ("perf(ddx-ad):
// transpose causal attention's contractions without their joins", section
// "What changed": transpose p = w/z per score, then p @ v).  The row-max
// shift contributes nothing (issue #243, item 1), so dS = P o (dP - D).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

template <bool B> using bool_c = std::integral_constant<bool, B>;

// ---------------------------------------------------------------------------
// Preprocess.  D[b, h, n] = sum_c dO[b, n, h, c] * O[b, n, h, c] in float32
// (the softmax-weighted sum of dP, since sum_j P_ij dP_ij = dO_i . O_i), and
// L2[b, h, n] = L[b, h, n] * log2(e), the row scalar in the base-2 units the
// kernels exponentiate in.  Both are stored negated (-D, -L2): the kernels
// add them, which lets them enter a matrix instruction as its C input.
// 16 lanes per row; a 256-thread block takes 16 consecutive positions of one
// (b, h), so its 16 results land side by side in the [B, H, N] outputs.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const T* __restrict__ O,
                                                             const T* __restrict__ dO,
                                                             const float* __restrict__ L,
                                                             float* __restrict__ Dout,
                                                             float* __restrict__ L2out, int B,
                                                             int H, int N, int d) {
  constexpr int VEC = Mma<T>::CHUNK;
  const int sub = threadIdx.x & 15;
  const int chunks = (N + 15) / 16;
  const long bh = blockIdx.x / chunks;                          // = b * H + h
  const int n = (int)(blockIdx.x % chunks) * 16 + (threadIdx.x >> 4);
  const int h = (int)(bh % H);
  const long b = bh / H;
  const long row = (b * N + n) * H + h;                         // input row of [B, N, H, d]
  float acc = 0.f;
  if (n < N) {
    const T* o = O + row * d;
    const T* g = dO + row * d;
    for (int c = sub * VEC; c < d; c += 16 * VEC) {
      if constexpr (sizeof(T) == 2) {
        acc = dot8_bf16(*reinterpret_cast<const bf16x8*>(o + c),
                        *reinterpret_cast<const bf16x8*>(g + c), acc);
      } else {
        f32x4 a = *reinterpret_cast<const f32x4*>(o + c);
        f32x4 b = *reinterpret_cast<const f32x4*>(g + c);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc += a[t] * b[t];
      }
    }
  }
  acc = sum16_lanes(acc);
  if (n < N && sub == 0) {
    const long i = bh * N + n;
    Dout[i] = -acc;
    // a row with no kept key (L = -inf) stores -inf, so every P of it is 0
    L2out[i] = L[i] == -__builtin_inff() ? -__builtin_inff() : -L[i] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 4 waves = one block of 128 key rows of one (b, h);
// wave w owns key rows kv0 + [0, 32).  K and V of those rows sit in
// registers as B operands of S = Q K^T and dP = dO V^T (column n = key row),
// so P and dS come out with the query rows along the registers and feed
// dV^T += dO^T P and dK^T += Q^T dS directly.  The accumulators hold dV^T
// and dK^T (rows = head dim, columns = key rows).  Query blocks of 64 rows
// (Q, dO and their L2, D) are double-buffered in LDS: the next block is
// copied in while the current one is consumed.  Causal: the walk starts at
// the diagonal; only the two diagonal blocks carry the element mask.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dws,
    T* __restrict__ dK, T* __restrict__ dV, int H, int N, int d, float scale_log2, float scale,
    const unsigned char* __restrict__ mask, int mask_heads) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BKV = 128, BQ = 64, KS = D / M::K, RS = 32 / M::K;
  // Wide heads (bf16 256 bucket, float32 128 bucket): each workgroup
  // accumulates DA of the output's columns (part = which DA) and recomputes S
  // and dP over the full head dim, so a (b, h) runs on D / DA workgroups per
  // block.
  constexpr int DA = out_cols<T, D>(), MA = DA / 32, NSPLIT = D / DA;
  using QT = Tile<T, BQ, D>;
  struct __align__(16) Buf {
    T q[QT::ELEMS];
    T o[QT::ELEMS];
    float l[BQ];
    float dd[BQ];
  };
  __shared__ Buf bufA, bufB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const BlockOrder bo = block_order();
  const int jb = bo.rank, head = bo.head / NSPLIT, b = bo.b;   // rank 0 = longest walk
  const int dofs = (bo.head % NSPLIT) * DA;          // first output column of this workgroup
  const long rs = (long)H * d;                       // elements between positions
  const long base = ((long)b * N * H + head) * d;    // (b, 0, head, 0)
  const float* Lh = L2 + ((long)b * H + head) * N;
  const float* Dh = Dws + ((long)b * H + head) * N;

  const int kvb = jb * BKV;
  const int kv0 = kvb + wave * 32;
  const int kv = kv0 + l32;                          // this lane's key row
  frag kf[KS], vf[KS];
  load_row_frags<T, D>(kf, K + base, rs, kv, N, d, h);
  load_row_frags<T, D>(vf, V + base, rs, kv, N, d, h);

  f32x16 dv_acc[MA], dk_acc[MA];
#pragma unroll
  for (int i = 0; i < MA; ++i) { dv_acc[i] = zero16(); dk_acc[i] = zero16(); }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kvb / BQ : 0;
  // the walk: query tiles qt0 .. nqt - 1, or (block-sparse mask) the ones whose
  // mask block (row of the tile, column jb of this key block) is kept
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

  // bf16 whole tiles: direct copies by a plan built once per workgroup (the
  // tile base in scalar registers, a 32-bit offset per lane and copy), waited
  // for at the end of each step
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
        if (wu == 0) fill_row64_untracked(B.l, Lh + q0, lane);
        if (wu == 1) fill_row64_untracked(B.dd, Dh + q0, lane);
        return;
      }
    }
    fill_sync(QT{B.q}, Q + base, rs, q0, N, d, tid);
    fill_sync(QT{B.o}, dO + base, rs, q0, N, d, tid);
    if (tid < BQ) {
      const int q = q0 + tid;
      B.l[tid] = q < N ? Lh[q] : -__builtin_inff();   // padded rows: P = 0 (-L2 stored)
      B.dd[tid] = q < N ? Dh[q] : 0.f;                // -D stored
    }
  };

  // One body for masked and unmasked tiles, its two sub-tiles in a loop: at
  // head dim 256 two inlined copies would not fit in registers.
  auto body = [&](const Buf& B, int q0, bool MASKED) ATTN_INLINE {
    const QT qt_{const_cast<T*>(B.q)}, ot_{const_cast<T*>(B.o)};
#pragma unroll 1
    for (int st = 0; st < BQ / 32; ++st) {
      const int qa = q0 + st * 32;                 // first query row of the sub-tile
      if (MASKED && qa + 31 < kv0) continue;       // every pair above the diagonal
      if constexpr (sizeof(T) == 2 && D > 128) {
        // bf16 head dim 256: the sub-tile's operands (Q, dO along the head
        // dim for S and dP; dO, Q across positions for dV and dK) are read
        // in one sequence, RA fragments ahead of their products through a
        // ring, with the order held by scheduling fences, so that no product
        // waits on a read issued right before it
        constexpr int RA = 3, NG = RS * MA, NOP = 2 * KS + 2 * NG;
        auto opnd = [&](int n) ATTN_INLINE -> frag {
          if (n < KS) return qt_.along_cols(st * 32 + l32, n, h);
          if (n < 2 * KS) return ot_.along_cols(st * 32 + l32, n - KS, h);
          const int j = (n - 2 * KS) % NG;
          const QT& src = n < 2 * KS + NG ? ot_ : qt_;
          return src.along_rows(dofs + (j % MA) * 32 + l32, st * 32, j / MA, h);
        };
        frag ring[RA];
#pragma unroll
        for (int n = 0; n < RA; ++n) ring[n] = opnd(n);
        auto take = [&](int n) ATTN_INLINE -> frag {
          const frag a = ring[n % RA];
          if (n + RA < NOP) ring[n % RA] = opnd(n + RA);
          return a;
        };
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int n = 0; n < 2 * KS; ++n) {
          const frag a = take(n);
          if (n < KS) s = M::mma(a, kf[n], s);
          else dp = M::mma(a, vf[n - KS], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 lg = *reinterpret_cast<const f32x4*>(&B.l[st * 32 + 8 * g + 4 * h]);
          const f32x4 dg = *reinterpret_cast<const f32x4*>(&B.dd[st * 32 + 8 * g + 4 * h]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, lg[i]));
            if (MASKED && kv > qa + acc_row(r, h)) p = 0.f;
            s[r] = p;
            dp[r] = p * (dp[r] + dg[i]);
          }
        }
        frag bp[RS], bds[RS];
#pragma unroll
        for (int ss = 0; ss < RS; ++ss) {
          bp[ss] = M::pack(s, ss);
          bds[ss] = M::pack(dp, ss);
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          dv_acc[j % MA] = M::mma(take(2 * KS + j), bp[j / MA], dv_acc[j % MA]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          dk_acc[j % MA] = M::mma(take(2 * KS + NG + j), bds[j / MA], dk_acc[j % MA]);
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      // S and dP: register r = query row qa + acc_row(r, h), column = key row kv
      frag aq[KS], ao[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) aq[ks] = qt_.along_cols(st * 32 + l32, ks, h);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ao[ks] = ot_.along_cols(st * 32 + l32, ks, h);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = M::mma(aq[ks], kf[ks], s);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dp = M::mma(ao[ks], vf[ks], dp);
      // P = exp2(S * scale * log2 e - L2), masked above the diagonal
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lg = *reinterpret_cast<const f32x4*>(&B.l[st * 32 + 8 * g + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, lg[i]));
          if (MASKED && kv > qa + acc_row(r, h)) p = 0.f;
          s[r] = p;
        }
      }
      frag bp[RS];
#pragma unroll
      for (int ss = 0; ss < RS; ++ss) bp[ss] = M::pack(s, ss);
      // dV^T += dO^T P
#pragma unroll
      for (int ss = 0; ss < RS; ++ss)
#pragma unroll
        for (int mt = 0; mt < MA; ++mt)
          dv_acc[mt] = M::mma(ot_.along_rows(dofs + mt * 32 + l32, st * 32, ss, h), bp[ss],
                              dv_acc[mt]);
      // dS = P o (dP - D)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 dg = *reinterpret_cast<const f32x4*>(&B.dd[st * 32 + 8 * g + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[4 * g + i] = s[4 * g + i] * (dp[4 * g + i] + dg[i]);
      }
      frag bds[RS];
#pragma unroll
      for (int ss = 0; ss < RS; ++ss) bds[ss] = M::pack(dp, ss);
      // dK^T += Q^T dS
#pragma unroll
      for (int ss = 0; ss < RS; ++ss)
#pragma unroll
        for (int mt = 0; mt < MA; ++mt)
          dk_acc[mt] = M::mma(qt_.along_rows(dofs + mt * 32 + l32, st * 32, ss, h), bds[ss],
                              dk_acc[mt]);
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

  if (ntiles > 0) {                               // a sparse walk may visit nothing
    fill(bufA, tile_at(0));
    wait_async_fills();
    __syncthreads();
  }
  for (int p = 0; p < ntiles; p += 2) {
    step(bufA, bufB, p);
    if (p + 1 < ntiles) step(bufB, bufA, p + 1);
  }

#pragma unroll
  for (int mt = 0; mt < MA; ++mt) {
    store_acc_transposed<T>(dv_acc[mt], dV + base, rs, kv0, dofs + mt * 32, N, d, 1.f, lane);
    store_acc_transposed<T>(dk_acc[mt], dK + base, rs, kv0, dofs + mt * 32, N, d, scale, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 4 waves = one block of 128 query rows of one (b, h); wave
// w owns query rows qw + [0, 32), whose Q and dO sit in registers as B
// operands of S^T = K Q^T and dP^T = V dO^T (column n = query row), so L2 and
// D are one scalar per lane and dS^T comes out with the key rows along the
// registers, ready for dQ^T += K^T dS^T.  Key blocks of 64 rows (K, V) are
// double-buffered in LDS.  Every dQ element is written once: no atomics.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dws,
    T* __restrict__ dQ, int H, int N, int d, float scale_log2, float scale,
    const unsigned char* __restrict__ mask, int mask_heads) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BQ = 128, BKV = 64, KS = D / M::K, RS = 32 / M::K;
  // Wide heads (bf16 256 bucket, float32 128 bucket): each workgroup
  // accumulates DA of the output's columns (part = which DA) and recomputes S
  // and dP over the full head dim, so a (b, h) runs on D / DA workgroups per
  // block.
  constexpr int DA = out_cols<T, D>(), MA = DA / 32, NSPLIT = D / DA;
  using KT = Tile<T, BKV, D>;
  struct __align__(16) Buf {
    T k[KT::ELEMS];
    T v[KT::ELEMS];
  };
  __shared__ Buf bufA, bufB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nqb = gridDim.x;
  const BlockOrder bo = block_order();
  const int ib = CAUSAL ? (nqb - 1 - bo.rank) : bo.rank;   // longest first
  const int head = bo.head / NSPLIT, b = bo.b;
  const int dofs = (bo.head % NSPLIT) * DA;          // first output column of this workgroup
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const float* Lh = L2 + ((long)b * H + head) * N;
  const float* Dh = Dws + ((long)b * H + head) * N;

  const int qb = ib * BQ;
  const int qw = qb + wave * 32;      // this wave's first query row
  const int q = qw + l32;             // this lane's query row (column of S^T)
  frag qf[KS], of[KS];
  load_row_frags<T, D>(qf, Q + base, rs, q, N, d, h);
  load_row_frags<T, D>(of, dO + base, rs, q, N, d, h);
  const float Lq = q < N ? Lh[q] : -__builtin_inff();   // -L2 stored; padded rows: P = 0
  const float Dq = q < N ? Dh[q] : 0.f;                  // -D stored

  f32x16 acc[MA];
#pragma unroll
  for (int i = 0; i < MA; ++i) acc[i] = zero16();

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int nkt = (kv_end + BKV - 1) / BKV;
  // the walk: key tiles 0 .. nkt - 1, or (block-sparse mask) the ones whose
  // mask block (row ib of this query block, column of the tile) is kept
  __shared__ unsigned short vis[kMaxVisit];
  __shared__ int nvis;
  int ntiles = nkt;
  if (mask) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mk = head_mask(mask, mask_heads, b, head, H, nb);
    ntiles = build_visits(vis, &nvis, nkt, [&](int t) ATTN_INLINE -> unsigned {
      return mk[ib * nb + t * BKV / kMaskBlock] ? (1u << 14) | (unsigned)t : 0u;
    });
  }
  auto tile_at = [&](int p) ATTN_INLINE -> int {
    return mask ? (int)(visit_entry(vis, p) & kVisitTile) : p;
  };

  // bf16 whole tiles: direct copies by a plan built once per workgroup
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
        return;
      }
    }
    fill_sync(KT{B.k}, K + base, rs, k0, N, d, tid);
    fill_sync(KT{B.v}, V + base, rs, k0, N, d, tid);
  };

  // MASKED tiles keep key rows up to the lane's query (causal) and below N:
  // the zero rows padding the sequence's ragged last tile give S = 0, so
  // P = exp(-L), which overflows for L below about -88 and must not reach the
  // products (0 * inf)
  const int klim = CAUSAL ? q : N - 1;              // last kept key of the lane's query
  const int wlim = CAUSAL ? qw + 31 : N - 1;        // ... of any query of the wave
  // (bf16 head dim 256: the operands of one sub-tile's S, dP and dQ products
  // are read in one sequence, RA fragments ahead of their products through a
  // ring, with the order held by scheduling fences; read all at once they
  // would take 128 registers and leave every product waiting on its read)
  constexpr bool RING = sizeof(T) == 2 && D > 128;
  constexpr int RA = 3;
  auto body = [&](const Buf& B, int k0, auto masked_c) ATTN_INLINE {
    constexpr bool MASKED = decltype(masked_c)::value;
    const KT kt_{const_cast<T*>(B.k)}, vt_{const_cast<T*>(B.v)};
#pragma unroll
    for (int st = 0; st < BKV / 32; ++st) {
      const int ka = k0 + st * 32;
      if (MASKED && ka > wlim) continue;           // every pair masked
      f32x16 s = zero16(), dp = zero16();
      if constexpr (RING) {
        // operand n of the sub-tile: K along the head dim (n < KS), V along
        // the head dim (KS <= n < 2 KS), K across positions (then)
        constexpr int NOP = 2 * KS + RS * MA;
        auto opnd = [&](int n) ATTN_INLINE -> frag {
          if (n < KS) return kt_.along_cols(st * 32 + l32, n, h);
          if (n < 2 * KS) return vt_.along_cols(st * 32 + l32, n - KS, h);
          const int j = n - 2 * KS;
          return kt_.along_rows(dofs + (j % MA) * 32 + l32, st * 32, j / MA, h);
        };
        frag ring[RA];
#pragma unroll
        for (int n = 0; n < RA; ++n) ring[n] = opnd(n);
#pragma unroll
        for (int n = 0; n < 2 * KS; ++n) {
          const frag a = ring[n % RA];
          if (n + RA < NOP) ring[n % RA] = opnd(n + RA);
          if (n < KS) s = M::mma(a, qf[n], s);
          else dp = M::mma(a, of[n - KS], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, Lq));
          if (MASKED && ka + acc_row(r, h) > klim) p = 0.f;
          dp[r] = p * (dp[r] + Dq);
        }
        frag bds[RS];
#pragma unroll
        for (int ss = 0; ss < RS; ++ss) bds[ss] = M::pack(dp, ss);
#pragma unroll
        for (int j = 0; j < RS * MA; ++j) {
          const int n = 2 * KS + j;
          const frag a = ring[n % RA];
          if (n + RA < NOP) ring[n % RA] = opnd(n + RA);
          acc[j % MA] = M::mma(a, bds[j / MA], acc[j % MA]);
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      frag ak[KS], av[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) ak[kk] = kt_.along_cols(st * 32 + l32, kk, h);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) av[kk] = vt_.along_cols(st * 32 + l32, kk, h);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) s = M::mma(ak[kk], qf[kk], s);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) dp = M::mma(av[kk], of[kk], dp);
      // register r = key row ka + acc_row(r, h), column = query row q
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, Lq));
        if (MASKED && ka + acc_row(r, h) > klim) p = 0.f;
        dp[r] = p * (dp[r] + Dq);
      }
      frag bds[RS];
#pragma unroll
      for (int ss = 0; ss < RS; ++ss) bds[ss] = M::pack(dp, ss);
#pragma unroll
      for (int ss = 0; ss < RS; ++ss)
#pragma unroll
        for (int mt = 0; mt < MA; ++mt)
          acc[mt] = M::mma(kt_.along_rows(dofs + mt * 32 + l32, st * 32, ss, h), bds[ss], acc[mt]);
    }
  };

  // step p: tile tile_at(p) in cur while tile tile_at(p + 1) is copied to nxt
  auto step = [&](const Buf& cur, Buf& nxt, int p) ATTN_INLINE {
    const int k0 = tile_at(p) * BKV;
    if (p + 1 < ntiles) fill(nxt, tile_at(p + 1));
    if ((CAUSAL && k0 + BKV - 1 > qb) || k0 + BKV > N)
      body(cur, k0, bool_c<true>{});
    else
      body(cur, k0, bool_c<false>{});
    wait_async_fills();
    __syncthreads();
  };

  if (ntiles > 0) {                               // a sparse walk may visit nothing
    fill(bufA, tile_at(0));
    wait_async_fills();
    __syncthreads();
  }
  for (int p = 0; p < ntiles; p += 2) {
    step(bufA, bufB, p);
    if (p + 1 < ntiles) step(bufB, bufA, p + 1);
  }
#pragma unroll
  for (int mt = 0; mt < MA; ++mt)
    store_acc_transposed<T>(acc[mt], dQ + base, rs, qw, dofs + mt * 32, N, d, scale, lane);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_bwd_preprocess_t(const void* O, const void* dO, const float* L, float* ws, int B,
                                   int H, int N, int d, hipStream_t stream) {
  const long rows = (long)B * N * H;
  const unsigned grid = (unsigned)((long)B * H * ((N + 15) / 16));
  hipLaunchKernelGGL(bwd_preprocess_kernel<T>, dim3(grid), dim3(256), 0, stream,
                     static_cast<const T*>(O), static_cast<const T*>(dO), L, ws, ws + rows, B, H,
                     N, d);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const void* O, const void* dO, const float* L, float* ws, int B,
                                 int H, int N, int d, int dtype, hipStream_t stream) {
  if (dtype == 1) return launch_bwd_preprocess_t<bf16>(O, dO, L, ws, B, H, N, d, stream);
  return launch_bwd_preprocess_t<float>(O, dO, L, ws, B, H, N, d, stream);
}

static inline long rows_of(const BwdArgs& a) { return (long)a.B * a.H * a.N; }

// workgroups per block: one per out_cols output columns
template <typename T, int D> constexpr int column_parts() { return D / out_cols<T, D>(); }

template <typename T, int D, bool C>
static hipError_t dkdv_go(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H * column_parts<T, D>(), a.B);
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, C>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.Dws + rows_of(a), a.Dws,
                     static_cast<T*>(a.dK), static_cast<T*>(a.dV), a.H, a.N, a.d,
                     a.scale * kLog2e, a.scale, a.mask, a.mask_heads);
  return hipGetLastError();
}

template <typename T, int D, bool C>
static hipError_t dq_go(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H * column_parts<T, D>(), a.B);
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, C>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.Dws + rows_of(a), a.Dws,
                     static_cast<T*>(a.dQ), a.H, a.N, a.d, a.scale * kLog2e, a.scale, a.mask,
                     a.mask_heads);
  return hipGetLastError();
}

#define ATTN_DISPATCH(FN, a, stream)                                                  \
  do {                                                                                \
    const int bucket = head_dim_bucket((a).d);                                        \
    if ((a).dtype == 1) {                                                             \
      if ((a).causal) {                                                               \
        if (bucket == 32) return FN<bf16, 32, true>(a, stream);                       \
        if (bucket == 64) return FN<bf16, 64, true>(a, stream);                       \
        if (bucket == 128) return FN<bf16, 128, true>(a, stream);                     \
        return FN<bf16, 256, true>(a, stream);                                        \
      }                                                                               \
      if (bucket == 32) return FN<bf16, 32, false>(a, stream);                        \
      if (bucket == 64) return FN<bf16, 64, false>(a, stream);                        \
      if (bucket == 128) return FN<bf16, 128, false>(a, stream);                      \
      return FN<bf16, 256, false>(a, stream);                                         \
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

// bf16 with a head dim of exactly 64 or 128 runs the software-pipelined
// kernels (they copy whole tiles only); everything else the generic ones.
static bool use_pipe(const BwdArgs& a) { return a.dtype == 1 && (a.d == 64 || a.d == 128); }

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  if (use_pipe(a)) return launch_bwd_dkdv_bf16_pipe(a, stream);
  ATTN_DISPATCH(dkdv_go, a, stream);
}
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  if (use_pipe(a)) return launch_bwd_dq_bf16_pipe(a, stream);
  ATTN_DISPATCH(dq_go, a, stream);
}

bool bwd_dq_fuses_preprocess(const BwdArgs& a) { return use_pipe(a); }
hipError_t launch_bwd_dq_fused(const BwdArgs& a, hipStream_t stream) {
  if (!use_pipe(a) || !a.O || !a.L || !a.ws_out) return hipErrorInvalidValue;
  return launch_bwd_dq_fused_bf16_pipe(a, stream);
}

}  // namespace attn
