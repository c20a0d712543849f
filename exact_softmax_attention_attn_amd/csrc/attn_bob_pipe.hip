// Backward of the backward, pass 2 (query-block outer: hQ, hdO), software-
// pipelined for bf16 at head dims 64 and 128.  Built with every builtin MFMA
// in VGPR form (its rebuilt scores feed the VALU), so it has a file of its
// own; the other passes are in attn_bob.hip, which also holds the launcher
// that picks this kernel.
//
// Source: the page headed "Approaching I/O-optimality for Approximate
// Attention", its first abstract (FlashBoB): the exact gradient of the
// backward pass with no N x N array in memory.  The formulas (derived from the
// chain rule) are those of attn_bob.hip:
//   dS2 = P o (A + (dP - D) o (G - r) - E),  W = P o (G - r),
//   hQ = scale (dS2 K + dS gK),  hdO = P gV + W V.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {
__device__ __forceinline__ f32x16 splat16(float v) {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = v;
  return z;
}
}  // namespace

// ---------------------------------------------------------------------------
// Pass 2, query-block outer, software-pipelined (bf16, D = 64 or 128): hQ, hdO.
// The same workgroup, walk and arithmetic as bob_q_kernel<PASS 2>, laid out as
// the first backward's pipelined kernels are:
// - Q, dO and gQ of the wave's rows (B operands) and the hQ^T, hdO^T
//   accumulators stay in AGPRs; the accumulating products are inline
//   (mma_acc_agpr), so the rebuilt S, G, dP, A come out in VGPRs;
// - key tiles of 32 rows (K, V, gK, gV) rotate through three LDS buffers, the
//   copy of tile j + 2 going out right after the barrier that publishes j + 1
//   (a ragged last tile is copied before the walk into a fourth);
// - step j runs the S, G, dP, A chains of tile j + 1 beside the elementwise
//   block and packing of tile j, then tile j's hQ / hdO products beside the
//   exponentials of tile j + 1, so each VALU stage reads chains that finished
//   a stage earlier and the matrix core is fed throughout.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bob_q2_pipe_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const bf16* __restrict__ gQ, const bf16* __restrict__ gK,
    const bf16* __restrict__ gV, const float* __restrict__ ws, bf16* __restrict__ hQ,
    bf16* __restrict__ hdO, int H, int N, int d, float scale_log2, float scale,
    const unsigned char* __restrict__ mask, int mask_heads) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int BQ = 128, BKV = 32, KS = D / 16, MT = D / 32, RS = 2;
  constexpr int VT = 64, SUB = VT / BKV;       // visit-list tiles: 64 rows, SUB walk tiles each
  constexpr int EPK = 16 / KS;                 // elementwise registers per chain step
  constexpr int EPG = 16 / (RS * MT);          // exponentials per product group
  static_assert(D == 64 || D == 128, "pipelined pass 2 serves D = 64 and 128");
  using KT = Tile<bf16, BKV, D>;
  struct __align__(16) Buf {
    bf16 k[KT::ELEMS];
    bf16 v[KT::ELEMS];
    bf16 gk[KT::ELEMS];
    bf16 gv[KT::ELEMS];
  };
  __shared__ Buf buf0, buf1, buf2, bufr;       // a ring of three; bufr: the ragged last tile

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int nqb = gridDim.x;
  const BlockOrder bo = block_order();
  const int ib = CAUSAL ? (nqb - 1 - bo.rank) : bo.rank;   // longest first
  const int head = bo.head, b = bo.b;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const long rows = (long)gridDim.z * H * N;
  const long rbase = ((long)b * H + head) * N;
  const float* nD = ws;
  const float* nL2 = ws + rows;
  const float* R = ws + 2 * rows;
  const float* E = ws + 3 * rows;

  const int qb = ib * BQ;
  const int qw = qb + wave * 32;
  const int q = qw + l32;
  frag qf[KS], of[KS], gqf[KS];
  load_row_frags<bf16, D>(qf, Q + base, rs, q, N, d, h);
  load_row_frags<bf16, D>(of, dO + base, rs, q, N, d, h);
  load_row_frags<bf16, D>(gqf, gQ + base, rs, q, N, d, h);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    pin_agpr(qf[kk]);
    pin_agpr(of[kk]);
    pin_agpr(gqf[kk]);
  }
  const float Lq = q < N ? nL2[rbase + q] : -__builtin_inff();   // padded rows: P = 0
  const float Dq = q < N ? nD[rbase + q] : 0.f;
  const float rq = q < N ? R[rbase + q] : 0.f;
  const float eq = q < N ? E[rbase + q] : 0.f;

  f32x16 acc[2][MT];                           // [0]: hQ^T, [1]: hdO^T
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) { acc[c][i] = zero16(); pin_agpr(acc[c][i]); }

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
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
  auto tile_at = [&](int p) ATTN_INLINE -> int {
    return mask ? SUB * (int)(visit_entry(vis, p / SUB) & kVisitTile) + p % SUB : p;
  };
  // a kept 64-row tile's second half past kv_end keeps no pair: dropped (it can
  // only be the walk's last tile)
  if (mask && ntiles > 0 && tile_at(ntiles - 1) * BKV >= kv_end) --ntiles;
  // Only the walk's last tile can reach past N (the sequence's ragged end).
  // It is copied by the register path into a buffer of its own before the
  // walk, so the walk's copies are all direct (no register-path loads whose
  // waits would land inside the pipelined steps).
  const bool last_ragged = ntiles > 0 && tile_at(ntiles - 1) * BKV + BKV > N;

  using FS = AsyncFillShape<BKV, D>;
  unsigned copy_off[FS::PER];
  async_fill_plan<BKV, D>(copy_off, rs, wave, lane);
  const LanePlan<D> plan(lane);
  // the buffer of walk tile j
  auto buf_of = [&](int j) ATTN_INLINE -> Buf& {
    if (last_ragged && j == ntiles - 1) return bufr;
    const int i = j % 3;
    return i == 0 ? buf0 : (i == 1 ? buf1 : buf2);
  };
  // walk tile j into its buffer (whole tiles; the ragged one is already there)
  auto fill = [&](int j) ATTN_INLINE {
    if (last_ragged && j == ntiles - 1) return;
    Buf& B = buf_of(j);
    const long at = base + (long)tile_at(j) * BKV * rs;
    async_fill_untracked<BKV, D>(KT{B.k}, K + at, copy_off, wave);
    async_fill_untracked<BKV, D>(KT{B.v}, V + at, copy_off, wave);
    async_fill_untracked<BKV, D>(KT{B.gk}, gK + at, copy_off, wave);
    async_fill_untracked<BKV, D>(KT{B.gv}, gV + at, copy_off, wave);
  };
  if (last_ragged) {
    const int k0 = tile_at(ntiles - 1) * BKV;
    fill_sync<bf16, BKV, D>(KT{bufr.k}, K + base, rs, k0, N, d, tid);
    fill_sync<bf16, BKV, D>(KT{bufr.v}, V + base, rs, k0, N, d, tid);
    fill_sync<bf16, BKV, D>(KT{bufr.gk}, gK + base, rs, k0, N, d, tid);
    fill_sync<bf16, BKV, D>(KT{bufr.gv}, gV + base, rs, k0, N, d, tid);
  }

  // registers of a tile: register r = key row k0 + acc_row(r, h), column =
  // the lane's query.  S becomes P, dP - D becomes dS, G becomes dS2, A - E
  // becomes W.
  struct Set { f32x16 s, dp, g, a; };
  const int klim = CAUSAL ? q : N - 1;         // last kept key of the lane's query
  auto masked_at = [&](int k0) ATTN_INLINE -> bool {
    return (CAUSAL && k0 + BKV - 1 > qb) || k0 + BKV > N;
  };
  auto exp_one = [&](Set& X, int r, int k0, bool masked) ATTN_INLINE {
    float p = fast_exp2(__builtin_fmaf(X.s[r], scale_log2, Lq));
    if (masked && k0 + acc_row(r, h) > klim) p = 0.f;
    X.s[r] = p;
  };
  auto elem_one = [&](Set& X, int r) ATTN_INLINE {
    const float p = X.s[r];
    const float dpd = X.dp[r];                               // dP - D
    const float t = __builtin_fmaf(X.g[r], scale, -rq);      // G - r
    X.dp[r] = p * dpd;                                       // dS
    X.g[r] = p * __builtin_fmaf(dpd, t, X.a[r]);             // dS2 (a = A - E)
    X.a[r] = p * t;                                          // W
  };
  // the S, G, dP, A chains of the tile in T into X, with `beside(kk)` (VALU
  // work on other registers) after the products of K step kk
  auto chains = [&](Set& X, const Buf& T, auto&& beside) ATTN_INLINE {
    // (the starting values are formed here each time: hoisted out of the
    // walk they would hold 32 registers for its whole length)
    float d0 = Dq, e0 = -eq;
    asm volatile("" : "+v"(d0), "+v"(e0));
    X.s = zero16();
    X.g = zero16();
    X.dp = splat16(d0);
    X.a = splat16(e0);
    // K, gK, V and gV of the next K step are read one step ahead
    frag kc = plan.cols(T.k, 0, 0), gkc = plan.cols(T.gk, 0, 0);
    frag vc = plan.cols(T.v, 0, 0), gvc = plan.cols(T.gv, 0, 0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const frag c0 = kc, c1 = gkc, c2 = vc, c3 = gvc;
      if (kk + 1 < KS) {
        kc = plan.cols(T.k, 0, kk + 1);
        gkc = plan.cols(T.gk, 0, kk + 1);
        vc = plan.cols(T.v, 0, kk + 1);
        gvc = plan.cols(T.gv, 0, kk + 1);
      }
      X.s = M::mma(c0, qf[kk], X.s);
      X.g = M::mma(c0, gqf[kk], X.g);
      X.g = M::mma(c1, qf[kk], X.g);
      X.dp = M::mma(c2, of[kk], X.dp);
      X.a = M::mma(c3, of[kk], X.a);
      beside(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // hQ^T += K^T dS2^T + gK^T dS^T;  hdO^T += gV^T P^T + V^T W^T for the tile in
  // T (packed operands), with `beside(i)` after product group i
  auto prods = [&](const Buf& T, const frag (&bp)[RS], const frag (&bds)[RS],
                   const frag (&bds2)[RS], const frag (&bw)[RS], auto&& beside) ATTN_INLINE {
    // K^T, gK^T, gV^T and V^T of the next group are read one group ahead
    frag nk = plan.rows(T.k, 0, 0, 0), ngk = plan.rows(T.gk, 0, 0, 0);
    frag ngv = plan.rows(T.gv, 0, 0, 0), nv = plan.rows(T.v, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < RS * MT; ++i) {
      const int ss = i / MT, mt = i % MT;
      const frag ok = nk, ogk = ngk, ogv = ngv, ov = nv;
      if (i + 1 < RS * MT) {
        nk = plan.rows(T.k, 0, (i + 1) / MT, (i + 1) % MT);
        ngk = plan.rows(T.gk, 0, (i + 1) / MT, (i + 1) % MT);
        ngv = plan.rows(T.gv, 0, (i + 1) / MT, (i + 1) % MT);
        nv = plan.rows(T.v, 0, (i + 1) / MT, (i + 1) % MT);
      }
      need_both(ok, ogk);
      mma_acc_agpr(acc[0][mt], ok, bds2[ss]);
      mma_acc_agpr(acc[0][mt], ogk, bds[ss]);
      need_both(ogv, ov);
      mma_acc_agpr(acc[1][mt], ogv, bp[ss]);
      mma_acc_agpr(acc[1][mt], ov, bw[ss]);
      beside(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: tiles 0 and 1 in flight, tile 0's chains and exponentials
  Set A, B;
  if (ntiles > 0) {
    fill(0);
    if (ntiles > 1) fill(1);
    wait_async_fills();
    lds_barrier();
    const int k0 = tile_at(0) * BKV;
    chains(A, buf_of(0), [&](int) ATTN_INLINE {});
    const bool m0 = masked_at(k0);
#pragma unroll
    for (int r = 0; r < 16; ++r) exp_one(A, r, k0, m0);
  }
  // step j: tile j's registers in X (P formed), tile j + 1's chains into Y
  // step j: tile j's registers in X (P formed), tile j + 1's chains into Y
  auto step = [&](Set& X, Set& Y, int j) ATTN_INLINE {
    const bool more = j + 1 < ntiles;
    // tile j + 1 has landed (every wave), and every wave is done with the
    // buffer of tile j - 1, which tile j + 2 now fills
    wait_async_fills();
    lds_barrier();
    if (j + 2 < ntiles) fill(j + 2);
    const Buf& cur = buf_of(j);
    const Buf& nxt = buf_of(j + 1);
    frag bp[RS], bds[RS], bds2[RS], bw[RS];
    auto pack = [&](int ss) ATTN_INLINE {
      bp[ss] = M::pack(X.s, ss);
      bds[ss] = M::pack(X.dp, ss);
      bds2[ss] = M::pack(X.g, ss);
      bw[ss] = M::pack(X.a, ss);
      pin_operand(bp[ss]);
      pin_operand(bds[ss]);
      pin_operand(bds2[ss]);
      pin_operand(bw[ss]);
    };
    if (more) {
      chains(Y, nxt, [&](int kk) ATTN_INLINE {
#pragma unroll
        for (int e = 0; e < EPK; ++e) elem_one(X, kk * EPK + e);
        if ((kk + 1) * EPK == 8) pack(0);
        if ((kk + 1) * EPK == 16) pack(1);
      });
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) elem_one(X, r);
      pack(0);
      pack(1);
    }
    mma_operand_guard();
    const int k1 = more ? tile_at(j + 1) * BKV : 0;
    const bool m1 = masked_at(k1);
    prods(cur, bp, bds, bds2, bw, [&](int i) ATTN_INLINE {
      if (more) {
#pragma unroll
        for (int e = 0; e < EPG; ++e) exp_one(Y, i * EPG + e, k1, m1);
      }
    });
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(A, B, j);
    if (j + 1 < ntiles) step(B, A, j + 1);
  }

  mma_acc_drain(acc);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    store_acc_transposed<bf16>(acc[0][mt], hQ + base, rs, qw, mt * 32, N, d, scale, lane);
    store_acc_transposed<bf16>(acc[1][mt], hdO + base, rs, qw, mt * 32, N, d, 1.f, lane);
  }
}

template <int D, bool C>
static hipError_t q2_pipe_run(const BobArgs& a, hipStream_t stream) {
  const dim3 gq((a.N + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((bob_q2_pipe_kernel<D, C>), gq, dim3(256), 0, stream,
                     static_cast<const bf16*>(a.Q), static_cast<const bf16*>(a.K),
                     static_cast<const bf16*>(a.V), static_cast<const bf16*>(a.dO),
                     static_cast<const bf16*>(a.gQ), static_cast<const bf16*>(a.gK),
                     static_cast<const bf16*>(a.gV), a.ws, static_cast<bf16*>(a.hQ),
                     static_cast<bf16*>(a.hdO), a.H, a.N, a.d, a.scale * kLog2e, a.scale,
                     a.mask, a.mask_heads);
  return hipGetLastError();
}

bool bob_q2_pipe_serves(const BobArgs& a) { return a.dtype == 1 && (a.d == 64 || a.d == 128); }

hipError_t launch_bob_q2_pipe(const BobArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? q2_pipe_run<64, true>(a, stream) : q2_pipe_run<64, false>(a, stream);
  return a.causal ? q2_pipe_run<128, true>(a, stream) : q2_pipe_run<128, false>(a, stream);
}

}  // namespace attn
