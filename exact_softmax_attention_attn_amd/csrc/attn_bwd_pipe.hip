// Software-pipelined bf16 backward kernels (dK/dV and dQ) for gfx950.
//
// Same method as the generic kernels (scores rebuilt per tile from Q, K and
// the saved row scalar, ddx issue #243 item 2; dS = P o (dP - D) with no
// row-max term, issue #243 item 1; PR #162's plan p = w/z then p @ v), shaped
// for one wave per SIMD:
//  - the long-lived operands (K, V or Q, dO of the wave's rows) and the
//    accumulators stay in AGPRs for the whole kernel; products that the VALU
//    reads next (S, dP) land in VGPRs;
//  - the streamed tile operands are read from LDS a few fragments ahead of the
//    product that consumes them, in a fixed order held by scheduling fences;
//  - the scores are scaled in float32 (one FMA with the row's -L log2 e per
//    score, ahead of its exp2), so they are the forward's to float32
//    rounding; -D is added by the matrix cores, so dS = P o (dP - D) is one
//    multiply per score;
//  - streamed tiles are copied global->LDS two steps ahead into a ring of
//    three separately named buffers, with direct-to-LDS copies that the
//    compiler does not track and explicit waits before each hand-off.
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
// owns key rows kv0 + [0, 32).  Its K and V rows sit in AGPRs as the B
// operands of S = Q K^T and dP = dO V^T (column n = key row), so the results
// hold query rows along the registers and the row scalars -L log2e and -D are
// per register: -D enters as the MFMA's C input, read from LDS straight into
// the accumulator registers, and -L2 is the addend of one FMA per element, so
//   P = exp2(c S - L2)  (c = scale log2 e, in float32: the forward's scores
//   to float32 rounding),   dP' = dO V^T - D,   dS = P o dP'.
// dV^T += dO^T P and dK^T += Q^T dS accumulate in AGPRs (asm MFMA).  The
// operand reads (Q, dO along the head dim; dO, Q across positions) run AH
// fragments ahead through a whole 64-row query tile.  Causal: only the two
// tiles on the diagonal carry the element mask.  SPARSE: the walk visits only
// the query tiles whose mask block (row of the tile, column of this key
// block) is kept.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ nL2, const float* __restrict__ nD,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int H, int N, int d, float scale_log2,
    float scale, const unsigned char* __restrict__ mask, int mask_heads, int pair_cus) {
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
  __shared__ Buf buf0, buf1, buf2, buf3;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  // (head dim 64: two workgroups per CU)
  const BlockOrder bo = block_order_paired(D == 64 ? pair_cus : 0);
  const int jb = bo.rank, head = bo.head, b = bo.b;   // rank 0 = longest walk
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const float* Lh = nL2 + ((long)b * H + head) * N;
  const float* Dh = nD + ((long)b * H + head) * N;

  const int kvb = jb * BKV;
  const int kv0 = kvb + wave * 32;
  const int kv = kv0 + l32;
  const LanePlan<D> plan(lane);
  using FS = AsyncFillShape<BQ, D>;
  unsigned copy_off[FS::PER];
  async_fill_plan<BQ, D>(copy_off, rs, wave, lane);
  // The block's K and V rows go to LDS first, by whole-row copies (buf2 holds
  // rows 0..63, buf3 rows 64..127; K in the q slot, V in the o slot; the
  // sequence's ragged last block by the register path with zero rows).  They
  // fly while the visit list is built and the walk's first two tiles are
  // requested, and each wave then reads its 32 rows into registers.
  if (kvb + BKV <= N) {
    async_fill_untracked<BQ, D>(QT{buf2.q}, K + base + kvb * rs, copy_off, wave);
    async_fill_untracked<BQ, D>(QT{buf2.o}, V + base + kvb * rs, copy_off, wave);
    async_fill_untracked<BQ, D>(QT{buf3.q}, K + base + (kvb + BQ) * rs, copy_off, wave);
    async_fill_untracked<BQ, D>(QT{buf3.o}, V + base + (kvb + BQ) * rs, copy_off, wave);
  } else {
    fill_sync(QT{buf2.q}, K + base, rs, kvb, N, d, tid);
    fill_sync(QT{buf2.o}, V + base, rs, kvb, N, d, tid);
    fill_sync(QT{buf3.q}, K + base, rs, kvb + BQ, N, d, tid);
    fill_sync(QT{buf3.o}, V + base, rs, kvb + BQ, N, d, tid);
  }
  frag kf[KS], vf[KS];                          // read from LDS before the walk
  f32x16 dv_acc[MT], dk_acc[MT];

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kvb / BQ : 0;
  int ntiles = nqt - qt0;
  // block-sparse: the kept query tiles, last first (this key block is mask
  // column jb, a query tile of 64 rows lies in one mask row)
  __shared__ unsigned short vis[SPARSE ? kMaxVisit : 1];
  __shared__ int nvis;
  if constexpr (SPARSE) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mk = head_mask(mask, mask_heads, b, head, H, nb);
    ntiles = build_visits(vis, &nvis, ntiles, [&](int i) ATTN_INLINE -> unsigned {
      const int t = nqt - 1 - i;
      return mk[(t * BQ / kMaskBlock) * nb + jb] ? (1u << 14) | (unsigned)t : 0u;
    });
  }

  // A query tile (Q, dO rows and their two row scalars) into LDS.  Whole
  // tiles go by direct global->LDS copies: 2 * PER instructions per wave,
  // plus one for the row scalars on waves 0 and 1.  The walk's first tile may
  // be the sequence's ragged last one: register path with zero padding.
  auto fill_whole = [&](Buf& B, int t) ATTN_INLINE {
    const int q0 = t * BQ;
    async_fill_untracked<BQ, D>(QT{B.q}, Q + base + q0 * rs, copy_off, wave);
    async_fill_untracked<BQ, D>(QT{B.o}, dO + base + q0 * rs, copy_off, wave);
    if (wave == 0) fill_row64_untracked(B.l, Lh + q0, lane);
    if (wave == 1) fill_row64_untracked(B.dd, Dh + q0, lane);
  };
  auto fill = [&](Buf& B, int t) ATTN_INLINE {
    const int q0 = t * BQ;
    if (q0 + BQ <= N) {
      fill_whole(B, t);
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

  // One step = one query tile t, sub-tiles a (rows 0..31) and b (32..63),
  // plus the dV / dK products of the previous tile's sub-tile b ("p"), whose
  // P and dS arrive packed in bpp / bdsp.  Chains of L = D / 16 products:
  //   dV_p | S_a | dK_p | dP_a | S_b | dV_a | dP_b | dK_a
  // Each VALU stage reads a chain that finished at least one chain earlier:
  // the exps of S_a run beside dK_p and dP_a, dS_a beside S_b, the exps of
  // S_b beside dV_a and dP_b, dS_b beside dK_a; P_b and dS_b leave packed for
  // the next step.  The row scalars (-L2 for the exps, -D as dP's C input)
  // are read from LDS one chain ahead, and operand reads run AH fragments ahead
  // through the step, so no chain starts on a fresh LDS read.
  constexpr int L = KS;                       // = 2 * MT
  static_assert(L == 2 * MT, "chain length");
  auto row_scalars = [&](const float* src, int r0) ATTN_INLINE {
    f32x16 v;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = lds_f32x4(&src[r0 + 8 * g + 4 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * g + i] = x[i];
    }
    return v;
  };
  // P from a raw score and its row's -L2
  auto pexp = [&](float sraw, float nl2) ATTN_INLINE {
    return fast_exp2(__builtin_fmaf(sraw, scale_log2, nl2));
  };
  auto mask_rows = [&](f32x16& p, int qa) ATTN_INLINE {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kv > qa + acc_row(r, h)) p[r] = 0.f;
  };
  // Copy slot j of a tile two steps ahead (issued during this step, into the
  // buffer freed by this step's barrier): j < PER Q, then dO, then the row
  // scalars (waves 0 and 1).  Spreading the slots over the step's chains
  // keeps the four waves from queueing their copies all at once.
  constexpr int NSLOT = 2 * FS::PER + 1;
  auto copy_slot = [&](Buf& A, int q0, int j) ATTN_INLINE {
    if (j < FS::PER) {
      async_fill_one_untracked<BQ, D>(QT{A.q}, Q + base + q0 * rs, copy_off, wave, j);
    } else if (j < 2 * FS::PER) {
      async_fill_one_untracked<BQ, D>(QT{A.o}, dO + base + q0 * rs, copy_off, wave, j - FS::PER);
    } else {
      if (wave == 0) fill_row64_untracked(A.l, Lh + q0, lane);
      if (wave == 1) fill_row64_untracked(A.dd, Dh + q0, lane);
    }
  };
  auto step_body = [&](auto has_prev, int t, const Buf& B, const Buf& Pv, bool masked,
                       frag (&bpp)[2], frag (&bdsp)[2], frag (&ring)[AH], auto&& copy) ATTN_INLINE {
    constexpr bool HP = decltype(has_prev)::value;
    // chain positions in the step (-1: chain absent in the walk's first step)
    constexpr int C_DVP = HP ? 0 : -1, C_SA = HP ? 1 : 0, C_DKP = HP ? 2 : -1, C_DPA = HP ? 3 : 1,
                  C_SB = HP ? 4 : 2, C_DVA = HP ? 5 : 3, C_DPB = HP ? 6 : 4, C_DKA = HP ? 7 : 5;
    constexpr int NCH = HP ? 8 : 6;
    constexpr int NOPS = NCH * L;
    // copy slot i * NCH + c goes out after product i of chain c
    auto slot = [&](int c, int i) ATTN_INLINE {
      if (i * NCH + c < NSLOT) copy(i * NCH + c);
    };
    auto opnd = [&](int n) ATTN_INLINE -> frag {
      const int c = n / L, i = n % L;
      if (c == C_SA) return plan.cols(B.q, 0, i);
      if (c == C_DPA) return plan.cols(B.o, 0, i);
      if (c == C_SB) return plan.cols(B.q, 32, i);
      if (c == C_DPB) return plan.cols(B.o, 32, i);
      if (c == C_DVA) return plan.rows(B.o, 0, i / MT, i % MT);
      if (c == C_DKA) return plan.rows(B.q, 0, i / MT, i % MT);
      if (c == C_DKP) return plan.rows(Pv.q, 32, i / MT, i % MT);
      if (c == C_DVP) return plan.rows(Pv.o, 32, i / MT, i % MT);
      // past the step: the next step's dV_p reads this tile's sub-tile b
      return plan.rows(B.o, 32, i / MT, i % MT);
    };
    // The ring arrives holding this step's first AH operands (the previous
    // step read them ahead) except in the walk's first step.
    if constexpr (!HP) {
#pragma unroll
      for (int n = 0; n < AH; ++n) ring[n] = opnd(n);
    }
    // take operand n, issue its product, then refill the slot: the read of
    // the next operand goes out after the product, not before it; the last
    // refills fetch the next step's first operands
    auto refill = [&](int n) ATTN_INLINE { ring[n % AH] = opnd(n + AH); };
    const int qa = t * BQ;                       // first query row of the tile
    constexpr int E = 8 / L;                     // exps per product (half a sub-tile per chain)
    constexpr int M2 = 16 / L;                   // dS multiplies per product
    // before product n of an even position, wait for operands n and n + 1
    auto pair_wait = [&](int n) ATTN_INLINE {
      if (n % 2 == 0) need_both(ring[n % AH], ring[(n + 1) % AH]);
    };
    auto s_chain = [&](int c, f32x16& acc) ATTN_INLINE {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        pair_wait(c * L + i);
        acc = M::mma(ring[(c * L + i) % AH], kf[i], acc);
        refill(c * L + i);
        slot(c, i);
        fence();
      }
    };
    const f32x16 la = row_scalars(B.l, 0);       // -L2 of S_a's rows, read during dV_p
    f32x16 sa = zero16();
    fence();
    // dV_p
    if constexpr (HP) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        pair_wait(C_DVP * L + i);
        mma_acc_agpr(dv_acc[i % MT], ring[(C_DVP * L + i) % AH], bpp[i / MT]);
        refill(C_DVP * L + i);
        slot(C_DVP, i);
        fence();
      }
    }
    // S_a
    s_chain(C_SA, sa);
    // dK_p | exps of S_a, first half
    f32x16 pa = row_scalars(B.dd, 0);            // dP_a's C input
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if constexpr (HP) {
        pair_wait(C_DKP * L + i);
        mma_acc_agpr(dk_acc[i % MT], ring[(C_DKP * L + i) % AH], bdsp[i / MT]);
        refill(C_DKP * L + i);
        slot(C_DKP, i);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) sa[i * E + e] = pexp(sa[i * E + e], la[i * E + e]);
      fence();
    }
    // dP_a | exps of S_a, second half
    const f32x16 lb = row_scalars(B.l, 32);      // -L2 of S_b's rows
#pragma unroll
    for (int i = 0; i < L; ++i) {
      pair_wait(C_DPA * L + i);
      pa = M::mma(ring[(C_DPA * L + i) % AH], vf[i], pa);
      refill(C_DPA * L + i);
      slot(C_DPA, i);
#pragma unroll
      for (int e = 0; e < E; ++e) sa[8 + i * E + e] = pexp(sa[8 + i * E + e], la[8 + i * E + e]);
      fence();
    }
    if (CAUSAL && masked) mask_rows(sa, qa);
    frag bpa[2] = {M::pack(sa, 0), M::pack(sa, 1)};
    pin_operand(bpa[0]);
    pin_operand(bpa[1]);
    fence();
    // S_b | dS_a = P_a o dP'_a
    f32x16 sb = zero16();
#pragma unroll
    for (int i = 0; i < L; ++i) {
      pair_wait(C_SB * L + i);
      sb = M::mma(ring[(C_SB * L + i) % AH], kf[i], sb);
      refill(C_SB * L + i);
      slot(C_SB, i);
#pragma unroll
      for (int e = 0; e < M2; ++e) pa[i * M2 + e] = sa[i * M2 + e] * pa[i * M2 + e];
      fence();
    }
    frag bdsa[2] = {M::pack(pa, 0), M::pack(pa, 1)};
    pin_operand(bdsa[0]);
    pin_operand(bdsa[1]);
    f32x16 pb = row_scalars(B.dd, 32);           // dP_b's C input
    fence();
    // dV_a | exps of S_b, first half
#pragma unroll
    for (int i = 0; i < L; ++i) {
      pair_wait(C_DVA * L + i);
      mma_acc_agpr(dv_acc[i % MT], ring[(C_DVA * L + i) % AH], bpa[i / MT]);
      refill(C_DVA * L + i);
      slot(C_DVA, i);
#pragma unroll
      for (int e = 0; e < E; ++e) sb[i * E + e] = pexp(sb[i * E + e], lb[i * E + e]);
      fence();
    }
    // dP_b | exps of S_b, second half
#pragma unroll
    for (int i = 0; i < L; ++i) {
      pair_wait(C_DPB * L + i);
      pb = M::mma(ring[(C_DPB * L + i) % AH], vf[i], pb);
      refill(C_DPB * L + i);
      slot(C_DPB, i);
#pragma unroll
      for (int e = 0; e < E; ++e) sb[8 + i * E + e] = pexp(sb[8 + i * E + e], lb[8 + i * E + e]);
      fence();
    }
    if (CAUSAL && masked) mask_rows(sb, qa + 32);
    bpp[0] = M::pack(sb, 0);
    bpp[1] = M::pack(sb, 1);
    pin_operand(bpp[0]);
    pin_operand(bpp[1]);
    fence();
    // dK_a | dS_b = P_b o dP'_b
#pragma unroll
    for (int i = 0; i < L; ++i) {
      pair_wait(C_DKA * L + i);
      mma_acc_agpr(dk_acc[i % MT], ring[(C_DKA * L + i) % AH], bdsa[i / MT]);
      refill(C_DKA * L + i);
      slot(C_DKA, i);
#pragma unroll
      for (int e = 0; e < M2; ++e) {
        float x = sb[i * M2 + e] * pb[i * M2 + e];
        asm volatile("" : "+v"(x));             // here, not bunched before the packs
        pb[i * M2 + e] = x;
      }
      fence();
    }
    bdsp[0] = M::pack(pb, 0);
    bdsp[1] = M::pack(pb, 1);
    pin_operand(bdsp[0]);
    pin_operand(bdsp[1]);
    fence();
  };
  // dV / dK of the last step's sub-tile b, once the walk is over
  auto flush = [&](const Buf& Pv, const frag (&bpp)[2], const frag (&bdsp)[2]) ATTN_INLINE {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      mma_acc_agpr(dv_acc[i % MT], plan.rows(Pv.o, 32, i / MT, i % MT), bpp[i / MT]);
      fence();
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      mma_acc_agpr(dk_acc[i % MT], plan.rows(Pv.q, 32, i / MT, i % MT), bdsp[i / MT]);
      fence();
    }
  };

  // Walk the query tiles from the last one back to the diagonal: every block
  // of a head starts on the same tiles at the same time, so they are shared
  // in L2 instead of each block streaming its own stretch.  Step k visits
  // tile tile_of(k) (nqt - 1 - k, or entry k of the visit list); causal: the
  // diagonal tiles (BKV = 2 BQ), the walk's last two steps when they are
  // visited, apply the element mask.  Tiles are copied two steps ahead
  // into a ring of four separately named buffers picked statically (the loop
  // is unrolled by four): a step reads its own tile and the previous one, and
  // a copy has two steps to land, so step k waits only for tile k's copy,
  // leaving tile k + 1's in flight.  A runtime choice between buffers would
  // make the compiler shuffle the accumulators between registers while
  // products are in flight.
  auto tile_of = [&](int k) ATTN_INLINE -> int {
    if constexpr (SPARSE) return wave_uniform(vis[k] & kVisitTile);
    else return nqt - 1 - k;
  };
  frag bpp[2], bdsp[2], ring[AH];
  auto step = [&](auto has_prev, int k, const Buf& cur, const Buf& prv, Buf& ahead) ATTN_INLINE {
    if (k + 1 < ntiles) wait_async_fills_but<2 * FS::PER>();   // tile k + 1's copy may fly
    else wait_async_fills();
    lds_barrier();
    const bool ahead_on = k + 2 < ntiles;
    const int qn = ahead_on ? tile_of(k + 2) * BQ : 0;
    const int t = tile_of(k);
    const bool masked = CAUSAL && (SPARSE ? t * BQ < kvb + BKV : k + 2 >= ntiles);
    step_body(has_prev, t, cur, prv, masked, bpp, bdsp, ring,
              [&](int j) ATTN_INLINE { if (ahead_on) copy_slot(ahead, qn, j); });
  };
  // Steps at least two ahead of the last are unmasked and have two tiles
  // after them: the main loop takes four of them at a time without a
  // branch, which keeps each step one straight block.
  auto step_inner = [&](int k, const Buf& cur, const Buf& prv, Buf& ahead) ATTN_INLINE {
    wait_async_fills_but<2 * FS::PER>();
    lds_barrier();
    const int qn = tile_of(k + 2) * BQ;
    step_body(bool_c<true>{}, tile_of(k), cur, prv, false, bpp, bdsp, ring,
              [&](int j) ATTN_INLINE { copy_slot(ahead, qn, j); });
  };
  if (ntiles > 0) {                             // a sparse walk may visit nothing
    fill(buf0, tile_of(0));
    if (ntiles > 1) fill_whole(buf1, tile_of(1));
  }
  // K and V have landed once at most the 2 PER copies of a tile issued after
  // them are in flight (a ragged first tile went by the register path, whose
  // loads were waited for in order after them); every wave's copies, then
  // the reads
  if (ntiles > 0) wait_async_fills_but<2 * FS::PER>();
  else wait_async_fills();
  lds_barrier();
  {
    const Buf& kvt = wave < 2 ? buf2 : buf3;
    const int r0 = (wave & 1) * 32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = plan.cols(kvt.q, r0, ks);
      vf[ks] = plan.cols(kvt.o, r0, ks);
      pin_agpr(kf[ks]);
      pin_agpr(vf[ks]);
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    dv_acc[i] = zero16(); pin_agpr(dv_acc[i]);
    dk_acc[i] = zero16(); pin_agpr(dk_acc[i]);
  }

  if (ntiles > 0) {
    // the first step's barrier also frees buf2 (its copies of tile 2 land
    // there) from the K, V reads above
    step(bool_c<false>{}, 0, buf0, buf3, buf2);
    int k = 1;
    for (; k + 6 <= ntiles; k += 4) {
      step_inner(k, buf1, buf0, buf3);
      step_inner(k + 1, buf2, buf1, buf0);
      step_inner(k + 2, buf3, buf2, buf1);
      step_inner(k + 3, buf0, buf3, buf2);
    }
    if (k < ntiles) step(bool_c<true>{}, k, buf1, buf0, buf3);
    if (k + 1 < ntiles) step(bool_c<true>{}, k + 1, buf2, buf1, buf0);
    if (k + 2 < ntiles) step(bool_c<true>{}, k + 2, buf3, buf2, buf1);
    if (k + 3 < ntiles) step(bool_c<true>{}, k + 3, buf0, buf3, buf2);
    if (k + 4 < ntiles) step(bool_c<true>{}, k + 4, buf1, buf0, buf3);
    const int last = (ntiles - 1) & 3;         // buffer of the last step
    const Buf& lb = last == 0 ? buf0 : last == 1 ? buf1 : last == 2 ? buf2 : buf3;
    flush(lb, bpp, bdsp);
  }

  mma_acc_drain(dv_acc);
#pragma unroll
  for (int i = 0; i < MT; ++i) asm volatile("" : "+a"(dk_acc[i]));
  // every wave is done with the ring: rows out through buf0 (waves 0, 1) and
  // buf1 (waves 2, 3), whole rows per store
  static_assert(2 * RowStage<D>::BYTES <= sizeof(Buf), "staging area");
  lds_barrier();
  bf16* stage = reinterpret_cast<bf16*>(wave < 2 ? &buf0 : &buf1) + (wave & 1) * (RowStage<D>::BYTES / 2);
  store_rows_via_lds<D>(dv_acc, dV + base, rs, kv0, N, 1.f, stage, lane);
  store_rows_via_lds<D>(dk_acc, dK + base, rs, kv0, N, scale, stage, lane);
}

// ---------------------------------------------------------------------------
// dQ (bf16).  Workgroup = NW waves = 256 query rows of one (b, h); wave w owns
// query rows qw + [0, WQ) as two halves of 32 rows.  Q and dO of the wave's
// rows and its dQ^T accumulators live in AGPRs for the whole kernel.  With two
// halves each LDS operand fragment feeds two matrix instructions.  Per key
// sub-tile of 32 rows:
//   S^T = K Q^T,  dP'^T = V dO^T - D,  P = exp2(c S - L2)  (c = scale log2 e),
//   dS = P o dP',  dQ^T += K^T dS^T.
// The scores are scaled in float32 (one FMA with the lane's -L2 per element,
// the query rows run along the lanes), so they are the forward's scores to
// float32 rounding.  -D enters as the C input of each dP chain's first
// product: every register of a lane belongs to the lane's query, so a tile
// holding the lane's -D in all 16 registers (fixed for the whole walk) adds
// it to every element, in float32.  The two halves' chains run
// one after the other, so each VALU stage sits beside a chain it does not feed.
// Key tiles are copied two steps ahead into a ring of three separately named
// LDS buffers.  No atomics.
//
// FUSE: the kernel also does the preprocess for its own rows -- D = rowsum(dO
// o O) with the preprocess kernel's lanes and summation order (so the same
// bits), and -L log2 e from the forward's L -- and writes both to the
// workspace (ws: -D [B, H, N], then -L log2 e), where the dK/dV kernel that
// runs after it reads them.  nL2 and nD are then unused; otherwise O, L and
// ws are.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int WQ, int NW, bool SPARSE, bool FUSE>
__global__ __launch_bounds__(NW * 64, WQ == 32 ? 2 : 1) void bwd_dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ nL2, const float* __restrict__ nD,
    bf16* __restrict__ dQ, int H, int N, int d, float scale_log2, float scale,
    const unsigned char* __restrict__ mask, int mask_heads, const bf16* __restrict__ O,
    const float* __restrict__ L, float* __restrict__ ws, int pair_cus) {
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int NH = WQ / 32;                  // 32-row halves per wave
  constexpr int BQ = NW * WQ, BKV = 64, KS = D / 16, MT = D / 32;
  constexpr int NT = NW * 64;
  using KT = Tile<bf16, BKV, D>;
  struct __align__(16) Buf {
    bf16 k[KT::ELEMS];
    bf16 v[KT::ELEMS];
  };
  __shared__ Buf buf0, buf1, buf2;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int nqb = gridDim.x;
  const BlockOrder bo = block_order_paired(NH == 1 ? pair_cus : 0);
  const int ib = CAUSAL ? (nqb - 1 - bo.rank) : bo.rank;   // longest first
  const int head = bo.head, b = bo.b;
  const long rs = (long)H * d;
  const long base = ((long)b * N * H + head) * d;
  const long rbase = ((long)b * H + head) * N;        // the (b, h) slice of [B, H, N]
  const float* Lh = FUSE ? L + rbase : nL2 + rbase;   // L (FUSE) or -L * log2(e)
  const float* Dh = nD + rbase;                       // -D (unless FUSE)

  const int qb = ib * BQ;
  const int qw = qb + wave * WQ;               // this wave's first query row
  LanePlan<D> plan(lane);
  frag qf[NH][KS], of[NH][KS];
  // -D of the lane's query in every register, per half: the C input of each
  // dP chain's first product
  f32x16 ndt[NH];
  float nl2[NH];                               // -L log2 e of the lane's query, per half

  f32x16 acc[NH][MT];
#pragma unroll
  for (int c = 0; c < NH; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      acc[c][i] = zero16();
      if constexpr (NH == 2) pin_agpr(acc[c][i]);
    }

  using FS = AsyncFillShape<BKV, D, NW>;
  unsigned copy_off[FS::PER];
  async_fill_plan<BKV, D, NW>(copy_off, rs, wave, lane);
  // 64 of the block's own rows (of Q or dO, from row r0) into an LDS tile:
  // direct copies (PER instructions per wave), or, for the sequence's ragged
  // end, the register path with zero rows
  auto fill_rows = [&](bf16* t, const bf16* src, int r0) ATTN_INLINE {
    if (r0 + BKV <= N) async_fill_untracked<BKV, D, NW>(KT{t}, src + base + r0 * rs, copy_off, wave);
    else fill_sync<bf16, BKV, D, NT>(KT{t}, src + base, rs, r0, N, d, tid);
  };
  // The block's Q and dO rows reach the waves' registers through LDS, by
  // whole-row copies (a lane loading its own row would touch 32 rows per
  // instruction), in two rounds since the three tile buffers hold 384 rows:
  // first Q (buf0, buf1) and dO rows 0..127 (buf2), then dO rows 128..255
  // (buf2) beside the walk's first two key tiles (buf0, buf1).  Each buffer
  // holds 128 rows as its k and v tiles; wave w's 64 rows are tile w % 2 of
  // buffer w / 2 (Q) and of buf2 (dO, round w / 2 + 1).
  // One-half form (WQ = 32, 128 rows per block): Q in buf0 and dO in buf1,
  // one round; wave w's 32 rows are rows 32 (w % 2) of tile w / 2.
  static_assert(NW == 4 && (WQ == BKV || WQ == 32), "wave rows per buffer");
  if constexpr (NH == 2) {
    fill_rows(buf0.k, Q, qb);
    fill_rows(buf0.v, Q, qb + 64);
    fill_rows(buf1.k, Q, qb + 128);
    fill_rows(buf1.v, Q, qb + 192);
    fill_rows(buf2.k, dO, qb);
    fill_rows(buf2.v, dO, qb + 64);
  } else {
    fill_rows(buf0.k, Q, qb);
    fill_rows(buf0.v, Q, qb + 64);
    fill_rows(buf1.k, dO, qb);
    fill_rows(buf1.v, dO, qb + 64);
  }
  // -L log2 e as the preprocess forms it (a row with no kept key, L = -inf,
  // gives -inf, so every P of it is 0)
  auto neg_l2 = [](float l) ATTN_INLINE -> float {
    return l == -__builtin_inff() ? -__builtin_inff() : -l * kLog2e;
  };
  // FUSE: -D and -L log2 e of the block's rows, kept here until the end,
  // where they go to the workspace as two whole-block stores
  __shared__ float sD[FUSE ? BQ : 1], sL2[FUSE ? BQ : 1];
  // The preprocess for rows qb .. qb + BQ - 1: 16 lanes per row, 16 rows per
  // pass.  Every pass's loads go out here, from clamped (in-bounds) addresses,
  // beside the round-1 copies (and a block mask's reads below); the sums are
  // formed once the visit list is built.  Lanes past the row or the head dim
  // count 0.
  static_assert(!FUSE || (NT == 256 && BQ % 16 == 0), "16 rows of 16 lanes per pass");
  // (d = D <= 128: the preprocess's column loop is one chunk per lane)
  static_assert(!FUSE || D <= 16 * 8, "one 8-column chunk per lane");
  constexpr int NP = FUSE ? BQ / 16 : 1;
  const int pl = tid & 15;                     // the lane's 8-column chunk of its row
  bf16x8 xo[NP], xg[NP];
  float lr[NP];
  if constexpr (FUSE) {
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
      const int n = min(qb + pass * 16 + (tid >> 4), N - 1);
      const long at = base + (long)n * rs + min(pl * 8, D - 8);
      xo[pass] = *reinterpret_cast<const bf16x8*>(O + at);
      xg[pass] = *reinterpret_cast<const bf16x8*>(dO + at);
      lr[pass] = Lh[n];
    }
  }
  float dq[NH];
#pragma unroll
  for (int c = 0; c < NH; ++c) {
    const int q = qw + 32 * c + l32;
    // padded rows (q >= N) and rows with no kept key (stored -inf): P = 0
    if constexpr (FUSE) nl2[c] = q < N ? neg_l2(Lh[q]) : -__builtin_inff();
    else nl2[c] = q < N ? Lh[q] : -__builtin_inff();
    dq[c] = (!FUSE && q < N) ? Dh[q] : 0.f;    // FUSE: from sD once it is published
  }

  const int kv_end = CAUSAL ? min(N, qb + BQ) : N;
  const int ntiles_all = (kv_end + BKV - 1) / BKV;
  // first tile holding key rows above some of the block's query rows
  const int diag0 = CAUSAL ? max(0, min(ntiles_all, qb / BKV)) : ntiles_all;
  // block-sparse: the key tiles kept by either mask row of the block's query
  // rows (rows qb .. qb + 255 span mask rows r0 and r0 + 1), in order; a wave
  // (64 rows, one mask row) zeroes P on the tiles its own row drops.
  __shared__ unsigned short vis[SPARSE ? kMaxVisit : 1];
  __shared__ int nvis;
  static_assert(!SPARSE || ((BQ == 2 * kMaskBlock || BQ == kMaskBlock) && WQ * 2 <= kMaskBlock),
                "mask rows per block and per wave");
  const int nb = (N + kMaskBlock - 1) / kMaskBlock;
  const int ntiles = !SPARSE ? ntiles_all : build_visits(vis, &nvis, ntiles_all,
      [&](int t) ATTN_INLINE -> unsigned {
        const unsigned char* mk = head_mask(mask, mask_heads, b, head, H, nb);
        const int r0 = qb / kMaskBlock, c = t * BKV / kMaskBlock;
        const unsigned code = (mk[r0 * nb + c] ? 1u : 0u) |
                              (BQ > kMaskBlock && r0 + 1 < nb && mk[(r0 + 1) * nb + c] ? 2u : 0u);
        return code ? (code << 14) | (unsigned)t : 0u;
      });
  if constexpr (FUSE) {
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
      const int rl = pass * 16 + (tid >> 4), n = qb + rl;
      float acc = dot8_bf16(xo[pass], xg[pass], 0.f);
      if (!(n < N && pl * 8 < D)) acc = 0.f;
      acc = sum16_lanes(acc);
      if (pl == 0) {
        sD[rl] = n < N ? -acc : 0.f;
        sL2[rl] = neg_l2(lr[pass]);
      }
    }
  }
  // walk positions below inner_end need no checks (unmasked, next two tiles
  // whole); a sparse walk takes every step through the checked form (one loop
  // keeps the register assignment the same all along the walk)
  const int inner_end = !SPARSE ? min(diag0, min(ntiles - 2, N / BKV - 2)) : 0;
  // tile index at walk position p, and whether this wave's mask row drops it
  auto tile_at = [&](int p) ATTN_INLINE -> int {
    if constexpr (SPARSE) return (int)(visit_entry(vis, p) & kVisitTile);
    else return p;
  };
  auto kill_at = [&](int p) ATTN_INLINE -> bool {
    if constexpr (SPARSE) return ((visit_entry(vis, p) >> (14 + wave * WQ / kMaskBlock)) & 1u) == 0u;
    else return false;
  };

  // A key tile (K and V rows) into LDS: whole tiles by direct copies (2 * PER
  // instructions per wave), the sequence's ragged last tile by the register
  // path with zero padding.
  auto fill = [&](Buf& B, int kt) ATTN_INLINE {
    const int k0 = kt * BKV;
    if (k0 + BKV <= N) {
      async_fill_untracked<BKV, D, NW>(KT{B.k}, K + base + k0 * rs, copy_off, wave);
      async_fill_untracked<BKV, D, NW>(KT{B.v}, V + base + k0 * rs, copy_off, wave);
    } else {
      fill_sync<bf16, BKV, D, NT>(KT{B.k}, K + base, rs, k0, N, d, tid);
      fill_sync<bf16, BKV, D, NT>(KT{B.v}, V + base, rs, k0, N, d, tid);
    }
  };

  // Operands of the 32 key rows at r0 of a tile: K along the head dim (S, in
  // kf), V along the head dim (dP, in vf), K across positions (dQ, in tf).
  // Per sub-tile the products run in chains (each dP chain starts from the
  // -D tile):
  //   S_0 | S_1 | dP_0 | dP_1 | dQ_0 | dQ_1        (index = query half)
  // and every VALU stage reads a chain that finished at least one product
  // earlier: exps of S_0 beside S_1, exps of S_1 beside dP_0, dS_0 beside
  // dP_1, dS_1 beside dQ_0.  One operand read feeds the two halves' chains
  // from registers.  V is read during S_1 and dP_0, K^T during dP_1 and dQ_0 (each
  // half a chain ahead of its use, which keeps few fragments live), and the
  // next sub-tile's K during dQ_1, which runs after the next step's barrier
  // for a tile's last sub-tile, so a tile starts on operands already read.
  // The copies of the tile two steps ahead go out during the S_0 chains.
  constexpr int NSLOT = 2 * FS::PER, SPS = NSLOT / 2;     // copy slots per tile, per sub-tile
  static_assert(KS % SPS == 0, "copy slots per sub-tile");
  static_assert(KS == 2 * MT, "one K fragment read per dQ_1 product");
  auto copy_slot = [&](Buf& A, int k0, int j) ATTN_INLINE {
    if (j < FS::PER) async_fill_one_untracked<BKV, D, NW>(KT{A.k}, K + base + k0 * rs, copy_off, wave, j);
    else async_fill_one_untracked<BKV, D, NW>(KT{A.v}, V + base + k0 * rs, copy_off, wave, j - FS::PER);
  };
  // (two-half form: kf, vf, tf, bds1; one-half form: kf, vf, tf for the
  // pending sub-tile's K^T, tfn, pp, dpp)
  frag kf[KS], vf[KS], tf[2 * MT], tfn[2 * MT], bds1[2];
  f32x16 pp, dpp;
  // dQ_1 of the pending sub-tile (K^T in tf, dS_1 packed in bds1), reading the
  // K fragments of the sub-tile at r0 of B beside it
  auto dq_half1 = [&](const Buf& B, int r0) ATTN_INLINE {
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      mma_acc_agpr(acc[NH - 1][i % MT], tf[i], bds1[i / MT]);
      kf[i] = plan.cols(B.k, r0, i);
      fence();
    }
  };
  // P = 0 above the diagonal (causal), on the padded keys of the sequence's
  // ragged last tile (whose zero rows give S = 0 and so P = exp(-L), which
  // overflows for L below about -88), or everywhere (the wave's mask row
  // drops the tile)
  auto mask_half = [&](f32x16& s, int c, int ka, bool kill) ATTN_INLINE {
    const int q = qw + 32 * c + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = ka + acc_row(r, h);
      if (kill || (CAUSAL && k > q) || k >= N) s[r] = 0.f;
    }
  };
  // sub-tile st of B (key rows ka ..), K fragments already in kf; leaves
  // dQ_1 pending in tf and bds1
  auto sub = [&](const Buf& B, int st, int ka, bool masked, bool kill, auto&& copy) ATTN_INLINE {
    const int r0 = st * 32;
    constexpr int E = 16 / KS;                  // elements per product in the exp and dS_0 stages
    f32x16 sc[2], pc[2];
    // S_0^T = K Q_0^T
    sc[0] = M::mma(kf[0], qf[0][0], zero16());
    copy(st * SPS);
    fence();
#pragma unroll
    for (int kk = 1; kk < KS; ++kk) {
      sc[0] = M::mma(kf[kk], qf[0][kk], sc[0]);
      if (kk % (KS / SPS) == 0) copy(st * SPS + kk / (KS / SPS));
      fence();
    }
    // S_1 | P_0 = exp2(c S_0 - L2); first half of V read (KS / 2 products ahead)
    sc[1] = zero16();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      sc[1] = M::mma(kf[kk], qf[1][kk], sc[1]);
      if (kk >= KS / 2) vf[kk - KS / 2] = plan.cols(B.v, r0, kk - KS / 2);
#pragma unroll
      for (int e = 0; e < E; ++e)
        sc[0][kk * E + e] = fast_exp2(__builtin_fmaf(sc[0][kk * E + e], scale_log2, nl2[0]));
      fence();
    }
    // (a use here keeps the exps beside the chain; otherwise the compiler
    // bunches some of them next to their first use, with no product beside)
    pin_operand(sc[0]);
    if (masked || kill) mask_half(sc[0], 0, ka, kill);
    // dP'_0 | P_1 = exp2(c S_1 - L2); second half of V read
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      pc[0] = M::mma(vf[kk], of[0][kk], kk == 0 ? ndt[0] : pc[0]);
      if (kk < KS / 2) vf[KS / 2 + kk] = plan.cols(B.v, r0, KS / 2 + kk);
#pragma unroll
      for (int e = 0; e < E; ++e)
        sc[1][kk * E + e] = fast_exp2(__builtin_fmaf(sc[1][kk * E + e], scale_log2, nl2[1]));
      fence();
    }
    pin_operand(sc[1]);
    if (masked || kill) mask_half(sc[1], 1, ka, kill);
    // dP'_1 | dS_0 = P_0 o dP'_0, packed; first half of K^T read
    frag bds0[2];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      pc[1] = M::mma(vf[kk], of[1][kk], kk == 0 ? ndt[1] : pc[1]);
      if (kk >= KS / 2) tf[kk - KS / 2] = plan.rows(B.k, r0, 0, kk - KS / 2);
#pragma unroll
      for (int e = 0; e < E; ++e) pc[0][kk * E + e] = sc[0][kk * E + e] * pc[0][kk * E + e];
      if (kk == KS / 2 - 1) {
        bds0[0] = M::pack(pc[0], 0);
        pin_operand(bds0[0]);
      }
      fence();
    }
    bds0[1] = M::pack(pc[0], 1);                // first read MT products into dQ_0
    pin_operand(bds0[1]);
    fence();
    // dQ_0^T += K^T dS_0^T | dS_1 = P_1 o dP'_1 over products 1 .. 2 MT - 1;
    // second half of K^T read MT products ahead of its use
    constexpr int S3 = 2 * MT - 1;
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      mma_acc_agpr(acc[0][i % MT], tf[i], bds0[i / MT]);
      if (i < MT) tf[MT + i] = plan.rows(B.k, r0, 1, i);
      if (i > 0) {
        const int lo = 16 * (i - 1) / S3, hi = 16 * i / S3;
#pragma unroll
        for (int r = lo; r < hi; ++r) pc[1][r] = sc[1][r] * pc[1][r];
        if (lo < 8 && hi >= 8) {
          bds1[0] = M::pack(pc[1], 0);
          pin_operand(bds1[0]);
        }
      }
      fence();
    }
    bds1[1] = M::pack(pc[1], 1);                // first read MT products into dQ_1
    pin_operand(bds1[1]);
    fence();
  };
  // One-half form (WQ = 32): the wave's 32 query rows are one half, and two
  // workgroups share a CU, so each SIMD runs two waves.  Per sub-tile j the
  // chains run
  //   S_j | dQ_{j-1} | dP_j
  // with dS_{j-1} = P_{j-1} o dP'_{j-1} (multiplies and packs) beside S_j,
  // P_j's exps beside dQ_{j-1} and dP_j, V_j read during S_j, K^T_j during
  // dQ_{j-1} and the tile's second K during dP_j; a tile's first K is read
  // after its barrier.  P_j, dP'_j and K^T_j stay pending (pp, dpp, tf).
  // Everything, the dQ^T accumulators included, lives in VGPRs with builtin
  // products: at two waves per SIMD a wave has 256 registers, and the
  // compiler would split them evenly between VGPRs and AGPRs if any AGPR
  // were pinned.
  auto sub1 = [&](const Buf& B, int st, int ka, bool masked, bool kill, auto&& copy) ATTN_INLINE {
    const int r0 = st * 32;
    constexpr int EM = 16 / KS;                 // dS multiplies per S product
    constexpr int EX = 16 / (2 * MT + KS);      // exps per dQ or dP product
    static_assert(EM * KS == 16 && EX * (2 * MT + KS) == 16 && EM <= 8, "elements per product");
    frag bd[2];
    // S_j^T = K Q^T | dS_{j-1}, packed; V_j read
    f32x16 sc = M::mma(kf[0], qf[0][0], zero16());
    copy(st * SPS);
#pragma unroll
    for (int e = 0; e < EM; ++e) dpp[e] = pp[e] * dpp[e];
    vf[0] = plan.cols(B.v, r0, 0);
    fence();
#pragma unroll
    for (int kk = 1; kk < KS; ++kk) {
      sc = M::mma(kf[kk], qf[0][kk], sc);
      if (kk % (KS / SPS) == 0) copy(st * SPS + kk / (KS / SPS));
#pragma unroll
      for (int e = 0; e < EM; ++e) dpp[kk * EM + e] = pp[kk * EM + e] * dpp[kk * EM + e];
      if (kk * EM + EM == 8) {
        bd[0] = M::pack(dpp, 0);
        pin_operand(bd[0]);
      }
      vf[kk] = plan.cols(B.v, r0, kk);
      fence();
    }
    bd[1] = M::pack(dpp, 1);                    // first read MT products into dQ_{j-1}
    pin_operand(bd[1]);
    fence();
    // dQ_{j-1}^T += K^T dS_{j-1}^T | P_j = exp2(c S_j - L2), first part; K^T_j read
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      acc[0][i % MT] = M::mma(tf[i], bd[i / MT], acc[0][i % MT]);
      tfn[i] = plan.rows(B.k, r0, i / MT, i % MT);
#pragma unroll
      for (int e = 0; e < EX; ++e)
        sc[i * EX + e] = fast_exp2(__builtin_fmaf(sc[i * EX + e], scale_log2, nl2[0]));
      fence();
    }
    pin_operand(sc);                            // keeps these exps beside the chain
    // dP'_j^T = V dO^T - D (the -D tile as C input) | the rest of P_j; the
    // tile's second K read
    f32x16 pc;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      pc = M::mma(vf[kk], of[0][kk], kk == 0 ? ndt[0] : pc);
      if (st == 0) kf[kk] = plan.cols(B.k, 32, kk);
#pragma unroll
      for (int e = 0; e < EX; ++e) {
        const int r = 2 * MT * EX + kk * EX + e;
        float p = fast_exp2(__builtin_fmaf(sc[r], scale_log2, nl2[0]));
        asm volatile("" : "+v"(p));             // here, not bunched at the chain's end
        sc[r] = p;
      }
      fence();
    }
    pin_operand(sc);
    if (masked || kill) mask_half(sc, 0, ka, kill);
    pp = sc;
    dpp = pc;
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) tf[i] = tfn[i];
  };
  // One key tile.  Two-half form: the pending dQ_1 of the previous tile while
  // this tile's first K fragments are read, then both sub-tiles.  One-half
  // form: this tile's first K fragments, then both sub-tiles.  Before the
  // first tile the pending products add zero (dS = 0), which keeps every
  // step alike.
  auto tile_body = [&](int kt, const Buf& B, bool masked, bool kill, auto&& copy) ATTN_INLINE {
    if constexpr (NH == 2) {
      dq_half1(B, 0);
      sub(B, 0, kt * BKV, masked, kill, copy);
      dq_half1(B, 32);
      sub(B, 1, kt * BKV + 32, masked, kill, copy);
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kf[kk] = plan.cols(B.k, 0, kk);
      sub1(B, 0, kt * BKV, masked, kill, copy);
      sub1(B, 1, kt * BKV + 32, masked, kill, copy);
    }
  };

  // Key tiles are copied two steps ahead into a ring of three separately
  // named buffers, picked statically (the loops are unrolled by three): step
  // kt waits only for tile kt's copy and leaves tile kt + 1's in flight
  // (unless that one went by the register path, the ragged last tile, which
  // leaves nothing to count against).  Tiles from diag0 on apply the causal
  // element mask, and a ragged last tile masks its padded keys.  kt is the
  // walk position; tile_at(kt) the tile.
  auto step = [&](int kt, const Buf& cur, Buf& ahead) ATTN_INLINE {
    const int t1 = !SPARSE ? kt + 1 : kt + 1 < ntiles ? tile_at(kt + 1) : 0;
    if (kt + 1 < ntiles && (t1 + 1) * BKV <= N) wait_async_fills_but<2 * FS::PER>();
    else wait_async_fills();
    lds_barrier();
    plan.rebind();
    const int t2 = !SPARSE ? kt + 2 : kt + 2 < ntiles ? tile_at(kt + 2) : 0;
    const int k2 = t2 * BKV;
    const bool spread = kt + 2 < ntiles && k2 + BKV <= N;
    if (kt + 2 < ntiles && !spread) fill(ahead, t2);         // ragged: register path now
    const int t = tile_at(kt);
    tile_body(t, cur, (CAUSAL && t >= diag0) || (t + 1) * BKV > N, kill_at(kt),
              [&](int j) ATTN_INLINE { if (spread) copy_slot(ahead, k2, j); });
  };
  // Steps below the diagonal whose tile two ahead is whole need none of the
  // checks above: the first loop takes three of them at a time without a
  // branch, which keeps each tile body one straight block.
  auto step_inner = [&](int kt, const Buf& cur, Buf& ahead) ATTN_INLINE {
    wait_async_fills_but<2 * FS::PER>();
    lds_barrier();
    plan.rebind();
    const int k2 = tile_at(kt + 2) * BKV;
    tile_body(tile_at(kt), cur, false, kill_at(kt),
              [&](int j) ATTN_INLINE { copy_slot(ahead, k2, j); });
  };
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i) tf[i] = frag{};
  bds1[0] = bds1[1] = frag{};
  pp = zero16();
  dpp = zero16();
  // round 1 landed (every wave's copies): Q for all waves, dO for waves 0, 1
  // (one-half form: dO for all waves) (and, FUSE, every row's -D is in sD)
  wait_async_fills();
  lds_barrier();
  if constexpr (FUSE) {
#pragma unroll
    for (int c = 0; c < NH; ++c) dq[c] = sD[wave * WQ + 32 * c + l32];
  }
  if constexpr (NH == 1) {
    const bf16* qt = wave < 2 ? buf0.k : buf0.v;
    const bf16* ot = wave < 2 ? buf1.k : buf1.v;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      qf[0][kk] = plan.cols(qt, 32 * (wave & 1), kk);
      of[0][kk] = plan.cols(ot, 32 * (wave & 1), kk);
    }
    lds_barrier();                             // buf0, buf1 free again
    if (ntiles > 0) fill(buf0, tile_at(0));     // a sparse walk may visit nothing
    if (ntiles > 1) fill(buf1, tile_at(1));
  } else {
  {
    const Buf& qb_buf = wave < 2 ? buf0 : buf1;
    const bf16* qt = (wave & 1) ? qb_buf.v : qb_buf.k;
    const bf16* ot = (wave & 1) ? buf2.v : buf2.k;
#pragma unroll
    for (int c = 0; c < NH; ++c)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        qf[c][kk] = plan.cols(qt, 32 * c, kk);
        if (wave < 2) of[c][kk] = plan.cols(ot, 32 * c, kk);
      }
  }
  lds_barrier();                               // buf0..2 free again
  // round 2: dO rows 128..255, then the walk's first two tiles
  fill_rows(buf2.k, dO, qb + 128);
  fill_rows(buf2.v, dO, qb + 192);
  if (ntiles > 0) fill(buf0, tile_at(0));       // a sparse walk may visit nothing
  if (ntiles > 1) fill(buf1, tile_at(1));
  // dO has landed once at most the 2 PER copies of a tile issued after it are
  // in flight (a ragged first tile went by the register path, whose loads
  // were waited for in order after it)
  if (ntiles > 0) wait_async_fills_but<2 * FS::PER>();
  else wait_async_fills();
  lds_barrier();
  {
    const bf16* ot = (wave & 1) ? buf2.v : buf2.k;
#pragma unroll
    for (int c = 0; c < NH; ++c)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        if (wave >= 2) of[c][kk] = plan.cols(ot, 32 * c, kk);
  }
  }
  // (the first step's barrier frees buf2, which its copies of tile 2 fill,
  // from these reads)
#pragma unroll
  for (int c = 0; c < NH; ++c) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (NH == 2) {
        pin_agpr(qf[c][kk]);
        pin_agpr(of[c][kk]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ndt[c][r] = dq[c];
  }
  int kt = 0;
  for (; kt + 3 <= inner_end; kt += 3) {
    step_inner(kt, buf0, buf2);
    step_inner(kt + 1, buf1, buf0);
    step_inner(kt + 2, buf2, buf1);
  }
  for (; kt + 3 <= ntiles; kt += 3) {
    step(kt, buf0, buf2);
    step(kt + 1, buf1, buf0);
    step(kt + 2, buf2, buf1);
  }
  if (kt < ntiles) step(kt, buf0, buf2);
  if (kt + 1 < ntiles) step(kt + 1, buf1, buf0);
  if constexpr (NH == 2) {
    // the last sub-tile's dQ_1
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      mma_acc_agpr(acc[NH - 1][i % MT], tf[i], bds1[i / MT]);
      fence();
    }
  } else {
    // the last sub-tile's dS and dQ
    frag bd[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) dpp[r] = pp[r] * dpp[r];
    bd[0] = M::pack(dpp, 0);
    bd[1] = M::pack(dpp, 1);
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) acc[0][i % MT] = M::mma(tf[i], bd[i / MT], acc[0][i % MT]);
  }

  if constexpr (NH == 2) mma_acc_drain(acc);
  // every wave is done with the key tiles: rows out through buf0 (waves 0, 1)
  // and buf1 (waves 2, 3), whole rows per store
  static_assert(NW == 4 && 2 * RowStage<D>::BYTES <= sizeof(Buf), "staging area");
  lds_barrier();
  bf16* stage = reinterpret_cast<bf16*>(wave < 2 ? &buf0 : &buf1) + (wave & 1) * (RowStage<D>::BYTES / 2);
#pragma unroll
  for (int c = 0; c < NH; ++c)
    store_rows_via_lds<D>(acc[c], dQ + base, rs, qw + 32 * c, N, scale, stage, lane);
  if constexpr (FUSE) {
    if (tid < BQ && qb + tid < N) {
      ws[rbase + qb + tid] = sD[tid];
      ws[(long)gridDim.z * H * N + rbase + qb + tid] = sL2[tid];
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers (bf16 only; the generic kernels serve f32)
// ---------------------------------------------------------------------------
static inline long rows_of(const BwdArgs& a) { return (long)a.B * a.H * a.N; }

// Compute units of the current device (0 if the query fails), once per device.
static int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cached[dev] = n;
  }
  return cached[dev];
}

template <int D, bool C, bool S>
static hipError_t dkdv_pipe_run(const BwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, C, S>), grid, dim3(256), 0, stream,
                     static_cast<const bf16*>(a.Q), static_cast<const bf16*>(a.K),
                     static_cast<const bf16*>(a.V), static_cast<const bf16*>(a.dO),
                     a.Dws + rows_of(a), a.Dws, static_cast<bf16*>(a.dK),
                     static_cast<bf16*>(a.dV), a.H, a.N, a.d, a.scale * kLog2e, a.scale,
                     a.mask, a.mask_heads, D == 64 ? device_cus() : 0);
  return hipGetLastError();
}
template <int D, bool C>
static hipError_t dkdv_pipe_go(const BwdArgs& a, hipStream_t stream) {
  return a.mask ? dkdv_pipe_run<D, C, true>(a, stream) : dkdv_pipe_run<D, C, false>(a, stream);
}

// 256 query rows per workgroup as DQ_NW waves of 256 / DQ_NW rows
#ifndef ATTN_DQ_NW
#define ATTN_DQ_NW 4
#endif
// (causal, head dim 64: the one-half form, 128 query rows per workgroup as
// four waves of 32, two workgroups per CU, so that the SIMDs whose waves walk
// the long rows near the sequence's end also take short ones)
template <int D, bool C, bool S, bool F>
static hipError_t dq_pipe_run(const BwdArgs& a, hipStream_t stream) {
  constexpr int NW = ATTN_DQ_NW, WQ = D == 64 && C ? 32 : 256 / NW, BQ = NW * WQ;
  dim3 grid((a.N + BQ - 1) / BQ, a.H, a.B);
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, C, WQ, NW, S, F>), grid, dim3(NW * 64), 0, stream,
                     static_cast<const bf16*>(a.Q), static_cast<const bf16*>(a.K),
                     static_cast<const bf16*>(a.V), static_cast<const bf16*>(a.dO),
                     F ? nullptr : a.Dws + rows_of(a), F ? nullptr : a.Dws,
                     static_cast<bf16*>(a.dQ), a.H, a.N, a.d, a.scale * kLog2e, a.scale, a.mask,
                     a.mask_heads, F ? static_cast<const bf16*>(a.O) : nullptr,
                     F ? a.L : nullptr, F ? a.ws_out : nullptr, WQ == 32 ? device_cus() : 0);
  return hipGetLastError();
}
template <int D, bool C>
static hipError_t dq_pipe_go(const BwdArgs& a, hipStream_t stream) {
  return a.mask ? dq_pipe_run<D, C, true, false>(a, stream)
                : dq_pipe_run<D, C, false, false>(a, stream);
}
template <int D, bool C>
static hipError_t dq_fused_pipe_go(const BwdArgs& a, hipStream_t stream) {
  return a.mask ? dq_pipe_run<D, C, true, true>(a, stream)
                : dq_pipe_run<D, C, false, true>(a, stream);
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
hipError_t launch_bwd_dq_fused_bf16_pipe(const BwdArgs& a, hipStream_t stream) {
  ATTN_PIPE_DISPATCH(dq_fused_pipe_go, a, stream);
}

}  // namespace attn
