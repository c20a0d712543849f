// Forward kernel that also writes the saved row scalar L = m + log z.
//
// O follows the attention loss of ddx issue #217 ("Backward of batched
// attention builds a contraction over every pair of sequences and heads",
// repro script, CTEs scores / weights / norm / heads); L is the one number
// per row that ddx issue #243 (item 2) says the backward needs to rebuild the
// scores.  The row max and sum are kept online across key blocks.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

// Workgroup = 4 waves = one block of 128 query rows of one (b, h).  Wave w
// owns query rows qw + [0, 32); its Q rows sit in registers as the B operand
// of S^T = K Q^T, so each lane owns one query row (column of S^T) and the row
// max / row sum reduce over the lane's 16 registers plus its partner lane in
// the other half-wave.  P^T then feeds O^T += V^T P^T straight from the
// registers.  Key blocks of 64 rows (K, V) are double-buffered in LDS.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_lse_kernel(const T* __restrict__ Q,
                                                         const T* __restrict__ K,
                                                         const T* __restrict__ V,
                                                         T* __restrict__ O, float* __restrict__ L,
                                                         int H, int N, int d, float scale_log2,
                                                         const unsigned char* __restrict__ mask,
                                                         int mask_heads) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int BQ = 128, BKV = 64, KS = D / M::K, RS = 32 / M::K;
  // Wide heads (bf16 256 bucket, float32 128 bucket): each workgroup
  // accumulates DA of O's columns (part = which DA) and recomputes the scores
  // over the full head dim; the part-0 workgroup writes L.
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

  const int qb = ib * BQ;
  const int qw = qb + wave * 32;
  const int q = qw + l32;
  frag qf[KS];
  load_row_frags<T, D>(qf, Q + base, rs, q, N, d, h);

  f32x16 acc[MA];
#pragma unroll
  for (int i = 0; i < MA; ++i) acc[i] = zero16();
  float m = -1e30f;   // running max of the scaled scores, log2 units
  float l = 0.f;      // running sum of exp2(score - m)

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

  // bf16 whole tiles: direct copies by a plan built once per workgroup (the
  // tile base in scalar registers, a 32-bit offset per lane and copy), waited
  // for at the end of each step
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

  auto body = [&](const Buf& B, int k0, auto masked_c) ATTN_INLINE {
    constexpr bool MASKED = decltype(masked_c)::value;
    const KT kt_{const_cast<T*>(B.k)}, vt_{const_cast<T*>(B.v)};
    // (not unrolled: two sub-tiles in flight at once overflow the registers
    // at the widest head dims)
#pragma unroll 1
    for (int st = 0; st < BKV / 32; ++st) {
      const int ka = k0 + st * 32;
      if (MASKED && CAUSAL && ka > qw + 31) continue;
      // (bf16 head dim 256: the sub-tile's K and V operands are read in one
      // sequence, RA fragments ahead of their products through a ring, with
      // the order held by scheduling fences, so that no product waits on a
      // read issued right before it)
      constexpr bool RING = sizeof(T) == 2 && D > 128;
      constexpr int RA = 3, NOP = KS + RS * MA;
      auto opnd = [&](int n) ATTN_INLINE -> frag {
        if (n < KS) return kt_.along_cols(st * 32 + l32, n, h);
        const int j = n - KS;
        return vt_.along_rows(dofs + (j % MA) * 32 + l32, st * 32, j / MA, h);
      };
      frag ring[RING ? RA : 1];
      if constexpr (RING) {
#pragma unroll
        for (int n = 0; n < RA; ++n) ring[n] = opnd(n);
      }
      auto take = [&](int n) ATTN_INLINE -> frag {
        if constexpr (RING) {
          const frag a = ring[n % RA];
          if (n + RA < NOP) ring[n % RA] = opnd(n + RA);
          return a;
        } else {
          return opnd(n);
        }
      };
      auto fence_if_ring = [&]() ATTN_INLINE {
        if constexpr (RING) __builtin_amdgcn_sched_barrier(0);
      };
      f32x16 s = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        s = M::mma(take(kk), qf[kk], s);
        fence_if_ring();
      }
      // register r = key row ka + acc_row(r, h), column = query row q.  The
      // row max is taken on the raw scores (scale > 0 keeps the order).
      float mx = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MASKED) {
          const int kv = ka + acc_row(r, h);
          if ((CAUSAL && kv > q) || kv >= N) s[r] = -__builtin_inff();
        }
        mx = fmaxf(mx, s[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
      // Lazy rescaling: the running max m moves only when a row's new max
      // exceeds it by more than 8 (log2 units), so P = exp2(s c - m) stays
      // below 2^8 and the accumulators are rescaled only when some row of
      // the wave moved (rarely, once the max has settled).
      const bool upd = mx > m + 8.f;
      if (__builtin_amdgcn_ballot_w64(upd)) {
        const float m_new = upd ? mx : m;
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
        m = m_new;
#pragma unroll
        for (int mt = 0; mt < MA; ++mt) acc[mt] *= alpha;
      }
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -m));
        s[r] = p;
        sum += p;
      }
      sum += __shfl_xor(sum, 32);
      l += sum;
#pragma unroll
      for (int ss = 0; ss < RS; ++ss) {
        const frag bp = M::pack(s, ss);
#pragma unroll
        for (int mt = 0; mt < MA; ++mt) {
          acc[mt] = M::mma(take(KS + ss * MA + mt), bp, acc[mt]);
          fence_if_ring();
        }
      }
    }
  };

  // step p: tile tile_at(p) in cur while tile tile_at(p + 1) is copied to nxt
  auto step = [&](const Buf& cur, Buf& nxt, int p) ATTN_INLINE {
    const int k0 = tile_at(p) * BKV;
    if (p + 1 < ntiles) fill(nxt, tile_at(p + 1));
    if ((CAUSAL && k0 + BKV - 1 > qb) || k0 + BKV > N)
      body(cur, k0, std::integral_constant<bool, true>{});
    else
      body(cur, k0, std::integral_constant<bool, false>{});
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
  // a row that keeps no key ends with l = 0: O = 0, L = -inf
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int mt = 0; mt < MA; ++mt)
    store_acc_transposed<T>(acc[mt], O + base, rs, qw, dofs + mt * 32, N, d, inv, lane);
  if (h == 0 && q < N && dofs == 0)
    L[((long)b * H + head) * N + q] =
        l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
}

template <typename T, int D, bool C>
static hipError_t fwd_go(const FwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H * (D / out_cols<T, D>()), a.B);
  hipLaunchKernelGGL((fwd_lse_kernel<T, D, C>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                     static_cast<const T*>(a.V), static_cast<T*>(a.O), a.L, a.H, a.N, a.d,
                     a.scale * kLog2e, a.mask, a.mask_heads);
  return hipGetLastError();
}

hipError_t launch_fwd_lse(const FwdArgs& a, hipStream_t stream) {
  if (a.dtype == 1 && (a.d == 64 || a.d == 128)) return launch_fwd_lse_bf16_pipe(a, stream);
  const int bucket = head_dim_bucket(a.d);
  if (a.dtype == 1) {
    if (a.causal) {
      if (bucket == 32) return fwd_go<bf16, 32, true>(a, stream);
      if (bucket == 64) return fwd_go<bf16, 64, true>(a, stream);
      if (bucket == 128) return fwd_go<bf16, 128, true>(a, stream);
      return fwd_go<bf16, 256, true>(a, stream);
    }
    if (bucket == 32) return fwd_go<bf16, 32, false>(a, stream);
    if (bucket == 64) return fwd_go<bf16, 64, false>(a, stream);
    if (bucket == 128) return fwd_go<bf16, 128, false>(a, stream);
    return fwd_go<bf16, 256, false>(a, stream);
  }
  if (a.causal) {
    if (bucket == 32) return fwd_go<float, 32, true>(a, stream);
    if (bucket == 64) return fwd_go<float, 64, true>(a, stream);
    return fwd_go<float, 128, true>(a, stream);
  }
  if (bucket == 32) return fwd_go<float, 32, false>(a, stream);
  if (bucket == 64) return fwd_go<float, 64, false>(a, stream);
  return fwd_go<float, 128, false>(a, stream);
}

}  // namespace attn
