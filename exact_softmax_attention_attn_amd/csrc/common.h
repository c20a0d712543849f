// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (32x32 MFMA, wave64):
//   lane l, half h = l / 32, l32 = l % 32
//   A operand (32 x K): lane holds row m = l32, the K slots of half h
//   B operand (K x 32): lane holds column n = l32, the K slots of half h
//   C/D (32 x 32), 16 floats per lane: register r holds
//        row m = 8 * (r / 4) + 4 * h + (r % 4), column n = l32
// A and B only have to agree on which logical K index sits in each
// (half, slot); the hardware sums over all of them.  That freedom lets an
// accumulator feed the B operand of the next product directly: its rows
// become the K dimension, in the order the registers hold them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Lambdas in kernels must inline: a call would pass the accumulators through
// memory-like calling conventions and wreck register allocation.
#define ATTN_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;   // every attention kernel runs 4 waves per workgroup

// Row (within a 32-row accumulator block) held by accumulator register r in half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + sum_t x[t] y[t] over one 8-element bf16 chunk, as four two-element
// dot products (the products are exact in float32).  The preprocess kernel
// and the dQ kernel's folded preprocess both form D with it, so they leave
// the same bits.
// Sum over each aligned group of 16 lanes, returned in all 16, by DPP moves
// (no LDS round trips): lane pairs (quad_perm 1,0,3,2), pairs of pairs
// (quad_perm 2,3,0,1), then the half-row and row mirrors pair quads and
// eights.  Every lane adds the same two values at each stage, so all 16 get
// the same bits.  The preprocess kernel and the dQ kernel's folded
// preprocess both reduce D with it.
template <int CTRL> __device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                                  0xF, 0xF, false));
}
__device__ __forceinline__ float sum16_lanes(float x) {
  x = dpp_add<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x141>(x);   // row_half_mirror
  x = dpp_add<0x140>(x);   // row_mirror
  return x;
}

typedef __bf16 bf16pair __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_bf16(const bf16x8& x, const bf16x8& y, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16pair{x[2 * i], x[2 * i + 1]},
                                          bf16pair{y[2 * i], y[2 * i + 1]}, acc, false);
  return acc;
}

// Keep a matrix-core operand that lives for the whole kernel in the
// accumulation register file: the MFMA reads A/B operands from AGPRs directly,
// and the architectural VGPRs stay free for the per-tile working set.
template <typename V>
__device__ __forceinline__ void pin_agpr(V& x) { asm volatile("" : "+a"(x)); }

// Accumulate into an AGPR-resident 32x32 tile: acc += A B with
// v_mfma_f32_32x32x16_bf16 in its AGPR form.  Kernels compiled with every
// builtin MFMA in VGPR form (their results feed the VALU) use this for the
// accumulators that only ever meet the matrix core.  The compiler cannot see
// into the asm, so it cannot add the two wait states a matrix instruction
// needs after a VALU write of its A/B operands: callers either write those
// operands at least two instructions earlier or put mma_operand_guard()
// between the write and the product (the library's assembly test checks
// this on the compiled kernels).  Back-to-back accumulation into the same
// registers needs no wait states.
__device__ __forceinline__ void mma_acc_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Two wait states: between a VALU write of an operand and mma_acc_agpr.
__device__ __forceinline__ void mma_operand_guard() { asm volatile("s_nop 1"); }
// Fix where an mma_acc_agpr operand is produced: the optimiser may otherwise
// sink a pure computation (a pack) down to just before its first product.
template <typename V> __device__ __forceinline__ void pin_operand(V& x) {
  asm volatile("" : "+v"(x));
}

// Wait for two operand fragments at once: an empty statement that reads both
// makes the compiler's wait before it cover the pair, so the second of two
// back-to-back products needs no wait of its own.
template <typename V> __device__ __forceinline__ void need_both(const V& a, const V& b) {
  asm volatile("" : : "v"(a), "v"(b));
}

// A value every lane of the wave agrees on, moved to a scalar register (so
// addresses built from it stay scalar).
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Block order.  The grid is (blocks per head, H, B); workgroups are
// dispatched in linear order and handed to the XCDs round-robin.  Numbering
// the linear index "rank-major" (all (b, h) of rank 0 first, then rank 1, ...)
// and giving rank 0 the longest block makes the dispatch longest-first across
// all heads, so no long block starts late, and it sends every block of a
// given (b, h) to the same XCD (when B*H is a multiple of the XCD count), so
// the tiles the blocks of a head share stay in that XCD's L2.
struct BlockOrder {
  int rank, head, b;
};
__device__ __forceinline__ BlockOrder block_order() {
  const int nbh = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int bh = lin % nbh;
  return {lin / nbh, bh % (int)gridDim.y, bh / (int)gridDim.y};
}
// The same for kernels that run two workgroups per CU, when the whole grid
// fits the chip at once (cus < blocks <= 2 cus): the dispatcher gives the
// first cus workgroups one CU each and the rest the CUs' second places in the
// same order, so the second wave is numbered shortest-first (per XCD lane,
// which keeps a head's blocks on one XCD): the CU that runs the longest block
// also runs the shortest.  cus = 0 keeps block_order().
__device__ __forceinline__ BlockOrder block_order_paired(int cus) {
  const int nbh = gridDim.y * gridDim.z;
  int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int total = gridDim.x * nbh;
  if (cus > 0 && cus % 8 == 0 && total > cus && total <= 2 * cus && (total - cus) % 8 == 0 &&
      lin >= cus) {
    const int m = (total - cus) / 8, j = (lin - cus) / 8, x = lin % 8;
    lin = cus + 8 * (m - 1 - j) + x;
  }
  const int bh = lin % nbh;
  return {lin / nbh, bh % (int)gridDim.y, bh / (int)gridDim.y};
}

// ---------------------------------------------------------------------------
// Block-sparse masks.  A mask keeps or drops whole blocks of kMaskBlock query
// rows by kMaskBlock key rows (ddx PR #162, section "What changed": a filter
// on grouping keys passes a whole group of rows or none of it); the causal
// rule applies on top.  One (b, h) reads nb x nb bytes, row-major, nb =
// ceil(N / kMaskBlock); mask_heads = 1 shares one mask, B * H gives each
// (b, h) its own.
//
// A walk over tiles becomes a walk over a visit list: the kept tiles, in walk
// order, compacted into LDS once per workgroup.  Entry = tile index (low 14
// bits) | code << 14, code = which of (up to) two mask rows the workgroup's
// query rows span keep the tile (bit 0: the first, bit 1: the second); a
// workgroup inside one mask row uses code 1.
// ---------------------------------------------------------------------------
constexpr int kMaskBlock = 128;
constexpr int kMaxVisit = 1024;          // tiles of 64 rows per walk: N <= 65536
constexpr int kVisitTile = 0x3fff;

__device__ __forceinline__ const unsigned char* head_mask(const unsigned char* mask,
                                                          int mask_heads, int b, int head, int H,
                                                          int nb) {
  return mask + (mask_heads == 1 ? 0L : ((long)b * H + head) * nb * nb);
}

// Wave 0 compacts the candidates i = 0 .. n - 1 whose entry(i) is nonzero into
// vis[0 ..), in candidate order, 64 per ballot; every thread gets the count
// after the workgroup barrier that ends the call.
template <typename F>
__device__ __forceinline__ int build_visits(unsigned short* vis, int* count, int n, F entry) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int c = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const unsigned e = i < n ? entry(i) : 0u;
      const unsigned long long bal = __ballot(e != 0u);
      if (e != 0u) vis[c + __popcll(bal & ((1ull << lane) - 1ull))] = (unsigned short)e;
      c += __popcll(bal);
    }
    if (lane == 0) *count = c;
  }
  __syncthreads();
  return *count;
}

// Entry p of a visit list, as a wave-uniform value.  The read waits for
// itself inside the same statement (and so for every earlier LDS operation of
// the wave): meant for the points right before or after a barrier, where
// nothing else is in flight, and kept out of the compiler's view so it does
// not reschedule it among the operand reads.
__device__ __forceinline__ unsigned visit_entry(const unsigned short* vis, int p) {
  unsigned v;
  const unsigned addr = (unsigned)(unsigned long)((const __attribute__((address_space(3))) unsigned short*)(vis + p));
  asm volatile("ds_read_u16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return (unsigned)__builtin_amdgcn_readfirstlane((int)v);
}

// Entries of an ascending visit list vis[0 .. n) whose tile index is below x.
__device__ __forceinline__ int visits_below(const unsigned short* vis, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int)(vis[mid] & kVisitTile) < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Before the VALU reads AGPR accumulators written by mma_acc_agpr: the last
// 32x32 matrix instruction must have written its results back (it takes 8
// passes of 4 cycles plus write-back latency).
__device__ __forceinline__ void mma_acc_drain() {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
}
// The drain above, then every accumulator tile re-declared by an empty
// volatile asm: volatile statements keep their order, so no read of an
// accumulator can be scheduled above the drain.
template <int N>
__device__ __forceinline__ void mma_acc_drain(f32x16 (&acc)[N]) {
  mma_acc_drain();
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(acc[i]));
}
template <int N, int M>
__device__ __forceinline__ void mma_acc_drain(f32x16 (&acc)[N][M]) {
  mma_acc_drain();
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < M; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// ---------------------------------------------------------------------------
// Element type traits: which 32x32 MFMA, how deep one instruction contracts,
// how accumulator registers become a B operand.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  using frag = bf16x8;
  using chunk = bf16x8;                  // 16 bytes of a row
  static constexpr int K = 16;           // v_mfma_f32_32x32x16_bf16
  static constexpr int CHUNK = 8;        // elements per 16-byte chunk
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // B fragment for K step s from accumulator registers 8s .. 8s+7 (rounded to
  // nearest even), i.e. rows 16 s + 8 (t / 4) + 4 h + (t % 4) of the block.
  static __device__ __forceinline__ frag pack(const f32x16& c, int s) {
    frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (bf16)c[8 * s + t];
    return f;
  }
};

template <> struct Mma<float> {
  using frag = float;
  using chunk = f32x4;
  static constexpr int K = 2;            // v_mfma_f32_32x32x2_f32
  static constexpr int CHUNK = 4;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // step s uses accumulator register s: row acc_row(s, h) of the block
  static __device__ __forceinline__ frag pack(const f32x16& c, int s) { return c[s]; }
};

// ---------------------------------------------------------------------------
// A ROWS x D tile of a [pos, row_stride] global matrix staged in LDS.
//
// bf16: row-major, 16-byte chunks permuted within each row: logical chunk c
// of row r sits at chunk c ^ swz(r).  A read is served 256 bytes (all 64
// banks) at a time; the permutation keeps every such group on distinct slots:
//   - along_cols (ds_read_b128, one chunk per lane): any 16 consecutive rows
//     of one chunk, and any 8 aligned rows of two neighbouring chunks.
//   - along_rows (ds_read_b64_tr_b16, 8 bytes per lane): 32 consecutive lanes
//     read 4 aligned rows x 4 neighbouring chunks, lanes {0-15, 32-47} read 8
//     aligned rows x 2 chunks; both land on 16 distinct slots.
// f32: row-major with 4 floats of padding per row (a 1-float fragment reads
//   any layout in one access).
//
// along_cols(r, ks, h): operand with K slots along row r (contraction over
//   the tile's columns, e.g. the head dim), K step ks.
// along_rows(c, r0, s, h): operand with K slots down column c, rows in the
//   order the accumulator registers of the 32-row block at r0 hold them (see
//   Mma::pack), K step s (contraction over the tile's rows, e.g. positions).
// ---------------------------------------------------------------------------
template <typename T, int ROWS, int D> struct Tile;

template <int ROWS, int D> struct Tile<bf16, ROWS, D> {
  static constexpr int ELEMS = ROWS * D;
  static constexpr int BYTES = ELEMS * 2;
  static constexpr int CPR = D / 8;                       // chunks per row
  static_assert(CPR >= 4 && CPR <= 32 && (CPR & (CPR - 1)) == 0,
                "head-dim bucket must be 32, 64, 128 or 256");
  bf16* p;

  // Bank slot of (row, physical chunk) = (row % (16 / CPR)) * CPR + chunk for
  // CPR <= 16, and chunk % 16 for CPR 32 (a row is two 256-byte lines, so its
  // slots repeat).  With row bits r3 r2 r1 r0: CPR 16 and 32 permute by
  // (r1 r0 r2 r3), CPR 8 by (r1 r2 r3), CPR 4 by (r2 r3); rows sharing a slot
  // line then differ in the chunk bits that each read group above spans.
  __host__ __device__ __forceinline__ static int swz(int r) {
    if constexpr (CPR >= 16) return ((r & 2) << 2) | ((r & 1) << 2) | ((r >> 1) & 2) | ((r >> 3) & 1);
    else if constexpr (CPR == 8) return ((r & 2) << 1) | ((r >> 1) & 2) | ((r >> 3) & 1);
    else return ((r >> 1) & 2) | ((r >> 3) & 1);
  }
  __host__ __device__ __forceinline__ static int off(int r, int chunk) {
    return r * D + ((chunk ^ swz(r)) << 3);
  }
  __device__ __forceinline__ bf16x8 along_cols(int r, int ks, int h) const {
    return *reinterpret_cast<const bf16x8*>(p + off(r, 2 * ks + h));
  }
  __device__ __forceinline__ bf16x8 along_rows(int c, int r0, int s, int h) const {
    // 16-lane group g = lane / 16 reads rows ra + j / 4 (j = lane % 16), columns
    // cb + 4 (j % 4); the transposing read hands lane j column cb + j, 4 rows.
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;
    const int cb = (c & ~31) + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    const int ra = r0 + 16 * s + 4 * h + (j >> 2);
    const int e0 = off(ra, cb >> 3) + (cb & 7);
    const int e1 = off(ra + 8, cb >> 3) + (cb & 7);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + e0));
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + e1));
    bf16x4 fa = __builtin_bit_cast(bf16x4, a);
    bf16x4 fb = __builtin_bit_cast(bf16x4, b);
    return bf16x8{fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
  }
  __device__ __forceinline__ void put(int r, int chunk, const bf16x8& v) const {
    *reinterpret_cast<bf16x8*>(p + off(r, chunk)) = v;
  }
};

// Per-lane LDS offsets for the swizzled bf16 tiles, computed once per kernel.
// The swizzle depends only on a row's position inside its 16-row group, so
// the offset of any operand read is  plan entry + (16-row-aligned row) * D:
// a register plus an instruction immediate.
//   col[n]    : along_cols, rows r0 + l32, K step n (logical chunk 2n + h)
//   tr[mt][e] : along_rows, columns mt*32 + (the lane's column), first (e=0)
//               or second (e=1) group of 4 rows of K step s
template <int D> struct LanePlan {
  static constexpr int CPR = D / 8;
  int col[D / 16];
  int tr[D / 32][2];
  __host__ __device__ __forceinline__ explicit LanePlan(int lane) {
    using TT = Tile<bf16, 32, D>;
    const int h = lane >> 5, l32 = lane & 31, j = lane & 15;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) col[n] = l32 * D + (((2 * n + h) ^ TT::swz(l32)) << 3);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      const int cb = mt * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int rr = 4 * h + (j >> 2) + 8 * e;
        tr[mt][e] = rr * D + (((cb >> 3) ^ TT::swz(rr)) << 3) + (cb & 7);
      }
    }
  }
  // Marks the offsets as changed here, so that the compiler cannot hoist
  // (buffer base + offset) sums out of a loop over several statically named
  // buffers (one register per buffer and offset); inside the loop the buffer
  // base then folds into the read's immediate offset.
  __device__ __forceinline__ void rebind() {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) asm volatile("" : "+v"(col[n]));
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) asm volatile("" : "+v"(tr[mt][0]), "+v"(tr[mt][1]));
  }
  // operand with K slots along row r0 + l32 (r0 a multiple of 16), K step n
  __device__ __forceinline__ bf16x8 cols(const bf16* t, int r0, int n) const {
    return *reinterpret_cast<const bf16x8*>(t + col[n] + r0 * D);
  }
  // operand with K slots down column mt*32 + (lane's column), rows of the
  // 32-row accumulator block at r0 in register order, K step s
  __device__ __forceinline__ bf16x8 rows(const bf16* t, int r0, int s, int mt) const {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const bf16* b = t + (r0 + 16 * s) * D;
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + tr[mt][0]));
    i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + tr[mt][1]));
    bf16x4 fa = __builtin_bit_cast(bf16x4, a);
    bf16x4 fc = __builtin_bit_cast(bf16x4, c);
    return bf16x8{fa[0], fa[1], fa[2], fa[3], fc[0], fc[1], fc[2], fc[3]};
  }
};

template <int ROWS, int D> struct Tile<float, ROWS, D> {
  static constexpr int LDR = D + 4;
  static constexpr int ELEMS = ROWS * LDR;
  static constexpr int BYTES = ELEMS * 4;
  static constexpr int CPR = D / 4;
  float* p;

  __device__ __forceinline__ float along_cols(int r, int ks, int h) const {
    return p[r * LDR + ks * 2 + h];
  }
  __device__ __forceinline__ float along_rows(int c, int r0, int s, int h) const {
    return p[(r0 + acc_row(s, h)) * LDR + c];
  }
  __device__ __forceinline__ void put(int r, int chunk, const f32x4& v) const {
    *reinterpret_cast<f32x4*>(p + r * LDR + chunk * 4) = v;
  }
};

// ---------------------------------------------------------------------------
// Filling a Tile with rows [row0, row0 + ROWS) x columns [0, D) of a global
// [pos, row_stride] matrix, by all 256 threads.
//
// async_fill (bf16, whole tiles only): global_load_lds_dwordx4 copies 16
// bytes per lane straight into LDS without passing through registers; one
// wave instruction fills 1 KB of LDS, lane l landing at byte 16 l.  Each lane
// therefore fetches the logical chunk that the swizzle stores at its LDS
// slot.  Completion: s_waitcnt vmcnt(0) before the barrier that publishes it.
// fill_sync: 16-byte loads into registers, then LDS stores; rows >= nrows and
// columns >= ncols read as 0 (ragged tiles and the f32 layout).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// The copy plan of one wave, built once per kernel: for each of the wave's
// copy instructions, the byte offset (from the tile's first row in global
// memory) of the chunk this lane fetches.  A fill then costs one copy
// instruction per 1 KB with the tile's base address in scalar registers and
// the lane's 32-bit offset in a vector register; no per-fill address math.
// The offsets fit in 32 bits: ROWS <= 128 and rs = H * d <= 65535 * 128.
template <int ROWS, int D, int NWAVES = 4> struct AsyncFillShape {
  static constexpr int CPR = D / 8;       // chunks per row
  static constexpr int RPI = 64 / CPR;    // rows per wave instruction
  static constexpr int NI = ROWS / RPI;   // wave instructions per tile
  static constexpr int PER = NI / NWAVES; // instructions per wave
  static_assert(NI % NWAVES == 0, "tile must split evenly over the waves");
};

template <int ROWS, int D, int NWAVES = 4>
__host__ __device__ __forceinline__ void async_fill_plan(unsigned* off, long rs, int wave,
                                                         int lane) {
  using S = AsyncFillShape<ROWS, D, NWAVES>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int r = (wave * S::PER + i) * S::RPI + lane / S::CPR;
    const int chunk = (lane % S::CPR) ^ Tile<bf16, ROWS, D>::swz(r);
    off[i] = (unsigned)(((long)r * rs + chunk * 8) * (long)sizeof(bf16));
  }
}

// Copy instruction i (of the wave's PER) of the plan above.
template <int ROWS, int D, int NWAVES = 4>
__device__ __forceinline__ void async_fill_one(const Tile<bf16, ROWS, D>& t, const bf16* tile_base,
                                               const unsigned* off, int wave, int i) {
  using S = AsyncFillShape<ROWS, D, NWAVES>;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(tile_base) + off[i],
                                   (lds_void*)(t.p + (wave * S::PER + i) * 512), 16, 0, 0);
}

// Rows [row0, row0 + ROWS) of a global matrix into t, by the plan above;
// tile_base = (address of row row0) is the same in every lane.
template <int ROWS, int D, int NWAVES = 4>
__device__ __forceinline__ void async_fill(const Tile<bf16, ROWS, D>& t, const bf16* tile_base,
                                           const unsigned* off, int wave) {
  using S = AsyncFillShape<ROWS, D, NWAVES>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) async_fill_one<ROWS, D, NWAVES>(t, tile_base, off, wave, i);
}

// The same copies written as assembly, for the software-pipelined kernels
// that keep copies in flight across barriers.  The compiler's wait insertion
// cannot tell which LDS buffer a tracked copy writes and would drain every
// copy before the next LDS read; it does not see these, so their users wait
// explicitly (wait_async_fills*) before reading what they wrote.  M0 (the
// LDS destination) is declared clobbered, so the compiler keeps nothing in it
// across a copy and no save and restore is needed.
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(unsigned long)((lds_void*)p);
}
__device__ __forceinline__ void lds_dma_b128(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      : : "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_b32(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      : : "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}

// Copy instruction i of the plan (assembly form); tile_base wave-uniform.
template <int ROWS, int D, int NWAVES = 4>
__device__ __forceinline__ void async_fill_one_untracked(const Tile<bf16, ROWS, D>& t,
                                                         const bf16* tile_base, const unsigned* off,
                                                         int wave, int i) {
  using S = AsyncFillShape<ROWS, D, NWAVES>;
  lds_dma_b128(tile_base, off[i], lds_address(t.p + (wave * S::PER + i) * 512));
}
template <int ROWS, int D, int NWAVES = 4>
__device__ __forceinline__ void async_fill_untracked(const Tile<bf16, ROWS, D>& t,
                                                     const bf16* tile_base, const unsigned* off,
                                                     int wave) {
  using S = AsyncFillShape<ROWS, D, NWAVES>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i)
    async_fill_one_untracked<ROWS, D, NWAVES>(t, tile_base, off, wave, i);
}
// 64 consecutive floats at g (wave-uniform) into LDS, assembly form.
__device__ __forceinline__ void fill_row64_untracked(float* lds, const float* g, int lane) {
  lds_dma_b32(g, (unsigned)lane * 4u, lds_address(lds));
}

// One-off form for kernels that do not keep a plan.
template <int ROWS, int D, int NWAVES = 4>
__device__ __forceinline__ void fill_async(const Tile<bf16, ROWS, D>& t, const bf16* g, long rs,
                                           int row0, int wave, int lane) {
  unsigned off[AsyncFillShape<ROWS, D, NWAVES>::PER];
  async_fill_plan<ROWS, D, NWAVES>(off, rs, wave, lane);
  async_fill<ROWS, D, NWAVES>(t, g + (long)row0 * rs, off, wave);
}

// 64 consecutive floats (one wave instruction, 4 bytes per lane) into LDS.
__device__ __forceinline__ void fill_async_row64(float* lds, const float* g) {
  __builtin_amdgcn_global_load_lds(g + (threadIdx.x & 63), (lds_void*)lds, 4, 0, 0);
}

// Workgroup barrier for handing LDS tiles between waves.  __syncthreads()
// also waits for every vector-memory operation of the wave (its release
// fence), which would drain the global->LDS copies meant to stay in flight;
// here the wave's own LDS operations complete, then all waves meet.  Copies
// that must have landed are waited for explicitly (wait_async_fills*) before.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until every global->LDS copy issued by this wave has landed.
__device__ __forceinline__ void wait_async_fills() {
  // vmcnt = 0; expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt(0x3F70);
}

// Wait until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order, so all but the last N have landed).
template <int N> __device__ __forceinline__ void wait_async_fills_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x3F70 | (N & 15) | ((N >> 4) << 14));
}

template <typename T, int ROWS, int D, int NT = kThreads>
__device__ __forceinline__ void fill_sync(const Tile<T, ROWS, D>& t, const T* g, long rs, int row0,
                                          int nrows, int ncols, int tid) {
  using chunk = typename Mma<T>::chunk;
  constexpr int CH = Mma<T>::CHUNK;
  constexpr int CPR = D / CH;
  constexpr int NCH = (ROWS * CPR + NT - 1) / NT;
  chunk v[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int u = tid + NT * i;
    const int r = u / CPR, c = (u % CPR) * CH;
    v[i] = chunk{};
    if (u < ROWS * CPR && row0 + r < nrows && c < ncols)
      v[i] = *reinterpret_cast<const chunk*>(g + (long)(row0 + r) * rs + c);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int u = tid + NT * i;
    if (u < ROWS * CPR) t.put(u / CPR, u % CPR, v[i]);
  }
}

// A register-resident operand for a contraction over the head dim: the
// lane's row `row` of a global [pos, row_stride] matrix, K slots along the
// columns.  Out-of-range rows or columns read as 0.
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(typename Mma<T>::frag (&f)[D / Mma<T>::K],
                                               const T* g, long row_stride, int row, int nrows,
                                               int ncols, int h) {
  constexpr int KS = D / Mma<T>::K;
  const bool ok = row < nrows;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (sizeof(T) == 2) {
      const int c = ks * 16 + h * 8;
      f[ks] = (ok && c < ncols) ? *reinterpret_cast<const bf16x8*>(g + (long)row * row_stride + c)
                                : bf16x8{};
    } else {
      const int c = ks * 2 + h;
      f[ks] = (ok && c < ncols) ? g[(long)row * row_stride + c] : 0.f;
    }
  }
}

// Store a 32 x 32 accumulator holding X^T (rows = head-dim columns c0..c0+31,
// columns = positions n0..n0+31) into a global [pos, row_stride] matrix,
// multiplied by `mul`.  Each lane writes 4 consecutive columns per group.
template <typename T>
__device__ __forceinline__ void store_acc_transposed(const f32x16& acc, T* g, long row_stride,
                                                     int n0, int c0, int nrows, int ncols,
                                                     float mul, int lane) {
  const int h = lane >> 5, n = n0 + (lane & 31);
  if (n >= nrows) return;
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int c = c0 + 8 * grp + 4 * h;
    if (c < ncols) {
      T* p = g + (long)n * row_stride + c;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v{(bf16)(acc[4 * grp + 0] * mul), (bf16)(acc[4 * grp + 1] * mul),
                 (bf16)(acc[4 * grp + 2] * mul), (bf16)(acc[4 * grp + 3] * mul)};
        *reinterpret_cast<bf16x4*>(p) = v;
      } else {
        f32x4 v{acc[4 * grp + 0] * mul, acc[4 * grp + 1] * mul, acc[4 * grp + 2] * mul,
                acc[4 * grp + 3] * mul};
        *reinterpret_cast<f32x4*>(p) = v;
      }
    }
  }
}

// Store a wave's 32 positions x D head-dim columns, held as D / 32 accumulators
// of X^T in the layout store_acc_transposed takes (accumulator mt: columns
// 32 mt .. 32 mt + 31 by positions n0 .. n0 + 31), into a global
// [pos, row_stride] bf16 matrix, times `mul`, by way of a wave-private LDS
// area of 32 rows x RowStage<D>::PITCH = D + 8 elements (the 16-byte pad keeps
// the reads aligned and spreads the writes of one column over the banks).  The
// lanes first put their 4-column pieces there, then read back 16-byte pieces
// of whole rows: each store instruction then writes 64 / (D / 8) complete
// rows instead of one 16-byte piece of each of 32 rows.  Positions >= nrows
// are not stored.  No other wave may use the area meanwhile.
template <int D> struct RowStage {
  static constexpr int PITCH = D + 8;
  static constexpr int BYTES = 32 * PITCH * 2;
};
template <int D>
__device__ __forceinline__ void store_rows_via_lds(const f32x16 (&acc)[D / 32], bf16* g,
                                                   long row_stride, int n0, int nrows, float mul,
                                                   bf16* stage, int lane) {
  constexpr int PITCH = RowStage<D>::PITCH;
  const int h = lane >> 5, r = lane & 31;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const bf16x4 v{(bf16)(acc[mt][4 * grp + 0] * mul), (bf16)(acc[mt][4 * grp + 1] * mul),
                     (bf16)(acc[mt][4 * grp + 2] * mul), (bf16)(acc[mt][4 * grp + 3] * mul)};
      *reinterpret_cast<bf16x4*>(stage + r * PITCH + mt * 32 + 8 * grp + 4 * h) = v;
    }
  // the wave's LDS writes land before its reads below
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int CPR = D / 8;                   // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;                // rows per instruction
#pragma unroll
  for (int j = 0; j < 32 / RPI; ++j) {
    const int rr = j * RPI + lane / CPR, c = (lane % CPR) * 8;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(stage + rr * PITCH + c);
    if (n0 + rr < nrows) *reinterpret_cast<bf16x8*>(g + (long)(n0 + rr) * row_stride + c) = v;
  }
  // the reads are done before the area is written again
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace attn
