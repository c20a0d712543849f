// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (CDNA3/CDNA4 32x32 MFMA, wave64):
//   lane l, half h = l / 32, l32 = l % 32
//   A operand (32 x K): lane holds row m = l32, K-slots of half h
//   B operand (K x 32): lane holds column n = l32, K-slots of half h
//   C/D (32 x 32), 16 floats per lane: register r holds
//        row m = 8 * (r / 4) + 4 * h + (r % 4), column n = l32
// A and B only need to agree on which logical K index sits in each
// (half, slot); the hardware then sums over all of them.  That freedom lets a
// C accumulator feed the B operand of the next product directly: its rows
// become the K dimension, in the order the registers hold them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// Element type traits: which 32x32 MFMA, how deep one instruction contracts,
// how fragments are packed.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  using frag = bf16x8;
  static constexpr int K = 16;           // v_mfma_f32_32x32x16_bf16
  static constexpr int VEC = 8;          // elements per 16-byte global access
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // B fragment for K step s taken from accumulator registers 8s .. 8s+7
  static __device__ __forceinline__ frag pack(const f32x16& c, int s) {
    frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (bf16)c[8 * s + t];
    return f;
  }
  static __device__ __forceinline__ frag zero() { return frag{}; }
};

template <> struct Mma<float> {
  using frag = float;
  static constexpr int K = 2;            // v_mfma_f32_32x32x2_f32
  static constexpr int VEC = 4;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag pack(const f32x16& c, int s) { return c[s]; }
  static __device__ __forceinline__ frag zero() { return 0.f; }
};

// Row index (within a 32-row accumulator block) of K slot t, step s, half h,
// when accumulator registers are used as a B operand.  bf16: slots 0..7 of
// step s are registers 8s+t; f32: the single slot of step s is register s.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// A ROWS x D tile staged in LDS.
//   rm: row-major, row stride LDR (padding keeps 32 lanes reading 32
//       different rows on distinct banks).
//   tr: (bf16 only) the transpose, D rows of ROWS entries, stride LDT, with
//       the row index XOR-swizzled by 4 * ((c >> 5) & 3) so that the staging
//       writes of 16 neighbouring column groups land on distinct banks.
// along_cols(): operand whose K slots run along a row (contraction over the
//               tile's columns, e.g. over the head dim).
// along_rows(): operand whose K slots run down a column, in the order the
//               accumulator registers of a 32-row block hold their rows
//               (contraction over the tile's rows, e.g. over positions).
// ---------------------------------------------------------------------------
template <typename T, int ROWS, int D, bool TRANS> struct Tile;

template <int ROWS, int D, bool TRANS> struct Tile<bf16, ROWS, D, TRANS> {
  static constexpr int LDR = D + 8;
  static constexpr int LDT = ROWS + 4;
  static constexpr int RM_ELEMS = ROWS * LDR;
  static constexpr int TR_ELEMS = TRANS ? D * LDT : 0;
  static constexpr int BYTES = (RM_ELEMS + TR_ELEMS) * 2;
  bf16* rm;
  bf16* tr;

  __device__ __forceinline__ static int swz(int c) { return ((c >> 5) & 3) << 2; }

  __device__ __forceinline__ bf16x8 along_cols(int r, int ks, int h) const {
    return *reinterpret_cast<const bf16x8*>(rm + r * LDR + ks * 16 + h * 8);
  }
  // rows r0 + 16 s + 8 (t / 4) + 4 h + (t % 4), column c
  __device__ __forceinline__ bf16x8 along_rows(int c, int r0, int s, int h) const {
    const int x = swz(c);
    const bf16* base = tr + c * LDT;
    const int ra = (r0 + 16 * s + 4 * h) ^ x;
    const int rb = (r0 + 16 * s + 8 + 4 * h) ^ x;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + ra);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + rb);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  // Cooperative copy of rows [row0, row0 + ROWS) x columns [0, D) of a global
  // [.., row_stride] matrix; rows >= nrows and columns >= ncols read as 0.
  template <int NT>
  __device__ __forceinline__ void stage(const bf16* g, long row_stride, int row0, int nrows,
                                       int ncols, int tid) const {
    if constexpr (TRANS) {
      // unit = 4 rows x 8 columns: four 16-byte reads, four 16-byte row-major
      // writes, eight 8-byte transposed writes
      constexpr int CG = D / 8;
      constexpr int UNITS = (ROWS / 4) * CG;
#pragma unroll
      for (int u0 = 0; u0 < UNITS; u0 += NT) {
        const int u = u0 + tid;
        if (UNITS % NT == 0 || u < UNITS) {
          const int cg = u % CG, rg = u / CG;
          const int c = cg * 8;
          bf16x8 x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = row0 + rg * 4 + i;
            if (r < nrows && c < ncols)
              x[i] = *reinterpret_cast<const bf16x8*>(g + (long)r * row_stride + c);
            else
              x[i] = bf16x8{};
            *reinterpret_cast<bf16x8*>(rm + (rg * 4 + i) * LDR + c) = x[i];
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int cc = c + t;
            bf16x4 y{x[0][t], x[1][t], x[2][t], x[3][t]};
            *reinterpret_cast<bf16x4*>(tr + cc * LDT + ((rg * 4) ^ swz(cc))) = y;
          }
        }
      }
    } else {
      constexpr int CG = D / 8;
      constexpr int UNITS = ROWS * CG;
#pragma unroll
      for (int u0 = 0; u0 < UNITS; u0 += NT) {
        const int u = u0 + tid;
        if (UNITS % NT == 0 || u < UNITS) {
          const int cg = u % CG, r = u / CG;
          const int c = cg * 8;
          bf16x8 x = bf16x8{};
          if (row0 + r < nrows && c < ncols)
            x = *reinterpret_cast<const bf16x8*>(g + (long)(row0 + r) * row_stride + c);
          *reinterpret_cast<bf16x8*>(rm + r * LDR + c) = x;
        }
      }
    }
  }
};

template <int ROWS, int D, bool TRANS> struct Tile<float, ROWS, D, TRANS> {
  static constexpr int LDR = D + 4;
  static constexpr int RM_ELEMS = ROWS * LDR;
  static constexpr int TR_ELEMS = 0;
  static constexpr int BYTES = RM_ELEMS * 4;
  float* rm;
  float* tr;  // unused: a one-element fragment reads any layout in one access

  __device__ __forceinline__ float along_cols(int r, int ks, int h) const {
    return rm[r * LDR + ks * 2 + h];
  }
  __device__ __forceinline__ float along_rows(int c, int r0, int s, int h) const {
    return rm[(r0 + acc_row(s, h)) * LDR + c];
  }

  template <int NT>
  __device__ __forceinline__ void stage(const float* g, long row_stride, int row0, int nrows,
                                       int ncols, int tid) const {
    constexpr int CG = D / 4;
    constexpr int UNITS = ROWS * CG;
#pragma unroll
    for (int u0 = 0; u0 < UNITS; u0 += NT) {
      const int u = u0 + tid;
      if (UNITS % NT == 0 || u < UNITS) {
        const int cg = u % CG, r = u / CG;
        const int c = cg * 4;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row0 + r < nrows && c < ncols)
          x = *reinterpret_cast<const f32x4*>(g + (long)(row0 + r) * row_stride + c);
        *reinterpret_cast<f32x4*>(rm + r * LDR + c) = x;
      }
    }
  }
};

// A register-resident operand for a contraction over the head dim: the
// lane's row `row` of a global [.., row_stride] matrix, K slots along the
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

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace attn
