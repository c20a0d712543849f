// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const float* Dws;   // workspace: D [B, H, N] then L * log2(e) [B, H, N]
  void* dQ;
  void* dK;
  void* dV;
  int B, H, N, d;
  int causal;
  float scale;
  int dtype;  // 0 = f32, 1 = bf16
  const unsigned char* mask = nullptr;   // block-sparse mask, or nullptr (every block kept)
  int mask_heads = 1;
  // dQ with the preprocess fused in (launch_bwd_dq_fused) only: the forward's
  // O and L, and the workspace (Dws) writable, which it fills
  const void* O = nullptr;
  const float* L = nullptr;
  float* ws_out = nullptr;
};

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int B, H, N, d;
  int causal;
  float scale;
  int dtype;
  const unsigned char* mask = nullptr;
  int mask_heads = 1;
};

// Backward of the backward: forward inputs, the output cotangent dO and the
// first backward's cotangents gQ, gK, gV -> hQ, hK, hV, hdO.
struct BobArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* L;
  const void* gQ;
  const void* gK;
  const void* gV;
  void* hQ;
  void* hK;
  void* hV;
  void* hdO;
  float* ws;   // -D, -L log2(e), r, E, each [B, H, N]
  int B, H, N, d;
  int causal;
  float scale;
  int dtype;
  const unsigned char* mask = nullptr;   // optional block mask (as BwdArgs)
  int mask_heads = 1;
};

// Head dims are served by kernels compiled for 32, 64, 128 or (bf16) 256
// columns; a smaller d runs in the next bucket with the extra columns read as
// zero.
inline int head_dim_bucket(int d) { return d <= 32 ? 32 : (d <= 64 ? 64 : (d <= 128 ? 128 : 256)); }

// Output columns one workgroup of a generic kernel accumulates: the whole head
// dim up to 128 (bf16) or 64 (float32, whose operands take twice the
// registers).  Wider heads split their output columns over D / out_cols
// workgroups per block, each rebuilding the scores over the full head dim, so
// the register footprint stays that of the largest unsplit bucket.
template <typename T, int D> constexpr int out_cols() {
  return sizeof(T) == 2 ? (D > 128 ? 128 : D) : (D > 64 ? 64 : D);
}
// The same split at run time: workgroups per block of the generic kernels for
// head dim d and dtype (0 = f32, 1 = bf16); their grid's y extent is H times this.
inline int column_parts(int d, int dtype) {
  const int bucket = head_dim_bucket(d);
  return dtype == 1 ? (bucket > 128 ? 2 : 1) : (bucket > 64 ? 2 : 1);
}

hipError_t launch_bwd_preprocess(const void* O, const void* dO, const float* L, float* ws, int B,
                                 int H, int N, int d, int dtype, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_lse(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16_pipe(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq_bf16_pipe(const BwdArgs& a, hipStream_t stream);
// Backward of the backward, pass 2 query-block outer (hQ, hdO), pipelined:
// serves bf16 at d = 64 and 128.
bool bob_q2_pipe_serves(const BobArgs& a);
hipError_t launch_bob_q2_pipe(const BobArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq_fused_bf16_pipe(const BwdArgs& a, hipStream_t stream);
// Whether launch_bwd_dq_fused serves these arguments (bf16, d 64 or 128); if
// so, it does the preprocess for dQ's own rows and writes the workspace, and
// launch_bwd_dkdv may follow it with no preprocess launch.
bool bwd_dq_fuses_preprocess(const BwdArgs& a);
hipError_t launch_bwd_dq_fused(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_lse_bf16_pipe(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bwd(const BobArgs& a, hipStream_t stream);

}  // namespace attn
