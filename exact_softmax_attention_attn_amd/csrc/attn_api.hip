// C-ABI layer of libattn.so: argument validation (no HIP call until every
// check passes), dispatch to the kernel launchers, status reporting.
#include <initializer_list>
#include <math.h>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"
#include "launch.h"

namespace {

thread_local char g_last_error[256] = "";

void set_error_text(const char* s) {
  strncpy(g_last_error, s, sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = '\0';
}

void set_hip_error(hipError_t e) {
  const char* s = hipGetErrorString(e);
  set_error_text(s ? s : "unknown HIP error");
}

// Workspace of attn_bwd_noalloc: one array per GPU, in the library's own
// device memory, held until the process ends.  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress (looked up once per device, with that device current)
// and is what the kernels receive.
constexpr size_t kScratchBytes = ATTN_NOALLOC_MAX_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the array (its address looked up on the
// device's first call).
int current_device_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_hip_error(e);
    return ATTN_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error_text("attn_bwd_noalloc: device index beyond the 64 the library tracks");
    return ATTN_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      set_hip_error(e);
      return ATTN_ERR_HIP;
    }
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    set_hip_error(e);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// Sizes: each >= 1; grid limits (B, H <= 65535); B*H*N < 2^31 rows, so with
// d <= 256 every element offset (64-bit in the kernels) is below 2^39.
int check_sizes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_ERR_INVALID;
  if (B > 65535 || H > 65535) return ATTN_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)B * H * N;
  if (rows >= ((int64_t)1 << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Head dim and dtype; then the generic kernels' grid: wide heads run
// column_parts(d, dtype) workgroups per block along the grid's y axis, so
// H * parts must stay within its 65535 limit.
int check_dtype_dim(int H, int d, int dtype) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d > (dtype == ATTN_BF16 ? 256 : 128)) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_F32 && d % 4 != 0) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_BF16 && d % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)H * attn::column_parts(d, dtype) > 65535) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int check_scale_causal(float scale, int causal) {
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

// Block masks: a mask given, one per (b, h) or one shared; the walks' visit
// lists hold up to 1024 tiles of 64 rows.
int check_mask(const unsigned char* mask, int mask_heads, int B, int H, int N) {
  if (mask == nullptr) return ATTN_ERR_INVALID;
  if (mask_heads != 1 && (int64_t)mask_heads != (int64_t)B * H) return ATTN_ERR_INVALID;
  if (N > 65536) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

#define ATTN_TRY(expr)           \
  do {                           \
    const int st_ = (expr);      \
    if (st_ != ATTN_OK) return st_; \
  } while (0)

attn::BwdArgs make_bwd(const void* Q, const void* K, const void* V, const void* dO,
                       const void* ws, void* dQ, void* dK, void* dV, int B, int H, int N, int d,
                       int causal, float scale, int dtype) {
  attn::BwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.dO = dO;
  a.Dws = static_cast<const float*>(ws);
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.causal = causal; a.scale = scale; a.dtype = dtype;
  return a;
}

}  // namespace

extern "C" {

int attn_fwd_lse(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H,
                 int N, int d, int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, L}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  attn::FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.causal = causal; a.scale = scale; a.dtype = dtype;
  return finish(attn::launch_fwd_lse(a, static_cast<hipStream_t>(stream)));
}

int attn_fwd_lse_masked(const void* Q, const void* K, const void* V, void* O, float* L,
                        const unsigned char* mask, int mask_heads, int B, int H, int N, int d,
                        int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, L}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  ATTN_TRY(check_mask(mask, mask_heads, B, H, N));
  attn::FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.causal = causal; a.scale = scale; a.dtype = dtype;
  a.mask = mask; a.mask_heads = mask_heads;
  return finish(attn::launch_fwd_lse(a, static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_sizes(B, H, N, d) != ATTN_OK) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

int attn_bwd_preprocess(const void* O, const void* dO, const float* L, void* workspace, int B,
                        int H, int N, int d, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({O, dO, L, workspace}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  return finish(attn::launch_bwd_preprocess(O, dO, L, static_cast<float*>(workspace), B, H, N, d,
                                            dtype, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                  const void* workspace, void* dK, void* dV, int B, int H, int N, int d,
                  int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, dO, workspace, dK, dV}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  const attn::BwdArgs a =
      make_bwd(Q, K, V, dO, workspace, nullptr, dK, dV, B, H, N, d, causal, scale, dtype);
  return finish(attn::launch_bwd_dkdv(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                const void* workspace, void* dQ, int B, int H, int N, int d, int causal,
                float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, dO, workspace, dQ}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  const attn::BwdArgs a =
      make_bwd(Q, K, V, dO, workspace, dQ, nullptr, nullptr, B, H, N, d, causal, scale, dtype);
  return finish(attn::launch_bwd_dq(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
// The stages of attn_bwd on a validated call, with workspace ws (a block mask
// optional).  Where the dQ kernel can do the preprocess for its own rows
// (bf16, d 64 or 128), it runs first and fills ws, then dK/dV: two launches.
// Otherwise preprocess, dK/dV, dQ.  Both orders leave the same bits in dQ,
// dK, dV and ws.
int run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
            const float* L, void* dQ, void* dK, void* dV, float* ws, int B, int H, int N, int d,
            int causal, float scale, int dtype, hipStream_t s,
            const unsigned char* mask = nullptr, int mask_heads = 1) {
  attn::BwdArgs a = make_bwd(Q, K, V, dO, ws, dQ, dK, dV, B, H, N, d, causal, scale, dtype);
  a.mask = mask;
  a.mask_heads = mask_heads;
  if (attn::bwd_dq_fuses_preprocess(a)) {
    a.O = O;
    a.L = L;
    a.ws_out = ws;
    hipError_t e = attn::launch_bwd_dq_fused(a, s);
    if (e != hipSuccess) return finish(e);
    return finish(attn::launch_bwd_dkdv(a, s));
  }
  hipError_t e = attn::launch_bwd_preprocess(O, dO, L, ws, B, H, N, d, dtype, s);
  if (e != hipSuccess) return finish(e);
  e = attn::launch_bwd_dkdv(a, s);
  if (e != hipSuccess) return finish(e);
  return finish(attn::launch_bwd_dq(a, s));
}

int run_bob(const void* Q, const void* K, const void* V, const void* O, const void* dO,
            const float* L, const void* gQ, const void* gK, const void* gV, void* hQ, void* hK,
            void* hV, void* hdO, void* workspace, const unsigned char* mask, int mask_heads,
            int B, int H, int N, int d, int causal, float scale, int dtype, void* stream) {
  attn::BobArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.L = L;
  a.gQ = gQ; a.gK = gK; a.gV = gV;
  a.hQ = hQ; a.hK = hK; a.hV = hV; a.hdO = hdO;
  a.ws = static_cast<float*>(workspace);
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.causal = causal; a.scale = scale; a.dtype = dtype;
  a.mask = mask; a.mask_heads = mask_heads;
  return finish(attn::launch_bwd_bwd(a, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* L, void* dQ, void* dK, void* dV, void* workspace, int B, int H, int N,
             int d, int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, dO, L, dQ, dK, dV, workspace}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  return run_bwd(Q, K, V, O, dO, L, dQ, dK, dV, static_cast<float*>(workspace), B, H, N, d,
                 causal, scale, dtype, static_cast<hipStream_t>(stream));
}

int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* L, void* dQ, void* dK, void* dV, int B, int H, int N, int d,
                     int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, dO, L, dQ, dK, dV}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  const size_t need = 2 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof(msg),
             "attn_bwd_noalloc: workspace of %zu bytes (2*B*H*N floats) exceeds the static "
             "%zu-byte array; call attn_bwd with a workspace instead",
             need, kScratchBytes);
    set_error_text(msg);
    return ATTN_ERR_UNSUPPORTED;
  }
  float* ws = nullptr;
  ATTN_TRY(current_device_scratch(&ws));
  return run_bwd(Q, K, V, O, dO, L, dQ, dK, dV, ws, B, H, N, d, causal, scale, dtype,
                 static_cast<hipStream_t>(stream));
}

int attn_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* L, void* dQ, void* dK, void* dV, void* workspace,
                    const unsigned char* mask, int mask_heads, int B, int H, int N, int d,
                    int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, dO, L, dQ, dK, dV, workspace}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  ATTN_TRY(check_mask(mask, mask_heads, B, H, N));
  return run_bwd(Q, K, V, O, dO, L, dQ, dK, dV, static_cast<float*>(workspace), B, H, N, d,
                 causal, scale, dtype, static_cast<hipStream_t>(stream), mask, mask_heads);
}

int attn_bwd_dkdv_masked(const void* Q, const void* K, const void* V, const void* dO,
                         const void* workspace, void* dK, void* dV, const unsigned char* mask,
                         int mask_heads, int B, int H, int N, int d, int causal, float scale,
                         int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, dO, workspace, dK, dV}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  ATTN_TRY(check_mask(mask, mask_heads, B, H, N));
  attn::BwdArgs a =
      make_bwd(Q, K, V, dO, workspace, nullptr, dK, dV, B, H, N, d, causal, scale, dtype);
  a.mask = mask;
  a.mask_heads = mask_heads;
  return finish(attn::launch_bwd_dkdv(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dq_masked(const void* Q, const void* K, const void* V, const void* dO,
                       const void* workspace, void* dQ, const unsigned char* mask,
                       int mask_heads, int B, int H, int N, int d, int causal, float scale,
                       int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, dO, workspace, dQ}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  ATTN_TRY(check_mask(mask, mask_heads, B, H, N));
  attn::BwdArgs a =
      make_bwd(Q, K, V, dO, workspace, dQ, nullptr, nullptr, B, H, N, d, causal, scale, dtype);
  a.mask = mask;
  a.mask_heads = mask_heads;
  return finish(attn::launch_bwd_dq(a, static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_sizes(B, H, N, d) != ATTN_OK) return 0;
  return 4 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

int attn_bwd_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* L, const void* gQ, const void* gK, const void* gV, void* hQ,
                 void* hK, void* hV, void* hdO, void* workspace, int B, int H, int N, int d,
                 int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, dO, L, gQ, gK, gV, hQ, hK, hV, hdO, workspace}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  if (d > (dtype == ATTN_BF16 ? 128 : 64)) return ATTN_ERR_UNSUPPORTED;
  return run_bob(Q, K, V, O, dO, L, gQ, gK, gV, hQ, hK, hV, hdO, workspace, nullptr, 1, B, H, N,
                 d, causal, scale, dtype, stream);
}

int attn_bwd_bwd_masked(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* L, const void* gQ, const void* gK,
                        const void* gV, void* hQ, void* hK, void* hV, void* hdO, void* workspace,
                        const unsigned char* mask, int mask_heads, int B, int H, int N, int d,
                        int causal, float scale, int dtype, void* stream) {
  ATTN_TRY(check_ptrs({Q, K, V, O, dO, L, gQ, gK, gV, hQ, hK, hV, hdO, workspace}));
  ATTN_TRY(check_sizes(B, H, N, d));
  ATTN_TRY(check_scale_causal(scale, causal));
  ATTN_TRY(check_dtype_dim(H, d, dtype));
  ATTN_TRY(check_mask(mask, mask_heads, B, H, N));
  if (d > (dtype == ATTN_BF16 ? 128 : 64)) return ATTN_ERR_UNSUPPORTED;
  return run_bob(Q, K, V, O, dO, L, gQ, gK, gV, hQ, hK, hV, hdO, workspace, mask, mask_heads, B,
                 H, N, d, causal, scale, dtype, stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported size, head dim or dtype";
    case ATTN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
