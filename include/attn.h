/*
 * attn.h -- C ABI of libattn.so: exact softmax attention forward (with the
 * saved row scalar) and its exact backward by score recomputation, for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  For each batch b and head h, with q_i, k_j, v_j the rows
 * of Q, K, V at (b, ., h, .):
 *
 *   S_ij = scale * q_i . k_j          kept for j <= i when causal (diagonal
 *                                     kept), every j otherwise
 *   P_ij = exp(S_ij - L_i),  L_i = m_i + log z_i,  m_i = max_j S_ij,
 *          z_i = sum_j exp(S_ij - m_i)
 *   O_i  = sum_j P_ij v_j
 *
 * This is the attention loss of ddx issue #217 ("Backward of batched
 * attention builds a contraction over every pair of sequences and heads",
 * repro script: CTEs scores, weights, norm, heads), with L the one saved
 * number per row of ddx issue #243, item 2 ("Attention's gradient: a softmax
 * shift's backward computed twice, and recomputing scores instead of saving
 * them").  The backward returns the gradient of sum(dO o O):
 *
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
 *   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q
 *
 * with no term for the row-max shift (issue #243, item 1: it cancels), and
 * with S and P rebuilt tile by tile from Q, K and L (issue #243, item 2), so
 * no N x N array is ever stored in device memory.
 *
 * Conventions shared by every entry point.
 *  - Layout.  Q, K, V, O, dO, dQ, dK, dV are dense, row-major [B, N, H, d]
 *    (sequence, position, head, channel), the index order of issue #217's
 *    tables.  L and the workspace are dense [B, H, N] float32.
 *  - dtype.  ATTN_F32: all [B, N, H, d] tensors are float32, arithmetic is
 *    float32.  ATTN_BF16: they are bfloat16; products run on bf16 matrix
 *    cores with float32 accumulation; P and dS are rounded to bf16 (nearest
 *    even) before they enter a product; outputs are rounded to bf16.
 *  - Pointers are device pointers (or host-coherent pointers the GPU can
 *    read), aligned to 16 bytes.  The caller owns every buffer; the library
 *    allocates nothing, frees nothing and keeps no pointer after returning
 *    (attn_bwd_noalloc's workspace is a static array of the library's own).
 *  - Outputs must not alias inputs or each other; they are overwritten.
 *  - stream is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work and return; results are visible after the stream is synchronised.
 *    Apart from attn_bwd_noalloc's per-GPU workspace array, there is no
 *    global mutable state, so calls are thread-safe.
 *  - Errors.  The return value is an attn_status_t.  On ATTN_ERR_INVALID or
 *    ATTN_ERR_UNSUPPORTED nothing was enqueued, no HIP call was made, and the
 *    outputs are untouched.  ATTN_ERR_HIP means a launch failed; the text of
 *    the HIP error is returned by attn_last_error() on the calling thread.
 *    Non-finite inputs are not checked; they propagate.
 *  - Limits.  B, H, N, d >= 1 (ATTN_ERR_INVALID otherwise); d <= 128 (f32) or
 *    d <= 256 (bf16); d % 4 == 0 (f32) or d % 8 == 0 (bf16); B, H <= 65535,
 *    and H <= 32767 where the head's output columns split over two workgroups
 *    (bf16 with d > 128, f32 with d > 64); B*H*N < 2^31, so B*N*H*d < 2^39
 *    (ATTN_ERR_UNSUPPORTED otherwise); scale finite and > 0.  causal is 1
 *    (keep j <= i) or 0 (keep every pair).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,      /* null pointer, size < 1, bad scale or flag */
  ATTN_ERR_UNSUPPORTED = 2,  /* d or dtype outside what the kernels take  */
  ATTN_ERR_HIP = 3           /* a HIP launch failed                       */
} attn_status_t;

/*
 * Forward pass that also saves the row scalar.
 *   in : Q, K, V  [B, N, H, d] (dtype)
 *   out: O        [B, N, H, d] (dtype)   O_i = sum_j P_ij v_j
 *        L        [B, H, N]    float32   L_i = m_i + log z_i (natural log)
 * Issue #217 repro (CTEs scores .. heads) for O; issue #243 item 2 for L.
 */
int attn_fwd_lse(const void* Q, const void* K, const void* V, void* O, float* L,
                 int B, int H, int N, int d, int causal, float scale, int dtype,
                 void* stream);

/* Bytes of device workspace attn_bwd needs: 2*B*H*N*sizeof(float).  It holds
 * -D [B, H, N] followed by -L * log2(e) [B, H, N] (the row scalars negated and,
 * for L, in the base-2 units the kernels exponentiate in).  Returns 0 when a
 * size is < 1 or the sizes are unsupported. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass by score recomputation, on one stream: the three stages below
 * in order (preprocess, dK/dV, dQ), or, for bf16 with d = 64 or 128, two
 * launches -- dQ first, doing the preprocess's arithmetic for its own rows and
 * writing -D and -L * log2(e) to the workspace, then dK/dV.  Both orders give
 * the same bits in dQ, dK, dV and the workspace.
 *   in : Q, K, V, O, dO [B, N, H, d] (dtype); L [B, H, N] float32 as written
 *        by attn_fwd_lse (or any L_i = log sum_j exp(S_ij) of the same kept set)
 *   out: dQ, dK, dV     [B, N, H, d] (dtype)
 *   workspace: >= attn_bwd_workspace_bytes(B, H, N, d) bytes of device memory,
 *        16-byte aligned; overwritten with -D and -L * log2(e).
 * PR #162 ("perf(ddx-ad): transpose causal attention's contractions without
 * their joins", section "What changed") names the plan: transpose p = w/z per
 * score, then p @ v.
 */
int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* L, void* dQ, void* dK, void* dV, void* workspace,
             int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * attn_bwd for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same launches and kernels, with the workspace taken from an array the
 * library holds in each GPU's memory (ATTN_NOALLOC_MAX_BYTES per GPU, from
 * the first call on that GPU until the process ends) instead of an argument.
 * The call allocates nothing.
 *   in, out: as attn_bwd; results are bitwise those of attn_bwd.
 *   Limit: the workspace attn_bwd would need, 2*B*H*N*sizeof(float), must not
 *   exceed ATTN_NOALLOC_MAX_BYTES (B*H*N <= 2,097,152 rows); larger calls
 *   return ATTN_ERR_UNSUPPORTED before any HIP call, with the reason in
 *   attn_last_error().
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *   last call's contents (nothing in it needs clearing: the first launch
 *   overwrites all that the later ones read).  Calls that overlap on one GPU -- on
 *   different streams, or from different threads without ordering -- race on
 *   it; calls on different GPUs do not.  The current device must be the one
 *   the pointers and the stream belong to.
 */
#define ATTN_NOALLOC_MAX_BYTES ((size_t)16 << 20)
int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* L, void* dQ, void* dK, void* dV,
                     int B, int H, int N, int d, int causal, float scale, int dtype,
                     void* stream);

/*
 * Stage 1 of attn_bwd: D_i = sum_c dO_ic O_ic in float32 (the softmax-weighted
 * sum of dP, issue #243 item 2, since sum_j P_ij dP_ij = dO_i . O_i) and
 * L_i * log2(e), written negated to workspace as two [B, H, N] float32 arrays.
 */
int attn_bwd_preprocess(const void* O, const void* dO, const float* L, void* workspace,
                        int B, int H, int N, int d, int dtype, void* stream);

/*
 * Stage 2 of attn_bwd: dK and dV.  One workgroup owns a block of key rows,
 * keeps K, V and the dK, dV accumulators on chip, and walks the query blocks
 * that can see them (from the diagonal down when causal), rebuilding S, P,
 * dP and dS per tile.  Reads -D and -L * log2(e) from workspace (stage 1 must
 * have run on the same workspace).
 */
int attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                  const void* workspace, void* dK, void* dV,
                  int B, int H, int N, int d, int causal, float scale, int dtype,
                  void* stream);

/*
 * Stage 3 of attn_bwd: dQ.  One workgroup owns a block of query rows and walks
 * the key blocks it can see, rebuilding S, P, dP and dS and accumulating
 * dS K on chip.  No atomics: every dQ element is written once by one thread,
 * so results are bitwise repeatable.  Reads -D and -L * log2(e) from workspace.
 */
int attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                const void* workspace, void* dQ,
                int B, int H, int N, int d, int causal, float scale, int dtype,
                void* stream);

/*
 * Block-sparse masks.  A mask keeps or drops whole blocks of ATTN_MASK_BLOCK
 * query rows by ATTN_MASK_BLOCK key rows, the group-level filter of ddx PR
 * #162 ("perf(ddx-ad): transpose causal attention's contractions without
 * their joins", section "What changed": a filter that reads only grouping
 * keys passes every row of a group or none).  Pair (i, j) is kept iff
 *     mask[., i / ATTN_MASK_BLOCK, j / ATTN_MASK_BLOCK] != 0
 * and, when causal, j <= i.  Tiles of dropped blocks are never visited.
 *   mask: device memory, uint8 [mask_heads, nb, nb] row-major, nb =
 *         ceil(N / ATTN_MASK_BLOCK); any alignment; read only.
 *   mask_heads: 1 (every (b, h) shares the mask) or B * H (entry b * H + h).
 * A row that keeps no key has O = 0 and L = -inf, and contributes nothing to
 * dK and dV; its dQ is 0.  Limits beyond the shared ones: N <= 65536
 * (ATTN_ERR_UNSUPPORTED otherwise); mask_heads not 1 or B * H, or a null mask,
 * is ATTN_ERR_INVALID.  The backward must be given the L of the masked
 * forward with the same mask.
 */
#define ATTN_MASK_BLOCK 128

/* attn_fwd_lse restricted to the pairs a block mask keeps. */
int attn_fwd_lse_masked(const void* Q, const void* K, const void* V, void* O, float* L,
                        const unsigned char* mask, int mask_heads,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        void* stream);

/* attn_bwd restricted to the pairs a block mask keeps (the same launches;
 * the preprocess is the same, dK/dV and dQ walk only kept tiles). */
int attn_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* L, void* dQ, void* dK, void* dV, void* workspace,
                    const unsigned char* mask, int mask_heads,
                    int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/* Stages 2 and 3 of attn_bwd_masked (stage 1 is attn_bwd_preprocess). */
int attn_bwd_dkdv_masked(const void* Q, const void* K, const void* V, const void* dO,
                         const void* workspace, void* dK, void* dV,
                         const unsigned char* mask, int mask_heads,
                         int B, int H, int N, int d, int causal, float scale, int dtype,
                         void* stream);
int attn_bwd_dq_masked(const void* Q, const void* K, const void* V, const void* dO,
                       const void* workspace, void* dQ,
                       const unsigned char* mask, int mask_heads,
                       int B, int H, int N, int d, int causal, float scale, int dtype,
                       void* stream);

/*
 * Backward of the backward.  The first backward maps (Q, K, V, dO) to
 * (dQ, dK, dV); given cotangents gQ, gK, gV of its outputs, this returns the
 * gradients of  l2 = <gQ, dQ> + <gK, dK> + <gV, dV>  with respect to Q, K, V
 * and dO: the exact gradient of the backward pass, whose goal (no N x N array
 * in memory, a pair of per-row quantities beyond the recomputed tiles) is set
 * by the page "Approaching I/O-optimality for Approximate Attention", its
 * first abstract (FlashBoB); the formulas are derived from the chain rule.
 * With P, dP, D
 * and dS as in attn_bwd, G = scale (gQ K^T + Q gK^T), A = dO gV^T,
 *   r_i = sum_j P_ij G_ij,   E_i = sum_j (P_ij A_ij + dS_ij G_ij),
 *   W = P o (G - r),         dS2 = P o (A + (dP - D) o (G - r) - E),
 *   hQ = scale (dS2 K + dS gK),  hK = scale (dS2^T Q + dS^T gQ),
 *   hV = W^T dO,                 hdO = P gV + W V.
 *   in : Q, K, V, O, dO, gQ, gK, gV [B, N, H, d] (dtype); L [B, H, N] float32
 *        from attn_fwd_lse
 *   out: hQ, hK, hV, hdO [B, N, H, d] (dtype)
 *   workspace: >= attn_bwd_bwd_workspace_bytes(B, H, N, d) bytes, 16-byte
 *        aligned; overwritten with -D, -L log2(e), r and E.
 * Four launches on one stream: the preprocess, a query-block pass for r and
 * E, a key-block pass for hK, hV and a query-block pass for hQ, hdO; no N x N
 * array in memory.  Limits beyond the shared ones: d <= 128 (bf16) or d <= 64
 * (f32), ATTN_ERR_UNSUPPORTED otherwise.
 */
size_t attn_bwd_bwd_workspace_bytes(int B, int H, int N, int d);
int attn_bwd_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* L, const void* gQ, const void* gK, const void* gV,
                 void* hQ, void* hK, void* hV, void* hdO, void* workspace,
                 int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/* attn_bwd_bwd restricted to the pairs a block mask keeps (mask and
 * mask_heads as in the block-sparse section above; L from attn_fwd_lse_masked
 * with the same mask).  Every pass walks only kept tiles; a query row that
 * keeps no key gets r = E = 0 and hQ = hdO = 0, and adds nothing to hK, hV.
 * Validation and limits are those of attn_bwd_bwd plus the mask's. */
int attn_bwd_bwd_masked(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* L, const void* gQ, const void* gK,
                        const void* gV, void* hQ, void* hK, void* hV, void* hdO, void* workspace,
                        const unsigned char* mask, int mask_heads,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        void* stream);

/* Static text for a status code ("ok", "invalid argument", ...). */
const char* attn_status_string(int status);

/* Text of the last ATTN_ERR_HIP on the calling thread, or of the last size
 * rejection by attn_bwd_noalloc ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
