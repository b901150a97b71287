/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The library computes exact softmax attention O = softmax(scale * Q K^T) V by
 * tiling: each workgroup keeps a block of query rows on chip, streams key and
 * value blocks past it, and keeps a running maximum, running sum and running
 * output per row, so the N x N score matrix never reaches device memory
 * ("Interrogating the GPU, part 5: FlashAttention", sections "How does tiling
 * remove the traffic?" and "How can you softmax a row you never see whole?").
 * The forward pass saves one log-sum-exp per row; the backward pass recomputes
 * each probability tile from Q, K and that statistic instead of storing P
 * (same page, "What does the backward pass do without P?"; "LLM flash
 * attention", aicassindra.com, section "End-to-end flow").
 *
 * Common conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and keeps no state between calls.
 *   - Layout: contiguous row-major [B, H, N, d] for q, k, v, o, dO, dq, dk,
 *     dv (bfloat16, 2 bytes per element); contiguous [B, H, N] float32 for
 *     lse.  Base pointers must be 16-byte aligned.
 *   - d must be 128.  B, H, N >= 0, B*H*N*d below 2^31 and N below 2^24 - 256;
 *     when any of B,
 *     H, N is 0 there is nothing to compute and the call returns FA_OK
 *     without touching any pointer.
 *   - scale must be finite and > 0 (the scores are scale * q . k).
 *   - causal: 0 = every key visible; 1 = key j visible to query i iff j <= i.
 *   - Inputs are read only.  Outputs are fully overwritten, never accumulated
 *     into.  No output may alias an input or another output (not detected).
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     enqueue work and return at once; kernel faults surface at the caller's
 *     next synchronisation.
 *   - Return value: FA_OK (0) or an fa_status code.  Argument errors are
 *     detected before anything is launched; nothing is printed, no exception
 *     or abort crosses the ABI.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, bad scale/causal */
  FA_ERR_UNSUPPORTED = 2,  /* d != 128, misaligned pointer, size overflow */
  FA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  FA_ERR_HIP = 4           /* the HIP runtime rejected a launch */
} fa_status;

/*
 * Forward pass.
 *   q, k, v : [B,H,N,d] bf16 inputs.
 *   o       : [B,H,N,d] bf16 output, O = softmax(scale Q K^T) V, rounded to
 *             nearest even from float32 accumulators.
 *   lse     : [B,H,N] float32 output, L_i = m_i + ln(l_i): the natural
 *             log-sum-exp of row i of the scaled (and masked) scores
 *             ("Interrogating the GPU, part 5", backward section, definition
 *             of L_i).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Bytes of device workspace the backward pass needs for these sizes:
 * 2*B*H*N float32 (rounded up to 256 bytes), laid out as [D | L*log2(e)],
 * with D_i = sum_k dO_ik O_ik and L the forward's log-sum-exp.  Returns 0
 * when the sizes are invalid or empty.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, int causal);

/*
 * Backward pass: gradients of the forward above.
 *   q, k, v, o, dO : [B,H,N,d] bf16 inputs (o is fa_fwd's output).
 *   lse            : [B,H,N] float32, fa_fwd's log-sum-exp output.
 *   dq, dk, dv     : [B,H,N,d] bf16 outputs.
 *   workspace      : device buffer of at least fa_bwd_workspace_size() bytes,
 *                    16-byte aligned; its contents on entry are ignored and
 *                    on exit hold [D | L*log2(e)].
 * P is recomputed tile by tile as exp(scale q.k - L_i); with
 * dP = dO V^T and D_i = sum_k dO_ik O_ik, dS = P o (dP - D), and
 * dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q ("Interrogating the GPU,
 * part 5", section "What does the backward pass do without P?"; dQ and dK
 * by the chain rule).  Deterministic: no atomics, so repeated calls give
 * bitwise identical gradients.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three stages fa_bwd runs, in order, on one stream.  Each is exposed so a
 * caller can schedule or time them separately; running all three with the
 * same arguments and workspace is exactly fa_bwd.  Arguments as for fa_bwd.
 *
 * fa_bwd_preprocess: fills the workspace with D_i = sum_k dO_ik O_ik, the row
 *   sum of dO o O that plays the role of delta in dS = P o (dP - delta)
 *   ("Interrogating the GPU, part 5", section "What does the backward pass do
 *   without P?"), and with L_i log2(e) for the exp2-based recomputation.
 * fa_bwd_dkdv: for each key block, recompute P = exp(scale q.k - L) over all
 *   visible queries and accumulate dV = P^T dO and dK = scale dS^T Q.
 * fa_bwd_dq: for each query block, recompute P and dS over all visible keys
 *   and accumulate dQ = scale dS K.
 * The last two read the workspace the first one wrote.
 */
int fa_bwd_preprocess(const void* o, const void* dO, const float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
              const void* workspace, size_t workspace_bytes, void* dq,
              int B, int H, int N, int d, float scale, int causal, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
