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
 *   - scale must be finite; any sign, and zero, is accepted (the scores are
 *     scale * q . k; scale = 0 gives uniform weights over the visible keys).
 *     The scaled scores are formed in float32, so |scale * q . k| must stay
 *     below 2^127 for the results to be finite.
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
  FA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, non-finite scale, bad causal */
  FA_ERR_UNSUPPORTED = 2,  /* d != 128, misaligned pointer, size overflow */
  FA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  FA_ERR_HIP = 4,          /* the HIP runtime rejected a launch */
  FA_ERR_TOO_LARGE = 5     /* fa_bwd_noalloc: B*H*N above FA_NOALLOC_MAX_ROWS */
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
 * The forward pass through its key-split kernel, whatever the sizes.  fa_fwd
 * runs it by itself when B * H * ceil(N / 256) is below 128 (below 256 when
 * causal), i.e. when one workgroup per 256 query rows leaves most of the
 * GPU's 256 CUs idle (few heads and a short sequence; "Interrogating the GPU,
 * part 5", FlashAttention-2 section: batch x heads alone does not fill the
 * GPU).  A workgroup then owns 32 query
 * rows and its four wavefronts each run the online softmax over a quarter of
 * the key tiles; the four partial results are merged with the same rescale
 * rule the online softmax uses between tiles.  Arguments, outputs and error
 * behaviour exactly as for fa_fwd; exported so that either kernel can be
 * tested and timed on any sizes.
 */
int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * The forward pass scheduled as a ping-pong ("Interrogating the GPU, part 5",
 * section "What did FlashAttention-3 do with Hopper?"; "FlashAttention
 * versions", section "FlashAttention-3": one group's softmax runs on the
 * vector units while the other group's matrix products run).  The row-block
 * tiling of fa_fwd (256 query rows per workgroup, 64-key tiles, eight
 * wavefronts, two per SIMD), with waves w and w + 4 of a SIMD alternating an
 * MFMA phase and a softmax phase one phase apart, so that one's matrix
 * products meet the other's exponentials.  Same arithmetic as fa_fwd's
 * row-block kernel (results equal to rounding order, not bitwise);
 * arguments, outputs and error behaviour as for fa_fwd.  Exported to measure
 * that schedule against fa_fwd's, whose two waves per SIMD interleave by
 * themselves.
 */
int fa_fwd_pingpong(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * The forward pass through its row-block kernel (whatever the sizes) with a
 * share of the exponentials evaluated in software on the FMA path instead of
 * the transcendental unit ("Interrogating the GPU, part 5", section "Why did
 * Blackwell need FlashAttention-4?": 2^x = 2^n 2^f with f in [0, 1) and 2^f
 * from the page's cubic, relative error about 1e-4).  software_share is how
 * many of each lane's 32 exponentials per 64-key tile take that path: 0, 8,
 * 16 or 32 (other values: FA_ERR_INVALID_ARG, before any launch).  With 0 the
 * results are bitwise those of the row-block kernel that fa_fwd runs for
 * large grids.  Other arguments, outputs and error behaviour as for fa_fwd;
 * the outputs differ from fa_fwd's by the cubic's error (LSE by about 1e-4).
 * On this GPU the transcendental unit is not the limit (an exponential costs
 * one instruction, the cubic ten), so fa_fwd keeps v_exp_f32; this entry
 * point exists to measure that.
 */
int fa_fwd_soft_exp2(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal, int software_share,
                     void* stream);

/*
 * Bytes of device workspace the backward pass needs for these sizes:
 * 2*B*H*N float32 (rounded up to 256 bytes), laid out as [-D | L*log2(e)],
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
 *                    on exit hold [-D | L*log2(e)].
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
 * The backward pass without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs, results
 * (bitwise those of fa_bwd) and error behaviour as fa_bwd, minus the
 * workspace.  It calls no allocator: the [-D | L*log2(e)] workspace lives in a
 * fixed array inside the library, FA_NOALLOC_SCRATCH_BYTES per GPU, which
 * each GPU the library runs on holds until the process ends.  Problems whose
 * workspace would not fit (B*H*N above FA_NOALLOC_MAX_ROWS) are rejected with
 * FA_ERR_TOO_LARGE before anything is launched.  All calls on one GPU share
 * that GPU's array: calls that may overlap on one GPU (different streams or
 * threads without ordering between them) race and must not be issued.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
#define FA_NOALLOC_MAX_ROWS (FA_NOALLOC_SCRATCH_BYTES / 8u)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Workspace bytes for fa_bwd_atomic_dq: the [-D | L*log2(e)] workspace of
 * fa_bwd padded to 256 bytes, then an fp32 dQ buffer of B*H*N*d floats.
 * Returns 0 when the sizes are invalid or empty.
 */
size_t fa_bwd_atomic_workspace_size(int B, int H, int N, int d, int causal);

/*
 * The backward pass with dQ fused into the dK/dV pass through fp32 atomics
 * ("LLM flash attention", section "End-to-end flow": each key block adds its
 * share of dQ_i = sum_j dS_ij K_j).  Four launches: the pre-pass (-D and
 * L*log2(e)), a clear of the fp32 dQ buffer, the fused kernel (128 keys per
 * workgroup: dK, dV, and dS K summed over the workgroup in LDS, then one
 * fp32 global atomic add per element and 32-query tile), and a conversion
 * of the buffer to bf16 dQ times the scale.  Same arguments, outputs and
 * tolerances as fa_bwd, with the workspace sized by
 * fa_bwd_atomic_workspace_size (its contents on entry are ignored); dK and
 * dV are deterministic, dQ is not bitwise reproducible (the order of the
 * atomic additions varies).  On this GPU it is slower than fa_bwd: the
 * atomic traffic alone outweighs the dQ kernel's two recomputed products,
 * which is why fa_bwd keeps the separate dQ kernel; exported to measure that.
 */
int fa_bwd_atomic_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int H, int N, int d, float scale, int causal,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The stages of the backward, each exposed so that a caller can schedule or
 * time them separately.  fa_bwd runs fa_bwd_dq, then fa_bwd_dkdv, on one
 * stream; running those two with the same arguments and workspace is exactly
 * fa_bwd.  Arguments as for fa_bwd.
 *
 * fa_bwd_dq: computes, for every query row, -D_i = -sum_k dO_ik O_ik (D plays
 *   the role of delta in dS = P o (dP - delta), "Interrogating the GPU,
 *   part 5", section "What does the backward pass do without P?"; stored
 *   negated because both gradient stages start their dP accumulations from
 *   it) and L_i log2(e) (for the exp2-based recomputation), writes them into
 *   the workspace as [-D | L*log2(e)], and for each query block recomputes P
 *   and dS over all visible keys and accumulates dQ = scale dS K.
 * fa_bwd_dkdv: for each key block, recomputes P = exp(scale q.k - L) and dS
 *   over all visible queries and accumulates dV = P^T dO and dK =
 *   scale dS^T Q; it reads the workspace that fa_bwd_dq (or
 *   fa_bwd_preprocess) wrote.
 * fa_bwd_preprocess: writes the same workspace contents as fa_bwd_dq, bit
 *   for bit, without computing dQ (for callers that need dK and dV alone).
 */
int fa_bwd_preprocess(const void* o, const void* dO, const float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* workspace, size_t workspace_bytes, void* dq,
              int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * FP8 forward with incoherent processing ("Interrogating the GPU, part 5:
 * FlashAttention", section "What did FlashAttention-3 do with Hopper?": keys
 * and values quantised per block after a random Hadamard rotation, which
 * spreads outliers across the block; "FlashAttention versions", section
 * "FlashAttention-3": block-level quantisation with incoherent processing).
 * An approximation of the forward above, with its own accuracy contract.
 *
 * With sigma a sign vector chosen by the caller (d float32 entries, each +1
 * or -1) and H the d x d Sylvester Hadamard matrix:
 *   X' = (X o sigma) H for X = Q, K, V, computed in float32 as a fast
 *   Walsh-Hadamard transform (stage s = 0..6 pairs entries i and i + 2^s,
 *   bit s of i clear, into (a + b, a - b));
 *   each block of 64 consecutive rows of a head (the last block may be
 *   shorter) gets the exponent e, the smallest integer with
 *   max|X'| <= 448 * 2^e (-127 for an all-zero block), and the codes
 *   E4M3(X' * 2^-e): OCP FP8 E4M3, round to nearest even;
 *   the forward then uses S = (scale / d) Q' K'^T, P rounded to E4M3 for the
 *   P V' product, and O = ((P V') H / d) o sigma.
 *
 * fa_fp8_quantize: x [B,H,N,d] bf16 -> codes and exps.
 *   layout FA_FP8_ROWS (0): codes [B,H,N,d] uint8, row-major (Q and K);
 *   layout FA_FP8_VT (1): codes [B,H,ceil(N/64),d,64] uint8: per 64-key tile,
 *     one 64-byte row per dimension; inside a row, block-local key r sits at
 *     32*((r>>2)&1) + 16*(r>>5) + 4*((r>>3)&3) + (r&3); keys past N are zero
 *     (V).
 *   exps: [B,H,ceil(N/64)] int32 block exponents.  signs: d float32 values,
 *   device memory.  fa_fp8_codes_size / fa_fp8_exps_size give the byte sizes
 *   (0 for invalid or empty sizes).
 * fa_fwd_fp8: q8 and k8 in FA_FP8_ROWS layout, v8 in FA_FP8_VT layout, with
 *   their exps and the same signs; o [B,H,N,d] bf16 and lse [B,H,N] float32
 *   as for fa_fwd (lse of the scores the FP8 path computes).
 * Accuracy (unit-variance inputs, d = 128): O within about 0.1 and LSE within
 * about 0.1 of exact attention; the E4M3 rounding of P dominates.  Shapes,
 * alignment, scale, causal, stream and error codes as for fa_fwd.
 */
enum { FA_FP8_ROWS = 0, FA_FP8_VT = 1 };
size_t fa_fp8_codes_size(int B, int H, int N, int d, int layout);
size_t fa_fp8_exps_size(int B, int H, int N, int d);
int fa_fp8_quantize(const void* x, const float* signs, void* codes, int* exps,
                    int B, int H, int N, int d, int layout, void* stream);
int fa_fwd_fp8(const void* q8, const int* qexp, const void* k8, const int* kexp,
               const void* v8, const int* vexp, const float* signs, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
