/*
 * attn.h - C ABI of libattn.so: exact blockwise attention forward and the (O, lse) merge on MI355X (gfx950).
 *
 * What is computed.  For every batch b and head h, with Q [N_q, d], K and V [N_kv, d]:
 *     S = scale * Q K^T,   P = row-softmax(S) over the visible keys,   O = P V,
 *     LSE_i = ln sum_{j visible} exp(S_ij).
 * This is the attention of "FlashAttention by hand" (paragraph on the three standard steps), computed the
 * way that page describes it (paragraphs on online softmax, the per-tile flow, rescaling and the final
 * division): key/value tiles stream through on-chip memory while each query row keeps a running max, a
 * running denominator and an unnormalised output; the N_q x N_kv score matrix is never written to memory.
 * The merge combines two partial results over disjoint key sets, the associative step of the
 * "ATTENTION2D" explainer (sections 2 and 3) that Ring Attention ("Ring Attention with Blockwise Parallel
 * Transformers" explainer, section 3) needs when key/value blocks arrive one after another.
 *
 * Conventions that hold for every entry point.
 *   Layout     Q, K, V, O are [B, H, N, d] row-major (d fastest, contiguous); LSE is [B, H, N_q] fp32.
 *   Causal     bottom-right aligned ("HOF SWIFT Attention", section 3, Transform stage, names causal
 *              masking without fixing the alignment): key j is visible to query i iff j <= i + offset,
 *              where offset = N_kv - N_q unless given explicitly.  Non-causal: every key is visible.
 *   Empty row  a query with no visible key gets O = 0 and LSE = -inf (the identity of the merge).
 *   LSE        natural log, includes the scale.
 *   Dtypes     ATTN_BF16: Q, K, V in bf16, fp32 accumulation and statistics, O rounded to bf16 (RNE);
 *              ATTN_F32: fp32 everywhere.  The input dtype picks the kernel; d in {64, 128} for bf16,
 *              1..256 for fp32.
 *   Ownership  the caller allocates and owns every buffer (device memory), including the chunked
 *              workspace; the library never allocates device memory and keeps no per-call state.
 *   Device     every device buffer and stream of a call belongs to the calling thread's current HIP
 *              device (hipSetDevice), where the kernels launch; the library keeps one set of launch
 *              settings per device.
 *   Streams    every call enqueues on `hip_stream` (a hipStream_t; NULL = the null stream) and returns
 *              without synchronising.  Faults inside kernels surface at the caller's next synchronise.
 *              With the environment variable ATTN_DEBUG=1 every launch is followed by a synchronise and
 *              an error check.
 *   Errors     the return value is an attn_status.  Every argument is validated before any HIP call, so
 *              a non-zero status means nothing was enqueued (except ATTN_ERR_HIP, reported after a failed
 *              launch).  attn_strerror() names a status; attn_last_error() describes the last failure on
 *              the calling thread.
 *   Aliasing   O and LSE must not overlap Q, K, V, each other, or the workspace.
 *   Sizes      B, H, N_q, N_kv >= 1; element offsets are 64-bit.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL_PTR = 1,           /* a required pointer is NULL */
    ATTN_ERR_BAD_SHAPE = 2,          /* B, H, N_q, N_kv, rows or P out of range, or a stride too small;
                                        also any array that would span 2^56 bytes or more.
                                        Launch limits: ceil(N_q/128)*B*H (bf16) or ceil(N_q/64)*B*H (fp32)
                                        below 2^31-8; bf16 K of one head and launch below 2^31 bytes, i.e.
                                        N_kv <= 8,388,607 at d = 128 and 16,777,215 at d = 64 (in the
                                        chunked modes per chunk: ceil(N_kv/P)) */
    ATTN_ERR_UNSUPPORTED_D = 3,      /* head dimension not supported for this dtype */
    ATTN_ERR_BAD_DTYPE = 4,          /* unknown dtype or unsupported dtype combination */
    ATTN_ERR_BAD_SCALE = 5,          /* scale is NaN or infinite */
    ATTN_ERR_WORKSPACE_TOO_SMALL = 6,/* chunked mode: workspace NULL or smaller than required */
    ATTN_ERR_BAD_ALIAS = 7,          /* outputs overlap inputs (or each other) where that is not allowed */
    ATTN_ERR_HIP = 8,                /* a HIP launch or runtime call failed */
    ATTN_ERR_MISALIGNED = 9          /* a pointer or stride is not aligned as the kernel needs (bf16: 16 bytes
                                        for Q, K, V, O and head strides; otherwise the element size) */
} attn_status;

/*
 * attn_fwd - exact attention forward, one pass over all keys.
 *   Q [B,H,N_q,d], K and V [B,H,N_kv,d] in `dtype`; O [B,H,N_q,d] in `dtype`; LSE [B,H,N_q] fp32.
 *   causal: 0 or 1 (offset N_kv - N_q).  scale: any finite float (1/sqrt(d) is the usual choice).
 * Source: "FlashAttention by hand", paragraphs on fused tiled attention, online softmax, the per-tile flow,
 * rescaling and the single final division.
 */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
             int B, int H, int N_q, int N_kv, int d, int causal, float scale,
             attn_dtype dtype, void* hip_stream);

/*
 * attn_fwd_ex - attn_fwd over a key range of a larger key/value tensor, with an explicit causal offset
 * and output dtype.  This is one chunk of the chunked mode, and one device's step of a ring.
 *   K, V            point at the first key of the range in head (0,0);
 *   kv_head_stride  elements between consecutive (b,h) heads of K and V (0 means N_kv*d, contiguous);
 *   causal_offset   key j of the range is visible to query i iff j <= i + causal_offset (when causal);
 *   out_dtype       dtype of O: ATTN_F32 (partials to be merged) or the input dtype.
 * Source: "Ring Attention with Blockwise Parallel Transformers" explainer, section 3 (blockwise
 * computation over key/value blocks), and "FlashAttention by hand" as for attn_fwd.
 */
int attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE,
                int B, int H, int N_q, int N_kv, int d, int causal, float scale,
                long long causal_offset, long long kv_head_stride,
                attn_dtype in_dtype, attn_dtype out_dtype, void* hip_stream);

/*
 * attn_fwd_acc - attn_fwd_ex folded into a running partial result in the same launch:
 *     (O, LSE) = merge((O_acc, lse_acc), attention of Q against this key range)
 * with the merge of attn_merge.  The kernel's epilogue reads the partial row by row and writes the merged
 * row, so no separate merge pass and no partial of this range ever reaches memory.
 *   O_acc [B,H,N_q,d] and lse_acc [B,H,N_q] fp32 hold the result over the keys seen so far (a row with
 *   lse_acc = -inf is empty); the other arguments are those of attn_fwd_ex.  O is fp32 or the input dtype.
 *   In place is allowed: O == O_acc (with an fp32 O) and LSE == lse_acc; any other overlap between O, LSE,
 *   O_acc, lse_acc, Q, K and V is ATTN_ERR_BAD_ALIAS.  O_acc must be 16-byte aligned for bf16 inputs.
 * Source: "ATTENTION2D" explainer, sections 2 and 3 (partial statistics combined as they arrive), applied
 * at the end of each key range of "Ring Attention with Blockwise Parallel Transformers", section 3.
 */
int attn_fwd_acc(const void* Q, const void* K, const void* V, const float* O_acc, const float* lse_acc,
                 void* O, float* LSE, int B, int H, int N_q, int N_kv, int d, int causal, float scale,
                 long long causal_offset, long long kv_head_stride,
                 attn_dtype in_dtype, attn_dtype out_dtype, void* hip_stream);

/*
 * attn_merge - combine two partial results over disjoint key sets, row by row:
 *     M = max(lse_a, lse_b);  w_x = exp(lse_x - M);  O = (w_a O_a + w_b O_b) / (w_a + w_b);
 *     lse = M + ln(w_a + w_b);  rows with M = -inf give (0, -inf).
 *   O_a, O_b [rows, d] in in_dtype; lse_a, lse_b, lse [rows] fp32; O [rows, d] in out_dtype.
 *   In place is allowed when O == O_a (or O_b) and in_dtype == out_dtype, and lse == lse_a (or lse_b);
 *   any other overlap is ATTN_ERR_BAD_ALIAS.  d >= 1.
 * Source: "ATTENTION2D" explainer, sections 2 and 3 (partial statistics combined by commutativity and
 * associativity); the rescale rule is the one of "FlashAttention by hand", paragraph on rescaling.
 */
int attn_merge(const void* O_a, const float* lse_a, const void* O_b, const float* lse_b,
               void* O, float* lse, long long rows, int d,
               attn_dtype in_dtype, attn_dtype out_dtype, void* hip_stream);

/*
 * attn_fwd_chunked_workspace_bytes - device workspace attn_fwd_chunked needs: one fp32 partial output
 * [B,H,N_q,d] and one fp32 lse row [B,H,N_q], each 256-byte aligned; 0 when P == 1.
 * Returns 0 as well for invalid arguments (attn_fwd_chunked reports those).
 */
size_t attn_fwd_chunked_workspace_bytes(int B, int H, int N_q, int d, int P);

/*
 * attn_fwd_chunked - the keys are cut into P contiguous chunks, chunk p covering
 * [floor(p*N_kv/P), floor((p+1)*N_kv/P)), and folded left to right: the first chunk is attended with
 * attn_fwd_ex into an fp32 partial in the workspace, every later one with attn_fwd_acc (in place in the
 * workspace, the last one writing O in `dtype` and LSE).  Chunks that are empty or entirely in the causal
 * future are skipped (they are the merge identity).  Result: equal to attn_fwd up to rounding.  P >= 1
 * (P > N_kv is allowed).  Everything is enqueued on one stream.
 * Source: "Ring Attention with Blockwise Parallel Transformers" explainer, section 3 (key/value blocks
 * visited one after another), and "ATTENTION2D" explainer, section 3 (staged combination).
 */
int attn_fwd_chunked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int H, int N_q, int N_kv, int d, int causal, float scale, int P,
                     attn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * attn_fwd_chunked_noalloc - attn_fwd_chunked without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  The
 * running fp32 partial lives in a fixed array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on, from the first call on that device until the process ends; the call itself allocates
 * nothing.  The arguments, chunks, kernels and result are those of attn_fwd_chunked (bit for bit), and
 * attn_fwd_chunked_workspace_bytes(B, H, N_q, d, P) must not exceed ATTN_NOALLOC_SCRATCH_BYTES (B*H*N_q up
 * to 130,055 at d = 128 and 258,111 at d = 64), else ATTN_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued.  All calls on one device share that array and it keeps the last call's contents: calls that
 * overlap in time on one device (other streams, other threads) race, so the caller orders them (one stream,
 * or events).  P == 1 does not touch it.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int attn_fwd_chunked_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int N_q, int N_kv, int d, int causal, float scale, int P,
                             attn_dtype dtype, void* hip_stream);

/*
 * attn_fwd_streamed_workspace_bytes - device workspace attn_fwd_streamed needs: the fp32 partial output
 * [B,H,N_q,d] and lse [B,H,N_q] of attn_fwd_chunked, plus two staging slots, each holding the K and the V
 * rows of one chunk for every (b, h) ([B*H, ceil(N_kv/P), d] in `dtype`); every piece 256-byte aligned.
 * Returns 0 for invalid arguments (attn_fwd_streamed reports those).
 */
size_t attn_fwd_streamed_workspace_bytes(int B, int H, int N_q, int N_kv, int d, int P, attn_dtype dtype);

/*
 * attn_fwd_streamed - attn_fwd_chunked with K and V in host memory: the chunks are copied to the device
 * one after another on `copy_stream` into two staging slots of the workspace, and chunk p+1 is copied
 * while chunk p is attended on `hip_stream`.  Q, O, LSE and the workspace are device memory; K_host and
 * V_host are host memory laid out [B,H,N_kv,d] (page-locked, e.g. from hipHostMalloc, for the copies to
 * overlap the computation; pageable memory gives the same result, serialised).  The chunks, their order,
 * the skipped chunks and the kernels are those of attn_fwd_chunked with the same P, so O and LSE equal its
 * result bit for bit.  Every launch and copy is enqueued and the call returns without synchronising;
 * the first copies wait for everything enqueued on `hip_stream` before the call (so back-to-back calls may
 * share one workspace and one copy stream), `hip_stream` waits for each chunk's copy, and when its work is
 * done every copy is done.  The caller keeps
 * K_host, V_host and the workspace alive until then.  The two streams must differ (NULL is the
 * default stream; a non-blocking copy stream keeps the copies independent of it).
 * Errors: those of attn_fwd_chunked (the workspace must not overlap Q, O or LSE), ATTN_ERR_BAD_ALIAS for equal
 * streams, ATTN_ERR_HIP for a failed copy, event or launch (work enqueued before it stays enqueued).
 * Source: "Ring Attention with Blockwise Parallel Transformers" explainer, section 3 (the next block's keys
 * and values arrive while the current block is computed) and section 4 (no added time when a transfer is
 * shorter than a block's computation).
 */
int attn_fwd_streamed(const void* Q, const void* K_host, const void* V_host, void* O, float* LSE,
                      int B, int H, int N_q, int N_kv, int d, int causal, float scale, int P,
                      attn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream,
                      void* copy_stream);

/*
 * Blockwise feed-forward, the other half of a blockwise transformer block ("Ring Attention with Blockwise
 * Parallel Transformers" explainer, section 3: the sequence is cut into contiguous blocks and
 * self-attention and the feedforward are applied block by block).  The page names the standard feedforward
 * without defining it; this computes, for every row x of X,
 *     FFN(x) = act(x W1^T + b1) W2^T + b2,     act = GELU (x * Phi(x), the exact erf form) or ReLU,
 * taking the rows in contiguous blocks of `block` rows (the last one ragged), so the hidden activations
 * exist for one block at a time, in the caller's workspace.
 *   X [M, d_model] bf16; W1 [d_ff, d_model] bf16 and W2 [d_model, d_ff] bf16 (the [out, in] layout of a
 *   linear layer); b1 [d_ff] and b2 [d_model] fp32, or NULL for none; Y [M, d_model] bf16.
 *   Each block is two bf16 GEMMs with fp32 accumulation on the matrix cores; the hidden block is rounded
 *   to bf16 between them (bias and activation applied in fp32 before the rounding).
 *   d_model and d_ff: positive multiples of 64.  A row block, its hidden block and each weight must stay
 *   below 2^31 bytes.  X, W1, W2, Y, b1, b2 and the workspace: 16-byte aligned.
 *   The workspace holds min(block, M) * d_ff bf16 values (attn_ffn_workspace_bytes, which returns 0 for
 *   non-positive arguments); it is overwritten.
 *   Y must not overlap any input or the workspace.  Enqueued on hip_stream like every call here.
 */
typedef enum { ATTN_ACT_NONE = 0, ATTN_ACT_RELU = 1, ATTN_ACT_GELU = 2 } attn_act;

size_t attn_ffn_workspace_bytes(long long M, int d_ff, long long block);
int attn_ffn_blockwise(const void* X, const void* W1, const float* b1, const void* W2, const float* b2, void* Y,
                       long long M, int d_model, int d_ff, long long block, attn_act act,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* attn_strerror - a static string naming a status code. */
const char* attn_strerror(int status);

/* attn_last_error - a description of the last failure on the calling thread ("" if none). */
const char* attn_last_error(void);

/*
 * Launch timing.  attn_timing_enable(1) makes every kernel launch and chunk copy of the library record a
 * pair of HIP events on its stream (kind 0 = attention forward kernel, 1 = merge kernel, 2 = the K and V
 * copy of one chunk in attn_fwd_streamed, 3 = a GEMM of attn_ffn_blockwise); attn_timing_read synchronises
 * those events, returns per-kind counts and summed durations in milliseconds (arrays of 4), and clears the
 * record.  attn_timing_enable(0)
 * stops recording.  Used by the benchmark to time the work on the stream it runs on; off by default.
 * Returns ATTN_ERR_HIP if an event call fails.
 */
int attn_timing_enable(int on);
int attn_timing_read(long long counts[4], double total_ms[4]);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
