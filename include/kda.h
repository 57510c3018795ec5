/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked forward of bounded-decay KDA.
 *
 * The operator (delta-rule linear attention with a per-channel log-decay):
 *
 *   g_t   = g_min * sigmoid(a_t)                 per key channel, g_min < 0
 *   S_t   = S_{t-1} diag(exp g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   S_0 = 0
 *   o_t   = S_t q_t
 *
 * S is dv x dk (row = value channel, column = key channel).
 *
 * Sources: the bounded log-decay g = g_min * Sigmoid(.) with g_min = -5, which
 * keeps the inverse cumulative decay 1/Gamma representable inside any 16-token
 * tile so that every causal tile (diagonal and off-diagonal) is a dense matrix
 * product -- "Trillion-Scale MoE Multimodal Models: Practical Techniques for
 * Ultra-Long Context and Sparse Expert Architectures", sec. 3.1-3.3, and
 * "Breaking Through Trillion-Parameter Multimodal MoE: Key Innovations from
 * Ultra-Long Context to Extreme Sparsity", sec. 2.1 (which names the delta rule,
 * "Delta Net", and the unbounded Log(sigma(x)) form it replaces).  The chunked
 * recursion with a constant-size state: "Trillion-Parameter MoE Multimodal
 * Models: Engineering Long-Context and Sparse Expert Architectures", sec. 3.2.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    keeps no pointer after the call returns and never allocates device memory.
 *  - Tensors are contiguous, row-major:
 *      q, k, a : [B][H][T][dk]      v, out : [B][H][T][dv]      beta : [B][H][T]
 *      final_state : [B][H][dv][dk] float32, final_state[b][h][i][j] = S_T[i][j]
 *      G_out : [B][H][T][dk] float32
 *    Element type of q, k, v, a, beta, out is given by io_dtype (KDA_BF16 or
 *    KDA_FP32); state, accumulation and G_out are float32.
 *  - q, k, v, a, out, final_state, G_out and the workspace must be 16-byte
 *    aligned; beta must be aligned to its element size.  A pointer to an
 *    array with zero elements (T == 0) may be NULL.
 *  - Supported: dk, dv in {64, 128}; chunk in {16, 32, 64}; T % chunk == 0;
 *    1 <= B, H <= 65535; T >= 0; B*H*T*max(dk,dv) < 2^40.  Bounded mode needs a finite
 *    g_min with KDA_G_MIN_LOWEST <= g_min < 0 (below that bound the decay factors
 *    of a 16-token tile leave the range in which 16-bit operands keep their
 *    precision); the ablation mode ignores g_min.
 *  - Every argument is validated on the host before anything is launched; on a
 *    bad argument a negative kda_status is returned and nothing is launched.
 *    Work is enqueued asynchronously on `stream` (0 = the null stream); device
 *    faults surface at the caller's next synchronisation.  KDA_ERR_HIP reports
 *    a launch error (hipGetLastError) after enqueueing.
 *  - Outputs are fully overwritten, never accumulated.  out must not alias any
 *    input.  Results are bitwise reproducible run to run (no float atomics).
 *  - No global mutable state: calls from several host threads are safe.  The one
 *    exception is kda_chunk_fwd_noalloc, whose calls on one GPU share a static
 *    device array.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 8
/* The most negative g_min accepted: the constant the method fixes.  Inside a
 * 16-token tile the key operands of the diagonal sub-tile grow by up to
 * e^(15 |g_min|) and the row operands shrink by as much; at g_min = -5 both stay
 * e^12 inside the bf16/fp32 normal range (largest e^88.7, smallest normal
 * e^-87.3), so a row-operand component flushes only below 4.4e-6.  Closer to
 * the edge the shrunk row operands of a tile's last rows turn subnormal while
 * their products with the grown key operands are O(1) entries of M and A: with
 * every gate saturated, g_min = -5.6 already misses the bf16 tolerance. */
#define KDA_G_MIN_LOWEST (-5.0f)

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,      /* a required pointer is NULL                       */
    KDA_ERR_SHAPE = -2,     /* B, H, T, dk or dv unsupported, or T % chunk != 0 */
    KDA_ERR_DTYPE = -3,     /* io_dtype not KDA_BF16 / KDA_FP32                 */
    KDA_ERR_CHUNK = -4,     /* chunk not in {16, 32, 64}                        */
    KDA_ERR_GMIN = -5,      /* g_min not finite or outside [KDA_G_MIN_LOWEST,0) */
    KDA_ERR_WORKSPACE = -6, /* workspace NULL or smaller than required          */
    KDA_ERR_HIP = -7,       /* a HIP call or kernel launch failed               */
    KDA_ERR_ALIGN = -8,     /* a pointer is not aligned as required             */
    KDA_ERR_MODE = -9,      /* gate_mode unknown                                */
    KDA_ERR_SCRATCH = -10   /* kda_chunk_fwd_noalloc: the problem needs more than
                               KDA_NOALLOC_SCRATCH_BYTES of device scratch      */
} kda_status;

/* Bytes of device scratch that kda_chunk_fwd_noalloc works in: a static device array of the
 * library, one per GPU it runs on, held until the process ends. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)

typedef enum { KDA_BF16 = 0, KDA_FP32 = 1 } kda_dtype;

typedef enum {
    KDA_GATE_BOUNDED = 0,   /* g = g_min * sigmoid(a)   (the method)                     */
    KDA_GATE_LOGSIGMOID = 1 /* g = log sigmoid(a)       (unbounded form, ablation only)  */
} kda_gate_mode;

/* Version of this ABI (KDA_ABI_VERSION). */
int kda_abi_version(void);

/* Static, NUL-terminated description of a kda_status value. */
const char *kda_status_string(int status);

/* Bytes of device workspace kda_chunk_fwd needs for this problem (0 for an
 * invalid problem).  The workspace holds the per-chunk operands the chunk-
 * parallel stage hands to the sequential state stage and, when that stage cuts
 * each sequence into segments walked side by side (fewer than 256 heads; the
 * segments' affine state maps composed as in context-parallel prefill, third
 * page sec. 3), each segment's float32 end state and transition: 2 x 64 KiB
 * per segment and head at dk = dv = 128. */
size_t kda_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int io_dtype);

/* Gate and per-chunk prefix sum (first page sec. 3.2 / third page sec. 2.1 for
 * the gate; the cumulative decay of the chunked form, first page sec. 3.1):
 *   g[t][c] = g_min * sigmoid(a[t][c])      (gate_mode = KDA_GATE_BOUNDED)
 *   g[t][c] = log sigmoid(a[t][c])          (gate_mode = KDA_GATE_LOGSIGMOID)
 *   G_out[t][c] = sum of g[s][c] over s from the start of t's chunk to t (inclusive),
 * natural-log units, float32.  Only a and G_out are touched. */
int kda_gate_cumsum(const void *a, float g_min, int chunk, int B, int H, int T, int dk,
                    int io_dtype, int gate_mode, float *G_out, hipStream_t stream);

/* Chunked forward: out[b][h][t] = o_t for every token; if final_state is not
 * NULL it receives S_T.  q, k and v may have any magnitude in the range of the
 * I/O type: every 16-bit operand inside the kernels is block-scaled by a power of
 * two taken from its own block, so scaling v (or q) by 2^e scales out by exactly
 * 2^e.  The delta rule's usual convention, L2-normalised q and k, is not needed;
 * the recurrence itself stays bounded only while beta |k|^2 <= 2 (each step
 * I - beta k k^T is then a contraction).  workspace: device buffer of at least
 * kda_chunk_fwd_workspace_bytes(...) bytes, contents undefined on entry and on
 * return; it must not overlap any other argument. */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *beta,
                  float g_min, int chunk, int B, int H, int T, int dk, int dv, int io_dtype,
                  void *out, float *final_state, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* As kda_chunk_fwd, plus the gate mode (KDA_GATE_LOGSIGMOID is the unbounded
 * form the pages replace, kept for the ablation), optional device counters
 * (NULL to skip; else a device pointer to 2 unsigned 64-bit integers that are
 * ADDED to, so zero them first):
 *   nonfinite_counts[0] += number of Gamma-scaled key operands of the diagonal
 *                          16-token tiles that are +-inf or NaN after rounding
 *                          to the operand type (the only scaled operands whose
 *                          scale factor exceeds 1);
 *   nonfinite_counts[1] += number of outputs that are +-inf or NaN,
 * and an optional initial state (NULL: S_0 = 0; else a device pointer to
 * [B][H][dv][dk] float32 in the layout of final_state), so that a sequence can
 * be processed in pieces, each continuing from the previous piece's final
 * state (the constant-size state carried across a long context, second page
 * sec. 3.2; context-parallel prefill, third page sec. 3).  initial_state may
 * be the same array as final_state (each part of the state is read before it
 * is overwritten); any other overlap with an argument is not allowed. */
int kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const void *a, const void *beta,
                     float g_min, int chunk, int B, int H, int T, int dk, int dv, int io_dtype,
                     void *out, float *final_state, void *workspace, size_t workspace_bytes,
                     hipStream_t stream, int gate_mode, unsigned long long *nonfinite_counts,
                     const float *initial_state);

/* The two stages kda_chunk_fwd_ex runs, in order, exposed so a caller can
 * time them separately or schedule other work between them.  Same arguments
 * and rules as kda_chunk_fwd_ex; the workspace carries everything from the
 * first call to the second and must not be touched in between.
 *
 * kda_chunk_intra -- chunk-parallel stage (one work-group per chunk and head):
 *   gate and within-chunk prefix sum G; the Gamma-scaled causal 16x16 sub-tiles
 *   of M = (Q K^T masked) and A = (diag(beta) K K^T strictly masked), all dense
 *   products with each 16-token row tile referenced to its own first row
 *   (first page sec. 3.1-3.3, third page sec. 2.1); the delta rule's WY/UT
 *   transform T = (I + A)^-1, W = T diag(beta) K e^G, U~ = T diag(beta) V; and
 *   Q e^G, K e^(G_last - G), e^(G_last).  Writes only the workspace and, when
 *   given, nonfinite_counts[0].
 * kda_chunk_state -- sequential stage over the chunks of each head (the
 *   constant-size state carried chunk to chunk, second page sec. 3.2), fused
 *   with the output combine: U = U~ - W S^T, O = Q e^G S^T + M U,
 *   S^T <- diag(e^(G_last)) S^T + (K e^(G_last - G))^T U.  Reads the workspace,
 *   writes out, final_state (if not NULL) and, when given, nonfinite_counts[1]. */
int kda_chunk_intra(const void *q, const void *k, const void *v, const void *a, const void *beta,
                    float g_min, int chunk, int B, int H, int T, int dk, int dv, int io_dtype,
                    void *workspace, size_t workspace_bytes, hipStream_t stream, int gate_mode,
                    unsigned long long *nonfinite_counts);
int kda_chunk_state(const void *workspace, size_t workspace_bytes, int chunk, int B, int H, int T,
                    int dk, int dv, int io_dtype, void *out, float *final_state, hipStream_t stream,
                    unsigned long long *nonfinite_counts, const float *initial_state);

/* As kda_chunk_fwd_ex, with the gate pre-activation formed inside the chunk
 * kernel from a rank-`rank` factor instead of being read from an a tensor:
 *   a[b][h][t][c] = exp(A_log[h][c]) * sum_j h[b][t][j] * z[h][c][j]
 * then g = g_min * sigmoid(a) as before (the gate e^A h z of the first page,
 * sec. 3.2, with h the per-token low-rank gate input shared by all heads and z
 * each head's map from it to the key channels).  The a tensor (dk values per
 * token and head) is never materialised; h adds rank values per token.
 *   h : [B][T][rank] (io_dtype)   z : [H][dk][rank] (io_dtype)   A_log : [H][dk] float32
 * rank is 16, 32, 64 or 128.  h and z must be 16-byte aligned,
 * A_log 4-byte aligned.  Workspace as kda_chunk_fwd_workspace_bytes(...).
 * Everything else as kda_chunk_fwd_ex. */
int kda_chunk_fwd_lowrank(const void *q, const void *k, const void *v, const void *h, const void *z,
                          const float *A_log, const void *beta, float g_min, int chunk, int B, int H,
                          int T, int dk, int dv, int rank, int io_dtype, void *out, float *final_state,
                          void *workspace, size_t workspace_bytes, hipStream_t stream, int gate_mode,
                          unsigned long long *nonfinite_counts, const float *initial_state);

/* Packed documents: N documents of any lengths laid end to end in one token
 * stream per head, each run through the recurrence on its own -- from its own
 * initial state, nothing carried across a boundary -- as when many short
 * documents are packed into one long training sequence (third page, sec. 3,
 * the 256K-1M phase).  Document i is tokens [cu_seqlens[i], cu_seqlens[i+1])
 * of the stream:
 *   q, k, a : [H][T][dk]     v, out : [H][T][dv]     beta : [H][T]   (io_dtype)
 *   cu_seqlens : DEVICE pointer to N + 1 int32, nondecreasing, cu_seqlens[0] = 0,
 *             cu_seqlens[N] = T (document lengths need not be multiples of chunk)
 *   initial_state, final_state : [N][H][dv][dk] float32 (NULL: zero / not wanted),
 *             indexed by document; they may be the same array
 * T is the stream length and need not be a multiple of chunk; N >= 1.
 * cu_seqlens is only read on the device (nothing synchronises with the host):
 * its values are clipped to [0, T] and made nondecreasing there, so contents
 * outside the contract cannot make a kernel access memory outside the
 * arguments; they give unspecified results, and out rows of tokens that no
 * document covers are not written.  workspace: at least
 * kda_chunk_fwd_varlen_workspace_bytes(N, H, T, dk, dv, chunk, io_dtype) bytes
 * (0 for an invalid problem).  Everything else (dtypes, g_min, gate_mode,
 * nonfinite_counts, alignment, validation, asynchrony) as kda_chunk_fwd_ex;
 * cu_seqlens must be 4-byte aligned. */
size_t kda_chunk_fwd_varlen_workspace_bytes(int N, int H, int T, int dk, int dv, int chunk, int io_dtype);
int kda_chunk_fwd_varlen(const void *q, const void *k, const void *v, const void *a, const void *beta,
                         float g_min, int chunk, const int *cu_seqlens, int N, int H, int T, int dk,
                         int dv, int io_dtype, void *out, float *final_state, void *workspace,
                         size_t workspace_bytes, hipStream_t stream, int gate_mode,
                         unsigned long long *nonfinite_counts, const float *initial_state);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kda_chunk_fwd_ex without a workspace argument.  It
 * allocates nothing (no hipMalloc, hipFree, memset or copy node): its chunk records go to a
 * static device array of KDA_NOALLOC_SCRATCH_BYTES, one per GPU, and the sequence is processed
 * in windows of whole chunks whose records fit there, the state carried from window to window
 * (in final_state when given, else in the same array).  Results match kda_chunk_fwd_ex within
 * the parity tolerance (the state is re-scaled at window boundaries, so not bit for bit).
 * Arguments, layouts, validation and asynchrony as kda_chunk_fwd_ex.  Returns KDA_ERR_SCRATCH,
 * before anything is launched, when one chunk of every head, plus the state if final_state is
 * NULL, does not fit: B*H*(record bytes of one chunk) + (final_state ? 0 : B*H*dv*dk*4) >
 * KDA_NOALLOC_SCRATCH_BYTES (about 1,600 heads at dk = dv = 128, chunk 64, bf16).  Every call on
 * one GPU uses that GPU's one array: calls that overlap in time on the same GPU (other streams,
 * other host threads) race and must be ordered by the caller. */
int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *a, const void *beta,
                          float g_min, int chunk, int B, int H, int T, int dk, int dv, int io_dtype,
                          void *out, float *final_state, hipStream_t stream, int gate_mode,
                          unsigned long long *nonfinite_counts, const float *initial_state);

/* Backward pass: the gradients of L = sum_t dout_t . o_t + <dfinal_state, S_T>
 * with respect to q, k, v, a, beta and the initial state, for training (the
 * third page, sec. 2.1: the bounded parameterisation changes the operator, not
 * the training scripts above it, so the operator supplies exactly these).
 * Inputs as kda_chunk_fwd_ex (B, H, T, dk, dv, io_dtype, gate_mode, g_min,
 * initial_state nullable), plus
 *   dout         : [B][H][T][dv] (io_dtype), the gradient of out
 *   dfinal_state : [B][H][dv][dk] float32 or NULL (zero)
 * Outputs, float32 whatever io_dtype, fully overwritten:
 *   dq_out, dk_out, da_out : [B][H][T][dk]   dv_out : [B][H][T][dv]   dbeta_out : [B][H][T]
 *   dinitial_state : [B][H][dv][dk] or NULL (not wanted)
 * da_out is the gradient of the gate pre-activation a (through g = g_min sigmoid(a),
 * or log sigmoid(a) in the ablation mode).  The backward works on 16-token
 * chunks whatever chunk the forward used (the gradients do not depend on it):
 * T % 16 == 0, and B*H <= 65535.  workspace: kda_chunk_bwd_workspace_bytes(...) bytes (the
 * recomputed chunk records and two float32 states per 16-token chunk and head,
 * B*H*T/16 * (record + 2*dk*dv*4) bytes; 0 for an invalid problem).  No output
 * may alias an input.  Validation, alignment (16 bytes; beta: element size,
 * dbeta: 4) and asynchrony as above.  Part of the work (the reverse pass over the chunks)
 * runs on a second stream the library makes once per GPU (default priority), forked from
 * stream and joined back to it with events inside the call: work enqueued on stream after
 * the call still starts only once all of it is done. */
size_t kda_chunk_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int io_dtype);
int kda_chunk_bwd(const void *q, const void *k, const void *v, const void *a, const void *beta,
                  float g_min, int B, int H, int T, int dk, int dv, int io_dtype, int gate_mode,
                  const float *initial_state, const void *dout, const float *dfinal_state,
                  float *dq_out, float *dk_out, float *dv_out, float *da_out, float *dbeta_out,
                  float *dinitial_state, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* One token of the recurrence per (batch, head), the state updated in place
 * (decoding after a prefill; the constant-size state of the second page,
 * sec. 3.2; the gate as in kda_gate_cumsum):
 *   S~ = S diag(exp g),  S <- S~ + beta (v - S~ k) k^T,  out = S q.
 *   q, k, a : [B][H][dk]     v, out : [B][H][dv]     beta : [B][H]   (io_dtype)
 *   state   : [B][H][dv][dk] float32, S[i][j] (i = value, j = key), read and
 *             overwritten; it must not overlap any other argument.
 * Same rules as above for dtypes, g_min, gate_mode, alignment (16 bytes;
 * beta: element size), validation and asynchrony.  Supported: dk, dv in
 * {64, 128}; B, H >= 1. */
int kda_decode_step(const void *q, const void *k, const void *v, const void *a, const void *beta,
                    float g_min, int B, int H, int dk, int dv, int io_dtype, int gate_mode,
                    float *state, void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
