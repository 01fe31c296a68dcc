/*
 * sqa.h - C ABI of libsqa, the Sparse Query Attention forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is defined in "Sparse Query Attention (SQA): A Computationally
 * Efficient Attention Mechanism with Query Heads Reduction" (arXiv 2510.01817,
 * abstract) and in the ReactiveAI/GQA-Ref-Micro and ReactiveAI/xSMQAT-m model
 * cards (descriptions). SQA is grouped-query attention with fewer query heads:
 *
 *   Q = X Wq  (H_q heads)   K = X Wk, V = X Wv  (H_kv heads), y = x W
 *   query head i reads key/value head floor(i / (H_q / H_kv))
 *   A_i = softmax(Q_i K^T / sqrt(d_head) [+ causal mask]) V     per head
 *   A = [A_0 | A_1 | ... | A_{H_q-1}]  (head-major columns)
 *   Y = A Wo
 *
 * d_head = d_model / H. H is the head count of the equally shaped MHA model,
 * and H_q <= H of those heads are used (the cards' "d/heads"). Causal means
 * that key c is visible to query r iff c <= r.
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a device pointer the caller owns. The buffers are
 *     contiguous, row-major and 16-byte aligned, with element type `dtype`
 *     (fp32 or bf16; one dtype for inputs, intermediates and output).
 *   - Work is enqueued on `stream` and runs asynchronously. The caller keeps
 *     the buffers alive until the stream has passed the call. The library
 *     retains no pointer after it returns.
 *   - Arguments are validated on the host before any HIP call. An invalid
 *     call returns a status, enqueues nothing and writes no buffer.
 *     sqa_last_error_message() names the failed check. Nothing is printed and
 *     no C++ exception crosses the ABI.
 *   - A kernel fault after a successful launch surfaces at the caller's next
 *     synchronisation, as for any HIP call.
 *   - Supported: d_head in {32, 64}; 1 <= H_kv <= H_q <= H; H_q % H_kv == 0;
 *     1 <= N <= SQA_MAX_N. A call with B*N == 0 is a no-op that returns SQA_OK.
 *   - Arithmetic: matrix products on the MFMA units with fp32 accumulation,
 *     softmax in fp32. Q, K, V, A and Y are each rounded once (to nearest,
 *     ties to even) to `dtype` when stored.
 *   - Calls on different streams may run concurrently. The library keeps one
 *     stream-ordered memory pool per device, and small workspaces per stream
 *     (see sqa_forward).
 */
#ifndef SQA_H
#define SQA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SQA_OK = 0,
  SQA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, inconsistent shape, aliasing */
  SQA_ERR_UNSUPPORTED = 2,   /* valid but not built: d_head not 32/64, unknown dtype, N too large */
  SQA_ERR_HIP = 3,           /* a HIP call failed (launch, pool, device query) */
  SQA_ERR_OUT_OF_MEMORY = 4  /* the workspace could not be allocated */
} sqa_status;

typedef enum { SQA_DTYPE_FP32 = 0, SQA_DTYPE_BF16 = 1 } sqa_dtype;

/* Largest sequence length accepted (keeps per-head offsets in 32 bits). */
#define SQA_MAX_N (1 << 24)

/*
 * sqa_forward - the whole SQA forward pass: projection, attention core and
 * output projection (the three steps of the definition above).
 *
 *   x   [B, N, d_model]        input tokens
 *   Wq  [d_model, H_q*d_head]  query projection, narrowed to the H_q used heads
 *   Wk  [d_model, H_kv*d_head] key projection
 *   Wv  [d_model, H_kv*d_head] value projection
 *   Wo  [H_q*d_head, d_model]  output projection, narrowed likewise
 *   out [B, N, d_model]        result Y; must not overlap any input
 *   causal: 0 or 1.
 *
 * Workspace: Q, K, V^T and A intermediates plus the two weight matrices
 * transposed, about elem_size * (B*Np*d_head*(H_q + 2*H_kv) + B*N*H_q*d_head
 * + d_model*d_head*(2*H_q + 2*H_kv)) bytes with Np = sqa_padded_length(N).
 * A workspace of up to SQA_STREAM_WORKSPACE_MAX bytes is kept per stream
 * between calls: taken on a stream's first call (or when a call needs more)
 * from a per-device stream-ordered memory pool and held until the process
 * ends; calls on one stream run in order and share it. A larger workspace is
 * taken from the pool (hipMallocFromPoolAsync) and returned to it
 * (hipFreeAsync) on `stream` by each call; the pool keeps freed memory for
 * reuse until the process ends. This holds for every entry point below that
 * needs a workspace.
 * Returns SQA_ERR_OUT_OF_MEMORY if the pool cannot supply the workspace.
 */
sqa_status sqa_forward(const void* x, const void* Wq, const void* Wk, const void* Wv,
                       const void* Wo, void* out, int64_t B, int64_t N, int64_t d_model,
                       int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head, int causal,
                       sqa_dtype dtype, hipStream_t stream);

/* Largest workspace that a call keeps with its stream (see sqa_forward). */
#define SQA_STREAM_WORKSPACE_MAX ((size_t)64 << 20)

/* Size of the fixed device array that sqa_forward_noalloc takes its workspace from. */
#define SQA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * sqa_forward_noalloc - sqa_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid allocation. Arguments, result and errors are those of sqa_forward,
 * and the result is bitwise the same (the same kernels run).
 *
 * The call allocates and frees nothing. Its workspace (Q, K, V^T, A and the
 * transposed weights, each rounded up to 256 bytes; see sqa_forward) comes
 * from one fixed device array of SQA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends. The first call on
 * a device looks the array's device address up (hipGetSymbolAddress with that
 * device current). A call whose workspace exceeds the array returns
 * SQA_ERR_UNSUPPORTED and enqueues nothing; with the headline head shape
 * (d_model 1024, H_q 8, H_kv 4, d_head 64, bf16) the limit is about 42k
 * tokens (B*N).
 *
 * The array keeps what the last call left in it; nothing in it needs to start
 * at zero (every region is written before it is read). Calls on one device
 * share the array: calls that may overlap in time on that device (different
 * streams without ordering between them) race and give wrong results. Calls
 * ordered on one stream are safe.
 */
sqa_status sqa_forward_noalloc(const void* x, const void* Wq, const void* Wk, const void* Wv,
                               const void* Wo, void* out, int64_t B, int64_t N, int64_t d_model,
                               int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head, int causal,
                               sqa_dtype dtype, hipStream_t stream);

/*
 * sqa_forward_varlen - sqa_forward over a batch of sequences of different
 * lengths, padded to a common N, as a training batch cut at a maximum sequence
 * length holds them (ReactiveAI/xSMQAT-m and ReactiveAI/GQA-Ref-Micro model
 * cards, training example).
 *
 *   lens  device array of B int32 values: sequence b is rows 0 .. lens[b]-1 of
 *         x[b]. Values outside [0, N] are clamped into it.
 *
 * Each sequence is one SQA forward over its own tokens: its keys end at
 * lens[b] (causal or not), whatever the padding rows of x hold. Rows t >= lens[b]
 * of out are written as zeros. Everything else (layouts, workspace, errors) is
 * as in sqa_forward. lens must be 4-byte aligned and must not overlap out;
 * SQA_ERR_INVALID_ARG if it is null (unless B*N == 0).
 */
sqa_status sqa_forward_varlen(const void* x, const void* Wq, const void* Wk, const void* Wv,
                              const void* Wo, void* out, const int32_t* lens, int64_t B, int64_t N,
                              int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv,
                              int64_t d_head, int causal, sqa_dtype dtype, hipStream_t stream);

/*
 * Autoregressive inference with a key/value cache. The model cards generate
 * text token by token (ReactiveAI/xSMQAT-m and ReactiveAI/GQA-Ref-Micro,
 * inference example). The caches are caller-owned device buffers
 *   k_cache, v_cache [B, H_kv, N_max, d_head]  (dtype; row t = token t)
 * with 1 <= N_max <= SQA_MAX_N. They must not overlap each other, the inputs
 * or out.
 *
 * sqa_prefill - sqa_forward with causal = 1 over x [B, N, d_model]
 * (N <= N_max), which also writes the keys and values of tokens 0..N-1 to rows
 * 0..N-1 of the caches. Rows N.. are not touched.
 */
sqa_status sqa_prefill(const void* x, const void* Wq, const void* Wk, const void* Wv,
                       const void* Wo, void* out, void* k_cache, void* v_cache, int64_t B,
                       int64_t N, int64_t N_max, int64_t d_model, int64_t H, int64_t H_q,
                       int64_t H_kv, int64_t d_head, sqa_dtype dtype, hipStream_t stream);

/*
 * sqa_decode_step - one new token per sequence.
 *   x_new [B, d_model]  the tokens
 *   pos   device array of B int32: token b's position in sequence b, i.e. the
 *         number of tokens already cached (clamped into [0, N_max-1])
 *   out   [B, d_model]
 * Projects the tokens and writes key and value of token b to cache row pos[b].
 * Query head i then attends over cache rows 0..pos[b] of key/value head
 * floor(i / (H_q/H_kv)), and out[b] = A Wo. The result is row pos[b] of
 * sqa_forward(causal = 1) over the sequence's first pos[b]+1 tokens, provided
 * that rows 0..pos[b]-1 of the caches hold those tokens' keys and values (from
 * sqa_prefill or earlier steps). Attention is split over key chunks, with
 * partial results in the workspace (see sqa_forward: a few hundred KB to a few
 * MB for decode shapes, so it stays with the stream between steps).
 * 1 <= B <= 65535; pos must be 4-byte aligned.
 */
sqa_status sqa_decode_step(const void* x_new, const void* Wq, const void* Wk, const void* Wv,
                           const void* Wo, void* out, void* k_cache, void* v_cache,
                           const int32_t* pos, int64_t B, int64_t N_max, int64_t d_model,
                           int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head, sqa_dtype dtype,
                           hipStream_t stream);

/*
 * Training. The model cards train this layer (ReactiveAI/xSMQAT-m and
 * ReactiveAI/GQA-Ref-Micro, training examples).
 *
 * sqa_training_saved_bytes - size of the activation buffer that
 * sqa_forward_train fills and sqa_backward reads: Q, K, V^T (the layouts of
 * sqa_qkv_projection), A [B*N, H_q*d_head], each row's softmax log-sum-exp
 * (fp32) and A before its rounding to dtype (fp32), about
 * elem_size*(B*Np*(H_q + 2*H_kv)*d_head + B*N*H_q*d_head) + 4*B*H_q*Np
 * + 4*B*N*H_q*d_head bytes. Returns 0 for an invalid shape or dtype.
 */
size_t sqa_training_saved_bytes(int64_t B, int64_t N, int64_t H_q, int64_t H_kv, int64_t d_head,
                                sqa_dtype dtype);

/*
 * sqa_forward_train - sqa_forward that also keeps its activations in `saved`
 * (a caller-owned device buffer of at least sqa_training_saved_bytes() bytes,
 * 16-byte aligned, overlapping no input and not out), for sqa_backward. `out`
 * is bitwise what sqa_forward writes. Its workspace is only the transposed
 * weights.
 */
sqa_status sqa_forward_train(const void* x, const void* Wq, const void* Wk, const void* Wv,
                             const void* Wo, void* out, void* saved, size_t saved_bytes, int64_t B,
                             int64_t N, int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv,
                             int64_t d_head, int causal, sqa_dtype dtype, hipStream_t stream);

/*
 * sqa_backward - gradients of the SQA layer: with Y = sqa_forward(x) and an
 * upstream gradient dy = dL/dY [B, N, d_model], writes
 *   dx  [B, N, d_model]         dL/dx
 *   dWq [d_model, H_q*d_head]   dL/dWq   (dWk, dWv [d_model, H_kv*d_head] likewise)
 *   dWo [H_q*d_head, d_model]   dL/dWo
 * By the chain rule through the definition above (P_i = the attention
 * weights of head i, O_i = P_i V_j):
 *   dA = dy Wo^T, dWo = A^T dy
 *   dS_i = P_i * (dA_i V_j^T - rowsum(dA_i * O_i)),  dQ_i = dS_i K_j / sqrt(d_head)
 *   dK_j = sum over the heads i of group j of dS_i^T Q_i / sqrt(d_head)
 *   dV_j = sum over the same heads of P_i^T dA_i
 *   dx = dQ Wq^T + dK Wk^T + dV Wv^T, dWq = x^T dQ, dWk = x^T dK, dWv = x^T dV
 * (weight gradients summed over the batch). The forward activations come from
 * `saved`, as sqa_forward_train wrote them for the same x, weights, shapes and
 * causal flag; if saved is NULL they are recomputed (saved_bytes is ignored).
 * Arithmetic: dA, dQ, dK, dV and the five outputs are each rounded once to
 * `dtype`; P, dS and the row sums are fp32; rowsum(dA_i * O_i) uses the
 * attention output before its rounding (fp32). The result does not depend on
 * the launch (no atomics).
 * Workspace: about elem_size * B*Np * (8*(H_q + H_kv)*d_head + 2*d_model)
 * bytes (less the saved activations when `saved` is given), 4*B*H_q*Np bytes
 * of fp32 row sums, and the fp32 split-K partial sums of the weight gradients,
 * (see sqa_forward). Outputs must not overlap
 * each other, any input or `saved`; other checks and errors as in sqa_forward.
 */
sqa_status sqa_backward(const void* x, const void* Wq, const void* Wk, const void* Wv,
                        const void* Wo, const void* dy, const void* saved, size_t saved_bytes,
                        void* dx, void* dWq, void* dWk, void* dWv, void* dWo, int64_t B, int64_t N,
                        int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv, int64_t d_head,
                        int causal, sqa_dtype dtype, hipStream_t stream);

/*
 * sqa_padded_length - Np, the sequence length of the Q/K/V^T layouts below:
 * N rounded up to a multiple of 256. Returns -1 for N < 0.
 */
int64_t sqa_padded_length(int64_t N);

/*
 * sqa_qkv_projection - step 1, Q = X Wq, K = X Wk, V = X Wv, written in the
 * layouts the attention step reads (Np = sqa_padded_length(N)):
 *   q  [B, H_q,  Np, d_head]   head-major; column h*d_head + c of X Wq is q[b, h, t, c]
 *   k  [B, H_kv, Np, d_head]
 *   vt [B, H_kv, d_head, Np]   V transposed per head: vt[b, h, c, t] = V[b, t, h*d_head + c]
 * Rows t in [N, Np) are written as zeros. x and the weights are as in sqa_forward.
 * Workspace: the transposed weights (elem_size * d_model*d_head*(H_q + 2*H_kv)
 * bytes), kept as sqa_forward's.
 */
sqa_status sqa_qkv_projection(const void* x, const void* Wq, const void* Wk, const void* Wv,
                              void* q, void* k, void* vt, int64_t B, int64_t N,
                              int64_t d_model, int64_t H, int64_t H_q, int64_t H_kv,
                              int64_t d_head, sqa_dtype dtype, hipStream_t stream);

/*
 * sqa_attention - step 2, the attention core of every query head:
 *   a[b*N + t, i*d_head + c] = sum_s softmax_s(q_i[t] . k_j[s] / sqrt(d_head)) vt_j[c, s]
 * with j = floor(i / (H_q/H_kv)), s over 0..N-1 (0..t if causal), in the q/k/vt
 * layouts of sqa_qkv_projection. Rows t in [N, Np) of q/k/vt must be finite
 * (sqa_qkv_projection writes zeros there). The output a is [B*N, H_q*d_head].
 */
sqa_status sqa_attention(const void* q, const void* k, const void* vt, void* a, int64_t B,
                         int64_t N, int64_t H_q, int64_t H_kv, int64_t d_head, int causal,
                         sqa_dtype dtype, hipStream_t stream);

/*
 * sqa_output_projection - step 3, out[M, d_model] = a[M, K] Wo[K, d_model].
 * K and d_model must be multiples of 32; out must not overlap a or Wo.
 * Workspace: Wo transposed (elem_size * K * d_model bytes), kept as
 * sqa_forward's.
 */
sqa_status sqa_output_projection(const void* a, const void* Wo, void* out, int64_t M,
                                 int64_t K, int64_t d_model, sqa_dtype dtype,
                                 hipStream_t stream);

/* Static description of a status code. Never NULL. */
const char* sqa_status_string(sqa_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* sqa_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* SQA_H */
