// Host-side launchers of the gfx950 kernels. The C ABI (include/sqa.h)
// validates every argument before it calls these; they assume valid shapes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sqa.h"

namespace sqa {

// Sequence padding granule of the Q/K/V^T layouts: a multiple of every query
// tile and key tile the attention kernel uses.
constexpr int64_t kSeqPad = 256;

inline int64_t padded_length(int64_t n) { return (n + kSeqPad - 1) / kSeqPad * kSeqPad; }

// Sequence lengths of a padded batch: lens is null (every sequence has N tokens)
// or a device array of B lengths, each clamped into [0, N] where it is read.

// Step 1: X [B*N, d_model] times [Wq | Wk | Wv] into q [B,H_q,Np,d], k [B,H_kv,Np,d],
// vt [B,H_kv,d,Np]; rows at or past a sequence's length are zero. wt is device
// scratch of qkv_wt_bytes() for the transposed weights.
size_t qkv_wt_bytes(sqa_dtype dt, int64_t d_model, int64_t H_q, int64_t H_kv, int64_t d_head);
hipError_t launch_qkv_projection(sqa_dtype dt, const void* x, const void* wq, const void* wk,
                                 const void* wv, void* wt, void* q, void* k, void* vt, int64_t B,
                                 int64_t N, int64_t Np, int64_t d_model, int64_t H_q, int64_t H_kv,
                                 int64_t d_head, const int32_t* lens, hipStream_t stream);

// Step 2: attention core into a [B*N, H_q*d]; keys end at each sequence's
// length, and rows at or past it are zero. With lse, also each row's base-2
// log-sum-exp of the scaled scores, [B, H_q, Np] fp32 (+inf on padding rows);
// with o32, also the output before its rounding, [B*N, H_q*d] fp32.
// With lens and order_ws (device scratch of attention_order_bytes()), the
// workgroups take the work items longest first.
// With split_ws (device scratch of attention_split_bytes(), at most
// attention_split_bound()), a non-causal bf16 grid whose last dispatch round is
// partial splits that round's work items over their keys and merges the parts.
size_t attention_order_bytes(int64_t B, int64_t N, int64_t H_q);
size_t attention_split_bytes(sqa_dtype dt, int64_t B, int64_t N, int64_t H_q, int64_t H_kv,
                             int64_t d_head, bool causal, bool varlen, hipStream_t stream);
size_t attention_split_bound(int64_t d_head);
hipError_t launch_attention(sqa_dtype dt, const void* q, const void* k, const void* vt, void* a,
                            int64_t B, int64_t N, int64_t Np, int64_t H_q, int64_t H_kv,
                            int64_t d_head, bool causal, const int32_t* lens, hipStream_t stream,
                            float* lse = nullptr, int32_t* order_ws = nullptr,
                            float* o32 = nullptr, float* split_ws = nullptr);

// Step 3: out [M, d_model] = a [M, K] * wo [K, d_model]. wt is device scratch of
// out_wt_bytes() for the transposed weights. With lens, row m is token m % seq_n
// of sequence m / seq_n, and rows in a sequence's padding may be stored as zeros
// without being computed (they are zero when a is).
size_t out_wt_bytes(sqa_dtype dt, int64_t K, int64_t d_model);
hipError_t launch_output_projection(sqa_dtype dt, const void* a, const void* wo, void* wt,
                                    void* out, int64_t M, int64_t K, int64_t d_model,
                                    const int32_t* lens, int64_t seq_n, hipStream_t stream);

// Other products on the projection GEMM, with W given transposed (wt [ncols, K],
// k-contiguous rows). K and ncols are multiples of 32; Np of 256.
//  heads:  out [B, ncols/d, Np, d] (head-major, rows t >= N zero) = x [B, N, K] wt^T
//  unpad:  out [B, N, ncols] = a [B*Np, K] wt^T, rows t >= N of each batch not stored
//  splitk: part [n_split, M, ncols] fp32 = a [M, K] wt^T, summed over the k of each split
hipError_t launch_gemm_heads(sqa_dtype dt, const void* x, const void* wt, void* out, int64_t B,
                             int64_t N, int64_t Np, int64_t K, int64_t ncols, int64_t d_head,
                             hipStream_t stream);
hipError_t launch_gemm_unpad(sqa_dtype dt, const void* a, const void* wt, void* out, int64_t B,
                             int64_t N, int64_t Np, int64_t K, int64_t ncols, hipStream_t stream);
struct SplitK { int64_t k_split, n_split; };
SplitK splitk_plan(int64_t M, int64_t K, int64_t ncols);
hipError_t launch_gemm_splitk(sqa_dtype dt, const void* a, const void* wt, float* part, int64_t M,
                              int64_t K, int64_t ncols, const SplitK& sk, hipStream_t stream);

// Activations a training forward keeps for the backward pass, at these byte
// offsets of one buffer: q, k, vt (the step-1 layouts), a [B*N, H_q*d], the
// per-row base-2 log-sum-exp [B, H_q, Np] fp32, and the attention output
// before rounding, o32 [B*N, H_q*d] fp32.
struct SavedLayout { int64_t q, k, vt, a, lse, o32, total; };
SavedLayout saved_layout(int64_t es, int64_t B, int64_t N, int64_t Np, int64_t H_q, int64_t H_kv,
                         int64_t d);

// Backward pass: dx [B,N,d_model] and dWq, dWk, dWv, dWo (the weights' shapes)
// for the upstream gradient dy [B,N,d_model]. The forward activations come
// from `saved` (saved_layout) or, if it is null, are recomputed. ws is device
// scratch of backward_workspace_bytes(..., saved != null).
size_t backward_workspace_bytes(sqa_dtype dt, int64_t B, int64_t N, int64_t Np, int64_t d_model,
                                int64_t H_q, int64_t H_kv, int64_t d_head, bool saved, bool causal);
hipError_t launch_backward(sqa_dtype dt, const void* x, const void* wq, const void* wk,
                           const void* wv, const void* wo, const void* dy, const void* saved,
                           void* dx, void* dwq, void* dwk, void* dwv, void* dwo, int64_t B,
                           int64_t N, int64_t Np, int64_t d_model, int64_t H_q, int64_t H_kv,
                           int64_t d_head, bool causal, void* ws, hipStream_t stream);

// Key/value caches [B, H_kv, N_max, d]: rows 0..N-1 from the step-1 layouts k and vt.
hipError_t launch_fill_cache(sqa_dtype dt, const void* k, const void* vt, void* kc, void* vc,
                             int64_t B, int64_t H_kv, int64_t N, int64_t Np, int64_t N_max,
                             int64_t d_head, hipStream_t stream);

// Decode step over B new tokens. decode_qkv projects x_new [B, d_model] into
// q [B, H_q*d] and writes token b's key and value straight to cache row pos[b]
// (clamped into [0, N_max-1]); decode_attention writes the states of its key
// chunks over cache rows 0..pos[b] to device scratch part of
// decode_partial_bytes() and, if a is not null, merges them into a [B, H_q*d];
// decode_out gives out [B, d_model] = a [B, K] * wo [K, d_model];
// decode_merge_out (where decode_merge_out_fits) merges the chunk states and
// projects them in one launch.
hipError_t launch_decode_qkv(sqa_dtype dt, const void* x_new, const void* wq, const void* wk,
                             const void* wv, const int32_t* pos, void* q, void* kc, void* vc,
                             int64_t B, int64_t d_model, int64_t H_q, int64_t H_kv, int64_t d_head,
                             int64_t N_max, hipStream_t stream);
size_t decode_partial_bytes(sqa_dtype dt, int64_t B, int64_t H_q, int64_t H_kv, int64_t N_max,
                            int64_t d_head);
hipError_t launch_decode_attention(sqa_dtype dt, const void* q, const void* kc, const void* vc,
                                   const int32_t* pos, void* a, void* part, int64_t B,
                                   int64_t N_max, int64_t H_q, int64_t H_kv, int64_t d_head,
                                   hipStream_t stream);
hipError_t launch_decode_out(sqa_dtype dt, const void* a, const void* wo, void* out, int64_t B,
                             int64_t K, int64_t d_model, hipStream_t stream);
bool decode_merge_out_fits(sqa_dtype dt, int64_t B, int64_t N_max, int64_t H_q, int64_t H_kv,
                           int64_t d_head, int64_t d_model);
hipError_t launch_decode_merge_out(sqa_dtype dt, const void* part, const int32_t* pos,
                                   const void* wo, void* out, int64_t B, int64_t N_max,
                                   int64_t H_q, int64_t H_kv, int64_t d_head, int64_t d_model,
                                   hipStream_t stream);

}  // namespace sqa
