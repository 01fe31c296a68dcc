// Key/value-cache kernels for autoregressive SQA inference on gfx950: filling
// the caches from a causal prefill, and one decode step, in which each
// sequence's new token attends over its cached keys.
//
// The model cards generate text token by token (ReactiveAI/xSMQAT-m and
// ReactiveAI/GQA-Ref-Micro, inference example). A decode step computes row t of
// the causal SQA forward over the sequence's first t+1 tokens. The paper's
// abstract notes that this regime is bound by memory traffic on keys and
// values, which SQA leaves at H_kv heads; it only cuts the query-side work.
//
// Cache layout: k_cache, v_cache [B, H_kv, N_max, d_head], row t of a head is
// token t's key (value): 16-byte aligned rows, contiguous in t.
//
// Decode attention is split over chunks of keys (split-K) so that a step keeps
// every CU busy. Each workgroup owns (sequence, key/value head, chunk) and
// serves all g = H_q / H_kv query heads of that head's group from one read of
// the chunk's keys and values, which is the reuse SQA and GQA rely on.
//  * Phase 1, one key per lane: the key row is loaded whole (16-byte pieces) and
//    dotted with each query head (queries in LDS, broadcast reads). The online
//    softmax runs in the exp2 domain per 64-key block, with wave-wide max and
//    sum; the block's probabilities go to a per-wave LDS slab.
//  * Phase 2, lanes as (key group, 16-byte column chunk): each lane adds p * v
//    for its chunk of head dims over the keys of its group. A fixed key group
//    reads whole consecutive value rows, so the loads are fully coalesced.
//  * The four waves' partial states, then the chunks' partial states (a second
//    kernel), are merged with the usual max/rescale rule.
#include <algorithm>

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int DEC_WAVES = 4, DEC_THREADS = 64 * DEC_WAVES, KB = 64;   // keys per wave block
constexpr float DEC_M_INIT = -1e30f;   // finite: exp2(M_INIT - m) is 0, never NaN

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }

// ---- prefill: K and V of tokens 0..N-1 into rows 0..N-1 of the caches ----

// k [BH, Np, d] -> kc [BH, N_max, d]: the first N rows are n16 contiguous chunks.
__global__ __launch_bounds__(256) void copy_rows(const Chunk* k, Chunk* kc, int64_t n16,
                                                 int64_t src_stride16, int64_t dst_stride16) {
  const int64_t bh = blockIdx.y;
  const Chunk* src = k + bh * src_stride16;
  Chunk* dst = kc + bh * dst_stride16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

// vt [BH, D, Np] -> vc [BH, N_max, D] for t < N, 64 tokens per workgroup through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void transpose_v(const T* vt, T* vc, int N, int64_t Np,
                                                   int64_t N_max) {
  __shared__ T tile[D][KB + 1];
  const int64_t bh = blockIdx.y;
  const int t0 = blockIdx.x * KB;
  const T* src = vt + bh * D * Np;
  T* dst = vc + bh * N_max * D;
  for (int i = threadIdx.x; i < D * KB; i += 256) {
    const int c = i / KB, t = i % KB;
    if (t0 + t < N) tile[c][t] = src[c * Np + t0 + t];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * KB; i += 256) {
    const int t = i / D, c = i % D;
    if (t0 + t < N) dst[(int64_t)(t0 + t) * D + c] = tile[c][t];
  }
}

// ---- decode: the new tokens' K and V into row pos[b] of the caches ----

// k [H_kv, Npb, D] and vt [H_kv, D, Npb] hold the step's tokens as rows b < B.
template <typename T>
__global__ void append_kv(const T* k, const T* vt, T* kc, T* vc, const int32_t* pos, int H_kv,
                          int D, int64_t Npb, int64_t N_max) {
  const int b = blockIdx.x / H_kv, h = blockIdx.x % H_kv, c = threadIdx.x;
  const int64_t p = min(max((int64_t)pos[b], (int64_t)0), N_max - 1);
  const int64_t dst = (((int64_t)b * H_kv + h) * N_max + p) * D + c;
  kc[dst] = k[((int64_t)h * Npb + b) * D + c];
  vc[dst] = vt[((int64_t)h * D + c) * Npb + b];
}

struct DecParams {
  const void* q;                 // [H_q, Npb, D]: query head i of token b at row b
  const void* kc; const void* vc;
  const int32_t* pos;
  float* part;                   // [B, H_q, n_chunks, D + 2]: o[D], m, l per chunk
  int64_t Npb, N_max;
  int H_q, H_kv, g, n_hg, n_chunks, chunk;   // chunk: keys per workgroup, a multiple of KB
  float c;                       // log2(e) / sqrt(D)
};

// Workgroup (chunk, kv head and head group, sequence): at most G query heads.
template <typename T, int D, int G>
__global__ __launch_bounds__(DEC_THREADS) void decode_partial(DecParams p) {
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int CPK = D / EPC;               // chunks per key row
  constexpr int KGS = 64 / CPK;              // key groups in phase 2
  static_assert(CPK * KGS == 64, "lane split");
  __shared__ float qs[G][D];
  __shared__ float ps[DEC_WAVES][KB][G];
  __shared__ float red_ml[DEC_WAVES][G][2];
  __shared__ float red_o[DEC_WAVES][G][D];

  const int chunk_id = blockIdx.x, h = blockIdx.y / p.n_hg, hg = blockIdx.y % p.n_hg;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = h * p.g + hg * G;             // first query head of this group
  const int gq = min(G, p.g - hg * G);         // query heads in this group
  const int64_t pb = min(max((int64_t)p.pos[b], (int64_t)0), p.N_max - 1);
  const int n_keys = (int)pb + 1;
  const int k_begin = chunk_id * p.chunk, k_end = min(k_begin + p.chunk, n_keys);
  float* part = p.part + (((int64_t)b * p.H_q + i0) * p.n_chunks + chunk_id) * (D + 2);
  const int64_t part_head = (int64_t)p.n_chunks * (D + 2);   // stride between query heads

  if (k_begin >= k_end) {   // the chunk lies past this sequence's keys (uniform per workgroup)
    for (int i = tid; i < gq * (D + 2); i += DEC_THREADS) {
      const int hd = i / (D + 2), e = i % (D + 2);
      part[hd * part_head + e] = e == D ? DEC_M_INIT : 0.f;
    }
    return;
  }

  const T* Q = (const T*)p.q;
  for (int i = tid; i < G * D; i += DEC_THREADS) {
    const int hd = i / D, e = i % D;
    qs[hd][e] = hd < gq ? to_f32(Q[((int64_t)(i0 + hd) * p.Npb + b) * D + e]) : 0.f;
  }
  __syncthreads();

  const int64_t row0 = ((int64_t)b * p.H_kv + h) * p.N_max;   // cache row of token 0
  const T* Kc = (const T*)p.kc + row0 * D;
  const T* Vc = (const T*)p.vc + row0 * D;
  const int kg = lane / CPK, dc = lane % CPK;

  float m[G], l[G], o[G][EPC];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = DEC_M_INIT;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[i][e] = 0.f;
  }

  for (int kb = k_begin + wave * KB; kb < k_end; kb += DEC_WAVES * KB) {
    // phase 1: lane = key
    const int j = kb + lane;
    const bool valid = j < k_end;
    const T* krow = Kc + (int64_t)(valid ? j : k_begin) * D;
    float s[G];
#pragma unroll
    for (int i = 0; i < G; ++i) s[i] = 0.f;
#pragma unroll
    for (int ck = 0; ck < CPK; ++ck) {
      const Chunk raw = *reinterpret_cast<const Chunk*>(krow + ck * EPC);
      const T* kv = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float kf = to_f32(kv[e]);
#pragma unroll
        for (int i = 0; i < G; ++i) s[i] = fmaf(qs[i][ck * EPC + e], kf, s[i]);
      }
    }
    float alpha[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float si = valid ? s[i] * p.c : -INFINITY;
      float bm = si;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
      const float m_new = fmaxf(m[i], bm);
      alpha[i] = __builtin_amdgcn_exp2f(m[i] - m_new);
      const float pi = __builtin_amdgcn_exp2f(si - m_new);
      float bs = pi;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) bs += __shfl_xor(bs, off);
      l[i] = l[i] * alpha[i] + bs;
      m[i] = m_new;
      ps[wave][lane][i] = pi;
    }
    // phase 2: lane = (key group kg, column chunk dc); same wave, LDS in order
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[i][e] *= alpha[i];
#pragma unroll
    for (int r = 0; r < CPK; ++r) {
      const int jl = r * KGS + kg;   // key within the block
      const int jj = kb + jl < k_end ? kb + jl : k_begin;   // in range; p is 0 past k_end
      const Chunk raw = *reinterpret_cast<const Chunk*>(Vc + (int64_t)jj * D + dc * EPC);
      const T* vv = reinterpret_cast<const T*>(&raw);
      float vf[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) vf[e] = to_f32(vv[e]);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float pj = ps[wave][jl][i];
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[i][e] = fmaf(pj, vf[e], o[i][e]);
      }
    }
  }

  // This wave's state: o summed over the key groups (lanes with the same dc).
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < EPC; ++e)
#pragma unroll
      for (int off = CPK; off < 64; off <<= 1) o[i][e] += __shfl_xor(o[i][e], off);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (lane == 0) { red_ml[wave][i][0] = m[i]; red_ml[wave][i][1] = l[i]; }
    if (lane < CPK) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) red_o[wave][i][dc * EPC + e] = o[i][e];
    }
  }
  __syncthreads();
  // Merge the waves; write the chunk's (o, m, l) per query head.
  for (int x = tid; x < gq * D; x += DEC_THREADS) {
    const int i = x / D, e = x % D;
    float M = DEC_M_INIT;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, red_ml[w][i][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float f = __builtin_amdgcn_exp2f(red_ml[w][i][0] - M);
      L += red_ml[w][i][1] * f;
      O += red_o[w][i][e] * f;
    }
    float* dst = part + i * part_head;
    dst[e] = O;
    if (e == 0) { dst[D] = M; dst[D + 1] = L; }
  }
}

// One workgroup of D threads per (sequence, query head): merges the chunks
// that hold keys of that sequence and writes a[b, i*D + e].
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine(const float* part, const int32_t* pos, T* a,
                                                    int H_q, int n_chunks, int chunk, int64_t N_max) {
  const int b = blockIdx.x / H_q, i = blockIdx.x % H_q, e = threadIdx.x;
  const int64_t pb = min(max((int64_t)pos[b], (int64_t)0), N_max - 1);
  const int n_valid = (int)min((int64_t)n_chunks, (pb + 1 + chunk - 1) / chunk);
  const float* src = part + ((int64_t)b * H_q + i) * n_chunks * (D + 2);
  float M = DEC_M_INIT;
  for (int c = 0; c < n_valid; ++c) M = fmaxf(M, src[c * (D + 2) + D]);
  float L = 0.f, O = 0.f;
  for (int c = 0; c < n_valid; ++c) {
    const float f = __builtin_amdgcn_exp2f(src[c * (D + 2) + D] - M);
    L += src[c * (D + 2) + D + 1] * f;
    O += src[c * (D + 2) + e] * f;
  }
  a[((int64_t)b * H_q + i) * D + e] = from_f32<T>(O / L);
}

// Chunking of a decode step: enough workgroups for the chip, chunks a multiple of KB.
struct DecodePlan { int G, n_hg, n_chunks, chunk; };

DecodePlan decode_plan(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_max) {
  const int g = (int)(H_q / H_kv);
  DecodePlan pl;
  pl.G = 1;
  while (pl.G < g && pl.G < 8) pl.G *= 2;   // 16 heads' accumulators would spill
  pl.n_hg = (g + pl.G - 1) / pl.G;
  const int64_t units = B * H_kv * pl.n_hg;
  const int64_t max_chunks = (N_max + KB - 1) / KB;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(max_chunks, (1024 + units - 1) / units));
  const int64_t per = (N_max + want - 1) / want;
  pl.chunk = (int)((per + KB - 1) / KB * KB);
  pl.n_chunks = (int)((N_max + pl.chunk - 1) / pl.chunk);
  return pl;
}

template <typename T, int D, int G>
hipError_t run_partial(const DecParams& p, dim3 grid, hipStream_t stream) {
  decode_partial<T, D, G><<<grid, DEC_THREADS, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t partial_for(int G, const DecParams& p, dim3 grid, hipStream_t stream) {
  switch (G) {
    case 1: return run_partial<T, D, 1>(p, grid, stream);
    case 2: return run_partial<T, D, 2>(p, grid, stream);
    case 4: return run_partial<T, D, 4>(p, grid, stream);
    default: return run_partial<T, D, 8>(p, grid, stream);
  }
}

template <typename T, int D>
hipError_t decode_impl(const void* q, const void* kc, const void* vc, const int32_t* pos, void* a,
                       float* part, int64_t B, int64_t Npb, int64_t N_max, int64_t H_q,
                       int64_t H_kv, hipStream_t stream) {
  const DecodePlan pl = decode_plan(B, H_q, H_kv, N_max);
  DecParams p;
  p.q = q; p.kc = kc; p.vc = vc; p.pos = pos; p.part = part;
  p.Npb = Npb; p.N_max = N_max;
  p.H_q = (int)H_q; p.H_kv = (int)H_kv; p.g = (int)(H_q / H_kv); p.n_hg = pl.n_hg;
  p.n_chunks = pl.n_chunks; p.chunk = pl.chunk;
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  const dim3 grid((unsigned)pl.n_chunks, (unsigned)(H_kv * pl.n_hg), (unsigned)B);
  hipError_t e = partial_for<T, D>(pl.G, p, grid, stream);
  if (e != hipSuccess) return e;
  decode_combine<T, D><<<(unsigned)(B * H_q), D, 0, stream>>>(part, pos, (T*)a, (int)H_q,
                                                            pl.n_chunks, pl.chunk, N_max);
  return hipGetLastError();
}

}  // namespace

size_t decode_partial_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_max, int64_t d_head) {
  const DecodePlan pl = decode_plan(B, H_q, H_kv, N_max);
  return (size_t)(B * H_q * pl.n_chunks * (d_head + 2)) * sizeof(float);
}

hipError_t launch_fill_cache(sqa_dtype dt, const void* k, const void* vt, void* kc, void* vc,
                             int64_t B, int64_t H_kv, int64_t N, int64_t Np, int64_t N_max,
                             int64_t d_head, hipStream_t stream) {
  const int64_t es = dt == SQA_DTYPE_BF16 ? 2 : 4;
  const int64_t BH = B * H_kv;
  if (BH > 65535) return hipErrorInvalidConfiguration;
  const int64_t n16 = N * d_head * es / 16;
  const unsigned gx = (unsigned)std::min<int64_t>(1024, (n16 + 255) / 256);
  copy_rows<<<dim3(gx, (unsigned)BH), 256, 0, stream>>>(
      (const Chunk*)k, (Chunk*)kc, n16, Np * d_head * es / 16, N_max * d_head * es / 16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + KB - 1) / KB), (unsigned)BH);
  if (dt == SQA_DTYPE_BF16) {
    if (d_head == 64) transpose_v<bf16, 64><<<grid, 256, 0, stream>>>((const bf16*)vt, (bf16*)vc, (int)N, Np, N_max);
    else transpose_v<bf16, 32><<<grid, 256, 0, stream>>>((const bf16*)vt, (bf16*)vc, (int)N, Np, N_max);
  } else {
    if (d_head == 64) transpose_v<float, 64><<<grid, 256, 0, stream>>>((const float*)vt, (float*)vc, (int)N, Np, N_max);
    else transpose_v<float, 32><<<grid, 256, 0, stream>>>((const float*)vt, (float*)vc, (int)N, Np, N_max);
  }
  return hipGetLastError();
}

hipError_t launch_append_kv(sqa_dtype dt, const void* k, const void* vt, void* kc, void* vc,
                            const int32_t* pos, int64_t B, int64_t H_kv, int64_t d_head,
                            int64_t Npb, int64_t N_max, hipStream_t stream) {
  const unsigned grid = (unsigned)(B * H_kv), threads = (unsigned)d_head;
  if (dt == SQA_DTYPE_BF16)
    append_kv<bf16><<<grid, threads, 0, stream>>>((const bf16*)k, (const bf16*)vt, (bf16*)kc,
                                                 (bf16*)vc, pos, (int)H_kv, (int)d_head, Npb, N_max);
  else
    append_kv<float><<<grid, threads, 0, stream>>>((const float*)k, (const float*)vt, (float*)kc,
                                                  (float*)vc, pos, (int)H_kv, (int)d_head, Npb, N_max);
  return hipGetLastError();
}

hipError_t launch_decode_attention(sqa_dtype dt, const void* q, const void* kc, const void* vc,
                                   const int32_t* pos, void* a, void* part, int64_t B, int64_t Npb,
                                   int64_t N_max, int64_t H_q, int64_t H_kv, int64_t d_head,
                                   hipStream_t stream) {
  if (B > 65535 || H_kv * ((H_q / H_kv + 7) / 8) > 65535) return hipErrorInvalidConfiguration;
  float* pf = (float*)part;
  if (dt == SQA_DTYPE_BF16)
    return d_head == 64 ? decode_impl<bf16, 64>(q, kc, vc, pos, a, pf, B, Npb, N_max, H_q, H_kv, stream)
                        : decode_impl<bf16, 32>(q, kc, vc, pos, a, pf, B, Npb, N_max, H_q, H_kv, stream);
  return d_head == 64 ? decode_impl<float, 64>(q, kc, vc, pos, a, pf, B, Npb, N_max, H_q, H_kv, stream)
                      : decode_impl<float, 32>(q, kc, vc, pos, a, pf, B, Npb, N_max, H_q, H_kv, stream);
}

}  // namespace sqa
