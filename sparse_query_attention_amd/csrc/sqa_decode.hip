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
#include <atomic>
#include <cstdint>
#include <type_traits>

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
// (sequence, head) pairs stride over the grid's y dimension (BH may pass 65535).
__global__ __launch_bounds__(256) void copy_rows(const Chunk* k, Chunk* kc, int64_t n16,
                                                 int64_t src_stride16, int64_t dst_stride16,
                                                 int64_t BH) {
  for (int64_t bh = blockIdx.y; bh < BH; bh += gridDim.y) {
    const Chunk* src = k + bh * src_stride16;
    Chunk* dst = kc + bh * dst_stride16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
      dst[i] = src[i];
  }
}

// vt [BH, D, Np] -> vc [BH, N_max, D] for t < N, 64 tokens per workgroup through LDS;
// (sequence, head) pairs stride over the grid's y dimension.
template <typename T, int D>
__global__ __launch_bounds__(256) void transpose_v(const T* vt, T* vc, int N, int64_t Np,
                                                   int64_t N_max, int64_t BH) {
  __shared__ T tile[D][KB + 1];
  const int t0 = blockIdx.x * KB;
  for (int64_t bh = blockIdx.y; bh < BH; bh += gridDim.y) {
    const T* src = vt + bh * D * Np;
    T* dst = vc + bh * N_max * D;
    __syncthreads();   // the previous pair's reads of the tile are done
    for (int i = threadIdx.x; i < D * KB; i += 256) {
      const int c = i / KB, t = i % KB;
      if (t0 + t < N) tile[c][t] = src[(int64_t)c * Np + t0 + t];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < D * KB; i += 256) {
      const int t = i / D, c = i % D;
      if (t0 + t < N) dst[(int64_t)(t0 + t) * D + c] = tile[c][t];
    }
  }
}

// ---- decode: projections of the B new tokens ----
// A decode step projects only B tokens, so these products are skinny: each
// weight element is used B times, and the step is bound by reading the weights
// once and, at a few MB, by latency. Each product is one launch. A workgroup
// owns SK_COLS output columns over all K rows and up to SK_BR tokens, and reads
// the weights in place from their [in, out] layout: one 16-byte chunk per
// thread and row, the rows of a K block split over the thread phases. The
// phases' fp32 sums meet in a reduce-scatter across the wave's lanes and then
// across the four waves through LDS, in a fixed order; the workgroup rounds
// once and stores its results itself (q and the new cache rows, or the output).

constexpr int SK_COLS = 8, SK_BR = 8, SK_J = 4;     // columns and tokens per workgroup, rows per thread

// Column block of workgroup x of a row of n: the dispatcher hands workgroup i
// to XCD i % 8, and each XCD has its own L2. Neighbouring column blocks share
// the 128-byte lines of every weight row, so the blocks are renumbered to run
// in contiguous runs of n/8 on one XCD, and each line reaches one L2 only
// (rather than up to eight, each fetching it from memory): 7.7 -> 6.8 us for
// the Q/K/V product of 8 tokens at d_model 1024. A grid of several rows keeps
// the assignment when n is a multiple of 8, the only case renumbered. (The
// merge kernel's 32-column blocks, two to a line, measured slower this way.)
__device__ inline int xcd_block(int x, int n) { return n % 8 ? x : x % 8 * (n / 8) + x / 8; }

// x staged as fp32 [k][token], 8 floats of padding after every 8 rows, so that
// the transposing writes (lanes over tokens, then over 16-byte chunks of k) and
// the row reads (two 16-byte reads per row) are free of bank conflicts.
__device__ inline int xs_at(int k, int b) { return (k + (k >> 3)) * SK_BR + b; }

// Cross-lane steps on the VALU (no LDS round trip). Lane partners by stride:
// 32 and 16 through v_permlane32_swap / v_permlane16_swap (they exchange the
// upper lanes of one register with the lower lanes of another), 8 through DPP
// row_ror:8 (lane ^ 8 within a row of 16), 2 and 1 through quad permutations;
// for 4, row_ror:12 and row_ror:4 bring lane + 4 and lane - 4 within the row
// (row_ror:n hands lane i the value of lane i - n), and the lane's bit 2 picks
// one (lane ^ 4). dpp_partner<7> is lane ^ 7 within
// 8 (row_half_mirror): enough for a full reduction, where every lane ends with
// the same total.
template <int M> __device__ inline float dpp_partner(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned r;
  if constexpr (M == 8) r = __builtin_amdgcn_update_dpp(0u, u, 0x128, 0xF, 0xF, false);
  else if constexpr (M == 7) r = __builtin_amdgcn_update_dpp(0u, u, 0x141, 0xF, 0xF, false);
  else if constexpr (M == 2) r = __builtin_amdgcn_update_dpp(0u, u, 0x4E, 0xF, 0xF, false);
  else r = __builtin_amdgcn_update_dpp(0u, u, 0xB1, 0xF, 0xF, false);
  return __builtin_bit_cast(float, r);
}
__device__ inline float dpp_xor4(float x, bool hi) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const unsigned up = __builtin_amdgcn_update_dpp(0u, u, 0x12C, 0xF, 0xF, false);     // lane + 4
  const unsigned down = __builtin_amdgcn_update_dpp(0u, u, 0x124, 0xF, 0xF, false);   // lane - 4
  return __builtin_bit_cast(float, hi ? down : up);
}
// One reduce-scatter step over lane bit M on pairs (v[i], v[n/2 + i]): a lane
// with the bit clear keeps v[i], one with it set keeps v[n/2 + i], and each
// adds its partner's copy of the half it keeps.
template <int M, int n, int NV> __device__ inline void rs_step(float (&v)[NV], int lane) {
  if constexpr (M >= 16) {
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const unsigned a = __builtin_bit_cast(unsigned, v[i]), b = __builtin_bit_cast(unsigned, v[n / 2 + i]);
      unsigned r0, r1;
      if constexpr (M == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        r0 = r[0]; r1 = r[1];
      } else {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        r0 = r[0]; r1 = r[1];
      }
      v[i] = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    }
  } else {
    const bool hi = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float keep = hi ? v[n / 2 + i] : v[i];
      const float give = hi ? v[i] : v[n / 2 + i];
      if constexpr (M == 4) v[i] = keep + dpp_xor4(give, hi);
      else v[i] = keep + dpp_partner<M>(give);
    }
  }
}
// The reduce-scatter of N values per lane down to OUT, over lane bits M, M/2, ...
template <int N, int M, int OUT, int NV> __device__ inline void rs_levels(float (&v)[NV], int lane) {
  if constexpr (N > OUT) {
    rs_step<M, N>(v, lane);
    rs_levels<N / 2, M / 2, OUT>(v, lane);
  }
}
// Reduction of x over the wave (every lane gets the result), in a fixed order.
template <bool MAX> __device__ inline float wave_reduce(float x) {
  auto op = [](float p, float q) { return MAX ? fmaxf(p, q) : p + q; };
  const unsigned u = __builtin_bit_cast(unsigned, x);
  {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = op(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  }
  {
    const unsigned w = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    x = op(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  }
  x = op(x, dpp_partner<8>(x));
  x = op(x, dpp_partner<7>(x));
  x = op(x, dpp_partner<2>(x));
  x = op(x, dpp_partner<1>(x));
  return x;
}

// out[b][n] = sum over k of x[b][k] * W[k][n] for W = [W0 | W1 | W2], x [B, K].
// Every segment width is a multiple of SK_COLS, so a workgroup's columns lie in
// one segment. K is a multiple of the chunk width (16 bytes of T).
template <typename T, typename Store>
__global__ __launch_bounds__(256) void skinny(const T* x, int B, int K, const T* w0, int n0w,
                                              const T* w1, int n1w, const T* w2, int n2w,
                                              Store store) {
  constexpr int EPC = 16 / (int)sizeof(T);   // columns per chunk
  constexpr int TPR = SK_COLS / EPC;         // threads per weight row (lanes tid % TPR)
  constexpr int PH = 256 / TPR;              // thread phases over K
  constexpr int KB = PH * SK_J;              // K rows per block
  constexpr int XC = KB / EPC;               // x chunks per token and block
  constexpr int XPT = XC * SK_BR / 256;      // x chunks per thread
  constexpr int NV = SK_BR * EPC;            // partial sums per thread
  constexpr int OUT = SK_BR * SK_COLS / 64;  // results per lane after the wave's reduce-scatter
  static_assert(XPT * 256 == XC * SK_BR && OUT * 64 == SK_BR * SK_COLS, "split");
  __shared__ __align__(16) float xs[(KB + KB / 8) * SK_BR];
  __shared__ __align__(16) float red[4][SK_BR * SK_COLS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid % TPR, kp = tid / TPR;
  const int n0 = xcd_block(blockIdx.x, gridDim.x) * SK_COLS;
  const T* W = w0;
  int ld = n0w, c0 = n0;
  if (n0 >= n0w + n1w) { W = w2; ld = n2w; c0 = n0 - n0w - n1w; }
  else if (n0 >= n0w) { W = w1; ld = n1w; c0 = n0 - n0w; }
  c0 += cc * EPC;
  const int b0 = blockIdx.y * SK_BR, nb = min(SK_BR, B - b0);

  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KB) {
    // Every load of the block is issued before any is used: row indexes are
    // clamped to valid rows and the values of rows past K cleared afterwards,
    // so no load sits behind a branch.
    Chunk raw[SK_J];
#pragma unroll
    for (int j = 0; j < SK_J; ++j) {
      const int k = k0 + kp + j * PH;
      raw[j] = *reinterpret_cast<const Chunk*>(W + (int64_t)(k < K ? k : 0) * ld + c0);
    }
    Chunk xr[XPT];
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int i = tid + u * 256, b = i % SK_BR, k = k0 + i / SK_BR * EPC;
      xr[u] = *reinterpret_cast<const Chunk*>(x + (int64_t)(b0 + (b < nb ? b : 0)) * K +
                                              (k < K ? k : 0));
    }
#pragma unroll
    for (int j = 0; j < SK_J; ++j) {
      const uint32_t keep = k0 + kp + j * PH < K ? ~0u : 0u;
#pragma unroll
      for (int w = 0; w < 4; ++w) raw[j].w[w] &= keep;
    }
    __syncthreads();   // the previous block's reads of xs are done
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int i = tid + u * 256, b = i % SK_BR, kk = i / SK_BR * EPC;
      const bool ok = b < nb && k0 + kk < K;
      const T* xv = reinterpret_cast<const T*>(&xr[u]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) xs[xs_at(kk + e, b)] = ok ? to_f32(xv[e]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SK_J; ++j) {
      const T* wv = reinterpret_cast<const T*>(&raw[j]);
      float wf[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) wf[e] = to_f32(wv[e]);
      const float4* xrow = reinterpret_cast<const float4*>(&xs[xs_at(kp + j * PH, 0)]);
#pragma unroll
      for (int b4 = 0; b4 < SK_BR / 4; ++b4) {
        const float4 xv = xrow[b4];
        const float xb[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            acc[(b4 * 4 + u) * EPC + e] = fmaf(xb[u], wf[e], acc[(b4 * 4 + u) * EPC + e]);
      }
    }
  }

  // Reduce-scatter over the wave's phases (lane bits above those of cc): at
  // the step over lane bit m a lane keeps the half of its sums selected by that
  // bit, adds its partner's copy of that half and hands over the other half.
  // After the last step a lane holds OUT consecutive flat indexes
  // (lane / TPR) * OUT + i of acc, flat index = token * EPC + column in chunk.
  rs_levels<NV, 32, OUT>(acc, lane);
  const float* v = acc;
  {
    const int f = (lane / TPR) * OUT, b = f / EPC, col = cc * EPC + f % EPC;
#pragma unroll
    for (int i = 0; i < OUT; ++i) red[wave][b * SK_COLS + col + i] = v[i];
  }
  __syncthreads();
  const int b = tid / SK_COLS, c = tid % SK_COLS;
  if (b < nb) {
    const float s = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    store(b0 + b, n0 + c, s);
  }
}

// Results of the Q/K/V product: q to [B, H_q*D]; the new key and value of
// token b straight to cache row pos[b] (clamped into [0, N_max-1]).
template <typename T>
struct QkvRows {
  T* q; T* kc; T* vc;
  const int32_t* pos;
  int wq_w, wkv_w, D, H_kv;
  int64_t N_max;
  __device__ void operator()(int b, int n, float v) const {
    const T r = from_f32<T>(v);
    if (n < wq_w) { q[(int64_t)b * wq_w + n] = r; return; }
    const int nk = (n - wq_w) % wkv_w, h = nk / D, c = nk % D;
    const int64_t p = min(max((int64_t)pos[b], (int64_t)0), N_max - 1);
    T* dst = n < wq_w + wkv_w ? kc : vc;
    dst[(((int64_t)b * H_kv + h) * N_max + p) * D + c] = r;
  }
};

template <typename T>
struct DenseRows {   // out [B, ncols]
  T* out;
  int ncols;
  __device__ void operator()(int b, int n, float v) const {
    out[(int64_t)b * ncols + n] = from_f32<T>(v);
  }
};

struct DecParams {
  const void* q;                 // [B, H_q * D]: query head i of token b at q[b][i*D ..]
  const void* kc; const void* vc;
  const int32_t* pos;
  float* part;                   // [B, H_q, n_chunks, D + 2]: o[D], m, l per chunk
  int64_t N_max;
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
  __shared__ __align__(16) float qs[G][D];
  __shared__ float ps[DEC_WAVES][KB][G];
  __shared__ float red_ml[DEC_WAVES][G][2];
  __shared__ float red_o[DEC_WAVES][G][D];

  const int chunk_id = blockIdx.x, h = blockIdx.y / p.n_hg, hg = blockIdx.y % p.n_hg;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
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

  const int64_t row0 = ((int64_t)b * p.H_kv + h) * p.N_max;   // cache row of token 0
  const T* Kc = (const T*)p.kc + row0 * D;
  const T* Vc = (const T*)p.vc + row0 * D;
  const int kg = lane / CPK, dc = lane % CPK;

  // Each wave streams its 64-key blocks with the next block's loads in flight
  // while the current one is computed: its key rows are requested as soon as
  // phase 1 has consumed the current ones, its value chunks as soon as phase 2
  // has. Rows past the chunk are clamped to its first row (one cache line for
  // the whole wave), so no load sits behind a branch; the loads issued in a
  // wave's last step are drained after the loop.
  constexpr int KSTEP = DEC_WAVES * KB;
  Chunk kraw[CPK], vraw[CPK];
  auto load_k = [&](int kb) {
    const int j = kb + lane;
    const T* krow = Kc + (int64_t)(j < k_end ? j : k_begin) * D;
#pragma unroll
    for (int ck = 0; ck < CPK; ++ck) kraw[ck] = *reinterpret_cast<const Chunk*>(krow + ck * EPC);
  };
  auto load_v = [&](int kb) {
#pragma unroll
    for (int r = 0; r < CPK; ++r) {
      const int jv = kb + r * KGS + kg;
      vraw[r] = *reinterpret_cast<const Chunk*>(Vc + (int64_t)(jv < k_end ? jv : k_begin) * D + dc * EPC);
    }
  };

  // The queries go to LDS as fp32. Their loads are issued first and the first
  // block's keys and values right behind them, so the staging waits for the
  // queries alone and phase 1 for the keys alone.
  constexpr int QPT = (G * D + DEC_THREADS - 1) / DEC_THREADS;
  const T* Q = (const T*)p.q;
  float qv[QPT];
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int i = tid + u * DEC_THREADS;
    const bool ok = i < G * D && i / D < gq;
    const int ic = ok ? i : 0;   // a valid element, so the load needs no branch
    const float v = to_f32(Q[((int64_t)b * p.H_q + i0 + ic / D) * D + ic % D]);
    qv[u] = ok ? v : 0.f;
  }
  __builtin_amdgcn_sched_barrier(0);
  load_k(k_begin + wave * KB);
  __builtin_amdgcn_sched_barrier(0);
  load_v(k_begin + wave * KB);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int i = tid + u * DEC_THREADS;
    if (i < G * D) qs[i / D][i % D] = qv[u];
  }
  __syncthreads();

  float m[G], l[G], o[G][EPC];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = DEC_M_INIT;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[i][e] = 0.f;
  }

  for (int kb = k_begin + wave * KB; kb < k_end; kb += KSTEP) {
    // phase 1: lane = key
    const int j = kb + lane;
    const bool valid = j < k_end;
    float s[G];
#pragma unroll
    for (int i = 0; i < G; ++i) s[i] = 0.f;
    // The queries are read from LDS in the loop: an opaque zero offset keeps
    // the compiler from hoisting G*D of them into registers, which at G >= 2
    // cost more occupancy than the broadcast reads cost time.
    int qo = 0;
    asm volatile("" : "+s"(qo));
    const float* qb = &qs[0][0] + qo;
#pragma unroll
    for (int ck = 0; ck < CPK; ++ck) {
      const T* kv = reinterpret_cast<const T*>(&kraw[ck]);
#pragma unroll
      for (int e4 = 0; e4 < EPC / 4; ++e4) {
        const float k0 = to_f32(kv[e4 * 4]), k1 = to_f32(kv[e4 * 4 + 1]),
                    k2 = to_f32(kv[e4 * 4 + 2]), k3 = to_f32(kv[e4 * 4 + 3]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float4 q4 = *reinterpret_cast<const float4*>(qb + i * D + ck * EPC + e4 * 4);
          s[i] = fmaf(q4.x, k0, s[i]); s[i] = fmaf(q4.y, k1, s[i]);
          s[i] = fmaf(q4.z, k2, s[i]); s[i] = fmaf(q4.w, k3, s[i]);
        }
      }
    }
    // The scheduler would otherwise move the next block's loads next to their
    // first use and pull the value conversions into phase 1, which then waits
    // for the values; the barriers keep each block's loads where they are.
    __builtin_amdgcn_sched_barrier(0);
    load_k(kb + KSTEP);   // phase 1 is done with kraw
    __builtin_amdgcn_sched_barrier(0);
    float alpha[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float si = valid ? s[i] * p.c : -INFINITY;
      const float bm = wave_reduce<true>(si);
      const float m_new = fmaxf(m[i], bm);
      alpha[i] = __builtin_amdgcn_exp2f(m[i] - m_new);
      const float pi = __builtin_amdgcn_exp2f(si - m_new);
      const float bs = wave_reduce<false>(pi);
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
      const int jl = r * KGS + kg;   // key within the block; past k_end it loaded a valid row, p = 0
      const T* vv = reinterpret_cast<const T*>(&vraw[r]);
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
    __builtin_amdgcn_sched_barrier(0);
    load_v(kb + KSTEP);   // phase 2 is done with vraw
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();   // the last step's loads, never used

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

// One 256-thread workgroup per (sequence, query head) merges the chunks that
// hold keys of that sequence and writes a[b, i*D + e]. Thread (group gr,
// column e) takes every (256/D)-th chunk from gr on and merges them as they
// arrive with the max/rescale rule, so all its loads are independent of each
// other; the groups' states then meet in LDS.

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine(const float* part, const int32_t* pos, T* a,
                                                      int H_q, int n_chunks, int chunk,
                                                      int64_t N_max) {
  constexpr int GR = 256 / D;
  __shared__ float mo[GR][D], mm[GR], ml[GR];
  const int b = blockIdx.x / H_q, i = blockIdx.x % H_q, tid = threadIdx.x;
  const int64_t pb = min(max((int64_t)pos[b], (int64_t)0), N_max - 1);
  const int n_valid = (int)min((int64_t)n_chunks, (pb + 1 + chunk - 1) / chunk);
  const float* src = part + ((int64_t)b * H_q + i) * n_chunks * (D + 2);
  const int gr = tid / D, e = tid % D;
  float M = DEC_M_INIT, L = 0.f, O = 0.f;
#pragma unroll 4
  for (int c = gr; c < n_valid; c += GR) {
    const float* st = src + (int64_t)c * (D + 2);
    const float m = st[D], l = st[D + 1], o = st[e];
    const float Mn = fmaxf(M, m);
    const float fa = __builtin_amdgcn_exp2f(M - Mn), fb = __builtin_amdgcn_exp2f(m - Mn);
    L = L * fa + l * fb;
    O = O * fa + o * fb;
    M = Mn;
  }
  mo[gr][e] = O;
  if (e == 0) { mm[gr] = M; ml[gr] = L; }
  __syncthreads();
  if (tid < D) {
    float Mt = DEC_M_INIT;
#pragma unroll
    for (int g2 = 0; g2 < GR; ++g2) Mt = fmaxf(Mt, mm[g2]);
    float Lt = 0.f, Ot = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < GR; ++g2) {
      const float f = __builtin_amdgcn_exp2f(mm[g2] - Mt);
      Lt += ml[g2] * f;
      Ot += mo[g2][tid] * f;
    }
    a[((int64_t)b * H_q + i) * D + tid] = from_f32<T>(Ot / Lt);   // Lt > 0: key 0 is in chunk 0
  }
}

// The merge of the key chunks fused with the output projection: workgroup
// (block of MC output columns, token b) merges the chunk states of every query
// head of token b into a[b] = o / l, rounded to T once (as decode_combine
// stores it), keeps a[b] in LDS as fp32 and forms
// out[b, n0 .. n0+MC) = a[b] * wo[:, n0 .. n0+MC). The merge takes two passes,
// so that no load waits on another: a wave per head reduces the chunks' m
// (max) and l (weighted sum) across its lanes and leaves each chunk's weight
// exp2(m_c - M) in LDS, then every element sums its chunks' o with those
// weights. Each of the d_model/MC workgroups of a token merges its states
// again (from L2 after the first), which costs less than the launch it
// saves. The first RJ rows per thread of wo are loaded before the merge, so
// their latency overlaps it. LDS: a[b] [K], the weights [H_q][n_valid], 1/L
// [H_q], then the phases' sums.
constexpr int MC = 32;
constexpr int MERGE_MAX_W = 4096;   // H_q * n_chunks weights in LDS
// FP: 1 where K <= 512, else 2 (the loads of the common shape cover K <= FP * 512).
template <typename T, int D, int FP>
__global__ __launch_bounds__(256) void decode_merge_out(const float* part, const int32_t* pos,
                                                        const T* wo, T* out, int H_q, int n_chunks,
                                                        int chunk, int64_t N_max, int d_model) {
  constexpr int EPC = 16 / (int)sizeof(T);   // columns per 16-byte chunk
  constexpr int TPR = MC / EPC;              // threads per row of the column block
  constexpr int PH = 256 / TPR;              // row phases
  constexpr int RJ = FP * 512 / PH < 16 ? FP * 512 / PH : 16;   // rows per thread and k block
  constexpr int KBLK = PH * RJ;
  constexpr int SEG = 8;                     // first-level groups of the phase sums
  static_assert(PH % SEG == 0 && 256 / MC == SEG, "split");
  extern __shared__ float smem_f[];
  const int K = H_q * D;
  const int b = blockIdx.y, n0 = blockIdx.x * MC, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t pb = min(max((int64_t)pos[b], (int64_t)0), N_max - 1);
  const int nv = (int)min((int64_t)n_chunks, (pb + 1 + chunk - 1) / chunk);   // >= 1
  float* a_s = smem_f;                       // [K]
  float* w_s = a_s + K;                      // [H_q][nv]
  float* il_s = w_s + H_q * nv;              // [H_q]
  float* red = il_s + H_q;                   // [PH][MC]
  float* red2 = red + PH * MC;               // [SEG][MC]
  const int cc = tid % TPR, ph = tid / TPR;
  const T* wcol = wo + n0 + cc * EPC;

  auto load_rows = [&](int k0, Chunk (&raw)[RJ]) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int k = k0 + ph + j * PH;
      raw[j] = *reinterpret_cast<const Chunk*>(wcol + (int64_t)(k < K ? k : 0) * d_model);
    }
  };
  Chunk raw[RJ];
  load_rows(0, raw);   // in flight during the merge

  const float* pbase = part + (int64_t)b * H_q * n_chunks * (D + 2);
  // Common shape (at most FC chunks, at most FH heads, K <= FP * 512): every
  // load the merge needs is issued at once, in the order of use (each wave's
  // heads' m and l, then o as pairs of elements), with the wo rows already in
  // flight behind them in the counter.
  constexpr int FC = 32, FH = 16;
  const bool fast = nv <= FC && H_q <= FH && K <= FP * 512;
  if (fast) {
    constexpr int HPW = FH / 4;   // heads per wave
    float mh[HPW], lh[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int i = wave + 4 * hh;
      const float* st = pbase + ((int64_t)(i < H_q ? i : 0) * n_chunks + (lane < nv ? lane : 0)) * (D + 2);
      mh[hh] = st[D];
      lh[hh] = st[D + 1];
    }
    float2 o_r[FP][FC];
#pragma unroll
    for (int r = 0; r < FP; ++r) {
      const int x = 2 * (tid + r * 256), xc = x < K ? x : 0;
      const float* src = pbase + (int64_t)(xc / D) * n_chunks * (D + 2) + xc % D;
#pragma unroll
      for (int c = 0; c < FC; ++c)
        o_r[r][c] = *reinterpret_cast<const float2*>(src + (int64_t)(c < nv ? c : 0) * (D + 2));
    }
    // pass 1: per head, M = max m_c, weights w_c = exp2(m_c - M), 1/L with L = sum w_c l_c
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int i = wave + 4 * hh;
      if (i < H_q) {   // uniform per wave
        const float mx = wave_reduce<true>(lane < nv ? mh[hh] : DEC_M_INIT);
        const float w = __builtin_amdgcn_exp2f(mh[hh] - mx);
        if (lane < nv) w_s[i * nv + lane] = w;
        const float ls = wave_reduce<false>(lane < nv ? w * lh[hh] : 0.f);
        if (lane == 0) il_s[i] = 1.f / ls;   // ls > 0: key 0 is in chunk 0
      }
    }
    __syncthreads();
    // pass 2: a[i*D + e] = (sum_c w_c o_c[e]) / L, chunks in order
#pragma unroll
    for (int r = 0; r < FP; ++r) {
      const int x = 2 * (tid + r * 256);
      if (x < K) {
        const int i = x / D;
        const float* wi = w_s + i * nv;
        float O0 = 0.f, O1 = 0.f;
#pragma unroll
        for (int c = 0; c < FC; ++c)
          if (c < nv) { O0 = fmaf(wi[c], o_r[r][c].x, O0); O1 = fmaf(wi[c], o_r[r][c].y, O1); }
        a_s[x] = to_f32(from_f32<T>(O0 * il_s[i]));
        a_s[x + 1] = to_f32(from_f32<T>(O1 * il_s[i]));
      }
    }
  } else {
    // pass 1 as above, a head per wave at a time
    for (int i = wave; i < H_q; i += 4) {
      const float* ph_ = pbase + (int64_t)i * n_chunks * (D + 2);
      float mx = DEC_M_INIT, ls = 0.f;
      for (int c = lane; c < nv; c += 64) mx = fmaxf(mx, ph_[(int64_t)c * (D + 2) + D]);
      mx = wave_reduce<true>(mx);
      for (int c = lane; c < nv; c += 64) {
        const float* st = ph_ + (int64_t)c * (D + 2);
        const float w = __builtin_amdgcn_exp2f(st[D] - mx);
        w_s[i * nv + c] = w;
        ls = fmaf(w, st[D + 1], ls);
      }
      ls = wave_reduce<false>(ls);
      if (lane == 0) il_s[i] = 1.f / ls;
    }
    __syncthreads();
    constexpr int OU = 8;   // chunk loads in flight per element
    for (int x = tid; x < K; x += 256) {
      const int i = x / D, e = x % D;
      const float* src = pbase + (int64_t)i * n_chunks * (D + 2) + e;
      const float* wi = w_s + i * nv;
      float O = 0.f;
      for (int c0 = 0; c0 < nv; c0 += OU) {
        float o[OU];
#pragma unroll
        for (int u = 0; u < OU; ++u) o[u] = c0 + u < nv ? src[(int64_t)(c0 + u) * (D + 2)] : 0.f;
#pragma unroll
        for (int u = 0; u < OU; ++u)
          if (c0 + u < nv) O = fmaf(wi[c0 + u], o[u], O);
      }
      a_s[x] = to_f32(from_f32<T>(O * il_s[i]));
    }
  }
  __syncthreads();

  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KBLK) {
    if (k0 > 0) load_rows(k0, raw);
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int k = k0 + ph + j * PH;
      if (k < K) {
        const T* wv = reinterpret_cast<const T*>(&raw[j]);
        const float av = a_s[k];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = fmaf(av, to_f32(wv[e]), acc[e]);
      }
    }
  }
  // sums over the phases in a fixed order
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[ph * MC + cc * EPC + e] = acc[e];
  __syncthreads();
  {
    const int col = tid % MC, sg = tid / MC;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < PH / SEG; ++q) sum += red[(sg * (PH / SEG) + q) * MC + col];
    red2[sg * MC + col] = sum;
  }
  __syncthreads();
  if (tid < MC) {
    float sum = 0.f;
#pragma unroll
    for (int sg = 0; sg < SEG; ++sg) sum += red2[sg * MC + tid];
    out[(int64_t)b * d_model + n0 + tid] = from_f32<T>(sum);
  }
}

// Workgroups of decode_partial<T, D, G> the current device holds at once: the
// kernel's occupancy per CU times the CUs (cached per device).
template <typename T, int D, int G> int64_t partial_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partial<T, D, G>, DEC_THREADS, 0) !=
            hipSuccess || per_cu <= 0)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    n = per_cu * cus;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename T, int D> int64_t partial_slots_for(int G) {
  switch (G) {
    case 1: return partial_slots<T, D, 1>();
    case 2: return partial_slots<T, D, 2>();
    case 4: return partial_slots<T, D, 4>();
    default: return partial_slots<T, D, 8>();
  }
}

// Chunking of a decode step: as many workgroups as the device holds at once
// (a second, partly filled round of them cost about a quarter of the step),
// chunks a multiple of KB.
struct DecodePlan { int G, n_hg, n_chunks, chunk; };

DecodePlan decode_plan(sqa_dtype dt, int64_t d_head, int64_t B, int64_t H_q, int64_t H_kv,
                       int64_t N_max) {
  const int g = (int)(H_q / H_kv);
  DecodePlan pl;
  pl.G = 1;
  while (pl.G < g && pl.G < 8) pl.G *= 2;   // 16 heads' accumulators would spill
  pl.n_hg = (g + pl.G - 1) / pl.G;
  const int64_t slots = dt == SQA_DTYPE_BF16
      ? (d_head == 64 ? partial_slots_for<bf16, 64>(pl.G) : partial_slots_for<bf16, 32>(pl.G))
      : (d_head == 64 ? partial_slots_for<float, 64>(pl.G) : partial_slots_for<float, 32>(pl.G));
  const int64_t units = B * H_kv * pl.n_hg;
  const int64_t max_chunks = (N_max + KB - 1) / KB;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(max_chunks, slots / units));
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

// The chunk states into part, then, with a, their merge into a [B, H_q*D]
// (without a, the caller merges them with decode_merge_out).
template <typename T, int D>
hipError_t decode_impl(const void* q, const void* kc, const void* vc, const int32_t* pos, void* a,
                       float* part, int64_t B, int64_t N_max, int64_t H_q, int64_t H_kv,
                       hipStream_t stream) {
  const DecodePlan pl =
      decode_plan(sizeof(T) == 2 ? SQA_DTYPE_BF16 : SQA_DTYPE_FP32, D, B, H_q, H_kv, N_max);
  DecParams p;
  p.q = q; p.kc = kc; p.vc = vc; p.pos = pos; p.part = part;
  p.N_max = N_max;
  p.H_q = (int)H_q; p.H_kv = (int)H_kv; p.g = (int)(H_q / H_kv); p.n_hg = pl.n_hg;
  p.n_chunks = pl.n_chunks; p.chunk = pl.chunk;
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  const dim3 grid((unsigned)pl.n_chunks, (unsigned)(H_kv * pl.n_hg), (unsigned)B);
  hipError_t e = partial_for<T, D>(pl.G, p, grid, stream);
  if (e != hipSuccess || !a) return e;
  decode_combine<T, D><<<(unsigned)(B * H_q), 256, 0, stream>>>(part, pos, (T*)a, (int)H_q,
                                                              pl.n_chunks, pl.chunk, N_max);
  return hipGetLastError();
}

}  // namespace

size_t decode_partial_bytes(sqa_dtype dt, int64_t B, int64_t H_q, int64_t H_kv, int64_t N_max,
                            int64_t d_head) {
  const DecodePlan pl = decode_plan(dt, d_head, B, H_q, H_kv, N_max);
  return (size_t)(B * H_q * pl.n_chunks * (d_head + 2)) * sizeof(float);
}

hipError_t launch_fill_cache(sqa_dtype dt, const void* k, const void* vt, void* kc, void* vc,
                             int64_t B, int64_t H_kv, int64_t N, int64_t Np, int64_t N_max,
                             int64_t d_head, hipStream_t stream) {
  const int64_t es = dt == SQA_DTYPE_BF16 ? 2 : 4;
  const int64_t BH = B * H_kv;
  const unsigned gy = (unsigned)std::min<int64_t>(BH, 65535);
  const int64_t n16 = N * d_head * es / 16;
  const unsigned gx = (unsigned)std::min<int64_t>(1024, (n16 + 255) / 256);
  copy_rows<<<dim3(gx, gy), 256, 0, stream>>>(
      (const Chunk*)k, (Chunk*)kc, n16, Np * d_head * es / 16, N_max * d_head * es / 16, BH);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + KB - 1) / KB), gy);
  if (dt == SQA_DTYPE_BF16) {
    if (d_head == 64) transpose_v<bf16, 64><<<grid, 256, 0, stream>>>((const bf16*)vt, (bf16*)vc, (int)N, Np, N_max, BH);
    else transpose_v<bf16, 32><<<grid, 256, 0, stream>>>((const bf16*)vt, (bf16*)vc, (int)N, Np, N_max, BH);
  } else {
    if (d_head == 64) transpose_v<float, 64><<<grid, 256, 0, stream>>>((const float*)vt, (float*)vc, (int)N, Np, N_max, BH);
    else transpose_v<float, 32><<<grid, 256, 0, stream>>>((const float*)vt, (float*)vc, (int)N, Np, N_max, BH);
  }
  return hipGetLastError();
}

namespace {
// Grid of a skinny product: SK_COLS columns by SK_BR tokens per workgroup.
template <typename T, typename Store>
hipError_t run_skinny(const void* x, int64_t B, int64_t K, const void* w0, int64_t n0w,
                      const void* w1, int64_t n1w, const void* w2, int64_t n2w, const Store& st,
                      hipStream_t stream) {
  const int64_t ncols = n0w + n1w + n2w, epc = 16 / (int64_t)sizeof(T);
  if (n0w % SK_COLS || n1w % SK_COLS || n2w % SK_COLS || K % epc || ncols / SK_COLS > 65535 ||
      (B + SK_BR - 1) / SK_BR > 65535 || K > INT32_MAX || ncols > INT32_MAX)
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(ncols / SK_COLS), (unsigned)((B + SK_BR - 1) / SK_BR));
  skinny<T, Store><<<grid, 256, 0, stream>>>((const T*)x, (int)B, (int)K, (const T*)w0, (int)n0w,
                                             (const T*)w1, (int)n1w, (const T*)w2, (int)n2w, st);
  return hipGetLastError();
}

template <typename T>
hipError_t decode_qkv(const void* x_new, const void* wq, const void* wk, const void* wv,
                      const int32_t* pos, void* q, void* kc, void* vc, int64_t B, int64_t d_model,
                      int64_t H_q, int64_t H_kv, int64_t d_head, int64_t N_max, hipStream_t stream) {
  const int64_t wq_w = H_q * d_head, wkv_w = H_kv * d_head;
  QkvRows<T> st;
  st.q = (T*)q; st.kc = (T*)kc; st.vc = (T*)vc; st.pos = pos;
  st.wq_w = (int)wq_w; st.wkv_w = (int)wkv_w; st.D = (int)d_head; st.H_kv = (int)H_kv;
  st.N_max = N_max;
  return run_skinny<T>(x_new, B, d_model, wq, wq_w, wk, wkv_w, wv, wkv_w, st, stream);
}

template <typename T>
hipError_t decode_out(const void* a, const void* wo, void* out, int64_t B, int64_t K,
                      int64_t d_model, hipStream_t stream) {
  DenseRows<T> st;
  st.out = (T*)out; st.ncols = (int)d_model;
  return run_skinny<T>(a, B, K, wo, d_model, nullptr, 0, nullptr, 0, st, stream);
}
}  // namespace

hipError_t launch_decode_qkv(sqa_dtype dt, const void* x_new, const void* wq, const void* wk,
                             const void* wv, const int32_t* pos, void* q, void* kc, void* vc,
                             int64_t B, int64_t d_model, int64_t H_q, int64_t H_kv, int64_t d_head,
                             int64_t N_max, hipStream_t stream) {
  return dt == SQA_DTYPE_BF16
      ? decode_qkv<bf16>(x_new, wq, wk, wv, pos, q, kc, vc, B, d_model, H_q, H_kv, d_head, N_max,
                         stream)
      : decode_qkv<float>(x_new, wq, wk, wv, pos, q, kc, vc, B, d_model, H_q, H_kv, d_head, N_max,
                          stream);
}

hipError_t launch_decode_out(sqa_dtype dt, const void* a, const void* wo, void* out, int64_t B,
                             int64_t K, int64_t d_model, hipStream_t stream) {
  return dt == SQA_DTYPE_BF16 ? decode_out<bf16>(a, wo, out, B, K, d_model, stream)
                              : decode_out<float>(a, wo, out, B, K, d_model, stream);
}

bool decode_merge_out_fits(sqa_dtype dt, int64_t B, int64_t N_max, int64_t H_q, int64_t H_kv,
                           int64_t d_head, int64_t d_model) {
  return H_q * d_head <= 8192 && d_model % MC == 0 && d_model / MC <= 0x7FFFFFFF && B <= 65535 &&
         H_q * decode_plan(dt, d_head, B, H_q, H_kv, N_max).n_chunks <= MERGE_MAX_W;
}

hipError_t launch_decode_merge_out(sqa_dtype dt, const void* part, const int32_t* pos,
                                   const void* wo, void* out, int64_t B, int64_t N_max,
                                   int64_t H_q, int64_t H_kv, int64_t d_head, int64_t d_model,
                                   hipStream_t stream) {
  if (!decode_merge_out_fits(dt, B, N_max, H_q, H_kv, d_head, d_model))
    return hipErrorInvalidConfiguration;
  const DecodePlan pl = decode_plan(dt, d_head, B, H_q, H_kv, N_max);
  const int tpr = MC / (dt == SQA_DTYPE_BF16 ? 8 : 4);
  const size_t lds =
      (size_t)(H_q * d_head + H_q * pl.n_chunks + H_q + (256 / tpr) * MC + 8 * MC) * sizeof(float);
  const dim3 grid((unsigned)(d_model / MC), (unsigned)B);
  const float* pf = (const float*)part;
  const int hq = (int)H_q, dm = (int)d_model;
  auto run = [&](auto tc, auto dc, auto fc) {
    using T = decltype(tc);
    decode_merge_out<T, decltype(dc)::value, decltype(fc)::value><<<grid, 256, lds, stream>>>(
        pf, pos, (const T*)wo, (T*)out, hq, pl.n_chunks, pl.chunk, N_max, dm);
  };
  auto run_fp = [&](auto tc, auto dc) {
    if (H_q * d_head <= 512) run(tc, dc, std::integral_constant<int, 1>{});
    else run(tc, dc, std::integral_constant<int, 2>{});
  };
  auto run_d = [&](auto tc) {
    if (d_head == 64) run_fp(tc, std::integral_constant<int, 64>{});
    else run_fp(tc, std::integral_constant<int, 32>{});
  };
  if (dt == SQA_DTYPE_BF16) run_d(bf16{});
  else run_d(0.f);
  return hipGetLastError();
}

hipError_t launch_decode_attention(sqa_dtype dt, const void* q, const void* kc, const void* vc,
                                   const int32_t* pos, void* a, void* part, int64_t B,
                                   int64_t N_max, int64_t H_q, int64_t H_kv, int64_t d_head,
                                   hipStream_t stream) {
  if (B > 65535 || H_kv * ((H_q / H_kv + 7) / 8) > 65535) return hipErrorInvalidConfiguration;
  float* pf = (float*)part;
  if (dt == SQA_DTYPE_BF16)
    return d_head == 64 ? decode_impl<bf16, 64>(q, kc, vc, pos, a, pf, B, N_max, H_q, H_kv, stream)
                        : decode_impl<bf16, 32>(q, kc, vc, pos, a, pf, B, N_max, H_q, H_kv, stream);
  return d_head == 64 ? decode_impl<float, 64>(q, kc, vc, pos, a, pf, B, N_max, H_q, H_kv, stream)
                      : decode_impl<float, 32>(q, kc, vc, pos, a, pf, B, N_max, H_q, H_kv, stream);
}

}  // namespace sqa
