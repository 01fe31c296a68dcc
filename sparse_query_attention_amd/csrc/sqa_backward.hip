// Backward pass of the SQA layer on gfx950: the gradients of L = sum(Y * dY)
// with respect to x and the four weight matrices, for an upstream gradient dY.
//
// The model cards train the SQA layer (ReactiveAI/xSMQAT-m and
// ReactiveAI/GQA-Ref-Micro, training examples), and the paper's abstract puts
// SQA's gains in training. By the chain rule through the forward:
//   dA = dY Wo^T,  dWo = A^T dY
//   per query head i and its key/value head j = floor(i / g), with
//   P = softmax(Q_i K_j^T / sqrt(d)) recomputed from the forward's per-row
//   log-sum-exp, D = rowsum(dO * O):
//     dS = P * (dO V_j^T - D),  dQ_i = dS K_j / sqrt(d)
//     dK_j = sum over the g heads of dS^T Q_i / sqrt(d),  dV_j = sum of P^T dO
//   dX = [dQ | dK | dV] [Wq | Wk | Wv]^T,  [dWq | dWk | dWv] = X^T [dQ | dK | dV]
//
// Attention backward runs as two kernels and needs no atomics:
//  * dkdv: a workgroup of 8 waves owns 256 keys of one key/value head (32 per
//    wave, held as MFMA operands in registers) and walks the query tiles of
//    all g heads of the group, so the g-way sum of dK and dV stays in
//    registers. Per 32-query block: S = Q K^T and dP = dO V^T (lane = key),
//    then dV^T += dO^T P and dK^T += Q^T dS with P and dS consumed from
//    registers as B operands.
//  * dq: a workgroup owns 256 queries of one head (64 per wave) and walks the
//    key tiles: S^T = K Q^T and dP^T = V dO^T (lane = query, so the row's
//    log-sum-exp and D are per-lane scalars), then dQ^T += K^T dS^T.
// Both stream their tiles through rings of LDS slots filled by direct loads,
// pair their tiles so that concurrent workgroups read the same tiles (L2
// reuse), and run the tiles that need no mask in loops without mask code.
// The contraction over the score rows needs the other operand with those rows
// contiguous, so Q^T, dO^T, K^T (tokens in swap23 order) and V row-major are
// written once by a transpose kernel. Token-contiguous copies of X, A, dY and
// [dQ|dK|dV] feed the weight-gradient products (split-K over all tokens).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

// The LDS pointer p, with a value the compiler cannot see: the address of a
// read at a constant offset from it is then one register (p plus the lane's
// part, computed once) and an immediate, where from a known base beyond the
// 64 KB reach of the immediate every offset would take a register of its own.
template <typename T> __device__ __attribute__((always_inline)) inline const T* opaque_lds(const T* p) {
  auto q = (__attribute__((address_space(3))) const T*)p;
  asm("" : "+v"(q));
  return (const T*)q;
}

// f(std::integral_constant<int, i>) for i = I .. N-1, in order.
template <int I, int N, typename F> __device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ inline float f32_of(float x) { return x; }
__device__ inline float f32_of(bf16 x) { return (float)x; }

// ---- layout helpers ----

// dst[b][c][r] = src[b][r][c] for r < r_valid, 0 for r_valid <= r < r_total;
// c < C. 64x64 tiles through LDS, 16-byte global accesses on both sides
// (C and r_total are multiples of 16 / sizeof(T)). With PERM the rows land in
// swap23 order within each group of 16: dst[b][c][swap23(r)] = src[b][r][c].
// The tiles of all batches are numbered along x, column tiles fastest (rows,
// columns and batches can each run past the 65535 limit of the y and z
// dimensions).
template <typename T, bool PERM>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, int64_t src_bs, int64_t src_ld,
                                                        int r_valid, int r_total, T* dst,
                                                        int64_t dst_bs, int64_t dst_ld, int C) {
  constexpr int EPC = 16 / (int)sizeof(T), TP = 64 + EPC;   // padded LDS row
  __shared__ __align__(16) T tile[64][TP];
  const int n_ct = (C + 63) / 64;
  const int64_t per_batch = (int64_t)((r_total + 63) / 64) * n_ct;
  const int64_t bz = blockIdx.x / per_batch, t = blockIdx.x % per_batch;
  const int c0 = (int)(t % n_ct) * 64, r0 = (int)(t / n_ct) * 64;
  src += bz * src_bs;
  dst += bz * dst_bs;
  constexpr int CPR = 64 / EPC;   // chunks per 64-element line
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, cc = (i % CPR) * EPC;
    Chunk v = zero_chunk();
    if (r0 + r < r_valid && c0 + cc < C)
      v = *reinterpret_cast<const Chunk*>(src + (int64_t)(r0 + r) * src_ld + c0 + cc);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int k = 0; k < EPC; ++k) tile[cc + k][PERM ? swap23(r) : r] = e[k];   // tile[c][r]
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int c = i / CPR, rr = (i % CPR) * EPC;
    if (c0 + c < C && r0 + rr < r_total)
      *reinterpret_cast<Chunk*>(dst + (int64_t)(c0 + c) * dst_ld + r0 + rr) =
          *reinterpret_cast<const Chunk*>(&tile[c][rr]);
  }
}

// W_all [d_model, wq + 2*wkv] rows = [Wq row | Wk row | Wv row].
template <typename T>
__global__ __launch_bounds__(256) void concat_weights(const T* wq, const T* wk, const T* wv, T* w,
                                                      int64_t d_model, int wq_w, int wkv_w) {
  const int W = wq_w + 2 * wkv_w;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= d_model * W) return;
  const int64_t r = i / W;
  int c = (int)(i % W);
  T v;
  if (c < wq_w) v = wq[r * wq_w + c];
  else if ((c -= wq_w) < wkv_w) v = wk[r * wkv_w + c];
  else v = wv[r * wkv_w + c - wkv_w];
  w[i] = v;
}

// dvec[b, i, t] = -D with D = sum_c dO[b, i, t, c] * O[b, t, i*d + c] for
// t < N, 0 on padding rows, with O the attention output before its rounding
// (fp32). The rounded A would put a relative 2^-9 error into D, and
// dS = P (dP - D) keeps it even where dP - D cancels (short sequences). It is
// stored negated because the dK/dV kernel starts its dP accumulation from it.
// nlse[b, i, t] = -lse / c (lse the base-2 log-sum-exp of the scaled scores,
// c = log2(e) / sqrt(d)), -inf on padding rows: the dK/dV kernel starts its
// S accumulation from it, so that a probability is exp2(c * acc).
// Eight lanes share a row, each with D/8 consecutive elements of it, so that a
// wave reads eight whole rows of dO and of O with vector loads (one row per
// thread had made every load instruction touch 64 lines: 1.6 TB/s). The eight
// partial sums meet in a fixed butterfly.
template <typename T, int D>
__global__ __launch_bounds__(256) void dvec_kernel(const T* dO, const float* a, const float* lse,
                                                   float c, float* dvec, float* nlse, int N,
                                                   int64_t Np, int H_q, int64_t rows) {
  constexpr int EPL = D / 8;   // elements per lane
  struct alignas(EPL * sizeof(T)) TV { T v[EPL]; };
  struct alignas(EPL * 4 >= 16 ? 16 : EPL * 4) FV { float v[EPL]; };
  const int64_t x = (int64_t)blockIdx.x * 32 + threadIdx.x / 8;
  const int sub = threadIdx.x % 8;
  const int64_t xr = x < rows ? x : rows - 1;   // every lane of the wave takes part in the butterfly
  const int64_t t = xr % Np, bi = xr / Np, i = bi % H_q, b = bi / H_q;
  float s = 0.f;
  if (t < N) {
    const TV o = *reinterpret_cast<const TV*>(dO + xr * D + sub * EPL);
    const FV av = *reinterpret_cast<const FV*>(a + ((b * N + t) * H_q + i) * D + sub * EPL);
#pragma unroll
    for (int k = 0; k < EPL; ++k) s = fmaf(f32_of(o.v[k]), av.v[k], s);
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (sub == 0 && x < rows) {
    dvec[x] = -s;
    nlse[x] = t < N ? -lse[x] / c : -INFINITY;
  }
}

// out segments [M, w0 | w1 | w2] = sum over the n_split partials, rounded once.
template <typename T>
__global__ __launch_bounds__(256) void reduce_splits(const float* part, int n_split, int64_t M,
                                                     int ncols, T* o0, int w0, T* o1, int w1, T* o2,
                                                     int w2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * ncols) return;
  const int64_t m = i / ncols;
  int n = (int)(i % ncols);
  float v = 0.f;
  for (int s = 0; s < n_split; ++s) v += part[(int64_t)s * M * ncols + i];
  const T r = from_f32<T>(v);
  if (n < w0) o0[m * w0 + n] = r;
  else if ((n -= w0) < w1) o1[m * w1 + n] = r;
  else o2[m * w2 + n - w1] = r;
}

// ---- attention backward ----

struct BwdParams {
  const void* q;     // [B, H_q, Np, d]
  const void* qt;    // [B, H_q, d, Np], tokens in swap23 order
  const void* k;     // [B, H_kv, Np, d]
  const void* kt;    // [B, H_kv, d, Np], tokens in swap23 order
  const void* v;     // [B, H_kv, Np, d]
  const void* dO;    // [B, H_q, Np, d]
  const void* dOt;   // [B, H_q, d, Np], tokens in swap23 order
  const float* lse;  // [B, H_q, Np], base 2, of the scaled scores
  const float* nlse; // [B, H_q, Np]: -lse / c
  const float* dvec; // [B, H_q, Np]: -D per row
  void* dqkv;        // [B, Np, W]: dQ heads, then dK heads, then dV heads
  int N, Np, H_q, H_kv, g, causal, W;
  float c;           // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
};

constexpr int BT = 64;   // tokens per LDS tile

// Operand tiles in LDS, as the direct loads place them: 16-byte chunks
// XOR-swizzled per row (swz) so that the rows one 16-byte read touches sit on
// distinct banks.
// Row-major tile [64 tokens][D]: the MFMA operand of row `row`, k-step st over
// the head dims.
template <typename T, int D>
__device__ inline typename Mfma<T>::Frag row_frag(const T* tile, int row, int st, int grp) {
  constexpr int EPC = 16 / (int)sizeof(T), RC = D / EPC;
  const int e = st * Mfma<T>::KS + grp * Mfma<T>::E;
  return *reinterpret_cast<const typename Mfma<T>::Frag*>(tile + row * D + ((e / EPC) ^ swz<RC>(row)) * EPC +
                                                           e % EPC);
}

// Transposed tile [D][64 tokens], tokens in swap23 order: the A operand of line
// `line` that matches a B operand packed from accumulator registers. For
// k-step `half` of the 32-row block at `base`, k-group grp holds rows
// base + 16*half + 8*(e/4) + 4*grp + e%4 (e = 0..7), at positions
// base + 16*half + 8*grp + e; for fp32, k-step st (0..15) holds row
// base + 8*(st/4) + 4*grp + st%4, at position base + 16*(st/8) + 8*grp + st%8.
template <typename T>
__device__ inline typename Mfma<T>::Frag line_frag(const T* tile, int line, int base, int half, int grp) {
  constexpr int EPC = 16 / (int)sizeof(T), LC = 64 / EPC;
  const int pos = sizeof(T) == 2 ? base + 16 * half + 8 * grp : base + 16 * (half / 8) + 8 * grp + half % 8;
  return *reinterpret_cast<const typename Mfma<T>::Frag*>(tile + line * 64 + ((pos / EPC) ^ swz<LC>(line)) * EPC +
                                                           pos % EPC);
}

// B operand from accumulator registers x (C layout): k-step `half`.
template <typename T>
__device__ inline typename Mfma<T>::Frag frag_regs(const f32x16& x, int half) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)x[8 * half + e];
    return f;
  } else {
    return x[half];
  }
}

template <typename T> constexpr int kHalves = sizeof(T) == 2 ? 2 : 16;   // k-steps per 32 rows

// dK, dV: workgroup = (key tiles of 256 keys, KV head j, batch b); 8 waves x
// 32 keys. The query-side operand tiles (Q, dO, Q^T, dO^T and the rows' lse
// and D) of each 64-query tile go straight from global memory into a ring of
// LDS slots (buffer loads into LDS), NBUF-1 tiles ahead of the one in use; no
// registers hold them in transit. Row-major tiles [64][D] and transposed tiles
// [D][64] keep their 16-byte chunks XOR-swizzled per row, so the MFMA operand
// reads are free of bank conflicts.
//
// Order of the work. Every query tile is read by every key tile at or before
// it, and the workgroups that run at once on an XCD share its L2 only if they
// read the same tiles at the same time. Causal: workgroup pr takes key tile
// pr, walking its query tiles from the last one down, then key tile
// n_kt-1-pr, walking up from its first. Each workgroup then has the same
// number of items, and at step tau every workgroup in its first half reads
// query tile qt_end-1-tau and every one in its second half the same tile
// 4*(n_kt-1)-qt_end+tau, whatever pr is. Without a mask every workgroup walks
// all query tiles upward. Within a query tile the g heads are adjacent.
template <typename T, int D>
__global__ __launch_bounds__(512, 2) void bwd_dkdv(BwdParams p) {
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  constexpr int WAVES = 8, KPW = 32, KPG = WAVES * KPW;   // keys per wave, per workgroup
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int RC = D / EPC, LC = BT / EPC;   // chunks per row [64][D], per line [D][64]
  constexpr int NS = D / MF::KS;               // k-steps over the head dims
  constexpr int TE = BT * D;                   // elements of one operand tile
  constexpr int SE = 2 * BT * 4 / (int)sizeof(T);   // elements holding the rows' -lse/c and -D (fp32)
  constexpr int NBUF = 4 * TE * (int)sizeof(T) <= 32768 ? 4 : 2;   // ring slots (LDS <= 130 KB)
  constexpr int INS = TE * (int)sizeof(T) / 1024;                 // 1 KB loads per operand tile
  constexpr int IPW = 4 * INS / WAVES;                            // per wave and tile
  constexpr int VM_PER_TILE = IPW + 1;                            // and one of row statistics
  static_assert(IPW * WAVES == 4 * INS && INS * 64 * EPC == TE, "tile split");
  // One array for every direct-load target: the compiler then sees the
  // ring's reads and the loads in flight into other slots as one object and
  // adds no waits of its own between them. It is laid out by operand: the
  // NBUF slots of Q rows, then those of dO rows, Q^T, dO^T and the row
  // statistics. The slots of the row tiles (Q, dO) then span 64 KB, as do
  // those of the line tiles (Q^T, dO^T), so where a slot is known at compile
  // time a fragment read's address is a per-lane register plus an immediate.
  __shared__ __align__(16) T smem[NBUF * (4 * TE + SE)];
  // operand tile a (0: Q, 1: dO, 2: Q^T, 3: dO^T) of ring slot s
  const T* line_tiles = opaque_lds<T>(smem + 2 * NBUF * TE);
  auto tile = [&](int a, int s) __attribute__((always_inline)) {
    return a < 2 ? (const T*)smem + (a * NBUF + s) * TE : line_tiles + ((a - 2) * NBUF + s) * TE;
  };
  // the rows' -lse/c (BT values), then their -D (BT values), in ring slot s
  const float* stat_tiles = opaque_lds<float>(reinterpret_cast<const float*>(smem + 4 * NBUF * TE));
  auto stats = [&](int s) __attribute__((always_inline)) { return stat_tiles + s * (SE * (int)sizeof(T) / 4); };

  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int col = lane & 31, grp = lane >> 5;
  const int n_kt = p.Np / KPG;
  const int n_bj = gridDim.x / (p.causal ? (n_kt + 1) / 2 : n_kt);
  const int pr = blockIdx.x / n_bj, bj = blockIdx.x % n_bj;
  const int j = bj % p.H_kv, b = bj / p.H_kv;
  const int kt0 = pr, kt1 = n_kt - 1 - pr;
  const int qt_end = (p.N + BT - 1) / BT;
  // Items: phase 0 is key tile kt0, phase 1 (causal, kt1 != kt0) key tile kt1.
  // Causal key tile kt sees the query tiles from the one holding its first
  // key. Every row of the tiles walked has its -lse/c and -D written: -inf
  // and 0 past N.
  const int first0 = p.causal ? kt0 * (KPG / BT) : 0;
  const int first1 = kt1 * (KPG / BT);
  const int n0 = max(0, qt_end - first0) * p.g;
  const int n_work = n0 + (p.causal && kt1 != kt0 ? max(0, qt_end - first1) * p.g : 0);

  // item -> query tile (the head within the group: (w < n0 ? w : w - n0) % g)
  auto item_tile = [&](int w) {
    if (w < n0) return p.causal ? qt_end - 1 - w / p.g : w / p.g;
    return first1 + (w - n0) / p.g;
  };

  const T* Kh = (const T*)p.k + ((int64_t)b * p.H_kv + j) * (int64_t)p.Np * D;
  const T* Vh = (const T*)p.v + ((int64_t)b * p.H_kv + j) * (int64_t)p.Np * D;

  // Loads of work item w into ring slot w % NBUF. Load `ins` of the tile's
  // 4*INS covers 64 16-byte chunks of one operand tile; lane L's chunk lands
  // at position 64*ins + L, which holds chunk (c ^ swz(row)) of its row. All
  // of a wave's loads fall in one operand tile (arr), and their per-lane byte
  // offsets are the same for every item, so they are computed once; an item
  // only moves the wave-uniform base.
  static_assert(INS % IPW == 0, "a wave's loads within one operand tile");
  const int arr = wave * IPW / INS;
  uint32_t loff[IPW];
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int pos = (wave * IPW + x) % INS * 64 + lane;
    if (arr < 2) {   // Q, dO rows
      const int r = pos / RC, c = pos % RC;
      loff[x] = (uint32_t)((r * D + (c ^ swz<RC>(r)) * EPC) * (int)sizeof(T));
    } else {         // Q^T, dO^T lines (tokens in swap23 order)
      const int r = pos / LC, c = pos % LC;
      loff[x] = (uint32_t)r * (uint32_t)p.Np * (uint32_t)sizeof(T) + (uint32_t)((c ^ swz<LC>(r)) * EPC * (int)sizeof(T));
    }
  }
  const T* arr_base = (const T*)(arr == 0 ? p.q : arr == 1 ? p.dO : arr == 2 ? p.qt : p.dOt);
  const int which = wave >> 2, part = wave & 3;   // row statistics: -lse/c (waves 0-3), -D (4-7)
  // Items are issued in order, so the next one's query tile and head are
  // stepped along instead of divided out of its index (item_tile, and the head):
  // the scalar work per item shrinks. it_soff = (b*H_q + head) * Np, the head's
  // offset in the row statistics; times D it is the head's element offset in
  // Q, dO ([.., Np, D]) and in Q^T, dO^T ([.., D, Np]) alike.
  int next_issue = 0;
  int it_tile = n0 > 0 ? (p.causal ? qt_end - 1 : 0) : first1, it_head = 0;
  const int64_t it_soff0 = ((int64_t)b * p.H_q + (int64_t)j * p.g) * p.Np;
  int64_t it_soff = it_soff0;
  auto issue_next = [&]() {
    const int w = next_issue++;
    if (w >= n_work) return;
    const int q0 = it_tile * BT;
    const int64_t hoff = it_soff * D;
    T* tb = smem + (arr * NBUF + w % NBUF) * TE;
    const T* base = arr_base + hoff + (arr < 2 ? (int64_t)q0 * D : (int64_t)q0);
    // Buffer loads: unlike global_load_lds, they count only in vmcnt, so the
    // compiler's waits for the LDS fragment reads in flight stay exact
    // (with a global_load_lds in flight it waits for every LDS read). The
    // byte offsets stay below 2^32: the host checks D * Np * sizeof(T).
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, (short)0, (int)(arr < 2 ? TE * (uint32_t)sizeof(T) : (uint32_t)(D - 1) * (uint32_t)p.Np * (uint32_t)sizeof(T) + BT * (uint32_t)sizeof(T)),
        0x00020000);
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int li = (wave * IPW + x) % INS;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(tb + li * 64 * EPC), 16, (int)loff[x], 0, 0, 0);
    }
    // row statistics: 16 values per wave
    const float* src = (which ? p.dvec : p.nlse) + it_soff + q0 + part * 16;
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, 64, 0x00020000);
    float* dst = reinterpret_cast<float*>(smem + 4 * NBUF * TE + (w % NBUF) * SE) + which * BT + part * 16;
    if (lane < 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (lds_ptr)dst, 4, lane * 4, 0, 0, 0);
    // step to item w + 1 (its query tile and head)
    if (w + 1 == n0) {
      it_tile = first1; it_head = 0; it_soff = it_soff0;
    } else if (++it_head == p.g) {
      it_head = 0; it_soff = it_soff0;
      it_tile += (w + 1 < n0 && p.causal) ? -1 : 1;
    } else {
      it_soff += p.Np;
    }
  };

  // This wave's K and V fragments (B operands of S = Q K^T and dP = dO V^T)
  // for the key tile starting at key k0, and the store of its dK and dV.
  Frag kf[NS], vf[NS];
  auto load_kv = [&](int kw) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int64_t key = kw + col;
      kf[s] = *reinterpret_cast<const Frag*>(Kh + key * D + s * MF::KS + grp * MF::E);
      vf[s] = *reinterpret_cast<const Frag*>(Vh + key * D + s * MF::KS + grp * MF::E);
    }
  };
  f32x16 dk[D / 32], dv[D / 32];
  // dK^T, dV^T: lane = key, register r = head dim 32*nb + 8*(r/4) + 4*grp + r%4.
  auto store_dkdv = [&](int kw) {
    T* row = (T*)p.dqkv + ((int64_t)b * p.Np + kw + col) * p.W;
    T* dkr = row + (int64_t)p.H_q * D + j * D;
    T* dvr = row + (int64_t)(p.H_q + p.H_kv) * D + j * D;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = nb * 32 + 8 * rq + 4 * grp;
        const f32x16& K_ = dk[nb];
        const f32x16& V_ = dv[nb];
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x4*>(dkr + c) =
              bf16x4{(bf16)(K_[4 * rq] * p.scale), (bf16)(K_[4 * rq + 1] * p.scale),
                     (bf16)(K_[4 * rq + 2] * p.scale), (bf16)(K_[4 * rq + 3] * p.scale)};
          *reinterpret_cast<bf16x4*>(dvr + c) =
              bf16x4{(bf16)V_[4 * rq], (bf16)V_[4 * rq + 1], (bf16)V_[4 * rq + 2], (bf16)V_[4 * rq + 3]};
        } else {
          *reinterpret_cast<f32x4*>(dkr + c) =
              f32x4{K_[4 * rq] * p.scale, K_[4 * rq + 1] * p.scale, K_[4 * rq + 2] * p.scale,
                    K_[4 * rq + 3] * p.scale};
          *reinterpret_cast<f32x4*>(dvr + c) = f32x4{V_[4 * rq], V_[4 * rq + 1], V_[4 * rq + 2], V_[4 * rq + 3]};
        }
      }
  };

  // Ring bookkeeping. Tiles [0, next_issue) have been issued; tile x lives in
  // slot x % NBUF. sync(R, F) waits until this wave's loads of the tiles up to
  // R have landed, then passes a barrier (every wave's loads of those tiles
  // are visible, and every wave is done with the tiles before F), then issues
  // the tiles whose slots that frees, up to F + NBUF - 1.
  auto sync = [&](int R, int F) {
    wait_vmcnt_tiles<VM_PER_TILE, NBUF - 2>(min(NBUF - 2, max(0, next_issue - 1 - R)));
    ring_barrier();
    const int last = min(F + NBUF - 1, n_work - 1);
    while (next_issue <= last) issue_next();
  };

  // Prologue: work items 0..NBUF-2 in flight, then the K and V fragments of
  // the first key tile, all landed before the loop, which then waits only on
  // its own loads.
  int kw = kt0 * KPG + KPW * wave;   // this wave's first key
  while (next_issue < min(NBUF - 1, n_work)) issue_next();
  load_kv(kw);
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = f32x16{}; dv[nb] = f32x16{}; }
  if constexpr (sizeof(T) == 2) {
    // The line tiles of the last slot start as zeros: a pipelined run that
    // starts at item 0 reads them as the tiles of its (absent) previous item
    // and multiplies them by zeros, which must not meet an Inf or NaN.
    constexpr int ZC = TE * (int)sizeof(T) / 16;   // 16-byte chunks per tile
#pragma unroll
    for (int a = 2; a < 4; ++a)
      for (int x = tid; x < ZC; x += WAVES * 64)
        reinterpret_cast<f32x4*>(smem + (a * NBUF + NBUF - 1) * TE)[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  wait_vmcnt<0>();
  __syncthreads();

  // The accumulators of S and dP - D for the 32 query rows at rb of a tile
  // start from the rows' -lse/c and -D (register r: row rb + 8*(r/4) + 4*grp
  // + r%4). The probability is then exp2(c * S) and dS = P (dP - D) one
  // product, with no per-score subtraction.
  auto init_scores = [&](int s, int rb, f32x16& sc, f32x16& dpc) __attribute__((always_inline)) {
    const float* st = stats(s);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&st[rb + 8 * r4 + 4 * grp]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&st[BT + rb + 8 * r4 + 4 * grp]);
#pragma unroll
      for (int e = 0; e < 4; ++e) { sc[4 * r4 + e] = n4[e]; dpc[4 * r4 + e] = d4[e]; }
    }
  };

  // Items [w0, w1), one at a time, each of its 32-query blocks through
  // scores, softmax gradient and the dV/dK products. Used for the items that
  // need a mask, and in fp32 for all.
  auto run_items = [&](int w0, int w1, auto mask_on) {
    constexpr bool MASK = decltype(mask_on)::value;
    for (int w = w0; w < w1; ++w) {
      // item w visible; every wave done with the items before it
      sync(w, w);
      const int sw = w % NBUF;
      const T* Qs = tile(0, sw);
      const T* Os = tile(1, sw);
      const T* QTs = tile(2, sw);
      const T* OTs = tile(3, sw);
      const int q0 = item_tile(w) * BT;
      // S and dP - D of 32-query block qs (lane = key)
      auto scores = [&](int qs, f32x16& sc, f32x16& dpc) {
        Frag qa[NS], oa[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          qa[st] = row_frag<T, D>(Qs, 32 * qs + col, st, grp);
          oa[st] = row_frag<T, D>(Os, 32 * qs + col, st, grp);
        }
        init_scores(sw, 32 * qs, sc, dpc);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          sc = MF::run(qa[st], kf[st], sc);
          dpc = MF::run(oa[st], vf[st], dpc);
        }
      };
      // P and dS in place (register r: query qb + 8*(r/4) + 4*grp + r%4; column:
      // key kw + col), then dV^T += dO^T P and dK^T += Q^T dS.
      auto grads = [&](int qs, f32x16& sc, f32x16& dpc) {
        const int qb = q0 + 32 * qs;
        const int key = kw + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb + 8 * (r / 4) + 4 * grp + r % 4;
          float pv = __builtin_amdgcn_exp2f(sc[r] * p.c);
          if (MASK) pv = key >= p.N || (p.causal && key > q) ? 0.f : pv;
          sc[r] = pv;                        // P
          dpc[r] = pv * dpc[r];              // dS = P (dP - D)
        }
#pragma unroll
        for (int h = 0; h < kHalves<T>; ++h)
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) {
            dv[nb] = MF::run(line_frag<T>(OTs, nb * 32 + col, 32 * qs, h, grp), frag_regs<T>(sc, h), dv[nb]);
            dk[nb] = MF::run(line_frag<T>(QTs, nb * 32 + col, 32 * qs, h, grp), frag_regs<T>(dpc, h), dk[nb]);
          }
      };
      if constexpr (!MASK) {
        f32x16 s0, dp0, s1, dp1;
        scores(0, s0, dp0);
        scores(1, s1, dp1);
        grads(0, s0, dp0);
        grads(1, s1, dp1);
      } else {
#pragma unroll
        for (int qs = 0; qs < BT / 32; ++qs) {
          const int qb = q0 + 32 * qs;
          // wave-uniform skips: every query before this wave's first key, or past N
          if ((p.causal && qb + 31 < kw) || qb >= p.N) continue;
          f32x16 sc, dpc;
          scores(qs, sc, dpc);
          grads(qs, sc, dpc);
        }
      }
    }
  };

  // bf16 items [w0, w1) that need no mask, as a software pipeline over the
  // 32-query blocks (two per item). A block passes three stages: its scores S
  // and dP - D (MFMA), the softmax gradient P and dS (VALU, packed to bf16),
  // and the products dV^T += dO^T P, dK^T += Q^T dS (MFMA). Iteration w runs
  // two phases of 2*NS + 4*D/32 MFMAs each:
  //   phase 0: dV/dK of block 1 of item w-1, scores of block 1 of item w;
  //            softmax gradient of block 0 of item w
  //   phase 1: dV/dK of block 0 of item w, scores of block 0 of item w+1;
  //            softmax gradient of block 1 of item w
  // so each phase's VALU work is independent of its MFMAs. Each MFMA forms a
  // group with an equal share of the phase's VALU work and the LDS read of
  // the fragment FA groups ahead; sched_barrier keeps the groups in order.
  // An iteration reads the tiles of items w-1, w and w+1, so the ring keeps
  // one item in flight beyond them.
  auto run_clear = [&](int w0, int w1) {
    if constexpr (sizeof(T) != 2) {
      run_items(w0, w1, std::false_type{});
      return;
    } else {
    if (w0 >= w1) return;
    constexpr int NB = D / 32;
    constexpr int NGG = 4 * NB;      // dV/dK MFMAs of a block
    constexpr int NGS = 2 * NS;      // S/dP MFMAs of a block
    constexpr int NGP = NGG + NGS;   // MFMAs (groups) of a phase
    constexpr int SPG = 16 / NGP;    // scores per group
    constexpr int FA = 3;            // fragment reads ahead
    static_assert(SPG * NGP == 16 && FA <= NGG, "groups");
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x16 sA, dA, sB, dB;           // S and dP - D of block 0 (A) and block 1 (B)
    u32x4 pA[2][2], pB[2][2];        // [P, dS][half]: bf16 pairs, B operands
    Frag fr[2 * NGP];                // the fragment of each MFMA of an iteration
    // The fragment of MFMA u of the iteration over the ring slots of items
    // w-1 (prev), w (cur) and w+1 (next).
    auto fetch = [&](auto uc, int prev, int cur, int next) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value, ph = u / NGP, k = u % NGP;
      if constexpr (k < NGG) {
        constexpr int h = k / (2 * NB), nb = (k / 2) % NB, which = k % 2;   // 0: dV (dO^T), 1: dK (Q^T)
        fr[u] = line_frag<T>(tile(which ? 2 : 3, ph == 0 ? prev : cur), nb * 32 + col, ph == 0 ? 32 : 0, h, grp);
      } else {
        constexpr int st = (k - NGG) / 2, which = (k - NGG) % 2;             // 0: S (Q), 1: dP (dO)
        fr[u] = row_frag<T, D>(tile(which, ph == 0 ? cur : next), (ph == 0 ? 32 : 0) + col, st, grp);
      }
    };
    // dV/dK MFMA k (< NGG) of a block with packed P and dS pk
    auto grad_mfma = [&](auto kc, const Frag& a, const u32x4 (&pk)[2][2]) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, h = k / (2 * NB), nb = (k / 2) % NB, which = k % 2;
      const Frag b = __builtin_bit_cast(Frag, pk[which][h]);
      if constexpr (which == 0) dv[nb] = MF::run(a, b, dv[nb]);
      else dk[nb] = MF::run(a, b, dk[nb]);
    };
    float ex[16], ds[16];
    auto group = [&](auto uc, int prev, int cur, int next) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value, ph = u / NGP, k = u % NGP;
      f32x16& s_sc = ph == 0 ? sB : sA;   // scored in this phase
      f32x16& d_sc = ph == 0 ? dB : dA;
      const f32x16& s_sm = ph == 0 ? sA : sB;   // softmax gradient in this phase
      const f32x16& d_sm = ph == 0 ? dA : dB;
      u32x4 (&p_sm)[2][2] = ph == 0 ? pA : pB;
      // the fragment FA groups ahead; past the iteration's end, the first
      // groups of the next one (dV/dK of block 1 of item w: tile cur)
      if constexpr (u + FA < 2 * NGP) fetch(std::integral_constant<int, u + FA>{}, prev, cur, next);
      else fetch(std::integral_constant<int, u + FA - 2 * NGP>{}, cur, cur, cur);
      if constexpr (k == NGG - FA) {   // accumulators of the block scored next, before its first MFMA
        if constexpr (ph == 0) init_scores(cur, 32, sB, dB);
        else init_scores(next, 0, sA, dA);
      }
      if constexpr (k < NGG) {
        grad_mfma(std::integral_constant<int, k>{}, fr[u], ph == 0 ? pB : pA);
      } else {
        constexpr int st = (k - NGG) / 2, which = (k - NGG) % 2;
        if constexpr (which == 0) s_sc = MF::run(fr[u], kf[st], s_sc);
        else d_sc = MF::run(fr[u], vf[st], d_sc);
      }
      // softmax gradient of scores [k*SPG, (k+1)*SPG); exponentials one group ahead
      if constexpr (k == 0) {
#pragma unroll
        for (int q = 0; q < SPG; ++q) ex[q] = __builtin_amdgcn_exp2f(s_sm[q] * p.c);
      }
#pragma unroll
      for (int q = 0; q < SPG; ++q) {
        const int r = k * SPG + q;
        if (k + 1 < NGP) ex[r + SPG] = __builtin_amdgcn_exp2f(s_sm[r + SPG] * p.c);
        ds[r] = ex[r] * d_sm[r];
        if (r % 2 == 1) {
          p_sm[0][r / 8][(r % 8) / 2] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{ex[r - 1], ex[r]}, bf16x2));
          p_sm[1][r / 8][(r % 8) / 2] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{ds[r - 1], ds[r]}, bf16x2));
        }
      }
      // within the group: the MFMA, the LDS reads, then the VALU work, so
      // that the MFMAs of consecutive groups never issue back to back
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: tile w0 visible; scores of its block 0. The P and dS of
    // block "1 of item w0-1" are zeros, so the first phase's dV/dK MFMAs add
    // exact zeros: their other operands, the tiles in the slot before w0's,
    // hold item w0-1 (finite) or, before item 0, zeros.
    sync(w0, w0);
    {
      const int s0 = w0 % NBUF;
      init_scores(s0, 0, sA, dA);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        sA = MF::run(row_frag<T, D>(tile(0, s0), col, st, grp), kf[st], sA);
        dA = MF::run(row_frag<T, D>(tile(1, s0), col, st, grp), vf[st], dA);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int h = 0; h < 2; ++h) pB[a][h] = u32x4{0u, 0u, 0u, 0u};
      static_for<0, FA>([&](auto uc) { fetch(uc, (s0 + NBUF - 1) % NBUF, s0, s0); });
    }
    // Iteration w reads the slots of items w-1 (prev), w (cur) and w+1
    // (next; past the loop's end, item w+1's scores are computed and
    // dropped). There is one copy of it per slot of w, so that every slot is
    // a compile-time constant.
    for (int w = w0; w < w1; ++w) {
      // items w and w+1 visible; every wave done with the items before w-1
      sync(w + 1, w - 1);
      const int m = w % NBUF;
      static_for<0, NBUF>([&](auto mc) {
        constexpr int c = decltype(mc)::value;
        if (m == c) static_for<0, 2 * NGP>([&](auto uc) { group(uc, (c + NBUF - 1) % NBUF, c, (c + 1) % NBUF); });
      });
    }
    // Epilogue: dV/dK of block 1 of the last item (its first FA fragments
    // were read in the last iteration).
    const int lt = (w1 - 1) % NBUF;
    static_for<0, NGG>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k >= FA) fetch(kc, lt, lt, lt);
      grad_mfma(kc, fr[k], pB);
    });
    }
  };

  // Query tiles walked for key tile kt that see all of its keys: with a mask
  // the ones after its last key, [4kt + 4, qt_end); without one, all. None if
  // the key tile reaches past N.
  auto clear_tiles = [&](int kt) {
    if ((kt + 1) * KPG > p.N) return 0;
    return p.causal ? max(0, qt_end - (kt + 1) * (KPG / BT)) : qt_end;
  };
  // Phase 0 walks its query tiles downward (upward without a mask, where they
  // are all clear or all masked): the clear ones first.
  const int c0 = min(n0, clear_tiles(kt0) * p.g);
  run_clear(0, c0);
  run_items(c0, n0, std::true_type{});
  if (n_work > n0) {   // second key tile: store the first one's gradients
    store_dkdv(kw);
    kw = kt1 * KPG + KPW * wave;
    load_kv(kw);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = f32x16{}; dv[nb] = f32x16{}; }
    wait_vmcnt<0>();
    // Phase 1 walks its query tiles upward: the clear ones last.
    const int m1 = max(n0, n_work - clear_tiles(kt1) * p.g);
    run_items(n0, m1, std::true_type{});
    run_clear(m1, n_work);
  }
  // The last key tile's gradients. A key tile that no query reaches (wholly
  // past N) stores zeros: the weight gradients read those padding rows.
  store_dkdv(kw);
  if (p.causal && kt1 != kt0 && n_work == n0) {
    kw = kt1 * KPG + KPW * wave;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = f32x16{}; dv[nb] = f32x16{}; }
    store_dkdv(kw);
  }
}

// dQ (fp32, and bf16 at d_head 32; bwd_dq_pipe below serves bf16 at d_head
// 64): workgroup = (query tiles of 256 queries, head i, batch b); 4 waves x 64
// queries. The key-side tiles (K, V and K^T, 64 keys each) go straight from
// global memory into a ring of LDS slots (buffer loads into LDS), NBUF-1 tiles
// ahead of the one in use, XOR-swizzled per row as in bwd_dkdv.
//
// Order of the work, for L2 reuse as in bwd_dkdv: causal workgroup pr takes
// query tile pr, walking its key tiles upward from the first, then query tile
// n_qt-1-pr, walking its key tiles down from the last one it sees. Every
// workgroup has the same number of items, and at each step all workgroups in
// the same half read the same key tile. Without a mask every workgroup walks
// all key tiles upward.
// (one wave per SIMD for fp32 at d_head 64: its fragments take more registers than two waves have)
template <typename T, int D>
__global__ __launch_bounds__(256, sizeof(T) == 2 || D < 64 ? 2 : 1) void bwd_dq(BwdParams p) {
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  constexpr int WAVES = 4;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int RC = D / EPC, LC = BT / EPC;   // chunks per row [64][D], per line [D][64]
  constexpr int NS = D / MF::KS;
  constexpr int QB = 2;                        // 32-query MFMA column blocks per wave
  constexpr int TE = BT * D;
  constexpr int TILE = 3 * TE;                 // K, V, K^T
  constexpr int NBUF = TILE * (int)sizeof(T) <= 24576 ? 3 : 2;   // two workgroups per CU
  constexpr int INS = TE * (int)sizeof(T) / 1024;
  constexpr int IPW = 3 * INS / WAVES;
  constexpr int VM_PER_TILE = IPW;
  static_assert(IPW * WAVES == 3 * INS && INS * 64 * EPC == TE, "tile split");
  __shared__ __align__(16) T smem[NBUF * TILE];

  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int col = lane & 31, grp = lane >> 5;
  const int n_qt = p.Np / 256;
  const int n_units = p.causal ? (n_qt + 1) / 2 : n_qt;
  const int pr = blockIdx.x % n_units, bi = blockIdx.x / n_units;
  const int i = bi % p.H_q, b = bi / p.H_q;
  const int j = i / p.g;
  const int qt0 = pr, qt1 = n_qt - 1 - pr;
  const int64_t hq = (int64_t)b * p.H_q + i, hk = (int64_t)b * p.H_kv + j;

  // Items: the key tiles of query tile qt0 (phase 0), then, causal and
  // qt1 != qt0, those of query tile qt1 (phase 1) in reverse.
  auto kv_tiles = [&](int qt) { return ((p.causal ? min(p.N, qt * 256 + 256) : p.N) + BT - 1) / BT; };
  const int n0 = kv_tiles(qt0);
  const int nt1 = p.causal && qt1 != qt0 ? kv_tiles(qt1) : 0;
  const int n_items = n0 + nt1;
  auto item_tile = [&](int t) { return t < n0 ? t : nt1 - 1 - (t - n0); };
  const T* Kh = (const T*)p.k + hk * p.Np * D;
  const T* Vh = (const T*)p.v + hk * p.Np * D;
  const T* KTh = (const T*)p.kt + hk * D * p.Np;

  // Loads of item t (a key tile) into ring slot t % NBUF (see bwd_dkdv's
  // issue): per-lane byte offsets computed once, wave-uniform bases per item.
  uint32_t loff[IPW];
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int ins = wave * IPW + x, arr = ins / INS, pos = ins % INS * 64 + lane;
    if (arr < 2) {   // K, V rows
      const int r = pos / RC, c = pos % RC;
      loff[x] = (uint32_t)((r * D + (c ^ swz<RC>(r)) * EPC) * (int)sizeof(T));
    } else {         // K^T lines (keys in swap23 order)
      const int r = pos / LC, c = pos % LC;
      loff[x] = (uint32_t)r * (uint32_t)p.Np * (uint32_t)sizeof(T) + (uint32_t)((c ^ swz<LC>(r)) * EPC * (int)sizeof(T));
    }
  }
  // Buffer loads (counted only in vmcnt, as in bwd_dkdv), byte offsets below 2^32.
  auto issue = [&](int t) {
    if (t >= n_items) return;
    const int k0 = item_tile(t) * BT;
    T* tb = smem + (t % NBUF) * TILE;
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int ins = wave * IPW + x, arr = ins / INS, li = ins % INS;
      const T* base = arr == 0 ? Kh + (int64_t)k0 * D : arr == 1 ? Vh + (int64_t)k0 * D : KTh + k0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)base, (short)0,
          (int)(arr < 2 ? TE * (uint32_t)sizeof(T) : (uint32_t)(D - 1) * (uint32_t)p.Np * (uint32_t)sizeof(T) + BT * (uint32_t)sizeof(T)),
          0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(tb + arr * TE + li * 64 * EPC), 16, (int)loff[x], 0, 0, 0);
    }
  };

  // This wave's Q and dO fragments (B operands of S^T = K Q^T and
  // dP^T = V dO^T) and its rows' statistics for the query tile at q0, and the
  // store of its dQ.
  Frag qf[QB][NS], of[QB][NS];
  float lse[QB], dvq[QB];
  f32x16 dq[QB][D / 32];
  auto load_q = [&](int qw) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int t = qw + 32 * qb + col;
      const T* qr = (const T*)p.q + (hq * p.Np + t) * D;
      const T* orow = (const T*)p.dO + (hq * p.Np + t) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qf[qb][s] = *reinterpret_cast<const Frag*>(qr + s * MF::KS + grp * MF::E);
        of[qb][s] = *reinterpret_cast<const Frag*>(orow + s * MF::KS + grp * MF::E);
      }
      lse[qb] = t < p.N ? p.lse[hq * p.Np + t] : INFINITY;
      dvq[qb] = t < p.N ? -p.dvec[hq * p.Np + t] : 0.f;   // D (stored negated)
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) dq[qb][nb] = f32x16{};
    }
  };
  // dQ^T: lane = query, register r = head dim 32*nb + 8*(r/4) + 4*grp + r%4.
  auto store_dq = [&](int qw) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int t = qw + 32 * qb + col;
      T* dqr = (T*)p.dqkv + ((int64_t)b * p.Np + t) * p.W + (int64_t)i * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int c = nb * 32 + 8 * rq + 4 * grp;
          const f32x16& a = dq[qb][nb];
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(dqr + c) =
                bf16x4{(bf16)(a[4 * rq] * p.scale), (bf16)(a[4 * rq + 1] * p.scale),
                       (bf16)(a[4 * rq + 2] * p.scale), (bf16)(a[4 * rq + 3] * p.scale)};
          } else {
            *reinterpret_cast<f32x4*>(dqr + c) =
                f32x4{a[4 * rq] * p.scale, a[4 * rq + 1] * p.scale, a[4 * rq + 2] * p.scale,
                      a[4 * rq + 3] * p.scale};
          }
        }
    }
  };

  // Prologue: items 0..NBUF-2 in flight, then the first query tile's
  // fragments, all landed before the loop, which then waits only on its own
  // loads.
  int qw = qt0 * 256 + 64 * wave;   // this wave's first query
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) issue(t);
  load_q(qw);
  wait_vmcnt<0>();
  __syncthreads();

  // Items [t0, t1). Key tiles left of the diagonal and before the sequence
  // end need no mask for any wave; the loop over them is compiled without the
  // mask code (a fifth of the VALU work per block), and the few others run in
  // a copy that keeps it. Separate loops, rather than a branch per block, keep
  // each one's registers within 256.
  auto run_items = [&](int t0, int t1, auto mask_on) {
    constexpr bool MASK = decltype(mask_on)::value;
    for (int t = t0; t < t1; ++t) {
      if (t > 0) {
        // item t visible (items t+1.. may still be in flight), and every wave
        // is done with slot (t-1) % NBUF, which takes item t+NBUF-1
        wait_vmcnt_tiles<VM_PER_TILE, NBUF - 2>(min(NBUF - 2, max(0, n_items - 1 - t)));
        ring_barrier();
      }
      issue(t + NBUF - 1);
      const T* Ks = smem + (t % NBUF) * TILE;
      const T* Vs = Ks + TE;
      const T* KTs = Ks + 2 * TE;
      const int k0 = item_tile(t) * BT;
#pragma unroll
      for (int jb = 0; jb < BT / 32; ++jb) {
        const int kb = k0 + 32 * jb;
        if (MASK && (kb >= p.N || (p.causal && kb > qw + 63))) continue;   // wave-uniform
        // LDS reads ahead of their use: K and V fragments before the S^T/dP^T
        // MFMAs, K^T fragments before the softmax work.
        Frag ka[NS], va[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          ka[st] = row_frag<T, D>(Ks, 32 * jb + col, st, grp);
          va[st] = row_frag<T, D>(Vs, 32 * jb + col, st, grp);
        }
        f32x16 s[QB], dp[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) { s[qb] = f32x16{}; dp[qb] = f32x16{}; }
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            s[qb] = MF::run(ka[st], qf[qb][st], s[qb]);
            dp[qb] = MF::run(va[st], of[qb][st], dp[qb]);
          }
        // register r: key kb + 8*(r/4) + 4*grp + r%4; column: query qw + 32*qb + col.
        // Register r holds key kb + 4*grp + o_r with o_r = 8*(r/4) + r%4. The
        // key is visible iff o_r < lim: lim = N - kb - 4*grp, and for causal
        // also <= q - kb - 4*grp.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int base = kb + 4 * grp;
          const int lim = p.causal ? min(p.N - base, qw + 32 * qb + col - base + 1) : p.N - base;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[qb][r], p.c, -lse[qb]));
            const float ds = pv * (dp[qb][r] - dvq[qb]);   // dS^T
            s[qb][r] = !MASK || 8 * (r / 4) + r % 4 < lim ? ds : 0.f;
          }
        }
#pragma unroll
        for (int h = 0; h < kHalves<T>; ++h)
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              dq[qb][nb] = MF::run(line_frag<T>(KTs, nb * 32 + col, 32 * jb, h, grp), frag_regs<T>(s[qb], h), dq[qb][nb]);
      }
    }
  };
  // Key tiles [0, clear) are fully visible to every query of query tile qt:
  // all of their keys precede the tile's first query (or any key is visible,
  // without a mask) and lie before N.
  auto clear_tiles = [&](int qt) { return min(p.causal ? qt * 256 / BT : p.N / BT, p.N / BT); };
  // Phase 0 walks key tiles upward: the clear ones first.
  const int d0 = min(clear_tiles(qt0), n0);
  run_items(0, d0, std::false_type{});
  run_items(d0, n0, std::true_type{});
  if (n_items > n0) {   // second query tile: store the first one's dQ
    store_dq(qw);
    qw = qt1 * 256 + 64 * wave;
    load_q(qw);
    wait_vmcnt<0>();
    // Phase 1 walks key tiles downward: the clear ones last.
    const int m1 = n0 + max(0, nt1 - clear_tiles(qt1));
    run_items(n0, m1, std::true_type{});
    run_items(m1, n_items, std::false_type{});
  }
  store_dq(qw);
}

// dQ for bf16 at d_head = 64, as a software pipeline: workgroup = (query
// tiles of 256 queries, head i, batch b) as in bwd_dq, but 8 waves of 32
// queries (two waves per SIMD at up to 256 VGPRs). The key-side tiles (K, V
// and K^T) of each 64-key tile come through a ring of NBUF LDS slots, laid
// out by operand as in bwd_dkdv so that a fragment read whose slot is known at
// compile time is a lane register plus an immediate. The rows' statistics sit
// in two accumulator tiles (every register of a lane holds its query's -lse/c,
// or its -D), the start of every S^T and dP^T chain, so that P = exp2(c S) and
// dS = P (dP - D) are one product each. The work items are the key tiles, in
// bwd_dq's order; those that need a mask run one 32-key block at a time, the
// others through a pipeline like bwd_dkdv's run_clear: iteration t (a key
// tile, two 32-key blocks) runs two phases of 2*NS + 2*D/32 MFMAs each,
//   phase 0: S^T and dP^T of block 1 of tile t, then dQ of block 1 of tile
//            t-1; softmax gradient of block 0 of tile t
//   phase 1: S^T and dP^T of block 0 of tile t+1, then dQ of block 0 of tile
//            t; softmax gradient of block 1 of tile t
// and each MFMA forms a group with a share of the phase's VALU work and the
// LDS read of the fragment FA groups ahead.
template <int D>
__global__ __launch_bounds__(512, 2) void bwd_dq_pipe(BwdParams p) {
  using T = bf16;
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  constexpr int WAVES = 8;
  constexpr int EPC = 8;
  constexpr int RC = D / EPC, LC = BT / EPC;   // chunks per row [64][D], per line [D][64]
  constexpr int NS = D / MF::KS;               // k-steps over the head dims
  constexpr int NB = D / 32;                   // 32-dim blocks of dQ
  constexpr int TE = BT * D;                   // elements of one operand tile
  constexpr int NBUF = 6;                      // ring slots: tiles t-1, t, t+1 and three in flight
  constexpr int INS = TE * 2 / 1024;           // 1 KB loads per operand tile
  constexpr int IPW = 3 * INS / WAVES;         // per wave and tile
  static_assert(IPW * WAVES == 3 * INS && INS * 64 * EPC == TE, "tile split");
  __shared__ __align__(16) T smem[3 * NBUF * TE];   // K rows, V rows, K^T lines; NBUF slots each

  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int col = lane & 31, grp = lane >> 5;
  const int n_qt = p.Np / 256;
  const int n_units = p.causal ? (n_qt + 1) / 2 : n_qt;
  const int pr = blockIdx.x % n_units, bi = blockIdx.x / n_units;
  const int i = bi % p.H_q, b = bi / p.H_q;
  const int j = i / p.g;
  const int qt0 = pr, qt1 = n_qt - 1 - pr;
  const int64_t hq = (int64_t)b * p.H_q + i, hk = (int64_t)b * p.H_kv + j;

  // Items: the key tiles of query tile qt0 (phase 0), then, causal and
  // qt1 != qt0, those of query tile qt1 (phase 1) in reverse.
  auto kv_tiles = [&](int qt) { return ((p.causal ? min(p.N, qt * 256 + 256) : p.N) + BT - 1) / BT; };
  const int n0 = kv_tiles(qt0);
  const int nt1 = p.causal && qt1 != qt0 ? kv_tiles(qt1) : 0;
  const int n_items = n0 + nt1;
  auto item_tile = [&](int t) { return t < n0 ? t : nt1 - 1 - (t - n0); };
  const T* Kh = (const T*)p.k + hk * p.Np * D;
  const T* Vh = (const T*)p.v + hk * p.Np * D;
  const T* KTh = (const T*)p.kt + hk * D * p.Np;

  // operand tile a (0: K, 1: V, 2: K^T) of ring slot s
  const T* v_tiles = opaque_lds<T>(smem + NBUF * TE);
  const T* line_tiles = opaque_lds<T>(smem + 2 * NBUF * TE);
  auto tile = [&](int a, int s) __attribute__((always_inline)) {
    return (a == 0 ? (const T*)smem : a == 1 ? v_tiles : line_tiles) + s * TE;
  };

  // Loads of item t into ring slot t % NBUF: load `ins` (of 3*INS) covers 64
  // 16-byte chunks of operand tile ins / INS; lane L's chunk lands at position
  // 64*(ins % INS) + L, which holds chunk (c ^ swz(row)) of its row. The
  // per-lane byte offsets are the same for every item and computed once.
  uint32_t loff[IPW];
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int ins = wave * IPW + x, arr = ins / INS, pos = ins % INS * 64 + lane;
    if (arr < 2) {   // K, V rows
      const int r = pos / RC, c = pos % RC;
      loff[x] = (uint32_t)((r * D + (c ^ swz<RC>(r)) * EPC) * 2);
    } else {         // K^T lines (keys in swap23 order)
      const int r = pos / LC, c = pos % LC;
      loff[x] = (uint32_t)r * (uint32_t)p.Np * 2u + (uint32_t)((c ^ swz<LC>(r)) * EPC * 2);
    }
  }
  int next_issue = 0;
  auto issue_next = [&]() {
    const int t = next_issue++;
    if (t >= n_items) return;
    const int k0 = item_tile(t) * BT;
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int ins = wave * IPW + x, arr = ins / INS, li = ins % INS;
      const T* base = arr == 0 ? Kh + (int64_t)k0 * D : arr == 1 ? Vh + (int64_t)k0 * D : KTh + k0;
      // byte offsets below 2^32: the host checks D * Np * sizeof(T)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)base, (short)0,
          (int)(arr < 2 ? TE * 2u : (uint32_t)(D - 1) * (uint32_t)p.Np * 2u + BT * 2u), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(smem + (arr * NBUF + t % NBUF) * TE + li * 64 * EPC),
                                               16, (int)loff[x], 0, 0, 0);
    }
  };
  // Ring bookkeeping as in bwd_dkdv: sync(R, F) waits for this wave's loads
  // of the tiles up to R, passes a barrier (every wave's loads of those tiles
  // are visible, every wave is done with the tiles before F) and issues the
  // tiles whose slots that frees, up to F + NBUF - 1.
  auto sync = [&](int R, int F) {
    wait_vmcnt_tiles<IPW, NBUF - 2>(min(NBUF - 2, max(0, next_issue - 1 - R)));
    ring_barrier();
    const int last = min(F + NBUF - 1, n_items - 1);
    while (next_issue <= last) issue_next();
  };

  // This wave's Q and dO fragments (B operands of S^T = K Q^T and
  // dP^T = V dO^T), the accumulator tiles of its rows' statistics, and its dQ.
  Frag qf[NS], of[NS];
  f32x16 s_init, d_init, dq[NB];
  auto load_q = [&](int qw) {
    const int t = qw + col;
    const T* qr = (const T*)p.q + (hq * p.Np + t) * D;
    const T* orow = (const T*)p.dO + (hq * p.Np + t) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = *reinterpret_cast<const Frag*>(qr + s * MF::KS + grp * MF::E);
      of[s] = *reinterpret_cast<const Frag*>(orow + s * MF::KS + grp * MF::E);
    }
    // -lse/c and -D of every row of the tiles walked: -inf and 0 past N
    const float nl = p.nlse[hq * p.Np + t], nd = p.dvec[hq * p.Np + t];
#pragma unroll
    for (int r = 0; r < 16; ++r) { s_init[r] = nl; d_init[r] = nd; }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) dq[nb] = f32x16{};
  };
  // dQ^T: lane = query, register r = head dim 32*nb + 8*(r/4) + 4*grp + r%4.
  auto store_dq = [&](int qw) {
    const int t = qw + col;
    T* dqr = (T*)p.dqkv + ((int64_t)b * p.Np + t) * p.W + (int64_t)i * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = nb * 32 + 8 * rq + 4 * grp;
        const f32x16& a = dq[nb];
        *reinterpret_cast<bf16x4*>(dqr + c) =
            bf16x4{(bf16)(a[4 * rq] * p.scale), (bf16)(a[4 * rq + 1] * p.scale),
                   (bf16)(a[4 * rq + 2] * p.scale), (bf16)(a[4 * rq + 3] * p.scale)};
      }
  };

  // Prologue: items 0..NBUF-2 in flight, then the first query tile's
  // fragments; the K^T tile of the last slot starts as zeros (a pipelined run
  // from item 0 reads it as its absent previous item's and multiplies it by
  // zeros, which must not meet an Inf or NaN).
  int qw = qt0 * 256 + 32 * wave;   // this wave's first query
  while (next_issue < min(NBUF - 1, n_items)) issue_next();
  load_q(qw);
  for (int x = tid; x < TE * 2 / 16; x += WAVES * 64)
    reinterpret_cast<f32x4*>(smem + (2 * NBUF + NBUF - 1) * TE)[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_vmcnt<0>();
  __syncthreads();

  // Items [t0, t1) that need a mask, one 32-key block at a time.
  auto run_masked = [&](int t0, int t1) {
    for (int t = t0; t < t1; ++t) {
      sync(t, t);   // item t visible; every wave done with the items before it
      const int sw = t % NBUF;
      const int k0 = item_tile(t) * BT;
#pragma unroll
      for (int jb = 0; jb < BT / 32; ++jb) {
        const int kb = k0 + 32 * jb;
        if (kb >= p.N || (p.causal && kb > qw + 31)) continue;   // wave-uniform
        f32x16 s = s_init, dp = d_init;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = MF::run(row_frag<T, D>(tile(0, sw), 32 * jb + col, st, grp), qf[st], s);
          dp = MF::run(row_frag<T, D>(tile(1, sw), 32 * jb + col, st, grp), of[st], dp);
        }
        // register r: key kb + 4*grp + o_r, o_r = 8*(r/4) + r%4; visible iff
        // o_r < lim (lim = N - kb - 4*grp, and for causal also <= q - kb - 4*grp)
        const int base = kb + 4 * grp;
        const int lim = p.causal ? min(p.N - base, qw + col - base + 1) : p.N - base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(s[r] * p.c);
          s[r] = 8 * (r / 4) + r % 4 < lim ? pv * dp[r] : 0.f;   // dS^T
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            dq[nb] = MF::run(line_frag<T>(tile(2, sw), nb * 32 + col, 32 * jb, h, grp), frag_regs<T>(s, h), dq[nb]);
      }
    }
  };

  // Items [t0, t1) without a mask, pipelined.
  auto run_clear = [&](int t0, int t1) {
    if (t0 >= t1) return;
    constexpr int NGG = 2 * NB;      // dQ MFMAs of a block
    constexpr int NGS = 2 * NS;      // S^T/dP^T MFMAs of a block
    constexpr int NGP = NGG + NGS;   // MFMAs (groups) of a phase
    constexpr int FA = 3;            // fragment reads ahead
    static_assert(FA <= NGS, "groups");
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x16 sA, dA, sB, dB;           // S^T and dP^T - D of block 0 (A) and block 1 (B)
    u32x4 pA[2], pB[2];              // dS^T as bf16 pairs, per k-step: B operands of dQ
    Frag fr[2 * NGP];                // the fragment of each MFMA of an iteration
    // The fragment of MFMA u of the iteration over the ring slots of items
    // t-1 (prev), t (cur) and t+1 (next). A phase's score MFMAs come first,
    // its dQ MFMAs last: the softmax work of the next phase then reads scores
    // whose MFMAs ended NGG groups before.
    auto fetch = [&](auto uc, int prev, int cur, int next) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value, ph = u / NGP, k = u % NGP;
      if constexpr (k < NGS) {
        constexpr int st = k / 2, which = k % 2;   // 0: S^T (K), 1: dP^T (V)
        fr[u] = row_frag<T, D>(tile(which, ph == 0 ? cur : next), (ph == 0 ? 32 : 0) + col, st, grp);
      } else {
        constexpr int h = (k - NGS) / NB, nb = (k - NGS) % NB;
        fr[u] = line_frag<T>(tile(2, ph == 0 ? prev : cur), nb * 32 + col, ph == 0 ? 32 : 0, h, grp);
      }
    };
    // dQ MFMA k (< NGG) of a block with packed dS^T pk
    auto grad_mfma = [&](auto kc, const Frag& a, const u32x4 (&pk)[2]) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, h = k / NB, nb = k % NB;
      dq[nb] = MF::run(a, __builtin_bit_cast(Frag, pk[h]), dq[nb]);
    };
    // the scores [lo(k), lo(k+1)) of a phase go with its group k
    auto lo = [](int k) constexpr { return 16 * k / NGP; };
    float ex[16];
    auto group = [&](auto uc, int prev, int cur, int next) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value, ph = u / NGP, k = u % NGP;
      f32x16& s_sc = ph == 0 ? sB : sA;   // scored in this phase
      f32x16& d_sc = ph == 0 ? dB : dA;
      const f32x16& s_sm = ph == 0 ? sA : sB;   // softmax gradient in this phase
      const f32x16& d_sm = ph == 0 ? dA : dB;
      u32x4 (&p_sm)[2] = ph == 0 ? pA : pB;
      // the fragment FA groups ahead; past the iteration's end, the first
      // groups of the next one (scores of block 1 of item t+1: tile next)
      if constexpr (u + FA < 2 * NGP) fetch(std::integral_constant<int, u + FA>{}, prev, cur, next);
      else fetch(std::integral_constant<int, u + FA - 2 * NGP>{}, cur, next, next);
      if constexpr (k < NGS) {
        constexpr int st = k / 2, which = k % 2;
        if constexpr (which == 0) s_sc = MF::run(fr[u], qf[st], st == 0 ? s_init : s_sc);
        else d_sc = MF::run(fr[u], of[st], st == 0 ? d_init : d_sc);
      } else {
        grad_mfma(std::integral_constant<int, k - NGS>{}, fr[u], ph == 0 ? pB : pA);
      }
      // softmax gradient of this group's scores; exponentials one group ahead
      constexpr int r0 = lo(k), r1 = lo(k + 1), r2 = k + 1 < NGP ? lo(k + 2) : 16;
      if constexpr (k == 0) {
#pragma unroll
        for (int r = r0; r < r1; ++r) ex[r] = __builtin_amdgcn_exp2f(s_sm[r] * p.c);
      }
#pragma unroll
      for (int r = r1; r < r2; ++r) ex[r] = __builtin_amdgcn_exp2f(s_sm[r] * p.c);
#pragma unroll
      for (int r = r0; r < r1; ++r) {
        ex[r] = ex[r] * d_sm[r];   // dS^T = P (dP - D)
        if (r % 2 == 1)
          p_sm[r / 8][(r % 8) / 2] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{ex[r - 1], ex[r]}, bf16x2));
      }
      // within the group: the MFMA, the fragment read, then the VALU work, so
      // that the MFMAs of consecutive groups never issue back to back
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: tile t0 visible; scores of its block 0. The dS of block "1 of
    // item t0-1" is zeros, so the first phase's dQ MFMAs add exact zeros:
    // their other operand, the K^T tile in the slot before t0's, holds item
    // t0-1 (finite) or, before item 0, zeros. Then the first FA fragments of
    // the first iteration (scores of block 1 of tile t0).
    sync(t0, t0);
    {
      const int s0 = t0 % NBUF;
      sA = s_init; dA = d_init;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        sA = MF::run(row_frag<T, D>(tile(0, s0), col, st, grp), qf[st], sA);
        dA = MF::run(row_frag<T, D>(tile(1, s0), col, st, grp), of[st], dA);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) pB[h] = u32x4{0u, 0u, 0u, 0u};
      static_for<0, FA>([&](auto uc) { fetch(uc, (s0 + NBUF - 1) % NBUF, s0, s0); });
    }
    // Iteration t reads the slots of items t-1 (prev), t (cur) and t+1
    // (next; past the loop's end, item t+1's scores are computed and
    // dropped, and its first fragments read and dropped). There is one copy
    // of it per slot of t.
    for (int t = t0; t < t1; ++t) {
      sync(t + 1, t - 1);   // items t and t+1 visible; every wave done with the items before t-1
      const int m = t % NBUF;
      static_for<0, NBUF>([&](auto mc) {
        constexpr int c = decltype(mc)::value;
        if (m == c) static_for<0, 2 * NGP>([&](auto uc) { group(uc, (c + NBUF - 1) % NBUF, c, (c + 1) % NBUF); });
      });
    }
    // Epilogue: dQ of block 1 of the last item.
    const int lt = (t1 - 1) % NBUF;
    static_for<0, NGG>([&](auto kc) { fetch(std::integral_constant<int, NGS + decltype(kc)::value>{}, lt, lt, lt); });
    static_for<0, NGG>([&](auto kc) { grad_mfma(kc, fr[NGS + decltype(kc)::value], pB); });
  };

  // Key tiles [0, clear) are fully visible to every query of query tile qt.
  auto clear_tiles = [&](int qt) { return min(p.causal ? qt * 256 / BT : p.N / BT, p.N / BT); };
  // Phase 0 walks key tiles upward: the clear ones first.
  const int d0 = min(clear_tiles(qt0), n0);
  run_clear(0, d0);
  run_masked(d0, n0);
  if (n_items > n0) {   // second query tile: store the first one's dQ
    store_dq(qw);
    qw = qt1 * 256 + 32 * wave;
    load_q(qw);
    wait_vmcnt<0>();
    // Phase 1 walks key tiles downward: the clear ones last.
    const int m1 = n0 + max(0, nt1 - clear_tiles(qt1));
    run_masked(n0, m1);
    run_clear(m1, n_items);
  }
  store_dq(qw);
}

template <typename T, bool PERM = false>
hipError_t transpose(const void* src, int64_t src_bs, int64_t src_ld, int64_t r_valid,
                     int64_t r_total, void* dst, int64_t dst_bs, int64_t dst_ld, int64_t C,
                     int64_t nbatch, hipStream_t stream) {
  const int64_t tiles = (r_total + 63) / 64 * ((C + 63) / 64) * nbatch;
  if (tiles > 0x7FFFFFFF || r_total > 0x7FFFFFFF || C > 0x7FFFFFFF)
    return hipErrorInvalidConfiguration;
  if (PERM && r_total % 64) return hipErrorInvalidValue;   // the permutation stays within 64-row tiles
  const dim3 grid((unsigned)tiles);
  transpose_kernel<T, PERM><<<grid, 256, 0, stream>>>((const T*)src, src_bs, src_ld, (int)r_valid,
                                                      (int)r_total, (T*)dst, dst_bs, dst_ld, (int)C);
  return hipGetLastError();
}

}  // namespace

SavedLayout saved_layout(int64_t es, int64_t B, int64_t N, int64_t Np, int64_t H_q, int64_t H_kv,
                         int64_t d) {
  auto r = [](int64_t x) { return (x + 255) / 256 * 256; };
  SavedLayout S;
  S.q = 0;
  S.k = S.q + r(es * B * H_q * Np * d);
  S.vt = S.k + r(es * B * H_kv * Np * d);
  S.a = S.vt + r(es * B * H_kv * Np * d);
  S.lse = S.a + r(es * B * N * H_q * d);
  S.o32 = S.lse + r(4 * B * H_q * Np);
  S.total = S.o32 + r(4 * B * N * H_q * d);
  return S;
}

namespace {

// Byte offsets of the backward workspace regions.
struct BwdLayout {
  int64_t q, k, vt, a, lse, o32, wt, dO, dvec, qt, kt, v, dOt, dqkv, dqkvT, xT, wall, aT, dyT, part;
  int64_t total;
};

inline int64_t r256(int64_t x) { return (x + 255) / 256 * 256; }

// With `saved`, the forward activations (q, k, vt, a, lse) come from a
// training forward in the caller's buffer, and those regions (and the weight
// transpose that recomputing them needs) take no workspace.
BwdLayout bwd_layout(int64_t es, int64_t B, int64_t N, int64_t Np, int64_t d_model, int64_t H_q,
                     int64_t H_kv, int64_t d, bool saved, bool causal) {
  const int64_t W = (H_q + 2 * H_kv) * d, T = B * Np;
  const SplitK s1 = splitk_plan(d_model, T, W), s2 = splitk_plan(H_q * d, T, d_model);
  // The region also holds the key-split parts of a recomputed non-causal
  // attention (bf16) before the weight gradients use it.
  const int64_t att = !saved && !causal && es == 2 ? (int64_t)attention_split_bound(d) : 0;
  const int64_t part = std::max(std::max(s1.n_split * d_model * W, s2.n_split * H_q * d * d_model) * 4, att);
  const int64_t f = saved ? 0 : 1;
  const int64_t sizes[] = {
      f * es * B * H_q * Np * d, f * es * B * H_kv * Np * d, f * es * B * H_kv * Np * d,
      f * es * B * N * H_q * d, f * 4 * B * H_q * Np, f * 4 * B * N * H_q * d,
      f * (int64_t)qkv_wt_bytes(es == 2 ? SQA_DTYPE_BF16 : SQA_DTYPE_FP32, d_model, H_q, H_kv, d),
      es * B * H_q * Np * d, 2 * 4 * B * H_q * Np, es * B * H_q * Np * d, es * B * H_kv * Np * d,
      es * B * H_kv * Np * d, es * B * H_q * Np * d, es * T * W, es * T * W, es * d_model * T,
      es * d_model * W, es * H_q * d * T, es * d_model * T, part};
  BwdLayout L;
  int64_t* out[] = {&L.q, &L.k, &L.vt, &L.a, &L.lse, &L.o32, &L.wt, &L.dO, &L.dvec, &L.qt, &L.kt,
                    &L.v, &L.dOt, &L.dqkv, &L.dqkvT, &L.xT, &L.wall, &L.aT, &L.dyT, &L.part};
  static_assert(sizeof(out) / sizeof(out[0]) == sizeof(sizes) / sizeof(sizes[0]), "regions");
  int64_t off = 0;
  for (int x = 0; x < (int)(sizeof(sizes) / sizeof(sizes[0])); ++x) {
    *out[x] = off;
    off += r256(sizes[x]);
  }
  L.total = off;
  return L;
}

template <typename T, int D>
hipError_t backward_impl(const void* x, const void* wq, const void* wk, const void* wv,
                         const void* wo, const void* dy, const char* saved, void* dx, void* dwq,
                         void* dwk, void* dwv, void* dwo, int64_t B, int64_t N, int64_t Np,
                         int64_t d_model, int64_t H_q, int64_t H_kv, bool causal, char* ws,
                         hipStream_t stream) {
  const sqa_dtype dt = sizeof(T) == 2 ? SQA_DTYPE_BF16 : SQA_DTYPE_FP32;
  const BwdLayout L = bwd_layout(sizeof(T), B, N, Np, d_model, H_q, H_kv, D, saved != nullptr, causal);
  const int64_t wq_w = H_q * D, wkv_w = H_kv * D, W = wq_w + 2 * wkv_w, TT = B * Np;
  void *q = ws + L.q, *k = ws + L.k, *vt = ws + L.vt, *a = ws + L.a, *wt = ws + L.wt;
  float* lse = (float*)(ws + L.lse);
  float* o32 = (float*)(ws + L.o32);
  if (saved) {
    const SavedLayout S = saved_layout(sizeof(T), B, N, Np, H_q, H_kv, D);
    char* sv = const_cast<char*>(saved);   // read only below
    q = sv + S.q; k = sv + S.k; vt = sv + S.vt; a = sv + S.a;
    lse = (float*)(sv + S.lse);
    o32 = (float*)(sv + S.o32);
  }
  float* dvec = (float*)(ws + L.dvec);   // -D, then -lse/c
  float* nlse = dvec + B * H_q * Np;
  void *dO = ws + L.dO, *qt = ws + L.qt, *kt = ws + L.kt, *v = ws + L.v, *dOt = ws + L.dOt;
  void *dqkv = ws + L.dqkv, *dqkvT = ws + L.dqkvT, *xT = ws + L.xT, *wall = ws + L.wall;
  void *aT = ws + L.aT, *dyT = ws + L.dyT;
  float* part = (float*)(ws + L.part);
  hipError_t e;
#define SQA_CK(call) do { e = (call); if (e != hipSuccess) return e; } while (0)
  // forward activations and each row's log-sum-exp, unless a training forward kept them
  if (!saved) {
    SQA_CK(launch_qkv_projection(dt, x, wq, wk, wv, wt, q, k, vt, B, N, Np, d_model, H_q, H_kv, D,
                                 nullptr, stream));
    SQA_CK(launch_attention(dt, q, k, vt, a, B, N, Np, H_q, H_kv, D, causal, nullptr, stream, lse,
                            nullptr, o32, (float*)(ws + L.part)));
  }
  // dO = dY Wo^T in the head layout of q (Wo [H_q*d, d_model] is W^T of that product)
  SQA_CK(launch_gemm_heads(dt, dy, wo, dO, B, N, Np, d_model, wq_w, D, stream));
  {
    const int64_t rows = B * H_q * Np;
    dvec_kernel<T, D><<<(unsigned)((rows + 31) / 32), 256, 0, stream>>>(
        (const T*)dO, o32, lse, (float)(1.4426950408889634 / sqrt((double)D)), dvec, nlse, (int)N, Np,
        (int)H_q, rows);
    SQA_CK(hipGetLastError());
  }
  // head-dim-major copies for the contractions over tokens (tokens in swap23
  // order, the k-order of operands packed from accumulators), V row-major
  SQA_CK((transpose<T, true>(q, Np * D, D, Np, Np, qt, D * Np, Np, D, B * H_q, stream)));
  SQA_CK((transpose<T, true>(k, Np * D, D, Np, Np, kt, D * Np, Np, D, B * H_kv, stream)));
  SQA_CK(transpose<T>(vt, D * Np, Np, D, D, v, Np * D, D, Np, B * H_kv, stream));
  SQA_CK((transpose<T, true>(dO, Np * D, D, Np, Np, dOt, D * Np, Np, D, B * H_q, stream)));
  BwdParams p;
  p.q = q; p.qt = qt; p.k = k; p.kt = kt; p.v = v; p.dO = dO; p.dOt = dOt;
  p.lse = lse; p.nlse = nlse; p.dvec = dvec; p.dqkv = dqkv;
  p.N = (int)N; p.Np = (int)Np; p.H_q = (int)H_q; p.H_kv = (int)H_kv; p.g = (int)(H_q / H_kv);
  p.causal = causal ? 1 : 0; p.W = (int)W;
  p.c = (float)(1.4426950408889634 / sqrt((double)D));
  p.scale = (float)(1.0 / sqrt((double)D));
  // grids, and the 32-bit byte offsets of bwd_dq's loads within a K^T head
  if ((Np / 256) * B * H_kv > 0x7FFFFFFF || (Np / 256) * B * H_q > 0x7FFFFFFF ||
      (int64_t)D * Np * (int64_t)sizeof(T) > 0xFFFFFFFFll)
    return hipErrorInvalidConfiguration;
  // causal: workgroups take pairs of 256-key tiles (kt, n_kt-1-kt)
  const int64_t n_kt = Np / 256;
  bwd_dkdv<T, D><<<(unsigned)((causal ? (n_kt + 1) / 2 : n_kt) * B * H_kv), 512, 0, stream>>>(p);
  SQA_CK(hipGetLastError());
  // causal: workgroups take pairs of 256-query tiles (qt, n_qt-1-qt)
  const int64_t n_qt = Np / 256;
  const unsigned dq_grid = (unsigned)((causal ? (n_qt + 1) / 2 : n_qt) * B * H_q);
  if constexpr (std::is_same_v<T, bf16> && D == 64) bwd_dq_pipe<D><<<dq_grid, 512, 0, stream>>>(p);
  else bwd_dq<T, D><<<dq_grid, 256, 0, stream>>>(p);
  SQA_CK(hipGetLastError());
  // dX = [dQ | dK | dV] [Wq | Wk | Wv]^T
  concat_weights<T><<<(unsigned)((d_model * W + 255) / 256), 256, 0, stream>>>(
      (const T*)wq, (const T*)wk, (const T*)wv, (T*)wall, d_model, (int)wq_w, (int)wkv_w);
  SQA_CK(hipGetLastError());
  SQA_CK(launch_gemm_unpad(dt, dqkv, wall, dx, B, N, Np, W, d_model, stream));
  // [dWq | dWk | dWv] = X^T [dQ | dK | dV] over all tokens (padding tokens are zero in X^T)
  SQA_CK(transpose<T>(x, N * d_model, d_model, N, Np, xT, Np, TT, d_model, B, stream));
  SQA_CK(transpose<T>(dqkv, 0, W, TT, TT, dqkvT, 0, TT, W, 1, stream));
  {
    const SplitK sk = splitk_plan(d_model, TT, W);
    SQA_CK(launch_gemm_splitk(dt, xT, dqkvT, part, d_model, TT, W, sk, stream));
    reduce_splits<T><<<(unsigned)((d_model * W + 255) / 256), 256, 0, stream>>>(
        part, (int)sk.n_split, d_model, (int)W, (T*)dwq, (int)wq_w, (T*)dwk, (int)wkv_w, (T*)dwv,
        (int)wkv_w);
    SQA_CK(hipGetLastError());
  }
  // dWo = A^T dY
  SQA_CK(transpose<T>(a, N * wq_w, wq_w, N, Np, aT, Np, TT, wq_w, B, stream));
  SQA_CK(transpose<T>(dy, N * d_model, d_model, N, Np, dyT, Np, TT, d_model, B, stream));
  {
    const SplitK sk = splitk_plan(wq_w, TT, d_model);
    SQA_CK(launch_gemm_splitk(dt, aT, dyT, part, wq_w, TT, d_model, sk, stream));
    reduce_splits<T><<<(unsigned)((wq_w * d_model + 255) / 256), 256, 0, stream>>>(
        part, (int)sk.n_split, wq_w, (int)d_model, (T*)dwo, (int)d_model, nullptr, 0, nullptr, 0);
    SQA_CK(hipGetLastError());
  }
#undef SQA_CK
  return hipSuccess;
}

}  // namespace

size_t backward_workspace_bytes(sqa_dtype dt, int64_t B, int64_t N, int64_t Np, int64_t d_model,
                                int64_t H_q, int64_t H_kv, int64_t d_head, bool saved, bool causal) {
  return (size_t)bwd_layout(dt == SQA_DTYPE_BF16 ? 2 : 4, B, N, Np, d_model, H_q, H_kv, d_head,
                            saved, causal).total;
}

hipError_t launch_backward(sqa_dtype dt, const void* x, const void* wq, const void* wk,
                           const void* wv, const void* wo, const void* dy, const void* saved,
                           void* dx, void* dwq,
                           void* dwk, void* dwv, void* dwo, int64_t B, int64_t N, int64_t Np,
                           int64_t d_model, int64_t H_q, int64_t H_kv, int64_t d_head, bool causal,
                           void* ws, hipStream_t stream) {
  char* w = (char*)ws;
  const char* sv = (const char*)saved;
  if (dt == SQA_DTYPE_BF16)
    return d_head == 64 ? backward_impl<bf16, 64>(x, wq, wk, wv, wo, dy, sv, dx, dwq, dwk, dwv, dwo, B, N,
                                                  Np, d_model, H_q, H_kv, causal, w, stream)
                        : backward_impl<bf16, 32>(x, wq, wk, wv, wo, dy, sv, dx, dwq, dwk, dwv, dwo, B, N,
                                                  Np, d_model, H_q, H_kv, causal, w, stream);
  return d_head == 64 ? backward_impl<float, 64>(x, wq, wk, wv, wo, dy, sv, dx, dwq, dwk, dwv, dwo, B, N,
                                                 Np, d_model, H_q, H_kv, causal, w, stream)
                      : backward_impl<float, 32>(x, wq, wk, wv, wo, dy, sv, dx, dwq, dwk, dwv, dwo, B, N,
                                                 Np, d_model, H_q, H_kv, causal, w, stream);
}

}  // namespace sqa
