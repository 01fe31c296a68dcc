// Attention core of the SQA forward pass on gfx950: per query head i,
//   A_i = softmax(Q_i K_j^T / sqrt(d)) V_j,   j = floor(i / (H_q/H_kv)),
// with an optional causal mask (key c visible to query r iff c <= r).
// SQA keeps GQA's key/value sharing and cuts the query heads, so the score
// work scales with H_q ("Sparse Query Attention (SQA)...", arXiv 2510.01817,
// abstract; ReactiveAI/GQA-Ref-Micro model card, description).
//
// Design (one workgroup = 8 waves of 64 lanes, or 4 for some grids):
//  * A workgroup owns one (batch, key/value head) pair, G query heads of that
//    head's group and a tile of queries: 512x1, 256x2, 128x4 or 64x8 queries x
//    heads with 8 waves (half that with 4). Every key/value tile staged in LDS
//    is read by all G heads, so repeated K/V is never materialised.
//  * Each wave owns 64 query rows of one head (two 32-query MFMA blocks). It
//    computes S^T = K Q^T, which puts one query per lane (lanes l and l+32
//    share query l%32). Row max and row sum then need a single cross-lane
//    exchange, and the exponentiated scores are already in the B-operand
//    layout of O^T += V^T P^T. No score tile goes through LDS or HBM.
//    Each K or V^T fragment read from LDS feeds two MFMAs, one per query block.
//  * Keys are stored in LDS with bits 2 and 3 of their in-tile index swapped.
//    This makes each lane's 16 score registers of a 32-key block cover two
//    runs of 8 consecutive keys, so P^T is consumed as-is and V^T fragments
//    are single 16-byte LDS reads.
//  * Online softmax in the exp2 domain with fp32 running max and sum. The
//    VALU, not the MFMA pipe, bounds this kernel at d_head = 64, so per score
//    it spends one FMA, one v_exp, half a v_cvt_pk_bf16 and half a v_dot2
//    (the row sum is taken on the bf16 P that the PV product consumes). No row
//    max is taken on the common path: the exponentials use a reference that
//    may lag the running max, and a block is redone against its exact max only
//    when its sums show that the reference fell too far behind.
//  * Causal: key tiles past a workgroup's last query are never loaded, and a
//    wave computes nothing for 32-key blocks past its own last query (it only
//    keeps passing the workgroup's barriers and issuing its share of the tile
//    loads). The two waves that share a SIMD take complementary query rows, so
//    every SIMD carries the same causal work. Only blocks that cross the
//    diagonal or the sequence end are masked. The heaviest query tiles are
//    dispatched first; a grid that fits one dispatch round instead runs as
//    4-wave workgroups, two per CU, each CU pairing a heavy tile with its
//    complement.
#include <math.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int KT = 64;       // keys per LDS tile (two 32-key blocks)
constexpr int NBUF = 4;      // LDS tile ring: in use, visible next, NBUF-2 in flight

// A block index known only at run time (the other form is
// std::integral_constant<int, j mod 2*NBUF>).
struct DynBlock {};

// f(std::integral_constant<int, i>) for i = I .. N-1, in order.
template <int I, int N, typename F> __device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
constexpr int QB = 2;             // 32-query MFMA column blocks per wave
constexpr int FETCH_AHEAD = 2;    // LDS fragments read ahead of their first MFMA
constexpr int QW = 32 * QB;       // query rows per wave
// Exponentials are taken against a reference m_ref (exp2 domain) set MARGIN
// binades above a row's running max when it is (re)computed, and clamped to
// [0, 1] (the clamp bit of v_exp_f32, free), so no weight can overflow however
// far the reference lags. While the row's max stays within MARGIN - 5 binades
// of where the reference was set, every weight is below 1/32 and a lane's sum
// of 16 weights stays at or below SUM_LIMIT. A larger sum (or NaN) means the
// reference fell too far behind for that block, possibly with clamped
// weights: only then is the block's exact max computed, O and l rescaled and
// the block redone. Weights more than 126 - MARGIN binades below a row's max
// underflow to zero; they are below 2^-62 of the largest weight.
constexpr float MARGIN = 64.0f;
constexpr float SUM_LIMIT = 0.5f;

struct AttnParams {
  const void* q; const void* k; const void* vt; void* a;
  const int32_t* lens;   // null, or each sequence's length (clamped into [0, N])
  float* lse;            // null, or [B, H_q, Np]: base-2 log-sum-exp of each row's scaled scores
  const int32_t* order;  // null, or the logical work item of each workgroup (lpt_order)
  float* o32;            // null, or [B*N, H_q*d]: the output before its rounding to T (fp32)
  int N, Np, H_q, H_kv, g, G, n_sub, q_per_wg, n_qt, causal;
  int chunk, remap_end;   // XCD-aware workgroup order (see the kernel's block decode)
  // Key-split tail (non-causal): work items from split_begin on run as n_split
  // workgroups each, part k taking keys [k*split_keys, (k+1)*split_keys), and
  // leave their unnormalised state (O rows in part, m_ref and l in part_ml)
  // for split_merge. split_begin is INT_MAX when nothing is split.
  int split_begin, n_split, split_keys;
  float* part; float* part_ml;
  // Paired order (causal, 4-wave workgroups, one dispatch round): blocks b and
  // b + pair_stride of each group of 2*pair_stride take a heavy query tile and
  // its complement in the same stream; 0 when off.
  int pair_stride;
  float c;  // log2(e) / sqrt(d_head)
};

// The dispatcher hands workgroup i to XCD i % XCDS, and each XCD has its own L2.
constexpr int XCDS = 8;

__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// A logical work item: query tile qt (heaviest first when causal), head group
// sub, key/value head h, sequence b.
struct WorkItem { int qt, sub, h, b; };

__device__ inline WorkItem decode_item(const AttnParams& p, int blk) {
  WorkItem w;
  w.qt = blk % p.n_qt;
  blk /= p.n_qt;
  if (p.causal) w.qt = p.n_qt - 1 - w.qt;
  w.sub = blk % p.n_sub;
  blk /= p.n_sub;
  w.h = blk % p.H_kv;
  w.b = blk / p.H_kv;
  return w;
}

// Keys a work item processes (each of its waves walks them all); 0 for a tile
// wholly in its sequence's padding.
__device__ inline int item_keys(const AttnParams& p, const WorkItem& w) {
  const int L = p.lens ? min(max(p.lens[w.b], 0), p.N) : p.N;
  const int q0 = w.qt * p.q_per_wg;
  if (q0 >= L) return 0;
  return p.causal ? min(L, q0 + p.q_per_wg) : L;
}

constexpr int LPT_MAX = 8192;   // work items the one-workgroup sort holds in LDS

// Longest-processing-time order of a ragged launch: one workgroup bitonic-sorts
// the grid's logical work items by their key counts, largest first (ties by
// index), so that the dispatcher starts the long tiles first and the short ones
// fill the tail. Sequences of different lengths otherwise leave CUs idle at the
// end of the grid.
__global__ __launch_bounds__(1024) void lpt_order(AttnParams p, int grid, int n_pow2,
                                                  int32_t* order) {
  __shared__ int key[LPT_MAX], val[LPT_MAX];
  for (int i = threadIdx.x; i < n_pow2; i += 1024) {
    key[i] = i < grid ? item_keys(p, decode_item(p, i)) : -1;
    val[i] = i;
  }
  __syncthreads();
  for (int k = 2; k <= n_pow2; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < n_pow2; i += 1024) {
        const int l = i ^ jj;
        if (l > i) {
          // descending by key, ascending by index among equal keys
          const bool i_first = key[i] > key[l] || (key[i] == key[l] && val[i] < val[l]);
          const bool want_i_first = (i & k) == 0;
          if (i_first != want_i_first) {
            const int tk = key[i], tv = val[i];
            key[i] = key[l]; val[i] = val[l];
            key[l] = tk; val[l] = tv;
          }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < grid; i += 1024) order[i] = val[i];
}

// Two waves per SIMD, except fp32 at d_head 64, whose operand fragments and
// accumulators take more than the 256 registers a wave has at that occupancy.
template <typename T, int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, sizeof(T) == 2 || D < 64 ? 2 : 1) void attn_kernel(AttnParams p) {
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int KCPR = D / EPC, VCPR = KT / EPC;
  constexpr int K_ELEMS = KT * D;              // elements of one tile's K (and of its V^T)
  constexpr int TILE = 2 * K_ELEMS;
  constexpr int K_INS = K_ELEMS / (64 * EPC);      // 1 KB direct loads of a tile's K (and of V^T)
  constexpr int INS = 2 * K_INS / WAVES;           // loads per wave per tile
  constexpr int VM_PER_TILE = INS;
  static_assert(INS * WAVES == 2 * K_INS && K_INS * 64 * EPC == K_ELEMS, "tile split");
  __shared__ __align__(16) T smem[NBUF * TILE];

  // The wave index is the same in every lane; readfirstlane lets the compiler
  // see that, so branches on it (the masked-block test) stay real branches
  // instead of predicated code that every step would execute.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;

  // Renumber the workgroups so that each XCD runs logical chunks of `chunk`
  // consecutive query tiles of one K/V stream, as many as the XCD holds at
  // once. The chunk's workgroups start together and walk the same K/V rows
  // within a few thousand keys of each other, so all but the first read of
  // each K/V tile hit that XCD's L2. In round r the XCDs take chunks 8r..8r+7,
  // in reverse order on odd rounds: the assignment to XCDs is static, and with
  // causal work falling linearly along the chunks this gives every XCD the same
  // total. Blocks from remap_end on keep their index.
  // A ragged launch may instead take its work items in a precomputed order.
  int blk = blockIdx.x, kpart = -1;
  bool light = false;   // the lighter tile of a pair: its waves take the slots in reverse
  if (p.order) {
    blk = p.order[blk];
  } else if (p.pair_stride) {
    const int ps = p.pair_stride, within = blk % (2 * ps);
    const int pi = blk / (2 * ps) * ps + within % ps, hn = p.n_qt / 2;
    light = within >= ps;
    const int r = pi % hn;   // 0: the stream's heaviest tile (decode_item reverses causal tiles)
    blk = pi / hn * p.n_qt + (light ? p.n_qt - 1 - r : r);
  } else if (blk >= p.split_begin) {   // part kpart of a split work item
    const int sidx = blk - p.split_begin;
    blk = p.split_begin + sidx / p.n_split;
    kpart = sidx % p.n_split;
  } else if (blk < p.remap_end) {
    const int xcd = blk % XCDS, s = blk / XCDS, r = s / p.chunk;
    blk = (r * XCDS + ((r & 1) ? XCDS - 1 - xcd : xcd)) * p.chunk + s % p.chunk;
  }
  const WorkItem item = decode_item(p, blk);   // causal: heaviest query tiles first
  const int qt = item.qt, sub = item.sub, h = item.h, b = item.b;
  const int waves_per_head = WAVES / p.G;
  // Waves w and w+4 of an 8-wave workgroup share a SIMD. The second four take
  // the (head, row block) slots in reverse order, so each SIMD pairs a low
  // row block with a high one and carries the same causal work.
  const int slot = (WAVES == 8 && wave >= 4) ? 11 - wave : light ? WAVES - 1 - wave : wave;
  const int head = h * p.g + sub * p.G + slot / waves_per_head;
  const int q0 = qt * p.q_per_wg;
  const int qw = q0 + (slot % waves_per_head) * QW;   // first query row of this wave
  // Tokens of this sequence: N, or its own length in a padded batch. Its keys
  // end there, and its rows from there on are zero.
  const int L = p.lens ? min(max(p.lens[b], 0), p.N) : p.N;
  // First key of this workgroup's range (0 unless it is part of a split item);
  // key indexes below count from it, and the sequence ends Lk keys after it.
  const int kb0 = kpart >= 0 ? kpart * p.split_keys : 0;
  const int Lk = L - kb0;

  // A query tile wholly in the padding: zero rows, no keys (uniform per workgroup).
  if (q0 >= L) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int t = qw + 32 * qb + col;
      if (p.lse && grp == 0 && t < p.Np)
        p.lse[((int64_t)b * p.H_q + head) * p.Np + t] = INFINITY;
      if (t < p.N) {
        T* arow = (T*)p.a + ((int64_t)b * p.N + t) * ((int64_t)p.H_q * D) + head * D;
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            T* dst = arow + nb * 32 + 8 * rq + 4 * grp;
            if constexpr (sizeof(T) == 2) *reinterpret_cast<bf16x4*>(dst) = bf16x4{};
            else *reinterpret_cast<f32x4*>(dst) = f32x4{};
            if (p.o32)
              *reinterpret_cast<f32x4*>(p.o32 + (arow - (T*)p.a) + nb * 32 + 8 * rq + 4 * grp) = f32x4{};
          }
      }
    }
    return;
  }

  const T* Qh = (const T*)p.q + ((int64_t)b * p.H_q + head) * (int64_t)p.Np * D;
  const T* Kh = (const T*)p.k + ((int64_t)b * p.H_kv + h) * (int64_t)p.Np * D + (int64_t)kb0 * D;
  const T* Vh = (const T*)p.vt + ((int64_t)b * p.H_kv + h) * (int64_t)D * p.Np + kb0;

  // Q as the B operand of S^T = K Q^T: lane -> query qw + 32*qb + col, k-group grp.
  // A query tile may reach past Np (tiles of 512 rows, Np a multiple of 256):
  // such rows read row Np-1 and are never stored.
  Frag qf[QB][D / MF::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < D / MF::KS; ++s)
      qf[qb][s] = *reinterpret_cast<const Frag*>(
          Qh + (int64_t)min(qw + 32 * qb + col, p.Np - 1) * D + s * MF::KS + grp * MF::E);

  // The workgroup stages the keys of its last query; this wave computes the
  // blocks up to its own last query (nblk_w) and only keeps pace with the
  // tile ring for the rest.
  const int kv_len = p.causal ? min(L, q0 + p.q_per_wg) : kpart >= 0 ? min(Lk, p.split_keys) : L;
  const int nblk = (kv_len + 31) / 32;
  const int nblk_w = p.causal ? (min(kv_len, qw + QW) + 31) / 32 : nblk;
  const int n_tiles = (kv_len + KT - 1) / KT;

  // Direct global->LDS loads of tile t into ring slot t % NBUF. Lane L of a
  // load lands at 16*L bytes past the load's LDS base, so the source address
  // chosen per lane realises the key permutation and the chunk swizzle. The
  // tile's 1 KB loads (K first, then V^T) are split evenly over the waves.
  // bf16 loads through buffer resources over this head's K and V^T: a 32-bit
  // per-lane offset fixed for the whole kernel and the tile's position as a
  // scalar offset. That keeps one VGPR per load instead of a 64-bit address
  // (the 4-wave form issues four loads per wave and spilled with addresses),
  // and buffer loads count only in vmcnt, so the compiler's waits for the LDS
  // fragment reads stay exact (with a global_load_lds in flight it waits for
  // every LDS read). A head's K or V^T holds at most 2^31 bytes in bf16
  // (N <= 2^24, d_head <= 64), so every offset, and the tile's scalar offset
  // k0 * D * 2 < 2^31, fits; the resources take the whole 32-bit range as
  // their size, which the in-range offsets never reach. fp32 heads can exceed
  // 32-bit offsets and keep 64-bit addresses.
  [[maybe_unused]] uint32_t loff[INS];
  [[maybe_unused]] __amdgpu_buffer_rsrc_t rsK, rsV;
  if constexpr (sizeof(T) == 2) {
    rsK = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, -1, 0x00020000);
    rsV = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < INS; ++i) {
      const int ins = wave * INS + i;
      if (ins < K_INS) {
        const int pos = ins * 64 + lane;
        const int r = pos / KCPR, slot = pos % KCPR;
        loff[i] = (uint32_t)((swap23(r) * D + (slot ^ swz<KCPR>(r)) * EPC) * (int)sizeof(T));
      } else {
        const int pos = (ins - K_INS) * 64 + lane;
        const int r = pos / VCPR, slot = pos % VCPR;
        loff[i] = (uint32_t)r * (uint32_t)p.Np * (uint32_t)sizeof(T) + (uint32_t)((slot ^ swz<VCPR>(r)) * EPC * (int)sizeof(T));
      }
    }
  }
  auto issue = [&](int t) {
    if (t >= n_tiles) return;
    T* kb = smem + (t % NBUF) * TILE;
    const int k0 = t * KT;
#pragma unroll
    for (int i = 0; i < INS; ++i) {
      const int ins = wave * INS + i;            // 0 .. 2*K_INS-1
      if constexpr (sizeof(T) == 2) {
        if (ins < K_INS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_ptr)(kb + ins * 64 * EPC), 16, (int)loff[i],
                                                   k0 * D * (int)sizeof(T), 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_ptr)(kb + K_ELEMS + (ins - K_INS) * 64 * EPC), 16,
                                                   (int)loff[i], k0 * (int)sizeof(T), 0, 0);
      } else if (ins < K_INS) {
        const int pos = ins * 64 + lane;
        const int r = pos / KCPR, slot = pos % KCPR;
        const T* src = Kh + (int64_t)(k0 + swap23(r)) * D + (slot ^ swz<KCPR>(r)) * EPC;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(kb + ins * 64 * EPC), 16, 0, 0);
      } else {
        const int vi = ins - K_INS;
        const int pos = vi * 64 + lane;
        const int r = pos / VCPR, slot = pos % VCPR;
        const T* src = Vh + (int64_t)r * p.Np + k0 + (slot ^ swz<VCPR>(r)) * EPC;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(kb + K_ELEMS + vi * 64 * EPC), 16, 0, 0);
      }
    }
  };

  // The ring slot and the parity of block j, from j itself or, as
  // std::integral_constant<int, M>, from M = j mod 2*NBUF known at compile
  // time. Then a fragment's LDS address is a lane part the loop does not
  // change plus a constant (the slot's byte offset fits a ds_read's 16-bit
  // immediate), and the step spends no VALU on addresses.
  auto slot_par = [&](int j, auto jm) {
    if constexpr (std::is_same_v<decltype(jm), DynBlock>) return std::pair<int, int>{(j >> 1) % NBUF, j & 1};
    else return std::pair<int, int>{(decltype(jm)::value >> 1) % NBUF, decltype(jm)::value & 1};
  };
  // K fragment (A operand of S^T) of global 32-key block j, k-step st.
  auto kfrag = [&](int j, int st, auto jm) -> Frag {
    const auto [sl, par] = slot_par(j, jm);
    const int r = par * 32 + col;
    const int e = st * MF::KS + grp * MF::E;
    const int off = sl * TILE + r * D + (((e / EPC) ^ swz<KCPR>(r)) * EPC) + e % EPC;
    return *reinterpret_cast<const Frag*>(&smem[off]);
  };
  // V^T fragment (A operand of O^T) of block j: head dims 32*nb + col,
  // keys kk.. of the block (8 consecutive for bf16, one for fp32).
  auto vfrag = [&](int j, int nb, int kk, auto jm) -> Frag {
    const auto [sl, par] = slot_par(j, jm);
    const int r = nb * 32 + col;
    const int key = par * 32 + kk;
    const int off = sl * TILE + K_ELEMS + r * KT + (((key / EPC) ^ swz<VCPR>(r)) * EPC) + key % EPC;
    return *reinterpret_cast<const Frag*>(&smem[off]);
  };

  f32x16 o[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[qb][nb] = f32x16{};
  float m_ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) l_run[qb] = 0.f;
  const float c = p.c;

  // S^T of block j for both query blocks. Register r of lane group grp holds
  // key 32*j + 16*(r/8) + 8*grp + r%8 (after the LDS row swap).
  auto qk = [&](int j, f32x16 (&s)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / MF::KS; ++st) {
      const Frag a = kfrag(j, st, DynBlock{});
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = MF::run(a, qf[qb][st], s[qb]);
    }
  };

  // After softmax, a block's probabilities live in its own S registers: bf16
  // pairs packed into the first 8 fp32 slots of each query block (fp32 runs
  // keep all 16 values). PV reads them there, before QK of a later block
  // overwrites the registers.
  auto pfrag = [&](const f32x16& sp, int half) -> Frag {
    if constexpr (sizeof(T) == 2) {
      const f32x4 v = {sp[4 * half], sp[4 * half + 1], sp[4 * half + 2], sp[4 * half + 3]};
      return __builtin_bit_cast(Frag, v);
    } else {
      return sp[half];
    }
  };

  // O^T += V^T P^T for block j, with P in sp.
  auto pv = [&](int j, const f32x16 (&sp)[QB]) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const Frag a = vfrag(j, nb, half * 16 + grp * 8, DynBlock{});
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][nb] = MF::run(a, pfrag(sp[qb], half), o[qb][nb]);
        }
    } else {
#pragma unroll
      for (int st = 0; st < 16; ++st)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const Frag a = vfrag(j, nb, 16 * (st >> 3) + 8 * grp + (st & 7), DynBlock{});
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][nb] = MF::run(a, pfrag(sp[qb], st), o[qb][nb]);
        }
    }
  };

  // The weight of score s against reference m: exp2(s*c - m) clamped to [0, 1]
  // (the median folds into the clamp bit of v_exp_f32).
  auto expw = [&](float sv, float m) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(fmaf(sv, c, -m)), 0.0f, 1.0f);
  };

  // p = exp2(s*c - m_ref) in place, packed as PV consumes it, and each lane's
  // block sums (taken on the rounded bf16 values that PV multiplies).
  auto exponentiate = [&](f32x16 (&s)[QB], float (&bsum)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mb = m_ref[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][r] = expw(s[qb][r], mb);
      if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
        float packed[8];
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bf16x2 pr = __builtin_convertvector(f32x2{s[qb][2 * e], s[qb][2 * e + 1]}, bf16x2);
          packed[e] = __builtin_bit_cast(float, pr);
          if (e & 1) acc1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc1, false);
          else acc0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc0, false);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s[qb][e] = packed[e];
        bsum[qb] = acc0 + acc1;
      } else {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += s[qb][r];
        bsum[qb] = acc;
      }
    }
  };

  auto mask = [&](f32x16 (&s)[QB], int j) __attribute__((always_inline)) {
    const int k0b = j * 32;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qw + 32 * qb + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0b + 16 * (r >> 3) + 8 * grp + (r & 7);
        if (key >= Lk || (p.causal && key > qi)) s[qb][r] = -INFINITY;
      }
    }
  };

  // Each row's max over the scores s of one block (-inf if all are masked).
  auto block_max = [&](const f32x16 (&s)[QB], float (&m)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float v = max3(s[qb][0], s[qb][1], s[qb][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) v = max3(v, s[qb][r], s[qb][r + 1]);
      v = fmaxf(v, s[qb][15]);
      m[qb] = fmaxf(v, __shfl_xor(v, 32));
    }
  };

  // Raise each row's reference to MARGIN binades above the max of the scores
  // s (never lower it), rescaling O and l by the change.
  auto rebase = [&](const f32x16 (&s)[QB]) __attribute__((always_inline)) {
    float m[QB];
    block_max(s, m);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = fmaxf(m_ref[qb], fmaf(m[qb], c, MARGIN));
      const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
      l_run[qb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[qb][nb] *= alpha;
      m_ref[qb] = m_new;
    }
  };

  // The exact fallback of block j's softmax, used only when its sums showed
  // that m_ref fell too far behind for it (before its PV product). Block j's
  // keys are still in the LDS ring, so its scores are recomputed, not kept.
  auto rescale = [&](int j, f32x16 (&s)[QB], float (&bsum)[QB], bool masked) __attribute__((always_inline)) {
    qk(j, s);
    if (masked) mask(s, j);
    rebase(s);
    exponentiate(s, bsum);
  };

  // The negated weights -P of scores s (bf16 path), packed as PV consumes
  // them: the sign flip happens before the rounding to bf16, which rounds
  // symmetrically, so they are exactly -P. (Flipping the sign bits of the
  // packed pairs afterwards, an xor on the f32 vector slots, was miscompiled:
  // the slots came out as copies of the first pair.)
  auto neg_weights = [&](f32x16 (&s)[QB]) __attribute__((always_inline)) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float packed[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16x2 pr = __builtin_convertvector(
            f32x2{-expw(s[qb][2 * e], m_ref[qb]), -expw(s[qb][2 * e + 1], m_ref[qb])}, bf16x2);
        packed[e] = __builtin_bit_cast(float, pr);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s[qb][e] = packed[e];
    }
  };

  // One pipeline step for block j (bf16). s_cur holds S(j); s_next holds
  // P(j-1). The MFMAs of O += V^T P(j-1), then of S(j+1) = K Q^T (into
  // s_next, once PV has read it), are independent of block j's softmax. The
  // step is laid out as one group per MFMA, each carrying the VALU work of one
  // pair of scores (the exponentials of the next pair and the bf16 packing and
  // row sum of the current one) and, every other group, the LDS fragment read
  // for the MFMA four groups ahead. sched_barrier keeps this order, so the
  // MFMA pipe and the VALU stay busy together and the register set stays what
  // the layout implies. S(j+1) of the last block and P(-1) = 0 are padding
  // that keeps each step straight-line.
  auto step_interleaved = [&](int j, f32x16 (&sc)[QB], f32x16 (&sn)[QB], float (&bsum)[QB], auto jm) __attribute__((always_inline)) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    constexpr int NB = D / 32, NST = D / MF::KS;
    constexpr int N_PV = 2 * NB * QB, N_QK = NST * QB, NG = N_PV + N_QK;
    constexpr int PAIRS = QB * 8, PPG = PAIRS / NG > 0 ? PAIRS / NG : 1;   // score pairs per group
    static_assert(sizeof(T) != 2 || PPG * NG == PAIRS, "pairs per group");
    const int jp = j > 0 ? j - 1 : 0;
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    Frag vf[2][NB], kf[NST];
    // the fragment whose first use is MFMA group u (u % QB == 0)
    auto fetch = [&](int u) {
      if (u < N_PV) {
        const int half = u / (NB * QB), nb = (u % (NB * QB)) / QB;
        if constexpr (std::is_same_v<decltype(jm), DynBlock>)
          vf[half][nb] = vfrag(jp, nb, half * 16 + grp * 8, jm);
        else   // a static step is never block 0, so jp = j - 1
          vf[half][nb] = vfrag(jp, nb, half * 16 + grp * 8,
                               std::integral_constant<int, (decltype(jm)::value + 2 * NBUF - 1) % (2 * NBUF)>{});
      } else if (u < NG) {
        const int st = (u - N_PV) / QB;
        if constexpr (std::is_same_v<decltype(jm), DynBlock>)
          kf[st] = kfrag(j + 1, st, jm);
        else
          kf[st] = kfrag(j + 1, st, std::integral_constant<int, (decltype(jm)::value + 1) % (2 * NBUF)>{});
      }
    };
    float acc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[qb][0] = acc[qb][1] = 0.f;
    float x[2 * PPG];   // exponentials of the pairs packed in the next group
    auto expo = [&](int pr, float* dst) {   // pair pr: scores 2e, 2e+1 of query block qb
      const int qb = pr / 8, e = pr % 8;
      dst[0] = expw(sc[qb][2 * e], m_ref[qb]);
      dst[1] = expw(sc[qb][2 * e + 1], m_ref[qb]);
    };
#pragma unroll
    for (int u = 0; u < FETCH_AHEAD * QB; u += QB) fetch(u);
#pragma unroll
    for (int k = 0; k < PPG; ++k) expo(k, &x[2 * k]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g % QB == 0) fetch(g + FETCH_AHEAD * QB);
      if (g < N_PV) {
        const int half = g / (NB * QB), nb = (g % (NB * QB)) / QB, qb = g % QB;
        o[qb][nb] = MF::run(vf[half][nb], pfrag(sn[qb], half), o[qb][nb]);
      } else {
        const int st = (g - N_PV) / QB, qb = g % QB;
        sn[qb] = MF::run(kf[st], qf[qb][st], st == 0 ? f32x16{} : sn[qb]);
      }
#pragma unroll
      for (int k = 0; k < PPG; ++k) {
        const int pr = g * PPG + k, qb = pr / 8, e = pr % 8;
        const bf16x2 pk = __builtin_convertvector(f32x2{x[2 * k], x[2 * k + 1]}, bf16x2);
        acc[qb][e & 1] = __builtin_amdgcn_fdot2_f32_bf16(pk, one, acc[qb][e & 1], false);
        sc[qb][e] = __builtin_bit_cast(float, pk);   // slot e: its own scores are already used
        if (pr + PPG < PAIRS) expo(pr + PPG, &x[2 * k]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bsum[qb] = acc[qb][0] + acc[qb][1];
    // Block j's weights and sums are dead on the rare path after this step
    // (it recomputes them), so the compiler would sink their computation
    // below that branch, out of the interleaved groups. This empty statement
    // reads and redefines them here, which keeps the exponentials beside the
    // MFMAs they were laid out with. (The row-sum dot2s still collect at the
    // end of the step; keeping them in their groups as well measured 4%
    // slower: each would wait on the bf16 pack just before it.)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(sc[qb]), "+v"(bsum[qb]));
  };

  // Masking touches only S(j), so it stays a small branch in front of the one
  // copy of the step body (two copies of the body would double its register
  // footprint at their merge). bsum carries the lane sums of the last block
  // whose check is still to come: in bf16, block j-1 on entry and block j on
  // exit (fp32 checks each block within its own step and leaves bsum at 0).
  // bf16 checks block j-1's sums at the end of step j, one step after they
  // were formed, so the branch never waits for them. If the check fails
  // (rarely: a row's max grew by more than about MARGIN - 5 binades), block
  // j-1's PV product is already in O: its clamped weights are recomputed
  // (the same scores against the same reference give the same values) and
  // that product is taken back out of O; then block j-1 is redone against its
  // exact max, and block j, exponentiated against the old reference, is
  // redone from its scores. s_cur serves as scratch; s_next keeps S(j+1).
  auto run_step = [&](int j, f32x16 (&s_cur)[QB], f32x16 (&s_next)[QB], auto mask_on,
                      float (&bsum)[QB], auto jm) __attribute__((always_inline)) {
    const bool masked =
        decltype(mask_on)::value && (j * 32 + 32 > Lk || (p.causal && j * 32 + 31 > qw));
    if (masked) mask(s_cur, j);
    float bcur[QB];
    if constexpr (sizeof(T) == 2) {
      step_interleaved(j, s_cur, s_next, bcur, jm);
      bool redo = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) redo |= !(bsum[qb] <= SUM_LIMIT);
      if (__builtin_expect(__any(redo), 0)) {   // j >= 1: block -1's sums are 0
        qk(j - 1, s_cur);
        if (decltype(mask_on)::value) mask(s_cur, j - 1);
        neg_weights(s_cur);
        pv(j - 1, s_cur);   // O -= V^T P^T
        rescale(j - 1, s_cur, bsum, decltype(mask_on)::value);
        pv(j - 1, s_cur);
        qk(j, s_cur);
        if (masked) mask(s_cur, j);
        exponentiate(s_cur, bcur);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) { l_run[qb] += bsum[qb]; bsum[qb] = bcur[qb]; }
    } else {
      pv(j > 0 ? j - 1 : 0, s_next);
      qk(j + 1, s_next);
      exponentiate(s_cur, bcur);
      bool redo = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) redo |= !(bcur[qb] <= SUM_LIMIT);
      if (__builtin_expect(__any(redo), 0)) rescale(j, s_cur, bcur, masked);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += bcur[qb];
    }
  };

  // After a wave's last step, block j (in s_cur): its pending check (bf16),
  // then its PV product.
  auto finish = [&](int j, f32x16 (&s_cur)[QB], float (&bsum)[QB]) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
      bool redo = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) redo |= !(bsum[qb] <= SUM_LIMIT);
      if (__builtin_expect(__any(redo), 0)) rescale(j, s_cur, bsum, true);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += bsum[qb];
    }
    pv(j, s_cur);
  };

  // Prologue: tiles 0..NBUF-2 in flight, tile 0 visible, S of block 0, and
  // each row's reference MARGIN binades above its max over block 0 (key 0 is
  // visible to every row, so that max is finite).
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) issue(t);
  wait_vmcnt<0>();
  __syncthreads();

  f32x16 sA[QB], sB[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) sB[qb] = f32x16{};   // P(-1) = 0
  qk(0, sA);
  if (32 > Lk || (p.causal && 31 > qw)) mask(sA, 0);
  {
    float m0[QB];
    block_max(sA, m0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = fmaf(m0[qb], c, MARGIN);
  }
  float bsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) bsum[qb] = 0.f;
  // Before odd block 2t+1: tile t+1 must be visible (loads of tiles t+2.. may
  // still be in flight), and tile t-1 is no longer read, so its slot takes
  // tile t+NBUF-1.
  auto advance = [&](int j) __attribute__((always_inline)) {
    const int t = j >> 1;
    wait_vmcnt_tiles<VM_PER_TILE, NBUF - 3>(min(NBUF - 3, max(0, n_tiles - (t + 2))));
    __syncthreads();
    issue(t + NBUF - 1);
  };
  // Blocks before jc (even) need no mask for this wave: their keys precede its
  // first query (causal) and the sequence end. That loop is compiled without
  // the mask code; the second keeps it. Every wave passes the barriers at the
  // same blocks, whichever loop it is in, and steps only up to nblk_w
  // (jc <= nblk_w). A wave's last block is finished right after its step: the
  // next advance() but one recycles that block's tile.
  const int jc = min(nblk, min(Lk / 32, p.causal ? qw / 32 : nblk)) & ~1;
  // The mask-free loop runs its first 2*NBUF blocks with the slot from j (block
  // 0's step reads block 0 for its padding PV), then NBUF tiles per iteration
  // with every slot known at compile time, then the rest with the slot from j.
  int j = 0;
  for (; j < jc && j < 2 * NBUF; j += 2) {
    run_step(j, sA, sB, std::false_type{}, bsum, DynBlock{});
    advance(j);   // j + 1 < jc <= nblk
    run_step(j + 1, sB, sA, std::false_type{}, bsum, DynBlock{});
  }
  if constexpr (sizeof(T) == 2) {
    for (; j + 2 * NBUF <= jc; j += 2 * NBUF) {   // j % (2 * NBUF) == 0
      static_for<0, NBUF>([&](auto tc) {
        constexpr int m = 2 * decltype(tc)::value;
        run_step(j + m, sA, sB, std::false_type{}, bsum, std::integral_constant<int, m>{});
        advance(j + m);
        run_step(j + m + 1, sB, sA, std::false_type{}, bsum, std::integral_constant<int, m + 1>{});
      });
    }
  }
  for (; j < jc; j += 2) {
    run_step(j, sA, sB, std::false_type{}, bsum, DynBlock{});
    advance(j);
    run_step(j + 1, sB, sA, std::false_type{}, bsum, DynBlock{});
  }
  for (; j < nblk; j += 2) {
    if (j < nblk_w) {
      run_step(j, sA, sB, std::true_type{}, bsum, DynBlock{});
      if (j + 1 == nblk_w) finish(j, sA, bsum);
    }
    if (j + 1 < nblk) {
      advance(j);
      if (j + 1 < nblk_w) {
        run_step(j + 1, sB, sA, std::true_type{}, bsum, DynBlock{});
        if (j + 2 == nblk_w) finish(j + 1, sB, bsum);
      }
    }
  }
  if (jc == nblk_w) finish(nblk_w - 1, sB, bsum);   // every block in the first loop (nblk_w even)

  if (kpart >= 0) {   // a part of a split item: its unnormalised state
    const int64_t rows_item = (int64_t)p.G * p.q_per_wg;
    const int64_t prow0 = (int64_t)((blk - p.split_begin) * p.n_split + kpart) * rows_item +
                          (int64_t)(slot / waves_per_head) * p.q_per_wg + (qw - q0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int64_t prow = prow0 + 32 * qb + col;
      const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
      float* po = p.part + prow * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *reinterpret_cast<f32x4*>(po + nb * 32 + 8 * rq + 4 * grp) =
              f32x4{o[qb][nb][4 * rq], o[qb][nb][4 * rq + 1], o[qb][nb][4 * rq + 2], o[qb][nb][4 * rq + 3]};
      if (grp == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * prow) = float2{m_ref[qb], l_tot};
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = qw + 32 * qb + col;
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.f / l_tot;
    const bool pad = t >= L;   // padding row of its sequence: stored as zeros
    // p = exp2(s*c - m_ref) / l_tot = exp2(s*c - (m_ref + log2 l_tot)); padding
    // rows get +inf, so every weight recomputed from it is 0
    if (p.lse && grp == 0 && t < p.Np)
      p.lse[((int64_t)b * p.H_q + head) * p.Np + t] = pad ? INFINITY : m_ref[qb] + log2f(l_tot);
    if (t < p.N) {
      T* arow = (T*)p.a + ((int64_t)b * p.N + t) * ((int64_t)p.H_q * D) + head * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          // rows 8*rq + 4*grp + 0..3 of this O^T tile are 4 consecutive head dims
          T* dst = arow + nb * 32 + 8 * rq + 4 * grp;
          const float v0 = pad ? 0.f : o[qb][nb][4 * rq] * inv;
          const float v1 = pad ? 0.f : o[qb][nb][4 * rq + 1] * inv;
          const float v2 = pad ? 0.f : o[qb][nb][4 * rq + 2] * inv;
          const float v3 = pad ? 0.f : o[qb][nb][4 * rq + 3] * inv;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(dst) =
                bf16x4{from_f32<T>(v0), from_f32<T>(v1), from_f32<T>(v2), from_f32<T>(v3)};
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
          }
          if (p.o32)   // the unrounded output, for the backward pass's rowsum(dO * O)
            *reinterpret_cast<f32x4*>(p.o32 + (dst - (T*)p.a)) = f32x4{v0, v1, v2, v3};
        }
    }
  }
}

// The parts of each split work item combined into its rows of A (and lse, o32):
// with part k's reference m_k, sum l_k and unnormalised O_k, and M the largest
// m_k, O = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k, and the row's
// log-sum-exp is M + log2 of that denominator. A thread takes four head dims of
// one row; rows past N are not stored (their lse is +inf, as in attn_kernel).
template <typename T, int D>
__global__ __launch_bounds__(256) void split_merge(AttnParams p, int n_items) {
  constexpr int GPR = D / 4, RPW = 256 / GPR;   // threads per row, rows per workgroup
  const int rows_item = p.G * p.q_per_wg;
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / GPR;
  if (row >= (int64_t)n_items * rows_item) return;
  const int dg = threadIdx.x % GPR;
  const int si = (int)(row / rows_item), rr = (int)(row % rows_item);
  const WorkItem it = decode_item(p, p.split_begin + si);
  const int head = it.h * p.g + it.sub * p.G + rr / p.q_per_wg;
  const int t = it.qt * p.q_per_wg + rr % p.q_per_wg;
  const int64_t prow0 = (int64_t)si * p.n_split * rows_item + rr;   // part k: prow0 + k * rows_item
  float M = -INFINITY;
  for (int k = 0; k < p.n_split; ++k) M = fmaxf(M, p.part_ml[2 * (prow0 + (int64_t)k * rows_item)]);
  float l = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  for (int k = 0; k < p.n_split; ++k) {
    const int64_t pr = prow0 + (int64_t)k * rows_item;
    const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + 2 * pr);
    const f32x4 ov = *reinterpret_cast<const f32x4*>(p.part + pr * D + 4 * dg);
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    l = fmaf(w, ml.y, l);
    o0 = fmaf(w, ov[0], o0); o1 = fmaf(w, ov[1], o1); o2 = fmaf(w, ov[2], o2); o3 = fmaf(w, ov[3], o3);
  }
  const bool pad = t >= p.N;
  if (p.lse && dg == 0 && t < p.Np)
    p.lse[((int64_t)it.b * p.H_q + head) * p.Np + t] = pad ? INFINITY : M + log2f(l);
  if (pad) return;
  const float inv = 1.f / l;
  const float v0 = o0 * inv, v1 = o1 * inv, v2 = o2 * inv, v3 = o3 * inv;
  const int64_t off = ((int64_t)it.b * p.N + t) * ((int64_t)p.H_q * D) + head * D + 4 * dg;
  T* dst = (T*)p.a + off;
  if constexpr (sizeof(T) == 2) *reinterpret_cast<bf16x4*>(dst) = bf16x4{from_f32<T>(v0), from_f32<T>(v1), from_f32<T>(v2), from_f32<T>(v3)};
  else *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
  if (p.o32) *reinterpret_cast<f32x4*>(p.o32 + off) = f32x4{v0, v1, v2, v3};
}

template <typename T, int D, int WAVES>
hipError_t run(const AttnParams& p, unsigned grid, hipStream_t stream) {
  attn_kernel<T, D, WAVES><<<grid, 64 * WAVES, 0, stream>>>(p);
  return hipGetLastError();
}

template <int WAVES>
int64_t plan(AttnParams& p, int64_t B, int64_t H_kv) {
  p.G = 1;   // heads per workgroup: the largest power of two <= WAVES dividing g
  while (p.G * 2 <= WAVES && p.g % (p.G * 2) == 0) p.G *= 2;
  p.n_sub = p.g / p.G;
  p.q_per_wg = QW * (WAVES / p.G);
  p.n_qt = (p.N + p.q_per_wg - 1) / p.q_per_wg;
  return (int64_t)p.n_qt * p.n_sub * H_kv * B;
}

// Chunks of the XCD-aware order: one chunk is what an XCD holds at once
// (two waves per SIMD: 8 / WAVES workgroups per CU). No renumbering when the
// CU count does not split evenly over the XCDs.
template <int WAVES>
void plan_order(AttnParams& p, int64_t grid, int64_t cus) {   // grid: the items to renumber
  p.chunk = (int)(cus / XCDS) * (8 / WAVES);
  p.remap_end = 0;
  if (cus % XCDS == 0 && p.chunk > 0)
    p.remap_end = (int)(grid / ((int64_t)XCDS * p.chunk) * XCDS * p.chunk);
}

template <int WAVES>
hipError_t dispatch(sqa_dtype dt, int64_t d_head, AttnParams& p, int64_t grid, int64_t cus,
                    int32_t* order_ws, hipStream_t stream, int64_t remap_items = -1) {
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  plan_order<WAVES>(p, remap_items < 0 ? grid : remap_items, cus);
  // Sequences of different lengths break the chunk order's premise (equal
  // streams whose work falls linearly), and its static XCD assignment then
  // unbalances the XCDs (5.5 against 4.8 ms for plain round-robin on a batch of
  // 8 sequences of 9k-28k tokens). They run longest first instead.
  p.order = nullptr;
  if (p.lens) {
    p.remap_end = 0;
    if (order_ws && grid <= LPT_MAX) {
      int n = 1;
      while (n < grid) n <<= 1;
      lpt_order<<<1, 1024, 0, stream>>>(p, (int)grid, n, order_ws);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      p.order = order_ws;
    }
  }
  if (dt == SQA_DTYPE_BF16)
    return d_head == 64 ? run<bf16, 64, WAVES>(p, (unsigned)grid, stream)
                        : run<bf16, 32, WAVES>(p, (unsigned)grid, stream);
  if constexpr (WAVES == 8) {   // fp32 at d_head 64 always takes 4-wave workgroups
    if (d_head == 64) return hipErrorInvalidValue;
    return run<float, 32, WAVES>(p, (unsigned)grid, stream);
  } else {
    return d_head == 64 ? run<float, 64, WAVES>(p, (unsigned)grid, stream)
                        : run<float, 32, WAVES>(p, (unsigned)grid, stream);
  }
}

// Compute units of the stream's device (cached per device).
int cu_count(hipStream_t stream) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 ||
      dev >= 64)
    return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

// Workgroup shape: 8 waves (one workgroup per CU, 512 query rows sharing each
// K/V tile) by default. A non-causal grid whose last dispatch round would be
// under half full runs with 4-wave workgroups instead (two per CU): every
// workgroup of a non-causal grid costs the same, and the smaller ones pack
// that tail round over more CUs. Causal grids, dispatched heaviest first,
// fill their tail with short workgroups; one that fits a single round of
// 8-wave workgroups pairs its heavy and light tiles on each CU instead. fp32
// at d_head 64 always runs with 4-wave workgroups: its 8-wave form needs more
// than the 256 registers that two waves per SIMD leave.
// Key-split tail of a non-causal grid. Every non-causal work item streams all
// of its sequence's keys, so a grid of R full dispatch rounds and a partial
// one takes R + 1 round times (the 200k-token xSMQA workload: 1563 items on
// 256 CUs, 6.1 rounds run in 7). The items of the partial round are split
// over their keys into up to cus / tail parts of at least SPLIT_MIN_KEYS keys,
// so that round shrinks to about 1 / n_split of a round, and split_merge
// combines the parts. At most SPLIT_MAX_WGS workgroups are split parts.
constexpr int64_t SPLIT_MIN_KEYS = 2048, SPLIT_MAX_WGS = 256;
struct SplitPlan { int64_t full = 0, tail = 0, n_split = 1, keys = 0, bytes = 0; };

SplitPlan split_plan(sqa_dtype dt, int64_t B, int64_t N, int64_t H_q, int64_t H_kv, int64_t d_head,
                     bool causal, bool varlen, int64_t cus) {
  SplitPlan sp;
  if (causal || varlen || dt != SQA_DTYPE_BF16 || B * N == 0) return sp;
  AttnParams p{};
  p.N = (int)N; p.g = (int)(H_q / H_kv);
  const int64_t grid = plan<8>(p, B, H_kv);
  const int64_t tail = grid % cus;
  if (grid < cus || tail == 0) return sp;
  int64_t n = std::min(std::min(cus, SPLIT_MAX_WGS) / tail, N / SPLIT_MIN_KEYS);
  if (n < 2) return sp;
  const int64_t keys = ((N + n - 1) / n + KT - 1) / KT * KT;
  n = (N + keys - 1) / keys;   // every part holds keys
  if (n < 2) return sp;
  sp.full = grid - tail; sp.tail = tail; sp.n_split = n; sp.keys = keys;
  sp.bytes = tail * n * p.G * p.q_per_wg * (d_head + 2) * (int64_t)sizeof(float);
  return sp;
}

size_t attention_order_bytes(int64_t B, int64_t N, int64_t H_q) {
  // a bound on the grid: query tiles of at least 64 rows, at most H_q head groups
  return (size_t)(B * ((N + 63) / 64) * H_q) * sizeof(int32_t);
}

size_t attention_split_bytes(sqa_dtype dt, int64_t B, int64_t N, int64_t H_q, int64_t H_kv,
                             int64_t d_head, bool causal, bool varlen, hipStream_t stream) {
  return (size_t)split_plan(dt, B, N, H_q, H_kv, d_head, causal, varlen, cu_count(stream)).bytes;
}

size_t attention_split_bound(int64_t d_head) {
  return (size_t)(SPLIT_MAX_WGS * 8 * QW * (d_head + 2) * (int64_t)sizeof(float));
}

hipError_t launch_attention(sqa_dtype dt, const void* q, const void* k, const void* vt, void* a,
                            int64_t B, int64_t N, int64_t Np, int64_t H_q, int64_t H_kv,
                            int64_t d_head, bool causal, const int32_t* lens, hipStream_t stream,
                            float* lse, int32_t* order_ws, float* o32, float* split_ws) {
  AttnParams p;
  p.q = q; p.k = k; p.vt = vt; p.a = a; p.lens = lens; p.lse = lse; p.o32 = o32;
  p.N = (int)N; p.Np = (int)Np; p.H_q = (int)H_q; p.H_kv = (int)H_kv;
  p.g = (int)(H_q / H_kv);
  p.causal = causal ? 1 : 0;
  p.c = (float)(1.4426950408889634 / sqrt((double)d_head));
  p.split_begin = 0x7FFFFFFF; p.n_split = 1; p.split_keys = 0;
  p.part = nullptr; p.part_ml = nullptr; p.pair_stride = 0;
  AttnParams p8 = p;
  const int64_t grid8 = plan<8>(p8, B, H_kv);
  const int64_t cus = cu_count(stream);
  const int64_t tail = grid8 % cus;
  // A causal grid that fits one round of 8-wave workgroups ends when its
  // heaviest tiles do, while CUs holding light tiles idle. Run it as 4-wave
  // workgroups, two per CU, each CU pairing a heavy tile with its complement
  // in the same stream (slots reversed in the light one), so every SIMD carries
  // about the same number of block steps.
  if (causal && dt == SQA_DTYPE_BF16 && !lens && grid8 <= cus) {
    AttnParams p4 = p;
    const int64_t grid4 = plan<4>(p4, B, H_kv);
    if (grid4 <= 2 * cus && p4.n_qt % 2 == 0) {   // grid4 = streams * n_qt: even
      // The dispatcher puts blocks b and b + grid/2 of a one-round grid on one
      // CU: the first half takes the heavy tiles, the second their complements
      // (measured: pairs of neighbouring blocks, or blocks 8 apart, ran 33-34
      // against 25 us on the 16x1024 sSQA workload; unpaired 8-wave 31.5 us).
      p4.pair_stride = (int)(grid4 / 2);
      return dispatch<4>(dt, d_head, p4, grid4, cus, nullptr, stream, 0);
    }
  }
  const SplitPlan sp = split_ws ? split_plan(dt, B, N, H_q, H_kv, d_head, causal, lens != nullptr, cus)
                                : SplitPlan{};
  if (sp.n_split >= 2) {
    const int64_t grid = sp.full + sp.tail * sp.n_split, rows = grid - sp.full;
    p8.split_begin = (int)sp.full; p8.n_split = (int)sp.n_split; p8.split_keys = (int)sp.keys;
    p8.part = split_ws;
    p8.part_ml = split_ws + rows * p8.G * p8.q_per_wg * d_head;
    hipError_t e = dispatch<8>(dt, d_head, p8, grid, cus, nullptr, stream, sp.full);
    if (e != hipSuccess) return e;
    const int rpw = 256 / (int)(d_head / 4);
    const int64_t merge_rows = sp.tail * p8.G * p8.q_per_wg;
    const unsigned mgrid = (unsigned)((merge_rows + rpw - 1) / rpw);
    if (d_head == 64) split_merge<bf16, 64><<<mgrid, 256, 0, stream>>>(p8, (int)sp.tail);
    else split_merge<bf16, 32><<<mgrid, 256, 0, stream>>>(p8, (int)sp.tail);
    return hipGetLastError();
  }
  if ((!causal && tail != 0 && 2 * tail <= cus) || (dt == SQA_DTYPE_FP32 && d_head == 64)) {
    const int64_t grid4 = plan<4>(p, B, H_kv);
    return dispatch<4>(dt, d_head, p, grid4, cus, order_ws, stream);
  }
  return dispatch<8>(dt, d_head, p8, grid8, cus, order_ws, stream);
}

}  // namespace sqa
