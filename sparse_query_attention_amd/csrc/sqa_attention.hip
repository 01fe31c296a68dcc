// Attention core of the SQA forward pass on gfx950: per query head i,
//   A_i = softmax(Q_i K_j^T / sqrt(d)) V_j,   j = floor(i / (H_q/H_kv)),
// with an optional causal mask (key c visible to query r iff c <= r).
// SQA keeps GQA's key/value sharing and cuts the query heads, so the score
// work scales with H_q ("Sparse Query Attention (SQA)...", arXiv 2510.01817,
// abstract; ReactiveAI/GQA-Ref-Micro model card, description).
//
// Design (one workgroup = 4 waves of 64 lanes):
//  * A workgroup owns one (batch, key/value head) pair, G query heads of that
//    head's group and a tile of queries: 256x1, 128x2 or 64x4 queries x heads.
//    Every key/value tile staged in LDS is read by all G heads, so repeated
//    K/V is never materialised.
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
//    it spends: half a v_max3, one FMA, one v_exp, half a v_cvt_pk_bf16 and
//    half a v_dot2 (the row sum is taken on the bf16 P that the PV product
//    consumes). The O accumulators are rescaled lazily, only when a row's max
//    outgrows the reference by 2^8.
//  * Causal: key tiles past a workgroup's last query are never loaded, and a
//    wave skips the MFMAs of 32-key blocks past its own last query. Only
//    blocks that cross the diagonal or the sequence end are masked. The
//    heaviest query tiles are dispatched first.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int KT = 64;       // keys per LDS tile (two 32-key blocks)
constexpr int NBUF = 4;      // LDS tile ring: in use, visible next, NBUF-2 in flight
constexpr int QB = 2;             // 32-query MFMA column blocks per wave
constexpr int FETCH_AHEAD = 2;    // LDS fragments read ahead of their first MFMA
constexpr int QW = 32 * QB;       // query rows per wave
// Exponentials are taken against a reference max m_ref that may lag the true
// running max. A lane's block sum above SUM_LIMIT (or inf/NaN) means the
// reference is too low for that block; only then is the block's exact max
// computed, O and l rescaled and the block's exponentials redone.
constexpr float SUM_LIMIT = 256.0f;
constexpr float M_INIT = -1e30f;   // finite, so masked scores give exp2(-inf) = 0

struct AttnParams {
  const void* q; const void* k; const void* vt; void* a;
  const int32_t* lens;   // null, or each sequence's length (clamped into [0, N])
  float* lse;            // null, or [B, H_q, Np]: base-2 log-sum-exp of each row's scaled scores
  const int32_t* order;  // null, or the logical work item of each workgroup (lpt_order)
  float* o32;            // null, or [B*N, H_q*d]: the output before its rounding to T (fp32)
  int N, Np, H_q, H_kv, g, G, n_sub, q_per_wg, n_qt, causal;
  int chunk, remap_end;   // XCD-aware workgroup order (see the kernel's block decode)
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

template <typename T, int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void attn_kernel(AttnParams p) {
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
  int blk = blockIdx.x;
  if (p.order) {
    blk = p.order[blk];
  } else if (blk < p.remap_end) {
    const int xcd = blk % XCDS, s = blk / XCDS, r = s / p.chunk;
    blk = (r * XCDS + ((r & 1) ? XCDS - 1 - xcd : xcd)) * p.chunk + s % p.chunk;
  }
  const WorkItem item = decode_item(p, blk);   // causal: heaviest query tiles first
  const int qt = item.qt, sub = item.sub, h = item.h, b = item.b;
  const int waves_per_head = WAVES / p.G;
  const int head = h * p.g + sub * p.G + wave / waves_per_head;
  const int q0 = qt * p.q_per_wg;
  const int qw = q0 + (wave % waves_per_head) * QW;   // first query row of this wave
  // Tokens of this sequence: N, or its own length in a padded batch. Its keys
  // end there, and its rows from there on are zero.
  const int L = p.lens ? min(max(p.lens[b], 0), p.N) : p.N;

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
  const T* Kh = (const T*)p.k + ((int64_t)b * p.H_kv + h) * (int64_t)p.Np * D;
  const T* Vh = (const T*)p.vt + ((int64_t)b * p.H_kv + h) * (int64_t)D * p.Np;

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

  // All waves of the workgroup walk the same key range; rows past a wave's own
  // causal horizon are masked to zero weight.
  const int kv_len = p.causal ? min(L, q0 + p.q_per_wg) : L;
  const int nblk = (kv_len + 31) / 32;
  const int n_tiles = (kv_len + KT - 1) / KT;

  // Direct global->LDS loads of tile t into ring slot t % NBUF. Lane L of a
  // load lands at 16*L bytes past the load's LDS base, so the source address
  // chosen per lane realises the key permutation and the chunk swizzle. The
  // tile's 1 KB loads (K first, then V^T) are split evenly over the waves.
  auto issue = [&](int t) {
    if (t >= n_tiles) return;
    T* kb = smem + (t % NBUF) * TILE;
    const int k0 = t * KT;
#pragma unroll
    for (int i = 0; i < INS; ++i) {
      const int ins = wave * INS + i;            // 0 .. 2*K_INS-1
      if (ins < K_INS) {
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

  // K fragment (A operand of S^T) of global 32-key block j, k-step st.
  auto kfrag = [&](int j, int st) -> Frag {
    const int r = (j & 1) * 32 + col;
    const int e = st * MF::KS + grp * MF::E;
    const int off = ((j >> 1) % NBUF) * TILE + r * D + (((e / EPC) ^ swz<KCPR>(r)) * EPC) + e % EPC;
    return *reinterpret_cast<const Frag*>(&smem[off]);
  };
  // V^T fragment (A operand of O^T) of block j: head dims 32*nb + col,
  // keys kk.. of the block (8 consecutive for bf16, one for fp32).
  auto vfrag = [&](int j, int nb, int kk) -> Frag {
    const int r = nb * 32 + col;
    const int key = (j & 1) * 32 + kk;
    const int off = ((j >> 1) % NBUF) * TILE + K_ELEMS + r * KT +
                    (((key / EPC) ^ swz<VCPR>(r)) * EPC) + key % EPC;
    return *reinterpret_cast<const Frag*>(&smem[off]);
  };

  f32x16 o[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[qb][nb] = f32x16{};
  float m_ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_ref[qb] = M_INIT; l_run[qb] = 0.f; }
  const float c = p.c;

  // S^T of block j for both query blocks. Register r of lane group grp holds
  // key 32*j + 16*(r/8) + 8*grp + r%8 (after the LDS row swap).
  auto qk = [&](int j, f32x16 (&s)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / MF::KS; ++st) {
      const Frag a = kfrag(j, st);
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
  auto pv = [&](int j, const f32x16 (&sp)[QB]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const Frag a = vfrag(j, nb, half * 16 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][nb] = MF::run(a, pfrag(sp[qb], half), o[qb][nb]);
        }
    } else {
#pragma unroll
      for (int st = 0; st < 16; ++st)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const Frag a = vfrag(j, nb, 16 * (st >> 3) + 8 * grp + (st & 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][nb] = MF::run(a, pfrag(sp[qb], st), o[qb][nb]);
        }
    }
  };

  // p = exp2(s*c - m_ref) in place, packed as PV consumes it, and each lane's
  // block sums (taken on the rounded bf16 values that PV multiplies).
  auto exponentiate = [&](f32x16 (&s)[QB], float (&bsum)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mb = m_ref[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][r] = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -mb));
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

  auto mask = [&](f32x16 (&s)[QB], int j) {
    const int k0b = j * 32;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qw + 32 * qb + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0b + 16 * (r >> 3) + 8 * grp + (r & 7);
        if (key >= L || (p.causal && key > qi)) s[qb][r] = -INFINITY;
      }
    }
  };

  // The exact-rescale fallback of block j's softmax, used only when a block
  // sum showed that m_ref was too low for it. Block j's keys are still in
  // the LDS ring, so its scores are recomputed rather than kept.
  auto rescale = [&](int j, f32x16 (&s)[QB], float (&bsum)[QB], bool masked) {
    qk(j, s);
    if (masked) mask(s, j);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = max3(s[qb][0], s[qb][1], s[qb][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = max3(m, s[qb][r], s[qb][r + 1]);
      m = fmaxf(m, s[qb][15]);
      m = fmaxf(m, __shfl_xor(m, 32));
      const float m_new = fmaxf(m_ref[qb], m * c);
      const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
      l_run[qb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[qb][nb] *= alpha;
      m_ref[qb] = m_new;
    }
    exponentiate(s, bsum);
  };

  // One pipeline step for block j. s_cur holds S(j); s_next holds P(j-1).
  // The MFMAs of O += V^T P(j-1), then of S(j+1) = K Q^T (into s_next, once
  // PV has read it), are independent of block j's softmax. The step is laid
  // out as one group per MFMA, each carrying the VALU work of one pair of
  // scores (the exponentials of the next pair and the bf16 packing and row
  // sum of the current one) and, every other group, the LDS fragment read for
  // the MFMA four groups ahead. sched_barrier keeps this order, so the MFMA
  // pipe and the VALU stay busy together and the register set stays what the
  // layout implies. S(j+1) of the last block and P(-1) = 0 are padding that
  // keeps each step straight-line.
  auto step_interleaved = [&](int j, f32x16 (&sc)[QB], f32x16 (&sn)[QB], float (&bsum)[QB]) {
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
        vf[half][nb] = vfrag(jp, nb, half * 16 + grp * 8);
      } else if (u < NG) {
        const int st = (u - N_PV) / QB;
        kf[st] = kfrag(j + 1, st);
      }
    };
    float acc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[qb][0] = acc[qb][1] = 0.f;
    float x[2 * PPG];   // exponentials of the pairs packed in the next group
    auto expo = [&](int pr, float* dst) {   // pair pr: scores 2e, 2e+1 of query block qb
      const int qb = pr / 8, e = pr % 8;
      dst[0] = __builtin_amdgcn_exp2f(fmaf(sc[qb][2 * e], c, -m_ref[qb]));
      dst[1] = __builtin_amdgcn_exp2f(fmaf(sc[qb][2 * e + 1], c, -m_ref[qb]));
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
  };

  // Masking touches only S(j), so it stays a small branch in front of the one
  // copy of the step body (two copies of the body would double its register
  // footprint at their merge).
  auto run_step = [&](int j, f32x16 (&s_cur)[QB], f32x16 (&s_next)[QB], auto mask_on) {
    const bool masked =
        decltype(mask_on)::value && (j * 32 + 32 > L || (p.causal && j * 32 + 31 > qw));
    if (masked) mask(s_cur, j);
    float bsum[QB];
    if constexpr (sizeof(T) == 2) {
      step_interleaved(j, s_cur, s_next, bsum);
    } else {
      pv(j > 0 ? j - 1 : 0, s_next);
      qk(j + 1, s_next);
      exponentiate(s_cur, bsum);
    }
    bool redo = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) redo |= !(bsum[qb] <= SUM_LIMIT);
    if (__any(redo)) rescale(j, s_cur, bsum, masked);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += bsum[qb];
  };

  // Prologue: tiles 0..NBUF-2 in flight, tile 0 visible, S of block 0.
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) issue(t);
  wait_vmcnt<0>();
  __syncthreads();

  f32x16 sA[QB], sB[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) sB[qb] = f32x16{};   // P(-1) = 0
  qk(0, sA);
  // Before odd block 2t+1: tile t+1 must be visible (loads of tiles t+2.. may
  // still be in flight), and tile t-1 is no longer read, so its slot takes
  // tile t+NBUF-1.
  auto advance = [&](int j) {
    const int t = j >> 1;
    wait_vmcnt_tiles<VM_PER_TILE, NBUF - 3>(min(NBUF - 3, max(0, n_tiles - (t + 2))));
    __syncthreads();
    issue(t + NBUF - 1);
  };
  // Blocks before jc (even) need no mask for this wave: their keys precede its
  // first query (causal) and the sequence end. That loop is compiled without
  // the mask code; the second keeps it. Every wave passes the barriers at the
  // same blocks, whichever loop it is in.
  const int jc = min(nblk, min(L / 32, p.causal ? qw / 32 : nblk)) & ~1;
  int j = 0;
  for (; j < jc; j += 2) {
    run_step(j, sA, sB, std::false_type{});
    advance(j);   // j + 1 < jc <= nblk
    run_step(j + 1, sB, sA, std::false_type{});
  }
  for (; j < nblk; j += 2) {
    run_step(j, sA, sB, std::true_type{});
    if (j + 1 < nblk) {
      advance(j);
      run_step(j + 1, sB, sA, std::true_type{});
    }
  }
  if (nblk & 1) pv(nblk - 1, sA); else pv(nblk - 1, sB);

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
void plan_order(AttnParams& p, int64_t grid, int64_t cus) {
  p.chunk = (int)(cus / XCDS) * (8 / WAVES);
  p.remap_end = 0;
  if (cus % XCDS == 0 && p.chunk > 0)
    p.remap_end = (int)(grid / ((int64_t)XCDS * p.chunk) * XCDS * p.chunk);
}

template <int WAVES>
hipError_t dispatch(sqa_dtype dt, int64_t d_head, AttnParams& p, int64_t grid, int64_t cus,
                    int32_t* order_ws, hipStream_t stream) {
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  plan_order<WAVES>(p, grid, cus);
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
// fill their tail with short workgroups. fp32 at d_head 64 always runs with
// 4-wave workgroups: its 8-wave form needs more than the 256 registers that
// two waves per SIMD leave.
size_t attention_order_bytes(int64_t B, int64_t N, int64_t H_q) {
  // a bound on the grid: query tiles of at least 64 rows, at most H_q head groups
  return (size_t)(B * ((N + 63) / 64) * H_q) * sizeof(int32_t);
}

hipError_t launch_attention(sqa_dtype dt, const void* q, const void* k, const void* vt, void* a,
                            int64_t B, int64_t N, int64_t Np, int64_t H_q, int64_t H_kv,
                            int64_t d_head, bool causal, const int32_t* lens, hipStream_t stream,
                            float* lse, int32_t* order_ws, float* o32) {
  AttnParams p;
  p.q = q; p.k = k; p.vt = vt; p.a = a; p.lens = lens; p.lse = lse; p.o32 = o32;
  p.N = (int)N; p.Np = (int)Np; p.H_q = (int)H_q; p.H_kv = (int)H_kv;
  p.g = (int)(H_q / H_kv);
  p.causal = causal ? 1 : 0;
  p.c = (float)(1.4426950408889634 / sqrt((double)d_head));
  AttnParams p8 = p;
  const int64_t grid8 = plan<8>(p8, B, H_kv);
  const int64_t cus = cu_count(stream);
  const int64_t tail = grid8 % cus;
  if ((!causal && tail != 0 && 2 * tail <= cus) || (dt == SQA_DTYPE_FP32 && d_head == 64)) {
    const int64_t grid4 = plan<4>(p, B, H_kv);
    return dispatch<4>(dt, d_head, p, grid4, cus, order_ws, stream);
  }
  return dispatch<8>(dt, d_head, p8, grid8, cus, order_ws, stream);
}

}  // namespace sqa
