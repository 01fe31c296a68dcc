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

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int KT = 64;       // keys per LDS tile (two 32-key MFMA blocks)
constexpr int WAVES = 4;
constexpr int QB = 2;        // 32-query MFMA column blocks per wave
constexpr int QW = 32 * QB;  // query rows per wave
constexpr int THREADS = 64 * WAVES;
// Lazy rescaling: exponentials are taken against a reference max that may lag
// the true running max by up to 2^TAU_LOG2 in the exp2 domain (so p <= 256);
// the O accumulators are rescaled only when a row's max outgrows that margin.
constexpr float TAU_LOG2 = 8.0f;

struct AttnParams {
  const void* q; const void* k; const void* vt; void* a;
  int N, Np, H_q, H_kv, g, G, n_sub, q_per_wg, n_qt, causal;
  float c;  // log2(e) / sqrt(d_head)
};

template <typename T, int D> struct AttnCfg {
  static constexpr int EPC = 16 / sizeof(T);
  static constexpr int KLD = D + EPC;         // LDS K row (one key), 16-byte pad
  static constexpr int VLD = KT + EPC;        // LDS V^T row (one head dim), 16-byte pad
  static constexpr int K_PER = KT * D / EPC / THREADS;
  static constexpr int V_PER = D * KT / EPC / THREADS;
  static_assert(K_PER * THREADS * EPC == KT * D, "K tile split");
  static_assert(V_PER * THREADS * EPC == KT * D, "V tile split");
};

// In-tile key index <-> LDS row: swap bits 2 and 3 (an involution).
__device__ inline int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Row sum of 8 bf16 probabilities with two v_dot2_f32_bf16 chains.
__device__ inline float sum8(bf16x8 p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float a0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[0], p[1]}, one, acc, false);
  float a1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[2], p[3]}, one, 0.f, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[4], p[5]}, one, a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[6], p[7]}, one, a1, false);
  return a0 + a1;
}

template <typename T, int D>
__global__ __launch_bounds__(THREADS, 2) void attn_kernel(AttnParams p) {
  using Cfg = AttnCfg<T, D>;
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  __shared__ __align__(16) T Ks[2][KT * Cfg::KLD];
  __shared__ __align__(16) T Vs[2][D * Cfg::VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;

  int blk = blockIdx.x;
  int qt = blk % p.n_qt;
  blk /= p.n_qt;
  if (p.causal) qt = p.n_qt - 1 - qt;   // heaviest query tiles first
  const int sub = blk % p.n_sub;
  blk /= p.n_sub;
  const int h = blk % p.H_kv, b = blk / p.H_kv;
  const int waves_per_head = WAVES / p.G;
  const int head = h * p.g + sub * p.G + wave / waves_per_head;
  const int q0 = qt * p.q_per_wg;
  const int qw = q0 + (wave % waves_per_head) * QW;   // first query row of this wave

  const T* Qh = (const T*)p.q + ((int64_t)b * p.H_q + head) * (int64_t)p.Np * D;
  const T* Kh = (const T*)p.k + ((int64_t)b * p.H_kv + h) * (int64_t)p.Np * D;
  const T* Vh = (const T*)p.vt + ((int64_t)b * p.H_kv + h) * (int64_t)D * p.Np;

  // Q as the B operand of S^T = K Q^T: lane -> query qw + 32*qb + col, k-group grp.
  Frag qf[QB][D / MF::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < D / MF::KS; ++s)
      qf[qb][s] = *reinterpret_cast<const Frag*>(Qh + (int64_t)(qw + 32 * qb + col) * D +
                                                 s * MF::KS + grp * MF::E);

  const int kv_len = p.causal ? min(p.N, q0 + p.q_per_wg) : p.N;
  const int n_tiles = (kv_len + KT - 1) / KT;

  Chunk kreg[Cfg::K_PER], vreg[Cfg::V_PER];
  auto load = [&](int kt) {
    const int k0 = kt * KT;
#pragma unroll
    for (int i = 0; i < Cfg::K_PER; ++i) {
      const int c = tid + i * THREADS;
      const int key = c / (D / Cfg::EPC), cc = c % (D / Cfg::EPC);
      kreg[i] = *reinterpret_cast<const Chunk*>(Kh + (int64_t)(k0 + key) * D + cc * Cfg::EPC);
    }
#pragma unroll
    for (int i = 0; i < Cfg::V_PER; ++i) {
      const int c = tid + i * THREADS;
      const int row = c / (KT / Cfg::EPC), cc = c % (KT / Cfg::EPC);
      vreg[i] = *reinterpret_cast<const Chunk*>(Vh + (int64_t)row * p.Np + k0 + cc * Cfg::EPC);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Cfg::K_PER; ++i) {
      const int c = tid + i * THREADS;
      const int key = c / (D / Cfg::EPC), cc = c % (D / Cfg::EPC);
      *reinterpret_cast<Chunk*>(&Ks[buf][swap23(key) * Cfg::KLD + cc * Cfg::EPC]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::V_PER; ++i) {
      const int c = tid + i * THREADS;
      const int row = c / (KT / Cfg::EPC), cc = c % (KT / Cfg::EPC);
      *reinterpret_cast<Chunk*>(&Vs[buf][row * Cfg::VLD + cc * Cfg::EPC]) = vreg[i];
    }
  };

  f32x16 o[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[qb][nb] = f32x16{};
  float m_ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_ref[qb] = -INFINITY; l_run[qb] = 0.f; }
  const float c = p.c;

  // S^T of one 32-key block for both query blocks. Register r of lane group
  // grp holds key 32*kb + 16*(r/8) + 8*grp + r%8 (after the LDS row swap).
  auto scores = [&](const T* ks, f32x16 (&s)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / MF::KS; ++st) {
      const Frag a = *reinterpret_cast<const Frag*>(&ks[col * Cfg::KLD + st * MF::KS + grp * MF::E]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = MF::run(a, qf[qb][st], s[qb]);
    }
  };

  // Online softmax of one 32-key block (first key k0b) followed by
  // O^T += V^T P^T. vs points at the block's first key column of V^T.
  auto softmax_pv = [&](f32x16 (&s)[QB], int k0b, const T* vs) {
    if (k0b + 32 > p.N || (p.causal && k0b + 31 > qw)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + 32 * qb + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0b + 16 * (r >> 3) + 8 * grp + (r & 7);
          if (key >= p.N || (p.causal && key > qi)) s[qb][r] = -INFINITY;
        }
      }
    }
    float mx[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = max3(s[qb][0], s[qb][1], s[qb][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = max3(m, s[qb][r], s[qb][r + 1]);
      m = fmaxf(m, s[qb][15]);
      m = fmaxf(m, __shfl_xor(m, 32)) * c;
      mx[qb] = m;
      grow |= m > m_ref[qb] + TAU_LOG2;
    }
    if (__any(grow)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_ref[qb], mx[qb]);
        const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) o[qb][nb] *= alpha;
        m_ref[qb] = m_new;
      }
    }
    if constexpr (sizeof(T) == 2) {
      Frag pf[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // a row with no visible key yet keeps m_ref = -inf; use 0 so that its
        // masked scores give exp2(-inf) = 0 rather than NaN
        const float mb = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pf[qb][half][e] = from_f32<T>(__builtin_amdgcn_exp2f(fmaf(s[qb][8 * half + e], c, -mb)));
          l_run[qb] = sum8(pf[qb][half], l_run[qb]);
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const Frag a = *reinterpret_cast<const Frag*>(
              &vs[(nb * 32 + col) * Cfg::VLD + half * 16 + grp * 8]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][nb] = MF::run(a, pf[qb][half], o[qb][nb]);
        }
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mb = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[qb][r] = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -mb));
          l_run[qb] += s[qb][r];
        }
      }
#pragma unroll
      for (int st = 0; st < 16; ++st)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const Frag a = *reinterpret_cast<const Frag*>(
              &vs[(nb * 32 + col) * Cfg::VLD + 16 * (st >> 3) + 8 * grp + (st & 7)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][nb] = MF::run(a, s[qb][st], o[qb][nb]);
        }
    }
  };

  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) load(kt + 1);
    const int k0 = kt * KT;
    // a 32-key block is skipped by a wave whose last query precedes its first key
    const bool act0 = !p.causal || k0 <= qw + QW - 1;
    const bool act1 = !p.causal || k0 + 32 <= qw + QW - 1;
    f32x16 s0[QB], s1[QB];
    if (act0) scores(&Ks[buf][0], s0);
    if (act1) scores(&Ks[buf][32 * Cfg::KLD], s1);
    if (act0) softmax_pv(s0, k0, &Vs[buf][0]);
    if (act1) softmax_pv(s1, k0 + 32, &Vs[buf][32]);
    if (kt + 1 < n_tiles) stash(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.f / (l_run[qb] + __shfl_xor(l_run[qb], 32));
    const int t = qw + 32 * qb + col;
    if (t < p.N) {
      T* arow = (T*)p.a + ((int64_t)b * p.N + t) * ((int64_t)p.H_q * D) + head * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          // rows 8*rq + 4*grp + 0..3 of this O^T tile are 4 consecutive head dims
          T* dst = arow + nb * 32 + 8 * rq + 4 * grp;
          const float v0 = o[qb][nb][4 * rq] * inv, v1 = o[qb][nb][4 * rq + 1] * inv;
          const float v2 = o[qb][nb][4 * rq + 2] * inv, v3 = o[qb][nb][4 * rq + 3] * inv;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(dst) =
                bf16x4{from_f32<T>(v0), from_f32<T>(v1), from_f32<T>(v2), from_f32<T>(v3)};
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
          }
        }
    }
  }
}

template <typename T, int D>
hipError_t run(const AttnParams& p, unsigned grid, hipStream_t stream) {
  attn_kernel<T, D><<<grid, THREADS, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(sqa_dtype dt, const void* q, const void* k, const void* vt, void* a,
                            int64_t B, int64_t N, int64_t Np, int64_t H_q, int64_t H_kv,
                            int64_t d_head, bool causal, hipStream_t stream) {
  AttnParams p;
  p.q = q; p.k = k; p.vt = vt; p.a = a;
  p.N = (int)N; p.Np = (int)Np; p.H_q = (int)H_q; p.H_kv = (int)H_kv;
  p.g = (int)(H_q / H_kv);
  p.G = p.g % 4 == 0 ? 4 : (p.g % 2 == 0 ? 2 : 1);   // heads per workgroup
  p.n_sub = p.g / p.G;
  p.q_per_wg = QW * (WAVES / p.G);
  p.n_qt = (int)((N + p.q_per_wg - 1) / p.q_per_wg);
  p.causal = causal ? 1 : 0;
  p.c = (float)(1.4426950408889634 / sqrt((double)d_head));
  const int64_t grid = (int64_t)p.n_qt * p.n_sub * H_kv * B;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (dt == SQA_DTYPE_BF16)
    return d_head == 64 ? run<bf16, 64>(p, (unsigned)grid, stream)
                        : run<bf16, 32>(p, (unsigned)grid, stream);
  return d_head == 64 ? run<float, 64>(p, (unsigned)grid, stream)
                      : run<float, 32>(p, (unsigned)grid, stream);
}

}  // namespace sqa
