// Attention core of the SQA forward pass on gfx950: per query head i,
//   A_i = softmax(Q_i K_j^T / sqrt(d)) V_j,   j = floor(i / (H_q/H_kv)),
// with an optional causal mask (key c visible to query r iff c <= r).
// SQA keeps GQA's key/value sharing and cuts the query heads, so the score
// work scales with H_q ("Sparse Query Attention (SQA)...", arXiv 2510.01817,
// abstract; ReactiveAI/GQA-Ref-Micro model card, description).
//
// Design (one workgroup = 4 waves of 64 lanes):
//  * A workgroup owns one (batch, key/value head) pair, G query heads of that
//    head's group and a tile of queries. 32x128, 64x2 or 128x1 queries x heads
//    give 128 query rows per workgroup. Every key/value tile staged in LDS is
//    read by all G heads, so repeated K/V is never materialised.
//  * Each wave owns 32 query rows of one head. It computes S^T = K Q^T, which
//    puts one query per lane (lanes l and l+32 share query l%32). Row max and
//    row sum then need a single cross-lane exchange, and the exponentiated
//    scores are already in the B-operand layout of O^T += V^T P^T. No score
//    tile ever goes through LDS or HBM.
//  * Keys are stored in LDS with bits 2 and 3 of their in-tile index swapped.
//    This makes each lane's 16 score registers of a 32-key block cover two
//    runs of 8 consecutive keys, so P^T is consumed as-is and V^T fragments
//    are single 16-byte LDS reads.
//  * Online softmax in the exp2 domain with fp32 running max and sum, one
//    rescale of the O^T accumulators per key tile.
//  * Causal: key tiles past a workgroup's last query are never loaded, and a
//    wave skips the MFMAs of tiles past its own last query. Only tiles that
//    cross the diagonal or the sequence end are masked. Heaviest query tiles
//    are dispatched first.
#include <math.h>

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int KT = 64;       // keys per tile
constexpr int WAVES = 4;
constexpr int QW = 32;       // query rows per wave
constexpr int THREADS = 64 * WAVES;

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

template <typename T, int D>
__global__ __launch_bounds__(THREADS) void attn_kernel(AttnParams p) {
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
  if (p.causal) qt = p.n_qt - 1 - qt;
  const int sub = blk % p.n_sub;
  blk /= p.n_sub;
  const int h = blk % p.H_kv, b = blk / p.H_kv;
  const int waves_per_head = WAVES / p.G;
  const int head = h * p.g + sub * p.G + wave / waves_per_head;
  const int q0 = qt * p.q_per_wg;
  const int qw = q0 + (wave % waves_per_head) * QW;

  const T* Qh = (const T*)p.q + ((int64_t)b * p.H_q + head) * (int64_t)p.Np * D;
  const T* Kh = (const T*)p.k + ((int64_t)b * p.H_kv + h) * (int64_t)p.Np * D;
  const T* Vh = (const T*)p.vt + ((int64_t)b * p.H_kv + h) * (int64_t)D * p.Np;

  // Q as the B operand of S^T = K Q^T: lane -> query qw + col, k-group grp.
  Frag qf[D / MF::KS];
#pragma unroll
  for (int s = 0; s < D / MF::KS; ++s)
    qf[s] = *reinterpret_cast<const Frag*>(Qh + (int64_t)(qw + col) * D + s * MF::KS + grp * MF::E);

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

  f32x16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) load(kt + 1);
    const int k0 = kt * KT;
    if (!p.causal || k0 <= qw + QW - 1) {
      // S^T for two 32-key blocks: register r of lane group grp is key
      // k0 + 32*kb + 16*(r/8) + 8*grp + r%8 (after the LDS row swap).
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int st = 0; st < D / MF::KS; ++st) {
          const Frag a = *reinterpret_cast<const Frag*>(
              &Ks[buf][(kb * 32 + col) * Cfg::KLD + st * MF::KS + grp * MF::E]);
          s[kb] = MF::run(a, qf[st], s[kb]);
        }
      }
      if (k0 + KT > p.N || (p.causal && k0 + KT - 1 > qw)) {
        const int qi = qw + col;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 16 * (r >> 3) + 8 * grp + (r & 7);
            if (key >= p.N || (p.causal && key > qi)) s[kb][r] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_new));
          s[kb][r] = e;
          rs += e;
        }
      l_run += rs;
      m_run = m_new;

      // O^T[d x 32 queries] += V^T[d x 64 keys] P^T[64 keys x 32 queries]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const Frag pf = {from_f32<T>(s[kb][8 * half + 0]), from_f32<T>(s[kb][8 * half + 1]),
                             from_f32<T>(s[kb][8 * half + 2]), from_f32<T>(s[kb][8 * half + 3]),
                             from_f32<T>(s[kb][8 * half + 4]), from_f32<T>(s[kb][8 * half + 5]),
                             from_f32<T>(s[kb][8 * half + 6]), from_f32<T>(s[kb][8 * half + 7])};
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) {
              const Frag a = *reinterpret_cast<const Frag*>(
                  &Vs[buf][(nb * 32 + col) * Cfg::VLD + kb * 32 + half * 16 + grp * 8]);
              o[nb] = MF::run(a, pf, o[nb]);
            }
          }
        } else {
#pragma unroll
          for (int st = 0; st < 16; ++st) {
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) {
              const Frag a = *reinterpret_cast<const Frag*>(
                  &Vs[buf][(nb * 32 + col) * Cfg::VLD + kb * 32 + 16 * (st >> 3) + 8 * grp + (st & 7)]);
              o[nb] = MF::run(a, s[kb][st], o[nb]);
            }
          }
        }
      }
    }
    if (kt + 1 < n_tiles) stash(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.f / (l_run + __shfl_xor(l_run, 32));
  const int t = qw + col;
  if (t < p.N) {
    T* arow = (T*)p.a + ((int64_t)b * p.N + t) * ((int64_t)p.H_q * D) + head * D;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        // rows 8*rq + 4*grp + 0..3 of this O^T tile are 4 consecutive head dims
        T* dst = arow + nb * 32 + 8 * rq + 4 * grp;
        const float v0 = o[nb][4 * rq] * inv, v1 = o[nb][4 * rq + 1] * inv;
        const float v2 = o[nb][4 * rq + 2] * inv, v3 = o[nb][4 * rq + 3] * inv;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x4*>(dst) =
              bf16x4{from_f32<T>(v0), from_f32<T>(v1), from_f32<T>(v2), from_f32<T>(v3)};
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
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
