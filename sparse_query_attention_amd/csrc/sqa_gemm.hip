// Projection GEMMs of the SQA forward pass on gfx950 MFMA.
//
// Step 1 (query/key/value projection) and step 3 (output projection) are both
// C[M, Ncols] = A[M, K] * W[K, Ncols] with W stored [in, out] row-major, as the
// SQA definition's y = x W. The query projection and the output projection are
// narrowed to the H_q used heads (ReactiveAI/xSMQAT-m model card, description).
// One kernel template serves both steps. Only where rows come from and where
// results go differ.
//
// Tiling: a 256-thread workgroup owns a 128x128 tile of C. Its four waves
// each own a 64x64 sub-tile, i.e. 2x2 MFMA 32x32 tiles. K advances in
// steps of 32 through double-buffered LDS; the next step's global loads are
// in flight while the current one feeds the MFMAs. W is stored transposed in
// LDS ([n][k]) so that both MFMA operands read k-contiguous 16-byte
// fragments.
#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int BM = 128, BN = 128, BK = 32, THREADS = 256;

template <typename T> struct GemmCfg {
  static constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int LD = BK + EPC;                    // LDS row length, 16-byte pad
  static constexpr int CPR = BK / EPC;                   // chunks per A-tile row
  static constexpr int A_PER = BM * CPR / THREADS;       // A chunks per thread
  static constexpr int RPT = sizeof(T) == 2 ? 2 : 1;     // W rows per task (fills 32-bit LDS words)
  static constexpr int B_TASKS = (BK / RPT) * (BN / EPC);
  static constexpr int B_PER = B_TASKS / THREADS;        // W tasks per thread
  static_assert(B_PER * THREADS == B_TASKS, "W tile split");
  static_assert(A_PER * THREADS == BM * CPR, "A tile split");
};

// Rows of X for step 1: output row gr = b*Np + t reads X row b*N + t when t < N,
// and zeros otherwise (the padded rows of the Q/K/V^T layouts).
template <typename T> struct PaddedRows {
  const T* x; int64_t N, Np; int K;
  __device__ const T* row(int64_t gr) const {
    const int64_t b = gr / Np, t = gr - b * Np;
    return t < N ? x + (b * N + t) * K : nullptr;
  }
};

// Rows of A for step 3: plain [M, K] with a ragged last tile.
template <typename T> struct DenseRows {
  const T* a; int64_t M; int K;
  __device__ const T* row(int64_t gr) const { return gr < M ? a + gr * K : nullptr; }
};

// Columns of [Wq | Wk | Wv] (widths wq, wkv, wkv). A 16-byte chunk never
// straddles two matrices because every width is a multiple of d_head >= 32.
template <typename T> struct QkvCols {
  const T* wq; const T* wk; const T* wv; int wq_w, wkv_w;
  __device__ const T* col(int n, int& ld) const {
    if (n < wq_w) { ld = wq_w; return wq + n; }
    n -= wq_w;
    if (n < wkv_w) { ld = wkv_w; return wk + n; }
    n -= wkv_w;
    if (n < wkv_w) { ld = wkv_w; return wv + n; }
    ld = 0; return nullptr;
  }
};

template <typename T> struct DenseCols {
  const T* w; int ncols;
  __device__ const T* col(int n, int& ld) const {
    ld = ncols; return n < ncols ? w + n : nullptr;
  }
};

// Step 1 epilogue: route column n to q, k or vt and row gr to (b, t).
template <typename T> struct QkvStore {
  T* q; T* k; T* vt; int64_t Np; int H_q, H_kv, D, wq_w, wkv_w;
  // v[i] is C[gr + i][n] for i = 0..3 (four consecutive rows, one column).
  __device__ void operator()(int64_t gr, int n, const float v[4]) const {
    const int64_t b = gr / Np, t = gr - b * Np;
    if (n < wq_w) {
      T* p = q + ((b * H_q + n / D) * Np + t) * D + n % D;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[(int64_t)i * D] = from_f32<T>(v[i]);
      return;
    }
    n -= wq_w;
    if (n < wkv_w) {
      T* p = k + ((b * H_kv + n / D) * Np + t) * D + n % D;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[(int64_t)i * D] = from_f32<T>(v[i]);
      return;
    }
    n -= wkv_w;
    if (n < wkv_w) {
      // V^T: the four rows are four consecutive t, contiguous in vt.
      T* p = vt + ((b * H_kv + n / D) * (int64_t)D + n % D) * Np + t;
      if constexpr (sizeof(T) == 2) {
        bf16x4 w = {from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
        *reinterpret_cast<bf16x4*>(p) = w;
      } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
      }
    }
  }
};

template <typename T> struct DenseStore {
  T* out; int64_t M; int ncols;
  __device__ void operator()(int64_t gr, int n, const float v[4]) const {
    if (n >= ncols) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (gr + i < M) out[(gr + i) * ncols + n] = from_f32<T>(v[i]);
  }
};

template <typename T, class Rows, class Cols, class Store>
__global__ __launch_bounds__(THREADS) void gemm_kernel(Rows rows, Cols cols, Store store, int K) {
  using C = GemmCfg<T>;
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  __shared__ __align__(16) T As[2][BM * C::LD];
  __shared__ __align__(16) T Bs[2][BN * C::LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;

  // Fixed per-thread source pointers of the A tile chunks and W tile tasks.
  const T* a_src[C::A_PER];
#pragma unroll
  for (int i = 0; i < C::A_PER; ++i) {
    const int c = tid + i * THREADS;
    const T* r = rows.row(m0 + c / C::CPR);
    a_src[i] = r ? r + (c % C::CPR) * C::EPC : nullptr;
  }
  const T* b_src[C::B_PER];
  int b_ld[C::B_PER];
#pragma unroll
  for (int i = 0; i < C::B_PER; ++i) {
    const int task = tid + i * THREADS;
    const int kp = task / (BN / C::EPC), nc = task % (BN / C::EPC);
    const T* p = cols.col(n0 + nc * C::EPC, b_ld[i]);
    b_src[i] = p ? p + (int64_t)kp * C::RPT * b_ld[i] : nullptr;
  }

  Chunk areg[C::A_PER];
  Chunk breg[C::B_PER][C::RPT];

  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i)
      areg[i] = a_src[i] ? *reinterpret_cast<const Chunk*>(a_src[i] + kt * BK) : zero_chunk();
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i)
#pragma unroll
      for (int j = 0; j < C::RPT; ++j)
        breg[i][j] = b_src[i]
            ? *reinterpret_cast<const Chunk*>(b_src[i] + ((int64_t)kt * BK + j) * b_ld[i])
            : zero_chunk();
  };

  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
      const int c = tid + i * THREADS;
      *reinterpret_cast<Chunk*>(&As[buf][(c / C::CPR) * C::LD + (c % C::CPR) * C::EPC]) = areg[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
      const int task = tid + i * THREADS;
      const int kp = task / (BN / C::EPC), nc = task % (BN / C::EPC);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&Bs[buf][(nc * C::EPC) * C::LD + kp * C::RPT]);
      constexpr int WSTRIDE = C::LD * sizeof(T) / 4;  // one LDS row in 32-bit words
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) {
        uint32_t w;
        if constexpr (sizeof(T) == 2) {
          const uint32_t lo = (breg[i][0].w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          const uint32_t hi = (breg[i][1].w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          w = lo | (hi << 16);
        } else {
          w = breg[i][0].w[e];
        }
        dst[e * WSTRIDE] = w;
      }
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 31, grp = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / MF::KS; ++s) {
      Frag a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const Frag*>(
            &As[buf][(wm * 64 + i * 32 + col) * C::LD + s * MF::KS + grp * MF::E]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const Frag*>(
            &Bs[buf][(wn * 64 + j * 32 + col) * C::LD + s * MF::KS + grp * MF::E]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MF::run(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float v[4] = {acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                            acc[i][j][4 * rq + 3]};
        store(m0 + wm * 64 + i * 32 + 8 * rq + 4 * grp, n0 + wn * 64 + j * 32 + col, v);
      }
}

template <typename T>
hipError_t qkv_impl(const void* x, const void* wq, const void* wk, const void* wv, void* q,
                    void* k, void* vt, int64_t B, int64_t N, int64_t Np, int64_t d_model,
                    int64_t H_q, int64_t H_kv, int64_t d, hipStream_t stream) {
  const int wq_w = (int)(H_q * d), wkv_w = (int)(H_kv * d);
  const int ncols = wq_w + 2 * wkv_w;
  PaddedRows<T> rows{(const T*)x, N, Np, (int)d_model};
  QkvCols<T> cols{(const T*)wq, (const T*)wk, (const T*)wv, wq_w, wkv_w};
  QkvStore<T> st{(T*)q, (T*)k, (T*)vt, Np, (int)H_q, (int)H_kv, (int)d, wq_w, wkv_w};
  dim3 grid((unsigned)(B * Np / BM), (unsigned)((ncols + BN - 1) / BN));
  gemm_kernel<T><<<grid, THREADS, 0, stream>>>(rows, cols, st, (int)d_model);
  return hipGetLastError();
}

template <typename T>
hipError_t out_impl(const void* a, const void* wo, void* out, int64_t M, int64_t K,
                    int64_t d_model, hipStream_t stream) {
  DenseRows<T> rows{(const T*)a, M, (int)K};
  DenseCols<T> cols{(const T*)wo, (int)d_model};
  DenseStore<T> st{(T*)out, M, (int)d_model};
  dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((d_model + BN - 1) / BN));
  gemm_kernel<T><<<grid, THREADS, 0, stream>>>(rows, cols, st, (int)K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_projection(sqa_dtype dt, const void* x, const void* wq, const void* wk,
                                 const void* wv, void* q, void* k, void* vt, int64_t B, int64_t N,
                                 int64_t Np, int64_t d_model, int64_t H_q, int64_t H_kv,
                                 int64_t d_head, hipStream_t stream) {
  if (dt == SQA_DTYPE_BF16)
    return qkv_impl<bf16>(x, wq, wk, wv, q, k, vt, B, N, Np, d_model, H_q, H_kv, d_head, stream);
  return qkv_impl<float>(x, wq, wk, wv, q, k, vt, B, N, Np, d_model, H_q, H_kv, d_head, stream);
}

hipError_t launch_output_projection(sqa_dtype dt, const void* a, const void* wo, void* out,
                                    int64_t M, int64_t K, int64_t d_model, hipStream_t stream) {
  if (dt == SQA_DTYPE_BF16) return out_impl<bf16>(a, wo, out, M, K, d_model, stream);
  return out_impl<float>(a, wo, out, M, K, d_model, stream);
}

}  // namespace sqa
