// Projection GEMMs of the SQA forward pass on gfx950 MFMA.
//
// Step 1 (query/key/value projection) and step 3 (output projection) are both
// C[M, Ncols] = A[M, K] * W[K, Ncols] with W stored [in, out] row-major, as the
// SQA definition's y = x W. The query projection and the output projection are
// narrowed to the H_q used heads (ReactiveAI/xSMQAT-m model card, description).
// One kernel template serves both steps. Only where rows come from and where
// results go differ.
//
// Design:
//  * W is first transposed to W^T [Ncols, K] (a few MB, once per call), so both
//    MFMA operands are k-contiguous rows.
//  * Two tilings. The bf16 forward projections run 512-thread workgroups that
//    own a 256x256 tile of C, eight waves of 128x64 (4x2 v_mfma_f32_32x32x16
//    tiles): six 16-byte LDS fragment reads feed eight MFMAs, and each
//    workgroup runs long enough that its pipeline fill and epilogue are small.
//    Every other product (fp32, the backward pass) runs 256-thread workgroups
//    on 128x128 tiles, four waves of 64x64 (2x2 MFMA tiles).
//  * K advances in steps of 32 through a 4-stage LDS ring filled by direct
//    loads into LDS (buffer_load_dwordx4 ... lds), three stages ahead, with one
//    barrier per step. Each load lands lane-contiguously, so 16-byte chunks are
//    XOR-swizzled per row against LDS bank conflicts.
//  * Workgroups are dispatched round-robin over the 8 XCDs, each with its own
//    L2. The 1-D grid is remapped so that every column tile of a row block
//    runs on one XCD, and that row block of A is fetched from memory once.
//  * LDS fragments are read one k-step of 16 ahead of the MFMAs that use them,
//    across the stage boundary too, into two alternating register sets, so LDS
//    latency overlaps the MFMAs.
//  * Rows past the end of A are loaded from a clamped, valid row and never
//    stored as computed: step 1 writes zeros there (the padded rows of the
//    Q/K/V^T layouts), step 3 skips them.
//  * The epilogue stages the C tile in LDS and writes it in 16-byte chunks that
//    run along contiguous memory: rows of Q, K and Y, sequence runs of V^T.
#include <algorithm>
#include <type_traits>

#include "sqa_device.h"
#include "sqa_internal.h"

namespace sqa {
namespace {

constexpr int BK = 32;
constexpr int XCDS = 8;

// A workgroup tiling: a BM x BN tile of C, WM x WN waves each owning
// 32*MI x 32*NJ (MI x NJ MFMA tiles of 32x32), an NST-stage LDS ring.
template <int BM_, int BN_, int WM_, int WN_, int NST_> struct Tiling {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NST = NST_;
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int MI = BM / WM / 32, NJ = BN / WN / 32;
  static constexpr int NBI = BM / 32, NBJ = BN / 32;   // 32x32 blocks per tile
  static_assert(MI * 32 * WM == BM && NJ * 32 * WN == BN, "wave tiles");
};
using SmallTiles = Tiling<128, 128, 2, 2, 4>;   // 4 waves of 64x64
using LargeTiles = Tiling<256, 256, 2, 4, 4>;   // 8 waves of 128x64 (bf16 only: 128 KB of LDS)

template <typename T, class TL> struct GemmCfg {
  static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int CPR = BK / EPC;                 // chunks per tile row (4 bf16, 8 fp32)
  static constexpr int A_ELEMS = TL::BM * BK, B_ELEMS = TL::BN * BK, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int A_INS = A_ELEMS / (64 * EPC) / TL::WAVES;   // 1 KB loads per wave
  static constexpr int B_INS = B_ELEMS / (64 * EPC) / TL::WAVES;
  static constexpr int VM = A_INS + B_INS;                          // loads per wave per stage
  static_assert(A_INS * TL::WAVES * 64 * EPC == A_ELEMS && B_INS * TL::WAVES * 64 * EPC == B_ELEMS,
                "split");
};

// Rows of X for step 1: output row gr = b*Np + t is X row b*N + t when t < N
// (padded rows load the sequence's last row and are stored as zeros).
template <typename T> struct PaddedRows {
  const T* x; int64_t N, Np; int K;
  __device__ const T* row(int64_t gr) const {
    const int64_t b = gr / Np, t = gr - b * Np;
    return x + (b * N + (t < N ? t : N - 1)) * K;
  }
};

// Rows of A for step 3: plain [M, K]; rows past M load row M-1 and are not stored.
template <typename T> struct DenseRows {
  const T* a; int64_t M; int K;
  __device__ const T* row(int64_t gr) const { return a + (gr < M ? gr : M - 1) * K; }
};

// Epilogue interface. The workgroup's C tile reaches memory in 16-byte chunks
// from LDS, one 32x32 block at a time. store.col_major(n) says whether the
// block whose first column is n is staged column by column (its chunks run
// along rows) or row by row (chunks run along columns). store.tile(m0) gives
// the tile whose rows start at m0, with rows r counted from m0:
//  * all_zero(): every row of the tile is stored as zeros (padding of its
//    sequence), so its products are not computed;
//  * zero_row(r): row r is stored as zeros (padding of the Q/K/V^T layouts);
//  * row_chunk(r, n, c): C[r][n .. n+E-1]; col_chunk(r, n, c): C[r .. r+E-1][n],
//    with E = 16 / sizeof(T).

// Step 1: column n goes to q, k or vt, row to (b, t). A tile of 128 or 256
// rows lies in one batch (Np is a multiple of 256). V^T blocks are column-major so that
// their chunks are runs of t, contiguous in vt.
template <typename T> struct QkvStore {
  static constexpr bool kDirect = false;
  T* q; T* k; T* vt; int64_t N, Np; int H_q, H_kv, dsh, wq_w, wkv_w;   // d_head = 1 << dsh
  const int32_t* lens;   // null, or each sequence's length (clamped into [0, N])
  __device__ bool col_major(int n) const { return n >= wq_w + wkv_w; }
  struct Tile {
    T* q; T* k; T* vt;   // batch b's slices, row t0
    int t0, n_valid, dsh, wq_w, wkv_w; int64_t Np;
    __device__ bool all_zero() const { return t0 >= n_valid; }
    __device__ bool zero_row(int r) const { return t0 + r >= n_valid; }
    __device__ void row_chunk(int r, int n, const Chunk& c) const {
      const int64_t t = t0 + r;
      T* p;
      if (n < wq_w) p = q + ((int64_t)(n >> dsh) * Np + t) * (1 << dsh) + (n & ((1 << dsh) - 1));
      else {
        n -= wq_w;
        p = k + ((int64_t)(n >> dsh) * Np + t) * (1 << dsh) + (n & ((1 << dsh) - 1));
      }
      *reinterpret_cast<Chunk*>(p) = c;
    }
    __device__ void col_chunk(int r, int n, const Chunk& c) const {
      n -= wq_w + wkv_w;   // V^T row (head n >> dsh, dim n & mask) is row n of batch b's block
      *reinterpret_cast<Chunk*>(vt + (int64_t)n * Np + t0 + r) = c;
    }
  };
  __device__ Tile tile(int64_t m0) const {
    const int64_t b = m0 / Np, t0 = m0 - b * Np;
    const int64_t d = (int64_t)1 << dsh;
    const int n_valid = lens ? min(max(lens[b], 0), (int)N) : (int)N;
    return Tile{q + b * H_q * Np * d, k + b * H_kv * Np * d, vt + b * H_kv * d * Np,
                (int)t0, n_valid, dsh, wq_w, wkv_w, Np};
  }
};

// Step 3: plain row-major out [M, ncols]; rows past M are not stored. With
// lens, row m is token m % seq_n of sequence m / seq_n, and a tile that lies in
// one sequence's padding is stored as zeros without computing it.
template <typename T> struct DenseStore {
  static constexpr bool kDirect = false;
  T* out; int64_t M; int ncols;
  const int32_t* lens; int64_t seq_n;
  int bm;   // rows per tile
  __device__ bool col_major(int) const { return false; }
  struct Tile {
    T* out; int64_t rows_left; int ncols; bool pad;   // rows from m0 on
    __device__ bool all_zero() const { return pad; }
    __device__ bool zero_row(int) const { return pad; }
    __device__ void row_chunk(int r, int n, const Chunk& c) const {
      if (r < rows_left) *reinterpret_cast<Chunk*>(out + (int64_t)r * ncols + n) = c;
    }
    __device__ void col_chunk(int, int, const Chunk&) const {}
  };
  __device__ Tile tile(int64_t m0) const {
    bool pad = false;
    if (lens) {
      const int64_t b = m0 / seq_n, t0 = m0 - b * seq_n;
      const int64_t L = min(max((int64_t)lens[b], (int64_t)0), seq_n);
      pad = t0 >= L && t0 + bm <= seq_n;   // the whole tile is padding of sequence b
    }
    return Tile{out + m0 * ncols, M - m0, ncols, pad};
  }
};

// Rows m = b*Np + t of a padded layout into out [B, N, ncols]: t >= N is not stored.
template <typename T> struct UnpadStore {
  static constexpr bool kDirect = false;
  T* out; int64_t N, Np; int ncols;
  __device__ bool col_major(int) const { return false; }
  struct Tile {
    T* out; int64_t rows_left; int ncols;   // rows from t0 on
    __device__ bool all_zero() const { return false; }
    __device__ bool zero_row(int) const { return false; }
    __device__ void row_chunk(int r, int n, const Chunk& c) const {
      if (r < rows_left) *reinterpret_cast<Chunk*>(out + (int64_t)r * ncols + n) = c;
    }
    __device__ void col_chunk(int, int, const Chunk&) const {}
  };
  __device__ Tile tile(int64_t m0) const {
    const int64_t b = m0 / Np, t0 = m0 - b * Np;
    return Tile{out + (b * N + t0) * ncols, N - t0, ncols};
  }
};

// Split-K partial sums, fp32 and unrounded: part[blockIdx.y][m][n] for m < M.
// The accumulators go straight from registers to memory (no LDS staging).
struct F32PartStore {
  static constexpr bool kDirect = true;
  float* part; int64_t M; int ncols;
  __device__ bool col_major(int) const { return false; }
  struct Tile {   // the staged epilogue's interface, unused by a direct store
    __device__ bool all_zero() const { return false; }
    __device__ bool zero_row(int) const { return false; }
    __device__ void row_chunk(int, int, const Chunk&) const {}
    __device__ void col_chunk(int, int, const Chunk&) const {}
  };
  __device__ Tile tile(int64_t) const { return Tile{}; }
  __device__ void put(int64_t m, int n, float v) const {
    if (m < M) part[((int64_t)blockIdx.y * M + m) * ncols + n] = v;
  }
};

// C = A * W with W given transposed (wt [ncols, K]); see the file header.
// Workgroup row blockIdx.y sums k in [y*k_split, min(K, (y+1)*k_split)), a
// multiple of BK (split-K; k_split = K otherwise).
template <typename T, class TL, class Rows, class Store>
__global__ __launch_bounds__(TL::THREADS) void gemm_kernel(Rows rows, const T* wt, int ncols,
                                                           Store store, int K, int n_rb, int n_ct,
                                                           int k_split) {
  using C = GemmCfg<T, TL>;
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  constexpr int BM = TL::BM, BN = TL::BN, NST = TL::NST, MI = TL::MI, NJ = TL::NJ;
  constexpr int NBJ = TL::NBJ, THREADS = TL::THREADS;
  __shared__ __align__(16) T smem[NST * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int col = lane & 31, grp = lane >> 5;
  // block L runs on XCD L % 8; XCD x owns row blocks x, x+8, ... in turn
  const int L = blockIdx.x, xcd = L % XCDS, k_in_xcd = L / XCDS;
  const int rb = (k_in_xcd / n_ct) * XCDS + xcd, ct = k_in_xcd % n_ct;
  if (rb >= n_rb) return;
  const int64_t m0 = (int64_t)rb * BM;
  const int n0 = ct * BN;
  const int k_begin = blockIdx.y * k_split;

  // Direct loads as buffer loads: unlike global_load_lds they count only in
  // vmcnt, so the compiler's waits for the fragment reads in flight stay
  // exact (with a global_load_lds in flight it waits for every LDS read).
  // Load i of a wave covers 64 chunks of the tile rows r0 .. r0 + 64/CPR - 1;
  // its buffer starts at row r0 (a row at or after it: clamped rows repeat a
  // later one), and each lane's byte offset in it (its row, its chunk
  // swizzled per row) is fixed, below 2^32 for these few rows of K elements.
  // Stage kt moves the scalar offset only.
  const T* a_base[C::A_INS];
  const T* b_base[C::B_INS];
  uint32_t a_off[C::A_INS], b_off[C::B_INS];
#pragma unroll
  for (int i = 0; i < C::A_INS; ++i) {
    const int pos = (wave * C::A_INS + i) * 64 + lane;
    const int r = pos / C::CPR, slot = pos % C::CPR, r0 = (wave * C::A_INS + i) * 64 / C::CPR;
    a_base[i] = rows.row(m0 + r0) + k_begin;
    a_off[i] = (uint32_t)((rows.row(m0 + r) + k_begin + (slot ^ swz<C::CPR>(r)) * C::EPC - a_base[i]) * (int64_t)sizeof(T));
  }
#pragma unroll
  for (int i = 0; i < C::B_INS; ++i) {
    const int pos = (wave * C::B_INS + i) * 64 + lane;
    const int r = pos / C::CPR, slot = pos % C::CPR, r0 = (wave * C::B_INS + i) * 64 / C::CPR;
    const int nb0 = min(n0 + r0, ncols - 1), n = min(n0 + r, ncols - 1);
    b_base[i] = wt + (int64_t)nb0 * K + k_begin;
    b_off[i] = (uint32_t)(((int64_t)(n - nb0) * K + (slot ^ swz<C::CPR>(r)) * C::EPC) * (int64_t)sizeof(T));
  }
  const int nk = (min(K, k_begin + k_split) - k_begin) / BK;
  auto issue = [&](int kt) {
    if (kt >= nk) return;
    T* st = smem + (kt % NST) * C::STAGE;
    const int koff = kt * BK * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < C::A_INS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)a_base[i], (short)0, -1, 0x00020000),
                                               (lds_ptr)(st + (wave * C::A_INS + i) * 64 * C::EPC), 16,
                                               (int)a_off[i], koff, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_INS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)b_base[i], (short)0, -1, 0x00020000),
                                               (lds_ptr)(st + C::A_ELEMS + (wave * C::B_INS + i) * 64 * C::EPC),
                                               16, (int)b_off[i], koff, 0, 0);
  };
  // MFMA fragment of tile row r (A or B part of a stage), k-step s.
  auto frag = [&](const T* part, int r, int s) -> Frag {
    const int e = s * MF::KS + grp * MF::E;
    return *reinterpret_cast<const Frag*>(
        &part[r * BK + (((e / C::EPC) ^ swz<C::CPR>(r)) * C::EPC) + e % C::EPC]);
  };

  const int wm = wave / TL::WN, wn = wave % TL::WN;
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  // Fragments of stage kt, k-step s, for this wave's MI x NJ MFMA tiles.
  constexpr int SUB = BK / MF::KS;
  auto read = [&](int kt, int s, Frag (&a)[MI], Frag (&b)[NJ]) {
    const T* st = smem + (kt % NST) * C::STAGE;
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = frag(st, wm * MI * 32 + i * 32 + col, s);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = frag(st + C::A_ELEMS, wn * NJ * 32 + j * 32 + col, s);
  };

  // The MFMA operand order fixes which way the accumulator's runs of four go:
  // A*B gives runs along rows, B*A (the tile transposed) runs along columns.
  // A workgroup whose blocks are all staged row-major takes B*A, so that it
  // stages four consecutive columns per write.
  bool rows_all = true;
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) rows_all &= n0 + 32 * bj >= ncols || !store.col_major(n0 + 32 * bj);

  auto main_loop = [&](auto transposed) {
    constexpr bool TR = decltype(transposed)::value;
    // All NST stages in flight; stage 0 visible; its first fragments read.
#pragma unroll
    for (int s = 0; s < NST; ++s) issue(s);
    wait_vmcnt_tiles<C::VM, NST - 1>(min(NST - 1, nk - 1));
    ring_barrier();
    // Fragments in two register sets: k-step s uses set s % 2 while the
    // reads of k-step s + 1 fill the other (SUB is even, so a stage's first
    // k-step always uses set 0 and no set is copied into another). The last
    // stage runs in a copy of its own, so that no branch joins the paths
    // before a k-step's MFMAs and their waits count the reads in flight
    // exactly.
    static_assert(SUB % 2 == 0, "k-steps per stage");
    Frag fa[2][MI], fb[2][NJ];
    read(0, 0, fa[0], fb[0]);
    auto stage = [&](int kt, auto last) {
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int cur = s % 2, nxt = (s + 1) % 2;
        if (s + 1 < SUB) {
          read(kt, s + 1, fa[nxt], fb[nxt]);
        } else if constexpr (!decltype(last)::value) {
          // Stage kt+1 complete for this wave (later stages may be in flight),
          // then visible to all; every wave's reads of stage kt are done, so
          // its slot takes stage kt+NST.
          wait_vmcnt_tiles<C::VM, NST - 2>(min(NST - 2, max(0, nk - 2 - kt)));
          ring_barrier();
          issue(kt + NST);
          read(kt + 1, 0, fa[nxt], fb[nxt]);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = TR ? MF::run(fb[cur][j], fa[cur][i], acc[i][j]) : MF::run(fa[cur][i], fb[cur][j], acc[i][j]);
        // the next k-step's reads before this one's MFMAs, so that their
        // latency hides behind all of them
        __builtin_amdgcn_sched_group_barrier(0x100, MI + NJ, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) stage(kt, std::false_type{});
    if (nk > 0) stage(nk - 1, std::true_type{});
  };
  if constexpr (Store::kDirect) {
    // register r of this lane: row 8*(r/4) + 4*grp + r%4, column col
    main_loop(std::false_type{});
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * NJ * 32 + j * 32 + col;
        if (n >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          store.put(m0 + wm * MI * 32 + i * 32 + 8 * (r / 4) + 4 * grp + r % 4, n, acc[i][j][r]);
      }
    return;
  }
  // A tile wholly in the padding of its sequence keeps zero accumulators.
  const auto tile = store.tile(m0);
  if (tile.all_zero()) {
  } else if (rows_all) {
    main_loop(std::true_type{});
  } else {
    main_loop(std::false_type{});
  }

  // Epilogue through LDS (the ring is free once every wave has passed the
  // first barrier). Block (bi, bj) is the 32x32 sub-tile at rows 32*bi,
  // columns 32*bj; each is staged row- or column-major as the store asks, in
  // lines of 32 elements with a 16-byte pad against bank conflicts. Then all
  // threads write 16-byte chunks, four (bf16) or eight (fp32) per line. When
  // the whole tile does not fit the ring, it goes out in WM passes of one wave
  // row each.
  constexpr int LINE = 32 * (int)sizeof(T) + 16;   // bytes per staged line
  constexpr int BLOCK = 32 * LINE;
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int PASSES = TL::NBI * NBJ * BLOCK <= NST * C::STAGE * (int)sizeof(T) ? 1 : TL::WM;
  constexpr int BI_PASS = TL::NBI / PASSES;          // block rows staged per pass
  static_assert(BI_PASS * NBJ * BLOCK <= NST * C::STAGE * (int)sizeof(T), "epilogue fits the ring");
  char* ep = reinterpret_cast<char*>(smem);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    __syncthreads();
    if (PASSES == 1 || wm == pass) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int bi = wm * MI + i, bj = wn * NJ + j;
          char* blk = ep + ((bi - pass * BI_PASS) * NBJ + bj) * BLOCK;
          if (rows_all) {
            // transposed: register r holds row col, column 8*(r/4) + 4*grp + r%4
            const bool z = tile.zero_row(32 * bi + col);
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = z ? 0.f : acc[i][j][4 * rq + e];
              T* dst = reinterpret_cast<T*>(blk + col * LINE) + 8 * rq + 4 * grp;
              if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<bf16x4*>(dst) =
                    bf16x4{from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
              } else {
                *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
              }
            }
          } else if (store.col_major(n0 + 32 * bj)) {
            // register r of this lane: row 8*(r/4) + 4*grp + r%4, column col
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int r0 = 8 * rq + 4 * grp;
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                v[e] = tile.zero_row(32 * bi + r0 + e) ? 0.f : acc[i][j][4 * rq + e];
              T* dst = reinterpret_cast<T*>(blk + col * LINE) + r0;
              if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<bf16x4*>(dst) =
                    bf16x4{from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
              } else {
                *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = 8 * (r / 4) + 4 * grp + r % 4;
              const bool z = tile.zero_row(32 * bi + row);
              reinterpret_cast<T*>(blk + row * LINE)[col] = from_f32<T>(z ? 0.f : acc[i][j][r]);
            }
          }
        }
    }
    __syncthreads();
    constexpr int CPL = 32 / EPC;                  // chunks per line
    constexpr int CHUNKS = BI_PASS * NBJ * 32 * CPL;
    static_assert(CHUNKS % THREADS == 0, "whole chunk rounds");
#pragma unroll
    for (int it = 0; it < CHUNKS / THREADS; ++it) {
      const int cidx = it * THREADS + tid;
      const int blkid = cidx / (32 * CPL), line = (cidx / CPL) % 32, qc = cidx % CPL;
      const int bi = pass * BI_PASS + blkid / NBJ, bj = blkid % NBJ;
      const int n_b = n0 + 32 * bj;
      if (n_b >= ncols) continue;
      const Chunk c = *reinterpret_cast<const Chunk*>(ep + blkid * BLOCK + line * LINE + qc * 16);
      if (store.col_major(n_b)) tile.col_chunk(32 * bi + qc * EPC, n_b + line, c);
      else tile.row_chunk(32 * bi + line, n_b + qc * EPC, c);
    }
  }
}

// W^T [ncols, K] from W = [W0 | W1 | W2] ([K, w0], [K, w1], [K, w2] row-major;
// w1, w2 may be 0). One 32x32 tile per workgroup through LDS.
template <typename T>
__global__ __launch_bounds__(256) void transpose_weights(const T* w0, int w0n, const T* w1, int w1n,
                                                         const T* w2, int w2n, T* wt, int K) {
  __shared__ T tile[32][33];
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
#pragma unroll
  for (int r = 0; r < 32; r += 8) {
    int n = n0 + tx;
    const T* src;
    int ld;
    if (n < w0n) { src = w0; ld = w0n; }
    else if ((n -= w0n) < w1n) { src = w1; ld = w1n; }
    else { n -= w1n; src = w2; ld = w2n; }
    tile[ty + r][tx] = src[(int64_t)(k0 + ty + r) * ld + n];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 32; r += 8)
    wt[(int64_t)(n0 + ty + r) * K + k0 + tx] = tile[tx][ty + r];
}

// Blocks for n_rb row blocks x n_ct column tiles under the XCD remap (row
// blocks rounded up to a multiple of 8; the extra blocks exit at once).
int64_t grid_size(int64_t n_rb, int64_t n_ct) { return (n_rb + XCDS - 1) / XCDS * XCDS * n_ct; }

bool grid_ok(int64_t n_rb, int64_t n_ct) {
  return n_rb > 0 && n_ct > 0 && grid_size(n_rb, n_ct) <= 0x7FFFFFFF;
}

template <typename T>
hipError_t transpose(const T* w0, int w0n, const T* w1, int w1n, const T* w2, int w2n, T* wt,
                     int K, hipStream_t stream) {
  const int ncols = w0n + w1n + w2n;
  dim3 grid((unsigned)(ncols / 32), (unsigned)(K / 32));
  transpose_weights<T><<<grid, 256, 0, stream>>>(w0, w0n, w1, w1n, w2, w2n, wt, K);
  return hipGetLastError();
}

// The tiling of the dense products over all tokens (the forward projections,
// dO = dY Wo^T and dX): large tiles for bf16 (their 128 KB ring would not fit
// the LDS with fp32 operands), the 128x128 tiling otherwise. The split-K
// weight gradients keep 128x128 tiles: larger ones would need 2-4x the fp32
// partial sums for the same number of workgroups.
template <typename T>
using ProjTiles = typename std::conditional<sizeof(T) == 2, LargeTiles, SmallTiles>::type;

template <typename T>
hipError_t qkv_impl(const void* x, const void* wq, const void* wk, const void* wv, void* wt,
                    void* q, void* k, void* vt, int64_t B, int64_t N, int64_t Np, int64_t d_model,
                    int64_t H_q, int64_t H_kv, int64_t d, const int32_t* lens,
                    hipStream_t stream) {
  using TL = ProjTiles<T>;
  const int wq_w = (int)(H_q * d), wkv_w = (int)(H_kv * d);
  const int ncols = wq_w + 2 * wkv_w;
  const int64_t n_rb = B * Np / TL::BM, n_ct = (ncols + TL::BN - 1) / TL::BN;
  if (!grid_ok(n_rb, n_ct)) return hipErrorInvalidConfiguration;
  hipError_t e = transpose<T>((const T*)wq, wq_w, (const T*)wk, wkv_w, (const T*)wv, wkv_w, (T*)wt,
                              (int)d_model, stream);
  if (e != hipSuccess) return e;
  PaddedRows<T> rows{(const T*)x, N, Np, (int)d_model};
  const int dsh = d == 64 ? 6 : 5;   // d_head is 32 or 64 (checked by the caller)
  QkvStore<T> st{(T*)q, (T*)k, (T*)vt, N, Np, (int)H_q, (int)H_kv, dsh, wq_w, wkv_w, lens};
  gemm_kernel<T, TL><<<(unsigned)grid_size(n_rb, n_ct), TL::THREADS, 0, stream>>>(
      rows, (const T*)wt, ncols, st, (int)d_model, (int)n_rb, (int)n_ct, (int)d_model);
  return hipGetLastError();
}

template <typename T>
hipError_t out_impl(const void* a, const void* wo, void* wt, void* out, int64_t M, int64_t K,
                    int64_t d_model, const int32_t* lens, int64_t seq_n, hipStream_t stream) {
  using TL = ProjTiles<T>;
  const int64_t n_rb = (M + TL::BM - 1) / TL::BM, n_ct = (d_model + TL::BN - 1) / TL::BN;
  if (!grid_ok(n_rb, n_ct)) return hipErrorInvalidConfiguration;
  hipError_t e = transpose<T>((const T*)wo, (int)d_model, nullptr, 0, nullptr, 0, (T*)wt, (int)K,
                              stream);
  if (e != hipSuccess) return e;
  DenseRows<T> rows{(const T*)a, M, (int)K};
  DenseStore<T> st{(T*)out, M, (int)d_model, lens, seq_n, TL::BM};
  gemm_kernel<T, TL><<<(unsigned)grid_size(n_rb, n_ct), TL::THREADS, 0, stream>>>(
      rows, (const T*)wt, (int)d_model, st, (int)K, (int)n_rb, (int)n_ct, (int)K);
  return hipGetLastError();
}

// out [B, ncols/d, Np, d] (head-major rows, zero past N) = x [B, N, K] * wt^T.
template <typename T>
hipError_t heads_impl(const void* x, const void* wt, void* out, int64_t B, int64_t N, int64_t Np,
                      int64_t K, int64_t ncols, int64_t d, hipStream_t stream) {
  using TL = ProjTiles<T>;
  const int64_t n_rb = B * Np / TL::BM, n_ct = (ncols + TL::BN - 1) / TL::BN;
  if (!grid_ok(n_rb, n_ct)) return hipErrorInvalidConfiguration;
  PaddedRows<T> rows{(const T*)x, N, Np, (int)K};
  const int dsh = d == 64 ? 6 : 5;
  QkvStore<T> st{(T*)out, nullptr, nullptr, N, Np, (int)(ncols / d), 0, dsh, (int)ncols, 0, nullptr};
  gemm_kernel<T, TL><<<(unsigned)grid_size(n_rb, n_ct), TL::THREADS, 0, stream>>>(
      rows, (const T*)wt, (int)ncols, st, (int)K, (int)n_rb, (int)n_ct, (int)K);
  return hipGetLastError();
}

// out [B, N, ncols] = a [B*Np, K] * wt^T, rows t >= N of each batch dropped.
template <typename T>
hipError_t unpad_impl(const void* a, const void* wt, void* out, int64_t B, int64_t N, int64_t Np,
                      int64_t K, int64_t ncols, hipStream_t stream) {
  using TL = ProjTiles<T>;   // Np is a multiple of 256: no tile spans two sequences
  const int64_t n_rb = B * Np / TL::BM, n_ct = (ncols + TL::BN - 1) / TL::BN;
  if (!grid_ok(n_rb, n_ct)) return hipErrorInvalidConfiguration;
  DenseRows<T> rows{(const T*)a, B * Np, (int)K};
  UnpadStore<T> st{(T*)out, N, Np, (int)ncols};
  gemm_kernel<T, TL><<<(unsigned)grid_size(n_rb, n_ct), TL::THREADS, 0, stream>>>(
      rows, (const T*)wt, (int)ncols, st, (int)K, (int)n_rb, (int)n_ct, (int)K);
  return hipGetLastError();
}

template <typename T>
hipError_t splitk_impl(const void* a, const void* wt, float* part, int64_t M, int64_t K,
                       int64_t ncols, int64_t k_split, int64_t n_split, hipStream_t stream) {
  using TL = SmallTiles;
  const int64_t n_rb = (M + TL::BM - 1) / TL::BM, n_ct = (ncols + TL::BN - 1) / TL::BN;
  if (!grid_ok(n_rb, n_ct) || n_split > 65535) return hipErrorInvalidConfiguration;
  DenseRows<T> rows{(const T*)a, M, (int)K};
  F32PartStore st{part, M, (int)ncols};
  gemm_kernel<T, TL><<<dim3((unsigned)grid_size(n_rb, n_ct), (unsigned)n_split), TL::THREADS, 0,
                       stream>>>(rows, (const T*)wt, (int)ncols, st, (int)K, (int)n_rb, (int)n_ct,
                                 (int)k_split);
  return hipGetLastError();
}

}  // namespace

SplitK splitk_plan(int64_t M, int64_t K, int64_t ncols) {
  const int64_t tiles = grid_size((M + SmallTiles::BM - 1) / SmallTiles::BM,
                                  (ncols + SmallTiles::BN - 1) / SmallTiles::BN);
  const int64_t steps = K / BK;
  // about 1024 workgroups, each with at least 32 k-steps
  int64_t n = std::max<int64_t>(1, std::min<int64_t>((1024 + tiles - 1) / tiles, steps / 32));
  SplitK p;
  p.k_split = (steps + n - 1) / n * BK;
  p.n_split = (K + p.k_split - 1) / p.k_split;
  return p;
}

size_t qkv_wt_bytes(sqa_dtype dt, int64_t d_model, int64_t H_q, int64_t H_kv, int64_t d_head) {
  return (size_t)(d_model * (H_q + 2 * H_kv) * d_head) * (dt == SQA_DTYPE_BF16 ? 2 : 4);
}

size_t out_wt_bytes(sqa_dtype dt, int64_t K, int64_t d_model) {
  return (size_t)(K * d_model) * (dt == SQA_DTYPE_BF16 ? 2 : 4);
}

hipError_t launch_qkv_projection(sqa_dtype dt, const void* x, const void* wq, const void* wk,
                                 const void* wv, void* wt, void* q, void* k, void* vt, int64_t B,
                                 int64_t N, int64_t Np, int64_t d_model, int64_t H_q, int64_t H_kv,
                                 int64_t d_head, const int32_t* lens, hipStream_t stream) {
  if (dt == SQA_DTYPE_BF16)
    return qkv_impl<bf16>(x, wq, wk, wv, wt, q, k, vt, B, N, Np, d_model, H_q, H_kv, d_head, lens,
                          stream);
  return qkv_impl<float>(x, wq, wk, wv, wt, q, k, vt, B, N, Np, d_model, H_q, H_kv, d_head, lens,
                         stream);
}

hipError_t launch_gemm_heads(sqa_dtype dt, const void* x, const void* wt, void* out, int64_t B,
                             int64_t N, int64_t Np, int64_t K, int64_t ncols, int64_t d_head,
                             hipStream_t stream) {
  return dt == SQA_DTYPE_BF16 ? heads_impl<bf16>(x, wt, out, B, N, Np, K, ncols, d_head, stream)
                              : heads_impl<float>(x, wt, out, B, N, Np, K, ncols, d_head, stream);
}

hipError_t launch_gemm_unpad(sqa_dtype dt, const void* a, const void* wt, void* out, int64_t B,
                             int64_t N, int64_t Np, int64_t K, int64_t ncols, hipStream_t stream) {
  return dt == SQA_DTYPE_BF16 ? unpad_impl<bf16>(a, wt, out, B, N, Np, K, ncols, stream)
                              : unpad_impl<float>(a, wt, out, B, N, Np, K, ncols, stream);
}

hipError_t launch_gemm_splitk(sqa_dtype dt, const void* a, const void* wt, float* part, int64_t M,
                              int64_t K, int64_t ncols, const SplitK& sk, hipStream_t stream) {
  return dt == SQA_DTYPE_BF16
      ? splitk_impl<bf16>(a, wt, part, M, K, ncols, sk.k_split, sk.n_split, stream)
      : splitk_impl<float>(a, wt, part, M, K, ncols, sk.k_split, sk.n_split, stream);
}

hipError_t launch_output_projection(sqa_dtype dt, const void* a, const void* wo, void* wt,
                                    void* out, int64_t M, int64_t K, int64_t d_model,
                                    const int32_t* lens, int64_t seq_n, hipStream_t stream) {
  if (dt == SQA_DTYPE_BF16)
    return out_impl<bf16>(a, wo, wt, out, M, K, d_model, lens, seq_n, stream);
  return out_impl<float>(a, wo, wt, out, M, K, d_model, lens, seq_n, stream);
}

}  // namespace sqa
