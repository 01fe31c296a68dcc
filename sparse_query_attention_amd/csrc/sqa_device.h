// Device-side building blocks shared by the gfx950 kernels: element types,
// the MFMA instructions each dtype uses, and the operand layouts they share.
//
// A 32x32 MFMA tile (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32)
// computes C[32][32] += A[32][K] * B[K][32] across one wave of 64 lanes:
//   A operand: lane l supplies row (l % 32), k-group (l / 32), E values
//   B operand: lane l supplies column (l % 32), k-group (l / 32), E values
//   C/D:       lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4)
//              for its 16 accumulator registers r = 0..15
// The k-group split only has to agree between A and B, so every operand below
// is loaded with "k-group g holds the E consecutive k at g*E of each step".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;

// bf16 inputs, fp32 accumulation: 32x32x16, 8 bf16 (16 bytes) per lane and operand.
template <> struct Mfma<bf16> {
  static constexpr int E = 8;
  static constexpr int KS = 16;
  typedef bf16x8 Frag;
  __device__ static inline f32x16 run(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// fp32 inputs and accumulation: 32x32x2, one float per lane and operand.
template <> struct Mfma<float> {
  static constexpr int E = 1;
  static constexpr int KS = 2;
  typedef float Frag;
  __device__ static inline f32x16 run(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Round-to-nearest-even conversion from fp32 (v_cvt_pk_bf16_f32 on gfx950).
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16-byte vector of T, the unit of every global<->LDS copy.
struct alignas(16) Chunk { uint32_t w[4]; };

__device__ inline Chunk zero_chunk() { Chunk c; c.w[0] = c.w[1] = c.w[2] = c.w[3] = 0u; return c; }

// Swap bits 2 and 3 of an index (an involution within each aligned group of
// 16). A B operand packed from accumulator registers carries, in k-step h of a
// 32-row block, rows 16h + 8*(e/4) + 4*grp + e%4 for its 8 slots e; after this
// permutation of the rows those are the 8 consecutive positions 16h + 8*grp + e,
// so the matching A operand is one 16-byte read.
__host__ __device__ inline int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// XOR swizzle of 16-byte chunks within an LDS row of CPR chunks. It spreads
// the rows that one ds_read_b128 touches over distinct banks.
template <int CPR> __device__ inline int swz(int r);
template <> __device__ inline int swz<16>(int r) { return r & 15; }
template <> __device__ inline int swz<8>(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <> __device__ inline int swz<4>(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Direct global->LDS loads (global_load_lds): lane L of a 16-byte load lands
// 16*L bytes past the load's LDS base, and the loads count in vmcnt.
// Wait until at most N of this wave's vector-memory operations are outstanding
// (N < 64: vmcnt bits [3:0] and [15:14]). The other counters are left unconstrained.
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait_vmcnt<n * PER>() for a runtime n in [0, MAXN].
template <int PER, int MAXN> __device__ inline void wait_vmcnt_tiles(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) { wait_vmcnt<MAXN * PER>(); return; }
    wait_vmcnt_tiles<PER, MAXN - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier between the steps of a ring of LDS slots filled by direct
// loads. The fences of __syncthreads() make the compiler drain every load in
// flight (direct loads count in vmcnt), which would empty the ring at each
// step. Callers first wait with wait_vmcnt for the loads the next step reads;
// every LDS read of the slot about to be refilled has returned, since its data
// was consumed before the barrier. The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ inline void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace sqa
