// Device helpers shared by the forward and backward kernels (gfx950): vector
// types, the 16-bit MFMA/pack wrappers, the LDS chunk swizzle, HBM -> LDS
// copies and memory-counter waits.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace attn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;

struct TypeBF16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> one packed pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

struct TypeF16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

// XOR pattern for the 16-byte chunk index of LDS row r (r taken mod 16).
// Rows 0..15 map to 16 distinct values, so the K operand reads (16 rows, one
// chunk each) cover all banks.  Within each group of 4 consecutive rows that
// starts at a multiple of 4 the pattern differs in bits 2-3 only, so the
// transposing V reads (4 rows x 4 adjacent chunks per 32 lanes) also land on
// 16 distinct chunk positions.
__device__ __forceinline__ int chunk_swizzle(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool SOFTCAP>
__device__ __forceinline__ float transform_score(float s, float pre, float cap) {
  if constexpr (SOFTCAP) {
    // cap * tanh(s * pre) with tanh(x) = 1 - 2 / (exp(2x) + 1); saturates to +-cap.
    float e = fast_exp2(s * pre * (2.0f * kLog2e));
    return cap * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
  } else {
    return s;
  }
}

// One 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4): lane l of
// the wave writes LDS bytes [lds + 16 l, lds + 16 l + 16); `lds` must be
// wave-uniform.  No VGPR is used for the data.
__device__ __forceinline__ void dma16(const void* g, const char* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}
// The same copy with a cache-policy operand (gfx950 CPOL bits: 1 = sc0,
// 2 = nt, 16 = sc1).  CPOL_NT marks data that is streamed once.
constexpr int CPOL_NT = 2;
template <int CPOL>
__device__ __forceinline__ void dma16_pol(const void* g, const char* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, CPOL);
}

// HBM -> LDS copies through a buffer resource: the tile's base address lives
// in scalar registers and each lane adds a 32-bit byte offset, so a copy
// costs one VGPR per lane instead of a 64-bit address.  Word 3 of the
// resource selects raw 32-bit data on gfx9-family parts (0x00020000); the
// record count is the whole 32-bit range, so an offset never reads past it
// and the hardware returns zero instead of faulting for an out-of-range one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
// One 16-byte copy per lane of tile byte `voff` into LDS bytes
// [lds + 16 lane, +16) (`lds` wave-uniform), with cache policy CPOL.
template <int CPOL>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, const char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16, voff, 0, 0,
                                           CPOL);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier of a tile pipeline: this wave's LDS reads and writes have
// retired (lgkmcnt(0)) and at most N vector-memory operations -- the newest,
// i.e. HBM -> LDS copies for later steps -- are still in flight.
// __syncthreads() would also drain those (its release fence waits for
// vmcnt(0)), so a copy issued two steps ahead would have to land within the
// current step.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier; the explicit wait gives the ordering
// the hardware needs.
// (s_waitcnt gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.)
template <int N>
__device__ __forceinline__ void barrier_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace attn
