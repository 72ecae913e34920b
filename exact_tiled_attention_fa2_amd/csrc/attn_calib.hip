// Matrix-core rate calibration for gfx950 (debug build only; the release
// library compiles nothing from this file).
//
// The attention kernels are priced against the published dense MFMA peak.
// Under sustained load the board's power limit pulls the clock below its
// maximum, and how far depends on what the matrix cores are fed.  This
// kernel measures the rate the matrix cores sustain with no memory traffic
// and no other vector work: every wave issues back-to-back 32x32x16 MFMAs of
// one 16-bit type into four independent accumulators (so no MFMA waits on
// the previous one's result), on operands read once from a caller buffer --
// random values, or zeros, which draw less power.
#if defined(ATTN_DEBUG_BUILD)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_mi355x.h"
#include "attn_mi355x_debug.h"

namespace attn {
namespace {

constexpr int kCalibThreads = 256;

// ops: 64 lanes x 8 16-byte chunks (lane-major): chunks 0-3 are the lane's A
// fragments, 4-7 its B fragments.  out: one float per thread.
template <class Ty>
__global__ void __launch_bounds__(kCalibThreads) calib_mfma_kernel(const u32x4* __restrict__ ops,
                                                                   float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[lane * 8 + i];
    b[i] = ops[lane * 8 + 4 + i];
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = Ty::mfma(a[(j + k) & 3], b[j], acc[k]);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace attn

extern "C" int attn_debug_calib_mfma(int32_t dtype, const void* operands, float* out, int32_t blocks,
                                     int32_t iters, void* stream) {
  if (operands == nullptr || out == nullptr) return ATTN_E_NULL;
  if ((reinterpret_cast<uintptr_t>(operands) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return ATTN_E_ALIGN;
  if (blocks < 1 || iters < 1) return ATTN_E_SHAPE;
  const attn::u32x4* ops = static_cast<const attn::u32x4*>(operands);
  const dim3 grid((unsigned)blocks), block(attn::kCalibThreads);
  if (dtype == ATTN_DTYPE_BF16) {
    hipLaunchKernelGGL(attn::calib_mfma_kernel<attn::TypeBF16>, grid, block, 0, (hipStream_t)stream, ops, out,
                       (int)iters);
  } else if (dtype == ATTN_DTYPE_F16) {
    hipLaunchKernelGGL(attn::calib_mfma_kernel<attn::TypeF16>, grid, block, 0, (hipStream_t)stream, ops, out,
                       (int)iters);
  } else {
    return ATTN_E_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

#endif  // ATTN_DEBUG_BUILD
