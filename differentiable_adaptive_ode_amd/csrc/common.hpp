// Device-side building blocks shared by the solve and gradient kernels.
//
// Arithmetic contract with the CPU oracle: this library is compiled with
// -ffp-contract=off, so a fused multiply-add happens exactly where fmaR() is
// written.  Divisions and square roots are IEEE-rounded (no fast-math), so a
// forward solve computes the same bits as any other implementation that
// follows the same contract.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dao {

enum : int32_t {
  TRAJ_OK = 0,
  TRAJ_MAX_STEPS = 1,
  TRAJ_NONFINITE = 2,
  TRAJ_DT_UNDERFLOW = 3,
  TRAJ_CAPACITY = 4,
};

constexpr int WAVE = 64;

__device__ __forceinline__ double fmaR(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float fmaR(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double absR(double a) { return __builtin_fabs(a); }
__device__ __forceinline__ float absR(float a) { return __builtin_fabsf(a); }
__device__ __forceinline__ double sqrtR(double a) { return __builtin_sqrt(a); }
__device__ __forceinline__ float sqrtR(float a) { return __builtin_sqrtf(a); }
__device__ __forceinline__ double powR(double a, double b) { return pow(a, b); }
__device__ __forceinline__ float powR(float a, float b) { return powf(a, b); }
__device__ __forceinline__ double maxR(double a, double b) { return a > b ? a : b; }
__device__ __forceinline__ float maxR(float a, float b) { return a > b ? a : b; }
__device__ __forceinline__ double minR(double a, double b) { return a < b ? a : b; }
__device__ __forceinline__ float minR(float a, float b) { return a < b ? a : b; }
__device__ __forceinline__ bool finiteR(double a) { return __builtin_isfinite(a); }
__device__ __forceinline__ bool finiteR(float a) { return __builtin_isfinite(a); }
__device__ __forceinline__ double nanR(double) { return __builtin_nan(""); }
__device__ __forceinline__ float nanR(float) { return __builtin_nanf(""); }

// Step-size factors are truncated to a few significant bits (16 explicit
// mantissa bits in binary64, 8 in binary32) so that the accepted mesh does
// not depend on the last-ulp behaviour of pow() in a given math library.
__device__ __forceinline__ double truncBits(double x) {
  unsigned long long u = __double_as_longlong(x);
  u &= ~((1ull << 36) - 1ull);
  return __longlong_as_double(u);
}
__device__ __forceinline__ float truncBits(float x) {
  unsigned int u = __float_as_uint(x);
  u &= ~((1u << 15) - 1u);
  return __uint_as_float(u);
}

// Lane index within the 64-wide wavefront and cross-lane helpers.
__device__ __forceinline__ int laneId() { return __lane_id(); }

}  // namespace dao
