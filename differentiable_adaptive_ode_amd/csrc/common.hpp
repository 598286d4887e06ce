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
constexpr int BLOCK_WAVES = 4;  // wavefronts per workgroup of the per-lane kernels

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

// Step-size controller power x^(-1/Q) (Q = 10 for Tsit5, 6 for Rosenbrock23;
// x is the mean square of the scaled error, so this is err^(-1/(order+1))).
// A libm pow costs about a thousand cycles of dependent FP64 work per call on
// one wavefront; this rule costs two short Horner chains:
//   clamp x to [lo, hi] (beyond it 0.9 x^(-1/Q) is outside the controller's
//   limits [0.2, 10] anyway), write x = m 2^e with m in [1, 2) and
//   e = Q a + b (0 <= b < Q), then
//   x^(-1/Q) = P(2m - 3) * E(2 b / Q - 1) * 2^(-a)
// with P ~ m^(-1/Q) on [1, 2] and E ~ 2^(-f) on f in [0, 1] (Chebyshev
// interpolants in monomial form; relative error below 1e-7).  Every step is
// IEEE-exact or an explicit fused multiply-add, so the result does not depend
// on any math library.
template <int Q>
struct CtrlRoot;
template <>
struct CtrlRoot<10> {
  static constexpr double lo = 1e-12, hi = 1e8;
  static constexpr double c[8] = {0.9602644780153649,     -0.03200878522189435,
                                  0.005869002336249675,   -0.0013696795740665145,
                                  0.0003502086621236076,  -9.523230976561381e-05,
                                  3.278285231379161e-05,  -9.803433032024717e-06};
};
template <>
struct CtrlRoot<6> {
  static constexpr double lo = 1e-8, hi = 1e5;
  static constexpr double c[8] = {0.9346552216460542,     -0.05192523185937651,
                                  0.010097959271667333,   -0.0024314560515976726,
                                  0.0006347021852295785,  -0.0001753744494318341,
                                  6.143024330877807e-05,  -1.8571447204984547e-05};
};
__device__ constexpr double EXP2_NEG[7] = {0.7071067811579441,    -0.24506454511279616,
                                           0.042466448938030865,  -0.004905842513716687,
                                           0.00042506069534188184, -2.9611051419632863e-05,
                                           1.7091800607644192e-06};

__device__ __forceinline__ double frexpR(double x, int* e) { return __builtin_frexp(x, e); }
__device__ __forceinline__ float frexpR(float x, int* e) { return __builtin_frexpf(x, e); }
__device__ __forceinline__ double ldexpR(double x, int e) { return __builtin_ldexp(x, e); }
__device__ __forceinline__ float ldexpR(float x, int e) { return __builtin_ldexpf(x, e); }

template <class R, int Q>
__device__ __forceinline__ R ctrl_root(R x) {
  using K = CtrlRoot<Q>;
  x = x > R(K::lo) ? x : R(K::lo);
  x = x < R(K::hi) ? x : R(K::hi);
  int e = 0;
  const R m = frexpR(x, &e) * R(2);  // x = m 2^(e-1)
  e -= 1;
  const int a = (e + 64 * Q) / Q - 64;  // floor(e / Q); e > -64 Q after the clamp
  const int b = e - Q * a;
  const R s = m * R(2) - R(3);
  R p = R(K::c[7]);
#pragma unroll
  for (int i = 6; i >= 0; --i) p = fmaR(p, s, R(K::c[i]));
  const R s2 = fmaR(R(b), R(2.0 / Q), R(-1));
  R q = R(EXP2_NEG[6]);
#pragma unroll
  for (int i = 5; i >= 0; --i) q = fmaR(q, s2, R(EXP2_NEG[i]));
  return ldexpR(p * q, -a);
}

// Lane index within the 64-wide wavefront and cross-lane helpers.
__device__ __forceinline__ int laneId() { return __lane_id(); }

}  // namespace dao
