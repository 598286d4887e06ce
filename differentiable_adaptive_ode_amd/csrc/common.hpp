// Device-side building blocks shared by the solve and gradient kernels.
//
// Arithmetic contract with the CPU oracle: this library is compiled with
// -ffp-contract=off, so a fused multiply-add happens exactly where fmaR() is
// written.  Divisions and square roots are IEEE-rounded (no fast-math): the
// quotients that feed a step are either the compiler's IEEE division or
// recipR / divR below, which return the same bits for operands of normal
// magnitude.  So a forward solve computes the same bits as any other
// implementation that follows the same contract.  The one exception is the
// error weights s / sc_c, formed as s times a reciprocal within 11 ulp (rcpW):
// they only scale the mean square that the accept test and the truncated
// controller factor read.
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
// max(|a|, |b|) as one v_max instruction with absolute-value operands (the
// comparison and select take three, and the library fmax adds a
// canonicalising max per operand).  Equal to the comparison's choice for
// every non-NaN pair; arithmetic only, no memory access.
__device__ __forceinline__ double absmaxR(double a, double b) {
  double r;
  asm("v_max_f64 %0, |%1|, |%2|" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float absmaxR(float a, float b) {
  float r;
  asm("v_max_f32 %0, |%1|, |%2|" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ bool finiteR(double a) { return __builtin_isfinite(a); }
__device__ __forceinline__ bool finiteR(float a) { return __builtin_isfinite(a); }
__device__ __forceinline__ double nanR(double) { return __builtin_nan(""); }
__device__ __forceinline__ float nanR(float) { return __builtin_nanf(""); }

// 1/x for a finite nonzero normal x: the hardware reciprocal refined by
// Newton steps e = 1 - x r, r += r e (two in binary64, one in binary32), five
// or three instructions where an IEEE quotient takes eleven.  In binary64 this
// is the correctly rounded quotient (recipR below); in binary32 it is within
// an ulp, and is used only where the result scales a quantity compared against
// a threshold that absorbs such differences (the solve's error weights).
__device__ __forceinline__ double rcpR(double x) {
  double r = __builtin_amdgcn_rcp(x);
  double e = __builtin_fma(-x, r, 1.0);
  r = __builtin_fma(r, e, r);
  e = __builtin_fma(-x, r, 1.0);
  return __builtin_fma(r, e, r);
}
__device__ __forceinline__ float rcpR(float x) {
  float r = __builtin_amdgcn_rcpf(x);
  const float e = __builtin_fmaf(-x, r, 1.0f);
  return __builtin_fmaf(r, e, r);
}

// 1/x within 11 ulp (binary64; the hardware estimate, up to 2^28 ulp off, and
// one Newton step: the worst case over 4.3e9 values of every exponent from
// -500 to 500 measured on gfx950), for the error weights only: they scale the
// mean square, whose accept test and truncated controller factor absorb it.
// In binary32 rcpR.
__device__ __forceinline__ double rcpW(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return __builtin_fma(r, __builtin_fma(-x, r, 1.0), r);
}
__device__ __forceinline__ float rcpW(float x) { return rcpR(x); }

// 1/x where the quotient feeds the step itself (pivots, field terms), so it
// must equal the IEEE quotient.  In binary64 rcpR does: two Newton steps from
// the hardware estimate leave a relative error near 2^-104 before the last
// rounding, so the result is the correctly rounded 1/x unless that lies within
// 2^-104 of a rounding midpoint; on gfx950 it matched the IEEE quotient bit for
// bit on 2.1e10 values of random sign and mantissa spread over every exponent
// from -1022 to 1022.  It differs only at x = 0, +-inf and subnormal x (NaN
// where the quotient gives +-inf or 0), which arise only in a step whose
// result is non-finite either way.  Six instructions where the quotient takes
// eleven.  In binary32 (one Newton step would not round correctly) the IEEE
// quotient.
__device__ __forceinline__ double recipR(double x) { return rcpR(x); }
__device__ __forceinline__ float recipR(float x) { return 1.0f / x; }

// a/b, equal to the IEEE quotient: with r the correctly rounded 1/b and
// q = a r within an ulp of a/b, the residual a - b q is exact in one fused
// multiply-add and q + r (a - b q), rounded once, is the correctly rounded
// quotient (Markstein's theorem on FMA-based division), provided nothing
// overflows or underflows.  On gfx950 it matched the IEEE quotient bit for bit
// on 1.3e10 random pairs with divisor exponents up to +-900 (the same check
// finds a r alone, rounded twice, wrong in 27 % of cases).  Eight
// instructions where the quotient takes eleven; binary32 keeps the quotient.
__device__ __forceinline__ double divR(double a, double b) {
  const double r = rcpR(b);
  const double q = a * r;
  return __builtin_fma(__builtin_fma(-b, q, a), r, q);
}
__device__ __forceinline__ float divR(float a, float b) { return a / b; }

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

// Step-size controller power x^(-1/Q) (Q = 10 for Tsit5, 14 for Verner 7, 6
// for Rosenbrock23; x is the mean square of the scaled error, so this is
// err^(-1/(p+1)) with p the pair's lower order).
// A libm pow costs about a thousand cycles of dependent FP64 work per call on
// one wavefront; this rule costs two short polynomial evaluations:
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
template <>
struct CtrlRoot<14> {
  static constexpr double lo = 1e-15, hi = 1e10;
  static constexpr double c[8] = {0.971453564346184,      -0.02312982604893814,
                                  0.004130813507010568,   -0.0009509085609683622,
                                  0.00024095017603375496, -6.506922272280208e-05,
                                  2.2232410031470908e-05, -6.6171886469205804e-06};
};
__device__ constexpr double EXP2_NEG[7] = {0.7071067811579441,    -0.24506454511279616,
                                           0.042466448938030865,  -0.004905842513716687,
                                           0.00042506069534188184, -2.9611051419632863e-05,
                                           1.7091800607644192e-06};

__device__ __forceinline__ double frexpR(double x, int* e) { return __builtin_frexp(x, e); }
__device__ __forceinline__ float frexpR(float x, int* e) { return __builtin_frexpf(x, e); }
__device__ __forceinline__ double ldexpR(double x, int e) { return __builtin_ldexp(x, e); }
__device__ __forceinline__ float ldexpR(float x, int e) { return __builtin_ldexpf(x, e); }

// The rule's coefficients as values: literals, or pinned to vector registers
// once per kernel where scalar registers are the scarce resource (an empty
// asm that claims to modify the value keeps the compiler from rebuilding the
// literal from scalar moves at each use).
template <class R, int Q>
struct CtrlCoef {
  R c[8], e[7];
  __device__ __forceinline__ static R pin_(R v) {
    asm volatile("" : "+v"(v));
    return v;
  }
  __device__ __forceinline__ static CtrlCoef make(bool pinned) {
    CtrlCoef K;
#pragma unroll
    for (int i = 0; i < 8; ++i) K.c[i] = pinned ? pin_(R(CtrlRoot<Q>::c[i])) : R(CtrlRoot<Q>::c[i]);
#pragma unroll
    for (int i = 0; i < 7; ++i) K.e[i] = pinned ? pin_(R(EXP2_NEG[i])) : R(EXP2_NEG[i]);
    return K;
  }
};

// E(2b/Q - 1) ~ 2^(-b/Q), the power's fractional factor; it takes only the Q
// values b = 0 .. Q-1, so a kernel may tabulate it once (ctrl_root_tab).
template <class R, int Q>
__device__ __forceinline__ R ctrl_frac(int b, const CtrlCoef<R, Q>& K) {
  const R t = fmaR(R(b), R(2.0 / Q), R(-1));
  const R t2 = t * t, t4 = t2 * t2;
  const R q01 = fmaR(K.e[1], t, K.e[0]), q23 = fmaR(K.e[3], t, K.e[2]);
  const R q45 = fmaR(K.e[5], t, K.e[4]);
  return fmaR(fmaR(K.e[6], t2, q45), t4, fmaR(q23, t2, q01));
}

// The power with E(b) from `tab` (tab[b] = ctrl_frac(b)) or, for a null tab,
// evaluated in place: the same values either way.
template <class R, int Q>
__device__ __forceinline__ R ctrl_root_tab(R x, const CtrlCoef<R, Q>& K, const R* tab) {
  using L = CtrlRoot<Q>;
  x = x > R(L::lo) ? x : R(L::lo);
  x = x < R(L::hi) ? x : R(L::hi);
  int e = 0;
  const R mh = frexpR(x, &e);  // x = mh 2^e, mh in [1/2, 1): m = 2 mh
  e -= 1;
  const int a = (e + 64 * Q) / Q - 64;  // floor(e / Q); e > -64 Q after the clamp
  const int b = e - Q * a;
  const R s = fmaR(mh, R(4), R(-3));  // 2 m - 3, exact
  // P(s), degree 7, and E(t), degree 6, by Estrin's scheme (pairs of
  // coefficients, then pairs of pairs): three dependent steps, not seven.
  const R s2 = s * s, s4 = s2 * s2;
  const R p01 = fmaR(K.c[1], s, K.c[0]), p23 = fmaR(K.c[3], s, K.c[2]);
  const R p45 = fmaR(K.c[5], s, K.c[4]), p67 = fmaR(K.c[7], s, K.c[6]);
  const R p = fmaR(fmaR(p67, s2, p45), s4, fmaR(p23, s2, p01));
  const R q = tab ? tab[b] : ctrl_frac<R, Q>(b, K);
  return ldexpR(p * q, -a);
}

template <class R, int Q>
__device__ __forceinline__ R ctrl_root(R x, const CtrlCoef<R, Q>& K) {
  return ctrl_root_tab<R, Q>(x, K, nullptr);
}

// Lane index within the 64-wide wavefront and cross-lane helpers.
__device__ __forceinline__ int laneId() { return __lane_id(); }

}  // namespace dao
