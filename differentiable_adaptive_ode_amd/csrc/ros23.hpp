// Rosenbrock23: the second-order linearly implicit Rosenbrock-Wanner method
// of Shampine & Reichelt (the ode23s triple), autonomous form.  arXiv
// 2609.02876 Sec. 3.1 names it as the stiff default of the fused kernels and
// Sec. 3.2 gives the structure: each stage solves with W = I - gamma h J,
// and the backward sweep needs one more solve per stage, against W^T.
//
//   F0 = f(y), W = I - h d J(y), d = 1/(2 + sqrt 2)
//   k1 = W^-1 F0
//   F1 = f(y + h/2 k1)
//   k2 = W^-1 (F1 - k1) + k1
//   y_new = y + h k2
//   F2 = f(y_new)                                   (reused as the next F0)
//   k3 = W^-1 (F2 - e32 (k2 - F1) - 2 (k1 - F0)),   e32 = 6 + sqrt 2
//   err = h/6 (k1 - 2 k2 + k3)   (trial() returns k1 - 2 k2 + k3; the
//                                 solve folds h/6 into its error weights)
//
// W is factored per lane as P W = L U with partial pivoting (first row of
// largest magnitude); the reciprocal pivots are formed once per
// factorisation and the elimination and every solve multiply by them.  The
// pivot index is data dependent, so rows are exchanged with selects on
// compile-time indices to keep every value in a register.  When no lane of
// the wavefront exchanges rows at a step (the usual case: for Robertson's W
// the diagonal always pivots), the selects of that step are skipped on a
// wavefront-uniform branch; they would leave every value as it is.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace dao {
namespace ros23 {

__device__ constexpr double GAMMA = 0.29289321881345248;  // 1 / (2 + sqrt 2)
__device__ constexpr double E32 = 7.4142135623730951;     // 6 + sqrt 2

// Keeps the compiler from turning a skippable block into selects executed
// every time (an empty asm statement cannot be speculated).
__device__ __forceinline__ void skip_point() { asm volatile("" ::: "memory"); }

template <class R, int D>
struct LU {
  R m[D][D];   // unit-lower L below the diagonal, U on and above
  R rp[D];     // reciprocal pivots 1 / u_kk (elimination and solves multiply by them)
  int piv[D];  // row exchanged with row k at elimination step k
  bool swaps;  // some lane of the wavefront exchanges rows (wavefront-uniform)
};

// Sparse systems.  A system may declare which entries of its Jacobian can be
// nonzero (static constexpr bool jac_nz(i, j)).  W then has that pattern plus
// the diagonal, and eliminating without row exchanges fills in only where
// lu_nz says (computed at compile time).  While no lane of the wavefront has
// exchanged rows, factor, solve and solve_t skip the entries outside it: the
// dense code would only add exact zeros there (a structurally zero multiplier
// or row entry), so every nonzero value is the dense code's own.  From the
// first step at which some lane exchanges rows, the dense code runs.
template <class Sys, class = void>
struct HasJacPattern : std::false_type {};
template <class Sys>
struct HasJacPattern<Sys, std::void_t<decltype(Sys::jac_nz(0, 0))>> : std::true_type {};

template <int D>
struct Pattern {
  bool nz[D][D];
};
template <class Sys>
constexpr Pattern<Sys::D> fill_pattern() {
  constexpr int D = Sys::D;
  Pattern<D> p{};
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) p.nz[i][j] = (i == j) || Sys::jac_nz(i, j);
  for (int k = 0; k < D; ++k)
    for (int i = k + 1; i < D; ++i)
      if (p.nz[i][k])
        for (int j = k + 1; j < D; ++j)
          if (p.nz[k][j]) p.nz[i][j] = true;
  return p;
}
template <class Sys>
__device__ constexpr Pattern<Sys::D> lu_nz = fill_pattern<Sys>();

// Whether J's entry (i, j) can be nonzero (every entry, for a system that
// declares no pattern).
template <class Sys>
__device__ constexpr bool jac_entry(int i, int j) {
  if constexpr (HasJacPattern<Sys>::value) {
    return Sys::jac_nz(i, j);
  } else {
    return true;
  }
}

// Whether factor/solve/solve_t take the sparse path for Sys (void: dense).
template <class Sys, bool SKIP>
constexpr bool sparse_lu() {
  if constexpr (std::is_void<Sys>::value) {
    return false;
  } else {
    return SKIP && HasJacPattern<Sys>::value;
  }
}

// SKIP (here and below): test, once per elimination step and per solve,
// whether any lane of the wavefront exchanges rows, and skip the exchange on
// a real branch when none does.  Without it the exchanges are selects in
// straight-line code, which suits kernels that run many independent solves
// per step (the sensitivity tangents), where branches would keep the
// compiler from interleaving them.
//
// One elimination step k of factor (a template parameter: the sparse and the
// dense step together are too large for the compiler to unroll a loop over k,
// and a loop left rolled would index the factors at run time, through
// scratch memory).
template <int K, class R, int D, bool SKIP, class Sys>
__device__ __forceinline__ void factor_step(LU<R, D>& f, bool& dense) {
  if constexpr (K < D) {
    constexpr int k = K;
    bool done = false;  // step k taken by the sparse code
    if constexpr (sparse_lu<Sys, SKIP>()) {
      if (!dense) {
        // pivot among the rows that can be nonzero in column k (a structural
        // zero never wins: 0 > best is false)
        int p = k;
        R best = absR(f.m[k][k]);
#pragma unroll
        for (int i = k + 1; i < D; ++i) {
          if (lu_nz<Sys>.nz[i][k]) {
            R v = absR(f.m[i][k]);
            if (v > best) { best = v; p = i; }
          }
        }
        if ((k + 1 < D) && __ballot(p != k) != 0ull) {
          dense = true;  // some lane exchanges rows at step k: the dense code from here on
        } else {
          f.piv[k] = k;
          f.rp[k] = recipR(f.m[k][k]);
#pragma unroll
          for (int i = k + 1; i < D; ++i) {
            if (lu_nz<Sys>.nz[i][k]) {
              R l = f.m[i][k] * f.rp[k];
              f.m[i][k] = l;
#pragma unroll
              for (int j = k + 1; j < D; ++j)
                if (lu_nz<Sys>.nz[k][j]) f.m[i][j] = fmaR(-l, f.m[k][j], f.m[i][j]);
            }
          }
          done = true;
        }
      }
    }
    if (!done) {
      int p = k;
      R best = absR(f.m[k][k]);
#pragma unroll
      for (int i = k + 1; i < D; ++i) {
        R v = absR(f.m[i][k]);
        if (v > best) { best = v; p = i; }
      }
      f.piv[k] = p;
      const bool any = !SKIP || ((k + 1 < D) && __ballot(p != k) != 0ull);
      f.swaps = f.swaps || any;
      if (any) {
        if (SKIP) skip_point();
#pragma unroll
        for (int i = k + 1; i < D; ++i) {
          const bool sw = (p == i);
#pragma unroll
          for (int j = 0; j < D; ++j) {
            R rk = f.m[k][j], ri = f.m[i][j];
            f.m[k][j] = sw ? ri : rk;
            f.m[i][j] = sw ? rk : ri;
          }
        }
      }
      f.rp[k] = recipR(f.m[k][k]);
#pragma unroll
      for (int i = k + 1; i < D; ++i) {
        R l = f.m[i][k] * f.rp[k];
        f.m[i][k] = l;
#pragma unroll
        for (int j = k + 1; j < D; ++j) f.m[i][j] = fmaR(-l, f.m[k][j], f.m[i][j]);
      }
    }
    factor_step<K + 1, R, D, SKIP, Sys>(f, dense);
  }
}

template <class R, int D, bool SKIP = true, class Sys = void>
__device__ __forceinline__ void factor(LU<R, D>& f) {
  bool dense = !sparse_lu<Sys, SKIP>();  // (wavefront-uniform) the dense code runs
  f.swaps = false;
  factor_step<0, R, D, SKIP, Sys>(f, dense);
}

// x = W^-1 b
template <class R, int D, bool SKIP = true, class Sys = void>
__device__ __forceinline__ void solve(const LU<R, D>& f, const R (&b)[D], R (&x)[D]) {
  if constexpr (sparse_lu<Sys, SKIP>()) {
    if (!f.swaps) {
      R z[D];
#pragma unroll
      for (int i = 0; i < D; ++i) {
        z[i] = b[i];
#pragma unroll
        for (int j = 0; j < D; ++j)
          if (j < i && lu_nz<Sys>.nz[i][j]) z[i] = fmaR(-f.m[i][j], z[j], z[i]);
      }
#pragma unroll
      for (int i = D - 1; i >= 0; --i) {
        R acc = z[i];
#pragma unroll
        for (int j = 0; j < D; ++j)
          if (j > i && lu_nz<Sys>.nz[i][j]) acc = fmaR(-f.m[i][j], x[j], acc);
        x[i] = acc * f.rp[i];
      }
      return;
    }
  }
  R z[D];
#pragma unroll
  for (int i = 0; i < D; ++i) z[i] = b[i];
  if (!SKIP || f.swaps) {
    if (SKIP) skip_point();
#pragma unroll
    for (int k = 0; k < D; ++k) {
#pragma unroll
      for (int i = k + 1; i < D; ++i) {
        const bool sw = (f.piv[k] == i);
        R zk = z[k], zi = z[i];
        z[k] = sw ? zi : zk;
        z[i] = sw ? zk : zi;
      }
    }
  }
#pragma unroll
  for (int i = 1; i < D; ++i)
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < i) z[i] = fmaR(-f.m[i][j], z[j], z[i]);
#pragma unroll
  for (int i = D - 1; i >= 0; --i) {
    R acc = z[i];
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j > i) acc = fmaR(-f.m[i][j], x[j], acc);
    x[i] = acc * f.rp[i];
  }
}

// x = W^-T b, with W = P^T L U:  U^T z = b,  L^T w = z,  x = P^T w.
template <class R, int D, bool SKIP = true, class Sys = void>
__device__ __forceinline__ void solve_t(const LU<R, D>& f, const R (&b)[D], R (&x)[D]) {
  if constexpr (sparse_lu<Sys, SKIP>()) {
    if (!f.swaps) {
      R z[D];
#pragma unroll
      for (int i = 0; i < D; ++i) {
        R acc = b[i];
#pragma unroll
        for (int j = 0; j < D; ++j)
          if (j < i && lu_nz<Sys>.nz[j][i]) acc = fmaR(-f.m[j][i], z[j], acc);
        z[i] = acc * f.rp[i];
      }
#pragma unroll
      for (int i = D - 1; i >= 0; --i) {
        R acc = z[i];
#pragma unroll
        for (int j = 0; j < D; ++j)
          if (j > i && lu_nz<Sys>.nz[j][i]) acc = fmaR(-f.m[j][i], x[j], acc);
        x[i] = acc;
      }
      return;
    }
  }
  R z[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    R acc = b[i];
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < i) acc = fmaR(-f.m[j][i], z[j], acc);
    z[i] = acc * f.rp[i];
  }
#pragma unroll
  for (int i = D - 1; i >= 0; --i) {
    R acc = z[i];
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j > i) acc = fmaR(-f.m[j][i], x[j], acc);
    x[i] = acc;
  }
  if (!SKIP || f.swaps) {
    if (SKIP) skip_point();
#pragma unroll
    for (int k = D - 1; k >= 0; --k) {
#pragma unroll
      for (int i = k + 1; i < D; ++i) {
        const bool sw = (f.piv[k] == i);
        R xk = x[k], xi = x[i];
        x[k] = sw ? xi : xk;
        x[i] = sw ? xk : xi;
      }
    }
  }
}

template <class R, class Sys, bool SKIP = true>
__device__ __forceinline__ void build_w(const Sys& sys, const R (&y)[Sys::D], R h,
                                        LU<R, Sys::D>& w) {
  constexpr int D = Sys::D;
  R J[D][D];
  sys.jac(y, J);
  R hd = h * R(GAMMA);
#pragma unroll
  for (int i = 0; i < D; ++i)
#pragma unroll
    for (int j = 0; j < D; ++j) w.m[i][j] = fmaR(-hd, J[i][j], R(i == j ? 1 : 0));
  factor<R, D, SKIP, Sys>(w);
}

// Trial step: F0 = f(y) on entry; returns ynew, F2 = f(ynew) and err.
template <class R, class Sys, bool SKIP = true>
__device__ __forceinline__ void trial(const Sys& sys, const R (&y)[Sys::D], R h,
                                      const R (&F0)[Sys::D], R (&ynew)[Sys::D], R (&F2)[Sys::D],
                                      R (&err)[Sys::D]) {
  constexpr int D = Sys::D;
  LU<R, D> w;
  build_w<R, Sys, SKIP>(sys, y, h, w);
  R k1[D], k2[D], Y1[D], F1[D], r[D], u[D], k3[D];
  solve<R, D, SKIP, Sys>(w, F0, k1);
  R hh = R(0.5) * h;
#pragma unroll
  for (int c = 0; c < D; ++c) Y1[c] = fmaR(hh, k1[c], y[c]);
  sys.f(Y1, F1);
#pragma unroll
  for (int c = 0; c < D; ++c) r[c] = F1[c] - k1[c];
  solve<R, D, SKIP, Sys>(w, r, u);
#pragma unroll
  for (int c = 0; c < D; ++c) k2[c] = u[c] + k1[c];
#pragma unroll
  for (int c = 0; c < D; ++c) ynew[c] = fmaR(h, k2[c], y[c]);
  sys.f(ynew, F2);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    R t2 = fmaR(R(-E32), k2[c] - F1[c], F2[c]);
    r[c] = fmaR(R(-2), k1[c] - F0[c], t2);
  }
  solve<R, D, SKIP, Sys>(w, r, k3);
  // the embedded error without its factor h/6 (in the error weights)
#pragma unroll
  for (int c = 0; c < D; ++c) err[c] = fmaR(R(-2), k2[c], k1[c]) + k3[c];
}

// Replay step y <- Phi(y; h) (no k3, no error estimate).
template <class R, class Sys>
__device__ __forceinline__ void replay(const Sys& sys, R (&y)[Sys::D], R h) {
  constexpr int D = Sys::D;
  LU<R, D> w;
  build_w(sys, y, h, w);
  R F0[D], k1[D], Y1[D], F1[D], r[D], u[D];
  sys.f(y, F0);
  solve<R, D, true, Sys>(w, F0, k1);
  R hh = R(0.5) * h;
#pragma unroll
  for (int c = 0; c < D; ++c) Y1[c] = fmaR(hh, k1[c], y[c]);
  sys.f(Y1, F1);
#pragma unroll
  for (int c = 0; c < D; ++c) r[c] = F1[c] - k1[c];
  solve<R, D, true, Sys>(w, r, u);
#pragma unroll
  for (int c = 0; c < D; ++c) y[c] = fmaR(h, u[c] + k1[c], y[c]);
}

// Reverse of one replay step, in two parts: the forward quantities of the
// step (they depend only on y_j and h_j), then the sweep that takes
// lam = dL/dy_{j+1} to dL/dy_j and accumulates dL/dtheta into pb.
template <class R, int D>
struct Stages {
  LU<R, D> w;   // factors of W = I - h d J(y)
  R y[D];       // y_j
  R k1[D];      // W^-1 F0
  R Y1[D];      // y + h/2 k1
  R u[D];       // W^-1 (F1 - k1)
};

template <class R, class Sys, bool SKIP = true>
__device__ __forceinline__ void stages(const Sys& sys, const R (&y)[Sys::D], R h,
                                       Stages<R, Sys::D>& S) {
  constexpr int D = Sys::D;
  build_w<R, Sys, SKIP>(sys, y, h, S.w);
  R F0[D], F1[D], r[D];
#pragma unroll
  for (int c = 0; c < D; ++c) S.y[c] = y[c];
  sys.f(y, F0);
  solve<R, D, SKIP, Sys>(S.w, F0, S.k1);
  R hh = R(0.5) * h;
#pragma unroll
  for (int c = 0; c < D; ++c) S.Y1[c] = fmaR(hh, S.k1[c], y[c]);
  sys.f(S.Y1, F1);
#pragma unroll
  for (int c = 0; c < D; ++c) r[c] = F1[c] - S.k1[c];
  solve<R, D, SKIP, Sys>(S.w, r, S.u);
}

template <class R, class Sys>
__device__ __forceinline__ void sweep(const Sys& sys, const Stages<R, Sys::D>& S, R h,
                                      R (&lam)[Sys::D], R (&pb)[Sys::P]) {
  constexpr int D = Sys::D;
  const R hh = R(0.5) * h;
  // y_new = y + h (u + k1)
  R ub[D], k1b[D], rb[D], tmp[D], F0b[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    ub[c] = h * lam[c];
    k1b[c] = ub[c];
  }
  // u = W^-1 r:  rb = W^-T ub,  Wb = -rb u^T
  solve_t<R, D, true, Sys>(S.w, ub, rb);
  // r = F1 - k1
#pragma unroll
  for (int c = 0; c < D; ++c) k1b[c] -= rb[c];
  // F1 = f(Y1), Y1 = y + h/2 k1
  sys.vjp(S.Y1, rb, tmp, pb);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    lam[c] += tmp[c];
    k1b[c] = fmaR(hh, tmp[c], k1b[c]);
  }
  // k1 = W^-1 F0:  F0b = W^-T k1b,  Wb -= F0b k1^T
  solve_t<R, D, true, Sys>(S.w, k1b, F0b);
  // F0 = f(y)
  sys.vjp(S.y, F0b, tmp, pb);
#pragma unroll
  for (int c = 0; c < D; ++c) lam[c] += tmp[c];
  // W = I - h d J(y, theta):  Jb = -h d Wb = h d (rb u^T + F0b k1^T)
  R hd = h * R(GAMMA);
  R Jb[D][D];
#pragma unroll
  for (int i = 0; i < D; ++i)
#pragma unroll
    for (int j = 0; j < D; ++j) Jb[i][j] = hd * fmaR(rb[i], S.u[j], F0b[i] * S.k1[j]);
  sys.jac_vjp(S.y, Jb, lam, pb);
}

// Tangent of one replay step along NT directions (arXiv 2609.28458 Sec. 2.3:
// the sensitivity equations with the steps held fixed), from the step's
// forward quantities St (stages() at the same y and h).  Direction t is the
// parameter dir[t] (none for dir[t] < 0 or >= P).  On entry S[c][t] = dy_c/dp_t,
// on exit the tangent of y_new = y + h (u + k1):
//   Wd = -h d Jd,  k1d = W^-1 (F0d - Wd k1),  Y1d = yd + h/2 k1d,
//   ud = W^-1 (F1d - k1d - Wd u),  y_new d = yd + h (ud + k1d),
// with F0d, F1d the field's tangents at y and Y1 and Jd the Jacobian's.
template <class R, class Sys, int NT, bool SKIP = true>
__device__ __forceinline__ void tangent(const Sys& sys, const Stages<R, Sys::D>& St, R h,
                                        const int (&dir)[NT], R (&S)[Sys::D][NT]) {
  constexpr int D = Sys::D;
  const R hh = R(0.5) * h, hd = h * R(GAMMA);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    R yd[D], F0d[D], F1d[D], k1d[D], Y1d[D], ud[D], r[D];
    R Jd[D][D];
#pragma unroll
    for (int c = 0; c < D; ++c) yd[c] = S[c][t];
    sys.jvp(St.y, yd, dir[t], F0d);
    sys.jac_jvp(St.y, yd, dir[t], Jd);
    // F0d - Wd k1 = F0d + h d Jd k1 (Jd has J's pattern: the structural
    // zeros would add exact zeros)
#pragma unroll
    for (int i = 0; i < D; ++i) {
      R acc = R(0);
#pragma unroll
      for (int j = 0; j < D; ++j)
        if (jac_entry<Sys>(i, j)) acc = fmaR(Jd[i][j], St.k1[j], acc);
      r[i] = fmaR(hd, acc, F0d[i]);
    }
    solve<R, D, SKIP>(St.w, r, k1d);
#pragma unroll
    for (int c = 0; c < D; ++c) Y1d[c] = fmaR(hh, k1d[c], yd[c]);
    sys.jvp(St.Y1, Y1d, dir[t], F1d);
    // F1d - k1d - Wd u = F1d - k1d + h d Jd u
#pragma unroll
    for (int i = 0; i < D; ++i) {
      R acc = R(0);
#pragma unroll
      for (int j = 0; j < D; ++j)
        if (jac_entry<Sys>(i, j)) acc = fmaR(Jd[i][j], St.u[j], acc);
      r[i] = fmaR(hd, acc, F1d[i] - k1d[i]);
    }
    solve<R, D, SKIP>(St.w, r, ud);
#pragma unroll
    for (int c = 0; c < D; ++c) S[c][t] = fmaR(h, ud[c] + k1d[c], yd[c]);
  }
}

}  // namespace ros23
}  // namespace dao
