// Rodas5P: G. Steinebach's eight-stage, stiffly accurate, L-stable
// Rosenbrock-Wanner method of order 5 with an embedded order-4 solution
// (arXiv 2609.02876 Sec. 3.1 names it as the library's general stiff engine;
// Sec. 3.2 gives the stage structure: one factorisation, one linear solve per
// stage, transposed solves in the adjoint).  With W = I/(gamma h) - J(y):
//
//   W u_i = f(Y_i) + (1/h) sum_{j<i} C_ij u_j          (i = 1..8, Y_1 = y)
//   Y_i   = y + sum_{j<i} a_ij u_j                      (i = 2..6)
//   Y_7   = Y_6 + u_6,   Y_8 = Y_7 + u_7,   y_new = Y_8 + u_8,
//
// and the error estimate is u_8 (y_new minus the embedded solution Y_8).  The
// systems are autonomous, so the method's df/dt terms vanish.  A zero-size
// step (the padding of a lockstep group, or a requested time on a step
// boundary) is the identity, the step map's limit as h -> 0; it is applied
// by selects because W and the stage sums carry 1/h.  The LU factorisation
// and the (transposed) solves are those of Rosenbrock23.
#pragma once

#include "common.hpp"
#include "ros23.hpp"

namespace dao {
namespace rodas5p {

__device__ constexpr double GAMMA = 0.21193756319429014;
__device__ constexpr double A[6][6] = {
    {0, 0, 0, 0, 0, 0},
    {3.0, 0, 0, 0, 0, 0},
    {2.849394379747939, 0.45842242204463923, 0, 0, 0, 0},
    {-6.954028509809101, 2.489845061869568, -10.358996098473584, 0, 0, 0},
    {2.8029986275628964, 0.5072464736228206, -0.3988312541770524, -0.04721187230404641, 0, 0},
    {-7.502846399306121, 2.561846144803919, -11.627539656261098, -0.18268767659942256,
     0.030198172008377946, 0}};
__device__ constexpr double C[8][8] = {
    {0, 0, 0, 0, 0, 0, 0, 0},
    {-14.155112264123755, 0, 0, 0, 0, 0, 0, 0},
    {-17.97296035885952, -2.859693295451294, 0, 0, 0, 0, 0, 0},
    {147.12150275711716, -1.41221402718213, 71.68940251302358, 0, 0, 0, 0, 0},
    {165.43517024871676, -0.4592823456491126, 42.90938336958603, -5.961986721573306, 0, 0, 0, 0},
    {24.854864614690072, -3.0009227002832186, 47.4931110020768, 5.5814197821558125,
     -0.6610691825249471, 0, 0, 0},
    {30.91273214028599, -3.1208243349937974, 77.79954646070892, 34.28646028294783,
     -19.097331116725623, -28.087943162872662, 0, 0},
    {37.80277123390563, -3.2571969029072276, 112.26918849496327, 66.9347231244047,
     -40.06618937091002, -54.66780262877968, -9.48861652309627, 0}};

// Everything of one step that depends only on (y, h): the factors of W, the
// stage states and the stage solutions.
template <class R, int D>
struct Stages {
  ros23::LU<R, D> w;
  R Y[8][D];  // Y_1 = y .. Y_8
  R u[8][D];
};

// The step's quantities from y, h and F0 = f(y); h must be nonzero.
template <class R, class Sys, bool SKIP = true>
__device__ __forceinline__ void run(const Sys& sys, const R (&y)[Sys::D], R h,
                                    const R (&F0)[Sys::D], Stages<R, Sys::D>& S) {
  constexpr int D = Sys::D;
  R J[D][D];
  sys.jac(y, J);
  const R ginv = recipR(R(GAMMA) * h);
  const R hinv = recipR(h);
#pragma unroll
  for (int i = 0; i < D; ++i)
#pragma unroll
    for (int j = 0; j < D; ++j) S.w.m[i][j] = (i == j) ? ginv - J[i][j] : -J[i][j];
  ros23::factor<R, D, SKIP, Sys>(S.w);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    R r[D];
    if (i == 0) {
#pragma unroll
      for (int c = 0; c < D; ++c) {
        S.Y[0][c] = y[c];
        r[c] = F0[c];
      }
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) {
        if (i <= 5) {
          R acc = R(A[i][0]) * S.u[0][c];
#pragma unroll
          for (int j = 1; j < 5; ++j)
            if (j < i) acc = fmaR(R(A[i][j]), S.u[j][c], acc);
          S.Y[i][c] = acc + y[c];
        } else {
          S.Y[i][c] = S.Y[i - 1][c] + S.u[i - 1][c];
        }
      }
      R F[D];
      sys.f(S.Y[i], F);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        R acc = R(C[i][0]) * S.u[0][c];
#pragma unroll
        for (int j = 1; j < 7; ++j)
          if (j < i) acc = fmaR(R(C[i][j]), S.u[j][c], acc);
        r[c] = fmaR(acc, hinv, F[c]);
      }
    }
    ros23::solve<R, D, SKIP, Sys>(S.w, r, S.u[i]);
  }
}

// Trial step: F0 = f(y) on entry; returns ynew and err = u_8.
template <class R, class Sys, bool SKIP = true>
__device__ __forceinline__ void trial(const Sys& sys, const R (&y)[Sys::D], R h,
                                      const R (&F0)[Sys::D], R (&ynew)[Sys::D],
                                      R (&err)[Sys::D]) {
  constexpr int D = Sys::D;
  Stages<R, D> S;
  run<R, Sys, SKIP>(sys, y, h, F0, S);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    ynew[c] = S.Y[7][c] + S.u[7][c];
    err[c] = S.u[7][c];
  }
}

// Replay step y <- Phi(y; h); a zero-size step leaves y as it is.
template <class R, class Sys>
__device__ __forceinline__ void replay(const Sys& sys, R (&y)[Sys::D], R h) {
  constexpr int D = Sys::D;
  const bool zero = (h == R(0));
  const R hs = zero ? R(1) : h;
  R F0[D];
  sys.f(y, F0);
  Stages<R, D> S;
  run<R, Sys>(sys, y, hs, F0, S);
#pragma unroll
  for (int c = 0; c < D; ++c) y[c] = zero ? y[c] : S.Y[7][c] + S.u[7][c];
}

template <class R, class Sys>
__device__ __forceinline__ void stages(const Sys& sys, const R (&y)[Sys::D], R h,
                                       Stages<R, Sys::D>& S) {
  constexpr int D = Sys::D;
  const R hs = (h == R(0)) ? R(1) : h;
  R F0[D];
  sys.f(y, F0);
  run<R, Sys>(sys, y, hs, F0, S);
}

// Reverse of one replay step: lam = dL/dy_new -> dL/dy, dL/dtheta added into
// pb.  Stage i's solve u_i = W^-1 r_i sends rb = W^-T ub_i to f(Y_i), to the
// earlier stages through (1/h) C_ij, and -rb u_i^T to W, i.e. +rb u_i^T to
// J(y, theta), pulled back once through the Jacobian's own derivatives.
template <class R, class Sys>
__device__ __forceinline__ void sweep(const Sys& sys, const Stages<R, Sys::D>& S, R h,
                                      R (&lam)[Sys::D], R (&pb)[Sys::P]) {
  constexpr int D = Sys::D, P = Sys::P;
  const bool zero = (h == R(0));
  const R hinv = recipR(zero ? R(1) : h);
  R ub[8][D], yb[D], Yb[D], Jb[D][D], pt[P];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    ub[7][c] = lam[c];  // y_new = Y_8 + u_8
    Yb[c] = lam[c];
    yb[c] = R(0);
  }
#pragma unroll
  for (int i = 0; i < 7; ++i)
#pragma unroll
    for (int c = 0; c < D; ++c) ub[i][c] = R(0);
#pragma unroll
  for (int a = 0; a < D; ++a)
#pragma unroll
    for (int b = 0; b < D; ++b) Jb[a][b] = R(0);
#pragma unroll
  for (int j = 0; j < P; ++j) pt[j] = R(0);
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    R rb[D], tmp[D];
    ros23::solve_t<R, D, true, Sys>(S.w, ub[i], rb);
#pragma unroll
    for (int a = 0; a < D; ++a)
#pragma unroll
      for (int b = 0; b < D; ++b) Jb[a][b] = fmaR(rb[a], S.u[i][b], Jb[a][b]);
    sys.vjp(S.Y[i], rb, tmp, pt);
    if (i == 0) {
#pragma unroll
      for (int c = 0; c < D; ++c) yb[c] += tmp[c];
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) Yb[c] += tmp[c];
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        if (j < i) {
          const R ch = R(C[i][j]) * hinv;
#pragma unroll
          for (int c = 0; c < D; ++c) ub[j][c] = fmaR(ch, rb[c], ub[j][c]);
        }
      }
      if (i >= 6) {
        // Y_i = Y_{i-1} + u_{i-1}: Yb carries on as the cotangent of Y_{i-1}
#pragma unroll
        for (int c = 0; c < D; ++c) ub[i - 1][c] += Yb[c];
      } else {
        // Y_i = y + sum_j a_ij u_j
#pragma unroll
        for (int c = 0; c < D; ++c) yb[c] += Yb[c];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          if (j < i) {
#pragma unroll
            for (int c = 0; c < D; ++c) ub[j][c] = fmaR(R(A[i][j]), Yb[c], ub[j][c]);
          }
        }
#pragma unroll
        for (int c = 0; c < D; ++c) Yb[c] = R(0);
      }
    }
  }
  sys.jac_vjp(S.Y[0], Jb, yb, pt);
  // a zero-size step is the identity: lam and pb pass unchanged
#pragma unroll
  for (int c = 0; c < D; ++c) lam[c] = zero ? lam[c] : yb[c];
#pragma unroll
  for (int j = 0; j < P; ++j) pb[j] += zero ? R(0) : pt[j];
}

// The same reverse step with the stage solutions in LDS, for systems whose
// step does not fit the registers (d = 8: the factors, the stage solutions,
// the stage states and the stage cotangents together are ~400 doubles).  us
// points at this lane's element of the wavefront's area [8][D][64]: u_i,c at
// us[(i D + c) 64].  The stage states are recomputed from y and the u_j with
// the operations run() used, so every value is run()'s own.  Each stage's
// loads are tied to that stage's incoming cotangent through an empty asm
// statement: without it the compiler issues every stage's loads and
// recomputed states at the top of the step and holds them all in registers.
// Its transposed solves run their row exchanges as selects (SKIP = false):
// the compiler barrier on the skip branches pins the loads around it, and
// the reverse step then spilled 630 registers and ran 3.8x slower.  The Jacobian cotangent
// rb u_i^T is pulled back stage by stage (the pull-back is linear), so only
// the entries the pull-back reads are ever formed.
template <class R, int D>
__device__ __forceinline__ void put_stages(const Stages<R, D>& S, R* us) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < D; ++c) us[(i * D + c) * WAVE] = S.u[i][c];
}

template <class R, class Sys>
__device__ __forceinline__ void sweep_lds(const Sys& sys, const ros23::LU<R, Sys::D>& w,
                                          const R (&y)[Sys::D], R h, const R* us_,
                                          R (&lam)[Sys::D], R (&pb)[Sys::P]) {
  constexpr int D = Sys::D, P = Sys::P;
  const R* us = us_;
  int dep = 0;  // always 0; the asm below makes it depend on the cotangent
  auto u = [&](int i, int c) -> R { return us[(i * D + c) * WAVE + dep]; };
  const bool zero = (h == R(0));
  const R hinv = recipR(zero ? R(1) : h);
  // stage state Y_i as run() forms it (Y_6 = Y_5 + u_5, Y_7 = Y_6 + u_6)
  auto stage_y = [&](int i, R (&Yi)[D]) {
#pragma unroll
    for (int c = 0; c < D; ++c) {
      const int i5 = i < 5 ? i : 5;
      R v = y[c];
      if (i5 > 0) {
        R acc = R(A[i5][0]) * u(0, c);
#pragma unroll
        for (int j = 1; j < 5; ++j)
          if (j < i5) acc = fmaR(R(A[i5][j]), u(j, c), acc);
        v = acc + y[c];
      }
      if (i >= 6) v = v + u(5, c);
      if (i >= 7) v = v + u(6, c);
      Yi[c] = v;
    }
  };
  R ub[8][D], yb[D], Yb[D], pt[P];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    ub[7][c] = lam[c];
    Yb[c] = lam[c];
    yb[c] = R(0);
  }
#pragma unroll
  for (int i = 0; i < 7; ++i)
#pragma unroll
    for (int c = 0; c < D; ++c) ub[i][c] = R(0);
#pragma unroll
  for (int j = 0; j < P; ++j) pt[j] = R(0);
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    // stage i's loads and recomputed state wait for ub_i to be complete
    asm volatile("" : "+v"(dep) : "v"(ub[i][0]));
    R Yi[D], rb[D], tmp[D];
    stage_y(i, Yi);
    ros23::solve_t<R, D, false>(w, ub[i], rb);
    {
      // W's cotangent -rb u_i^T is +rb u_i^T on J(y, theta), pulled back at
      // once (the pull-back is linear; only the entries it reads are formed)
      R ui[D], Jo[D][D];
#pragma unroll
      for (int b = 0; b < D; ++b) ui[b] = u(i, b);
#pragma unroll
      for (int a = 0; a < D; ++a)
#pragma unroll
        for (int b = 0; b < D; ++b) Jo[a][b] = rb[a] * ui[b];
      sys.jac_vjp(y, Jo, yb, pt);
    }
    sys.vjp(Yi, rb, tmp, pt);
    if (i == 0) {
#pragma unroll
      for (int c = 0; c < D; ++c) yb[c] += tmp[c];
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) Yb[c] += tmp[c];
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        if (j < i) {
          const R ch = R(C[i][j]) * hinv;
#pragma unroll
          for (int c = 0; c < D; ++c) ub[j][c] = fmaR(ch, rb[c], ub[j][c]);
        }
      }
      if (i >= 6) {
#pragma unroll
        for (int c = 0; c < D; ++c) ub[i - 1][c] += Yb[c];
      } else {
#pragma unroll
        for (int c = 0; c < D; ++c) yb[c] += Yb[c];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          if (j < i) {
#pragma unroll
            for (int c = 0; c < D; ++c) ub[j][c] = fmaR(R(A[i][j]), Yb[c], ub[j][c]);
          }
        }
#pragma unroll
        for (int c = 0; c < D; ++c) Yb[c] = R(0);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < D; ++c) lam[c] = zero ? lam[c] : yb[c];
#pragma unroll
  for (int j = 0; j < P; ++j) pb[j] += zero ? R(0) : pt[j];
}

}  // namespace rodas5p
}  // namespace dao
