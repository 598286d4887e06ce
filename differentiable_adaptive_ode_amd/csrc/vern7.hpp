// Verner 7(6): the ten-stage explicit pair of J. H. Verner's "most efficient"
// seventh-order family (arXiv 2609.02876 lists it among the library's
// engines; the application paper, arXiv 2609.28458, integrates its
// precession ensemble with it).  The seventh-order weights b use stages 1 and
// 4-9, the sixth-order weights bhat stages 1, 4-7 and 10; stage 10 exists for
// the error estimate only, and the pair is not FSAL: f(y_new) is a new
// evaluation after an accepted step.
//
// Per lane, all stage values live in registers.  Stage i (0-based) is
//   Y_i = y + h * (a_i0 k_0 + sum_{j=1}^{i-1} a_ij k_j)   (fma chain, j ascending,
//                                                        zero entries skipped)
//   k_i = f(Y_i)
// y_new = y + h * sum_j b_j k_j and the error estimate (without its factor h)
// sum_j (b_j - bhat_j) k_j.
#pragma once

#include "common.hpp"

namespace dao {
namespace vern7 {

__device__ constexpr double A[10][10] = {
    {0, 0, 0, 0, 0, 0, 0, 0, 0, 0},
    {0.005, 0, 0, 0, 0, 0, 0, 0, 0, 0},
    {-1.07679012345679, 1.185679012345679, 0, 0, 0, 0, 0, 0, 0, 0},
    {0.04083333333333333, 0, 0.1225, 0, 0, 0, 0, 0, 0, 0},
    {0.6389139236255726, 0, -2.455672638223657, 2.272258714598084, 0, 0, 0, 0, 0, 0},
    {-2.6615773750187572, 0, 10.804513886456137, -8.3539146573962, 0.820487594956657, 0, 0, 0,
     0, 0},
    {6.067741434696772, 0, -24.711273635911088, 20.427517930788895, -1.9061579788166472,
     1.006172249242068, 0, 0, 0, 0},
    {12.054670076253203, 0, -49.75478495046899, 41.142888638604674, -4.461760149974004,
     2.042334822239175, -0.09834843665406107, 0, 0, 0},
    {10.138146522881808, 0, -42.6411360317175, 35.76384003992257, -4.3480228403929075,
     2.0098622683770357, 0.3487490460338272, -0.27143900510483127, 0, 0},
    {-45.030072034298676, 0, 187.3272437654589, -154.02882369350186, 18.56465306347536,
     -7.141809679295079, 1.3088085781613787, 0, 0, 0}};
__device__ constexpr double B[10] = {0.04715561848627222, 0, 0, 0.25750564298434153,
                                     0.26216653977412624, 0.15216092656738558,
                                     0.4939969170032485, -0.29430311714032503,
                                     0.08131747232495111, 0};
__device__ constexpr double BH[10] = {0.044608606606341174, 0, 0, 0.26716403785713727,
                                      0.22010183001772932, 0.2188431703143157,
                                      0.22898717054112028, 0, 0, 0.02029518466335628};

// The error weights b - bhat, formed in binary64 like every other coefficient.
__device__ __forceinline__ constexpr double bt(int j) { return B[j] - BH[j]; }

// Stage state Y_i from y and k_0 .. k_{i-1}.
template <class R, int D, int NK>
__device__ __forceinline__ void stage_state(int i, const R (&y)[D], R h, const R (&k)[NK][D],
                                            R (&Y)[D]) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    R acc = R(A[i][0]) * k[0][c];
#pragma unroll
    for (int j = 1; j < 9; ++j)
      if (j < i && A[i][j] != 0.0) acc = fmaR(R(A[i][j]), k[j][c], acc);
    Y[c] = fmaR(h, acc, y[c]);
  }
}

// y_new = y + h sum_j b_j k_j (stages 1, 4-9).
template <class R, int D, int NK>
__device__ __forceinline__ void combine(const R (&y)[D], R h, const R (&k)[NK][D],
                                        R (&ynew)[D]) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    R acc = R(B[0]) * k[0][c];
#pragma unroll
    for (int j = 1; j < 9; ++j)
      if (B[j] != 0.0) acc = fmaR(R(B[j]), k[j][c], acc);
    ynew[c] = fmaR(h, acc, y[c]);
  }
}

// One trial step: k[0] = f(y) on entry; fills k[1..9], ynew and err.
template <class R, class Sys>
__device__ __forceinline__ void trial(const Sys& sys, const R (&y)[Sys::D], R h,
                                      R (&k)[10][Sys::D], R (&ynew)[Sys::D], R (&err)[Sys::D]) {
  constexpr int D = Sys::D;
  R Y[D];
#pragma unroll
  for (int i = 1; i < 9; ++i) {
    stage_state<R, D, 10>(i, y, h, k, Y);
    sys.f(Y, k[i]);
  }
  combine<R, D, 10>(y, h, k, ynew);
  stage_state<R, D, 10>(9, y, h, k, Y);
  sys.f(Y, k[9]);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    R acc = R(bt(0)) * k[0][c];
#pragma unroll
    for (int j = 1; j < 10; ++j)
      if (bt(j) != 0.0) acc = fmaR(R(bt(j)), k[j][c], acc);
    err[c] = acc;  // the embedded error without its factor h (in the error weights)
  }
}

// One replay step y <- Phi(y; h): nine evaluations, no error estimate.
template <class R, class Sys>
__device__ __forceinline__ void replay(const Sys& sys, R (&y)[Sys::D], R h) {
  constexpr int D = Sys::D;
  R k[9][D];
  R Y[D];
  sys.f(y, k[0]);
#pragma unroll
  for (int i = 1; i < 9; ++i) {
    stage_state<R, D, 9>(i, y, h, k, Y);
    sys.f(Y, k[i]);
  }
  combine<R, D, 9>(y, h, k, Y);
#pragma unroll
  for (int c = 0; c < D; ++c) y[c] = Y[c];
}

// Reverse of one replay step (states kept, stages recomputed, as the
// in-kernel adjoint of arXiv 2609.02876 Sec. 3.3 does): `stages` recomputes
// the nine stage states of step j from y_j and h_j; `sweep` takes
// lam = dL/dy_{j+1} to dL/dy_j and adds dL/dtheta into pb.
template <class R, int D>
struct Stages {
  R Y[9][D];  // stage states Y_1 .. Y_9 (Y_1 = y_j)
};

template <class R, class Sys>
__device__ __forceinline__ void stages(const Sys& sys, const R (&y)[Sys::D], R h,
                                       Stages<R, Sys::D>& S) {
  constexpr int D = Sys::D;
  // Each stage's sum is built as the k_j appear, j ascending with the zero
  // entries skipped (the order stage_state uses, so the same bits); each k_j
  // dies once added, so the live set is the open sums plus the stage states
  // kept, not every k_j beside every stage state.
  R acc[9][D];
  R k[D];
#pragma unroll
  for (int c = 0; c < D; ++c) S.Y[0][c] = y[c];
  sys.f(S.Y[0], k);
#pragma unroll
  for (int i = 1; i < 9; ++i)
#pragma unroll
    for (int c = 0; c < D; ++c) acc[i][c] = R(A[i][0]) * k[c];
#pragma unroll
  for (int j = 1; j < 9; ++j) {
#pragma unroll
    for (int c = 0; c < D; ++c) S.Y[j][c] = fmaR(h, acc[j][c], y[c]);
    if (j < 8) {
      sys.f(S.Y[j], k);
#pragma unroll
      for (int i = 2; i < 9; ++i)
        if (i > j && A[i][j] != 0.0) {
#pragma unroll
          for (int c = 0; c < D; ++c) acc[i][c] = fmaR(R(A[i][j]), k[c], acc[i][c]);
        }
    }
  }
}

template <class R, class Sys>
__device__ __forceinline__ void sweep(const Sys& sys, const Stages<R, Sys::D>& S, R h,
                                      R (&lam)[Sys::D], R (&pb)[Sys::P]) {
  constexpr int D = Sys::D;
  // y_new = y + h sum_j b_j k_j and Y_i = y + h sum_{j<i} a_ij k_j, so
  //   kb_i = h b_i lam + sum_{m > i} h a_mi yb_m,  yb_m = (df/dy)(Y_m)^T kb_m,
  // with lam as it was on entry (b_i = 0 for stages 2, 3: the sum alone).
  // kb_i is formed when stage i is reached, from the yb of the stages already
  // swept, added m = 8, 7, ..., i + 1 (the order in which each would be
  // pushed into it; the same bits): only the yb of swept stages are live.
  R lam0[D];
#pragma unroll
  for (int c = 0; c < D; ++c) lam0[c] = lam[c];
  R yb[9][D];
#pragma unroll
  for (int i = 8; i >= 0; --i) {
    R kb[D];
    const R hb = h * R(B[i]);
#pragma unroll
    for (int c = 0; c < D; ++c) kb[c] = (B[i] != 0.0) ? hb * lam0[c] : R(0);
#pragma unroll
    for (int m = 8; m > 0; --m)
      if (m > i && i < 8 && A[m][i] != 0.0) {
        const R ha = h * R(A[m][i]);
#pragma unroll
        for (int c = 0; c < D; ++c) kb[c] = fmaR(ha, yb[m][c], kb[c]);
      }
    sys.vjp(S.Y[i], kb, yb[i], pb);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] += yb[i][c];
  }
}

}  // namespace vern7
}  // namespace dao
