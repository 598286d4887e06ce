// Tsit5: the Tsitouras 5(4) explicit pair with 7 stages and FSAL
// (arXiv 2609.02876 Sec. 2.1 names it as the default non-stiff method; the
// coefficients are the published ones, Tsitouras 2011, Table 1).
//
// Per lane, all stage values live in registers.  Stage i (0-based) is
//   Y_i = y + h * (a_i0 k_0 + sum_{j=1}^{i-1} a_ij k_j)        (fma chain, j ascending)
//   k_i = f(Y_i)
// and y_new = Y_6 (the weights b equal the last row of A).  The error estimate
// is e = h * (bt_0 k_0 + sum_{j=1}^{6} bt_j k_j) with bt = b - bhat.
#pragma once

#include "common.hpp"

namespace dao {
namespace tsit5 {

__device__ constexpr double A10 = 0.161;
__device__ constexpr double A20 = -0.008480655492356989, A21 = 0.335480655492357;
__device__ constexpr double A30 = 2.897153057105493, A31 = -6.359448489975075,
                            A32 = 4.3622954328695815;
__device__ constexpr double A40 = 5.325864828439257, A41 = -11.748883564062828,
                            A42 = 7.4955393428898365, A43 = -0.09249506636175525;
__device__ constexpr double A50 = 5.86145544294642, A51 = -12.92096931784711,
                            A52 = 8.159367898576159, A53 = -0.071584973281401,
                            A54 = -0.028269050394068383;
__device__ constexpr double A60 = 0.09646076681806523, A61 = 0.01, A62 = 0.4798896504144996,
                            A63 = 1.379008574103742, A64 = -3.290069515436081,
                            A65 = 2.324710524099774;
__device__ constexpr double E0 = -0.00178001105222577714, E1 = -0.0008164344596567469,
                            E2 = 0.007880878010261995, E3 = -0.1447110071732629,
                            E4 = 0.5823571654525552, E5 = -0.45808210592918697,
                            E6 = 0.015151515151515152;

// Coefficient lookup with compile-time indices (the stage loops below are
// fully unrolled, so every access resolves to a literal).
template <class R>
__device__ __forceinline__ constexpr R a(int i, int j) {
  return R(i == 1 ? A10
         : i == 2 ? (j == 0 ? A20 : A21)
         : i == 3 ? (j == 0 ? A30 : j == 1 ? A31 : A32)
         : i == 4 ? (j == 0 ? A40 : j == 1 ? A41 : j == 2 ? A42 : A43)
         : i == 5 ? (j == 0 ? A50 : j == 1 ? A51 : j == 2 ? A52 : j == 3 ? A53 : A54)
                  : (j == 0 ? A60 : j == 1 ? A61 : j == 2 ? A62 : j == 3 ? A63 : j == 4 ? A64 : A65));
}
template <class R>
__device__ __forceinline__ constexpr R e(int j) {
  return R(j == 0 ? E0 : j == 1 ? E1 : j == 2 ? E2 : j == 3 ? E3 : j == 4 ? E4 : j == 5 ? E5 : E6);
}

// The coefficients as values held in registers for a whole kernel.  As plain
// literals every binary64 coefficient is rebuilt from two scalar moves at each
// use; pinning them to vector registers once (an empty asm that claims to
// modify the value keeps the compiler from re-materialising the literal)
// removes those moves from the step loops.
template <class R>
__device__ __forceinline__ R pin(R v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <class R>
struct Coef {
  R a[7][6];  // a[i][j], j < i
  R e[7];     // error weights b - bhat
  __device__ __forceinline__ static Coef pinned() {
    Coef C;
#pragma unroll
    for (int i = 1; i < 7; ++i)
#pragma unroll
      for (int j = 0; j < 6; ++j)
        if (j < i) C.a[i][j] = pin(tsit5::a<R>(i, j));
#pragma unroll
    for (int j = 0; j < 7; ++j) C.e[j] = pin(tsit5::e<R>(j));
    return C;
  }
  __device__ __forceinline__ static Coef literal() {
    Coef C;
#pragma unroll
    for (int i = 1; i < 7; ++i)
#pragma unroll
      for (int j = 0; j < 6; ++j)
        if (j < i) C.a[i][j] = tsit5::a<R>(i, j);
#pragma unroll
    for (int j = 0; j < 7; ++j) C.e[j] = tsit5::e<R>(j);
    return C;
  }
};

// Stage state Y_i from y and k_0..k_{i-1}.
template <class R, int D>
__device__ __forceinline__ void stage_state(const Coef<R>& C, int i, const R (&y)[D], R h,
                                            const R (&k)[7][D], R (&Y)[D]) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    R acc = C.a[i][0] * k[0][c];
#pragma unroll
    for (int j = 1; j < 6; ++j)
      if (j < i) acc = fmaR(C.a[i][j], k[j][c], acc);
    Y[c] = fmaR(h, acc, y[c]);
  }
}

// One trial step: k[0] = f(y) on entry; fills k[1..6], ynew and err.
template <class R, class Sys>
__device__ __forceinline__ void trial(const Coef<R>& C, const Sys& sys, const R (&y)[Sys::D], R h,
                                      R (&k)[7][Sys::D], R (&ynew)[Sys::D], R (&err)[Sys::D]) {
  constexpr int D = Sys::D;
  R Y[D];
#pragma unroll
  for (int i = 1; i < 7; ++i) {
    stage_state<R, D>(C, i, y, h, k, Y);
    sys.f(Y, k[i]);
  }
#pragma unroll
  for (int c = 0; c < D; ++c) ynew[c] = Y[c];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    R acc = C.e[0] * k[0][c];
#pragma unroll
    for (int j = 1; j < 7; ++j) acc = fmaR(C.e[j], k[j][c], acc);
    err[c] = acc;  // the embedded error without its factor h (in the error weights)
  }
}

// One replay step y <- Phi(y; h): six evaluations, no error estimate.
template <class R, class Sys>
__device__ __forceinline__ void replay(const Coef<R>& C, const Sys& sys, R (&y)[Sys::D], R h) {
  constexpr int D = Sys::D;
  R k[7][D];
  R Y[D];
  sys.f(y, k[0]);
#pragma unroll
  for (int i = 1; i < 6; ++i) {
    stage_state<R, D>(C, i, y, h, k, Y);
    sys.f(Y, k[i]);
  }
  stage_state<R, D>(C, 6, y, h, k, Y);
#pragma unroll
  for (int c = 0; c < D; ++c) y[c] = Y[c];
}

// Forward sensitivities through one step (arXiv 2609.28458 Sec. 2.3: the
// sensitivity equations integrated beside the state with the state's own
// steps; with the steps held fixed this is the exact tangent of the step).
// On entry S[c][t] = dy_c/dp_t for NT directions, direction t being the
// parameter dir[t] (or none, for an initial-state direction: dir[t] < 0 or
// >= P); k[0..5] are the step's stage derivatives at (y, h).  On exit S holds
// the tangent of y_new.  Stage tangents: Yd_i = S + h sum_j a_ij K_j,
// K_i = (df/dy)(Y_i) Yd_i + df/dtheta_dir(Y_i).
template <class R, class Sys, int NT>
__device__ __forceinline__ void tangent(const Coef<R>& C, const Sys& sys, const R (&y)[Sys::D],
                                        R h, const R (&k)[7][Sys::D], const int (&dir)[NT],
                                        R (&S)[Sys::D][NT]) {
  constexpr int D = Sys::D;
  R K[6][NT][D];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    R Y[D];
    if (i == 0) {
#pragma unroll
      for (int c = 0; c < D; ++c) Y[c] = y[c];
    } else {
      stage_state<R, D>(C, i, y, h, k, Y);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      R Yd[D];
#pragma unroll
      for (int c = 0; c < D; ++c) {
        if (i == 0) {
          Yd[c] = S[c][t];
        } else {
          R acc = C.a[i][0] * K[0][t][c];
#pragma unroll
          for (int j = 1; j < 5; ++j)
            if (j < i) acc = fmaR(C.a[i][j], K[j][t][c], acc);
          Yd[c] = fmaR(h, acc, S[c][t]);
        }
      }
      sys.jvp(Y, Yd, dir[t], K[i][t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < D; ++c) {
      R acc = C.a[6][0] * K[0][t][c];
#pragma unroll
      for (int j = 1; j < 6; ++j) acc = fmaR(C.a[6][j], K[j][t][c], acc);
      S[c][t] = fmaR(h, acc, S[c][t]);
    }
}

// Reverse of one replay step, in two parts.  The stage states depend only
// on y_j and h_j (store-the-state, recompute-the-stages, as the in-kernel
// adjoint of Sec. 3.3 does); the sweep takes lam = dL/dy_{j+1} to
// lam = dL/dy_j and accumulates dL/dtheta into pb.  Keeping them apart lets a
// caller recompute one step's stages while it sweeps back through another.
template <class R, int D>
struct Stages {
  R Y[6][D];  // stage states Y_1 .. Y_6 (Y_1 = y_j)
};

template <class R, class Sys>
__device__ __forceinline__ void stages(const Coef<R>& C, const Sys& sys, const R (&y)[Sys::D], R h,
                                       Stages<R, Sys::D>& S) {
  constexpr int D = Sys::D;
  // Each stage's sum is built as the k_j appear, j ascending, and each k_j
  // dies as soon as it is added: the live set is the sums still open plus
  // the stage states kept, not every k_j beside every stage state.  From
  // d = 3 on the sums are y + sum_j (h a_ij) k_j: one product h a_ij per
  // coupling instead of a product per component, and Y_i is the sum itself,
  // one multiply-add earlier.  The stage states then round differently from
  // the solve's (y + h sum_j a_ij k_j); they only feed the stage VJPs, and the
  // step's y_j and y_{j+1} stay the replay's.
  constexpr bool HA = D >= 3;
  R acc[6][D];
  R k[D];
#pragma unroll
  for (int c = 0; c < D; ++c) S.Y[0][c] = y[c];
  sys.f(S.Y[0], k);
#pragma unroll
  for (int i = 1; i < 6; ++i) {
    const R ha = h * C.a[i][0];
#pragma unroll
    for (int c = 0; c < D; ++c) acc[i][c] = HA ? fmaR(ha, k[c], y[c]) : C.a[i][0] * k[c];
  }
#pragma unroll
  for (int j = 1; j < 6; ++j) {
#pragma unroll
    for (int c = 0; c < D; ++c) S.Y[j][c] = HA ? acc[j][c] : fmaR(h, acc[j][c], y[c]);
    if (j < 5) {
      sys.f(S.Y[j], k);
#pragma unroll
      for (int i = 2; i < 6; ++i)
        if (i > j) {
          const R a = HA ? h * C.a[i][j] : C.a[i][j];
#pragma unroll
          for (int c = 0; c < D; ++c) acc[i][c] = fmaR(a, k[c], acc[i][c]);
        }
    }
  }
}

template <class R, class Sys>
__device__ __forceinline__ void sweep(const Coef<R>& C, const Sys& sys, const Stages<R, Sys::D>& S,
                                      R h, R (&lam)[Sys::D], R (&pb)[Sys::P]) {
  constexpr int D = Sys::D;
  // y_new = y + h sum_j b_j k_j (b_j = a(6, j)) and Y_i = y + h sum_{j<i} a_ij k_j,
  // so the cotangent of k_i is
  //   kb_i = h b_i lam + sum_{m > i} h a_mi yb_m,  yb_m = (df/dy)(Y_m)^T kb_m,
  // with lam = dL/dy_{j+1} as it was on entry.  kb_i is formed when stage i
  // is reached, from the yb of the stages already swept, added m = 5, 4, ...,
  // i + 1 (the order in which each would be pushed into it as it appears;
  // the same bits): only the yb of swept stages are live, not an open
  // cotangent for every stage.
  R lam0[D];
#pragma unroll
  for (int c = 0; c < D; ++c) lam0[c] = lam[c];
  R yb[6][D];
#pragma unroll
  for (int i = 5; i >= 0; --i) {
    R kb[D];
    const R hb = h * C.a[6][i];
#pragma unroll
    for (int c = 0; c < D; ++c) kb[c] = hb * lam0[c];
#pragma unroll
    for (int m = 5; m > 0; --m)
      if (m > i) {
        const R ha = h * C.a[m][i];
#pragma unroll
        for (int c = 0; c < D; ++c) kb[c] = fmaR(ha, yb[m][c], kb[c]);
      }
    sys.vjp(S.Y[i], kb, yb[i], pb);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] += yb[i][c];
  }
}

}  // namespace tsit5
}  // namespace dao
