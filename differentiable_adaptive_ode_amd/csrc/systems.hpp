// Built-in right-hand sides for the per-lane kernels.
//
// Every system exposes, for one trajectory held in one lane's registers:
//   load(theta, n, k)      gather the trajectory's parameters from SoA theta[p][n]
//                          and precompute per-trajectory constants
//   f(y, dy)               the field, with the rounding contract of the solve
//   vjp(y, v, yb, pb)      yb = (df/dy)^T v ;  pb += (df/dtheta)^T v
//   jac(y, J)              J = df/dy (Rosenbrock stages)
//   jac_vjp(y, Jb, yb, pb) yb += d/dy <Jb, J(y,theta)> ; pb += d/dtheta <Jb, J>
//                          (the Jacobian's own dependence, needed by the
//                          Rosenbrock adjoint; arXiv 2609.02876 Sec. 3.2 notes
//                          the backward sweep differentiates through J)
//   jvp(y, yd, j, fd)      fd = (df/dy) yd + df/dtheta_j (no parameter term for
//                          j outside [0, P)): one column of the sensitivity
//                          equations S' = (df/dy) S + df/dtheta (arXiv
//                          2609.28458 Sec. 2.3)
//   jac_jvp(y, yd, j, Jd)  Jd = d/de J(y + e yd, theta + e e_j) at e = 0: the
//                          tangent of the Jacobian, which the tangent of a
//                          Rosenbrock step needs (W = I - gamma h J moves too)
// The vector-Jacobian products are derived by hand from the formulas below.
#pragma once

#include "common.hpp"

namespace dao {

// y' = -theta y.
template <class R>
struct Decay {
  static constexpr int D = 1, P = 1;
  R th;
  __device__ void load(const R* theta, int64_t n, int64_t k) { (void)n; th = theta[k]; }
  __device__ void f(const R (&y)[D], R (&dy)[D]) const { dy[0] = -(th * y[0]); }
  __device__ void vjp(const R (&y)[D], const R (&v)[D], R (&yb)[D], R (&pb)[P]) const {
    yb[0] = -th * v[0];
    pb[0] = fmaR(-y[0], v[0], pb[0]);
  }
  __device__ void jac(const R (&y)[D], R (&J)[D][D]) const { (void)y; J[0][0] = -th; }
  __device__ void jac_vjp(const R (&y)[D], const R (&Jb)[D][D], R (&yb)[D], R (&pb)[P]) const {
    (void)y; (void)yb;
    pb[0] -= Jb[0][0];
  }
  __device__ void jvp(const R (&y)[D], const R (&yd)[D], int j, R (&fd)[D]) const {
    fd[0] = (j == 0) ? -fmaR(th, yd[0], y[0]) : -(th * yd[0]);
  }
  __device__ void jac_jvp(const R (&y)[D], const R (&yd)[D], int j, R (&Jd)[D][D]) const {
    (void)y; (void)yd;
    Jd[0][0] = (j == 0) ? R(-1) : R(0);
  }
};

// Lotka-Volterra, theta = (a, b, g, d): y1' = y1 (a - b y2), y2' = y2 (d y1 - g).
template <class R>
struct LotkaVolterra {
  static constexpr int D = 2, P = 4;
  R a, b, g, d;
  __device__ void load(const R* theta, int64_t n, int64_t k) {
    a = theta[k]; b = theta[n + k]; g = theta[2 * n + k]; d = theta[3 * n + k];
  }
  __device__ void f(const R (&y)[D], R (&dy)[D]) const {
    dy[0] = y[0] * fmaR(-b, y[1], a);
    dy[1] = y[1] * fmaR(d, y[0], -g);
  }
  __device__ void vjp(const R (&y)[D], const R (&v)[D], R (&yb)[D], R (&pb)[P]) const {
    R j11 = fmaR(-b, y[1], a), j22 = fmaR(d, y[0], -g);
    yb[0] = fmaR(j11, v[0], (d * y[1]) * v[1]);
    yb[1] = fmaR(j22, v[1], -(b * y[0]) * v[0]);
    R y12 = y[0] * y[1];
    pb[0] = fmaR(y[0], v[0], pb[0]);
    pb[1] = fmaR(-y12, v[0], pb[1]);
    pb[2] = fmaR(-y[1], v[1], pb[2]);
    pb[3] = fmaR(y12, v[1], pb[3]);
  }
  __device__ void jac(const R (&y)[D], R (&J)[D][D]) const {
    J[0][0] = fmaR(-b, y[1], a);
    J[0][1] = -(b * y[0]);
    J[1][0] = d * y[1];
    J[1][1] = fmaR(d, y[0], -g);
  }
  __device__ void jac_vjp(const R (&y)[D], const R (&Jb)[D][D], R (&yb)[D], R (&pb)[P]) const {
    yb[0] += fmaR(d, Jb[1][1], -b * Jb[0][1]);
    yb[1] += fmaR(d, Jb[1][0], -b * Jb[0][0]);
    pb[0] += Jb[0][0];
    pb[1] -= fmaR(y[1], Jb[0][0], y[0] * Jb[0][1]);
    pb[2] -= Jb[1][1];
    pb[3] += fmaR(y[1], Jb[1][0], y[0] * Jb[1][1]);
  }
  __device__ void jvp(const R (&y)[D], const R (&yd)[D], int j, R (&fd)[D]) const {
    const R y12 = y[0] * y[1];
    R p0 = (j == 0) ? y[0] : (j == 1) ? -y12 : R(0);
    R p1 = (j == 2) ? -y[1] : (j == 3) ? y12 : R(0);
    fd[0] = fmaR(fmaR(-b, y[1], a), yd[0], fmaR(-(b * y[0]), yd[1], p0));
    fd[1] = fmaR(d * y[1], yd[0], fmaR(fmaR(d, y[0], -g), yd[1], p1));
  }
  __device__ void jac_jvp(const R (&y)[D], const R (&yd)[D], int j, R (&Jd)[D][D]) const {
    const R ad = (j == 0) ? R(1) : R(0), bd = (j == 1) ? R(1) : R(0);
    const R gd = (j == 2) ? R(1) : R(0), dd = (j == 3) ? R(1) : R(0);
    Jd[0][0] = ad - fmaR(bd, y[1], b * yd[1]);
    Jd[0][1] = -fmaR(bd, y[0], b * yd[0]);
    Jd[1][0] = fmaR(dd, y[1], d * yd[1]);
    Jd[1][1] = fmaR(dd, y[0], d * yd[0]) - gd;
  }
};

// Lorenz-63, theta = (sigma, rho, beta).
template <class R>
struct Lorenz63 {
  static constexpr int D = 3, P = 3;
  R s, r, b;
  __device__ void load(const R* theta, int64_t n, int64_t k) {
    s = theta[k]; r = theta[n + k]; b = theta[2 * n + k];
  }
  __device__ void f(const R (&y)[D], R (&dy)[D]) const {
    dy[0] = s * (y[1] - y[0]);
    dy[1] = fmaR(y[0], r - y[2], -y[1]);
    dy[2] = fmaR(y[0], y[1], -(b * y[2]));
  }
  __device__ void vjp(const R (&y)[D], const R (&v)[D], R (&yb)[D], R (&pb)[P]) const {
    R sv = s * v[0];
    yb[0] = fmaR(r - y[2], v[1], fmaR(y[1], v[2], -sv));
    yb[1] = fmaR(y[0], v[2], sv - v[1]);
    yb[2] = -fmaR(y[0], v[1], b * v[2]);
    pb[0] = fmaR(y[1] - y[0], v[0], pb[0]);
    pb[1] = fmaR(y[0], v[1], pb[1]);
    pb[2] = fmaR(-y[2], v[2], pb[2]);
  }
  __device__ void jac(const R (&y)[D], R (&J)[D][D]) const {
    J[0][0] = -s; J[0][1] = s; J[0][2] = R(0);
    J[1][0] = r - y[2]; J[1][1] = R(-1); J[1][2] = -y[0];
    J[2][0] = y[1]; J[2][1] = y[0]; J[2][2] = -b;
  }
  __device__ void jac_vjp(const R (&y)[D], const R (&Jb)[D][D], R (&yb)[D], R (&pb)[P]) const {
    (void)y;
    yb[0] += Jb[2][1] - Jb[1][2];
    yb[1] += Jb[2][0];
    yb[2] -= Jb[1][0];
    pb[0] += Jb[0][1] - Jb[0][0];
    pb[1] += Jb[1][0];
    pb[2] -= Jb[2][2];
  }
  __device__ void jvp(const R (&y)[D], const R (&yd)[D], int j, R (&fd)[D]) const {
    const R d10 = yd[1] - yd[0];
    fd[0] = (j == 0) ? fmaR(s, d10, y[1] - y[0]) : s * d10;
    fd[1] = fmaR(r - y[2], yd[0], fmaR(-y[0], yd[2], (j == 1) ? y[0] - yd[1] : -yd[1]));
    fd[2] = fmaR(y[1], yd[0], fmaR(y[0], yd[1], -fmaR(b, yd[2], (j == 2) ? y[2] : R(0))));
  }
  __device__ void jac_jvp(const R (&y)[D], const R (&yd)[D], int j, R (&Jd)[D][D]) const {
    (void)y;
    const R sd = (j == 0) ? R(1) : R(0), rd = (j == 1) ? R(1) : R(0), bd = (j == 2) ? R(1) : R(0);
    Jd[0][0] = -sd; Jd[0][1] = sd; Jd[0][2] = R(0);
    Jd[1][0] = rd - yd[2]; Jd[1][1] = R(0); Jd[1][2] = -yd[0];
    Jd[2][0] = yd[1]; Jd[2][1] = yd[0]; Jd[2][2] = -bd;
  }
};

// Robertson kinetics, theta = (k1, k2, k3):
//   y1' = -k1 y1 + k3 y2 y3,  y2' = k1 y1 - k2 y2^2 - k3 y2 y3,  y3' = k2 y2^2.
template <class R>
struct Robertson {
  static constexpr int D = 3, P = 3;
  R k1, k2, k3;
  __device__ void load(const R* theta, int64_t n, int64_t k) {
    k1 = theta[k]; k2 = theta[n + k]; k3 = theta[2 * n + k];
  }
  __device__ void f(const R (&y)[D], R (&dy)[D]) const {
    R a = k1 * y[0];
    R b = k2 * (y[1] * y[1]);
    R c = k3 * (y[1] * y[2]);
    dy[0] = c - a;
    dy[1] = (a - b) - c;
    dy[2] = b;
  }
  __device__ void vjp(const R (&y)[D], const R (&v)[D], R (&yb)[D], R (&pb)[P]) const {
    R v21 = v[1] - v[0], v12 = v[0] - v[1], v32 = v[2] - v[1];
    R t2 = (R(2) * k2) * y[1];
    yb[0] = k1 * v21;
    yb[1] = fmaR(k3 * y[2], v12, t2 * v32);
    yb[2] = (k3 * y[1]) * v12;
    pb[0] = fmaR(y[0], v21, pb[0]);
    pb[1] = fmaR(y[1] * y[1], v32, pb[1]);
    pb[2] = fmaR(y[1] * y[2], v12, pb[2]);
  }
  __device__ void jac(const R (&y)[D], R (&J)[D][D]) const {
    R j12 = k3 * y[2];
    R j13 = k3 * y[1];
    R t = (R(2) * k2) * y[1];
    J[0][0] = -k1; J[0][1] = j12;        J[0][2] = j13;
    J[1][0] = k1;  J[1][1] = -(t + j12); J[1][2] = -j13;
    J[2][0] = R(0); J[2][1] = t;         J[2][2] = R(0);
  }
  __device__ void jac_vjp(const R (&y)[D], const R (&Jb)[D][D], R (&yb)[D], R (&pb)[P]) const {
    // <Jb, J> = -k1 Jb00 + k3 y3 Jb01 + k3 y2 Jb02 + k1 Jb10 - (2 k2 y2 + k3 y3) Jb11
    //           - k3 y2 Jb12 + 2 k2 y2 Jb21
    R w21 = Jb[2][1] - Jb[1][1];
    R w02 = Jb[0][2] - Jb[1][2];
    R w01 = Jb[0][1] - Jb[1][1];
    yb[1] += fmaR(k3, w02, (R(2) * k2) * w21);
    yb[2] += k3 * w01;
    pb[0] += Jb[1][0] - Jb[0][0];
    pb[1] += (R(2) * y[1]) * w21;
    pb[2] += fmaR(y[2], w01, y[1] * w02);
  }
  __device__ void jvp(const R (&y)[D], const R (&yd)[D], int j, R (&fd)[D]) const {
    // tangents of a = k1 y1, b = k2 y2^2, c = k3 y2 y3
    const R ad = fmaR(k1, yd[0], (j == 0) ? y[0] : R(0));
    const R bd = fmaR((R(2) * k2) * y[1], yd[1], (j == 1) ? y[1] * y[1] : R(0));
    const R cd = fmaR(k3, fmaR(y[2], yd[1], y[1] * yd[2]), (j == 2) ? y[1] * y[2] : R(0));
    fd[0] = cd - ad;
    fd[1] = (ad - bd) - cd;
    fd[2] = bd;
  }
  __device__ void jac_jvp(const R (&y)[D], const R (&yd)[D], int j, R (&Jd)[D][D]) const {
    const R k1d = (j == 0) ? R(1) : R(0), k2d = (j == 1) ? R(1) : R(0), k3d = (j == 2) ? R(1) : R(0);
    const R j12 = fmaR(k3d, y[2], k3 * yd[2]);                        // (k3 y3)'
    const R j13 = fmaR(k3d, y[1], k3 * yd[1]);                        // (k3 y2)'
    const R t = R(2) * fmaR(k2d, y[1], k2 * yd[1]);                   // (2 k2 y2)'
    Jd[0][0] = -k1d; Jd[0][1] = j12;        Jd[0][2] = j13;
    Jd[1][0] = k1d;  Jd[1][1] = -(t + j12); Jd[1][2] = -j13;
    Jd[2][0] = R(0); Jd[2][1] = t;          Jd[2][2] = R(0);
  }
};

// HIRES, the eight-species photomorphogenesis model (Schaefer 1975, in the
// form of Hairer & Wanner, Solving ODEs II, Sec. IV.10; arXiv 2609.02876
// Sec. 3.1 lists it among the fused kernels' stiff fields), with its twelve
// distinct rate constants theta = (k1 .. k12):
//   y1' = -k1 y1 + k2 y2 + k3 y3 + k4        y2' = k1 y1 - k5 y2
//   y3' = -k6 y3 + k2 y4 + k7 y5             y4' = k3 y2 + k1 y3 - k8 y4
//   y5' = -k9 y5 + k2 (y6 + y7)
//   y6' = k11 (y4 + y7) + k1 y5 - (k2 y6 + a),  a = k10 y6 y8
//   y7' = a - k12 y7                         y8' = k12 y7 - a
// (indices below are 0-based: y[5] is y6, y[7] is y8).  Only a couples
// states nonlinearly, so J is constant apart from four entries.
template <class R>
struct Hires {
  static constexpr int D = 8, P = 12;
  // entries of the Jacobian that can be nonzero (those jac() sets), row by
  // row as bit masks over the columns: the linear solves skip the others
  static constexpr bool jac_nz(int i, int j) {
    constexpr unsigned rows[D] = {0x07, 0x03, 0x1C, 0x0E, 0x70, 0xF8, 0xE0, 0xE0};
    return (rows[i] >> j) & 1u;
  }
  R k[P];
  __device__ void load(const R* theta, int64_t n, int64_t kk) {
#pragma unroll
    for (int i = 0; i < P; ++i) k[i] = theta[i * n + kk];
  }
  __device__ void f(const R (&y)[D], R (&dy)[D]) const {
    const R a = k[9] * (y[5] * y[7]);
    const R b = k[11] * y[6];
    dy[0] = fmaR(-k[0], y[0], fmaR(k[1], y[1], fmaR(k[2], y[2], k[3])));
    dy[1] = fmaR(k[0], y[0], -(k[4] * y[1]));
    dy[2] = fmaR(-k[5], y[2], fmaR(k[1], y[3], k[6] * y[4]));
    dy[3] = fmaR(k[2], y[1], fmaR(k[0], y[2], -(k[7] * y[3])));
    dy[4] = fmaR(-k[8], y[4], k[1] * (y[5] + y[6]));
    dy[5] = fmaR(k[10], y[3] + y[6], fmaR(k[0], y[4], -fmaR(k[1], y[5], a)));
    dy[6] = a - b;
    dy[7] = b - a;
  }
  // yb = J^T v;  pb += (df/dk)^T v
  __device__ void vjp(const R (&y)[D], const R (&v)[D], R (&yb)[D], R (&pb)[P]) const {
    const R u = k[9] * y[7], w = k[9] * y[5];
    const R s5 = (v[6] - v[7]) - v[5];  // weight of a in (f5, f6, f7)
    const R s6 = v[7] - v[6];           // weight of k12 y7 in (f6, f7)
    yb[0] = k[0] * (v[1] - v[0]);
    yb[1] = fmaR(k[1], v[0], fmaR(k[2], v[3], -(k[4] * v[1])));
    yb[2] = fmaR(k[2], v[0], fmaR(k[0], v[3], -(k[5] * v[2])));
    yb[3] = fmaR(k[1], v[2], fmaR(k[10], v[5], -(k[7] * v[3])));
    yb[4] = fmaR(k[6], v[2], fmaR(k[0], v[5], -(k[8] * v[4])));
    yb[5] = fmaR(k[1], v[4] - v[5], u * s5);
    yb[6] = fmaR(k[1], v[4], fmaR(k[10], v[5], k[11] * s6));
    yb[7] = w * s5;
    pb[0] = fmaR(y[0], v[1] - v[0], fmaR(y[2], v[3], fmaR(y[4], v[5], pb[0])));
    pb[1] = fmaR(y[1], v[0], fmaR(y[3], v[2], fmaR(y[5] + y[6], v[4], fmaR(-y[5], v[5], pb[1]))));
    pb[2] = fmaR(y[2], v[0], fmaR(y[1], v[3], pb[2]));
    pb[3] = pb[3] + v[0];
    pb[4] = fmaR(-y[1], v[1], pb[4]);
    pb[5] = fmaR(-y[2], v[2], pb[5]);
    pb[6] = fmaR(y[4], v[2], pb[6]);
    pb[7] = fmaR(-y[3], v[3], pb[7]);
    pb[8] = fmaR(-y[4], v[4], pb[8]);
    pb[9] = fmaR(y[5] * y[7], s5, pb[9]);
    pb[10] = fmaR(y[3] + y[6], v[5], pb[10]);
    pb[11] = fmaR(y[6], s6, pb[11]);
  }
  __device__ void jac(const R (&y)[D], R (&J)[D][D]) const {
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
      for (int j = 0; j < D; ++j) J[i][j] = R(0);
    const R u = k[9] * y[7], w = k[9] * y[5];
    J[0][0] = -k[0]; J[0][1] = k[1]; J[0][2] = k[2];
    J[1][0] = k[0];  J[1][1] = -k[4];
    J[2][2] = -k[5]; J[2][3] = k[1]; J[2][4] = k[6];
    J[3][1] = k[2];  J[3][2] = k[0]; J[3][3] = -k[7];
    J[4][4] = -k[8]; J[4][5] = k[1]; J[4][6] = k[1];
    J[5][3] = k[10]; J[5][4] = k[0]; J[5][5] = -(k[1] + u); J[5][6] = k[10]; J[5][7] = -w;
    J[6][5] = u;     J[6][6] = -k[11]; J[6][7] = w;
    J[7][5] = -u;    J[7][6] = k[11];  J[7][7] = -w;
  }
  // <Jb, J>: y6 and y8 enter through u = k10 y8 (J55, J65, J75) and
  // w = k10 y6 (J57, J67, J77); the rate constants through every entry.
  __device__ void jac_vjp(const R (&y)[D], const R (&Jb)[D][D], R (&yb)[D], R (&pb)[P]) const {
    const R gu = (Jb[6][5] - Jb[5][5]) - Jb[7][5];
    const R gw = (Jb[6][7] - Jb[5][7]) - Jb[7][7];
    yb[7] = fmaR(k[9], gu, yb[7]);
    yb[5] = fmaR(k[9], gw, yb[5]);
    pb[0] += ((Jb[1][0] - Jb[0][0]) + Jb[3][2]) + Jb[5][4];
    pb[1] += (((Jb[0][1] + Jb[2][3]) + Jb[4][5]) + Jb[4][6]) - Jb[5][5];
    pb[2] += Jb[0][2] + Jb[3][1];
    pb[4] -= Jb[1][1];
    pb[5] -= Jb[2][2];
    pb[6] += Jb[2][4];
    pb[7] -= Jb[3][3];
    pb[8] -= Jb[4][4];
    pb[9] += fmaR(y[7], gu, y[5] * gw);
    pb[10] += Jb[5][3] + Jb[5][6];
    pb[11] += Jb[7][6] - Jb[6][6];
  }
  // fd = J yd + df/dk_j
  __device__ void jvp(const R (&y)[D], const R (&yd)[D], int j, R (&fd)[D]) const {
    R e[P];
#pragma unroll
    for (int i = 0; i < P; ++i) e[i] = (j == i) ? R(1) : R(0);
    const R ad = fmaR(e[9], y[5] * y[7], k[9] * fmaR(yd[5], y[7], y[5] * yd[7]));
    const R bd = fmaR(e[11], y[6], k[11] * yd[6]);
    fd[0] = fmaR(-k[0], yd[0], fmaR(k[1], yd[1], fmaR(k[2], yd[2],
            fmaR(-e[0], y[0], fmaR(e[1], y[1], fmaR(e[2], y[2], e[3]))))));
    fd[1] = fmaR(k[0], yd[0], fmaR(-k[4], yd[1], fmaR(e[0], y[0], -(e[4] * y[1]))));
    fd[2] = fmaR(-k[5], yd[2], fmaR(k[1], yd[3], fmaR(k[6], yd[4],
            fmaR(-e[5], y[2], fmaR(e[1], y[3], e[6] * y[4])))));
    fd[3] = fmaR(k[2], yd[1], fmaR(k[0], yd[2], fmaR(-k[7], yd[3],
            fmaR(e[2], y[1], fmaR(e[0], y[2], -(e[7] * y[3]))))));
    fd[4] = fmaR(-k[8], yd[4], fmaR(k[1], yd[5] + yd[6], fmaR(-e[8], y[4], e[1] * (y[5] + y[6]))));
    fd[5] = fmaR(k[10], yd[3] + yd[6], fmaR(k[0], yd[4], fmaR(-k[1], yd[5],
            fmaR(e[10], y[3] + y[6], fmaR(e[0], y[4], fmaR(-e[1], y[5], -ad))))));
    fd[6] = ad - bd;
    fd[7] = bd - ad;
  }
  __device__ void jac_jvp(const R (&y)[D], const R (&yd)[D], int j, R (&Jd)[D][D]) const {
    R e[P];
#pragma unroll
    for (int i = 0; i < P; ++i) e[i] = (j == i) ? R(1) : R(0);
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
      for (int c = 0; c < D; ++c) Jd[i][c] = R(0);
    const R ud = fmaR(e[9], y[7], k[9] * yd[7]);
    const R wd = fmaR(e[9], y[5], k[9] * yd[5]);
    Jd[0][0] = -e[0]; Jd[0][1] = e[1]; Jd[0][2] = e[2];
    Jd[1][0] = e[0];  Jd[1][1] = -e[4];
    Jd[2][2] = -e[5]; Jd[2][3] = e[1]; Jd[2][4] = e[6];
    Jd[3][1] = e[2];  Jd[3][2] = e[0]; Jd[3][3] = -e[7];
    Jd[4][4] = -e[8]; Jd[4][5] = e[1]; Jd[4][6] = e[1];
    Jd[5][3] = e[10]; Jd[5][4] = e[0]; Jd[5][5] = -(e[1] + ud); Jd[5][6] = e[10]; Jd[5][7] = -wd;
    Jd[6][5] = ud;    Jd[6][6] = -e[11]; Jd[6][7] = wd;
    Jd[7][5] = -ud;   Jd[7][6] = e[11];  Jd[7][7] = -wd;
  }
};

// Star in a flattened logarithmic halo, Phi = 1/2 v0^2 ln(Rc^2 + x^2 + y^2 + z^2/q^2).
// State (x, y, z, vx, vy, vz), theta = (v0, Rc, q).
template <class R>
struct LogHalo {
  static constexpr int D = 6, P = 3;
  R v0, rc, q, v2, r2, iq2, diq2;
  __device__ void load(const R* theta, int64_t n, int64_t k) {
    v0 = theta[k]; rc = theta[n + k]; q = theta[2 * n + k];
    v2 = v0 * v0;
    r2 = rc * rc;
    iq2 = R(1) / (q * q);
    diq2 = (R(-2) * iq2) / q;  // d(1/q^2)/dq, once per trajectory
  }
  __device__ void f(const R (&y)[D], R (&dy)[D]) const {
    R zq = y[2] * iq2;
    R Dn = fmaR(y[0], y[0], fmaR(y[1], y[1], fmaR(y[2], zq, r2)));
    R A = divR(v2, Dn);
    dy[0] = y[3];
    dy[1] = y[4];
    dy[2] = y[5];
    dy[3] = -(A * y[0]);
    dy[4] = -(A * y[1]);
    dy[5] = -(A * zq);
  }
  // a = -A g with g = (x, y, z/q^2), A = v0^2 / Dn.  With s = <w, g> for the
  // acceleration cotangent w and u = s A / Dn:
  //   d/dx = -A w_x + 2 x u, d/dy = -A w_y + 2 y u, d/dz = -A w_z / q^2 + 2 (z/q^2) u,
  //   d/dv0 = -2 s v0 / Dn, d/dRc = 2 Rc u, d/dq = (u z^2 - A w_z z) (-2 / (q^3)).
  __device__ void vjp(const R (&y)[D], const R (&v)[D], R (&yb)[D], R (&pb)[P]) const {
    R zq = y[2] * iq2;
    R Dn = fmaR(y[0], y[0], fmaR(y[1], y[1], fmaR(y[2], zq, r2)));
    R iD = recipR(Dn);
    R A = v2 * iD;
    R s = fmaR(v[3], y[0], fmaR(v[4], y[1], v[5] * zq));
    R u = (s * A) * iD;
    R u2 = u + u;
    yb[0] = fmaR(u2, y[0], -A * v[3]);
    yb[1] = fmaR(u2, y[1], -A * v[4]);
    yb[2] = fmaR(u2, zq, -(A * iq2) * v[5]);
    yb[3] = v[0];
    yb[4] = v[1];
    yb[5] = v[2];
    pb[0] = fmaR(-(s + s) * v0, iD, pb[0]);
    pb[1] = fmaR(u2, rc, pb[1]);
    pb[2] = fmaR(fmaR(u, y[2], -A * v[5]) * y[2], diq2, pb[2]);
  }
  __device__ void jac(const R (&y)[D], R (&J)[D][D]) const {
    R zq = y[2] * iq2;
    R Dn = fmaR(y[0], y[0], fmaR(y[1], y[1], fmaR(y[2], zq, r2)));
    R iD = recipR(Dn);
    R A = v2 * iD;
    R g[3] = {y[0], y[1], zq};
    R dD[3] = {R(2) * y[0], R(2) * y[1], R(2) * zq};
#pragma unroll
    for (int i = 0; i < 6; ++i)
#pragma unroll
      for (int j = 0; j < 6; ++j) J[i][j] = R(0);
#pragma unroll
    for (int i = 0; i < 3; ++i) J[i][3 + i] = R(1);
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        R dg = (i == j) ? ((i == 2) ? iq2 : R(1)) : R(0);
        J[3 + i][j] = (A * g[i]) * dD[j] * iD - A * dg;
      }
  }
  __device__ void jac_vjp(const R (&y)[D], const R (&Jb)[D][D], R (&yb)[D], R (&pb)[P]) const {
    // Not used: the halo has no Rosenbrock path (dao_solve/dao_grad refuse it).
    (void)y; (void)Jb; (void)yb; (void)pb;
  }
  __device__ void jac_jvp(const R (&y)[D], const R (&yd)[D], int j, R (&Jd)[D][D]) const {
    // Not used: the halo has no Rosenbrock path.
    (void)y; (void)yd; (void)j;
#pragma unroll
    for (int a = 0; a < D; ++a)
#pragma unroll
      for (int c = 0; c < D; ++c) Jd[a][c] = R(0);
  }
  // a = -A g: ad = -(Ad g + A gd) with Dnd = 2 <g, (xd, yd, zd)> + dRc^2 + z^2 d(1/q^2),
  // Ad = d(v0^2) / Dn - A Dnd / Dn, gd = (xd, yd, zd / q^2 + z d(1/q^2)).
  __device__ void jvp(const R (&y)[D], const R (&yd)[D], int j, R (&fd)[D]) const {
    const R zq = y[2] * iq2;
    const R Dn = fmaR(y[0], y[0], fmaR(y[1], y[1], fmaR(y[2], zq, r2)));
    const R iD = recipR(Dn);
    const R A = v2 * iD;
    const R dq2 = (j == 2) ? diq2 : R(0);  // d(1/q^2)/dq along direction j
    const R gzd = fmaR(yd[2], iq2, y[2] * dq2);
    R Dnd = R(2) * fmaR(y[0], yd[0], fmaR(y[1], yd[1], zq * yd[2]));
    Dnd = fmaR(y[2] * y[2], dq2, (j == 1) ? fmaR(R(2) * rc, R(1), Dnd) : Dnd);
    const R Ad = fmaR(-A, Dnd, (j == 0) ? R(2) * v0 : R(0)) * iD;
    fd[0] = yd[3];
    fd[1] = yd[4];
    fd[2] = yd[5];
    fd[3] = -fmaR(Ad, y[0], A * yd[0]);
    fd[4] = -fmaR(Ad, y[1], A * yd[1]);
    fd[5] = -fmaR(Ad, zq, A * gzd);
  }
};

}  // namespace dao
