// Neural right-hand side y' = W3 tanh(W2 tanh(W1 y + b1) + b2) + b3 (4-64-64-4,
// weights shared by the whole ensemble), solved and differentiated with the
// batched MLP on the matrix cores (v_mfma_f32_16x16x4f32).  The gradsolve
// paper (arXiv 2609.02876) Sec. 2.2 notes that theta may be the thousands of
// weights of a neural right-hand side; Sec. 4.8 trains one with the replay.
//
// Lane geometry.  One wavefront carries 16 trajectories ("slots").  Lane
// l = 16 g + j holds component g (0..3) of slot j (0..15).  This is exactly
// the B-operand layout of the 16x16x4 MFMA (k = l / 16, n = l % 16), and the
// result tile D (lane l, register r: row 4 g + r, column j) feeds the next
// contraction directly: its rows serve as that contraction's k index in the
// permuted order {4 g + r : g = 0..3} for k-block r, so a whole MLP forward
// pass, and the chain of its vector-Jacobian product, runs without moving
// data between lanes.  The weight gradients contract over the batch of 16
// trajectories instead; their operands are the transposes of those tiles,
// taken through a per-wavefront LDS buffer.
//
// Adaptive control (Sec. 2.1) is per slot: the four lanes of a slot hold the
// same t, h, counters and decisions, computed from the same values in the
// same order.
#pragma once

#include "common.hpp"
#include "tsit5.hpp"

namespace dao {
namespace mlp {

constexpr int NH = 64;  // hidden width
constexpr int OW1 = 0, OB1 = 256, OW2 = 320, OB2 = 4416, OW3 = 4480, OB3 = 4736, NP = 4740;
constexpr int SLOTS = 16;

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// Value of lane (16 c + j) for c = 0..3, gathered into every lane of slot j,
// in component order (the same four values in the same order in all four
// lanes of a slot).
__device__ __forceinline__ void gather4(float x, int j, float (&out)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = __shfl(x, 16 * c + j);
}

// Operands of the forward pass held in registers for the whole kernel.
struct Fwd {
  float w1[4];    // layer 1, output tile T: A[i][k] = W1[16T + i][k]
  f4 b1[4];       // C of output tile T: b1[16T + 4g + r]
  float w2[64];   // layer 2, [T2 * 16 + T * 4 + r]: A[i][g] = W2[16T2 + i][16T + 4g + r]
  f4 b2[4];
  float w3[16];   // layer 3, rows padded to 16 (row 4o = output o): [T * 4 + r]
  f4 b3;          // C: {b3[g], 0, 0, 0}

  // with_w2 = false: W2, b1 and b2 are read from LDS instead (gradient kernel).
  __device__ __forceinline__ void load(const float* th, int g, int j, bool with_w2 = true) {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      w1[T] = th[OW1 + (16 * T + j) * 4 + g];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (with_w2) {
          b1[T][r] = th[OB1 + 16 * T + 4 * g + r];
          b2[T][r] = th[OB2 + 16 * T + 4 * g + r];
        }
        w3[T * 4 + r] = (j % 4 == 0) ? th[OW3 + (j / 4) * NH + 16 * T + 4 * g + r] : 0.f;
      }
    }
    if (with_w2) {
#pragma unroll
      for (int T2 = 0; T2 < 4; ++T2)
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            w2[T2 * 16 + T * 4 + r] = th[OW2 + (16 * T2 + j) * NH + 16 * T + 4 * g + r];
    }
    b3 = f4{th[OB3 + g], 0.f, 0.f, 0.f};
  }
};

// Operands of the vector-Jacobian product.
struct Bwd {
  float w3t[4];   // dh2 = W3^T v, tile T: A[i][g] = W3[g][16T + i]
  float w1t[16];  // ybar = W1^T dz1, rows padded (row 4c = input c): [T * 4 + r]
  // dh1 = W2^T dz2 reads A[i][g] = W2[16T2 + 4g + r][16T1 + i] from LDS.

  __device__ __forceinline__ void load(const float* th, int g, int j) {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      w3t[T] = th[OW3 + g * NH + 16 * T + j];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        w1t[T * 4 + r] = (j % 4 == 0) ? th[OW1 + (16 * T + 4 * g + r) * 4 + j / 4] : 0.f;
    }
  }
};

// tanh in binary32: for |x| < 1/4 the odd Taylor polynomial to x^9 (relative
// truncation error below 4e-8 there), otherwise 1 - 2 / (exp(2|x|) + 1) with
// the hardware base-2 exponential and reciprocal (absolute error ~2e-7);
// sign restored at the end.  Large |x| saturate to +-1.
__device__ __forceinline__ float tanh_(float x) {
  const float ax = __builtin_fabsf(x);
  const float x2 = ax * ax;
  float p = fmaR(x2, 62.0f / 2835.0f, -17.0f / 315.0f);
  p = fmaR(p, x2, 2.0f / 15.0f);
  p = fmaR(p, x2, -1.0f / 3.0f);
  p = fmaR(p * x2, ax, ax);
  const float e = __builtin_amdgcn_exp2f(ax * 2.8853900817779268f);  // exp(2|x|)
  const float q = fmaR(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
  return __builtin_copysignf(ax < 0.25f ? p : q, x);
}

// W2 kept once in LDS for the gradient kernel, row u2 = 64 floats, column u1
// stored at u1 ^ swz(u2).  swz sends bits (0, 1, 3, 2) of u2 mod 16 to bits
// (0, 1, 3, 4): the forward operand reads (row 16T2 + j, column
// 16T + 4g + r) and the transposed reads (row 16T2 + 4g + r, column
// 16T1 + j) both hit 32 distinct banks in each half-wavefront.
__device__ __forceinline__ int swz(int u2) {
  return (u2 & 3) | (((u2 >> 3) & 1) << 3) | (((u2 >> 2) & 1) << 4);
}
__device__ __forceinline__ int w2_index(int u2, int u1) { return u2 * NH + (u1 ^ swz(u2 & 15)); }

// Operand sources for the layer-2 forward product (A of output tile T2,
// k-block (T, r)).
// Operand sources for the layer-2 forward product (A of output tile T2,
// k-block (T, r)) and for the hidden-layer biases (C of tile T).
struct W2Regs {
  const Fwd& P;
  __device__ float operator()(int T2, int T, int r, int, int) const { return P.w2[T2 * 16 + T * 4 + r]; }
  __device__ f4 b1(int T, int) const { return P.b1[T]; }
  __device__ f4 b2(int T, int) const { return P.b2[T]; }
};
// LDS copy of the gradient kernel: W2 swizzled (w2_index), then b1 and b2.
struct W2Lds {
  const float* w;
  __device__ float operator()(int T2, int T, int r, int g, int j) const {
    return w[w2_index(16 * T2 + j, 16 * T + 4 * g + r)];
  }
  __device__ f4 b1(int T, int g) const { return *(const f4*)(w + NH * NH + 16 * T + 4 * g); }
  __device__ f4 b2(int T, int g) const { return *(const f4*)(w + NH * NH + NH + 16 * T + 4 * g); }
};

// Forward pass for the 16 slots: y in the state layout; returns f in the
// state layout and the hidden activations as D tiles (unit 16T + 4g + r of
// slot j in h[T][r]).
template <class W2, bool OUT = true>
__device__ __forceinline__ float forward(const Fwd& P, const W2& w2, int g, int j, float y,
                                         f4 (&h1)[4], f4 (&h2)[4]) {
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const f4 z = mma(P.w1[T], y, w2.b1(T, g));
#pragma unroll
    for (int r = 0; r < 4; ++r) h1[T][r] = tanh_(z[r]);
  }
#pragma unroll
  for (int T2 = 0; T2 < 4; ++T2) {
    f4 acc = w2.b2(T2, g);
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mma(w2(T2, T, r, g, j), h1[T][r], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) h2[T2][r] = tanh_(acc[r]);
  }
  if constexpr (!OUT) return 0.f;
  f4 out = P.b3;
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) out = mma(P.w3[T * 4 + r], h2[T][r], out);
  return out[0];
}

__device__ __forceinline__ float rhs(const Fwd& P, float y) {
  f4 h1[4], h2[4];
  return forward(P, W2Regs{P}, 0, 0, y, h1, h2);
}
template <class W2>
__device__ __forceinline__ float rhs(const Fwd& P, const W2& w2, int g, int j, float y) {
  f4 h1[4], h2[4];
  return forward(P, w2, g, j, y, h1, h2);
}

// Tsit5 trial step for the slot (one component per lane); k[0] = f(y) on
// entry.  Same stage sums, in the same order, as tsit5::trial.
__device__ __forceinline__ void trial(const Fwd& P, float y, float h, float (&k)[7], float& ynew,
                                      float& err) {
  float Y = y;
#pragma unroll
  for (int i = 1; i < 7; ++i) {
    float acc = tsit5::a<float>(i, 0) * k[0];
#pragma unroll
    for (int j = 1; j < 6; ++j)
      if (j < i) acc = fmaR(tsit5::a<float>(i, j), k[j], acc);
    Y = fmaR(h, acc, y);
    k[i] = rhs(P, Y);
  }
  ynew = Y;
  float acc = tsit5::e<float>(0) * k[0];
#pragma unroll
  for (int j = 1; j < 7; ++j) acc = fmaR(tsit5::e<float>(j), k[j], acc);
  err = acc;  // the embedded error without its factor h (in the error weight)
}

// Stage state i from y and k[0..i-1] (one component).
__device__ __forceinline__ float stage(int i, float y, float h, const float (&k)[7]) {
  float acc = tsit5::a<float>(i, 0) * k[0];
#pragma unroll
  for (int j = 1; j < 6; ++j)
    if (j < i) acc = fmaR(tsit5::a<float>(i, j), k[j], acc);
  return fmaR(h, acc, y);
}

// The attempt's error test for the slot: the unscaled error a times the
// weight w = h / sc (formed while the last stage is evaluated), squared and
// averaged over the slot's four components in component order.
__device__ __forceinline__ float slot_error_msq(float a, float w, int j) {
  float r[4];
  gather4(a * w, j, r);
  float acc = r[0] * r[0];
#pragma unroll
  for (int c = 1; c < 4; ++c) acc = fmaR(r[c], r[c], acc);
  return acc * (1.0f / 4.0f);
}

// Mean square of a slot vector e / sc, summed in component order.
__device__ __forceinline__ float slot_mean_sq(float e, float sc, int j) {
  float r[4];
  gather4(e / sc, j, r);
  float acc = r[0] * r[0];
#pragma unroll
  for (int c = 1; c < 4; ++c) acc = fmaR(r[c], r[c], acc);
  return acc * (1.0f / 4.0f);
}

// Mean square of a slot vector x / sc (for the starting step), component order.
__device__ __forceinline__ float slot_rms(float x, float sc, int j) {
  return sqrtR(slot_mean_sq(x, sc, j));
}

struct SolveArgs {
  int64_t n;
  const float* theta;  // [4740]
  const float* y0;     // [4][n]
  float t0, t1, rtol, atol, dt0;
  int64_t max_steps;
  float* y1;
  int64_t s_cap;
  float* t_rec;
  float* h_rec;
  int32_t* count;
  int32_t* nrej;
  int32_t* status;
  unsigned long long* queue;
  float* trash;  // [64][2]
};

// Adaptive Tsit5 solve of the neural field, 16 trajectories per wavefront,
// slots refilled from a work queue.  The MLP evaluations are wave-wide: every
// slot takes one attempt per iteration with its own step size.
__global__ void __launch_bounds__(256) solve_kernel(SolveArgs a) {
  constexpr int32_t RUNNING = -1;
  const int lane = laneId();
  const int g = lane >> 4, j = lane & 15;
  Fwd P;
  P.load(a.theta, g, j);
  float* const trash = a.trash + 2 * lane;
  const CtrlCoef<float, 10> KC = CtrlCoef<float, 10>::make(false);

  float y = 0.f, k[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) k[i] = 0.f;
  float t = 0.f, h = 0.f;
  int32_t nacc = 0, nrej = 0;
  int64_t attempts = 0;
  bool prev_rej = false;
  int64_t traj = -1;
  bool live = true;
  bool drained = false;

  for (;;) {
    // ---- refill: slots are claimed from the queue together (one atomic per
    // wavefront); all four lanes of a slot compute the same index.
    const bool need = live && traj < 0;
    if (drained && need) live = false;
    const unsigned long long m = drained ? 0ull : (__ballot(need) & 0xFFFFull);  // slot bits
    bool fresh = false;
    if (m) {
      unsigned long long base = 0;
      if (lane == 0) base = atomicAdd(a.queue, (unsigned long long)__popcll(m));
      base = __shfl(base, 0);
      if (base + (unsigned long long)__popcll(m) >= (unsigned long long)a.n) drained = true;
      if (need) {
        const unsigned long long kk = base + (unsigned long long)__popcll(m & ((1ull << j) - 1ull));
        if (kk < (unsigned long long)a.n) {
          traj = (int64_t)kk;
          y = a.y0[g * a.n + traj];
          __builtin_amdgcn_s_waitcnt(0);
          t = a.t0;
          nacc = 0;
          nrej = 0;
          attempts = 0;
          prev_rej = false;
          fresh = true;
        } else {
          live = false;
        }
      }
    }
    if (__ballot(live) == 0ull) break;
    // Starting step for the fresh slots (two wave-wide field evaluations).
    if (__ballot(fresh)) {
      const float f0 = rhs(P, y);
      const float sc = fmaR(a.rtol, absR(y), a.atol);
      const float d0 = slot_rms(y, sc, j);
      const float d1 = slot_rms(f0, sc, j);
      const float span = a.t1 - a.t0;
      float hh = (d0 < 1e-5f || d1 < 1e-5f) ? 1e-6f : 0.01f * (d0 / d1);
      hh = (span < hh) ? span : hh;
      const float f1 = rhs(P, fmaR(hh, f0, y));
      const float d2 = slot_rms(f1 - f0, sc, j) / hh;
      const float mm = (d1 < d2) ? d2 : d1;
      float h1;
      if (mm <= 1e-15f) {
        const float tt = hh * 1e-3f;
        h1 = (1e-6f < tt) ? tt : 1e-6f;
      } else {
        h1 = powf(0.01f / mm, 1.0f / 5.0f);
      }
      const float h100 = 100.0f * hh;
      const float h0 = truncBits((h1 < h100) ? h1 : h100);
      if (fresh) {
        k[0] = f0;
        h = (a.dt0 > 0.f) ? a.dt0 : h0;
        if (!(a.t1 > a.t0)) {
          // Zero span: nothing to integrate.
          if (g == 0) {
            a.count[traj] = 0;
            if (a.nrej) a.nrej[traj] = 0;
            a.status[traj] = TRAJ_OK;
          }
          a.y1[g * a.n + traj] = y;
          traj = -1;
        }
      }
    }
    if (__ballot(traj >= 0) == 0ull) continue;

    // ---- one attempt for every active slot (selects, one rare exit)
    const bool act = traj >= 0;
    attempts += act ? 1 : 0;
    const bool last = (t + h >= a.t1);
    const float hs = last ? (a.t1 - t) : h;
    float ynew, err;
    trial(P, y, hs, k, ynew, err);
    const float ay = absR(y), an = absR(ynew);
    const float wt = hs / fmaR(a.rtol, (ay < an) ? an : ay, a.atol);
    const float msq = slot_error_msq(err, wt, j);
    const bool acc = msq <= 1.f;
    const float root = ctrl_root<float, 10>(msq, KC);
    const float fq = (msq == 0.f) ? 10.f : truncBits(0.9f * root);
    const float fmin = (0.2f < fq) ? fq : 0.2f;
    int32_t st = (acc && nacc >= a.s_cap) ? TRAJ_CAPACITY : RUNNING;
    st = finiteR(msq) ? st : TRAJ_NONFINITE;
    st = (t + hs > t) ? st : TRAJ_DT_UNDERFLOW;
    st = finiteR(hs) ? st : TRAJ_NONFINITE;
    if (act && g == 0) {
      const bool room = nacc < a.s_cap;
      *(room ? a.h_rec + traj * a.s_cap + nacc : trash) = hs;
      if (a.t_rec) *(room ? a.t_rec + traj * a.s_cap + nacc : trash + 1) = t;
    }
    const bool take = act && (st == RUNNING) && acc;
    const float tn = last ? a.t1 : t + hs;
    y = take ? ynew : y;
    k[0] = take ? k[6] : k[0];
    t = take ? tn : t;
    nacc += take ? 1 : 0;
    nrej += (act && st == RUNNING && !acc) ? 1 : 0;
    float fa = (fmin < 10.f) ? fmin : 10.f;
    fa = (prev_rej && fa > 1.f) ? 1.f : fa;
    h = act ? hs * (acc ? fa : fmin) : h;
    prev_rej = act ? !acc : prev_rej;
    if (act && st == RUNNING) {
      if (take && !(tn < a.t1)) st = TRAJ_OK;
      else if (attempts >= a.max_steps) st = TRAJ_MAX_STEPS;
    }
    if (act && st != RUNNING) {
      a.y1[g * a.n + traj] = (st == TRAJ_OK) ? y : nanR(0.f);
      if (g == 0) {
        a.count[traj] = nacc;
        if (a.nrej) a.nrej[traj] = nrej;
        a.status[traj] = st;
      }
      traj = -1;
    }
  }
}

// ---------------------------------------------------------------- gradient

struct GradArgs {
  int64_t n;
  const float* theta;
  const float* y0;
  int64_t s_cap;
  const float* h_rec;
  const int32_t* count;
  const int32_t* status;
  int64_t s_max;
  const float* dLdy1;
  float* dLdy0;
  float* scratch;          // per resident wavefront: [s_max][64]
  float* partial;          // per chunk: [NP] weight-gradient partial sums
  int64_t chunks;          // chunk c holds the groups c, c + chunks, c + 2 chunks, ...
  const int32_t* perm;
  unsigned long long* groups;  // chunk queue counter (zero at launch)
};

// Chunks of the shared-weight gradient: at most this many rows of partial
// sums, so their number (and with it every rounding of the sum) depends on n
// alone, not on the grid or on which wavefront claims which chunk.
constexpr int64_t MAX_CHUNKS = 2048;
inline int64_t grad_chunks(int64_t n) {
  const int64_t ngroups = (n + SLOTS - 1) / SLOTS;
  return ngroups < MAX_CHUNKS ? (ngroups > 0 ? ngroups : 1) : MAX_CHUNKS;
}

// Transpose through LDS: x holds unit 16T + 4g + r of slot j in x[T][r]; the
// result holds, in xt[T][r], unit 16T + j of slot 4g + r (the operand
// layout of a contraction over the slots).  buf: this wavefront's 4 x 16 x 17
// floats.
__device__ __forceinline__ void transpose(float* buf, const f4 (&x)[4], f4 (&xt)[4], int g, int j) {
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) buf[T * 272 + (4 * g + r) * 17 + j] = x[T][r];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) xt[T][r] = buf[T * 272 + j * 17 + 4 * g + r];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over the 16 slots of a transposed tile: the four slots 4g + r of this
// lane, then the four rows g.
__device__ __forceinline__ float slot_sum(const f4& x) {
  float s = (x[0] + x[1]) + (x[2] + x[3]);
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  return s;
}

// Weight-gradient accumulators of one wavefront.
struct GradAcc {
  f4 w2[16];   // dW2 tile (T2, T1) at [T2 * 4 + T1]: row 16T2 + 4g + r, column 16T1 + j
  f4 w3t[4];   // dW3^T tile T: row (unit) 16T + 4g + r, column (output) j < 4
  f4 w1t[4];   // dW1^T tile T: row (unit) 16T + 4g + r, column (input) j < 4
  float b1[4];  // dz1 summed over the slots, unit 16T + j (the same in every row g)
  float b2[4];  // dz2 likewise
  float b3;     // per-lane partial sum of v (output g, slot j)
};

// Reverse of one field evaluation at Y (state layout) with output cotangent
// v: returns ybar = (df/dy)^T v and accumulates the weight cotangents.  The
// second hidden layer's activations come from h2c (what forward() returned
// at this Y when the stage was recomputed, 16 values per lane at
// h2c[(4 T + r) 64]); the first layer is evaluated again (4 products), with
// the operations forward() uses, so both are the forward pass's bits.
__device__ __forceinline__ float vjp(const Fwd& P, const Bwd& Q, const float* w2s, float* buf,
                                     const float* h2c, float Y, float v, GradAcc& G, int g,
                                     int j) {
  const W2Lds w2{w2s};
  f4 h1[4], h2[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const f4 z = mma(P.w1[T], Y, w2.b1(T, g));
#pragma unroll
    for (int r = 0; r < 4; ++r) h1[T][r] = tanh_(z[r]);
  }
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) h2[T][r] = h2c[(4 * T + r) * WAVE];
  // dh2 = W3^T v, dz2 = dh2 (1 - h2^2)
  f4 dz2[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const f4 d = mma(Q.w3t[T], v, zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) dz2[T][r] = d[r] * fmaR(-h2[T][r], h2[T][r], 1.f);
  }
  // dh1 = W2^T dz2, dz1 = dh1 (1 - h1^2)
  f4 dz1[4];
#pragma unroll
  for (int T1 = 0; T1 < 4; ++T1) {
    f4 acc = zero4();
#pragma unroll
    for (int T2 = 0; T2 < 4; ++T2)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc = mma(w2s[w2_index(16 * T2 + 4 * g + r, 16 * T1 + j)], dz2[T2][r], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) dz1[T1][r] = acc[r] * fmaR(-h1[T1][r], h1[T1][r], 1.f);
  }
  // ybar = W1^T dz1 (padded rows: row 4c = input c)
  f4 yb = zero4();
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) yb = mma(Q.w1t[T * 4 + r], dz1[T][r], yb);

  G.b3 += v;
  // Weight cotangents: contractions over the 16 slots.
  f4 dz2t[4], h1t[4];
  transpose(buf, dz2, dz2t, g, j);
  transpose(buf, h1, h1t, g, j);
  // Bias cotangent of layer 2: dz2t[T][r] is unit 16T + j at slot 4g + r.
#pragma unroll
  for (int T = 0; T < 4; ++T) G.b2[T] += slot_sum(dz2t[T]);
#pragma unroll
  for (int T2 = 0; T2 < 4; ++T2)
#pragma unroll
    for (int T1 = 0; T1 < 4; ++T1)
#pragma unroll
      for (int r = 0; r < 4; ++r) G.w2[T2 * 4 + T1] = mma(dz2t[T2][r], h1t[T1][r], G.w2[T2 * 4 + T1]);
  // Slot-indexed operands: lane (g, j) takes v / Y of input j (< 4) at slot 4g + r.
  float vg[4], yg[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int src = 16 * (j & 3) + 4 * g + r;
    const float vs = __shfl(v, src), ys = __shfl(Y, src);
    vg[r] = (j < 4) ? vs : 0.f;
    yg[r] = (j < 4) ? ys : 0.f;
  }
  f4 h2t[4], dz1t[4];
  transpose(buf, h2, h2t, g, j);
  transpose(buf, dz1, dz1t, g, j);
#pragma unroll
  for (int T = 0; T < 4; ++T) G.b1[T] += slot_sum(dz1t[T]);
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      G.w3t[T] = mma(h2t[T][r], vg[r], G.w3t[T]);
      G.w1t[T] = mma(dz1t[T][r], yg[r], G.w1t[T]);
    }
  return yb[0];
}

// One replay step of the slot (one component per lane).
__device__ __forceinline__ float replay(const Fwd& P, const float* w2s, int g, int j, float y,
                                        float h) {
  const W2Lds w2{w2s};
  float k[7];
  k[0] = rhs(P, w2, g, j, y);
#pragma unroll
  for (int i = 1; i < 6; ++i) k[i] = rhs(P, w2, g, j, stage(i, y, h, k));
  return stage(6, y, h, k);
}

// Tsit5 stage coefficients a(i, j) for the reverse loop, whose stage index is
// a run-time (wavefront-uniform) value; the values are tsit5::a<float>.
__constant__ float TS_A_F32[6][5] = {
    {0.f, 0.f, 0.f, 0.f, 0.f},
    {(float)tsit5::A10, 0.f, 0.f, 0.f, 0.f},
    {(float)tsit5::A20, (float)tsit5::A21, 0.f, 0.f, 0.f},
    {(float)tsit5::A30, (float)tsit5::A31, (float)tsit5::A32, 0.f, 0.f},
    {(float)tsit5::A40, (float)tsit5::A41, (float)tsit5::A42, (float)tsit5::A43, 0.f},
    {(float)tsit5::A50, (float)tsit5::A51, (float)tsit5::A52, (float)tsit5::A53, (float)tsit5::A54}};

// Reverse of one replay step from y_j: lam = dL/dy_{j+1} in, dL/dy_j out.
// The stage states and stage cotangents sit in the wavefront's LDS area
// (st[0..5] = Y_i, st[6..11] = kbar_i, 64 lanes each) so that the six
// stage VJPs run as one loop body.
__device__ __forceinline__ void reverse(const Fwd& P, const Bwd& Q, const float* w2s, float* buf,
                                        float* st, float* h2s, float y, float h, float& lam,
                                        GradAcc& G, int g, int j) {
  const W2Lds w2{w2s};
  const int lane = 16 * g + j;
  // h2s: the second hidden layer of each stage's evaluation, [6][16][64]
  auto keep_h2 = [&](int i, const f4 (&h2)[4]) {
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) h2s[(16 * i + 4 * T + r) * WAVE + lane] = h2[T][r];
  };
  float k[7];
  float Yi = y;
  st[lane] = Yi;
  {
    f4 h1[4], h2[4];
    k[0] = forward(P, w2, g, j, y, h1, h2);
    keep_h2(0, h2);
  }
#pragma unroll
  for (int i = 1; i < 6; ++i) {
    Yi = stage(i, y, h, k);
    st[i * WAVE + lane] = Yi;
    f4 h1[4], h2[4];
    if (i < 5) {
      k[i] = forward(P, w2, g, j, Yi, h1, h2);
    } else {
      (void)forward<W2Lds, false>(P, w2, g, j, Yi, h1, h2);  // f itself is not needed
    }
    keep_h2(i, h2);
  }
#pragma unroll
  for (int i = 0; i < 6; ++i) st[(6 + i) * WAVE + lane] = (h * tsit5::a<float>(6, i)) * lam;
#pragma unroll 1
  for (int i = 5; i >= 0; --i) {
    const float yb = vjp(P, Q, w2s, buf, h2s + 16 * i * WAVE + lane, st[i * WAVE + lane],
                         st[(6 + i) * WAVE + lane], G, g, j);
    lam += yb;
    for (int jj = 0; jj < i; ++jj) {
      float& kb = st[(6 + jj) * WAVE + lane];
      kb = fmaR(h * TS_A_F32[i][jj], yb, kb);
    }
  }
}

// Sum over the 16 lanes of a row (lanes 16g .. 16g + 15).
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ void __launch_bounds__(256) grad_kernel(GradArgs a) {
  __shared__ float lds[4][4 * 272];
  __shared__ float stage_lds[4][12 * WAVE];
  __shared__ float h2_lds[4][6 * 16 * WAVE];
  __shared__ __attribute__((aligned(16))) float w2s[NH * NH + 2 * NH];
  const int lane = laneId();
  const int g = lane >> 4, j = lane & 15;
  const int wv = threadIdx.x / WAVE;
  float* buf = lds[wv];
  const int64_t slot = (int64_t)blockIdx.x * (blockDim.x / WAVE) + wv;
  float* scr = a.scratch + slot * (a.s_max * WAVE) + lane;
  const unsigned long long ngroups = (unsigned long long)((a.n + SLOTS - 1) / SLOTS);

  for (int e = threadIdx.x; e < NH * NH; e += blockDim.x)
    w2s[w2_index(e / NH, e % NH)] = a.theta[OW2 + e];
  for (int e = threadIdx.x; e < NH; e += blockDim.x) {
    w2s[NH * NH + e] = a.theta[OB1 + e];
    w2s[NH * NH + NH + e] = a.theta[OB2 + e];
  }
  __syncthreads();
  Fwd P;
  P.load(a.theta, g, j, false);
  Bwd Q;
  Q.load(a.theta, g, j);
  GradAcc G;
  // A trajectory of the ensemble that failed, or holds more than s_max steps,
  // has no gradient: its chunk's partial sum becomes NaN, so the summed
  // shared-weight gradient is NaN rather than silently partial.
  bool failed = false;
  auto fill = [&](float v) {
    const f4 v4 = {v, v, v, v};
#pragma unroll
    for (int i = 0; i < 16; ++i) G.w2[i] = v4;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      G.w3t[T] = v4;
      G.w1t[T] = v4;
      G.b1[T] = v;
      G.b2[T] = v;
    }
    G.b3 = v;
  };
  for (;;) {
    unsigned long long chunk = 0;
    if (lane == 0) chunk = atomicAdd(a.groups, 1ull);
    chunk = __shfl(chunk, 0);
    if (chunk >= (unsigned long long)a.chunks) break;
    fill(0.f);
    failed = false;
    for (unsigned long long grp = chunk; grp < ngroups; grp += (unsigned long long)a.chunks) {
      const int64_t idx = (int64_t)grp * SLOTS + j;
      int64_t k = -1;
      int cnt = 0;
      bool ok = false;
      if (idx < a.n) {
        k = a.perm ? (int64_t)a.perm[idx] : idx;
        if (k < 0 || k >= a.n) {
          k = -1;  // an order that is not this record's: nothing is read or written
        } else {
          cnt = a.count[k];
          ok = cnt >= 0 && cnt <= a.s_max && (a.status == nullptr || a.status[k] == TRAJ_OK);
          if (!ok) cnt = 0;
          failed = failed || !ok;
        }
      }
      int mx = cnt;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int o = __shfl_xor(mx, off);
        mx = (o > mx) ? o : mx;
      }
      // A slot that is empty or failed carries a zero state and cotangent, so it
      // contributes exactly nothing to the shared-weight gradient.
      float y = 0.f, lam = 0.f;
      const float* hrow = a.h_rec;
      if (ok) {
        y = a.y0[g * a.n + k];
        lam = a.dLdy1[g * a.n + k];
        hrow = a.h_rec + k * a.s_cap;
      }
      // Forward replay storing y_i (zero-size steps past a slot's count).
      for (int i = 0; i < mx; ++i) {
        const float hi = (i < cnt) ? hrow[i] : 0.f;
        scr[(int64_t)i * WAVE] = y;
        y = replay(P, w2s, g, j, y, hi);
      }
      for (int i = mx - 1; i >= 0; --i) {
        const float yi = scr[(int64_t)i * WAVE];
        const float hi = (i < cnt) ? hrow[i] : 0.f;
        reverse(P, Q, w2s, buf, stage_lds[wv], h2_lds[wv], yi, hi, lam, G, g, j);
      }
      if (k >= 0 && a.dLdy0) a.dLdy0[g * a.n + k] = ok ? lam : nanR(0.f);
    }

    // Write this chunk's partial weight gradient (packed like theta).
    if (__ballot(failed) != 0ull) fill(nanR(0.f));
    // Stores from one base per block of the row (it moves with the chunk)
    // and constant offsets.
    float* out = a.partial + (int64_t)chunk * NP;
    float* o2 = out + OW2 + 4 * g * NH + j;
#pragma unroll
    for (int T2 = 0; T2 < 4; ++T2)
#pragma unroll
      for (int T1 = 0; T1 < 4; ++T1)
#pragma unroll
        for (int r = 0; r < 4; ++r) o2[(16 * T2 + r) * NH + 16 * T1] = G.w2[T2 * 4 + T1][r];
    float* o3 = out + OW3 + j * NH + 4 * g;
    float* o1 = out + OW1 + 16 * g + j;
    float* ob = out + OB1 + j;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      if (j < 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o3[16 * T + r] = G.w3t[T][r];
          o1[(16 * T + r) * 4] = G.w1t[T][r];
        }
      }
      if (g == 0) {
        ob[16 * T] = G.b1[T];
        ob[OB2 - OB1 + 16 * T] = G.b2[T];
      }
    }
    const float s3 = row_sum(G.b3);
    if (j == 0) out[OB3 + g] = s3;
  }
}

// dL/dtheta[p] = sum over the chunks' rows w of partial[w][p], in a fixed
// order: pass 1 sums each run of REDUCE_CHUNK consecutive rows into the run's
// first row (block (x, c): columns 256x .. 256x + 255 of run c, so every row
// read is coalesced and a column of a run belongs to one thread); pass 2 sums
// those rows in order.
constexpr int REDUCE_CHUNK = 64;
__global__ void __launch_bounds__(256) reduce_chunks_kernel(float* partial, int64_t nw) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= NP) return;
  const int64_t w0 = (int64_t)blockIdx.y * REDUCE_CHUNK;
  const int64_t w1 = (w0 + REDUCE_CHUNK < nw) ? w0 + REDUCE_CHUNK : nw;
  float s = 0.f;
  for (int64_t w = w0; w < w1; ++w) s += partial[w * NP + p];
  partial[w0 * NP + p] = s;
}
__global__ void __launch_bounds__(256) reduce_kernel(const float* partial, int64_t nw, float* out) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= NP) return;
  float s = 0.f;
  for (int64_t w = 0; w < nw; w += REDUCE_CHUNK) s += partial[w * NP + p];
  out[p] = s;
}

}  // namespace mlp
}  // namespace dao
