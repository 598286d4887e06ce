// Solve and gradient kernels: one trajectory per lane.
//
// Solve (arXiv 2609.02876 Sec. 2.1 loop, Sec. 3.1 record): a persistent grid
// of wavefronts pulls trajectories from a global work queue.  Whenever lanes
// of a wavefront finish their trajectory, the wavefront ballots the idle
// lanes, claims that many new trajectory indices with ONE atomic add, and
// hands them out by rank among the idle lanes (mbcnt).  So a wavefront never
// waits for its slowest trajectory while work remains.  Each accepted step
// appends (t_n, h_n) to the lane's own record row.
//
// Gradient (Sec. 3.1 replay chain, reverse sweep): trajectories are visited in
// order of decreasing step count, 64 at a time (one wavefront); the 64 lanes
// replay their meshes in lockstep, store every state y_j in a per-wavefront
// scratch tile laid out [step][component][lane] (each store and load is one
// contiguous 512-byte row), then sweep backward, recomputing each step's
// stages from y_j.
#pragma once

#include "common.hpp"
#include "mlp.hpp"
#include "rodas5p.hpp"
#include "ros23.hpp"
#include "systems.hpp"
#include "tsit5.hpp"
#include "vern7.hpp"

namespace dao {

enum Method : int { M_TSIT5 = 0, M_ROS23 = 1, M_VERN7 = 2, M_RODAS5P = 3 };

// Values per trajectory in the two-phase solve's parking area: y, f(y), t, h
// and room for the sensitivities, rounded up to whole 64-byte lines.  A
// trajectory's record is contiguous, so the phase-2 resume, which visits
// trajectories in an order unrelated to their index, reads one or two lines
// per trajectory instead of one line per value.
template <class R, int D, int P>
constexpr int save_stride() {
  constexpr int v = 2 * D + 2 + D * P, u = 64 / (int)sizeof(R);
  return (v + u - 1) / u * u;
}

template <class R>
struct SolveArgs {
  int64_t n;
  const R* theta;
  const R* y0;
  R t0, t1, rtol, atol, dt0;
  int64_t max_steps;
  R* y1;
  int64_t s_cap;
  R* t_rec;
  R* h_rec;
  int32_t* count;
  int32_t* nrej;
  int32_t* status;
  R* y_rec;  // optional [n][s_cap][D]: the state at the start of each accepted step
  unsigned long long* queue;  // trajectories handed out so far (zero at launch)
  R* trash;  // [64][2] scratch target of record stores that have no row
  R* S_theta;  // forward sensitivities dy1/dtheta [D][P][n] (solve_kernel<..., true>)
  // Two-phase solve (solve_kernel<..., PHASED>): phase 1 runs the first
  // `probe` attempts of every trajectory and suspends the unfinished ones
  // (state into `save`, an ordering key into `key`); phase 2 resumes them in
  // the queue order `order`.
  int phase;              // 1 or 2
  int32_t probe;          // attempts per trajectory in phase 1
  R* save;                // [n][save_stride]: y, f(y), t, h (and S) of a suspended trajectory
  int32_t* save_i;        // [n][2]: accepted count; rejected count * 2 + last-rejected flag
  int32_t* key;           // [n] phase 1: predicted remaining attempts, log scale
  const int32_t* order;   // [n] phase 2: queue position -> trajectory
};

// Ordering key of a suspended trajectory: its remaining attempts predicted
// from the time the probe attempts covered, 200 log2(1 + r) capped at
// ORDER_KEY_MAX (the sort's bins).
constexpr int ORDER_KEY_MAX = 4095;

template <class R>
struct GradArgs {
  int64_t n;
  const R* theta;
  const R* y0;
  int64_t s_cap;
  const R* h_rec;
  const int32_t* count;
  const int32_t* status;
  int64_t s_max;
  const R* dLdy1;
  R* dLdtheta;
  R* dLdy0;
  R* scratch;
  const R* y_rec;  // optional recorded states [n][s_cap][D] (skip the forward replay)
  const int32_t* perm;
  unsigned long long* groups;
  // Cotangents at requested times (grad_kernel<..., true>): L also holds
  // sum_q <dLdyq[q], y(tq[q])>, y(tau) the shortened step of the method from
  // the start of the accepted step that holds tau.  m times tq[m] shared by
  // the ensemble, ascending in [t0, t1]; dLdyq [m][D][n]; dLdy1 may be null.
  int64_t m;
  const R* tq;
  const R* dLdyq;
  R t0, t1;
};

// The attempt's error test: the embedded error is e_c = s a_c (a_c the
// unscaled stage combination, s = h for Tsit5 and h/6 for Rosenbrock23) and
// its scaled component e_c / sc_c is formed as a_c w_c with the weight
// w_c = s / sc_c.  The weights depend only on h and the two states, so their
// divisions run while the last stage is still being evaluated and only one
// multiply sits between the last stage and the accept decision.  Mean of
// squares in component order, times the constant 1/D.
template <class R, int D>
__device__ __forceinline__ R error_msq(const R (&a)[D], const R (&w)[D]) {
  R r = a[0] * w[0];
  R acc = r * r;
#pragma unroll
  for (int c = 1; c < D; ++c) {
    r = a[c] * w[c];
    acc = fmaR(r, r, acc);
  }
  return acc * R(1.0 / D);
}

// Mean of squares of x_c / sc_c (the starting step's norms): summed in
// component order, the mean taken as a product with the constant 1/D.
template <class R, int D>
__device__ __forceinline__ R mean_sq(const R (&e)[D], const R (&sc)[D]) {
  R r = e[0] / sc[0];
  R acc = r * r;
#pragma unroll
  for (int c = 1; c < D; ++c) {
    r = e[c] / sc[c];
    acc = fmaR(r, r, acc);
  }
  return acc * R(1.0 / D);
}

// Starting step: Hairer, Norsett & Wanner, Solving ODEs I, Sec. II.4, with
// exponent 1/order; truncated like the controller factors.
template <class R, class Sys>
__device__ R initial_step(const Sys& sys, const R (&y0)[Sys::D], const R (&f0)[Sys::D], R span,
                          R rtol, R atol, int order) {
  constexpr int D = Sys::D;
  R sc[D], y1[D], f1[D], df[D];
#pragma unroll
  for (int c = 0; c < D; ++c) sc[c] = fmaR(rtol, absR(y0[c]), atol);
  R d0 = sqrtR(mean_sq<R, D>(y0, sc));
  R d1 = sqrtR(mean_sq<R, D>(f0, sc));
  R h0 = (d0 < R(1e-5) || d1 < R(1e-5)) ? R(1e-6) : R(0.01) * (d0 / d1);
  h0 = (span < h0) ? span : h0;
#pragma unroll
  for (int c = 0; c < D; ++c) y1[c] = fmaR(h0, f0[c], y0[c]);
  sys.f(y1, f1);
#pragma unroll
  for (int c = 0; c < D; ++c) df[c] = f1[c] - f0[c];
  R d2 = sqrtR(mean_sq<R, D>(df, sc)) / h0;
  R m = (d1 < d2) ? d2 : d1;
  R h1;
  if (m <= R(1e-15)) {
    R t = h0 * R(1e-3);
    h1 = (R(1e-6) < t) ? t : R(1e-6);
  } else {
    h1 = powR(R(0.01) / m, R(1) / R(order));
  }
  R h100 = R(100) * h0;
  return truncBits((h1 < h100) ? h1 : h100);
}

// SENS: also integrate the forward sensitivities S = dy/dtheta beside the
// state, with the steps chosen on the state alone (arXiv 2609.28458 Sec. 2.3
// and Sec. 3).  S starts at zero, takes the tangent of every accepted step
// and is written to S_theta when the trajectory finishes.
template <class R, class Sys, int METHOD, bool SENS = false, bool PHASED = false>
__global__ void __launch_bounds__(256) solve_kernel(SolveArgs<R> a) {
  constexpr int D = Sys::D;
  constexpr int NS = SENS ? Sys::P : 1;
  R Sv[D][NS];
  int sdir[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) sdir[j] = j;
  constexpr int ORDER = (METHOD == M_VERN7) ? 7 : (METHOD == M_ROS23) ? 2 : 5;
  // msq^(-1/Q) = err^(-1/(p+1)), p the pair's lower order (Tsit5 and Rodas5P 4,
  // Verner 7 6, Rosenbrock23 2)
  constexpr int CTRL_Q = (METHOD == M_VERN7) ? 14 : (METHOD == M_ROS23) ? 6 : 10;
  constexpr int NK = (METHOD == M_VERN7) ? 10 : 7;  // stage derivatives per attempt
  constexpr int32_t RUNNING = -1;
  const int lane = laneId();
  R* const trash = a.trash + 2 * lane;
  // Tsit5 coefficients pinned to registers where the state is small enough
  // that the extra 56 registers cost no occupancy (larger states keep the
  // literals: more resident wavefronts matter more there).
  tsit5::Coef<R> C5;
  if constexpr (METHOD == M_TSIT5) C5 = (Sys::D <= 4) ? tsit5::Coef<R>::pinned() : tsit5::Coef<R>::literal();
  // the controller's coefficients likewise (with the Tsit5 table pinned the
  // scalar registers would otherwise overflow)
  const CtrlCoef<R, CTRL_Q> KC = CtrlCoef<R, CTRL_Q>::make(METHOD == M_TSIT5 && Sys::D <= 4);
  // the power's fractional factor for its CTRL_Q possible arguments, once
  __shared__ R ctrl_tab[16];
  if (threadIdx.x < CTRL_Q) ctrl_tab[threadIdx.x] = ctrl_frac<R, CTRL_Q>((int)threadIdx.x, KC);
  __syncthreads();

  Sys sys;
  R y[D];
  R k[NK][D];  // stages, k[0] = f(y) (Tsit5: FSAL); Rosenbrock23: k[0] = F0 = f(y)
  R t = R(0), h = R(0);
  int32_t nacc = 0, nrej = 0;
  int64_t attempts = 0;
  bool prev_rej = false;
  int64_t traj = -1;
  bool live = true;
  R* hrow = nullptr;
  R* trow = nullptr;
  R* yrow = nullptr;

  // Record staging.  A lane keeps its last STAGE entries (t, h and, when
  // states are recorded, y) in an LDS ring (slot-major, lane-minor) and
  // writes them out as one aligned chunk per array whenever its count
  // reaches a multiple of STAGE, so the record reaches memory in whole
  // chunks instead of 8-byte pieces scattered over 64 rows.  A trajectory's
  // last partial chunk is written entry by entry when it finishes.  Records
  // whose capacity is not a multiple of STAGE are written directly.  The
  // ring is dynamic LDS: ring_arrays(with states) x STAGE x 64 values per
  // wavefront.
  constexpr int STAGE = 8;
  const bool with_t = a.t_rec != nullptr;
  const bool with_y = a.y_rec != nullptr;
  HIP_DYNAMIC_SHARED(unsigned char, dyn_lds)
  R* const wring = (R*)dyn_lds + (threadIdx.x / WAVE) * ((with_y ? 2 + D : 2) * STAGE * WAVE);
  R(*const hring)[WAVE] = (R(*)[WAVE])wring;
  R(*const tring)[WAVE] = (R(*)[WAVE])(wring + STAGE * WAVE);
  auto yring = [&](int c, int slot) -> R& { return wring[((2 + c) * STAGE + slot) * WAVE + lane]; };
  const bool staged = (a.s_cap % STAGE) == 0 && ((uintptr_t)a.h_rec % 16) == 0 &&
                      ((uintptr_t)a.t_rec % 16) == 0 && ((uintptr_t)a.y_rec % 16) == 0;

  auto finish = [&](int32_t st) {
#pragma unroll
    for (int c = 0; c < D; ++c) a.y1[c * a.n + traj] = (st == TRAJ_OK) ? y[c] : nanR(R(0));
    a.count[traj] = nacc;
    if (a.nrej) a.nrej[traj] = nrej;
    a.status[traj] = st;
    if constexpr (PHASED) {
      if (a.phase == 1) a.key[traj] = 0;  // done: nothing left to order
    }
    if constexpr (SENS) {
#pragma unroll
      for (int c = 0; c < D; ++c)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          a.S_theta[(c * NS + j) * a.n + traj] = (st == TRAJ_OK) ? Sv[c][j] : nanR(R(0));
    }
    if (staged) {
      const int32_t lo = nacc & ~(STAGE - 1);
      for (int32_t r = lo; r < nacc; ++r) {
        hrow[r] = hring[r & (STAGE - 1)][lane];
        if (with_t) trow[r] = tring[r & (STAGE - 1)][lane];
        if (with_y) {
#pragma unroll
          for (int c = 0; c < D; ++c) yrow[r * D + c] = yring(c, r & (STAGE - 1));
        }
      }
    }
    traj = -1;
  };

  // Phase 1 of a two-phase solve: park an unfinished trajectory.  Its state
  // for the next attempt goes to a.save, its unwritten record rows to memory
  // (phase 2 reloads them into the ring), and status stays RUNNING.
  auto suspend = [&]() {
    R* const sv = a.save + traj * save_stride<R, D, Sys::P>();
#pragma unroll
    for (int c = 0; c < D; ++c) {
      sv[c] = y[c];
      sv[D + c] = k[0][c];
    }
    sv[2 * D] = t;
    sv[2 * D + 1] = h;
    if constexpr (SENS) {
#pragma unroll
      for (int c = 0; c < D; ++c)
#pragma unroll
        for (int j = 0; j < NS; ++j) sv[2 * D + 2 + c * NS + j] = Sv[c][j];
    }
    a.save_i[2 * traj] = nacc;
    a.save_i[2 * traj + 1] = nrej * 2 + (prev_rej ? 1 : 0);
    a.status[traj] = RUNNING;
    const double done = (double)(t - a.t0), left = (double)(a.t1 - t);
    const double rem = (done > 0.0) ? (double)attempts * left / done : 1e30;
    const double kf = 200.0 * log2(1.0 + (rem < 1e30 ? rem : 1e30));
    a.key[traj] = (kf < (double)ORDER_KEY_MAX) ? (int32_t)kf : ORDER_KEY_MAX;
    if (staged) {
      for (int32_t r = nacc & ~(STAGE - 1); r < nacc; ++r) {
        hrow[r] = hring[r & (STAGE - 1)][lane];
        if (with_t) trow[r] = tring[r & (STAGE - 1)][lane];
        if (with_y) {
#pragma unroll
          for (int c = 0; c < D; ++c) yrow[r * D + c] = yring(c, r & (STAGE - 1));
        }
      }
    }
    traj = -1;
  };

  // Work distribution.  The queue hands out batches of 64 consecutive
  // trajectories, one device-scope atomic per batch; within its batch a
  // wavefront gives the next index to whichever lane asks first (a
  // wave-uniform cursor).  Batches keep the atomic rate low when trajectories
  // are short and many per lane (one queue hit per finished trajectory
  // serialises every wavefront on one counter), while the ensemble stays
  // balanced across wavefronts.
  constexpr int64_t BATCH = WAVE;
  int64_t cursor = 0, bend = 0;  // the wavefront's current batch [cursor, bend)
  bool drained = false;          // the queue has nothing left
  for (;;) {
    const bool need = live && traj < 0;
    const unsigned long long m = __ballot(need);
    if (m) {
      const int64_t cnt_w = (int64_t)__popcll(m);
      const int64_t rank = (int64_t)__popcll(m & ((1ull << lane) - 1ull));
      const int64_t left = bend - cursor;           // indices left in the batch
      const bool more = cnt_w > left && !drained;  // take a new batch (one atomic)
      int64_t base = a.n;
      if (more) {
        unsigned long long b = 0;
        if (lane == 0) b = atomicAdd(a.queue, (unsigned long long)BATCH);
        base = (int64_t)__shfl(b, 0);
        if (base + BATCH >= a.n) drained = true;
      }
      // ranks below `left` take the rest of the batch, the others the start
      // of the new one (rank - left < 64, as at most 64 lanes ask at once)
      const int64_t kk = (rank < left) ? cursor + rank : (more ? base + (rank - left) : a.n);
      if (more) {
        bend = (base + BATCH < a.n) ? base + BATCH : a.n;
        cursor = base + (cnt_w - left);
        if (cursor > bend) cursor = bend;
      } else {
        cursor = (cursor + cnt_w < bend) ? cursor + cnt_w : bend;
      }
      if (need && kk >= a.n) live = false;  // nothing left for this lane
      // Phase 2 takes trajectories in the given order and resumes only the
      // suspended ones (a lane that drew a finished one claims again).
      int64_t tk = kk;
      bool go = need && kk < a.n;
      if (PHASED && a.phase == 2 && go) {
        tk = a.order[kk];
        go = a.status[tk] == RUNNING;
      }
      if (PHASED && a.phase == 2 && go) {
        traj = tk;
        sys.load(a.theta, a.n, traj);
        const R* const sv = a.save + traj * save_stride<R, D, Sys::P>();
#pragma unroll
        for (int c = 0; c < D; ++c) {
          y[c] = sv[c];
          k[0][c] = sv[D + c];
        }
        t = sv[2 * D];
        h = sv[2 * D + 1];
        if constexpr (SENS) {
#pragma unroll
          for (int c = 0; c < D; ++c)
#pragma unroll
            for (int j = 0; j < NS; ++j) Sv[c][j] = sv[2 * D + 2 + c * NS + j];
        }
        nacc = a.save_i[2 * traj];
        const int32_t rj = a.save_i[2 * traj + 1];
        __builtin_amdgcn_s_waitcnt(0);
        nrej = rj >> 1;
        prev_rej = (rj & 1) != 0;
        attempts = a.probe;
        hrow = a.h_rec + traj * a.s_cap;
        trow = a.t_rec ? a.t_rec + traj * a.s_cap : nullptr;
        yrow = a.y_rec ? a.y_rec + traj * a.s_cap * D : nullptr;
        if (staged) {
          // the rows of the current chunk that phase 1 wrote, back into the ring
          for (int32_t r = nacc & ~(STAGE - 1); r < nacc; ++r) {
            hring[r & (STAGE - 1)][lane] = hrow[r];
            if (with_t) tring[r & (STAGE - 1)][lane] = trow[r];
            if (with_y) {
#pragma unroll
              for (int c = 0; c < D; ++c) yring(c, r & (STAGE - 1)) = yrow[r * D + c];
            }
          }
          __builtin_amdgcn_s_waitcnt(0);
        }
      } else if (go) {
        traj = tk;
        sys.load(a.theta, a.n, traj);
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] = a.y0[c * a.n + traj];
        // Loads and stores share one in-order counter (vmcnt).  Waiting here,
        // once per trajectory, keeps the attempt loop free of waits on these
        // loads, which would otherwise also drain the record stores of every
        // previous attempt.
        __builtin_amdgcn_s_waitcnt(0);
        hrow = a.h_rec + traj * a.s_cap;
        trow = a.t_rec ? a.t_rec + traj * a.s_cap : nullptr;
        yrow = a.y_rec ? a.y_rec + traj * a.s_cap * D : nullptr;
        t = a.t0;
        nacc = 0;
        nrej = 0;
        if constexpr (SENS) {
#pragma unroll
          for (int c = 0; c < D; ++c)
#pragma unroll
            for (int j = 0; j < NS; ++j) Sv[c][j] = R(0);
        }
        attempts = 0;
        prev_rej = false;
        if (!(a.t1 > a.t0)) {
          finish(TRAJ_OK);
        } else {
          sys.f(y, k[0]);
          h = (a.dt0 > R(0)) ? a.dt0 : initial_step<R, Sys>(sys, y, k[0], a.t1 - a.t0, a.rtol, a.atol, ORDER);
        }
      }
    }
    if (__ballot(live) == 0ull) break;
    if (traj < 0) continue;

    // ---- one attempted step.  Both outcomes are applied by selects; the
    // only branch is the (rare) exit of a finished or failed trajectory.
    ++attempts;
    const bool last = (t + h >= a.t1);
    const R hs = last ? (a.t1 - t) : h;
    R ynew[D], err[D], F2[D];
    if constexpr (METHOD == M_TSIT5) {
      tsit5::trial<R, Sys>(C5, sys, y, hs, k, ynew, err);
    } else if constexpr (METHOD == M_VERN7) {
      vern7::trial<R, Sys>(sys, y, hs, k, ynew, err);
      sys.f(ynew, F2);  // not FSAL: f at the new state, kept if the step is taken
    } else if constexpr (METHOD == M_RODAS5P) {
      rodas5p::trial<R, Sys>(sys, y, hs, k[0], ynew, err);
      sys.f(ynew, F2);  // not FSAL
    } else {
      ros23::trial<R, Sys, !SENS>(sys, y, hs, k[0], ynew, F2, err);
    }
    // the estimate's factor: h (explicit pairs), h/6 (Rosenbrock23), 1 (Rodas5P).
    // The weights s / sc_c only scale the mean square, whose accept test and
    // 16-bit-truncated controller factor absorb differences of a few ulp (a
    // flip needs msq within ~3e-15 relative of 1 or of a truncation
    // boundary), so they are formed with the hardware reciprocal and one
    // Newton step (rcpW, within 11 ulp), not IEEE division.
    // max(|y_c|, |y_new,c|) is one instruction (absmaxR: equal to the
    // comparison's choice for every non-NaN pair; a NaN state fails the step
    // either way, through msq).
    const R es = (METHOD == M_ROS23) ? hs * R(1.0 / 6.0) : (METHOD == M_RODAS5P) ? R(1) : hs;
    R wt[D];
#pragma unroll
    for (int c = 0; c < D; ++c)
      wt[c] = es * rcpW(fmaR(a.rtol, absmaxR(y[c], ynew[c]), a.atol));
    const R msq = error_msq<R, D>(err, wt);
    const bool acc = msq <= R(1);
    // One controller evaluation serves both outcomes.
    const R root = ctrl_root_tab<R, CTRL_Q>(msq, KC, ctrl_tab);
    const R fq = (msq == R(0)) ? R(10) : truncBits(R(0.9) * root);
    const R fmin = (R(0.2) < fq) ? fq : R(0.2);

    // Failure checks in the solve's order of precedence, as selects (the
    // lowest-precedence check is applied first and overridden).
    int32_t st = (acc && nacc >= a.s_cap) ? TRAJ_CAPACITY : RUNNING;
    st = finiteR(msq) ? st : TRAJ_NONFINITE;
    st = (t + hs > t) ? st : TRAJ_DT_UNDERFLOW;
    st = finiteR(hs) ? st : TRAJ_NONFINITE;

    // Record row nacc: an accepted step keeps it, a rejected one is
    // overwritten by the next accepted step (rows past count are unused).
    if (staged) {
      hring[nacc & (STAGE - 1)][lane] = hs;
      if (with_t) tring[nacc & (STAGE - 1)][lane] = t;
      if (with_y) {
#pragma unroll
        for (int c = 0; c < D; ++c) yring(c, nacc & (STAGE - 1)) = y[c];
      }
    } else {
      // With the record full, the store goes to the lane's trash slot.
      const bool room = nacc < a.s_cap;
      *(room ? hrow + nacc : trash) = hs;
      if (with_t) *(room ? trow + nacc : trash + 1) = t;
      if (with_y && room) {
#pragma unroll
        for (int c = 0; c < D; ++c) yrow[nacc * D + c] = y[c];
      }
    }

    const bool take = (st == RUNNING) && acc;
    const R tn = last ? a.t1 : t + hs;
    static_assert(!(SENS && (METHOD == M_VERN7 || METHOD == M_RODAS5P)),
                  "in-solve sensitivities are for Tsit5 and Rosenbrock23");
    if constexpr (SENS) {
      if (take) {
        if constexpr (METHOD == M_TSIT5) {
          tsit5::tangent<R, Sys, NS>(C5, sys, y, hs, k, sdir, Sv);
        } else {
          ros23::Stages<R, D> St;  // the step's factors and stages, recomputed
          ros23::stages<R, Sys, false>(sys, y, hs, St);
          ros23::tangent<R, Sys, NS, false>(sys, St, hs, sdir, Sv);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = take ? ynew[c] : y[c];
    if constexpr (METHOD == M_TSIT5) {
#pragma unroll
      for (int c = 0; c < D; ++c) k[0][c] = take ? k[6][c] : k[0][c];
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) k[0][c] = take ? F2[c] : k[0][c];
    }
    t = take ? tn : t;
    nacc += take ? 1 : 0;
    nrej += (st == RUNNING && !acc) ? 1 : 0;
    if (staged && take && (nacc & (STAGE - 1)) == 0) {
      // A full chunk: rows [nacc - STAGE, nacc), 64-byte aligned.
      const int32_t lo = nacc - STAGE;
      typedef R R2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int r = 0; r < STAGE; r += 2) {
        *(R2*)(hrow + lo + r) = R2{hring[r][lane], hring[r + 1][lane]};
        if (with_t) *(R2*)(trow + lo + r) = R2{tring[r][lane], tring[r + 1][lane]};
      }
      if (with_y) {
        // rows lo .. lo + STAGE - 1 of D values each: STAGE * D contiguous values
#pragma unroll
        for (int e = 0; e < STAGE * D; e += 2)
          *(R2*)(yrow + lo * D + e) =
              R2{yring(e % D, e / D), yring((e + 1) % D, (e + 1) / D)};
      }
    }
    R fa = (fmin < R(10)) ? fmin : R(10);
    fa = (prev_rej && fa > R(1)) ? R(1) : fa;
    h = hs * (acc ? fa : fmin);
    prev_rej = !acc;
    if (st == RUNNING) {
      if (take && !(tn < a.t1)) st = TRAJ_OK;
      else if (attempts >= a.max_steps) st = TRAJ_MAX_STEPS;
    }
    if (st != RUNNING) finish(st);
    else if (PHASED && a.phase == 1 && attempts >= a.probe) suspend();
  }
}

// Reads one record row per lane forward in a loop whose step index is the
// same in every lane.  Each lane reads its own row: read eight bytes per
// step, a row's lines are fetched again whenever they leave the cache
// between two steps, and the record is read several times over.  Here the
// row goes in 64-byte chunks (four 16-byte loads per lane) through an LDS
// ring of two 8-step chunks (ring: this wavefront's 16 x 64 values); the
// chunk after the current one is requested when the current one enters the
// ring, so each piece is fetched once and has a chunk's worth of steps to
// arrive.  Call at(i) for i = 0, 1, 2, ... < mx in order.  Requires
// s_cap % 8 == 0 (a chunk at 8c < mx <= s_cap stays in the row) and a
// 16-byte aligned row.
template <class R>
struct RowRing {
  typedef R R2 __attribute__((ext_vector_type(2)));
  R (*ring)[WAVE];
  const R* row;
  int mx, lane;
  R nx[8];
  __device__ __forceinline__ void request(int c) {
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const R2 v = *(const R2*)(row + 8 * c + u);
      nx[u] = v.x;
      nx[u + 1] = v.y;
    }
  }
  __device__ __forceinline__ void put(int c) {
#pragma unroll
    for (int u = 0; u < 8; ++u) ring[8 * (c & 1) + u][lane] = nx[u];
  }
  __device__ __forceinline__ void init(R (*ring_)[WAVE], const R* row_, int mx_, int lane_) {
    ring = ring_;
    row = row_;
    mx = mx_;
    lane = lane_;
#pragma unroll
    for (int u = 0; u < 8; ++u) nx[u] = R(0);
    if (mx > 0) {
      request(0);
      put(0);
      if (8 < mx) request(1);
    }
  }
  __device__ __forceinline__ R at(int i) {
    if (i > 0 && (i & 7) == 0) {
      put(i >> 3);
      if (i + 8 < mx) request((i >> 3) + 1);
    }
    return ring[i & 15][lane];
  }
};

// The gradient kernel's LDS per wavefront (reals): the forward replay's ring
// of record h (16 x 64), and, for Rodas5P on systems whose reverse step does
// not fit the registers, the reverse step's stage solutions (8 x D x 64; the
// ring is dead by then, so the two share the area).
template <class Sys, int METHOD>
constexpr bool rodas_stages_in_lds() {
  return METHOD == M_RODAS5P && Sys::D >= 8;
}
template <class Sys, int METHOD>
constexpr int grad_lds_reals() {
  return (rodas_stages_in_lds<Sys, METHOD>() && 8 * Sys::D > 16 ? 8 * Sys::D : 16) * WAVE;
}

// AT: the loss also holds cotangents of the states at requested times
// (application paper arXiv 2609.28458 Sec. 2.3 fits residuals at observation
// times; the states are those of states_kernel).  The forward pass assigns
// each requested time to the step that holds it (per lane: that step's index
// and the offset tau - t_j, in a table after the wavefront's tile); before
// the reverse sweep every lane takes the vector-Jacobian product of the
// shortened step Phi(y_J; tau - t_J) with each time's cotangent (time by
// time, all lanes together), and the sweep adds it to lam once it has taken
// lam through step J.
//
// Register budgets (measured choices): Rosenbrock23 with d <= 3 is held to
// 128 registers, four wavefronts per SIMD; Verner 7 without requested times
// to 256, two wavefronts per SIMD (one wavefront with its overflow in
// accumulation registers was slower); with requested times the spills would
// be many and one wavefront is faster.  Tsit5 with requested times and
// d <= 6 is held to 256 as well: the orbit's kernel needs two registers more
// (two spilled; without the cap it ran one wavefront per SIMD, ~10 % slower).
template <class R, class Sys, int METHOD, bool AT = false>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu((METHOD == M_ROS23 && Sys::D <= 3) ? 4
                                   : ((METHOD == M_VERN7 && !AT) ||
                                      (METHOD == M_TSIT5 && AT && Sys::D <= 6)) ? 2 : 1)))
grad_kernel(GradArgs<R> a) {
  constexpr int D = Sys::D, P = Sys::P;
  const int lane = laneId();
  // Tsit5 coefficients pinned to registers where the state is small enough
  // that the extra 56 registers cost no occupancy (larger states keep the
  // literals: more resident wavefronts matter more there).
  tsit5::Coef<R> C5;
  if constexpr (METHOD == M_TSIT5) C5 = (Sys::D <= 4) ? tsit5::Coef<R>::pinned() : tsit5::Coef<R>::literal();
  const int64_t slot = (int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  // per wavefront: the tile [s_max][D + 1][64], then (AT) the tables
  // [m][2][64] (step index and offset of each time) and [m][D][64] (its VJP)
  const int64_t tile = (a.s_max > 0 ? a.s_max : 1) * (D + 1) * WAVE;
  R* scr = a.scratch + slot * (tile + (AT ? a.m * (2 + D) * WAVE : 0)) + lane;
  R* const qt = scr + tile;
  // (AT) the requested times must be ascending in [t0, t1]; otherwise every
  // output is NaN (the same test for every lane)
  bool tq_ok = true;
  if constexpr (AT) {
    R prev = a.t0;
    for (int64_t q = 0; q < a.m; ++q) {
      const R tau = a.tq[q];
      tq_ok = tq_ok && tau >= a.t0 && tau <= a.t1 && tau >= prev;
      prev = tau;
    }
  }
  const unsigned long long ngroups = (unsigned long long)((a.n + WAVE - 1) / WAVE);

  for (;;) {
    unsigned long long g = 0;
    if (lane == 0) g = atomicAdd(a.groups, 1ull);
    g = __shfl(g, 0);
    if (g >= ngroups) break;
    const int64_t idx = (int64_t)g * WAVE + lane;
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
      }
    }
    int mx = cnt;
#pragma unroll
    for (int off = WAVE / 2; off > 0; off >>= 1) {
      const int o = __shfl_xor(mx, off);
      mx = (o > mx) ? o : mx;
    }

    // Lanes past the end of the ensemble (k < 0, count 0) run the loops below
    // on trajectory 0's parameters with a zero state; nothing of theirs is
    // written.
    Sys sys;
    R y[D], lam[D], pb[P];
    sys.load(a.theta, a.n, k >= 0 ? k : 0);
    const R* hrow = a.h_rec;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      y[c] = R(0);
      lam[c] = R(0);
    }
    if (k >= 0) {
#pragma unroll
      for (int c = 0; c < D; ++c) {
        y[c] = a.y0[c * a.n + k];
        lam[c] = (!AT || a.dLdy1) ? a.dLdy1[c * a.n + k] : R(0);
      }
      hrow = a.h_rec + k * a.s_cap;
    }
#pragma unroll
    for (int j = 0; j < P; ++j) pb[j] = R(0);

    // The group's lanes step in lockstep for mx steps.  A lane past its own
    // count takes steps of size zero: for a finite state, a zero step leaves y
    // unchanged, and its reverse leaves lam and the parameter cotangent
    // unchanged (every update is a multiple of h), so those steps are exact
    // no-ops and the loops need no per-lane branches.  Rows i < mx <= s_max
    // <= s_cap of a record are in bounds whatever their contents; rows past a
    // lane's count are loaded but not used.
    //
    // Forward replay, storing y_j before step j.  Each step's h is loaded one
    // step ahead: loads and stores retire in order (one vmcnt counter), so a
    // load issued before this step's stores is ready by the next step without
    // waiting for those stores.
    // With states recorded by the solve (valid at the theta it ran with) the
    // forward replay is skipped and y_j is read from the record, row j.
    // The states are written once and read once, long after (a wavefront's
    // tile is s_max x d x 512 bytes): they stream through the L2 as
    // nontemporal accesses, which leaves the lines of the h rows, each read
    // eight bytes per step, resident between their steps.
    // The scratch tile holds, per step, the D state components and the
    // step's h (zero past the lane's count), so that the reverse sweep reads
    // both as whole 512-byte rows instead of h again from 64 record rows.
    const bool rec_y = !AT && a.y_rec != nullptr;
    constexpr int SD = D + 1;
    int64_t qf = 0;    // (AT) requested times assigned so far
    R tcur = a.t0;     // (AT) t_j, the solve's running time
    R tnext = R(0);    // (AT) the next time to assign, kept in a register
    if constexpr (AT) {
      if (a.m > 0) tnext = a.tq[0];
    }
    const R* ysrc = rec_y ? a.y_rec + (k >= 0 ? k : 0) * a.s_cap * D : scr;
    const int64_t istr = rec_y ? D : (int64_t)SD * WAVE, cstr = rec_y ? 1 : WAVE;
    R h_nx = (mx > 0) ? hrow[0] : R(0);
    if (!rec_y) {
      // (the record's h a chunk at a time through the LDS ring, where the
      // record's layout allows it)
      const bool rows8 = (a.s_cap % 8) == 0 && ((uintptr_t)a.h_rec % 16) == 0;
      auto fwd = [&](int i, R hv) {
        const R hj = (i < cnt) ? hv : R(0);
        if constexpr (AT) {
          if (i < cnt) {
            // the times step i holds: tau < t_i + h_i, or all that are left at
            // the last step (it holds up to t1)
            while (qf < a.m) {
              if (!(i == cnt - 1 || tnext < tcur + hj)) break;
              qt[(qf * 2) * WAVE] = R(i);
              qt[(qf * 2 + 1) * WAVE] = tnext - tcur;
              ++qf;
              if (qf < a.m) tnext = a.tq[qf];
            }
            tcur = tcur + hj;
          }
        }
#pragma unroll
        for (int c = 0; c < D; ++c)
          __builtin_nontemporal_store(y[c], &scr[((int64_t)i * SD + c) * WAVE]);
        __builtin_nontemporal_store(hj, &scr[((int64_t)i * SD + D) * WAVE]);
        if constexpr (METHOD == M_TSIT5)
          tsit5::replay<R, Sys>(C5, sys, y, hj);
        else if constexpr (METHOD == M_VERN7)
          vern7::replay<R, Sys>(sys, y, hj);
        else if constexpr (METHOD == M_RODAS5P)
          rodas5p::replay<R, Sys>(sys, y, hj);
        else
          ros23::replay<R, Sys>(sys, y, hj);
      };
      if (rows8) {
        HIP_DYNAMIC_SHARED(unsigned char, gr_lds)
        RowRing<R> rr;
        rr.init((R(*)[WAVE])((R*)gr_lds + (threadIdx.x / WAVE) * grad_lds_reals<Sys, METHOD>()),
                hrow, mx, lane);
        for (int i = 0; i < mx; ++i) fwd(i, rr.at(i));
      } else {
        for (int i = 0; i < mx; ++i) {
          const R hv = h_nx;
          if (i + 1 < mx) h_nx = hrow[i + 1];
          fwd(i, hv);
        }
      }
    }
    // (AT) Phase A: the reverse of the shortened step to every requested
    // time, v_q = (d Phi(y_J; tau_q - t_J) / d y_J)^T dLdyq[q] with its
    // parameter part added to pb.  None of it depends on lam, so all lanes
    // take time q together (one unit each per iteration, whatever step holds
    // it); the reverse sweep below adds v_q to lam_J once step J is done.
    R* const vt = qt + a.m * 2 * WAVE;  // table [m][D][64]
    int64_t qp = qf;                     // times whose v_q is not yet added
    R nextJ = R(-1);                     // the step holding time qp - 1
    if constexpr (AT) {
      for (int64_t q = 0; q < a.m; ++q) {
        const bool has = q < qf;  // assigned (lanes with steps have all m)
        R hq = R(0), yq[D], lq[D];
#pragma unroll
        for (int c = 0; c < D; ++c) yq[c] = lq[c] = R(0);
        if (has) {
          const int64_t J = (int64_t)qt[(q * 2) * WAVE];
          hq = qt[(q * 2 + 1) * WAVE];
#pragma unroll
          for (int c = 0; c < D; ++c) {
            yq[c] = __builtin_nontemporal_load(&scr[(J * SD + c) * WAVE]);
            lq[c] = a.dLdyq[(q * D + c) * a.n + k];
          }
        }
        if constexpr (METHOD == M_TSIT5) {
          tsit5::Stages<R, D> S;
          tsit5::stages<R, Sys>(C5, sys, yq, hq, S);
          tsit5::sweep<R, Sys>(C5, sys, S, hq, lq, pb);
        } else if constexpr (METHOD == M_VERN7) {
          vern7::Stages<R, D> S;
          vern7::stages<R, Sys>(sys, yq, hq, S);
          vern7::sweep<R, Sys>(sys, S, hq, lq, pb);
        } else if constexpr (METHOD == M_RODAS5P) {
          rodas5p::Stages<R, D> S;
          rodas5p::stages<R, Sys>(sys, yq, hq, S);
          rodas5p::sweep<R, Sys>(sys, S, hq, lq, pb);
        } else {
          ros23::Stages<R, D> S;
          ros23::stages<R, Sys>(sys, yq, hq, S);
          ros23::sweep<R, Sys>(sys, S, hq, lq, pb);
        }
        if (has) {
#pragma unroll
          for (int c = 0; c < D; ++c) vt[(q * D + c) * WAVE] = lq[c];
        }
      }
      if (qp > 0) nextJ = qt[((qp - 1) * 2) * WAVE];
    }
    {
      // Reverse sweep, with y_j and h_j of the next step (j - 1) prefetched the
      // same way.  Past a lane's count the state is taken as zero (recorded rows
      // there are unspecified), which keeps the zero-size steps exact no-ops.
      // (Recomputing step j - 1's stages during step j's sweep, for two
      // independent chains per iteration, measured no faster on any workload.)
      R y_nx[D];
#pragma unroll
      for (int c = 0; c < D; ++c) y_nx[c] = R(0);
      h_nx = R(0);
      // h of row i: from the tile (zero past the count already), or the record
      auto h_at = [&](int i) -> R {
        return rec_y ? hrow[i] : __builtin_nontemporal_load(&scr[((int64_t)i * SD + D) * WAVE]);
      };
      if (mx > 0) {
#pragma unroll
        for (int c = 0; c < D; ++c)
          y_nx[c] = __builtin_nontemporal_load(&ysrc[(int64_t)(mx - 1) * istr + c * cstr]);
        h_nx = h_at(mx - 1);
      }
      for (int i = mx - 1; i >= 0; --i) {
        R yj[D];
        const R hj = (i < cnt) ? h_nx : R(0);
#pragma unroll
        for (int c = 0; c < D; ++c) yj[c] = (i < cnt) ? y_nx[c] : R(0);
        if (i >= 1) {
#pragma unroll
          for (int c = 0; c < D; ++c)
            y_nx[c] = __builtin_nontemporal_load(&ysrc[(int64_t)(i - 1) * istr + c * cstr]);
          h_nx = h_at(i - 1);
        }
        if constexpr (METHOD == M_TSIT5) {
          tsit5::Stages<R, D> S;
          tsit5::stages<R, Sys>(C5, sys, yj, hj, S);
          tsit5::sweep<R, Sys>(C5, sys, S, hj, lam, pb);
        } else if constexpr (METHOD == M_VERN7) {
          vern7::Stages<R, D> S;
          vern7::stages<R, Sys>(sys, yj, hj, S);
          vern7::sweep<R, Sys>(sys, S, hj, lam, pb);
        } else if constexpr (METHOD == M_RODAS5P) {
          rodas5p::Stages<R, D> S;
          rodas5p::stages<R, Sys>(sys, yj, hj, S);
          if constexpr (rodas_stages_in_lds<Sys, METHOD>()) {
            HIP_DYNAMIC_SHARED(unsigned char, rs_lds)
            R* const us = (R*)rs_lds + (threadIdx.x / WAVE) * grad_lds_reals<Sys, METHOD>() + lane;
            rodas5p::put_stages(S, us);
            rodas5p::sweep_lds<R, Sys>(sys, S.w, yj, hj, us, lam, pb);
          } else {
            rodas5p::sweep<R, Sys>(sys, S, hj, lam, pb);
          }
        } else {
          ros23::Stages<R, D> S;
          ros23::stages<R, Sys>(sys, yj, hj, S);
          ros23::sweep<R, Sys>(sys, S, hj, lam, pb);
        }
        if constexpr (AT) {
          // lam_i gains v_q of every time step i holds
          while (qp > 0 && nextJ == R(i)) {
#pragma unroll
            for (int c = 0; c < D; ++c) lam[c] += vt[((qp - 1) * D + c) * WAVE];
            --qp;
            nextJ = (qp > 0) ? qt[((qp - 1) * 2) * WAVE] : R(-1);
          }
        }
      }
    }
    if constexpr (AT) {
      // a trajectory with no steps (t0 = t1): y(tau) = y0 for every time
      if (tq_ok && k >= 0 && ok && cnt == 0) {
        for (int64_t q = 0; q < a.m; ++q)
#pragma unroll
          for (int c = 0; c < D; ++c) lam[c] += a.dLdyq[(q * D + c) * a.n + k];
      }
    }
    if (k >= 0) {
      if (!ok || !tq_ok) {
#pragma unroll
        for (int c = 0; c < D; ++c) lam[c] = nanR(R(0));
#pragma unroll
        for (int j = 0; j < P; ++j) pb[j] = nanR(R(0));
      }
      if (a.dLdtheta) {
#pragma unroll
        for (int j = 0; j < P; ++j) a.dLdtheta[j * a.n + k] = pb[j];
      }
      if (a.dLdy0) {
#pragma unroll
        for (int c = 0; c < D; ++c) a.dLdy0[c * a.n + k] = lam[c];
      }
    }
  }
}

// ------------------------------------------------------------------------
// Forward sensitivities through the replay of a record (arXiv 2609.28458
// Sec. 2.3; arXiv 2609.02876 Sec. 3.1 replays the recorded steps): per
// trajectory, the tangent of y_{j+1} = Phi(y_j; h_j, theta) along NT
// directions dir0 .. dir0 + NT - 1 of (theta_0 .. theta_{P-1}, y0_0 ..
// y0_{D-1}); directions past the last are carried as zero columns and not
// written.  Trajectories are visited in the gradient's sorted groups of 64.
template <class R>
struct SensArgs {
  int64_t n;
  const R* theta;
  const R* y0;
  int64_t s_cap;
  const R* h_rec;
  const int32_t* count;
  const int32_t* status;
  int64_t s_max;
  R* S_theta;  // [D][P][n] or null
  R* S_y0;     // [D][D][n] or null
  int dir0;    // first direction of this pass
  const int32_t* perm;
  unsigned long long* groups;
  bool chunked;  // read h in chunks through an LDS ring (16 x 64 values per wavefront)
};

template <class R, class Sys, int METHOD, int NT>
__global__ void __launch_bounds__(256) sens_kernel(SensArgs<R> a) {
  constexpr int D = Sys::D, P = Sys::P;
  const int lane = laneId();
  const tsit5::Coef<R> C5 = tsit5::Coef<R>::literal();
  int dir[NT], pdir[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    dir[t] = a.dir0 + t;
    pdir[t] = dir[t] < P ? dir[t] : -1;  // parameter index, or none
  }
  const unsigned long long ngroups = (unsigned long long)((a.n + WAVE - 1) / WAVE);
  for (;;) {
    unsigned long long g = 0;
    if (lane == 0) g = atomicAdd(a.groups, 1ull);
    g = __shfl(g, 0);
    if (g >= ngroups) break;
    const int64_t idx = (int64_t)g * WAVE + lane;
    int64_t k = -1;
    int cnt = 0;
    bool ok = false;
    if (idx < a.n) {
      k = a.perm ? (int64_t)a.perm[idx] : idx;
      if (k < 0 || k >= a.n) {
        k = -1;
      } else {
        cnt = a.count[k];
        ok = cnt >= 0 && cnt <= a.s_max && (a.status == nullptr || a.status[k] == TRAJ_OK);
        if (!ok) cnt = 0;
      }
    }
    int mx = cnt;
#pragma unroll
    for (int off = WAVE / 2; off > 0; off >>= 1) {
      const int o = __shfl_xor(mx, off);
      mx = (o > mx) ? o : mx;
    }
    Sys sys;
    sys.load(a.theta, a.n, k >= 0 ? k : 0);
    R y[D], S[D][NT];
    const R* hrow = a.h_rec;
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = (k >= 0) ? a.y0[c * a.n + k] : R(0);
    if (k >= 0) hrow = a.h_rec + k * a.s_cap;
#pragma unroll
    for (int c = 0; c < D; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) S[c][t] = (dir[t] - P == c) ? R(1) : R(0);
    // Lockstep steps; past a lane's count h = 0, which leaves y and S
    // unchanged.  h is read a chunk at a time through the LDS ring where the
    // record's layout allows (a.chunked), else loaded one step ahead.
    auto step = [&](int i, R hv) {
      const R hj = (i < cnt) ? hv : R(0);
      if constexpr (METHOD == M_TSIT5) {
        R kk[7][D], Y[D];
        sys.f(y, kk[0]);
#pragma unroll
        for (int st = 1; st < 6; ++st) {
          tsit5::stage_state<R, D>(C5, st, y, hj, kk, Y);
          sys.f(Y, kk[st]);
        }
        tsit5::tangent<R, Sys, NT>(C5, sys, y, hj, kk, pdir, S);
        tsit5::stage_state<R, D>(C5, 6, y, hj, kk, Y);
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] = Y[c];
      } else {
        ros23::Stages<R, D> St;
        ros23::stages<R, Sys, false>(sys, y, hj, St);
        ros23::tangent<R, Sys, NT, false>(sys, St, hj, pdir, S);
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] = fmaR(hj, St.u[c] + St.k1[c], y[c]);  // as ros23::replay
      }
    };
    if (a.chunked) {
      HIP_DYNAMIC_SHARED(unsigned char, sn_lds)
      RowRing<R> rr;
      rr.init((R(*)[WAVE])((R*)sn_lds + (threadIdx.x / WAVE) * (16 * WAVE)), hrow, mx, lane);
      for (int i = 0; i < mx; ++i) step(i, rr.at(i));
    } else {
      R h_nx = (mx > 0) ? hrow[0] : R(0);
      for (int i = 0; i < mx; ++i) {
        const R hv = h_nx;
        if (i + 1 < mx) h_nx = hrow[i + 1];
        step(i, hv);
      }
    }
    if (k >= 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = dir[t];
#pragma unroll
        for (int c = 0; c < D; ++c) {
          const R v = ok ? S[c][t] : nanR(R(0));
          if (d < P) {
            if (a.S_theta) a.S_theta[(c * P + d) * a.n + k] = v;
          } else if (d < P + D) {
            if (a.S_y0) a.S_y0[(c * D + (d - P)) * a.n + k] = v;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// States at requested times on a recorded mesh (arXiv 2609.28458 Sec. 2.3
// and Appendix A: a shortened step from the start of the accepted step that
// holds the time; arXiv 2609.02876: the replay engines integrate one extra
// step to each requested time).  Step j spans [t_j, t_j + h_j], t_0 = t0,
// t_{j+1} = t_j + h_j (the solve's own time update); the last step holds up
// to t1.  Each lane walks its trajectory's steps and the shared, ascending
// requested times together; every iteration takes exactly one step of the
// method per lane, either the next recorded step (advance) or the shortened
// step to the next requested time (write), so the lockstep loop is
// branch-free.  A requested time outside [t0, t1], not a number, or below its
// predecessor gives NaN; a failed trajectory gives NaN throughout.
template <class R>
struct StatesArgs {
  int64_t n;
  const R* theta;
  const R* y0;
  R t0, t1;
  int64_t s_cap;
  const R* h_rec;
  const int32_t* count;
  const int32_t* status;
  int64_t s_max;
  int64_t m;
  const R* tq;  // [m]
  R* yq;        // [m][D][n]
  const int32_t* perm;
  unsigned long long* groups;
  bool chunked;  // read h in chunks staged through LDS (2 x 8 slots x 64 lanes per wavefront)
};

template <class R, class Sys, int METHOD>
__global__ void __launch_bounds__(256) states_kernel(StatesArgs<R> a) {
  constexpr int D = Sys::D;
  const int lane = laneId();
  tsit5::Coef<R> C5;
  if constexpr (METHOD == M_TSIT5) C5 = tsit5::Coef<R>::literal();
  const unsigned long long ngroups = (unsigned long long)((a.n + WAVE - 1) / WAVE);
  for (;;) {
    unsigned long long g = 0;
    if (lane == 0) g = atomicAdd(a.groups, 1ull);
    g = __shfl(g, 0);
    if (g >= ngroups) break;
    const int64_t idx = (int64_t)g * WAVE + lane;
    int64_t k = -1;
    int cnt = 0;
    bool ok = false;
    if (idx < a.n) {
      k = a.perm ? (int64_t)a.perm[idx] : idx;
      if (k < 0 || k >= a.n) {
        k = -1;
      } else {
        cnt = a.count[k];
        ok = cnt >= 0 && cnt <= a.s_max && (a.status == nullptr || a.status[k] == TRAJ_OK);
        if (!ok) cnt = 0;
      }
    }
    Sys sys;
    sys.load(a.theta, a.n, k >= 0 ? k : 0);
    R y[D];
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = (k >= 0) ? a.y0[c * a.n + k] : R(0);
    const R* hrow = (k >= 0) ? a.h_rec + k * a.s_cap : a.h_rec;
    R t = a.t0, prev = a.t0;
    int j = 0;
    int64_t q = (k >= 0) ? 0 : a.m;  // lanes without a trajectory are done
    // h of step r: read step by step, or (a.chunked) from an LDS ring of two
    // 8-step chunks per lane.  A lane's row is read in 64-byte chunks (four
    // 16-byte loads), each requested one chunk before it enters the ring, so
    // every piece of the row is fetched once (read eight bytes per step the
    // row's lines were fetched again and again).  Chunk c sits in slots
    // 8 (c & 1) .. 8 (c & 1) + 7; when step 8c is first needed, chunk c goes
    // from registers (nx) into the ring and chunk c + 1 is requested.
    typedef R R2 __attribute__((ext_vector_type(2)));
    HIP_DYNAMIC_SHARED(unsigned char, st_lds)
    R(*const ring)[WAVE] = (R(*)[WAVE])((R*)st_lds + (threadIdx.x / WAVE) * (16 * WAVE));
    R nx[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) nx[u] = R(0);
    auto request = [&](int c) {  // chunk c into nx (rows 8c .. 8c + 7 < s_cap)
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        const R2 v = *(const R2*)(hrow + 8 * c + u);
        nx[u] = v.x;
        nx[u + 1] = v.y;
      }
    };
    auto put_ring = [&](int c) {
#pragma unroll
      for (int u = 0; u < 8; ++u) ring[8 * (c & 1) + u][lane] = nx[u];
    };
    R hc = R(0), hn = R(0);
    if (a.chunked) {
      if (cnt > 0) {
        request(0);
        put_ring(0);
        if (8 < cnt) request(1);
        hc = ring[0][lane];
        hn = ring[1][lane];
      }
    } else {
      hc = (cnt > 0) ? hrow[0] : R(0);
      hn = (cnt > 1) ? hrow[1] : R(0);
    }
    R tau = (q < a.m) ? a.tq[q] : R(0);
    while (__ballot(q < a.m)) {
      const bool live = q < a.m;
      const bool bad = !(tau >= a.t0 && tau <= a.t1) || tau < prev || !ok;
      const bool adv = live && !bad && (j < cnt - 1) && (tau >= t + hc);
      const bool put = live && !adv;
      // one step of the method: the recorded step, or the shortened step to tau
      R hs = adv ? hc : ((put && !bad && cnt > 0) ? tau - t : R(0));
      R ys[D];
#pragma unroll
      for (int c = 0; c < D; ++c) ys[c] = y[c];
      if constexpr (METHOD == M_TSIT5)
        tsit5::replay<R, Sys>(C5, sys, ys, hs);
      else if constexpr (METHOD == M_VERN7)
        vern7::replay<R, Sys>(sys, ys, hs);
      else if constexpr (METHOD == M_RODAS5P)
        rodas5p::replay<R, Sys>(sys, ys, hs);
      else
        ros23::replay<R, Sys>(sys, ys, hs);
      if (adv) {
#pragma unroll
        for (int c = 0; c < D; ++c) y[c] = ys[c];
        t = t + hc;
        ++j;
        hc = hn;
        const int r = j + 1;
        if (r < cnt) {
          if (a.chunked) {
            if ((r & 7) == 0) {
              put_ring(r >> 3);
              if (r + 8 < cnt) request((r >> 3) + 1);
            }
            hn = ring[r & 15][lane];
          } else {
            hn = hrow[r];
          }
        }
      }
      if (put) {
#pragma unroll
        for (int c = 0; c < D; ++c) a.yq[(q * D + c) * a.n + k] = bad ? nanR(R(0)) : ys[c];
        if (!bad) prev = tau;
        ++q;
        if (q < a.m) tau = a.tq[q];
      }
    }
  }
}

// ---- trajectory ordering by step count (counting sort, decreasing count)
constexpr int ORDER_BINS = 4096;
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v);
__global__ void order_hist_kernel(const int32_t* count, int64_t n, int64_t s_max, int shift, int nb,
                                  uint32_t* hist);
__global__ void scan_buckets_kernel(uint32_t* hist, int64_t nb);
__global__ void order_scatter_kernel(const int32_t* count, int64_t n, int64_t s_max, int shift,
                                     int nb, uint32_t* off, int32_t* perm);
__global__ void order_slice_hist_kernel(const int32_t* count, int64_t n, int64_t s_max, int shift,
                                        int nb, int64_t len, uint32_t* table);
__global__ void order_slice_scan_kernel(uint32_t* table, int64_t slices, int nb, uint32_t* hist);
__global__ void order_stable_scatter_kernel(const int32_t* count, int64_t n, int64_t s_max,
                                            int shift, int nb, int64_t len, const uint32_t* table,
                                            const uint32_t* off, int32_t* perm);

}  // namespace dao
