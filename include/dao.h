/*
 * dao.h -- C ABI of the MI355X ensemble ODE library: adaptive solve with a
 * step record, and the discrete-adjoint gradient on the recorded mesh.
 *
 * Method (arXiv 2609.02876, "gradsolve: fast exact gradients for ODE
 * ensembles on GPUs"):
 *   - Section 2.1: each trajectory is integrated by an embedded explicit
 *     Runge-Kutta pair (Tsit5) or a linearly implicit Rosenbrock-Wanner step
 *     (Rosenbrock23), accepting a trial step when the RMS of
 *     e / (atol + rtol * max(|y|, |y_new|)) is at most one.
 *   - Section 3.1 (Fig. 2, Eq. 4): the record keeps the accepted step sizes;
 *     the gradient is the exact reverse-mode derivative of the fixed-step
 *     replay of that mesh, with the step sizes held constant.
 *   - Section 3.2: the Rosenbrock stage solves with I - gamma h J, and its
 *     adjoint solves with the transpose.
 *
 * Conventions shared by every entry point:
 *   - "real" is double for DAO_F64 and float for DAO_F32.
 *   - All array pointers are DEVICE pointers unless stated otherwise; the
 *     caller allocates and owns them, the library never frees them and never
 *     allocates device memory itself.
 *   - Layouts are structure-of-arrays: parameters theta[p][n] (index
 *     i*n + k), states y[d][n]; the shared MLP weights are one vector
 *     theta[4740].  Record rows are trajectory-major: h[k*s_cap + j] is the
 *     j-th accepted step of trajectory k.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; results are ready when the stream
 *     is.  Argument checks happen before anything is enqueued; a call that
 *     fails them returns DAO_EINVAL (or DAO_EUNSUPPORTED / DAO_EWORKSPACE)
 *     and enqueues nothing.  dao_last_error() then names the argument.
 *   - Per-trajectory failures are not call failures: they are written to
 *     record.status, and that trajectory's outputs are NaN.
 *   - Calls on one stream are ordered; calls that share a workspace must
 *     not overlap in time.
 */
#ifndef DAO_H
#define DAO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DAO_OK = 0,
  DAO_EINVAL = 1,       /* an argument is invalid; dao_last_error() names it       */
  DAO_EDEVICE = 2,      /* a HIP runtime call or kernel launch failed              */
  DAO_EWORKSPACE = 3,   /* the workspace is smaller than the call needs            */
  DAO_EUNSUPPORTED = 4  /* system / method / dtype combination is not provided     */
} dao_status;

/* Built-in right-hand sides (d = state size, p = parameters per trajectory). */
typedef enum {
  DAO_SYS_DECAY = 0,          /* y' = -theta y; d=1, p=1                                     */
  DAO_SYS_LOTKA_VOLTERRA = 1, /* theta=(a,b,g,d): y1'=y1(a-b y2), y2'=y2(d y1-g); d=2, p=4    */
  DAO_SYS_LORENZ63 = 2,       /* theta=(sigma,rho,beta); d=3, p=3                            */
  DAO_SYS_MLP = 3,            /* y'=W3 tanh(W2 tanh(W1 y+b1)+b2)+b3, 4-64-64-4, shared
                                 theta[4740] = [W1(64x4) b1 W2(64x64) b2 W3(4x64) b3]; d=4   */
  DAO_SYS_ROBERTSON = 4,      /* theta=(k1,k2,k3): Robertson kinetics; d=3, p=3              */
  DAO_SYS_LOGHALO = 5,        /* theta=(v0,Rc,q), y=(x,y,z,vx,vy,vz), potential
                                 1/2 v0^2 ln(Rc^2+x^2+y^2+z^2/q^2); d=6, p=3                 */
  DAO_SYS_HIRES = 6           /* HIRES photomorphogenesis kinetics (Sec. 3.1 lists it among
                                 the stiff fields), theta = its twelve rate constants
                                 (k1..k12, nominal 1.71 0.43 8.32 0.0007 8.75 10.03 0.035
                                 1.12 1.745 280 0.69 1.81); d=8, p=12; f64 with either
                                 method, f32 with Rosenbrock23                               */
} dao_system;

typedef enum {
  DAO_TSIT5 = 0,        /* Tsitouras 5(4) pair, 7 stages, FSAL (Sec. 2.1)                  */
  DAO_ROSENBROCK23 = 1, /* Shampine-Reichelt second-order Rosenbrock, autonomous (Sec. 3.2) */
  DAO_VERNER7 = 2,      /* Verner 7(6) pair, 10 stages, not FSAL (Sec. 3.1 method list);
                           binary64 with decay, Lotka-Volterra, Lorenz-63 and the log halo;
                           solve, gradients and states at requested times (no forward
                           sensitivities: DAO_EUNSUPPORTED)                               */
  DAO_RODAS5P = 3       /* Rodas5P, 8-stage stiffly accurate L-stable Rosenbrock-Wanner
                           method of order 5(4) (Sec. 3.1: the general stiff engine;
                           Sec. 3.2: one factorisation of I/(gamma h) - J per step, one
                           solve per stage); autonomous systems; binary64 with decay,
                           Lotka-Volterra, Robertson and HIRES; solve, gradients and
                           states at requested times (no forward sensitivities)           */
} dao_method;

typedef enum { DAO_F64 = 0, DAO_F32 = 1 } dao_dtype;

/* Per-trajectory status codes (record.status). */
enum {
  DAO_TRAJ_OK = 0,
  DAO_TRAJ_MAX_STEPS = 1,    /* more than tol.max_steps attempts                          */
  DAO_TRAJ_NONFINITE = 2,    /* error estimate or step size not finite                    */
  DAO_TRAJ_DT_UNDERFLOW = 3, /* t + h == t                                                */
  DAO_TRAJ_CAPACITY = 4      /* more accepted steps than record.s_cap (or the grad's s_max) */
};

/* Tolerances and step controls (host struct, read during the call). */
typedef struct {
  double rtol;       /* relative tolerance, > 0                                         */
  double atol;       /* absolute tolerance, > 0                                         */
  double dt0;        /* > 0: first trial step; <= 0: automatic starting step           */
  int64_t max_steps; /* cap on attempted steps per trajectory, >= 1                     */
  int32_t phases;    /* work order of dao_solve / dao_solve_sens: 0 = automatic, 1 = one
                        phase, 2 = two phases whenever the workspace holds them (see
                        dao_solve); the outputs are the same bit for bit either way      */
} dao_tol;

/* Step record (Sec. 3, Fig. 2): host struct of caller-owned device arrays.
 * Rows past count[k] are never read, and after dao_solve they hold
 * unspecified values (a rejected attempt may write the next row).           */
typedef struct {
  int64_t s_cap;   /* rows per trajectory (capacity), >= 0                       */
  void* t;         /* real[n][s_cap]: start time of each accepted step; may be NULL */
  void* h;         /* real[n][s_cap]: accepted step sizes                          */
  int32_t* count;  /* int32[n]: accepted steps                                     */
  int32_t* nrej;   /* int32[n]: rejected attempts; may be NULL                     */
  int32_t* status; /* int32[n]: DAO_TRAJ_* code                                    */
  void* y;         /* optional real[n][s_cap][d]: the state at the start of each
                      accepted step (the accepted states the in-kernel adjoint of
                      Sec. 3.3 keeps); NULL = not recorded.  Not provided for
                      DAO_SYS_MLP.                                                */
} dao_record;

/* State size d, parameter count p, and whether theta is shared (MLP).
 * Returns DAO_EINVAL for an unknown system.                                 */
dao_status dao_system_dims(dao_system sys, int* d, int* p, int* shared);

/* Workspace (device bytes) dao_solve and dao_solve_sens need for n
 * trajectories.  Except for the neural field this includes the two-phase
 * solve's saved states (with room for the sensitivities), ordering keys and
 * order, about (2d + 2 + dp) x 8 + 16 bytes per trajectory in binary64.     */
size_t dao_solve_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n);

/*
 * dao_solve -- adaptive solve of n independent trajectories on [t0, t1]
 * (Sec. 2.1): per trajectory, FSAL Tsit5 or Rosenbrock23 trial steps, RMS
 * acceptance test, integral step-size controller, last step clipped to t1.
 * Writes y1[d][n] (NaN where status != DAO_TRAJ_OK) and the record of
 * accepted steps (Sec. 3, Fig. 2): rec->h (and rec->t if not NULL) rows,
 * rec->count, rec->nrej (if not NULL) and rec->status.
 *   theta    real[p][n] (or real[4740] for DAO_SYS_MLP), y0 real[d][n]
 *   t0 <= t1, both finite; tol as above
 *   rec      required; rec->h may be NULL only when rec->s_cap == 0
 *   workspace >= dao_solve_workspace_size() device bytes (work-queue
 *            counter and trash slots); its contents need no initialisation.
 *            With tol->phases = 0, ensembles of at least four times the
 *            lanes the solve keeps resident with rec->s_cap >= 1024 are
 *            solved in two phases: the first 64 attempts of every
 *            trajectory, then the unfinished ones resumed longest-predicted
 *            first (the remaining attempts extrapolated from the time the
 *            first ones covered), so that long trajectories do not run alone
 *            at the end.  tol->phases = 1 or 2 forces one or two phases.  Two
 *            phases need the whole dao_solve_workspace_size(); a smaller
 *            workspace (at least dao_solve_workspace_size() for n = 0)
 *            runs one phase.  Every trajectory
 *            takes the same attempts either way: the outputs are identical
 *            bit for bit.  The library reads no environment variable.
 * Errors: DAO_EINVAL (NULL array with n > 0, t1 < t0, bad tolerances,
 * tol->phases outside 0..2, rec NULL, rec->s_cap < 0), DAO_EUNSUPPORTED,
 * DAO_EWORKSPACE, DAO_EDEVICE.  Trajectories that fail do not fail the call
 * (it returns before they run): dao_record_stats counts them, stream-ordered.
 */
dao_status dao_solve(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                     const void* theta, const void* y0, double t0, double t1,
                     const dao_tol* tol, void* y1, const dao_record* rec,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace (device bytes) dao_grad needs for n trajectories whose records
 * hold at most s_max accepted steps.  Less is accepted (down to
 * dao_grad_workspace_min) and runs fewer trajectories at once.               */
size_t dao_grad_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                               int64_t s_max);
size_t dao_grad_workspace_min(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                              int64_t s_max);

/*
 * dao_grad -- discrete-adjoint gradient on the recorded mesh (Sec. 3.1):
 * replays y_{j+1} = Phi(y_j; h_j, theta) for j < count[k] from y0 with the
 * recorded h_j as constants, then sweeps backward from dL/dy1 through every
 * stage (Tsit5), or through both stage solves with the transposed LU factors
 * and the Jacobian's own dependence on y and theta (Rosenbrock23, Sec. 3.2).
 * theta may differ from the theta of the solve that wrote the record: the
 * derivative is then taken at theta on the old mesh (Sec. 3.1, 4.8).
 * When rec->y is not NULL the forward pass of the replay is skipped and the
 * recorded states are used instead; they are the replay's states only at the
 * theta (and y0) the solve ran with, so a call at another theta must pass a
 * record whose y is NULL.
 *   theta, y0 as in dao_solve; rec->h and rec->count are read
 *   s_max    >= max_k count[k] and <= rec->s_cap (trajectories with more
 *            steps get NaN outputs)
 *   dLdy1    real[d][n], the cotangent of the final state
 *   dLdtheta real[p][n], or real[4740] summed over the ensemble (MLP);
 *            may be NULL.  A trajectory whose status is not DAO_TRAJ_OK, or
 *            whose count exceeds s_max, gets NaN in its entries; for the
 *            shared weights of DAO_SYS_MLP one such trajectory makes the
 *            whole summed gradient NaN (a partial sum is never returned).
 *            The MLP's sum runs in an order fixed by n alone: the same
 *            inputs give the same bits whatever the workspace size, stream
 *            or scheduling.
 *   dLdy0    real[d][n]; may be NULL
 * Errors: DAO_EINVAL, DAO_EUNSUPPORTED, DAO_EWORKSPACE, DAO_EDEVICE.
 */
dao_status dao_grad(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                    const void* theta, const void* y0, const dao_record* rec, int64_t s_max,
                    const void* dLdy1, void* dLdtheta, void* dLdy0,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * dao_grad in two parts.  The gradient runs trajectories in groups of similar
 * step count; dao_grad_order sorts the record's trajectories by count[k] into
 * the workspace (a stable sort: equal counts keep index order, so the order
 * depends on the counts alone), and dao_grad_ordered runs the gradient with
 * the order the workspace holds.  dao_grad does both.  One order serves any number of
 * dao_grad_ordered calls on the same record counts, n and s_max (Sec. 3.1
 * and 4.8 reuse one record while theta moves: theta, y0 and dLdy1 may change
 * between them), provided nothing else writes the workspace in between (a
 * dao_grad call with it, or its use as a dao_solve workspace, does).
 * dao_grad_order reads rec->count and rec->s_cap only; theta, y0 and dLdy1
 * are not touched.  Arguments, errors and results otherwise as dao_grad; with
 * a workspace that holds no order for this record, dao_grad_ordered's
 * results are unspecified (every access stays within the workspace and the
 * record).
 */
dao_status dao_grad_order(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                          const dao_record* rec, int64_t s_max, void* workspace,
                          size_t workspace_bytes, void* stream);
dao_status dao_grad_ordered(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                            const void* theta, const void* y0, const dao_record* rec,
                            int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * dao_grad_noalloc -- dao_grad for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same gradient, bit for bit, with its scratch (queue
 * counter, step-count histogram, trajectory order, per-wavefront tiles and
 * the neural field's partial sums) in a static device array of the library
 * instead of a workspace argument.  Arguments, results and errors as
 * dao_grad.
 *   Limit: the array is 64 MiB (67,108,864 bytes) per GPU, held from the
 *   library's first use on that GPU until the process ends.  A call whose
 *   dao_grad_workspace_min(sys, method, dtype, n, s_max) exceeds it returns
 *   DAO_EWORKSPACE before anything is enqueued; below that, the gradient runs
 *   as many trajectory groups at once as the array holds (fewer than with
 *   the full dao_grad_workspace_size, so it may be slower).
 *   The call allocates nothing: no hipMalloc, no hipFree.  Its first call on
 *   a GPU looks up the array's device address (hipGetSymbolAddress).
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind (each call clears what it counts with first): calls that overlap
 *   in time on one GPU, on any streams, race and give wrong results.
 */
dao_status dao_grad_noalloc(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                            const void* theta, const void* y0, const dao_record* rec,
                            int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0,
                            void* stream);

/*
 * dao_grad_at -- the discrete-adjoint gradient of a loss that also holds the
 * states at requested times (the application paper, arXiv 2609.28458,
 * Sec. 2.3, fits residuals at observation times):
 *   L = sum_q <dLdyq[q], y(tq[q])> + <dLdy1, y(t1)>,
 * y(tau) exactly as dao_states_at returns it (a shortened step of the method
 * from the start of the accepted step that holds tau).  The reverse sweep
 * adds, at each step, the vector-Jacobian products of the shortened steps to
 * the times that step holds; the recorded h, the running time and each
 * tau - t_j are constants (sg[h], Sec. 3.1).
 *   t0, t1   the span of the solve that wrote the record
 *   m, tq    m requested times (device, real[m]) shared by the ensemble,
 *            ascending in [t0, t1]; otherwise every output is NaN
 *   dLdyq    real[m][d][n], the cotangents of the states at tq
 *   dLdy1    real[d][n] or NULL (no final-state term)
 *   rec->y   not used (the forward replay assigns the times to steps)
 *   others   as dao_grad; per-trajectory systems (not DAO_SYS_MLP)
 * Workspace: dao_grad_at_workspace_size (per resident wavefront the tile
 * of dao_grad plus a table of m step indices and offsets).
 * Errors: DAO_EINVAL, DAO_EUNSUPPORTED, DAO_EWORKSPACE, DAO_EDEVICE.
 */
size_t dao_grad_at_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                                  int64_t s_max, int64_t m);
dao_status dao_grad_at(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                       const void* theta, const void* y0, double t0, double t1,
                       const dao_record* rec, int64_t s_max, int64_t m, const void* tq,
                       const void* dLdyq, const void* dLdy1, void* dLdtheta, void* dLdy0,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward sensitivities of the final state, S = dy1/dtheta (and dy1/dy0):
 * the derivatives the application paper (arXiv 2609.28458, "Differentiable
 * astrophysics at scale") obtains in the same kernel as the solve by
 * integrating the sensitivity equations S' = (df/dy) S + df/dtheta beside the
 * state, with the step size chosen on the state alone (its Sec. 2.3 and
 * Sec. 3; eq. 2).  With the steps held fixed that is the exact derivative of
 * the discrete solution on the recorded mesh, the same quantity the forward
 * mode through the replay of the record gives (gradsolve Sec. 3.1).  Both
 * methods; for Rosenbrock23 the tangent of W = I - gamma h J is included.
 * Per-trajectory parameters only: DAO_EUNSUPPORTED for the neural field
 * (whose 4740 shared weights are a reverse-mode case).  Layouts: S_theta real[d][p][n] with S_theta[(c p + j) n + k] =
 * dy1_c/dtheta_j of trajectory k; S_y0 real[d][d][n] likewise.  Failed
 * trajectories get NaN.
 *
 * dao_solve_sens -- dao_solve (same arguments, record and results, the same
 * steps bit for bit) plus S_theta (required).
 */
dao_status dao_solve_sens(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                          const void* theta, const void* y0, double t0, double t1,
                          const dao_tol* tol, void* y1, const dao_record* rec, void* S_theta,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace (device bytes) dao_sens needs; 0 for an unsupported combination. */
size_t dao_sens_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                               int64_t s_max);

/*
 * dao_sens -- the same sensitivities by forward mode through the replay of a
 * record (rec->h, rec->count, rec->status read), at theta (which may differ
 * from the solve's) and y0.  S_theta or S_y0 may be NULL, not both.  With
 * the record of a dao_solve_sens call at the same theta, S_theta equals that
 * call's bit for bit.  s_max as in dao_grad.  The workspace holds the sorted
 * order of the record (its contents need no initialisation).
 * Errors: DAO_EINVAL, DAO_EUNSUPPORTED, DAO_EWORKSPACE, DAO_EDEVICE.
 */
dao_status dao_sens(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                    const void* theta, const void* y0, const dao_record* rec, int64_t s_max,
                    void* S_theta, void* S_y0, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace (device bytes) dao_states_at needs; 0 for an unsupported combination. */
size_t dao_states_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                                 int64_t s_max);

/*
 * dao_states_at -- the state of every trajectory at m requested times on its
 * recorded mesh: a shortened step of the method from the start of the
 * accepted step that holds the time (application paper arXiv 2609.28458,
 * Sec. 2.3 and Appendix A; gradsolve's replay engines integrate one extra
 * step to each requested time).  Step j spans [t_j, t_j + h_j] with t_0 = t0
 * and t_{j+1} = t_j + h_j, the solve's own time update, so a time on a step
 * boundary returns the replay's state there bit for bit and t1 the final
 * state.  The record's mesh is not changed.
 *   theta, y0  as in dao_solve (the theta may differ from the solve's)
 *   t0, t1     the span of the solve that wrote the record
 *   rec        rec->h, rec->count and rec->status are read
 *   s_max      as in dao_grad
 *   tq         real[m], shared by all trajectories, ascending in [t0, t1];
 *              a time outside that range, not a number, or below its
 *              predecessor gives NaN (so do failed trajectories)
 *   yq         real[m][d][n]: yq[(q d + c) n + k] = component c of
 *              trajectory k at tq[q]
 * Not provided for DAO_SYS_MLP.  Errors: DAO_EINVAL, DAO_EUNSUPPORTED,
 * DAO_EWORKSPACE, DAO_EDEVICE.
 */
dao_status dao_states_at(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                         const void* theta, const void* y0, double t0, double t1,
                         const dao_record* rec, int64_t s_max, int64_t m, const void* tq,
                         void* yq, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dao_record_stats -- summary of a record, computed on the device in stream
 * order (so a caller that must not synchronise can still size a gradient or
 * detect failed trajectories at a point of its choosing).  gradsolve Sec. 3
 * (Fig. 2): the record is the accepted steps of every trajectory, padded to
 * a common length for the replay, whose length is the longest record; Sec.
 * 3.4: a call that cannot produce its result says so.
 *   n        trajectories in the record (>= 0)
 *   rec      rec->count and rec->status are read (rec->nrej if not NULL)
 *   out      device int64[4], written after every earlier call on the
 *            stream:
 *              out[0] = max_k count[k]   (the s_max a gradient needs; 0 if n = 0)
 *              out[1] = sum_k count[k]   (accepted steps of the ensemble)
 *              out[2] = number of k with status[k] != DAO_TRAJ_OK
 *              out[3] = sum_k nrej[k]    (0 when rec->nrej is NULL)
 * Errors: DAO_EINVAL (n < 0, rec / count / status / out NULL with n > 0 --
 * out must not be NULL even for n = 0), DAO_EDEVICE.
 */
dao_status dao_record_stats(int64_t n, const dao_record* rec, int64_t* out, void* stream);

/*
 * dao_sqerr_cotangent -- cotangent of a squared-error loss (the misfit
 * l(y(t1)) of Sec. 2.2's calibration loss), out[c][k] = scale *
 * (y1[c][k] - target[c][k]) for components c < d_used, 0 for the rest.
 *   y1, target, out real[d][n]; 0 <= d_used <= d
 */
dao_status dao_sqerr_cotangent(dao_dtype dtype, int64_t n, int d, int d_used, const void* y1,
                               const void* target, double scale, void* out, void* stream);

/* Message describing the last failed call on this thread ("" if none). */
const char* dao_last_error(void);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* dao_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DAO_H */
