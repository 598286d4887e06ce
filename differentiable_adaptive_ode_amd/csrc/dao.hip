// C ABI of the ensemble ODE library (declared in include/dao.h): argument
// checks, workspace carving, kernel dispatch.  No device memory is allocated
// here; every buffer is the caller's.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dao.h"
#include "kernels.hpp"

namespace dao {

// ------------------------------------------------------------- small kernels
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Trajectory ordering for the gradient: a counting sort by decreasing
// accepted-step count, so that the 64 lanes of a wavefront replay meshes of
// similar length.  Counts are binned as
//   bucket = ((s_max + 1) - min(count, s_max + 1)) >> shift
// with shift chosen so that at most ORDER_BINS bins exist.  This order (the
// two-phase solve's) is arbitrary within a bin: a trajectory's solve does not
// depend on its neighbours.
// Both passes histogram in LDS first, so global atomics are one per non-empty
// bin per workgroup rather than one per trajectory.
__device__ __forceinline__ int bucket_of(int32_t c, int64_t s_max, int shift) {
  int64_t cc = c < 0 ? 0 : (int64_t)c;
  if (cc > s_max + 1) cc = s_max + 1;
  return (int)(((s_max + 1) - cc) >> shift);
}

__global__ void __launch_bounds__(256) order_hist_kernel(const int32_t* count, int64_t n,
                                                         int64_t s_max, int shift, int nb,
                                                         uint32_t* hist) {
  __shared__ uint32_t lh[ORDER_BINS];
  for (int b = threadIdx.x; b < nb; b += blockDim.x) lh[b] = 0u;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    atomicAdd(&lh[bucket_of(count[i], s_max, shift)], 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x)
    if (lh[b]) atomicAdd(&hist[b], lh[b]);
}

// In-place exclusive scan of hist[0..nb) by one 1024-thread workgroup.
__global__ void __launch_bounds__(1024) scan_buckets_kernel(uint32_t* hist, int64_t nb) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t chunk = (nb + 1023) / 1024;
  const int64_t lo = tid * chunk;
  const int64_t hi = (lo + chunk < nb) ? lo + chunk : nb;
  uint32_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += hist[i];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint32_t v = (tid >= off) ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  uint32_t run = part[tid] - s;  // exclusive prefix of this thread's chunk
  for (int64_t i = lo; i < hi; ++i) {
    const uint32_t v = hist[i];
    hist[i] = run;
    run += v;
  }
}

// Each workgroup owns the contiguous slice [lo, hi) of trajectories: it counts
// its slice per bin in LDS, reserves each bin's range in the global offsets
// with one atomic, then places its trajectories with LDS atomics.
__global__ void __launch_bounds__(256) order_scatter_kernel(const int32_t* count, int64_t n,
                                                            int64_t s_max, int shift, int nb,
                                                            uint32_t* off, int32_t* perm) {
  __shared__ uint32_t lh[ORDER_BINS];
  const int64_t chunk = (n + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = (lo + chunk < n) ? lo + chunk : n;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) lh[b] = 0u;
  __syncthreads();
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x)
    atomicAdd(&lh[bucket_of(count[i], s_max, shift)], 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x)
    if (lh[b]) lh[b] = atomicAdd(&off[b], lh[b]);
  __syncthreads();
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x)
    perm[atomicAdd(&lh[bucket_of(count[i], s_max, shift)], 1u)] = (int32_t)i;
}

// Stable variant, for the replays of a record (gradient, sensitivities,
// states at requested times): within a bin the trajectories keep their index
// order, so the order, and with it which trajectories share a wavefront, is a
// function of the counts alone.  The ensemble is cut into slices of whole
// 64-trajectory tiles (order_slice_len); order_slice_hist_kernel writes each
// slice's histogram into a table [slice][bin], order_slice_scan_kernel turns
// each bin's column into the slices' starting ranks within the bin (and the
// bin's total into hist), scan_buckets_kernel makes hist the bins' starting
// positions, and order_stable_scatter_kernel, one workgroup per slice, places
// the slice's trajectories tile by tile: a trajectory's position is its bin's
// next free position plus the number of lower lanes of its tile in the same
// bin.
__global__ void __launch_bounds__(256) order_slice_hist_kernel(const int32_t* count, int64_t n,
                                                               int64_t s_max, int shift, int nb,
                                                               int64_t len, uint32_t* table) {
  __shared__ uint32_t lh[ORDER_BINS];
  for (int b = threadIdx.x; b < nb; b += blockDim.x) lh[b] = 0u;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * len;
  const int64_t hi = (lo + len < n) ? lo + len : n;
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x)
    atomicAdd(&lh[bucket_of(count[i], s_max, shift)], 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x) table[(int64_t)blockIdx.x * nb + b] = lh[b];
}

// One thread per bin: exclusive prefix of the bin's column over the slices,
// in place, and the bin's total into hist[b].
__global__ void __launch_bounds__(256) order_slice_scan_kernel(uint32_t* table, int64_t slices,
                                                               int nb, uint32_t* hist) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  uint32_t run = 0;
  int64_t s = 0;
  for (; s + 8 <= slices; s += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = table[(s + u) * nb + b];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      table[(s + u) * nb + b] = run;
      run += v[u];
    }
  }
  for (; s < slices; ++s) {
    const uint32_t v = table[s * nb + b];
    table[s * nb + b] = run;
    run += v;
  }
  hist[b] = run;
}

constexpr int ORDER_BATCH = 8;  // tiles whose counts are loaded at once
// The workgroup's four wavefronts place a quarter of the slice's tiles each:
// a histogram per wavefront in LDS, then for every bin its slice's starting
// position plus the counts of the lower wavefronts, then each wavefront walks
// its tiles in order.  Lanes of a tile in the same bin are those whose bin
// agrees in every bit: one ballot per bit, and m ^ (bit ? 0 : ~0) keeps the
// lanes that agree with this lane on it.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__global__ void __launch_bounds__(256) order_stable_scatter_kernel(
    const int32_t* count, int64_t n, int64_t s_max, int shift, int nb, int64_t len,
    const uint32_t* table, const uint32_t* off, int32_t* perm) {
  __shared__ uint32_t next[4][ORDER_BINS];
  const int lane = threadIdx.x % WAVE;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  for (int b = threadIdx.x; b < 4 * ORDER_BINS; b += 256) (&next[0][0])[b] = 0u;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * len;
  const int64_t hi = (lo + len < n) ? lo + len : n;
  const int64_t tiles = (hi - lo + WAVE - 1) / WAVE;
  const int64_t per = (tiles + 3) / 4;
  const int64_t t0 = wv * per, t1 = (t0 + per < tiles) ? t0 + per : tiles;
  // bins of ORDER_BATCH tiles at a time (-1: past the slice); the loads
  // are unconditional (index clamped into the slice) so that they overlap
  auto load = [&](int64_t tb, int (&bk)[ORDER_BATCH]) {
    int32_t c[ORDER_BATCH];
#pragma unroll
    for (int u = 0; u < ORDER_BATCH; ++u) {
      const int64_t i = lo + (tb + u) * WAVE + lane;
      c[u] = count[i < hi ? i : hi - 1];
    }
#pragma unroll
    for (int u = 0; u < ORDER_BATCH; ++u) {
      const int64_t i = lo + (tb + u) * WAVE + lane;
      bk[u] = (tb + u < t1 && i < hi) ? bucket_of(c[u], s_max, shift) : -1;
    }
  };
  for (int64_t tb = t0; tb < t1; tb += ORDER_BATCH) {
    int bk[ORDER_BATCH];
    load(tb, bk);
#pragma unroll
    for (int u = 0; u < ORDER_BATCH; ++u)
      if (bk[u] >= 0) atomicAdd(&next[wv][bk[u]], 1u);
  }
  __syncthreads();
  const uint32_t* row = table + (int64_t)blockIdx.x * nb;
  for (int b = threadIdx.x; b < nb; b += 256) {
    uint32_t run = off[b] + row[b];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = next[w][b];
      next[w][b] = run;
      run += v;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  uint32_t* nx = next[wv];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int64_t tb = t0; tb < t1; tb += ORDER_BATCH) {
    int bks[ORDER_BATCH];
    load(tb, bks);
#pragma unroll
    for (int u = 0; u < ORDER_BATCH; ++u) {
      if (tb + u >= t1) break;  // the same for every lane
      const bool valid = bks[u] >= 0;
      const int bk = valid ? bks[u] : 0;
      unsigned long long peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const unsigned long long m = __ballot((bk >> bit) & 1);
        peers &= m ^ ((unsigned long long)((bk >> bit) & 1) - 1ull);
      }
      const uint32_t p = valid ? nx[bk] + (uint32_t)__popcll(peers & below) : 0u;
      wave_sync();
      // the highest lane of each bin advances the bin's next position
      if (valid && (peers >> lane) == 1ull) nx[bk] += (uint32_t)__popcll(peers);
      wave_sync();
      if (valid) perm[p] = (int32_t)(lo + (tb + u) * WAVE + lane);
    }
  }
}

// Record summary: max and sum of count, failed trajectories, sum of nrej.
// Each workgroup reduces its grid-stride share in LDS, then one lane adds it
// into out[] with device atomics (out[] cleared by the fill kernel first).
__global__ void __launch_bounds__(256) record_stats_kernel(const int32_t* count,
                                                           const int32_t* status,
                                                           const int32_t* nrej, int64_t n,
                                                           unsigned long long* out) {
  __shared__ unsigned long long red[4][256];
  unsigned long long mx = 0, sum = 0, bad = 0, rej = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int32_t c = count[i];
    const unsigned long long cu = c > 0 ? (unsigned long long)c : 0ull;
    mx = cu > mx ? cu : mx;
    sum += cu;
    bad += (status[i] != TRAJ_OK) ? 1ull : 0ull;
    if (nrej) rej += nrej[i] > 0 ? (unsigned long long)nrej[i] : 0ull;
  }
  const int t = threadIdx.x;
  red[0][t] = mx;
  red[1][t] = sum;
  red[2][t] = bad;
  red[3][t] = rej;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) {
      red[0][t] = red[0][t + off] > red[0][t] ? red[0][t + off] : red[0][t];
      red[1][t] += red[1][t + off];
      red[2][t] += red[2][t + off];
      red[3][t] += red[3][t + off];
    }
    __syncthreads();
  }
  if (t == 0) {
    atomicMax(&out[0], red[0][0]);
    atomicAdd(&out[1], red[1][0]);
    atomicAdd(&out[2], red[2][0]);
    atomicAdd(&out[3], red[3][0]);
  }
}

template <class R>
__global__ void sqerr_cotangent_kernel(int64_t n, int d, int d_used, const R* y1, const R* tgt,
                                       R scale, R* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * d) return;
  const int c = (int)(i / n);
  out[i] = (c < d_used) ? scale * (y1[i] - tgt[i]) : R(0);
}

}  // namespace dao

using namespace dao;

// ------------------------------------------------------------- error state
namespace {

thread_local char g_err[512] = "";

dao_status fail(dao_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

dao_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return DAO_OK;
  return fail(DAO_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

const int SYS_D[7] = {1, 2, 3, 4, 3, 6, 8};
const int SYS_P[7] = {1, 4, 3, 4740, 3, 3, 12};

bool sys_ok(int sys) { return sys >= 0 && sys <= 6; }
bool method_ok(int m) { return m >= DAO_TSIT5 && m <= DAO_RODAS5P; }

struct DevInfo {
  int cus = 0;
};

DevInfo dev_info() {
  static std::mutex mu;
  static std::vector<DevInfo> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DevInfo{256};
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1);
  if (cache[dev].cus == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].cus = v;
  }
  return cache[dev];
}

constexpr int BLOCK = BLOCK_WAVES * WAVE;
constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Resident workgroups for a kernel at BLOCK threads and `lds` bytes of
// dynamic LDS.
template <class K>
int64_t resident_blocks(K kernel, size_t lds = 0) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, BLOCK, lds) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  return (int64_t)per_cu * dev_info().cus;
}

// --------------------------------------------------------- typed launchers
void launch_order(const int32_t* count, int64_t n, int64_t s_max, uint32_t* hist, int32_t* perm,
                  hipStream_t stream);

// Two-phase solve of large ensembles.  When the ensemble is several times
// the solve's resident lanes, the order in which trajectories are handed out
// decides how long the last ones run alone: phase 1 takes the first
// SOLVE_PROBE attempts of every trajectory and predicts each one's remaining
// attempts from the time those covered (64 attempts, about a tenth of a
// log-halo orbit trajectory on average, rank them well enough); the
// suspended trajectories are sorted by that prediction and phase 2 resumes
// them longest first.  Every
// trajectory takes the same attempts as in one phase, bit for bit.
constexpr int32_t SOLVE_PROBE = 64;

size_t solve_base_bytes() { return ALIGN + align_up((size_t)WAVE * 2 * sizeof(double)); }

// save (the state of a suspended trajectory, with room for its
// sensitivities; one contiguous record per trajectory), save_i, key, perm,
// histogram
template <class R, int D, int P>
size_t solve_save_reals() { return (size_t)save_stride<R, D, P>(); }
template <class R, int D, int P>
size_t solve_phase_bytes(int64_t n) {
  return align_up(solve_save_reals<R, D, P>() * n * sizeof(R)) + align_up((size_t)2 * n * 4) +
         2 * align_up((size_t)n * 4) + align_up((size_t)ORDER_BINS * 4);
}

// Whether a solve of n trajectories takes two phases.  phases = 1 or 2 (the
// caller's dao_tol) forces one or two; 0 chooses two for n at least four
// times the resident lanes and a record capacity of at least 1024 steps.
// The capacity is the caller's bound on a trajectory's length: resuming a
// trajectory costs its wavefront a few memory round trips, which short
// trajectories (tens of steps) do not repay, while long ones are where a
// late start runs alone.
template <class R, class Sys, int M>
bool solve_two_phase(int64_t n, int64_t s_cap, int phases) {
  if (n <= 0 || phases == 1) return false;
  if (phases == 2) return true;
  if (s_cap < 1024) return false;
  auto kern = solve_kernel<R, Sys, M, false, true>;
  const size_t lds = (size_t)BLOCK_WAVES * 2 * 8 * WAVE * sizeof(R);
  return n >= 4 * resident_blocks(kern, lds) * BLOCK;
}

// Workspace of a solve: the queue and trash slots, and room for two phases
// (which any solve may be asked to take).
template <class R, class Sys, int M>
size_t solve_ws_bytes(int64_t n) {
  return solve_base_bytes() + (n > 0 ? solve_phase_bytes<R, Sys::D, Sys::P>(n) : 0);
}

template <class R, class Sys, int M, bool SENS = false>
dao_status launch_solve(int64_t n, const void* theta, const void* y0, double t0, double t1,
                        const dao_tol* tol, void* y1, const dao_record* rec, void* ws,
                        size_t ws_bytes, hipStream_t stream, void* S_theta = nullptr) {
  SolveArgs<R> a;
  a.S_theta = (R*)S_theta;
  a.n = n;
  a.theta = (const R*)theta;
  a.y0 = (const R*)y0;
  a.t0 = R(t0);
  a.t1 = R(t1);
  a.rtol = R(tol->rtol);
  a.atol = R(tol->atol);
  a.dt0 = R(tol->dt0);
  a.max_steps = tol->max_steps;
  a.y1 = (R*)y1;
  a.s_cap = rec->s_cap;
  a.t_rec = (R*)rec->t;
  a.h_rec = (R*)rec->h;
  a.count = rec->count;
  a.nrej = rec->nrej;
  a.status = rec->status;
  a.y_rec = (R*)rec->y;
  a.queue = (unsigned long long*)ws;
  a.trash = (R*)((char*)ws + ALIGN);
  a.phase = 0;
  a.probe = 0;
  a.save = nullptr;
  a.save_i = nullptr;
  a.key = nullptr;
  a.order = nullptr;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)ws, (int64_t)2, 0u);
  // record staging ring: (t, h [, y]) x 8 slots x 64 lanes per wavefront
  const size_t lds = (size_t)BLOCK_WAVES * (rec->y ? 2 + Sys::D : 2) * 8 * WAVE * sizeof(R);
  {
    if (solve_two_phase<R, Sys, M>(n, rec->s_cap, tol->phases) &&
        ws_bytes >= solve_base_bytes() + solve_phase_bytes<R, Sys::D, Sys::P>(n)) {
      char* p = (char*)ws + solve_base_bytes();
      a.save = (R*)p;
      p += align_up(solve_save_reals<R, Sys::D, Sys::P>() * n * sizeof(R));
      a.save_i = (int32_t*)p;
      p += align_up((size_t)2 * n * 4);
      a.key = (int32_t*)p;
      p += align_up((size_t)n * 4);
      int32_t* perm = (int32_t*)p;
      p += align_up((size_t)n * 4);
      uint32_t* hist = (uint32_t*)p;
      auto kern = solve_kernel<R, Sys, M, SENS, true>;
      int64_t blocks = (n + BLOCK - 1) / BLOCK;
      const int64_t res = resident_blocks(kern, lds);
      if (blocks > res) blocks = res;
      a.phase = 1;
      a.probe = SOLVE_PROBE;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(BLOCK), lds, stream, a);
      launch_order(a.key, n, ORDER_KEY_MAX, hist, perm, stream);
      hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)ws, (int64_t)2,
                         0u);
      a.phase = 2;
      a.order = perm;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(BLOCK), lds, stream, a);
      return check_hip(hipGetLastError(), "solve kernel launch");
    }
  }
  auto kern = solve_kernel<R, Sys, M, SENS>;
  int64_t blocks = (n + BLOCK - 1) / BLOCK;
  const int64_t res = resident_blocks(kern, lds);
  if (blocks > res) blocks = res;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(BLOCK), lds, stream, a);
  return check_hip(hipGetLastError(), "solve kernel launch");
}

// Per-wavefront scratch tile of the gradient: per step the D state
// components and h, 64 lanes each.
template <class R, int D>
size_t grad_slot_bytes(int64_t s_max, int64_t m = 0) {
  // the tile, then (cotangents at m requested times) the tables [m][2][64]
  // and [m][D][64]
  return ((size_t)(s_max > 0 ? s_max : 1) * (D + 1) + (size_t)m * (2 + D)) * WAVE * sizeof(R);
}

// Cotangents at requested times (dao_grad_at).
struct AtArgs {
  int64_t m;
  const void* tq;
  const void* dLdyq;
  double t0, t1;
};

// The stable order's slices: at most ORDER_SLICES of them, each a whole
// number of 64-trajectory tiles and at least ORDER_SLICE_MIN long.
constexpr int64_t ORDER_SLICES = 128;
constexpr int64_t ORDER_SLICE_MIN = 1024;
int64_t order_slice_len(int64_t n) {
  int64_t len = (n + ORDER_SLICES - 1) / ORDER_SLICES;
  len = (len + WAVE - 1) / WAVE * WAVE;
  return len < ORDER_SLICE_MIN ? ORDER_SLICE_MIN : len;
}
int64_t order_slice_count(int64_t n) {
  const int64_t k = (n + order_slice_len(n) - 1) / order_slice_len(n);
  return k < 1 ? 1 : k;
}
// Bins of the order by step count: bin = ((s_max + 1) - min(count, s_max + 1)) >> shift.
int order_shift(int64_t s_max) {
  int shift = 0;
  while (((s_max + 1) >> shift) + 1 > ORDER_BINS) ++shift;
  return shift;
}
int order_bins(int64_t s_max) { return (int)(((s_max + 1) >> order_shift(s_max)) + 1); }

// Head of the workspace of a record's replays: queue counter, bin offsets,
// the order, and the stable order's slice table.
size_t grad_header_bytes(int64_t n, int64_t s_max) {
  return align_up(16) + align_up((size_t)ORDER_BINS * 4) + align_up((size_t)(n > 0 ? n : 1) * 4) +
         align_up((size_t)order_slice_count(n) * order_bins(s_max) * 4);
}
struct OrderWs {
  unsigned long long* groups;
  uint32_t* hist;
  int32_t* perm;
  uint32_t* table;
};
OrderWs order_ws(void* ws, int64_t n) {
  char* base = (char*)ws;
  OrderWs o;
  o.groups = (unsigned long long*)base;
  o.hist = (uint32_t*)(base + align_up(16));
  o.perm = (int32_t*)(base + align_up(16) + align_up((size_t)ORDER_BINS * 4));
  o.table = (uint32_t*)(base + align_up(16) + align_up((size_t)ORDER_BINS * 4) +
                        align_up((size_t)(n > 0 ? n : 1) * 4));
  return o;
}

// Orders a record's trajectories by decreasing step count into o.perm, equal
// bins in index order.
void launch_order_stable(const int32_t* count, int64_t n, int64_t s_max, const OrderWs& o,
                         hipStream_t stream) {
  const int shift = order_shift(s_max), nb = order_bins(s_max);
  const int64_t len = order_slice_len(n), slices = order_slice_count(n);
  hipLaunchKernelGGL(order_slice_hist_kernel, dim3((unsigned)slices), dim3(256), 0, stream, count,
                     n, s_max, shift, nb, len, o.table);
  hipLaunchKernelGGL(order_slice_scan_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                     stream, o.table, slices, nb, o.hist);
  hipLaunchKernelGGL(scan_buckets_kernel, dim3(1), dim3(1024), 0, stream, o.hist, (int64_t)nb);
  hipLaunchKernelGGL(order_stable_scatter_kernel, dim3((unsigned)slices), dim3(256), 0, stream,
                     count, n, s_max, shift, nb, len, (const uint32_t*)o.table,
                     (const uint32_t*)o.hist, o.perm);
}

// Orders trajectories by decreasing step count into perm.
void launch_order(const int32_t* count, int64_t n, int64_t s_max, uint32_t* hist, int32_t* perm,
                  hipStream_t stream) {
  int shift = 0;
  while (((s_max + 1) >> shift) + 1 > ORDER_BINS) ++shift;
  const int nb = (int)(((s_max + 1) >> shift) + 1);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream,
                     hist, (int64_t)nb, 0u);
  int64_t oblk = (n + 255) / 256;
  if (oblk > 1024) oblk = 1024;
  hipLaunchKernelGGL(order_hist_kernel, dim3((unsigned)oblk), dim3(256), 0, stream, count, n,
                     s_max, shift, nb, hist);
  hipLaunchKernelGGL(scan_buckets_kernel, dim3(1), dim3(1024), 0, stream, hist, (int64_t)nb);
  hipLaunchKernelGGL(order_scatter_kernel, dim3((unsigned)oblk), dim3(256), 0, stream, count, n,
                     s_max, shift, nb, hist, perm);
}

// What a gradient call does: order the trajectories by step count into the
// workspace, run the gradient with the order the workspace holds, or both.
enum { GRAD_ORDER = 1, GRAD_RUN = 2 };

template <class R, class Sys, int M, bool AT = false>
dao_status launch_grad(int mode, int64_t n, const void* theta, const void* y0, const dao_record* rec,
                       int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0, void* ws,
                       size_t ws_bytes, hipStream_t stream, const AtArgs* at = nullptr) {
  constexpr int D = Sys::D;
  char* base = (char*)ws;
  const OrderWs ow = order_ws(ws, n);
  unsigned long long* groups = ow.groups;
  int32_t* perm = ow.perm;
  const size_t hdr = grad_header_bytes(n, s_max);
  R* scratch = (R*)(base + hdr);
  const size_t slot = grad_slot_bytes<R, D>(s_max, AT ? at->m : 0);
  int64_t slots = (int64_t)((ws_bytes - hdr) / slot);

  auto kern = grad_kernel<R, Sys, M, AT>;
  const int64_t ngroups = (n + WAVE - 1) / WAVE;
  const int64_t waves_per_block = BLOCK / WAVE;
  int64_t blocks = (ngroups + waves_per_block - 1) / waves_per_block;
  // the LDS ring through which the forward pass reads the record's h (and,
  // for Rodas5P on large systems, the reverse step's stage solutions)
  const size_t lds = (size_t)BLOCK_WAVES * grad_lds_reals<Sys, M>() * sizeof(R);
  const int64_t res = resident_blocks(kern, lds);
  if (blocks > res) blocks = res;
  if (blocks > slots / waves_per_block) blocks = slots / waves_per_block;
  if (blocks < 1) return fail(DAO_EWORKSPACE, "dao_grad: workspace too small");

  if (mode & GRAD_ORDER) launch_order_stable(rec->count, n, s_max, ow, stream);
  if (!(mode & GRAD_RUN)) return check_hip(hipGetLastError(), "order kernel launch");
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)groups, (int64_t)2, 0u);

  GradArgs<R> a;
  a.n = n;
  a.theta = (const R*)theta;
  a.y0 = (const R*)y0;
  a.s_cap = rec->s_cap;
  a.h_rec = (const R*)rec->h;
  a.count = rec->count;
  a.status = rec->status;
  a.s_max = s_max;
  a.dLdy1 = (const R*)dLdy1;
  a.dLdtheta = (R*)dLdtheta;
  a.dLdy0 = (R*)dLdy0;
  a.scratch = scratch;
  a.y_rec = (const R*)rec->y;
  a.perm = perm;
  a.groups = groups;
  a.m = 0;
  a.tq = nullptr;
  a.dLdyq = nullptr;
  a.t0 = a.t1 = R(0);
  if (AT) {
    a.m = at->m;
    a.tq = (const R*)at->tq;
    a.dLdyq = (const R*)at->dLdyq;
    a.t0 = R(at->t0);
    a.t1 = R(at->t1);
    a.y_rec = nullptr;  // the forward replay assigns the times to steps
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(BLOCK), lds, stream, a);
  return check_hip(hipGetLastError(), "grad kernel launch");
}

// Forward sensitivities through the replay: the record's trajectories are
// sorted once, then one pass of sens_kernel per P directions (the
// parameters, then the initial-state components).
template <class R, class Sys, int M>
dao_status launch_sens(int64_t n, const void* theta, const void* y0, const dao_record* rec,
                       int64_t s_max, void* S_theta, void* S_y0, void* ws, hipStream_t stream) {
  constexpr int D = Sys::D, P = Sys::P;
  char* base = (char*)ws;
  const OrderWs ow = order_ws(ws, n);
  unsigned long long* groups = ow.groups;
  int32_t* perm = ow.perm;
  auto kern = sens_kernel<R, Sys, M, P>;
  const int64_t ngroups = (n + WAVE - 1) / WAVE;
  int64_t blocks = (ngroups + BLOCK / WAVE - 1) / (BLOCK / WAVE);
  // h read in chunks through an LDS ring when the record's rows allow it
  const bool chunked = rec->s_cap % 8 == 0 && ((uintptr_t)rec->h % 16) == 0;
  const size_t lds = chunked ? (size_t)BLOCK_WAVES * 16 * WAVE * sizeof(R) : 0;
  const int64_t res = resident_blocks(kern, lds);
  if (blocks > res) blocks = res;
  launch_order_stable(rec->count, n, s_max, ow, stream);
  SensArgs<R> a;
  a.chunked = chunked;
  a.n = n;
  a.theta = (const R*)theta;
  a.y0 = (const R*)y0;
  a.s_cap = rec->s_cap;
  a.h_rec = (const R*)rec->h;
  a.count = rec->count;
  a.status = rec->status;
  a.s_max = s_max;
  a.S_theta = (R*)S_theta;
  a.S_y0 = (R*)S_y0;
  a.perm = perm;
  a.groups = groups;
  const int first = S_theta ? 0 : P, last = S_y0 ? P + D : P;
  for (int d0 = first; d0 < last; d0 += P) {
    a.dir0 = d0;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)groups, (int64_t)2, 0u);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(BLOCK), lds, stream, a);
  }
  return check_hip(hipGetLastError(), "sensitivity kernel launch");
}

// States at requested times: the record's trajectories sorted once, then one
// states_kernel launch.
template <class R, class Sys, int M>
dao_status launch_states(int64_t n, const void* theta, const void* y0, double t0, double t1,
                         const dao_record* rec, int64_t s_max, int64_t m, const void* tq, void* yq,
                         void* ws, hipStream_t stream) {
  char* base = (char*)ws;
  const OrderWs ow = order_ws(ws, n);
  unsigned long long* groups = ow.groups;
  int32_t* perm = ow.perm;
  auto kern = states_kernel<R, Sys, M>;
  // h read in chunks staged through LDS when the record's rows allow it
  const bool chunked = rec->s_cap % 8 == 0 && ((uintptr_t)rec->h % 16) == 0;
  const size_t lds = chunked ? (size_t)BLOCK_WAVES * 16 * WAVE * sizeof(R) : 0;
  const int64_t ngroups = (n + WAVE - 1) / WAVE;
  int64_t blocks = (ngroups + BLOCK / WAVE - 1) / (BLOCK / WAVE);
  const int64_t res = resident_blocks(kern, lds);
  if (blocks > res) blocks = res;
  launch_order_stable(rec->count, n, s_max, ow, stream);
  StatesArgs<R> a;
  a.chunked = chunked;
  a.n = n;
  a.theta = (const R*)theta;
  a.y0 = (const R*)y0;
  a.t0 = R(t0);
  a.t1 = R(t1);
  a.s_cap = rec->s_cap;
  a.h_rec = (const R*)rec->h;
  a.count = rec->count;
  a.status = rec->status;
  a.s_max = s_max;
  a.m = m;
  a.tq = (const R*)tq;
  a.yq = (R*)yq;
  a.perm = perm;
  a.groups = groups;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)groups, (int64_t)2, 0u);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(BLOCK), lds, stream, a);
  return check_hip(hipGetLastError(), "states kernel launch");
}

// ------------------------------------------------- neural right-hand side
dao_status launch_mlp_solve(int64_t n, const void* theta, const void* y0, double t0, double t1,
                            const dao_tol* tol, void* y1, const dao_record* rec, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  mlp::SolveArgs a;
  a.n = n;
  a.theta = (const float*)theta;
  a.y0 = (const float*)y0;
  a.t0 = (float)t0;
  a.t1 = (float)t1;
  a.rtol = (float)tol->rtol;
  a.atol = (float)tol->atol;
  a.dt0 = (float)tol->dt0;
  a.max_steps = tol->max_steps;
  a.y1 = (float*)y1;
  a.s_cap = rec->s_cap;
  a.t_rec = (float*)rec->t;
  a.h_rec = (float*)rec->h;
  a.count = rec->count;
  a.nrej = rec->nrej;
  a.status = rec->status;
  a.queue = (unsigned long long*)ws;
  a.trash = (float*)((char*)ws + ALIGN);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)ws, (int64_t)2, 0u);
  const int64_t groups = (n + mlp::SLOTS - 1) / mlp::SLOTS;
  int64_t blocks = (groups + BLOCK / WAVE - 1) / (BLOCK / WAVE);
  const int64_t res = resident_blocks(mlp::solve_kernel);
  if (blocks > res) blocks = res;
  hipLaunchKernelGGL(mlp::solve_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, stream, a);
  return check_hip(hipGetLastError(), "mlp solve kernel launch");
}

// Per-wavefront workspace of the neural gradient: the state tile
// [s_max][64] floats.
size_t mlp_slot_bytes(int64_t s_max) {
  return align_up((size_t)(s_max > 0 ? s_max : 1) * WAVE * sizeof(float));
}

// Workspace of the neural gradient that depends on n alone: one row of
// partial weight-gradient sums [4740] floats per chunk.
size_t mlp_fixed_bytes(int64_t n) {
  return align_up((size_t)mlp::grad_chunks(n) * mlp::NP * sizeof(float));
}

dao_status launch_mlp_grad(int mode, int64_t n, const void* theta, const void* y0, const dao_record* rec,
                           int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  char* base = (char*)ws;
  const OrderWs ow = order_ws(ws, n);
  unsigned long long* groups = ow.groups;
  int32_t* perm = ow.perm;
  const size_t hdr = grad_header_bytes(n, s_max);
  const size_t fixed = mlp_fixed_bytes(n);
  const int64_t chunks = mlp::grad_chunks(n);
  const size_t slot = mlp_slot_bytes(s_max);
  if (ws_bytes < hdr + fixed) return fail(DAO_EWORKSPACE, "dao_grad: workspace too small");
  const int64_t slots = (int64_t)((ws_bytes - hdr - fixed) / slot);
  const int64_t ngroups = (n + mlp::SLOTS - 1) / mlp::SLOTS;
  const int64_t waves_per_block = BLOCK / WAVE;
  int64_t blocks = (ngroups + waves_per_block - 1) / waves_per_block;
  const int64_t res = resident_blocks(mlp::grad_kernel);
  if (blocks > res) blocks = res;
  if (blocks > slots / waves_per_block) blocks = slots / waves_per_block;
  if (blocks < 1) return fail(DAO_EWORKSPACE, "dao_grad: workspace too small");
  float* partial = (float*)(base + hdr);
  float* scratch = (float*)(base + hdr + fixed);

  if (mode & GRAD_ORDER) launch_order_stable(rec->count, n, s_max, ow, stream);
  if (!(mode & GRAD_RUN)) return check_hip(hipGetLastError(), "order kernel launch");
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)groups, (int64_t)2, 0u);

  mlp::GradArgs a;
  a.n = n;
  a.theta = (const float*)theta;
  a.y0 = (const float*)y0;
  a.s_cap = rec->s_cap;
  a.h_rec = (const float*)rec->h;
  a.count = rec->count;
  a.status = rec->status;
  a.s_max = s_max;
  a.dLdy1 = (const float*)dLdy1;
  a.dLdy0 = (float*)dLdy0;
  a.scratch = scratch;
  a.partial = partial;
  a.chunks = chunks;
  a.perm = perm;
  a.groups = groups;
  hipLaunchKernelGGL(mlp::grad_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, stream, a);
  dao_status st = check_hip(hipGetLastError(), "mlp grad kernel launch");
  if (st != DAO_OK) return st;
  if (dLdtheta) {
    const int64_t runs = (chunks + mlp::REDUCE_CHUNK - 1) / mlp::REDUCE_CHUNK;
    hipLaunchKernelGGL(mlp::reduce_chunks_kernel, dim3((mlp::NP + 255) / 256, (unsigned)runs),
                       dim3(256), 0, stream, partial, chunks);
    hipLaunchKernelGGL(mlp::reduce_kernel, dim3((mlp::NP + 255) / 256), dim3(256), 0, stream,
                       (const float*)partial, chunks, (float*)dLdtheta);
    st = check_hip(hipGetLastError(), "mlp reduce kernel launch");
  }
  return st;
}

// Dispatch table over (system, method, dtype).
template <class R, template <class> class S, int M>
struct Entry {
  static dao_status solve(int64_t n, const void* th, const void* y0, double t0, double t1,
                          const dao_tol* tol, void* y1, const dao_record* rec, void* ws,
                          size_t wsb, hipStream_t st) {
    return launch_solve<R, S<R>, M>(n, th, y0, t0, t1, tol, y1, rec, ws, wsb, st);
  }
  static size_t solve_ws(int64_t n) { return solve_ws_bytes<R, S<R>, M>(n); }
  static dao_status grad(int mode, int64_t n, const void* th, const void* y0, const dao_record* rec,
                         int64_t s_max, const void* g, void* dth, void* dy0, void* ws,
                         size_t wsb, hipStream_t st) {
    return launch_grad<R, S<R>, M>(mode, n, th, y0, rec, s_max, g, dth, dy0, ws, wsb, st);
  }
  static dao_status solve_sens(int64_t n, const void* th, const void* y0, double t0, double t1,
                               const dao_tol* tol, void* y1, const dao_record* rec, void* ws,
                               size_t wsb, hipStream_t st, void* S_theta) {
    return launch_solve<R, S<R>, M, true>(n, th, y0, t0, t1, tol, y1, rec, ws, wsb, st, S_theta);
  }
  static dao_status sens(int64_t n, const void* th, const void* y0, const dao_record* rec,
                         int64_t s_max, void* S_theta, void* S_y0, void* ws, hipStream_t st) {
    return launch_sens<R, S<R>, M>(n, th, y0, rec, s_max, S_theta, S_y0, ws, st);
  }
  static dao_status states(int64_t n, const void* th, const void* y0, double t0, double t1,
                           const dao_record* rec, int64_t s_max, int64_t m, const void* tq,
                           void* yq, void* ws, hipStream_t st) {
    return launch_states<R, S<R>, M>(n, th, y0, t0, t1, rec, s_max, m, tq, yq, ws, st);
  }
  static dao_status grad_at(int64_t n, const void* th, const void* y0, const dao_record* rec,
                            int64_t s_max, const void* g, void* dth, void* dy0, void* ws,
                            size_t wsb, hipStream_t st, const AtArgs* at) {
    return launch_grad<R, S<R>, M, true>(GRAD_ORDER | GRAD_RUN, n, th, y0, rec, s_max, g, dth, dy0,
                                         ws, wsb, st, at);
  }
  static size_t slot_at_bytes(int64_t s_max, int64_t m) {
    return grad_slot_bytes<R, S<R>::D>(s_max, m);
  }
  static size_t slot_bytes(int64_t s_max) { return grad_slot_bytes<R, S<R>::D>(s_max); }
  static int64_t resident_waves() {
    return resident_blocks(grad_kernel<R, S<R>, M>) * (BLOCK / WAVE);
  }
};

typedef dao_status (*solve_fn)(int64_t, const void*, const void*, double, double, const dao_tol*,
                               void*, const dao_record*, void*, size_t, hipStream_t);
typedef size_t (*solve_ws_fn)(int64_t);
typedef dao_status (*grad_fn)(int, int64_t, const void*, const void*, const dao_record*, int64_t,
                              const void*, void*, void*, void*, size_t, hipStream_t);
typedef dao_status (*solve_sens_fn)(int64_t, const void*, const void*, double, double,
                                    const dao_tol*, void*, const dao_record*, void*, size_t,
                                    hipStream_t, void*);
typedef dao_status (*sens_fn)(int64_t, const void*, const void*, const dao_record*, int64_t, void*,
                              void*, void*, hipStream_t);
typedef dao_status (*states_fn)(int64_t, const void*, const void*, double, double,
                                const dao_record*, int64_t, int64_t, const void*, void*, void*,
                                hipStream_t);
typedef size_t (*slot_fn)(int64_t);
typedef int64_t (*res_fn)();
typedef dao_status (*grad_at_fn)(int64_t, const void*, const void*, const dao_record*, int64_t,
                                 const void*, void*, void*, void*, size_t, hipStream_t,
                                 const AtArgs*);
typedef size_t (*slot_at_fn)(int64_t, int64_t);

struct Impl {
  solve_fn solve;
  grad_fn grad;
  slot_fn slot;
  res_fn resident;
  int group;  // trajectories per wavefront in the gradient
  solve_sens_fn solve_sens;  // forward sensitivities (per-trajectory theta), else null
  sens_fn sens;
  states_fn states;  // states at requested times (per-lane systems), else null
  solve_ws_fn solve_ws;  // workspace of dao_solve for n trajectories
  grad_at_fn grad_at;    // gradient with cotangents at requested times, else null
  slot_at_fn slot_at;
  solve_ws_fn grad_fixed;  // gradient workspace that depends on n alone, else null
};

int64_t mlp_resident_waves() { return resident_blocks(mlp::grad_kernel) * (BLOCK / WAVE); }
size_t mlp_solve_ws(int64_t) { return solve_base_bytes(); }

template <class R, template <class> class S, int M>
Impl make_impl() {
  return Impl{&Entry<R, S, M>::solve, &Entry<R, S, M>::grad, &Entry<R, S, M>::slot_bytes,
              &Entry<R, S, M>::resident_waves, WAVE, &Entry<R, S, M>::solve_sens,
              &Entry<R, S, M>::sens, &Entry<R, S, M>::states, &Entry<R, S, M>::solve_ws,
              &Entry<R, S, M>::grad_at, &Entry<R, S, M>::slot_at_bytes};
}

// Verner 7 and Rodas5P: solve, gradient, states and gradient at requested
// times; no forward sensitivities.
template <class R, template <class> class S, int M>
Impl make_impl_no_sens() {
  using E = Entry<R, S, M>;
  return Impl{&E::solve, &E::grad, &E::slot_bytes, &E::resident_waves, WAVE, nullptr, nullptr,
              &E::states, &E::solve_ws, &E::grad_at, &E::slot_at_bytes};
}

const Impl* find_impl(int sys, int method, int dtype) {
  static Impl table[7][4][2];
  static bool init = false;
  static std::mutex mu;
  std::lock_guard<std::mutex> lk(mu);
  if (!init) {
    std::memset(table, 0, sizeof(table));
    table[DAO_SYS_DECAY][M_TSIT5][DAO_F64] = make_impl<double, Decay, M_TSIT5>();
    table[DAO_SYS_DECAY][M_TSIT5][DAO_F32] = make_impl<float, Decay, M_TSIT5>();
    table[DAO_SYS_DECAY][M_ROS23][DAO_F64] = make_impl<double, Decay, M_ROS23>();
    table[DAO_SYS_DECAY][M_ROS23][DAO_F32] = make_impl<float, Decay, M_ROS23>();
    table[DAO_SYS_LOTKA_VOLTERRA][M_TSIT5][DAO_F64] = make_impl<double, LotkaVolterra, M_TSIT5>();
    table[DAO_SYS_LOTKA_VOLTERRA][M_TSIT5][DAO_F32] = make_impl<float, LotkaVolterra, M_TSIT5>();
    table[DAO_SYS_LOTKA_VOLTERRA][M_ROS23][DAO_F64] = make_impl<double, LotkaVolterra, M_ROS23>();
    table[DAO_SYS_LOTKA_VOLTERRA][M_ROS23][DAO_F32] = make_impl<float, LotkaVolterra, M_ROS23>();
    table[DAO_SYS_LORENZ63][M_TSIT5][DAO_F64] = make_impl<double, Lorenz63, M_TSIT5>();
    table[DAO_SYS_LORENZ63][M_TSIT5][DAO_F32] = make_impl<float, Lorenz63, M_TSIT5>();
    table[DAO_SYS_LORENZ63][M_ROS23][DAO_F64] = make_impl<double, Lorenz63, M_ROS23>();
    table[DAO_SYS_LORENZ63][M_ROS23][DAO_F32] = make_impl<float, Lorenz63, M_ROS23>();
    table[DAO_SYS_ROBERTSON][M_TSIT5][DAO_F64] = make_impl<double, Robertson, M_TSIT5>();
    table[DAO_SYS_ROBERTSON][M_TSIT5][DAO_F32] = make_impl<float, Robertson, M_TSIT5>();
    table[DAO_SYS_ROBERTSON][M_ROS23][DAO_F64] = make_impl<double, Robertson, M_ROS23>();
    table[DAO_SYS_ROBERTSON][M_ROS23][DAO_F32] = make_impl<float, Robertson, M_ROS23>();
    table[DAO_SYS_LOGHALO][M_TSIT5][DAO_F64] = make_impl<double, LogHalo, M_TSIT5>();
    table[DAO_SYS_LOGHALO][M_TSIT5][DAO_F32] = make_impl<float, LogHalo, M_TSIT5>();
    table[DAO_SYS_HIRES][M_TSIT5][DAO_F64] = make_impl<double, Hires, M_TSIT5>();
    table[DAO_SYS_HIRES][M_ROS23][DAO_F64] = make_impl<double, Hires, M_ROS23>();
    table[DAO_SYS_HIRES][M_ROS23][DAO_F32] = make_impl<float, Hires, M_ROS23>();
    table[DAO_SYS_DECAY][M_VERN7][DAO_F64] = make_impl_no_sens<double, Decay, M_VERN7>();
    table[DAO_SYS_LOTKA_VOLTERRA][M_VERN7][DAO_F64] =
        make_impl_no_sens<double, LotkaVolterra, M_VERN7>();
    table[DAO_SYS_LORENZ63][M_VERN7][DAO_F64] = make_impl_no_sens<double, Lorenz63, M_VERN7>();
    table[DAO_SYS_LOGHALO][M_VERN7][DAO_F64] = make_impl_no_sens<double, LogHalo, M_VERN7>();
    table[DAO_SYS_DECAY][M_RODAS5P][DAO_F64] = make_impl_no_sens<double, Decay, M_RODAS5P>();
    table[DAO_SYS_LOTKA_VOLTERRA][M_RODAS5P][DAO_F64] =
        make_impl_no_sens<double, LotkaVolterra, M_RODAS5P>();
    table[DAO_SYS_ROBERTSON][M_RODAS5P][DAO_F64] =
        make_impl_no_sens<double, Robertson, M_RODAS5P>();
    table[DAO_SYS_HIRES][M_RODAS5P][DAO_F64] = make_impl_no_sens<double, Hires, M_RODAS5P>();
    table[DAO_SYS_MLP][M_TSIT5][DAO_F32] =
        Impl{&launch_mlp_solve, &launch_mlp_grad, &mlp_slot_bytes, &mlp_resident_waves, mlp::SLOTS,
             nullptr, nullptr, nullptr, &mlp_solve_ws, nullptr, nullptr, &mlp_fixed_bytes};
    init = true;
  }
  if (!sys_ok(sys) || !method_ok(method) || dtype < 0 || dtype > 1) return nullptr;
  const Impl* im = &table[sys][method][dtype];
  return im->solve ? im : nullptr;
}

bool is_fin(double x) { return std::isfinite(x); }

// ------------------------------------------- static scratch (dao_grad_noalloc)
// For callers that cannot allocate device memory: the gradient's workspace
// (queue counter, step-count histogram, trajectory order, per-wavefront
// tiles) in one file-scope device array.  Every GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` only names the
// symbol: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever passed to kernels.
constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// The device address of `scratch` on the current device (looked up on the
// first call per device), or null with the error set.
void* scratch_address(dao_status* st) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = check_hip(e, "dao_grad_noalloc: hipGetDevice");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = check_hip(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "dao_grad_noalloc: hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    addr[dev] = p;
  }
  *st = DAO_OK;
  return addr[dev];
}

}  // namespace

// ================================================================== C ABI
extern "C" {

const char* dao_last_error(void) { return g_err; }

const char* dao_version(void) { return "0.1.0 gfx950"; }

dao_status dao_system_dims(dao_system sys, int* d, int* p, int* shared) {
  if (!sys_ok(sys)) return fail(DAO_EINVAL, "dao_system_dims: unknown system %d", (int)sys);
  if (d) *d = SYS_D[sys];
  if (p) *p = SYS_P[sys];
  if (shared) *shared = (sys == DAO_SYS_MLP);
  return DAO_OK;
}

size_t dao_solve_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n) {
  // queue counter and trash slots; for large ensembles also the two-phase
  // solve's saved states, ordering keys and order
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || n < 0) return solve_base_bytes();
  return im->solve_ws(n);
}

}  // extern "C"

namespace {

// Argument checks of the solve's entry points; S_theta (the forward
// sensitivities) is non-null only for dao_solve_sens, whose name `fn` then is.
dao_status solve_call(const char* fn, dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                      const void* theta, const void* y0, double t0, double t1, const dao_tol* tol,
                      void* y1, const dao_record* rec, void* S_theta, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const bool sens = std::strcmp(fn, "dao_solve_sens") == 0;
  g_err[0] = 0;
  if (!sys_ok(sys)) return fail(DAO_EINVAL, "%s: unknown system %d", fn, (int)sys);
  if (!method_ok(method))
    return fail(DAO_EINVAL, "%s: unknown method %d", fn, (int)method);
  if (dtype != DAO_F64 && dtype != DAO_F32) return fail(DAO_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
  if (n < 0 || n > (int64_t)INT32_MAX) return fail(DAO_EINVAL, "%s: n = %lld out of range", fn, (long long)n);
  if (!tol) return fail(DAO_EINVAL, "%s: tol is NULL", fn);
  if (!(is_fin(t0) && is_fin(t1))) return fail(DAO_EINVAL, "%s: t0/t1 not finite", fn);
  if (!(t1 >= t0)) return fail(DAO_EINVAL, "%s: t1 < t0", fn);
  if (!(tol->rtol > 0) || !is_fin(tol->rtol)) return fail(DAO_EINVAL, "%s: rtol must be > 0", fn);
  if (!(tol->atol > 0) || !is_fin(tol->atol)) return fail(DAO_EINVAL, "%s: atol must be > 0", fn);
  if (!is_fin(tol->dt0)) return fail(DAO_EINVAL, "%s: dt0 not finite", fn);
  if (tol->max_steps < 1) return fail(DAO_EINVAL, "%s: max_steps must be >= 1", fn);
  if (tol->phases < 0 || tol->phases > 2)
    return fail(DAO_EINVAL, "%s: tol->phases must be 0 (automatic), 1 or 2", fn);
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || (sens && !im->solve_sens))
    return fail(DAO_EUNSUPPORTED, "%s: system %d with method %d dtype %d is not provided", fn,
                (int)sys, (int)method, (int)dtype);
  if (n == 0) return DAO_OK;
  if (!theta) return fail(DAO_EINVAL, "%s: theta is NULL", fn);
  if (!y0) return fail(DAO_EINVAL, "%s: y0 is NULL", fn);
  if (!y1) return fail(DAO_EINVAL, "%s: y1 is NULL", fn);
  if (sens && !S_theta) return fail(DAO_EINVAL, "%s: S_theta is NULL", fn);
  if (!rec) return fail(DAO_EINVAL, "%s: rec is NULL (count and status are written there)", fn);
  if (rec->s_cap < 0) return fail(DAO_EINVAL, "%s: rec->s_cap < 0", fn);
  if (!rec->count) return fail(DAO_EINVAL, "%s: rec->count is NULL", fn);
  if (!rec->status) return fail(DAO_EINVAL, "%s: rec->status is NULL", fn);
  if (rec->s_cap > 0 && !rec->h) return fail(DAO_EINVAL, "%s: rec->h is NULL", fn);
  if (rec->y && sys == DAO_SYS_MLP)
    return fail(DAO_EUNSUPPORTED, "%s: recorded states (rec->y) are not provided for the neural field", fn);
  if (!workspace || workspace_bytes < solve_base_bytes())
    return fail(DAO_EWORKSPACE, "%s: workspace needs at least %zu bytes (%zu for two phases)", fn,
                solve_base_bytes(), dao_solve_workspace_size(sys, method, dtype, n));
  if (sens)
    return im->solve_sens(n, theta, y0, t0, t1, tol, y1, rec, workspace, workspace_bytes,
                          (hipStream_t)stream, S_theta);
  return im->solve(n, theta, y0, t0, t1, tol, y1, rec, workspace, workspace_bytes,
                   (hipStream_t)stream);
}

}  // namespace

extern "C" {

dao_status dao_solve(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                     const void* theta, const void* y0, double t0, double t1, const dao_tol* tol,
                     void* y1, const dao_record* rec, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return solve_call("dao_solve", sys, method, dtype, n, theta, y0, t0, t1, tol, y1, rec, nullptr,
                    workspace, workspace_bytes, stream);
}

dao_status dao_solve_sens(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                          const void* theta, const void* y0, double t0, double t1,
                          const dao_tol* tol, void* y1, const dao_record* rec, void* S_theta,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return solve_call("dao_solve_sens", sys, method, dtype, n, theta, y0, t0, t1, tol, y1, rec,
                    S_theta, workspace, workspace_bytes, stream);
}

size_t dao_sens_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                               int64_t s_max) {
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || !im->sens || n < 0 || s_max < 0) return 0;
  return grad_header_bytes(n, s_max);
}

size_t dao_states_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                                 int64_t s_max) {
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || !im->states || n < 0 || s_max < 0) return 0;
  return grad_header_bytes(n, s_max);
}

dao_status dao_states_at(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                         const void* theta, const void* y0, double t0, double t1,
                         const dao_record* rec, int64_t s_max, int64_t m, const void* tq,
                         void* yq, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "dao_states_at";
  g_err[0] = 0;
  if (!sys_ok(sys)) return fail(DAO_EINVAL, "%s: unknown system %d", fn, (int)sys);
  if (!method_ok(method))
    return fail(DAO_EINVAL, "%s: unknown method %d", fn, (int)method);
  if (dtype != DAO_F64 && dtype != DAO_F32) return fail(DAO_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
  if (n < 0 || n > (int64_t)INT32_MAX) return fail(DAO_EINVAL, "%s: n = %lld out of range", fn, (long long)n);
  if (m < 0) return fail(DAO_EINVAL, "%s: m < 0", fn);
  if (!(is_fin(t0) && is_fin(t1))) return fail(DAO_EINVAL, "%s: t0/t1 not finite", fn);
  if (!(t1 >= t0)) return fail(DAO_EINVAL, "%s: t1 < t0", fn);
  if (!rec) return fail(DAO_EINVAL, "%s: rec is NULL", fn);
  if (rec->s_cap < 0) return fail(DAO_EINVAL, "%s: rec->s_cap < 0", fn);
  if (s_max < 0 || s_max > rec->s_cap) return fail(DAO_EINVAL, "%s: s_max must be in [0, rec->s_cap]", fn);
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || !im->states)
    return fail(DAO_EUNSUPPORTED, "%s: system %d with method %d dtype %d is not provided", fn,
                (int)sys, (int)method, (int)dtype);
  if (n == 0 || m == 0) return DAO_OK;
  if (!theta) return fail(DAO_EINVAL, "%s: theta is NULL", fn);
  if (!y0) return fail(DAO_EINVAL, "%s: y0 is NULL", fn);
  if (!tq) return fail(DAO_EINVAL, "%s: tq is NULL", fn);
  if (!yq) return fail(DAO_EINVAL, "%s: yq is NULL", fn);
  if (!rec->count) return fail(DAO_EINVAL, "%s: rec->count is NULL", fn);
  if (s_max > 0 && !rec->h) return fail(DAO_EINVAL, "%s: rec->h is NULL", fn);
  const size_t need = dao_states_workspace_size(sys, method, dtype, n, s_max);
  if (!workspace || workspace_bytes < need)
    return fail(DAO_EWORKSPACE, "%s: workspace needs at least %zu bytes", fn, need);
  return im->states(n, theta, y0, t0, t1, rec, s_max, m, tq, yq, workspace, (hipStream_t)stream);
}

dao_status dao_sens(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                    const void* theta, const void* y0, const dao_record* rec, int64_t s_max,
                    void* S_theta, void* S_y0, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* fn = "dao_sens";
  g_err[0] = 0;
  if (!sys_ok(sys)) return fail(DAO_EINVAL, "%s: unknown system %d", fn, (int)sys);
  if (!method_ok(method))
    return fail(DAO_EINVAL, "%s: unknown method %d", fn, (int)method);
  if (dtype != DAO_F64 && dtype != DAO_F32) return fail(DAO_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
  if (n < 0 || n > (int64_t)INT32_MAX) return fail(DAO_EINVAL, "%s: n = %lld out of range", fn, (long long)n);
  if (!rec) return fail(DAO_EINVAL, "%s: rec is NULL", fn);
  if (rec->s_cap < 0) return fail(DAO_EINVAL, "%s: rec->s_cap < 0", fn);
  if (s_max < 0 || s_max > rec->s_cap) return fail(DAO_EINVAL, "%s: s_max must be in [0, rec->s_cap]", fn);
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || !im->sens)
    return fail(DAO_EUNSUPPORTED, "%s: system %d with method %d dtype %d is not provided", fn,
                (int)sys, (int)method, (int)dtype);
  if (n == 0) return DAO_OK;
  if (!S_theta && !S_y0) return fail(DAO_EINVAL, "%s: S_theta and S_y0 are both NULL", fn);
  if (!theta) return fail(DAO_EINVAL, "%s: theta is NULL", fn);
  if (!y0) return fail(DAO_EINVAL, "%s: y0 is NULL", fn);
  if (!rec->count) return fail(DAO_EINVAL, "%s: rec->count is NULL", fn);
  if (s_max > 0 && !rec->h) return fail(DAO_EINVAL, "%s: rec->h is NULL", fn);
  const size_t need = dao_sens_workspace_size(sys, method, dtype, n, s_max);
  if (!workspace || workspace_bytes < need)
    return fail(DAO_EWORKSPACE, "%s: workspace needs at least %zu bytes", fn, need);
  return im->sens(n, theta, y0, rec, s_max, S_theta, S_y0, workspace, (hipStream_t)stream);
}

size_t dao_grad_workspace_min(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                              int64_t s_max) {
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || n < 0 || s_max < 0) return 0;
  return grad_header_bytes(n, s_max) + (im->grad_fixed ? im->grad_fixed(n) : 0) +
         (size_t)(BLOCK / WAVE) * im->slot(s_max);
}

size_t dao_grad_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                               int64_t s_max) {
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || n < 0 || s_max < 0) return 0;
  int64_t waves = (n + im->group - 1) / im->group;
  waves = (waves + BLOCK / WAVE - 1) / (BLOCK / WAVE) * (BLOCK / WAVE);
  const int64_t res = im->resident();
  if (waves > res) waves = res;
  if (waves < BLOCK / WAVE) waves = BLOCK / WAVE;
  return grad_header_bytes(n, s_max) + (im->grad_fixed ? im->grad_fixed(n) : 0) +
         (size_t)waves * im->slot(s_max);
}

}  // extern "C"

namespace {

// Argument checks shared by the gradient's entry points; `fn` names the entry
// point in the message.  The order step reads only rec->count (and status), so
// theta, y0 and dLdy1 are checked only when the gradient itself runs.
dao_status grad_call(const char* fn, int mode, dao_system sys, dao_method method, dao_dtype dtype,
                     int64_t n, const void* theta, const void* y0, const dao_record* rec,
                     int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0,
                     void* workspace, size_t workspace_bytes, void* stream,
                     bool static_scratch = false) {
  g_err[0] = 0;
  if (!sys_ok(sys)) return fail(DAO_EINVAL, "%s: unknown system %d", fn, (int)sys);
  if (!method_ok(method))
    return fail(DAO_EINVAL, "%s: unknown method %d", fn, (int)method);
  if (dtype != DAO_F64 && dtype != DAO_F32) return fail(DAO_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
  if (n < 0 || n > (int64_t)INT32_MAX) return fail(DAO_EINVAL, "%s: n = %lld out of range", fn, (long long)n);
  if (!rec) return fail(DAO_EINVAL, "%s: rec is NULL", fn);
  if (rec->s_cap < 0) return fail(DAO_EINVAL, "%s: rec->s_cap < 0", fn);
  if (s_max < 0 || s_max > rec->s_cap) return fail(DAO_EINVAL, "%s: s_max must be in [0, rec->s_cap]", fn);
  const Impl* im = find_impl(sys, method, dtype);
  if (!im) return fail(DAO_EUNSUPPORTED, "%s: system %d with method %d dtype %d is not provided",
                       fn, (int)sys, (int)method, (int)dtype);
  if (n == 0) return DAO_OK;
  if (!rec->count) return fail(DAO_EINVAL, "%s: rec->count is NULL", fn);
  if (mode & GRAD_RUN) {
    if (!theta) return fail(DAO_EINVAL, "%s: theta is NULL", fn);
    if (!y0) return fail(DAO_EINVAL, "%s: y0 is NULL", fn);
    if (s_max > 0 && !rec->h) return fail(DAO_EINVAL, "%s: rec->h is NULL", fn);
    if (!dLdy1) return fail(DAO_EINVAL, "%s: dLdy1 is NULL", fn);
    if (rec->y && sys == DAO_SYS_MLP)
      return fail(DAO_EUNSUPPORTED, "%s: recorded states (rec->y) are not provided for the neural field", fn);
  }
  const size_t need = dao_grad_workspace_min(sys, method, dtype, n, s_max);
  if (static_scratch) {
    if (need > SCRATCH_BYTES)
      return fail(DAO_EWORKSPACE,
                  "%s: n = %lld with s_max = %lld needs at least %zu bytes of scratch, more than "
                  "the library's static %zu bytes (use dao_grad with a workspace)",
                  fn, (long long)n, (long long)s_max, need, SCRATCH_BYTES);
    dao_status st = DAO_OK;
    workspace = scratch_address(&st);
    if (!workspace) return st;
    workspace_bytes = SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < need)
    return fail(DAO_EWORKSPACE, "%s: workspace needs at least %zu bytes", fn, need);
  return im->grad(mode, n, theta, y0, rec, s_max, dLdy1, dLdtheta, dLdy0, workspace,
                  workspace_bytes, (hipStream_t)stream);
}

}  // namespace

extern "C" {

dao_status dao_grad(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                    const void* theta, const void* y0, const dao_record* rec, int64_t s_max,
                    const void* dLdy1, void* dLdtheta, void* dLdy0, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return grad_call("dao_grad", GRAD_ORDER | GRAD_RUN, sys, method, dtype, n, theta, y0, rec, s_max,
                   dLdy1, dLdtheta, dLdy0, workspace, workspace_bytes, stream);
}

dao_status dao_grad_order(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                          const dao_record* rec, int64_t s_max, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return grad_call("dao_grad_order", GRAD_ORDER, sys, method, dtype, n, nullptr, nullptr, rec,
                   s_max, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

dao_status dao_grad_ordered(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                            const void* theta, const void* y0, const dao_record* rec,
                            int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return grad_call("dao_grad_ordered", GRAD_RUN, sys, method, dtype, n, theta, y0, rec, s_max,
                   dLdy1, dLdtheta, dLdy0, workspace, workspace_bytes, stream);
}

dao_status dao_grad_noalloc(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                            const void* theta, const void* y0, const dao_record* rec,
                            int64_t s_max, const void* dLdy1, void* dLdtheta, void* dLdy0,
                            void* stream) {
  return grad_call("dao_grad_noalloc", GRAD_ORDER | GRAD_RUN, sys, method, dtype, n, theta, y0,
                   rec, s_max, dLdy1, dLdtheta, dLdy0, nullptr, 0, stream, true);
}

size_t dao_grad_at_workspace_size(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                                  int64_t s_max, int64_t m) {
  const Impl* im = find_impl(sys, method, dtype);
  if (!im || !im->grad_at || n < 0 || s_max < 0 || m < 0) return 0;
  int64_t waves = (n + WAVE - 1) / WAVE;
  waves = (waves + BLOCK / WAVE - 1) / (BLOCK / WAVE) * (BLOCK / WAVE);
  const int64_t res = im->resident();
  if (waves > res) waves = res;
  if (waves < BLOCK / WAVE) waves = BLOCK / WAVE;
  return grad_header_bytes(n, s_max) + (size_t)waves * im->slot_at(s_max, m);
}

dao_status dao_grad_at(dao_system sys, dao_method method, dao_dtype dtype, int64_t n,
                       const void* theta, const void* y0, double t0, double t1,
                       const dao_record* rec, int64_t s_max, int64_t m, const void* tq,
                       const void* dLdyq, const void* dLdy1, void* dLdtheta, void* dLdy0,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "dao_grad_at";
  g_err[0] = 0;
  if (!sys_ok(sys)) return fail(DAO_EINVAL, "%s: unknown system %d", fn, (int)sys);
  if (!method_ok(method))
    return fail(DAO_EINVAL, "%s: unknown method %d", fn, (int)method);
  if (dtype != DAO_F64 && dtype != DAO_F32) return fail(DAO_EINVAL, "%s: unknown dtype %d", fn, (int)dtype);
  if (n < 0 || n > (int64_t)INT32_MAX) return fail(DAO_EINVAL, "%s: n = %lld out of range", fn, (long long)n);
  if (m < 0 || m > (int64_t)INT32_MAX) return fail(DAO_EINVAL, "%s: m = %lld out of range", fn, (long long)m);
  if (!is_fin(t0) || !is_fin(t1) || t1 < t0) return fail(DAO_EINVAL, "%s: need finite t0 <= t1", fn);
  if (!rec) return fail(DAO_EINVAL, "%s: rec is NULL", fn);
  if (rec->s_cap < 0) return fail(DAO_EINVAL, "%s: rec->s_cap < 0", fn);
  if (s_max < 0 || s_max > rec->s_cap) return fail(DAO_EINVAL, "%s: s_max must be in [0, rec->s_cap]", fn);
  const Impl* im = find_impl(sys, method, dtype);
  if (!im) return fail(DAO_EUNSUPPORTED, "%s: system %d with method %d dtype %d is not provided",
                       fn, (int)sys, (int)method, (int)dtype);
  if (!im->grad_at)
    return fail(DAO_EUNSUPPORTED, "%s: cotangents at requested times are provided for the "
                "per-trajectory systems, not the neural field", fn);
  if (n == 0) return DAO_OK;
  if (!rec->count) return fail(DAO_EINVAL, "%s: rec->count is NULL", fn);
  if (!theta) return fail(DAO_EINVAL, "%s: theta is NULL", fn);
  if (!y0) return fail(DAO_EINVAL, "%s: y0 is NULL", fn);
  if (s_max > 0 && !rec->h) return fail(DAO_EINVAL, "%s: rec->h is NULL", fn);
  if (m > 0 && (!tq || !dLdyq)) return fail(DAO_EINVAL, "%s: tq or dLdyq is NULL", fn);
  const size_t need = grad_header_bytes(n, s_max) + (size_t)(BLOCK / WAVE) * im->slot_at(s_max, m);
  if (!workspace || workspace_bytes < need)
    return fail(DAO_EWORKSPACE, "%s: workspace needs at least %zu bytes", fn, need);
  AtArgs at{m, tq, dLdyq, t0, t1};
  return im->grad_at(n, theta, y0, rec, s_max, dLdy1, dLdtheta, dLdy0, workspace, workspace_bytes,
                     (hipStream_t)stream, &at);
}

dao_status dao_record_stats(int64_t n, const dao_record* rec, int64_t* out, void* stream) {
  g_err[0] = 0;
  if (n < 0 || n > (int64_t)INT32_MAX)
    return fail(DAO_EINVAL, "dao_record_stats: n = %lld out of range", (long long)n);
  if (!out) return fail(DAO_EINVAL, "dao_record_stats: out is NULL");
  if (n > 0 && !rec) return fail(DAO_EINVAL, "dao_record_stats: rec is NULL");
  if (n > 0 && (!rec->count || !rec->status))
    return fail(DAO_EINVAL, "dao_record_stats: rec->count or rec->status is NULL");
  hipStream_t st = (hipStream_t)stream;
  // out[0..3] (int64) cleared as eight 32-bit words by a fill kernel, not a
  // memset, so the call may be captured into a graph
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, st, (uint32_t*)out, (int64_t)8, 0u);
  if (n > 0) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(record_stats_kernel, dim3((unsigned)blocks), dim3(256), 0, st, rec->count,
                       rec->status, rec->nrej, n, (unsigned long long*)out);
  }
  return check_hip(hipGetLastError(), "record stats kernel launch");
}

dao_status dao_sqerr_cotangent(dao_dtype dtype, int64_t n, int d, int d_used, const void* y1,
                               const void* target, double scale, void* out, void* stream) {
  g_err[0] = 0;
  if (dtype != DAO_F64 && dtype != DAO_F32) return fail(DAO_EINVAL, "dao_sqerr_cotangent: unknown dtype");
  if (n < 0 || d < 1 || d_used < 0 || d_used > d)
    return fail(DAO_EINVAL, "dao_sqerr_cotangent: bad sizes");
  if (!is_fin(scale)) return fail(DAO_EINVAL, "dao_sqerr_cotangent: scale not finite");
  if (n == 0) return DAO_OK;
  if (!y1 || !target || !out) return fail(DAO_EINVAL, "dao_sqerr_cotangent: NULL array");
  const int64_t tot = n * d;
  const unsigned blocks = (unsigned)((tot + 255) / 256);
  if (dtype == DAO_F64)
    hipLaunchKernelGGL(sqerr_cotangent_kernel<double>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       n, d, d_used, (const double*)y1, (const double*)target, scale, (double*)out);
  else
    hipLaunchKernelGGL(sqerr_cotangent_kernel<float>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       n, d, d_used, (const float*)y1, (const float*)target, (float)scale, (float*)out);
  return check_hip(hipGetLastError(), "cotangent kernel launch");
}

}  // extern "C"
