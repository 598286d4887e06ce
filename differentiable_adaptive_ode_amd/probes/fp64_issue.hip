// FP64 issue-rate probe for one MI355X SIMD: how many FP64 fused multiply-adds
// per second the chip completes when each SIMD holds 1, 2 or 4 wavefronts,
// with all 64 lanes or only part of them active, at 3, 4 or 8 independent
// dependency chains per lane.  It bounds what a per-lane ODE kernel with one
// wavefront per SIMD can reach.  Build and run:
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -o /tmp/fp64_issue fp64_issue.hip && /tmp/fp64_issue
// Each active lane runs C independent FMA chains for `iters` steps.
// active = lanes per wavefront that work (64, 32, 16); waves per SIMD set by the grid.
#include <hip/hip_runtime.h>
#include <cstdio>
template <int C>
__global__ void __launch_bounds__(256) chains(double* out, int iters, double a, double b, int active) {
  const int lane = threadIdx.x & 63;
  double s = 0;
  if (lane < active) {
    double x[C];
#pragma unroll
    for (int c = 0; c < C; ++c) x[c] = threadIdx.x * 1e-3 + c;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < C; ++c) x[c] = __builtin_fma(x[c], a, b);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) s += x[c];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}
template <int C>
float run(int blocks, double* out, int iters, int active) {
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  hipLaunchKernelGGL(chains<C>, dim3(blocks), dim3(256), 0, 0, out, iters, 0.999, 1e-3, active);
  (void)hipEventRecord(e0);
  hipLaunchKernelGGL(chains<C>, dim3(blocks), dim3(256), 0, 0, out, iters, 0.999, 1e-3, active);
  (void)hipEventRecord(e1);
  (void)hipEventSynchronize(e1);
  float ms;
  (void)hipEventElapsedTime(&ms, e0, e1);
  return ms;
}
int main() {
  const int maxblocks = 256 * 8;
  double* out;
  if (hipMalloc(&out, (size_t)maxblocks * 256 * sizeof(double)) != hipSuccess) return 1;
  const int iters = 20000;
  // useful lane-FMAs per SIMD held fixed at 64 lanes x C x iters: waves/SIMD = 64 / active
  struct Cfg { int wps, active; };
  Cfg cfgs[] = {{1, 64}, {2, 32}, {4, 16}, {2, 64}, {4, 64}};
  for (auto c : cfgs) {
    const int blocks = 256 * c.wps;  // 4 waves per block, 256 CUs
    float t4 = run<4>(blocks, out, iters, c.active);
    float t8 = run<8>(blocks, out, iters, c.active);
    float t3 = run<3>(blocks, out, iters, c.active);
    const double lanefma = 64.0 * 4 * 256 * c.wps * (c.active / 64.0);  // active lanes on the chip
    printf("waves/SIMD %d active %2d: C3 %.3f ms (%.2f TF)  C4 %.3f ms (%.2f TF)  C8 %.3f ms (%.2f TF)\n",
           c.wps, c.active, t3, lanefma * 3 * iters * 2 / (t3 * 1e9), t4,
           lanefma * 4 * iters * 2 / (t4 * 1e9), t8, lanefma * 8 * iters * 2 / (t8 * 1e9));
  }
  printf("ok\n");
  return 0;
}
