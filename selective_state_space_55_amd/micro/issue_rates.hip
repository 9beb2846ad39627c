// issue_rates.hip -- gfx950 issue-rate and bandwidth microbenchmark: v_exp_f32 / v_log_f32 vs v_fma_f32
// throughput, whether transcendental and plain VALU issue overlap, and 1 GiB copy / read bandwidth.
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops -o issue_rates issue_rates.hip
// All buffers are sized from the launch grid below; every index is < n.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)

constexpr int ITERS = 2048;

__global__ void k_fma(float* out, float a, float b) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], a, b);
  }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void k_exp(float* out) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-4f + i * 0.01f;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void k_log(float* out) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = 1.5f + threadIdx.x * 1e-4f + i * 0.01f;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_logf(x[i]) + 2.0f;  // 1 log + 1 add
  }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// R independent fmas per exp, on separate registers: measures whether the
// transcendental issue overlaps plain VALU issue.
template <int R>
__global__ void k_mix(float* out, float a, float b) {
  float x[8], y[8 * R];
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-4f + i * 0.01f;
  for (int i = 0; i < 8 * R; ++i) y[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = __builtin_amdgcn_exp2f(-x[i]);
#pragma unroll
      for (int r = 0; r < R; ++r) y[i * R + r] = fmaf(y[i * R + r], a, b);
    }
  }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i];
  for (int i = 0; i < 8 * R; ++i) s += y[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void k_copy(const float4* __restrict__ src, float4* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ void k_read(const float4* __restrict__ src, float* out, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  float s = 0;
  for (; i < n; i += stride) { float4 v = src[i]; s += v.x + v.y + v.z + v.w; }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <typename F>
float time_ms(F f, int reps = 5) {
  hipEvent_t a, b; CHK(hipEventCreate(&a)); CHK(hipEventCreate(&b));
  f(); CHK(hipDeviceSynchronize());
  CHK(hipEventRecord(a));
  for (int r = 0; r < reps; ++r) f();
  CHK(hipEventRecord(b)); CHK(hipEventSynchronize(b));
  float ms; CHK(hipEventElapsedTime(&ms, a, b));
  return ms / reps;
}

int main() {
  hipDeviceProp_t p; CHK(hipGetDeviceProperties(&p, 0));
  printf("device %s gcnArch %s CUs %d clock %d kHz\n", p.name, p.gcnArchName, p.multiProcessorCount, p.clockRate);
  fflush(stdout);
  const int cus = p.multiProcessorCount;
  float* out;
  const int maxBlocks = cus * 16, bs = 256;
  CHK(hipMalloc(&out, sizeof(float) * maxBlocks * bs));
  // configs: (blocks, threads) -> waves per SIMD = blocks*threads/64/(4*cus)
  struct Cfg { int blocks, threads; const char* name; };
  Cfg cfgs[] = { {cus * 4, 64, "1 wave/SIMD"}, {cus * 8, 64, "2 waves/SIMD"}, {cus * 8, 256, "8 waves/SIMD"} };
  for (auto c : cfgs) {
    double lanes = (double)c.blocks * c.threads;
    double ops = lanes * ITERS * 8;  // per chain-instruction count
    float t_fma = time_ms([&] { hipLaunchKernelGGL(k_fma, dim3(c.blocks), dim3(c.threads), 0, 0, out, 0.999f, 0.001f); });
    float t_exp = time_ms([&] { hipLaunchKernelGGL(k_exp, dim3(c.blocks), dim3(c.threads), 0, 0, out); });
    float t_log = time_ms([&] { hipLaunchKernelGGL(k_log, dim3(c.blocks), dim3(c.threads), 0, 0, out); });
    float t_m1 = time_ms([&] { hipLaunchKernelGGL(k_mix<1>, dim3(c.blocks), dim3(c.threads), 0, 0, out, 0.999f, 0.001f); });
    float t_m2 = time_ms([&] { hipLaunchKernelGGL(k_mix<2>, dim3(c.blocks), dim3(c.threads), 0, 0, out, 0.999f, 0.001f); });
    float t_m4 = time_ms([&] { hipLaunchKernelGGL(k_mix<4>, dim3(c.blocks), dim3(c.threads), 0, 0, out, 0.999f, 0.001f); });
    float t_m6 = time_ms([&] { hipLaunchKernelGGL(k_mix<6>, dim3(c.blocks), dim3(c.threads), 0, 0, out, 0.999f, 0.001f); });
    // lane-ops per CU per cycle at 2.4 GHz
    auto rate = [&](double n, float ms) { return n / (ms * 1e-3) / cus / 2.4e9; };
    printf("[%s] fma: %.3f ms  %.2f lane-op/CU/clk | exp: %.3f ms %.2f | log+add: %.3f ms %.2f (pairs)\n", c.name,
           t_fma, rate(ops, t_fma), t_exp, rate(ops, t_exp), t_log, rate(ops, t_log));
    printf("[%s] mix R=1: %.3f ms  R=2: %.3f ms  R=4: %.3f ms  R=6: %.3f ms  (fma-only equiv per R: %.3f ms)\n", c.name,
           t_m1, t_m2, t_m4, t_m6, t_fma);
    fflush(stdout);
  }
  // bandwidth
  size_t bytes = (size_t)1 << 30, n4 = bytes / 16;
  float4 *src, *dst; CHK(hipMalloc(&src, bytes)); CHK(hipMalloc(&dst, bytes));
  CHK(hipMemset(src, 0, bytes)); CHK(hipMemset(dst, 0, bytes));
  for (int wpc : {4, 8, 16}) {
    int blocks = cus * wpc;
    float tc = time_ms([&] { hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, 0, src, dst, n4); }, 10);
    float tr = time_ms([&] { hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, 0, src, out, n4); }, 10);
    printf("copy 1GiB (blocks=%d): %.3f ms -> %.1f GB/s (r+w) | read 1GiB: %.3f ms -> %.1f GB/s\n", blocks, tc,
           2.0 * bytes / (tc * 1e-3) / 1e9, tr, 1.0 * bytes / (tr * 1e-3) / 1e9);
    fflush(stdout);
  }
  float td = time_ms([&] { CHK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, 0)); }, 10);
  printf("hipMemcpy D2D 1GiB: %.3f ms -> %.1f GB/s (r+w)\n", td, 2.0 * bytes / (td * 1e-3) / 1e9);
  CHK(hipFree(src)); CHK(hipFree(dst)); CHK(hipFree(out));
  return 0;
}
