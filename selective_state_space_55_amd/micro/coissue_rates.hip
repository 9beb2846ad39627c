// coissue_rates.hip -- gfx950 VALU issue rate by instruction form and operand kind, and of pairs
// of forms, at 1, 2, 4 and 8 waves per SIMD.  Each thread runs 8 independent register-only chains
// (the asm statements name VGPR/SGPR operands only, no memory); a workgroup of 4 x wps waves per CU
// (two workgroups of 1024 at 8 waves/SIMD).  Reported: lanes per SIMD per s_memtime tick (with the
// tick rate from s_memrealtime, 100 MHz), and lanes per CU per nominal 2.4 GHz clock from the
// HIP-event wall time of the launch.  Pair rows count pairs (two instructions per statement).
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops -o coissue coissue_rates.hip
// Buffers: out has one float per thread of the grid, cyc two longs per workgroup.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#define CHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)
constexpr int ITERS = 8192;
#define BODY(ASM, ...) \
  float x[8]; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f + threadIdx.x * 1e-7f; \
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i; \
  __builtin_amdgcn_s_barrier(); \
  long t0 = __builtin_amdgcn_s_memtime(); long r0 = __builtin_amdgcn_s_memrealtime(); \
  for (int it = 0; it < ITERS; ++it) { _Pragma("unroll") for (int i = 0; i < 8; ++i) asm volatile(ASM : "+v"(x[i]) : __VA_ARGS__); } \
  long t1 = __builtin_amdgcn_s_memtime(); long r1 = __builtin_amdgcn_s_memrealtime(); \
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; \
  out[blockIdx.x * blockDim.x + threadIdx.x] = s; \
  if (threadIdx.x == 0) { cyc[2 * blockIdx.x] = t1 - t0; cyc[2 * blockIdx.x + 1] = r1 - r0; }
#define K(NAME, ASM, ...) __global__ void NAME(float* out, long* cyc, float a0) { BODY(ASM, __VA_ARGS__) }
K(k_fmac_vv, "v_fmac_f32_e32 %0, %1, %2", "v"(a), "v"(b))
K(k_add_vv, "v_add_f32_e32 %0, %0, %1", "v"(b))
K(k_add_lit, "v_add_f32_e32 %0, 0xbf7ffffe, %0", "v"(b))
K(k_add_inl, "v_add_f32_e32 %0, 1.0, %0", "v"(b))
K(k_fmamk, "v_fmamk_f32 %0, %0, 0x3e75fdf0, %1", "v"(b))
K(k_min_vv, "v_min_f32_e32 %0, %0, %1", "v"(b))
K(k_fma3_vvv, "v_fma_f32 %0, %1, %0, %2", "v"(a), "v"(b))
K(k_fmac_sv, "v_fmac_f32_e32 %0, %1, %2", "s"(a0), "v"(b))
K(k_mul_dpp, "v_mul_f32_dpp %0, %1, %2 row_newbcast:3 row_mask:0xf bank_mask:0xf", "v"(a), "v"(b))
K(k_exp, "v_exp_f32_e64 %0, -%0", "v"(b))
K(k_mov, "v_mov_b32_e32 %0, %1", "v"(b))
__global__ void k_perm32(float* out, long* cyc, float a0) {   // swap writes both operands
  float x[8], y[8];
  for (int i = 0; i < 8; ++i) { x[i] = threadIdx.x * 1e-3f + i; y[i] = i; }
  __builtin_amdgcn_s_barrier();
  long t0 = __builtin_amdgcn_s_memtime(); long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("v_permlane32_swap_b32_e32 %0, %1" : "+v"(x[i]), "+v"(y[i]));
  }
  long t1 = __builtin_amdgcn_s_memtime(); long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i] + y[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s + a0;
  if (threadIdx.x == 0) { cyc[2 * blockIdx.x] = t1 - t0; cyc[2 * blockIdx.x + 1] = r1 - r0; }
}
K(k_max_vv, "v_max_f32_e32 %0, %0, %1", "v"(b))
K(k_med3, "v_med3_f32 %0, %0, %1, %2", "v"(a), "v"(b))
K(k_sub_clamp, "v_sub_f32_e64 %0, %0, %1 clamp", "v"(b))
K(k_lshl, "v_lshlrev_b32_e32 %0, 16, %0", "v"(b))
K(k_and_lit, "v_and_b32_e32 %0, 0xffff0000, %0", "v"(b))
K(k_fma_neg, "v_fma_f32 %0, %1, %0, -%2", "v"(a), "v"(b))
K(k_cndmask, "v_cndmask_b32_e64 %0, %0, %1, s[0:1]", "v"(b))
K(k_mix_fmac_min, "v_fmac_f32_e32 %0, %1, %2\n v_min_f32_e32 %0, %0, %2", "v"(a), "v"(b))
K(k_mix_fmac_dpp, "v_fmac_f32_e32 %0, %1, %2\n v_mul_f32_dpp %0, %1, %2 row_newbcast:3 row_mask:0xf bank_mask:0xf", "v"(a), "v"(b))
K(k_mix_fmac_exp, "v_fmac_f32_e32 %0, %1, %2\n v_exp_f32_e32 %0, %0", "v"(a), "v"(b))
K(k_mix_3fmac_exp, "v_fmac_f32_e32 %0, %1, %2\n v_fmac_f32_e32 %0, %1, %2\n v_fmac_f32_e32 %0, %1, %2\n v_exp_f32_e32 %0, %0", "v"(a), "v"(b))
// a dependent chain (latency)
__global__ void k_chain(float* out, long* cyc, float a0) {
  float x = threadIdx.x * 1e-3f; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f;
  __builtin_amdgcn_s_barrier();
  long t0 = __builtin_amdgcn_s_memtime(); long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < ITERS * 8; ++it) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
  long t1 = __builtin_amdgcn_s_memtime(); long r1 = __builtin_amdgcn_s_memrealtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = x;
  if (threadIdx.x == 0) { cyc[2 * blockIdx.x] = t1 - t0; cyc[2 * blockIdx.x + 1] = r1 - r0; }
}
int main() {
  hipDeviceProp_t p; CHK(hipGetDeviceProperties(&p, 0)); const int cus = p.multiProcessorCount;
  const int maxw = 8;
  float* out; long* cyc;
  CHK(hipMalloc(&out, sizeof(float) * cus * 4 * maxw * 64));
  CHK(hipMalloc(&cyc, sizeof(long) * 2 * 2 * cus));
  long* hc = (long*)malloc(sizeof(long) * 2 * 2 * cus);
  hipEvent_t e0, e1; CHK(hipEventCreate(&e0)); CHK(hipEventCreate(&e1));
  struct { const char* n; void (*k)(float*, long*, float); } ks[] = {
    {"fmac_vv", k_fmac_vv}, {"add_vv", k_add_vv}, {"add_lit", k_add_lit}, {"add_inl", k_add_inl}, {"fmamk", k_fmamk},
    {"min_vv", k_min_vv}, {"fma3_vvv", k_fma3_vvv}, {"fmac_sv", k_fmac_sv}, {"mul_dpp", k_mul_dpp}, {"exp", k_exp},
    {"mov", k_mov}, {"perm32", k_perm32}, {"chain", k_chain}, {"max_vv", k_max_vv}, {"med3", k_med3},
    {"sub_clamp", k_sub_clamp}, {"lshl", k_lshl}, {"and_lit", k_and_lit}, {"fma_neg", k_fma_neg}, {"cndmask", k_cndmask},
    {"fmac+min", k_mix_fmac_min}, {"fmac+dpp", k_mix_fmac_dpp}, {"fmac+exp", k_mix_fmac_exp}, {"3fmac+exp", k_mix_3fmac_exp}};
  printf("lanes/SIMD/cycle = waves_per_SIMD * 64 * 8 * ITERS / median wave cycles (16 = one wave64 op per 4 cycles)\n");
  for (auto& kk : ks) {
    printf("%-9s", kk.n);
    for (int wps = 1; wps <= maxw; wps *= 2) {
      // workgroups of wps*4 waves, one per CU (4 SIMDs); 8 waves/SIMD as two workgroups of 1024 per CU
      const int per = wps > 4 ? 2 : 1;
      const int threads = 64 * 4 * wps / per, blocks = cus * per;
      for (int rep = 0; rep < 3; ++rep) hipLaunchKernelGGL(kk.k, dim3(blocks), dim3(threads), 0, 0, out, cyc, 1.0f);
      CHK(hipEventRecord(e0));
      hipLaunchKernelGGL(kk.k, dim3(blocks), dim3(threads), 0, 0, out, cyc, 1.0f);
      CHK(hipEventRecord(e1)); CHK(hipEventSynchronize(e1));
      float ms; CHK(hipEventElapsedTime(&ms, e0, e1));
      CHK(hipMemcpy(hc, cyc, sizeof(long) * 2 * blocks, hipMemcpyDeviceToHost));
      double s = 0, r = 0; for (int i = 0; i < blocks; ++i) { s += hc[2 * i]; r += hc[2 * i + 1]; }
      double c = s / blocks, rt = r / blocks;                 // ticks, realtime ticks (100 MHz)
      double lanes = wps * 64.0 * 8 * ITERS / c;              // lanes per SIMD per memtime tick (all wps waves run for c ticks)
      double ghz = c / (rt * 10.0);                           // memtime ticks per ns
      double wall = 64.0 * 8 * ITERS * threads / 64 * blocks / (ms * 1e6) / cus / 2.4;   // lanes (statements) per CU per nominal 2.4 GHz clock
      printf("  %dw %6.2f/t (%.2f GHz) wall %6.1f/CU/clk", wps, lanes, ghz, wall);
    }
    printf("\n"); fflush(stdout);
  }
  return 0;
}
