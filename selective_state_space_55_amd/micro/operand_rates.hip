// operand_rates.hip -- gfx950 VALU issue rates by operand kind and by waves per SIMD,
// and the throughput of the selective scan's per-(token, state) instruction mix.
// Part 1: v_fmac_f32 with VGPR / SGPR / DPP row_newbcast operands, v_mul_f32,
// VOP3 v_fma_f32, v_exp_f32, an exp+fma pair and one dependent fmac chain, each
// as 8 independent chains per thread (inline asm fixes the instruction form).
// Part 2: the scan's inner step (Abar = exp2(Delta A), s = B u / A,
// h = Abar (h + s) - s, y += C h) for 4 or 2 states per lane, with B and C taken
// through DPP broadcast, from an SGPR, or from a per-lane VGPR.
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//          -o operand_rates operand_rates.hip
// Every thread writes one float to out[blockIdx.x * blockDim.x + threadIdx.x]; out is
// sized for the largest grid launched.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include "../csrc/io.h"
#define CHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)
using namespace mscan;
constexpr int ITERS = 1024;
#define CHAINS(OP) _Pragma("unroll") for (int i = 0; i < 8; ++i) OP;
__global__ void k_vv(float* out, float a0) {   // v_fmac_f32 with VGPR operands
  float x[8]; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f + threadIdx.x * 1e-7f;
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) { CHAINS(asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(x[i]) : "v"(a), "v"(b))) }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_sv(float* out, float a0) {   // one SGPR operand
  float x[8]; float b = 0.999f + threadIdx.x * 1e-7f;
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) { CHAINS(asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(x[i]) : "s"(a0), "v"(b))) }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_mul(float* out, float a0) {   // v_mul_f32 VGPR
  float x[8]; float b = 0.999f + threadIdx.x * 1e-7f;
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) { CHAINS(asm volatile("v_mul_f32_e32 %0, %0, %1" : "+v"(x[i]) : "v"(b))) }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_fma3(float* out, float a0) {   // v_fma_f32 (VOP3) with neg modifier
  float x[8]; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f + threadIdx.x * 1e-7f;
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) { CHAINS(asm volatile("v_fma_f32 %0, %1, %0, -%2" : "+v"(x[i]) : "v"(a), "v"(b))) }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_dpp(float* out, float a0) {
  float x[8]; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f + threadIdx.x * 1e-7f;
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  for (int it = 0; it < ITERS; ++it) { CHAINS(asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:3 row_mask:0xf bank_mask:0xf" : "+v"(x[i]) : "v"(a), "v"(b))) }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_exp(float* out, float a0) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-4f + i * 0.01f;
  for (int it = 0; it < ITERS; ++it) { CHAINS(asm volatile("v_exp_f32_e64 %0, -%0" : "+v"(x[i]))) }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_expfma(float* out, float a0) {   // 8 exp + 8 fma per iteration on separate chains
  float x[8], y[8]; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f + threadIdx.x * 1e-7f;
  for (int i = 0; i < 8; ++i) { x[i] = threadIdx.x * 1e-4f + i * 0.01f; y[i] = i; }
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      asm volatile("v_exp_f32_e64 %0, -%0" : "+v"(x[i]));
      asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(y[i]) : "v"(a), "v"(b));
    }
  }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i] + y[i]; out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ void k_chain1(float* out, float a0) {   // one dependent chain: latency
  float x = threadIdx.x * 1e-3f; float a = a0 + threadIdx.x * 1e-6f, b = 0.999f;
  for (int it = 0; it < ITERS * 8; ++it) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
  out[blockIdx.x * blockDim.x + threadIdx.x] = x;
}
constexpr int TOK = 2048;
// MODE 0: current form (3 vv + 3 dpp + exp); 1: h+s as vv add (4 vv + 2 dpp + exp);
// 2: B, C from SGPR (uniform); 3: B, C from per-lane VGPR (no broadcast); 4: exp only+arg; 5: no exp (exp replaced by mul)
template <int NPW, int MODE>
__global__ __launch_bounds__(256) void hot(float* out, float s0, float sB, float sC) {
  const int lane = threadIdx.x & 63;
  float A[NPW], iA[NPW], h[NPW];
  for (int j = 0; j < NPW; ++j) { A[j] = -(j + 1) * 1.4426950f; iA[j] = -1.0f / (j + 1); h[j] = 0.01f * lane; }
  float dl0 = 0.05f + lane * 1e-4f, uu0 = 0.3f - lane * 1e-3f;
  float bq = 0.5f + lane * 1e-3f, cq = -0.25f + lane * 2e-3f;
  float ysum = 0.0f;
  const float bs = __builtin_amdgcn_readfirstlane(__float_as_uint(sB)) ? sB : sB;  // uniform
  for (int t = 0; t < TOK; t += 4) {
    float yy[4];
    static_for<4>([&](auto kk_c) {
      constexpr int kk = decltype(kk_c)::value;
      const float dl = dl0 + kk * 1e-3f, uu = uu0 - kk * 1e-3f;
      float acc = 0.0f;
      static_for<NPW>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        constexpr int src = (4 * j + kk) & 15;
        float av;
        if constexpr (MODE == 5) av = dl * A[j] + 1.0f; else av = __builtin_amdgcn_exp2f(dl * A[j]);
        const float v = uu * iA[j];
        float sv, hs;
        if constexpr (MODE == 0) { sv = dpp_bcast_mul<src>(bq, v); hs = dpp_bcast_fmac<src>(h[j], bq, v); }
        else if constexpr (MODE == 1 || MODE == 5) { sv = dpp_bcast_mul<src>(bq, v); hs = h[j] + sv; }
        else if constexpr (MODE == 2) { sv = sB * v; hs = h[j] + sv; }
        else if constexpr (MODE == 3) { sv = bq * v; hs = h[j] + sv; }
        else { sv = v; hs = h[j] + sv; }
        h[j] = fmaf(av, hs, -sv);
        if constexpr (MODE == 0 || MODE == 1 || MODE == 5) acc = j == 0 ? dpp_bcast_mul<src>(cq, h[j]) : dpp_bcast_fmac<src>(acc, cq, h[j]);
        else if constexpr (MODE == 2) acc = fmaf(sC, h[j], acc);
        else if constexpr (MODE == 3) acc = fmaf(cq, h[j], acc);
        else acc += h[j];
      });
      yy[kk] = acc;
    });
    ysum += (yy[0] + yy[1]) + (yy[2] + yy[3]);
    dl0 = dl0 * 0.999f; uu0 = uu0 + 1e-4f;
  }
  float hs = 0; for (int j = 0; j < NPW; ++j) hs += h[j];
  out[blockIdx.x * 64 + lane] = ysum + hs + s0;
}
template <typename F> float time_ms(F f, int reps = 5) {
  hipEvent_t e0, e1; CHK(hipEventCreate(&e0)); CHK(hipEventCreate(&e1));
  f(); CHK(hipDeviceSynchronize()); CHK(hipEventRecord(e0));
  for (int r = 0; r < reps; ++r) f();
  CHK(hipEventRecord(e1)); CHK(hipEventSynchronize(e1));
  float ms; CHK(hipEventElapsedTime(&ms, e0, e1)); return ms / reps;
}
int main() {
  hipDeviceProp_t p; CHK(hipGetDeviceProperties(&p, 0)); const int cus = p.multiProcessorCount;
  float* out; CHK(hipMalloc(&out, sizeof(float) * cus * 4 * 8 * 64));
  printf("part 1: lane-ops per CU per clock at 2.4 GHz (8 chains x %d iters per thread)\n", ITERS);
  for (int wps : {1, 2, 4, 8}) {
    const int blocks = cus * 4 * wps, threads = 64;   // one wave per block
    double ops = (double)blocks * threads * ITERS * 8;
    auto rate = [&](float ms) { return ops / (ms * 1e-3) / cus / 2.4e9; };
#define T(K) time_ms([&] { hipLaunchKernelGGL(K, dim3(blocks), dim3(threads), 0, 0, out, 1.0f); })
    float tvv = T(k_vv), tsv = T(k_sv), tmul = T(k_mul), tf3 = T(k_fma3), tdpp = T(k_dpp), texp = T(k_exp), tef = T(k_expfma), tc1 = T(k_chain1);
#undef T
    printf("[%d waves/SIMD] fmac_vv %.1f  fmac_sv %.1f  mul %.1f  fma_vop3 %.1f  fmac_dpp %.1f  exp %.1f  | exp+fma pair %.3f ms (exp %.3f + fma %.3f) | 1-chain fmac %.1f\n",
           wps, rate(tvv), rate(tsv), rate(tmul), rate(tf3), rate(tdpp), rate(texp), tef, texp, tvv, rate(tc1));
    fflush(stdout);
  }
  printf("part 2: CU-clocks per 64 lane-(token, state) updates at 2.4 GHz (lower is better)\n");
  printf("  cur: B and C by DPP, h + s by DPP fmac; add: h + s by plain add; sgpr / vgpr: B, C from SGPR / per-lane VGPR;\n");
  printf("  noBC: no B/C operands; noexp: exp replaced by one fma\n");
  for (int wps : {1, 2, 4, 8}) {
    const int blocks = cus * 4 * wps;
    auto cost = [&](float ms, int npw) { double upd = (double)blocks * 64 * TOK * npw; return ms * 1e-3 * 2.4e9 * cus / upd * 64; };
#define T(NPW, M) cost(time_ms([&] { hipLaunchKernelGGL((hot<NPW, M>), dim3(blocks), dim3(64), 0, 0, out, 1.0f, 0.5f, -0.25f); }), NPW)
    printf("[%d w/SIMD] 4 states/lane: cur %.2f  add %.2f  sgpr %.2f  vgpr %.2f  noBC %.2f  noexp %.2f | 2 states/lane: cur %.2f add %.2f sgpr %.2f vgpr %.2f\n", wps,
           T(4, 0), T(4, 1), T(4, 2), T(4, 3), T(4, 4), T(4, 5), T(2, 0), T(2, 1), T(2, 2), T(2, 3));
#undef T
    fflush(stdout);
  }
  return 0;
}
