// hot_loop_mix.hip -- the forward scan's per-(token, state) step (two states per lane, four-token
// groups, as in the forward kernel) in variants, timed alone: CU-clocks (nominal 2.4 GHz) per 64
// (token, state) updates, from the HIP-event wall time of a launch at 2, 3 and 4 waves per SIMD.
// Register-only loop (no memory but one store per thread at the end, one float per thread of the grid).
// Build (from the repo root): hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//   -o hotmix selective_state_space_55_amd/micro/hot_loop_mix.hip
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include "../csrc/io.h"
#define CHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)
using namespace mscan;
constexpr int TOK = 4096;
// MODE: 0 B and C through DPP row broadcasts; 1 B and C as per-lane VGPR operands (the kernel's form);
// 2 as 1 with decay_m1's constants in VGPRs and a plain min; 3 as 1 with m = ab - 1 (the imprecise
// decrement); 4 as 1 with the exp replaced by an fma (exp cost); 5 the earlier update form
// Abar (h + s) - s with DPP operands; 6 as 1 with decay_m1 written out (the clamped-fma form)
template <int MODE>
__global__ __launch_bounds__(256) void hot(float* out, float s0, float kc0, float kc1, float kc2) {
  const int lane = threadIdx.x & 63;
  float A[2], iA[2], h[2];
  for (int j = 0; j < 2; ++j) { A[j] = -(j + 1) * 1.4426950f - lane * 1e-4f; iA[j] = -1.0f / (j + 1); h[j] = 0.01f * lane; }
  float dl0 = 0.05f + lane * 1e-4f, uu0 = 0.3f - lane * 1e-3f;
  float bq = 0.5f + lane * 1e-3f, cq = -0.25f + lane * 2e-3f;
  float bv[2][4], cv[2][4];
  for (int j = 0; j < 2; ++j) for (int k = 0; k < 4; ++k) { bv[j][k] = bq + j * 0.1f + k * 0.01f; cv[j][k] = cq - j * 0.1f + k * 0.02f; }
  // constants: MODE 2 keeps them in VGPRs (values opaque to the compiler)
  float c0 = kc0 + lane * 0.0f, c1 = kc1 + lane * 0.0f, c2 = kc2 + lane * 0.0f;
  float ysum = 0.0f;
  for (int t = 0; t < TOK; t += 4) {
    float yy[4];
    static_for<4>([&](auto kk_c) {
      constexpr int kk = decltype(kk_c)::value;
      const float dl = dl0 + kk * 1e-3f, uu = uu0 - kk * 1e-3f;
      float acc = 0.0f;
      static_for<2>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        constexpr int src = 4 * j + kk;
        const float y = dl * A[j];
        float m;
        if constexpr (MODE == 5) {
          const float av = __builtin_amdgcn_exp2f(y);
          const float sv = dpp_bcast_mul<src>(bq, uu * iA[j]);
          h[j] = fmaf(av, h[j] + sv, -sv);
        } else {
          const float ab = MODE == 4 ? fmaf(y, 0.7f, 1.0f) : __builtin_amdgcn_exp2f(y);
          if constexpr (MODE == 2) {
            const float p2 = y * fmaf(y, c2, c1);
            m = fminf(ab - c0, p2);
          } else if constexpr (MODE == 6) {
            const float p2 = y * fmaf(y, 0.2402265069591007f, 0.6931471805599453f);
            const float m0 = ab - 0.99999988079071044921875f;
            m = m0 - __builtin_amdgcn_fmed3f(m0 - p2, 0.0f, 1.0f);
          } else if constexpr (MODE == 3) {
            m = ab - 1.0f;
          } else {
            m = decay_m1<false>(y, ab);
          }
          float sv;
          if constexpr (MODE == 0) sv = dpp_bcast_mul<src>(bq, uu * iA[j]);
          else sv = bv[j][kk] * (uu * iA[j]);
          h[j] = fmaf(m, h[j] + sv, h[j]);
        }
        if constexpr (MODE == 0 || MODE == 5) acc = j == 0 ? dpp_bcast_mul<src>(cq, h[j]) : dpp_bcast_fmac<src>(acc, cq, h[j]);
        else acc = j == 0 ? cv[j][kk] * h[j] : fmaf(cv[j][kk], h[j], acc);
      });
      yy[kk] = acc;
    });
    ysum += (yy[0] + yy[1]) + (yy[2] + yy[3]);
    dl0 = dl0 * 0.999f; uu0 = uu0 + 1e-4f;
  }
  out[blockIdx.x * 256 + threadIdx.x] = ysum + h[0] + h[1] + s0;
}
template <typename F> float time_ms(F f, int reps = 5) {
  hipEvent_t e0, e1; CHK(hipEventCreate(&e0)); CHK(hipEventCreate(&e1));
  for (int r = 0; r < 3; ++r) f();
  CHK(hipDeviceSynchronize()); CHK(hipEventRecord(e0));
  for (int r = 0; r < reps; ++r) f();
  CHK(hipEventRecord(e1)); CHK(hipEventSynchronize(e1));
  float ms; CHK(hipEventElapsedTime(&ms, e0, e1)); return ms / reps;
}
int main() {
  hipDeviceProp_t p; CHK(hipGetDeviceProperties(&p, 0)); const int cus = p.multiProcessorCount;
  float* out; CHK(hipMalloc(&out, sizeof(float) * cus * 4 * 256));
  printf("CU-clocks (2.4 GHz nominal) per 64 (token, state) updates, 2 states per lane; 256-thread blocks\n");
  for (int wps : {2, 3, 4}) {
    const int blocks = cus * wps;   // 4 waves per block: wps blocks per CU -> wps waves per SIMD
    auto cost = [&](float ms) { double upd = (double)blocks * 256 * TOK * 2; return ms * 1e-3 * 2.4e9 * cus / upd * 64; };
#define T(M) cost(time_ms([&] { hipLaunchKernelGGL((hot<M>), dim3(blocks), dim3(256), 0, 0, out, 1.0f, 0.99999988079071044921875f, 0.6931471805599453f, 0.2402265069591007f); }))
    printf("[%d w/SIMD] dppBC %.2f | vgprBC %.2f | +vgpr consts, min %.2f | m = ab-1 %.2f | no exp %.2f | Abar(h+s)-s %.2f | clamp %.2f\n", wps,
           T(0), T(1), T(2), T(3), T(4), T(5), T(6));
#undef T
    fflush(stdout);
  }
  return 0;
}
