// scan_step.hip -- single-token recurrent update (O(1) decoding) on gfx950.
//
// One iteration of the forward recurrence applied to a caller-held fp32
// state (State space models and Mamba, jonathanding.github.io, §3, recurrence
// mode; Mamba notes, awesome.papernotes.org, 设计 2: a fixed (d, N) state
// instead of a KV cache).  The step is a pure stream over the state: it reads
// and writes 2 * N * 4 bytes per (batch, channel) and a handful of bf16/fp32
// scalars, so the kernel is laid out for coalesced 16-byte state traffic:
// four lanes own one (batch, channel), lane q holding states 4q .. 4q+3 as one
// float4; consecutive quads cover consecutive channels, so a wave moves 1 KB
// of contiguous state per access.  The readout sum over the four lanes uses
// two cross-lane adds in a fixed order, so results are deterministic.
#include "internal.h"
#include "io.h"

namespace mscan {
namespace {

struct SArgs {
  float* state;
  const void* x;
  const void* dt;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* y;
  int64_t batch, dim;
  int dstate, softplus, vec_ok;
};

template <typename IoT>
__global__ __launch_bounds__(256) void scan_step_kernel(SArgs a) {
  using IO = Io<IoT>;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bd = gid >> 2;
  const int q = (int)(gid & 3);
  const int64_t nbd = a.batch * a.dim;
  const bool live = bd < nbd;   // whole quads share bd, so a quad is live or dead together
  const int64_t bdc = live ? bd : 0;
  const int64_t b = bdc / a.dim;
  const int64_t d = bdc % a.dim;

  const IoT* gx = static_cast<const IoT*>(a.x);
  const IoT* gdt = static_cast<const IoT*>(a.dt);
  const IoT* gB = static_cast<const IoT*>(a.B);
  const IoT* gC = static_cast<const IoT*>(a.C);

  const float xv = live ? IO::load1(gx + bdc) : 0.0f;
  const float xr = (live ? IO::load1(gdt + bdc) : 0.0f) + (a.bias ? a.bias[d] : 0.0f);
  const float dl = a.softplus ? softplus_log2e(xr) : xr * 1.4426950408889634f;   // Delta * log2e

  float hs[4];
  float* st = a.state + bdc * a.dstate + 4 * q;
  if (live && a.vec_ok) {
    const float4 v = *reinterpret_cast<const float4*>(st);
    hs[0] = v.x; hs[1] = v.y; hs[2] = v.z; hs[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) hs[j] = (live && 4 * q + j < a.dstate) ? st[j] : 0.0f;
  }

  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * q + j;
    if (n < a.dstate) {
      const float An = -expf(a.A_log[d * a.dstate + n]);
      const float Bn = IO::load1(gB + b * a.dstate + n);
      const float Cn = IO::load1(gC + b * a.dstate + n);
      const float av = __builtin_amdgcn_exp2f(dl * An);
      const float s = Bn * (xv * (1.0f / An));
      hs[j] = fmaf(av, hs[j] + s, -s);
      acc = fmaf(Cn, hs[j], acc);
    }
  }
  // sum over the quad: (q0 + q1) + (q2 + q3)
  acc += __shfl_xor(acc, 1, 4);
  acc += __shfl_xor(acc, 2, 4);

  if (!live) return;
  if (a.vec_ok) {
    *reinterpret_cast<float4*>(st) = make_float4(hs[0], hs[1], hs[2], hs[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * q + j < a.dstate) st[j] = hs[j];
  }
  if (q == 0) {
    float yv = fmaf(a.D ? a.D[d] : 0.0f, xv, acc);
    if (a.z) yv *= silu(IO::load1(static_cast<const IoT*>(a.z) + bdc));
    IO::store1(static_cast<IoT*>(a.y) + bdc, yv);
  }
}

template <typename IoT>
hipError_t run_step(const StepArgs& s, hipStream_t stream) {
  SArgs a{};
  a.state = s.state; a.x = s.x; a.dt = s.dt; a.A_log = s.A_log; a.B = s.B; a.C = s.C; a.D = s.D; a.z = s.z;
  a.bias = s.bias; a.y = s.y; a.batch = s.batch; a.dim = s.dim; a.dstate = (int)s.dstate;
  a.softplus = s.softplus;
  a.vec_ok = (s.dstate == 16) && ((reinterpret_cast<uintptr_t>(s.state) & 15) == 0);
  const int64_t threads = s.batch * s.dim * 4;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(scan_step_kernel<IoT>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  return a.io_bf16 ? run_step<uint16_t>(a, stream) : run_step<float>(a, stream);
}

}  // namespace mscan
