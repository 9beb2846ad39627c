// conv1d.hip -- causal depthwise conv1d + SiLU on gfx950, the step in front of
// the scan in the Mamba block (Mamba notes, awesome.papernotes.org, 设计 3
// block pseudo-code, kernel size 4; State space models and Mamba,
// jonathanding.github.io, Mamba block architecture: Conv1d -> SiLU -> SSM).
//
//   a[t] = bias[d] + sum_{k<K} w[d,k] x[t - (K-1) + k],   u[t] = a[t] sigmoid(a[t])
//
// with x at negative times taken from the caller's conv state (the K-1 inputs
// before the sequence, oldest first) or zero.  The work is a pure stream
// (read x once, write u once), so each thread owns 8 consecutive tokens of one
// row: one 16-byte load for its tokens plus the previous 8 tokens' load for
// the K-1 history values (the same cache line or its neighbour, served from
// L1/L2), fp32 arithmetic, one store.  Consecutive threads cover consecutive
// tokens of a row, so every wave reads and writes contiguous memory.
#include "internal.h"
#include "io.h"

namespace mscan {
namespace {

struct CArgs {
  const void* x;
  const float* w;
  const float* bias;
  const void* state_in;
  void* state_out;
  void* u;
  int64_t rows, seqlen, nchunk, dim;
  int K, silu;
};

template <typename IoT, bool kVec, int K>
__global__ __launch_bounds__(256) void conv1d_kernel(CArgs a) {
  using IO = Io<IoT>;
  using V8 = typename IO::V8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= a.rows * a.nchunk) return;
  const int64_t row = gid / a.nchunk;
  const int64_t t0 = (gid % a.nchunk) * 8;
  const int64_t d = row % a.dim;
  const IoT* xr = static_cast<const IoT*>(a.x) + row * a.seqlen;
  const IoT* st = a.state_in ? static_cast<const IoT*>(a.state_in) + row * (K - 1) : nullptr;
  const int nv = (int)min((int64_t)8, a.seqlen - t0);

  // xx[0..2]: inputs at t0-3 .. t0-1, xx[3..10]: inputs at t0 .. t0+7
  float xx[11];
  {
    float cur[8];
    if (kVec && nv == 8) {
      IO::to_f32(IO::load8(xr + t0), cur);
    } else {
      IO::to_f32(IO::load_n(xr + t0, nv), cur);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) xx[3 + i] = cur[i];
    if (t0 >= 8) {
      float prev[8];
      if (kVec)
        IO::to_f32(IO::load8(xr + t0 - 8), prev);
      else
        IO::to_f32(IO::load_n(xr + t0 - 8, 8), prev);
      xx[0] = prev[5]; xx[1] = prev[6]; xx[2] = prev[7];
    } else {
      // t0 == 0: history from the conv state (K-1 values, oldest first) or zero
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int back = 3 - i;   // input time -back
        xx[i] = (st && back <= K - 1) ? IO::load1(st + (K - 1 - back)) : 0.0f;
      }
    }
  }
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = a.w[d * K + k];
  const float bi = a.bias ? a.bias[d] : 0.0f;
  constexpr int base = 4 - K;   // xx index of tap 0 for output i = 0

  float out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float acc = bi;
#pragma unroll
    for (int k = 0; k < K; ++k) acc = fmaf(wk[k], xx[base + i + k], acc);   // input time t0 + i - (K-1) + k
    out[i] = a.silu ? acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * 1.4426950408889634f)) : acc;
  }
  IoT* ur = static_cast<IoT*>(a.u) + row * a.seqlen;
  if (kVec && nv == 8)
    IO::store8(ur + t0, IO::from_f32(out));
  else
    IO::store_n(ur + t0, IO::from_f32(out), nv);
}

// The K-1 inputs before the end of the sequence, oldest first (one thread per
// row, in increasing order, so the state may be updated in place).
template <typename IoT>
__global__ __launch_bounds__(256) void conv_state_kernel(CArgs a) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= a.rows) return;
  const int S = a.K - 1;
  const IoT* xr = static_cast<const IoT*>(a.x) + row * a.seqlen;
  const IoT* si = a.state_in ? static_cast<const IoT*>(a.state_in) + row * S : nullptr;
  IoT* so = static_cast<IoT*>(a.state_out) + row * S;
  for (int i = 0; i < S; ++i) {
    const int64_t tt = a.seqlen - S + i;
    IoT v;
    if (tt >= 0)
      v = xr[tt];
    else
      v = si ? si[S + tt] : IoT(0);
    so[i] = v;
  }
}

template <typename IoT>
hipError_t run_conv(const ConvArgs& c, hipStream_t s) {
  CArgs a{};
  a.x = c.x; a.w = c.weight; a.bias = c.bias; a.state_in = c.state_in; a.state_out = c.state_out; a.u = c.u;
  a.rows = c.batch * c.dim; a.seqlen = c.seqlen; a.dim = c.dim; a.K = (int)c.K; a.silu = c.silu;
  a.nchunk = (c.seqlen + 7) / 8;
  if (c.seqlen > 0) {
    const uintptr_t mis = reinterpret_cast<uintptr_t>(c.x) | reinterpret_cast<uintptr_t>(c.u);
    const bool vec = ((mis & 15) == 0) && ((c.seqlen * (int64_t)sizeof(IoT)) % 16 == 0);
    const int64_t n = a.rows * a.nchunk;
    const dim3 grid((unsigned)((n + 255) / 256));
    switch ((int)c.K) {
#define MSCAN_CONV_LAUNCH(KK)                                                          \
  case KK:                                                                             \
    if (vec)                                                                           \
      hipLaunchKernelGGL((conv1d_kernel<IoT, true, KK>), grid, dim3(256), 0, s, a);    \
    else                                                                               \
      hipLaunchKernelGGL((conv1d_kernel<IoT, false, KK>), grid, dim3(256), 0, s, a);   \
    break;
      MSCAN_CONV_LAUNCH(1)
      MSCAN_CONV_LAUNCH(2)
      MSCAN_CONV_LAUNCH(3)
      MSCAN_CONV_LAUNCH(4)
#undef MSCAN_CONV_LAUNCH
      default:
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (c.state_out && c.K > 1) {
    hipLaunchKernelGGL(conv_state_kernel<IoT>, dim3((unsigned)((a.rows + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
  return a.io_bf16 ? run_conv<uint16_t>(a, stream) : run_conv<float>(a, stream);
}

}  // namespace mscan
