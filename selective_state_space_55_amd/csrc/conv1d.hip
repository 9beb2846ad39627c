// conv1d.hip -- causal depthwise conv1d + SiLU on gfx950, the step in front of
// the scan in the Mamba block: conv, then SiLU, then the SSM (Mamba concept
// page, compassingai.com, §3.3 flow; State space models and Mamba,
// jonathanding.github.io, Mamba block architecture -- the Mamba notes' 设计 3
// pseudo-code, which applies SiLU first, is not followed), kernel size 4 (Mamba
// notes, awesome.papernotes.org, 设计 3).
//
//   a[t] = bias[d] + sum_{k<K} w[d,k] x[t - (K-1) + k],   u[t] = a[t] sigmoid(a[t])
//
// with x at negative times taken from the caller's conv state (the K-1 inputs
// before the sequence, oldest first) or zero.  The work is a pure stream
// (read x once, write u once, a few flops per element), so the layout is the
// one a plain copy runs at full speed with: each wave owns 512 consecutive
// tokens of one (batch, channel) row, lane l the 8 tokens at 8l .. 8l+7 (one
// 16-byte load and store per lane for bf16), so every load instruction of a
// wave covers 1 KB of contiguous memory.  The K-1 inputs before a lane's
// piece are the last ones of the lane below, fetched with a cross-lane read;
// only lane 0 goes to memory (or to the conv state) for them.  The grid is
// (segment groups, channels, batch rows), so a wave finds its row and channel
// from the block indices without a division; a workgroup holds up to four
// waves (fewer for rows shorter than 2048 tokens).  Arithmetic is fp32.
#include "internal.h"
#include "io.h"

#include <algorithm>

namespace mscan {
namespace {

constexpr int kSeg = 512;   // tokens per wave

struct CArgs {
  const void* x;
  const float* w;
  const float* bias;
  const void* state_in;
  void* state_out;
  void* u;
  int64_t rows, seqlen, nseg, dim;
  int64_t d0, b0;   // channel and batch offsets of this launch
  int K, silu;
};

template <typename IoT, bool kVec, int K>
__global__ __launch_bounds__(256) void conv1d_kernel(CArgs a) {
  using IO = Io<IoT>;
  const int lane = threadIdx.x & 63;
  const int64_t seg =
      (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (seg >= a.nseg) return;   // whole waves
  const int64_t d = a.d0 + blockIdx.y;
  const int64_t row = (a.b0 + blockIdx.z) * a.dim + d;
  const int64_t base = seg * kSeg;
  const IoT* xr = static_cast<const IoT*>(a.x) + row * a.seqlen;
  const int64_t t0 = base + 8 * lane;
  const int nv = (int)max((int64_t)0, min((int64_t)8, a.seqlen - t0));

  // every load is issued before the first wait: taps, bias, the lane's
  // inputs, and lane 0's three inputs before the segment (from x, or from the
  // conv state at the start of the row)
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = a.w[d * K + k];
  const float bi = a.bias ? a.bias[d] : 0.0f;
  float cur[8];
  if (kVec && nv == 8)
    IO::to_f32(IO::load8(xr + t0), cur);
  else
    IO::to_f32(IO::load_n(xr + t0, nv), cur);
  float h0[3] = {0.0f, 0.0f, 0.0f};   // inputs at base-3 .. base-1
  if (lane == 0) {
    if (base > 0) {
#pragma unroll
      for (int i = 0; i < 3; ++i) h0[i] = IO::load1(xr + base - 3 + i);
    } else if (a.state_in) {
      const IoT* st = static_cast<const IoT*>(a.state_in) + row * (K - 1);
#pragma unroll
      for (int i = 3 - (K - 1); i < 3; ++i) h0[i] = IO::load1(st + (i - 3 + (K - 1)));
    }
  }

  // xx[0..2]: inputs at t0-3 .. t0-1 (the last three of the lane below),
  // xx[3..10]: inputs at t0 .. t0+7
  float xx[11];
#pragma unroll
  for (int i = 0; i < 8; ++i) xx[3 + i] = cur[i];
  const int src = (lane + 63) & 63;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const float v = __shfl(xx[8 + i], src);
    xx[i] = lane == 0 ? h0[i] : v;
  }
  if (nv == 0) return;
  constexpr int kb = 4 - K;   // xx index of tap 0 for output i = 0

  float out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float acc = bi;
#pragma unroll
    for (int k = 0; k < K; ++k) acc = fmaf(wk[k], xx[kb + i + k], acc);   // input time t0 + i - (K-1) + k
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
  a.nseg = (c.seqlen + kSeg - 1) / kSeg;
  if (c.seqlen > 0) {
    const uintptr_t mis = reinterpret_cast<uintptr_t>(c.x) | reinterpret_cast<uintptr_t>(c.u);
    const bool vec = ((mis & 15) == 0) && ((c.seqlen * (int64_t)sizeof(IoT)) % 16 == 0);
    int dev = 0, maxy = 65535, maxz = 65535;
    if (hipGetDevice(&dev) == hipSuccess) {
      (void)hipDeviceGetAttribute(&maxy, hipDeviceAttributeMaxGridDimY, dev);
      (void)hipDeviceGetAttribute(&maxz, hipDeviceAttributeMaxGridDimZ, dev);
    }
    const int wpb = (int)std::min<int64_t>(4, a.nseg);   // waves per workgroup
    const unsigned gx = (unsigned)((a.nseg + wpb - 1) / wpb);
    for (int64_t b0 = 0; b0 < c.batch; b0 += maxz) {
      for (int64_t d0 = 0; d0 < c.dim; d0 += maxy) {
        a.b0 = b0;
        a.d0 = d0;
        const dim3 grid(gx, (unsigned)std::min<int64_t>(maxy, c.dim - d0), (unsigned)std::min<int64_t>(maxz, c.batch - b0));
        switch ((int)c.K) {
#define MSCAN_CONV_LAUNCH(KK)                                                          \
  case KK:                                                                             \
    if (vec)                                                                           \
      hipLaunchKernelGGL((conv1d_kernel<IoT, true, KK>), grid, dim3(64 * wpb), 0, s, a); \
    else                                                                               \
      hipLaunchKernelGGL((conv1d_kernel<IoT, false, KK>), grid, dim3(64 * wpb), 0, s, a);\
    break;
          MSCAN_CONV_LAUNCH(1)
          MSCAN_CONV_LAUNCH(2)
          MSCAN_CONV_LAUNCH(3)
          MSCAN_CONV_LAUNCH(4)
#undef MSCAN_CONV_LAUNCH
          default:
            return hipErrorInvalidValue;
        }
      }
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

template <typename IoT>
hipError_t run_conv_state(const ConvArgs& c, hipStream_t s) {
  if (!c.state_out || c.K <= 1) return hipSuccess;
  CArgs a{};
  a.x = c.x; a.state_in = c.state_in; a.state_out = c.state_out;
  a.rows = c.batch * c.dim; a.seqlen = c.seqlen; a.dim = c.dim; a.K = (int)c.K;
  hipLaunchKernelGGL(conv_state_kernel<IoT>, dim3((unsigned)((a.rows + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
  return a.io_bf16 ? run_conv<uint16_t>(a, stream) : run_conv<float>(a, stream);
}

hipError_t launch_conv_state(const ConvArgs& a, hipStream_t stream) {
  return a.io_bf16 ? run_conv_state<uint16_t>(a, stream) : run_conv_state<float>(a, stream);
}

}  // namespace mscan
