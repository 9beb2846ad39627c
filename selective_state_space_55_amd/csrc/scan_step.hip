// scan_step.hip -- single-token recurrent update (O(1) decoding) on gfx950.
//
// One iteration of the forward recurrence applied to a caller-held fp32
// state (State space models and Mamba, jonathanding.github.io, §3, recurrence
// mode; Mamba notes, awesome.papernotes.org, 设计 2: a fixed (d, N) state
// instead of a KV cache).  The step is a pure stream over the state: it reads
// and writes 2 * N * 4 bytes per (batch, channel) and a handful of bf16/fp32
// scalars, so the kernel is laid out for coalesced 16-byte state traffic:
// LPC lanes own one channel (4, 8 or 16 for up to 16, 32 or 64 states), lane
// q holding states 4q .. 4q+3 as one float4; consecutive lane groups cover
// consecutive channels, so a wave moves 1 KB of contiguous state per access.  Each thread walks kRows batch rows of its
// channel, so A = -exp(A_log) and 1/A are formed once per channel and reused,
// and all rows' loads are issued before the arithmetic.  The readout sum over
// a channel's lanes uses cross-lane adds in a fixed order, so results are
// deterministic.  For d_state 16 (the common case) a variant lets lane q of
// a channel's quad do the per-(batch, channel) scalar work of row q once.
// The update is the forward scan's: h = h + m (h + B u / A) with the decay
// decrement m = Abar - 1 formed accurately for small Delta |A| (decay_m1).
#include "internal.h"
#include "io.h"

namespace mscan {
namespace {

constexpr int kRows = 4;   // batch rows per thread

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
  int dstate, softplus, euler;
};

// B or C values of states 4q .. 4q+3 of batch row b (zero past dstate)
template <typename IoT, bool kVec>
__device__ __forceinline__ void load_bc4(const IoT* p, int64_t b, int q, int dstate, float (&f)[4]) {
  using IO = Io<IoT>;
  const IoT* r = p + b * dstate + 4 * q;
  if constexpr (kVec) {
    if constexpr (sizeof(IoT) == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(r);
      f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    } else {
      const float4 v = *reinterpret_cast<const float4*>(r);
      f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = (4 * q + j < dstate) ? IO::load1(r + j) : 0.0f;
  }
}

// kVec: dstate == 4 * LPC and the state, B and C rows are vector aligned
template <typename IoT, bool kVec, int LPC>
__global__ __launch_bounds__(256) void scan_step_kernel(SArgs a) {
  using IO = Io<IoT>;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t dq = gid / LPC;          // channel
  const int q = (int)(gid % LPC);
  const bool live_d = dq < a.dim;        // whole lane groups share the channel
  const int64_t d = live_d ? dq : 0;
  const int64_t b0 = (int64_t)blockIdx.y * kRows;

  const IoT* gx = static_cast<const IoT*>(a.x);
  const IoT* gdt = static_cast<const IoT*>(a.dt);
  const IoT* gz = static_cast<const IoT*>(a.z);
  const IoT* gB = static_cast<const IoT*>(a.B);
  const IoT* gC = static_cast<const IoT*>(a.C);

  // per-channel constants, shared by the thread's batch rows
  float An[4], iA[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * q + j;
    const bool ok = n < a.dstate;
    An[j] = ok ? -expf(a.A_log[d * a.dstate + n]) : 0.0f;
    iA[j] = ok ? 1.0f / An[j] : 0.0f;
  }
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const float Dd = a.D ? a.D[d] : 0.0f;

  // all loads of the thread's rows first
  float xv[kRows], xr[kRows], zv[kRows], Bv[kRows][4], Cv[kRows][4], hs[kRows][4];
  bool live[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t b = b0 + r;
    live[r] = live_d && b < a.batch;
    const int64_t bc = live[r] ? b : 0;
    const int64_t bd = bc * a.dim + d;
    xv[r] = live[r] ? IO::load1(gx + bd) : 0.0f;
    xr[r] = live[r] ? IO::load1(gdt + bd) : 0.0f;
    zv[r] = (live[r] && gz) ? IO::load1(gz + bd) : 0.0f;
    load_bc4<IoT, kVec>(gB, bc, q, a.dstate, Bv[r]);
    load_bc4<IoT, kVec>(gC, bc, q, a.dstate, Cv[r]);
    const float* st = a.state + bd * a.dstate + 4 * q;
    if constexpr (kVec) {
      const float4 v = live[r] ? *reinterpret_cast<const float4*>(st) : make_float4(0, 0, 0, 0);
      hs[r][0] = v.x; hs[r][1] = v.y; hs[r][2] = v.z; hs[r][3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) hs[r][j] = (live[r] && 4 * q + j < a.dstate) ? st[j] : 0.0f;
    }
  }

#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const float x = xr[r] + bias;
    const float dl = a.softplus ? softplus_log2e(x) : x * 1.4426950408889634f;   // Delta * log2e
    float acc = 0.0f;
    if (a.euler) {
      const float du = (dl * 0.6931471805599453f) * xv[r];   // Delta u
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float yv = dl * An[j];
        const float m = decay_m1<true>(yv, __builtin_amdgcn_exp2f(yv));
        hs[r][j] += fmaf(m, hs[r][j], Bv[r][j] * du);   // h + (m h + Delta B u)
        acc = fmaf(Cv[r][j], hs[r][j], acc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float yv = dl * An[j];
        const float m = decay_m1<true>(yv, __builtin_amdgcn_exp2f(yv));
        const float s = Bv[r][j] * (xv[r] * iA[j]);   // B u / A (zero for states past dstate)
        hs[r][j] = fmaf(m, hs[r][j] + s, hs[r][j]);    // h + m (h + s)
        acc = fmaf(Cv[r][j], hs[r][j], acc);
      }
    }
    // sum over the channel's lanes: pairs, then pairs of pairs, ...
#pragma unroll
    for (int m = 1; m < LPC; m <<= 1) acc += __shfl_xor(acc, m, LPC);
    if (!live[r]) continue;
    const int64_t bd = (b0 + r) * a.dim + d;
    float* st = a.state + bd * a.dstate + 4 * q;
    if constexpr (kVec) {
      *reinterpret_cast<float4*>(st) = make_float4(hs[r][0], hs[r][1], hs[r][2], hs[r][3]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * q + j < a.dstate) st[j] = hs[r][j];
    }
    if (q == 0) {
      float yv = fmaf(Dd, xv[r], acc);
      if (gz) yv *= silu(zv[r]);
      IO::store1(static_cast<IoT*>(a.y) + bd, yv);
    }
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// value of lane R of the lane's quad (DPP quad_perm [R, R, R, R])
template <int R>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), R * 0x55, 0xf, 0xf, false));
}
// value of lane l ^ 1 (CTRL 0xB1) or l ^ 2 (CTRL 0x4E) of the quad
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// d_state 16 with vector-aligned rows: the quad of lanes of a channel walks
// four batch rows, and lane q does the per-(batch, channel) work of row q --
// loads of x, dt, z, softplus, the gate and the output -- once for the quad
// (the general kernel repeats it on every lane); Delta and x of row r reach
// the other lanes by a DPP broadcast.  Same arithmetic in the same order as
// the general kernel, so the results are identical.  Offsets are 32-bit from
// per-workgroup base addresses (4 rows x dim x 64 bytes < 4 GiB, checked on
// the host).  kFull: batch % 4 == 0 and 4 dim % 256 == 0, so no lane is idle.
template <typename IoT, bool kFull, bool kEuler>
__global__ __launch_bounds__(256) void scan_step_quad_kernel(SArgs a) {
  using IO = Io<IoT>;
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  const uint32_t dq = gid >> 2;
  const int q = (int)(gid & 3);
  const uint32_t dim = (uint32_t)a.dim;
  const bool live_d = kFull || dq < dim;
  const uint32_t d = live_d ? dq : 0u;
  const int64_t b0 = (int64_t)blockIdx.y * 4;

  const IoT* gx = static_cast<const IoT*>(a.x) + b0 * a.dim;
  const IoT* gdt = static_cast<const IoT*>(a.dt) + b0 * a.dim;
  const IoT* gz = a.z ? static_cast<const IoT*>(a.z) + b0 * a.dim : nullptr;
  const IoT* gB = static_cast<const IoT*>(a.B) + b0 * 16;
  const IoT* gC = static_cast<const IoT*>(a.C) + b0 * 16;
  float* gst = a.state + b0 * a.dim * 16;
  IoT* gy = static_cast<IoT*>(a.y) + b0 * a.dim;

  // row q's scalars
  const bool live_q = kFull || (live_d && b0 + q < a.batch);
  const uint32_t oq = live_q ? (uint32_t)q * dim + d : 0u;
  const float xq = live_q ? IO::load1(gx + oq) : 0.0f;
  const float rq = live_q ? IO::load1(gdt + oq) : 0.0f;
  const float zq = (live_q && gz) ? IO::load1(gz + oq) : 0.0f;

  // every row's B, C and states 4q .. 4q+3
  float Bv[4][4], Cv[4][4], hs[4][4];
  bool live[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    live[r] = kFull || (live_d && b0 + r < a.batch);
    const uint32_t rr = live[r] ? (uint32_t)r : 0u;
    load_bc4<IoT, true>(gB, rr, q, 16, Bv[r]);
    load_bc4<IoT, true>(gC, rr, q, 16, Cv[r]);
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live[r]) v = *reinterpret_cast<const f32x4*>(gst + (rr * dim + d) * 16u + 4u * q);
    hs[r][0] = v.x; hs[r][1] = v.y; hs[r][2] = v.z; hs[r][3] = v.w;
  }
  float An[4], iA[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    An[j] = -expf(a.A_log[d * 16u + 4u * q + j]);
    iA[j] = 1.0f / An[j];
  }
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const float Dd = a.D ? a.D[d] : 0.0f;
  const float xb = rq + bias;
  const float dlq = a.softplus ? softplus_log2e(xb) : xb * 1.4426950408889634f;   // Delta * log2e of row q
  const float gq = gz ? silu(zq) : 1.0f;

  static_for<4>([&](auto r_c) {
    constexpr int r = decltype(r_c)::value;
    const float dl = quad_bcast<r>(dlq);
    const float xv = quad_bcast<r>(xq);
    float acc = 0.0f;
    if constexpr (kEuler) {
      const float du = (dl * 0.6931471805599453f) * xv;   // Delta u
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float yv = dl * An[j];
        const float m = decay_m1<true>(yv, __builtin_amdgcn_exp2f(yv));
        hs[r][j] += fmaf(m, hs[r][j], Bv[r][j] * du);   // h + (m h + Delta B u)
        acc = fmaf(Cv[r][j], hs[r][j], acc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float yv = dl * An[j];
        const float m = decay_m1<true>(yv, __builtin_amdgcn_exp2f(yv));
        const float s = Bv[r][j] * (xv * iA[j]);   // B u / A
        hs[r][j] = fmaf(m, hs[r][j] + s, hs[r][j]);    // h + m (h + s)
        acc = fmaf(Cv[r][j], hs[r][j], acc);
      }
    }
    acc += quad_swap<0xB1>(acc);   // pairs, then pairs of pairs, as the general kernel
    acc += quad_swap<0x4E>(acc);
    if (live[r]) {
      const f32x4 v = {hs[r][0], hs[r][1], hs[r][2], hs[r][3]};
      *reinterpret_cast<f32x4*>(gst + ((uint32_t)r * dim + d) * 16u + 4u * q) = v;
      if (q == r) IO::store1(gy + oq, fmaf(Dd, xq, acc) * gq);
    }
  });
}

// The same idea for d_state 32 and 64 (LPC = 8 or 16 lanes per channel, dstate
// = 4 LPC, vector-aligned rows): lanes q < 4 of a channel's group do row q's
// scalar work, and Delta and x of row r reach the group's other lanes by a
// cross-lane read.  Identical results to the general kernel.
template <typename IoT, int LPC, bool kFull, bool kEuler>
__global__ __launch_bounds__(256) void scan_step_rows_kernel(SArgs a) {
  using IO = Io<IoT>;
  static_assert(LPC == 8 || LPC == 16, "lanes per channel");
  constexpr uint32_t N = 4 * LPC;
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  const uint32_t dq = gid / LPC;
  const int q = (int)(gid % LPC);
  const int lane = (int)(threadIdx.x & 63);
  const int gbase = lane & ~(LPC - 1);   // first lane of the channel's group
  const uint32_t dim = (uint32_t)a.dim;
  const bool live_d = kFull || dq < dim;
  const uint32_t d = live_d ? dq : 0u;
  const int64_t b0 = (int64_t)blockIdx.y * 4;

  const IoT* gx = static_cast<const IoT*>(a.x) + b0 * a.dim;
  const IoT* gdt = static_cast<const IoT*>(a.dt) + b0 * a.dim;
  const IoT* gz = a.z ? static_cast<const IoT*>(a.z) + b0 * a.dim : nullptr;
  const IoT* gB = static_cast<const IoT*>(a.B) + b0 * N;
  const IoT* gC = static_cast<const IoT*>(a.C) + b0 * N;
  float* gst = a.state + b0 * a.dim * N;
  IoT* gy = static_cast<IoT*>(a.y) + b0 * a.dim;

  // lanes 0-3 of the group: row q's scalars
  const bool own = q < 4;
  const bool live_q = own && (kFull || (live_d && b0 + q < a.batch));
  const uint32_t oq = live_q ? (uint32_t)q * dim + d : 0u;
  const float xq = live_q ? IO::load1(gx + oq) : 0.0f;
  const float rq = live_q ? IO::load1(gdt + oq) : 0.0f;
  const float zq = (live_q && gz) ? IO::load1(gz + oq) : 0.0f;

  float Bv[4][4], Cv[4][4], hs[4][4];
  bool live[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    live[r] = kFull || (live_d && b0 + r < a.batch);
    const uint32_t rr = live[r] ? (uint32_t)r : 0u;
    load_bc4<IoT, true>(gB, rr, q, N, Bv[r]);
    load_bc4<IoT, true>(gC, rr, q, N, Cv[r]);
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live[r]) v = *reinterpret_cast<const f32x4*>(gst + (rr * dim + d) * N + 4u * q);
    hs[r][0] = v.x; hs[r][1] = v.y; hs[r][2] = v.z; hs[r][3] = v.w;
  }
  float An[4], iA[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    An[j] = -expf(a.A_log[d * N + 4u * q + j]);
    iA[j] = 1.0f / An[j];
  }
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const float Dd = a.D ? a.D[d] : 0.0f;
  const float xb = rq + bias;
  const float dlq = a.softplus ? softplus_log2e(xb) : xb * 1.4426950408889634f;   // Delta * log2e of row q
  const float gq = gz ? silu(zq) : 1.0f;

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float dl = __shfl(dlq, gbase + r);
    const float xv = __shfl(xq, gbase + r);
    float acc = 0.0f;
    if constexpr (kEuler) {
      const float du = (dl * 0.6931471805599453f) * xv;   // Delta u
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float yv = dl * An[j];
        const float m = decay_m1<true>(yv, __builtin_amdgcn_exp2f(yv));
        hs[r][j] += fmaf(m, hs[r][j], Bv[r][j] * du);   // h + (m h + Delta B u)
        acc = fmaf(Cv[r][j], hs[r][j], acc);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float yv = dl * An[j];
        const float m = decay_m1<true>(yv, __builtin_amdgcn_exp2f(yv));
        const float s = Bv[r][j] * (xv * iA[j]);   // B u / A
        hs[r][j] = fmaf(m, hs[r][j] + s, hs[r][j]);    // h + m (h + s)
        acc = fmaf(Cv[r][j], hs[r][j], acc);
      }
    }
#pragma unroll
    for (int m = 1; m < LPC; m <<= 1) acc += __shfl_xor(acc, m, LPC);   // as the general kernel
    if (live[r]) {
      const f32x4 v = {hs[r][0], hs[r][1], hs[r][2], hs[r][3]};
      *reinterpret_cast<f32x4*>(gst + ((uint32_t)r * dim + d) * N + 4u * q) = v;
      if (q == r) IO::store1(gy + oq, fmaf(Dd, xq, acc) * gq);
    }
  }
}

template <typename IoT>
hipError_t run_step(const StepArgs& s, hipStream_t stream) {
  SArgs a{};
  a.state = s.state; a.x = s.x; a.dt = s.dt; a.A_log = s.A_log; a.B = s.B; a.C = s.C; a.D = s.D; a.z = s.z;
  a.bias = s.bias; a.y = s.y; a.batch = s.batch; a.dim = s.dim; a.dstate = (int)s.dstate;
  a.softplus = s.softplus;
  a.euler = s.euler;
  const uintptr_t bc_mis = reinterpret_cast<uintptr_t>(s.B) | reinterpret_cast<uintptr_t>(s.C);
  const int lpc = s.dstate <= 16 ? 4 : (s.dstate <= 32 ? 8 : 16);   // lanes per channel
  const bool vec = (s.dstate == 4 * lpc) && ((reinterpret_cast<uintptr_t>(s.state) & 15) == 0) &&
                   ((bc_mis & (4 * sizeof(IoT) - 1)) == 0);
  const int64_t threads = s.dim * lpc;
  if (vec && lpc == 4 && s.dim < (int64_t(1) << 26)) {
    const dim3 g4((unsigned)((threads + 255) / 256), (unsigned)((s.batch + 3) / 4));
    const bool full = (s.batch % 4 == 0) && (threads % 256 == 0);
    auto k = full ? (s.euler ? scan_step_quad_kernel<IoT, true, true> : scan_step_quad_kernel<IoT, true, false>)
                  : (s.euler ? scan_step_quad_kernel<IoT, false, true> : scan_step_quad_kernel<IoT, false, false>);
    hipLaunchKernelGGL(k, g4, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (vec && lpc > 4 && s.dim * s.dstate < (int64_t(1) << 27)) {
    const dim3 g4((unsigned)((threads + 255) / 256), (unsigned)((s.batch + 3) / 4));
    const bool full = (s.batch % 4 == 0) && (threads % 256 == 0);
#define MSCAN_STEP_ROWS(L)                                                                               \
    {                                                                                                    \
      auto k = full ? (s.euler ? scan_step_rows_kernel<IoT, L, true, true> : scan_step_rows_kernel<IoT, L, true, false>) \
                    : (s.euler ? scan_step_rows_kernel<IoT, L, false, true> : scan_step_rows_kernel<IoT, L, false, false>); \
      hipLaunchKernelGGL(k, g4, dim3(256), 0, stream, a);                                               \
    }
    if (lpc == 8) MSCAN_STEP_ROWS(8) else MSCAN_STEP_ROWS(16)
#undef MSCAN_STEP_ROWS
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)((s.batch + kRows - 1) / kRows));
  switch (lpc * 2 + (vec ? 1 : 0)) {
    case 9: hipLaunchKernelGGL((scan_step_kernel<IoT, true, 4>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((scan_step_kernel<IoT, false, 4>), grid, dim3(256), 0, stream, a); break;
    case 17: hipLaunchKernelGGL((scan_step_kernel<IoT, true, 8>), grid, dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((scan_step_kernel<IoT, false, 8>), grid, dim3(256), 0, stream, a); break;
    case 33: hipLaunchKernelGGL((scan_step_kernel<IoT, true, 16>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((scan_step_kernel<IoT, false, 16>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  return a.io_bf16 ? run_step<uint16_t>(a, stream) : run_step<float>(a, stream);
}

}  // namespace mscan
