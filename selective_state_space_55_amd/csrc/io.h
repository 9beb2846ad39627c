// io.h -- device-side element access for float32 and bfloat16 tensors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bfloat16 storage is handled as raw uint16_t bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bfloat16 (round to nearest even) packed low|high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return
// zero (hardware range check).  Third dword 0x00020000: 32-bit data format,
// the value used for the gfx9 family.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const T* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, bytes, 0x00020000);
}

template <typename IoT>
struct Io;

// Eight consecutive elements, as raw storage.
template <>
struct Io<uint16_t> {
  struct V8 {
    uint4 w;
  };
  static __device__ __forceinline__ V8 zero() { return V8{make_uint4(0, 0, 0, 0)}; }
  static __device__ __forceinline__ V8 load8(const uint16_t* p) { return V8{*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ V8 load_n(const uint16_t* p, int n) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (j < n) ? p[j] : (uint16_t)0;
    V8 v;
    v.w.x = e[0] | ((uint32_t)e[1] << 16);
    v.w.y = e[2] | ((uint32_t)e[3] << 16);
    v.w.z = e[4] | ((uint32_t)e[5] << 16);
    v.w.w = e[6] | ((uint32_t)e[7] << 16);
    return v;
  }
  static __device__ __forceinline__ void to_f32(const V8& v, float (&f)[8]) {
    f[0] = bf16_lo(v.w.x); f[1] = bf16_hi(v.w.x);
    f[2] = bf16_lo(v.w.y); f[3] = bf16_hi(v.w.y);
    f[4] = bf16_lo(v.w.z); f[5] = bf16_hi(v.w.z);
    f[6] = bf16_lo(v.w.w); f[7] = bf16_hi(v.w.w);
  }
  static __device__ __forceinline__ V8 from_f32(const float (&f)[8]) {
    V8 v;
    v.w.x = pack_bf16x2(f[0], f[1]);
    v.w.y = pack_bf16x2(f[2], f[3]);
    v.w.z = pack_bf16x2(f[4], f[5]);
    v.w.w = pack_bf16x2(f[6], f[7]);
    return v;
  }
  static __device__ __forceinline__ void store8(uint16_t* p, const V8& v) { *reinterpret_cast<uint4*>(p) = v.w; }
  // 8 elements at byte offset off; stores past the descriptor are dropped.
  static __device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, const V8& v, bool vec) {
    if (vec) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v.w),
                                             r, off, 0, 0);
      return;
    }
    const uint32_t w[4] = {v.w.x, v.w.y, v.w.z, v.w.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu)), r,
                                            off + 2 * j, 0, 0);
  }
  static __device__ __forceinline__ void store_n(uint16_t* p, const V8& v, int n) {
    const uint32_t w[4] = {v.w.x, v.w.y, v.w.z, v.w.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < n) p[j] = (uint16_t)((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu));
  }
  // 8 elements at byte offset off: one 16-byte load when rows are 16-byte
  // aligned, else 8 element loads; bytes past the descriptor read as zero.
  static __device__ __forceinline__ V8 buf_load8(__amdgpu_buffer_rsrc_t r, int off, int vec) {
    if (vec) return V8{__builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0))};
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * j, 0, 0);
    return V8{make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16))};
  }
  // Four consecutive elements.
  struct V4 {
    uint2 w;
  };
  static __device__ __forceinline__ V4 buf_load4(__amdgpu_buffer_rsrc_t r, int off, int vec) {
    if (vec) return V4{__builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0))};
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * j, 0, 0);
    return V4{make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16))};
  }
  static __device__ __forceinline__ void to_f32(const V4& v, float (&f)[4]) {
    f[0] = bf16_lo(v.w.x); f[1] = bf16_hi(v.w.x);
    f[2] = bf16_lo(v.w.y); f[3] = bf16_hi(v.w.y);
  }
  static __device__ __forceinline__ V4 from_f32(const float (&f)[4]) {
    return V4{make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]))};
  }
  // 4 elements at byte offset off; stores past the descriptor are dropped.
  static __device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, int off, const V4& v, bool vec) {
    if (vec) {
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v.w),
                                            r, off, 0, 0);
      return;
    }
    const uint32_t w[2] = {v.w.x, v.w.y};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu)), r,
                                            off + 2 * j, 0, 0);
  }
  static __device__ __forceinline__ void store_n(uint16_t* p, const V4& v, int n) {
    const uint32_t w[2] = {v.w.x, v.w.y};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < n) p[j] = (uint16_t)((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu));
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
  static __device__ __forceinline__ void store1(uint16_t* p, float f) {
    *p = (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
  }
};

template <>
struct Io<float> {
  struct V8 {
    float4 a, b;
  };
  static __device__ __forceinline__ V8 zero() { return V8{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)}; }
  static __device__ __forceinline__ V8 load8(const float* p) {
    return V8{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  static __device__ __forceinline__ V8 load_n(const float* p, int n) {
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (j < n) ? p[j] : 0.0f;
    return V8{make_float4(e[0], e[1], e[2], e[3]), make_float4(e[4], e[5], e[6], e[7])};
  }
  static __device__ __forceinline__ void to_f32(const V8& v, float (&f)[8]) {
    f[0] = v.a.x; f[1] = v.a.y; f[2] = v.a.z; f[3] = v.a.w;
    f[4] = v.b.x; f[5] = v.b.y; f[6] = v.b.z; f[7] = v.b.w;
  }
  static __device__ __forceinline__ V8 from_f32(const float (&f)[8]) {
    return V8{make_float4(f[0], f[1], f[2], f[3]), make_float4(f[4], f[5], f[6], f[7])};
  }
  static __device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, const V8& v, bool vec) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    if (vec) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v.a), r, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v.b), r, off + 16, 0, 0);
      return;
    }
    const float e[8] = {v.a.x, v.a.y, v.a.z, v.a.w, v.b.x, v.b.y, v.b.z, v.b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, e[j]), r, off + 4 * j, 0, 0);
  }
  static __device__ __forceinline__ void store8(float* p, const V8& v) {
    reinterpret_cast<float4*>(p)[0] = v.a;
    reinterpret_cast<float4*>(p)[1] = v.b;
  }
  static __device__ __forceinline__ void store_n(float* p, const V8& v, int n) {
    const float e[8] = {v.a.x, v.a.y, v.a.z, v.a.w, v.b.x, v.b.y, v.b.z, v.b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < n) p[j] = e[j];
  }
  static __device__ __forceinline__ V8 buf_load8(__amdgpu_buffer_rsrc_t r, int off, int vec) {
    if (vec)
      return V8{__builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0)),
                __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0))};
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * j, 0, 0));
    return V8{make_float4(e[0], e[1], e[2], e[3]), make_float4(e[4], e[5], e[6], e[7])};
  }
  struct V4 {
    float4 a;
  };
  static __device__ __forceinline__ V4 buf_load4(__amdgpu_buffer_rsrc_t r, int off, int vec) {
    if (vec) return V4{__builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0))};
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * j, 0, 0));
    return V4{make_float4(e[0], e[1], e[2], e[3])};
  }
  static __device__ __forceinline__ void to_f32(const V4& v, float (&f)[4]) {
    f[0] = v.a.x; f[1] = v.a.y; f[2] = v.a.z; f[3] = v.a.w;
  }
  static __device__ __forceinline__ V4 from_f32(const float (&f)[4]) { return V4{make_float4(f[0], f[1], f[2], f[3])}; }
  static __device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, int off, const V4& v, bool vec) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    if (vec) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v.a), r, off, 0, 0);
      return;
    }
    const float e[4] = {v.a.x, v.a.y, v.a.z, v.a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, e[j]), r, off + 4 * j, 0, 0);
  }
  static __device__ __forceinline__ void store_n(float* p, const V4& v, int n) {
    const float e[4] = {v.a.x, v.a.y, v.a.z, v.a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < n) p[j] = e[j];
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float f) { *p = f; }
};

// softplus(x) * log2(e) = log2(1 + 2^(x*log2 e)), evaluated as
// max(x,0)*log2e + log2(1 + e), e = 2^(-|x| log2e); the rounding error of
// w = 1 + e is added back to first order so small e keeps full relative
// accuracy (log2(1+e) ~ log2(w) + (e - (w-1)) * log2e).
__device__ __forceinline__ float softplus_log2e(float x) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float r = e - (w - 1.0f);
  const float l = fmaf(r, kLog2e, __builtin_amdgcn_logf(w));
  return fmaf(fmaxf(x, 0.0f), kLog2e, l);
}

// The decrement of a decay, m = Abar - 1 = expm1(x) with x = y ln 2, from the
// base-2 exponent y = Delta A log2(e) and ab = 2^y (the hardware exp2).
// Abar - 1 alone carries exp2's absolute rounding error (a few 1e-8), which is
// a large relative error of m once |x| is small, and over the ~1/|x| steps a
// state remembers its input that error adds up (State space models and Mamba,
// jonathanding.github.io, §4: a small step keeps the state for a long time).
// For x <= 0 two upper bounds of expm1(x) are taken and the smaller kept:
//   x + x^2/2 (Taylor remainder x^3/6 e^xi < 0), relative error x^2/6;
//   ab - 1 + 2^-23 (exp2 within two units in the last place below 1).
// The smaller is within ~2e-5 relative of expm1(x) for every x <= 0, and is
// exactly 0 at x = 0 (Delta = 0 leaves the state unchanged).  For y <= 0 the
// minimum is taken as m0 - clamp(m0 - p2) with clamp to [0, 1] (m0 - p2 <= 1
// since p2 >= -1/2 and m0 <= 2^-23): the compiler folds p2 into that
// subtraction as one fma with the clamp modifier, and every instruction of
// the sequence is a plain two-VGPR-operand op, which gfx950 issues from two
// waves at about twice the rate of v_min_f32.  kAnySign: y may be positive
// (Delta without softplus); there x + x^2/2 is a lower bound, and the larger
// of it and ab - 1 - 2^-23 is taken.
constexpr float kDecayC1 = 0.6931471805599453f;            // ln 2
constexpr float kDecayC2 = 0.2402265069591007f;            // (ln 2)^2 / 2
constexpr float kDecayHi = 0.99999988079071044921875f;     // 1 - 2^-23
template <bool kAnySign>
__device__ __forceinline__ float decay_m1(float y, float ab) {
  const float p2 = y * fmaf(y, kDecayC2, kDecayC1);   // x + x^2 / 2
  const float m0 = ab - kDecayHi;                     // ab - (1 - 2^-23)
  if constexpr (!kAnySign) return m0 - __builtin_amdgcn_fmed3f(m0 - p2, 0.0f, 1.0f);   // min(m0, p2)
  return fmaxf(fminf(m0, p2), ab - 1.00000011920928955078125f);   // ab - (1 + 2^-23)
}

// decay_m1 of four tokens (Delta*log2e in dl) times two states (A in A), laid out
// for the issue order: the eight exp2 first, each of decay_m1's steps eight at a
// time (scheduling barriers keep the phases apart), so no instruction reads a
// result issued just before it -- a scan's h-independent work, formed before the
// recurrence meets it.
template <bool kAnySign>
__device__ __forceinline__ void decay_m1_4x2(const float (&dl)[4], const float (&A)[2], float (&m)[4][2]) {
  float y[4][2], ab[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 2; ++j) y[q][j] = dl[q] * A[j];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 2; ++j) ab[q][j] = __builtin_amdgcn_exp2f(y[q][j]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kAnySign) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j) m[q][j] = decay_m1<true>(y[q][j], ab[q][j]);
  } else {
    float p1[4][2], m0[4][2], t[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        p1[q][j] = fmaf(y[q][j], kDecayC2, kDecayC1);
        m0[q][j] = ab[q][j] - kDecayHi;
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j) t[q][j] = __builtin_amdgcn_fmed3f(m0[q][j] - y[q][j] * p1[q][j], 0.0f, 1.0f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j) m[q][j] = m0[q][j] - t[q][j];   // min(m0, p2), as in decay_m1
  }
}

// z * sigmoid(z) = z / (1 + 2^(-z log2e))
__device__ __forceinline__ float silu(float z) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Calls f(IntC<0>{}) .. f(IntC<N-1>{}) (compile-time loop index).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

// a * b and c + a * b where a is read from lane SRC of the same 16-lane row
// (DPP row_newbcast on the first source): a wave-wide broadcast of one of 16
// per-row values, folded into the arithmetic instruction.  The DPP source must
// not be written by a VALU instruction in the two preceding instructions; the
// callers pass registers loaded from LDS only.
template <int SRC>
__device__ __forceinline__ float dpp_bcast_mul(float a, float b) {
  static_assert(SRC >= 0 && SRC < 16, "row lane");
  float r;
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(a), "v"(b), "n"(SRC));
  return r;
}

template <int SRC>
__device__ __forceinline__ float dpp_bcast_fmac(float c, float a, float b) {
  static_assert(SRC >= 0 && SRC < 16, "row lane");
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(c) : "v"(a), "v"(b), "n"(SRC));
  return c;
}

// Sum of a value over lanes l and l ^ 32, for two values at once: lanes 0-31
// return a[l] + a[l+32], lanes 32-63 return b[l-32] + b[l]
// (v_permlane32_swap exchanges the upper half of a with the lower half of b).
__device__ __forceinline__ float half_sum2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Barrier for LDS producer/consumer hand-off only: orders LDS accesses, does
// not wait for outstanding global loads or stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Debug builds (-DMSCAN_LDS_POISON): a kernel fills its floating-point LDS
// arrays with all-ones words (NaN as fp32 and as bf16) before first use, and
// the SSD kernel refills its staging tiles before each chunk; a read of a word
// that no thread has written since then turns into NaN in the outputs (a
// missing barrier or an unwritten row).  Whole workgroup; ends at a barrier.
// In normal builds it is empty.
__device__ __forceinline__ void lds_poison(void* p, int bytes) {
#ifdef MSCAN_LDS_POISON
  __syncthreads();
  uint32_t* q = static_cast<uint32_t*>(p);
  for (int i = (int)threadIdx.x; i < bytes / 4; i += (int)blockDim.x) q[i] = 0xffffffffu;
  __syncthreads();
#else
  (void)p;
  (void)bytes;
#endif
}

}  // namespace mscan
