// ssd_fwd.hip -- multi-head SSM with a scalar decay per head (the
// state-space-duality form) on gfx950 matrix cores.
//
// Method (State space models and Mamba, jonathanding.github.io, §5): the P
// channels of a head share A, so the decay a_t = exp(Delta_t A_h) is one scalar
// per (batch, token, head); the sequence is cut into chunks of Q tokens; inside
// a chunk the output is a Q x Q masked matrix product (the dual,
// attention-like form with mask Lambda_ij = prod_{t=j+1..i} a_t), and only the
// N x P state crosses chunk boundaries.  Per chunk, with cum_i the running sum
// of log a_t inside the chunk and w_j the input weight ((a_j - 1)/A_h, or
// Delta_j for the Euler input term):
//
//   G      = B C^T                               (Q x Q, over N)
//   M_ij   = G_ji exp(cum_i - cum_j) w_j  (j <= i, else 0)
//   Y      = diag(exp(cum)) C S_in + M X + D X   (Q x P), times SiLU(z)
//   S_out  = exp(cum_Q) S_in + (B diag(exp(cum_Q - cum_j) w_j))^T X   (N x P)
//
// Mapping.  One workgroup owns one (batch, head, P-channel slice) and walks its
// chunks in order, keeping S (N x P, fp32) in MFMA accumulators -- nothing but
// x, dt, B, C, z in and y, the final state out touches HBM.  Q = 64, N = 64 or
// 128, P = 64 (head dims 64, 128, 192, 256) or 32 (head dims 32, 96, 160, 224).
// Every product is a 32x32x16 MFMA with bf16 operands and fp32 accumulation;
// the operand layouts (lane l holds 8 consecutive k) make each operand one
// 16-byte LDS read.  Wave roles, 8 waves (two per SIMD):
//   waves 0-2  the three causal 32 x 32 tiles of B C^T and the masked, decayed M
//   waves 4-7  the Y tiles (C S_in, M X) -- waves 4-5 at P = 32
//   waves 0-7  one 32 x 32 tile of S each (those that exist: 8 at (N, P) =
//              (128, 64), 2 to 4 otherwise)
//   wave 3     the decay terms (wave 7 at P = 32)
//   all        stage x (waves 0-3 at P = 32) and run the epilogue
// and at (N, P) = (128, 64) 16 waves, four per SIMD, so that one role's waits
// overlap another's work: waves 0-7 the S tiles, 8-11 the Y tiles, 12-14 B C^T
// and M, 15 the decay terms; all 16 stage x and run the epilogue, 4 channels
// of a token per thread.  Per chunk:
//   stage   -- x, B, C as loaded (token-major rows, coalesced 16-byte writes),
//              and x scaled by exp(cum_Q - cum_j) w_j as two bf16 parts (hi,
//              and bf16 of the rest); the chunk's decay terms were computed
//              during the previous chunk (one wave turns dt into log a
//              (softplus, A_h), w and a running sum over the chunk with a DPP
//              prefix scan, into the other of two buffers)
//   A2      -- B C^T -> M; the Y tiles' C S_in (S_in as bf16 hi + lo from
//              LDS), rows scaled by exp(cum_i); S = exp(cum_Q) S + B^T Xs over
//              both parts of the scaled x
//   A3      -- Y += M X, Y to LDS (token-major); S to LDS as hi + lo
//   epilogue -- y = Y + D x, SiLU(z) gate, one 16-byte store per thread
// At P = 32 a barrier ends each of the first three phases (three per chunk).
// At P = 64 (two x and two M tiles in LDS) chunk c's A3 moves into chunk c+1's
// A2 -- the Y waves first finish chunk c's Y with M X and store it -- and its
// epilogue into chunk c+1's last phase, so a chunk has two barriers; the decay
// terms of chunk c+1 are computed in chunk c's A2 from a dt loaded a chunk
// earlier.
// Operands whose k (token) index must be contiguous per lane -- x for M x, B
// and the scaled x for the state update -- are read straight from the
// token-major tiles with ds_read_b64_tr_b16 (gfx950's transposing LDS read:
// in each 16-lane group, lane 4a + c receives element c of the 4-element row
// pieces addressed by lanes a, a + 4, a + 8, a + 12), so nothing is transposed
// explicitly.  Chunk c+1's global loads are issued at the start of A2 of chunk c.
//
// Ranges: every operand is bf16 with fp32's exponent range; the hi + lo splits
// carry S and the scaled x to ~2^-17 relative.
#include "internal.h"
#include "io.h"

namespace mscan {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQ = 64;      // tokens per chunk
constexpr int kPadH = 8;    // LDS row padding, bf16 elements (keeps rows 16-byte aligned)

struct SArgs {
  const uint16_t* x;        // (batch, L, H, P) bf16
  const uint16_t* dt;       // (batch, L, H)
  const float* A_log;       // (H)
  const uint16_t* B;        // (batch, L, N)
  const uint16_t* C;        // (batch, L, N)
  const float* D;           // (H) or null
  const uint16_t* z;        // (batch, L, H, P) or null
  const float* dt_bias;     // (H) or null
  const float* h0;          // (batch, H, P, N) or null
  float* hT;                // (batch, H, P, N) or null
  uint16_t* y;              // (batch, L, H, P)
  int64_t L;
  int H, S, softplus, euler;   // S: P-channel slices per head (head dim P S)
};

template <int N, int P>
struct SsdLds {
  static constexpr int kRowQ = kQ + kPadH;    // rows over Q tokens
  static constexpr int kRowN = N + kPadH;     // rows over N states
  // B's rows take 16 elements of padding: its transposing reads take 32 bytes
  // from each of 4 consecutive rows, which a 288-byte pitch puts in distinct banks
  static constexpr int kRowNB = N + 2 * kPadH;
  // rows over P channels (the x tile and the scaled x); their transposing reads
  // take 64 bytes from each of 4 consecutive rows, which a pitch of 192 bytes at
  // P = 64 puts in distinct banks (144 bytes overlapped rows r and r + 2)
  static constexpr int kRowP = P == 64 ? P + 4 * kPadH : P + kPadH;
  static constexpr int kXtm = kQ * kRowP;     // x     [j][p]
  static constexpr int kCs = kQ * kRowN;      // C     [i][n]
  static constexpr int kBs = kQ * kRowNB;     // B     [j][n]
  static constexpr int kXs = kQ * kRowP;      // scaled x [j][p], twice: bf16 and bf16 of the rest
  static constexpr int kMs = kQ * kRowQ;      // M     [i][j]
  static constexpr int kST = P * kRowN;      // S^T   [p][n], twice: bf16 S and bf16 (S - that)
  // P = 64 keeps two x tiles and two M tiles: chunk c's M X runs in chunk c+1's
  // second phase (one barrier fewer per chunk)
  static constexpr int kBuf = P == 64 ? 2 : 1;
  static constexpr int kHalves = kBuf * kXtm + kCs + kBs + 2 * kXs + kBuf * kMs + 2 * kST;
  // Y fp32 [i][p]; at P = 64 a 288-byte pitch puts the two half-waves' rows (4
  // apart) in disjoint banks
  static constexpr int kYRow = P == 64 ? P + 8 : P + 4;
  // At P = 32 the fp32 Y tile takes the M tile's place (the same 144-byte rows):
  // a Y wave writes only the rows of M it has just multiplied, and M is next
  // written after the following stage barrier.  This keeps two workgroups per CU.
  static constexpr bool kYinM = P == 32;
  static_assert(!kYinM || (kYRow * 4 == kRowQ * 2 && kBuf == 1), "Y rows must match M rows");
  static constexpr int kFloats = (kYinM ? 0 : kQ * kYRow) + 2 * (4 * kQ + 4);   // Y, then two sets of decay terms
  static constexpr size_t bytes() { return 2 * (size_t)kHalves + 4 * (size_t)kFloats; }
};

__device__ __forceinline__ bf16x8 lds_b8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


__device__ __forceinline__ float bf(uint32_t h16) { return __uint_as_float(h16 << 16); }

// exp(x) - 1 without cancellation for small |x| (Taylor to x^3 below 1e-2)
__device__ __forceinline__ float expm1_f(float x) {
  if (fabsf(x) < 1e-2f) return x * (1.0f + x * (0.5f + x * (1.0f / 6.0f)));
  return __expf(x) - 1.0f;
}

// v from another lane (DPP move; lanes with no source get 0)
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add_src(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, true));
}

// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then row 0's total into row 1, rows 0-1's into rows 2-3, etc.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_add_src<0x111, 0xf>(v);   // row_shr:1
  v += dpp_add_src<0x112, 0xf>(v);   // row_shr:2
  v += dpp_add_src<0x114, 0xf>(v);   // row_shr:4
  v += dpp_add_src<0x118, 0xf>(v);   // row_shr:8
  v += dpp_add_src<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_add_src<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Operand of a 32x32x16 MFMA whose k index runs along the rows of a row-major
// bf16 tile: lane l gets rows k0 + 8 (l / 32) .. + 7 of column n0 + l % 32.
// Two transposing reads of 4 rows each; in 16-lane group g the lane
// m = a + 4 kk addresses row k0 + 8 (g / 2) + kk, columns n0 + 16 (g % 2) + 4 a .. + 3.
__device__ __forceinline__ bf16x8 lds_opnd_tr(const uint16_t* base, int stride, int k0, int n0, int lane) {
  const int g = lane >> 4, m = lane & 15;
  const uint16_t* p = base + (k0 + 8 * (g >> 1) + (m >> 2)) * stride + n0 + 16 * (g & 1) + 4 * (m & 3);
  const uint2 lo = lds_tr16(p);
  const uint2 hi = lds_tr16(p + 4 * stride);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// NW: waves per workgroup, 8 or (at N = 128, P = 64) 16, with the roles above.
template <int N, int P, int NW>
__global__ __launch_bounds__(NW * 64, P == 32 ? 4 : 1) void ssd_fwd_kernel(SArgs a) {
  using L = SsdLds<N, P>;
  constexpr int kNT = NW * 64;   // threads per workgroup
  constexpr bool kW16 = NW == 16;
  static_assert(NW == 8 || (kW16 && P == 64 && N == 128), "16 waves only at P = 64, N = 128");
  constexpr int kRowQ = L::kRowQ, kRowN = L::kRowN, kRowNB = L::kRowNB, kRowP = L::kRowP, kYRow = L::kYRow;
  extern __shared__ __align__(16) uint16_t sm[];
  uint16_t* Xtm = sm;
  uint16_t* Cs = Xtm + L::kBuf * L::kXtm;
  uint16_t* Bs = Cs + L::kCs;
  uint16_t* Xs = Bs + L::kBs;     // x exp(cum_Q - cum_j) w_j: bf16 part
  uint16_t* XsLo = Xs + L::kXs;   // and bf16 of what that leaves
  uint16_t* Ms = XsLo + L::kXs;
  uint16_t* ST = Ms + L::kBuf * L::kMs;
  uint16_t* STlo = ST + L::kST;
  float* Yf = L::kYinM ? reinterpret_cast<float*>(Ms) : reinterpret_cast<float*>(STlo + L::kST);   // [i][p]
  // decay terms of a chunk, double-buffered (chunk c uses set c & 1, while one wave
  // computes chunk c+1's into the other set): [set][cum | ecum | scl | wv | atot]
  float* dterms = L::kYinM ? reinterpret_cast<float*>(STlo + L::kST) : Yf + kQ * kYRow;
  lds_poison(sm, (int)L::bytes());
  constexpr int kDSet = 4 * kQ + 4;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int H = a.H;
  const int HS = H * a.S;   // (head, P-channel slice) items per batch row
  // A head of dim P S is S independent slices of P channels sharing the
  // head's decay, B and C; a workgroup owns one slice.  XCD-aware placement:
  // workgroup ids are dealt round-robin over the 8 XCDs; give each XCD a
  // contiguous range of (batch, head, slice) items, so the heads of a batch row
  // (which all read the same B and C) share an L2
  const int64_t nwg = gridDim.x;
  const int64_t bh = (nwg & 7) == 0 ? (int64_t)(blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int64_t b = bh / HS;
  const int hs = (int)(bh % HS);
  const int h = hs / a.S;
  const int64_t Lq = a.L;
  const int64_t nchunk = (Lq + kQ - 1) / kQ;

  const int64_t xs_t = (int64_t)HS * P;   // x/z/y token stride (H heads of dim P S)
  const uint16_t* xb = a.x + b * Lq * xs_t + (int64_t)hs * P;
  const uint16_t* zb = a.z ? a.z + b * Lq * xs_t + (int64_t)hs * P : nullptr;
  uint16_t* yb = a.y + b * Lq * xs_t + (int64_t)hs * P;
  const uint16_t* Bb = a.B + b * Lq * N;
  const uint16_t* Cb = a.C + b * Lq * N;
  const uint16_t* dtb = a.dt + b * Lq * H + h;

  const float Ah = -__expf(a.A_log[h]);
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;

  // x / z / y piece of this thread: token xj, channels xp8 .. xp8 + kXC - 1 (kXC = 8:
  // the first kQ P / 8 threads, all 8 waves at P = 64, waves 0-3 at P = 32; with 16
  // waves kXC = 4, all of them, so staging and epilogue work is spread over every
  // wave).  A piece is held as a uint4 whose first kXC / 2 words are used.
  constexpr int kXC = kW16 ? 4 : 8;
  constexpr int kXW = kXC / 2;
  constexpr int kXT = kQ * P / kXC;
  const bool has_x = kXT == kNT || tid < kXT;   // uniform per wave
  const int xt = kXT == kNT ? tid : tid % kXT;
  const int xj = xt / (P / kXC), xp8 = (xt % (P / kXC)) * kXC;
  // B / C pieces: e = tid + kNT r -> token e / (N/8), states 8 (e % (N/8))
  constexpr int kBCr = kQ * (N / 8) / kNT;    // 1 (N = 64 or 16 waves) or 2 (N = 128)
  static_assert(kBCr >= 1, "one B/C piece per thread at least");
  constexpr int kDtWave = kW16 ? 15 : P == 64 ? 3 : 7;   // at P = 32 a wave with no other role
  // B C^T tiles: waves 0-2 (12-14 with 16 waves)
  const int gw = kW16 ? w - 12 : w;
  const bool has_g = gw >= 0 && gw < 3;
  // At P = 32 (two workgroups per CU, 128 registers) a chunk's z is loaded at
  // its own stage instead of one chunk ahead, and the epilogue reads the
  // thread's x piece back from the x tile (which only this thread rewrites, at
  // the next stage) instead of keeping it in registers
  constexpr bool kLean = P == 32;
  // At P = 64, chunk c's M X, Y store and epilogue run in chunk c+1 (after its
  // C S_in, in the same phase as B C^T and the state update), so a chunk has two
  // barriers; the decay terms of chunk c+1 are then computed in chunk c's second
  // phase, from a dt loaded one chunk earlier
  constexpr bool kDefer = P == 64;

  struct Pf {
    uint4 x, z;
    uint4 bq[kBCr], cq[kBCr];
    uint32_t dt;
  };
  // Global traffic goes through buffer descriptors over the chunk's rows (built
  // in scalar registers per chunk): the per-thread offsets stay fixed, and rows
  // past the sequence's end fall outside the descriptor, so their loads return
  // 0 and their stores are dropped -- no per-lane bounds checks or 64-bit
  // address arithmetic.  Tokens t0 .. t0 + 63 of a (token, element) array with
  // tstride elements per token, of which the first tail belong to this thread
  // block: the descriptor ends at the tail of the chunk's last token inside the
  // sequence (at the largest accepted width, nheads * headdim = 2^24, that is
  // 63 * 2^25 + 2 P bytes, inside the 32-bit range).
  auto rs_chunk = [&](const uint16_t* base, int64_t t0, int64_t tstride, int tail) {
    const int64_t left = Lq - t0;
    const int64_t rows = left < kQ ? left : kQ;
    const int64_t bytes = left <= 0 ? 0 : ((rows - 1) * tstride + tail) * 2;
    return make_rsrc(base + (left <= 0 ? 0 : t0 * tstride), (int)bytes);
  };
  auto ld16 = [&](__amdgpu_buffer_rsrc_t r, int off) -> uint4 {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  };
  // an x / z piece from global memory, and an x piece to LDS
  auto ldx = [&](__amdgpu_buffer_rsrc_t r, int off) -> uint4 {
    if constexpr (kXC == 8) {
      return ld16(r, off);
    } else {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      return make_uint4(v.x, v.y, 0u, 0u);
    }
  };
  auto stx = [&](uint16_t* p, uint4 v) {
    if constexpr (kXC == 8)
      *reinterpret_cast<uint4*>(p) = v;
    else
      *reinterpret_cast<uint2*>(p) = make_uint2(v.x, v.y);
  };
  // per-thread byte offsets inside a chunk's rows
  const int x_off = (xj * (int)xs_t + xp8) * 2;
  int bc_off[kBCr];
#pragma unroll
  for (int r = 0; r < kBCr; ++r) {
    const int e = tid + kNT * r;
    bc_off[r] = ((e / (N / 8)) * N + (e % (N / 8)) * 8) * 2;
  }
  auto prefetch = [&](int64_t c, Pf& f) {
    const int64_t t0 = c * kQ;
    if (has_x) {
      f.x = ldx(rs_chunk(xb, t0, xs_t, P), x_off);
      if (!kLean && !kW16) f.z = zb ? ldx(rs_chunk(zb, t0, xs_t, P), x_off) : make_uint4(0, 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rb = rs_chunk(Bb, t0, N, N), rc = rs_chunk(Cb, t0, N, N);
#pragma unroll
    for (int r = 0; r < kBCr; ++r) {
      f.bq[r] = ld16(rb, bc_off[r]);
      f.cq[r] = ld16(rc, bc_off[r]);
    }
    if (w == kDtWave)
      f.dt = __builtin_amdgcn_raw_buffer_load_b16(rs_chunk(dtb, t0 + (kDefer ? kQ : 0), H, 1), lane * H * 2, 0, 0);
  };

  // ---- state tiles: S[n][p] rows 32 nb .., columns 32 pb .. ----
  constexpr int kSTiles = (N / 32) * (P / 32);      // (N, P) = (128, 64): 8, (64, 64) or (128, 32): 4, (64, 32): 2
  const bool has_s = w < kSTiles;
  const int s_nb = w / (P / 32), s_pb = w % (P / 32);
  f32x16 S = {};
  if (has_s) {
    const int p = s_pb * 32 + l32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = s_nb * 32 + 8 * q + 4 * h32;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.h0) v = *reinterpret_cast<const float4*>(a.h0 + ((bh * P + p) * N + n));
      S[4 * q + 0] = v.x; S[4 * q + 1] = v.y; S[4 * q + 2] = v.z; S[4 * q + 3] = v.w;
    }
  }
  // S for the next chunk's C S_in as two bf16 parts, hi = bf16(S) and
  // lo = bf16(S - hi) (S - hi is exact in fp32): C hi + C lo carries S to 2^-17,
  // where hi alone (2^-9) is read by every token of the chunk and, once the
  // decay is slow, by many chunks -- the same rounding each time
  auto write_ST = [&]() {
    if (!has_s) return;
    const int p = s_pb * 32 + l32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = s_nb * 32 + 8 * q + 4 * h32;
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float s0 = S[4 * q + 2 * k], s1 = S[4 * q + 2 * k + 1];
        hw[k] = pack_bf16x2(s0, s1);
        lw[k] = pack_bf16x2(s0 - bf(hw[k] & 0xffffu), s1 - bf(hw[k] >> 16));
      }
      *reinterpret_cast<uint2*>(ST + p * kRowN + n) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2*>(STlo + p * kRowN + n) = make_uint2(lw[0], lw[1]);
    }
  };
  write_ST();

  // Y tiles (waves 4-7 at P = 64, 4-5 at P = 32, 8-11 with 16 waves): rows 32 yi .., columns 32 yp ..
  constexpr int kYT = 2 * (P / 32);
  const bool has_y = kW16 ? (w >= 8 && w < 12) : (w >= 4 && (kYT == 4 || w < 4 + kYT));
  const int yi = P == 64 ? (w >> 1) & 1 : w & 1, yp = P == 64 ? w & 1 : 0;

  // one wave turns a chunk's dt into its decay terms (written to set `set`)
  auto dt_terms = [&](uint32_t dtv, int64_t tc0, int set) {
    const bool ok = tc0 + lane < Lq;
    const float x = bf(dtv) + bias;
    float Delta = a.softplus ? softplus_log2e(x) * 0.6931471805599453f : x;
    Delta = ok ? Delta : 0.0f;                       // past the end: a = 1, w = 0 (state unchanged)
    const float la = Delta * Ah;
    const float wj = a.euler ? Delta : (Ah != 0.0f ? expm1_f(la) / Ah : Delta);
    const float cs = wave_prefix_sum(la);
    const float tot = __shfl(cs, 63);
    float* o = dterms + set * kDSet;
    o[lane] = cs;
    o[kQ + lane] = __expf(cs);
    o[2 * kQ + lane] = __expf(tot - cs) * wj;
    o[3 * kQ + lane] = wj;
    if (lane == 0) o[4 * kQ] = __expf(tot);
  };

  // Y += M X over a Y tile's causal k range, then the tile to LDS (token-major)
  auto mx_store = [&](f32x16& acc, const uint16_t* Mb, const uint16_t* Xb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (yi == 0 && s >= 2) break;                 // rows 0..31 see tokens 0..31 only
      acc = mfma(lds_b8(Mb + (yi * 32 + l32) * kRowQ + 16 * s + 8 * h32), lds_opnd_tr(Xb, kRowP, 16 * s, yp * 32, lane),
                 acc);
    }
    const int p = yp * 32 + l32;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) Yf[(yi * 32 + 8 * q + 4 * h32 + r) * kYRow + p] = acc[4 * q + r];
  };
  // token xj, channels xp8 .. xp8 + kXC - 1 of chunk ce: y = Y + D x, gate, store (x
  // from the thread's registers, or its own piece of the x tile Xb)
  auto epilogue = [&](int64_t ce, const uint16_t* Xb, uint4 xreg, uint4 zreg) {
    if (has_x) {
      const float4 y0 = *reinterpret_cast<const float4*>(Yf + xj * kYRow + xp8);
      const float4 y1 = kXC == 8 ? *reinterpret_cast<const float4*>(Yf + xj * kYRow + xp8 + 4) : y0;
      const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      uint4 xe = xreg;
      if (kLean || kDefer) {
        if constexpr (kXC == 8) {
          xe = *reinterpret_cast<const uint4*>(Xb + xj * kRowP + xp8);
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(Xb + xj * kRowP + xp8);
          xe = make_uint4(v.x, v.y, 0u, 0u);
        }
      }
      const uint32_t xw[4] = {xe.x, xe.y, xe.z, xe.w};
      const uint32_t zw[4] = {zreg.x, zreg.y, zreg.z, zreg.w};
      uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < kXW; ++q) {
        float v0 = fmaf(Dh, bf(xw[q] & 0xffffu), yv[2 * q]);
        float v1 = fmaf(Dh, bf(xw[q] >> 16), yv[2 * q + 1]);
        if (zb) {
          v0 *= silu(bf(zw[q] & 0xffffu));
          v1 *= silu(bf(zw[q] >> 16));
        }
        o[q] = pack_bf16x2(v0, v1);
      }
      if constexpr (kXC == 8)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, make_uint4(o[0], o[1], o[2], o[3])),
            rs_chunk(yb, ce * kQ, xs_t, P), x_off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, make_uint2(o[0], o[1])),
            rs_chunk(yb, ce * kQ, xs_t, P), x_off, 0, 0);
    }
  };

  Pf pf;
  prefetch(0, pf);
  uint4 xcur, zcur, zprev = make_uint4(0, 0, 0, 0);
  f32x16 yprev = {};   // chunk c-1's C S_in, waiting for its M X (kDefer)
  if (w == kDtWave) {
    uint32_t dt0 = pf.dt;
    if constexpr (kDefer) dt0 = __builtin_amdgcn_raw_buffer_load_b16(rs_chunk(dtb, 0, H, 1), lane * H * 2, 0, 0);
    dt_terms(dt0, 0, 0);
  }
  lds_barrier();   // chunk 0's decay terms, read at its stage

  for (int64_t c = 0; c < nchunk; ++c) {
    const int64_t t0 = c * kQ;
    // ---- stage: rows as loaded; decay terms ----
    xcur = pf.x;
    if constexpr (kLean) {
      zcur = has_x && zb ? ldx(rs_chunk(zb, t0, xs_t, P), x_off) : make_uint4(0, 0, 0, 0);
    } else if constexpr (!kW16) {
      zcur = pf.z;
    }
    uint16_t* const Xc = Xtm + (kDefer ? (int)(c & 1) * L::kXtm : 0);   // this chunk's x and M tiles
    uint16_t* const Mc = Ms + (kDefer ? (int)(c & 1) * L::kMs : 0);
    uint16_t* const Xprev = Xtm + (kDefer ? (int)((c + 1) & 1) * L::kXtm : 0);   // chunk c-1's
    uint16_t* const Mprev = Ms + (kDefer ? (int)((c + 1) & 1) * L::kMs : 0);
#ifdef MSCAN_LDS_POISON
    // every tile this chunk writes before reading it: C, B, the scaled x, this chunk's x and M
    // tiles and Y (none of them still holds data a later phase reads)
    lds_poison(Cs, 2 * (L::kCs + L::kBs + 2 * L::kXs));
    lds_poison(Xc, 2 * L::kXtm);
    lds_poison(Mc, 2 * L::kMs);
    if constexpr (!L::kYinM) lds_poison(Yf, 4 * kQ * kYRow);
#endif
    if (has_x) stx(Xc + xj * kRowP + xp8, pf.x);
#pragma unroll
    for (int r = 0; r < kBCr; ++r) {
      const int e = tid + kNT * r;
      const int j = e / (N / 8), n8 = (e % (N / 8)) * 8;
      *reinterpret_cast<uint4*>(Cs + j * kRowN + n8) = pf.cq[r];
      *reinterpret_cast<uint4*>(Bs + j * kRowNB + n8) = pf.bq[r];
    }
    const int dset = (int)(c & 1);
    const float* cum = dterms + dset * kDSet;   // running sum of log a in the chunk
    const float* ecum = cum + kQ;               // exp(cum_i)
    const float* scl = ecum + kQ;               // exp(cum_Q - cum_j) w_j
    const float* wv = scl + kQ;                 // w_j
    const float* atot = wv + kQ;                // exp(cum_Q)
    if (has_x) {
      // the thread's own x piece (token xj, channels xp8 ..) scaled by exp(cum_Q - cum_j) w_j, as
      // two bf16 parts hi + lo (the rest after hi is exact in fp32): 16 significant bits over
      // fp32's range
      const float sc = scl[xj];
      const uint32_t cw[4] = {xcur.x, xcur.y, xcur.z, xcur.w};
      uint32_t hv[4] = {0u, 0u, 0u, 0u}, lv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < kXW; ++k) {
        const float v0 = bf(cw[k] & 0xffffu) * sc, v1 = bf(cw[k] >> 16) * sc;
        hv[k] = pack_bf16x2(v0, v1);
        lv[k] = pack_bf16x2(v0 - bf(hv[k] & 0xffffu), v1 - bf(hv[k] >> 16));
      }
      stx(Xs + xj * kRowP + xp8, make_uint4(hv[0], hv[1], hv[2], hv[3]));
      stx(XsLo + xj * kRowP + xp8, make_uint4(lv[0], lv[1], lv[2], lv[3]));
    }
    lds_barrier();

    // ---- A2: next loads; G -> M (waves 0-2); C S_in (waves 4-7); state update ----
    const uint32_t dt_next = pf.dt;   // kDefer: chunk c+1's dt, loaded during chunk c-1
    // this phase's critical path runs through the B C^T / M and Y waves (the state waves end it
    // early): raised issue priority puts their instructions ahead of the others' on a shared
    // SIMD (0.325 -> 0.316 ms, same-box A/B over six rounds)
    if (has_g || has_y) __builtin_amdgcn_s_setprio(3);
    if (c + 1 < nchunk) prefetch(c + 1, pf);
    // with 16 waves (registers short) chunk c-1's z is loaded here, for its epilogue in this
    // chunk's last phase, instead of riding along from its own prefetch
    uint4 zE = make_uint4(0, 0, 0, 0);
    if constexpr (kW16) {
      if (has_x && zb && c > 0) zE = ldx(rs_chunk(zb, t0 - kQ, xs_t, P), x_off);
    }
    if constexpr (kDefer) {
      if (has_y && c > 0) mx_store(yprev, Mprev, Xprev);   // chunk c-1's Y, read after this phase
    }
    f32x16 yacc = {};
    if (has_g) {
      // G^T tile (rows j-block jb, columns i-block ib) over N, two accumulation chains
      const int jb = gw == 2 ? 1 : 0, ib = gw == 0 ? 0 : 1;
      // (one chain at P = 32, where two workgroups share a CU and registers are short)
      f32x16 g0 = {}, g1 = {};
#pragma unroll
      for (int s = 0; s < N / 16; s += 2) {
        g0 = mfma(lds_b8(Bs + (jb * 32 + l32) * kRowNB + 16 * s + 8 * h32),
                  lds_b8(Cs + (ib * 32 + l32) * kRowN + 16 * s + 8 * h32), g0);
        f32x16& g = (P == 64 && !kW16) ? g1 : g0;
        g = mfma(lds_b8(Bs + (jb * 32 + l32) * kRowNB + 16 * (s + 1) + 8 * h32),
                 lds_b8(Cs + (ib * 32 + l32) * kRowN + 16 * (s + 1) + 8 * h32), g);
      }
      // M[i][j] = G^T[j][i] exp(cum_i - cum_j) w_j for j <= i: the lane holds column i, rows j in runs of 4
      const int i = ib * 32 + l32;
      const float ci = cum[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j0 = jb * 32 + 8 * q + 4 * h32;
        const float4 cj = *reinterpret_cast<const float4*>(cum + j0);
        const float4 wj = *reinterpret_cast<const float4*>(wv + j0);
        const float cja[4] = {cj.x, cj.y, cj.z, cj.w}, wja[4] = {wj.x, wj.y, wj.z, wj.w};
        float m4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // exp(-200) is 0 in fp32, so the upper triangle comes out 0 from the same
          // instructions (no branch per element)
          const float d = j0 + r <= i ? ci - cja[r] : -200.0f;
          const float g = (P == 64 && !kW16) ? g0[4 * q + r] + g1[4 * q + r] : g0[4 * q + r];
          m4[r] = g * __expf(d) * wja[r];
        }
        *reinterpret_cast<uint2*>(Mc + i * kRowQ + j0) = make_uint2(pack_bf16x2(m4[0], m4[1]), pack_bf16x2(m4[2], m4[3]));
      }
    } else if (has_y) {
      // C S_in = C hi + C lo over N (two chains), rows scaled by exp(cum_i)
      f32x16 y1 = {};
#pragma unroll
      for (int s = 0; s < N / 16; s += 2) {
        const bf16x8 c0 = lds_b8(Cs + (yi * 32 + l32) * kRowN + 16 * s + 8 * h32);
        const bf16x8 c1 = lds_b8(Cs + (yi * 32 + l32) * kRowN + 16 * (s + 1) + 8 * h32);
        const int o0 = (yp * 32 + l32) * kRowN + 16 * s + 8 * h32, o1 = o0 + 16;
        f32x16& y = (P == 64 && !kW16) ? y1 : yacc;
        yacc = mfma(c0, lds_b8(STlo + o0), yacc);
        y = mfma(c1, lds_b8(STlo + o1), y);
        yacc = mfma(c0, lds_b8(ST + o0), yacc);
        y = mfma(c1, lds_b8(ST + o1), y);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 e = *reinterpret_cast<const float4*>(ecum + yi * 32 + 8 * q + 4 * h32);
        const float ev[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          yacc[4 * q + r] = ((P == 64 && !kW16) ? yacc[4 * q + r] + y1[4 * q + r] : yacc[4 * q + r]) * ev[r];
      }
    }
    if (has_s) {
      // S = exp(cum_Q) S + B^T (x exp(cum_Q - cum_j) w_j), the scaled x as hi + lo
      const float at = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(atot[0])));
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] *= at;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 bv = lds_opnd_tr(Bs, kRowNB, 16 * s, s_nb * 32, lane);
        S = mfma(bv, lds_opnd_tr(XsLo, kRowP, 16 * s, s_pb * 32, lane), S);
        S = mfma(bv, lds_opnd_tr(Xs, kRowP, 16 * s, s_pb * 32, lane), S);
      }
    }
    if constexpr (kDefer) {
      if (w == kDtWave && c + 1 < nchunk) dt_terms(dt_next, t0 + kQ, dset ^ 1);   // the next chunk's
    }
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();

    if constexpr (!kDefer) {
      // ---- A3: Y += M x (waves 4-7) -> Yf; S -> LDS for the next chunk's C S_in ----
      if (has_y) mx_store(yacc, Mc, Xc);
#ifdef MSCAN_LDS_POISON
      lds_poison(ST, 4 * L::kST);   // hi and lo: read last in this chunk's second phase
#endif
      if (w == kDtWave && c + 1 < nchunk) dt_terms(pf.dt, t0 + kQ, dset ^ 1);   // the next chunk's, off the stage path
      write_ST();
      lds_barrier();
      // ---- epilogue ----
      epilogue(c, Xc, xcur, zcur);
    } else {
      // ---- S -> LDS for the next chunk's C S_in; chunk c-1's epilogue ----
#ifdef MSCAN_LDS_POISON
      lds_poison(ST, 4 * L::kST);   // hi and lo: read last in this chunk's second phase
#endif
      write_ST();
      if (c > 0) epilogue(c - 1, Xprev, xcur, kW16 ? zE : zprev);
      yprev = yacc;
      if constexpr (!kW16) zprev = zcur;
    }
  }
  if constexpr (kDefer) {
    if (nchunk > 0) {   // the last chunk's M X and epilogue
      const int64_t cl = nchunk - 1;
      uint16_t* const Xl = Xtm + (int)(cl & 1) * L::kXtm;
      lds_barrier();   // the previous epilogue has read Y
      if (has_y) mx_store(yprev, Ms + (int)(cl & 1) * L::kMs, Xl);
      lds_barrier();
      if constexpr (kW16) {
        const uint4 zl = has_x && zb ? ldx(rs_chunk(zb, cl * kQ, xs_t, P), x_off) : make_uint4(0, 0, 0, 0);
        epilogue(cl, Xl, xcur, zl);
      } else {
        epilogue(cl, Xl, xcur, zprev);
      }
    }
  }

  // ---- final state ----
  if (a.hT && has_s) {
    const int p = s_pb * 32 + l32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = s_nb * 32 + 8 * q + 4 * h32;
      *reinterpret_cast<float4*>(a.hT + ((bh * P + p) * N + n)) =
          make_float4(S[4 * q], S[4 * q + 1], S[4 * q + 2], S[4 * q + 3]);
    }
  }
}

template <int N, int P, int NW = 8>
hipError_t run_ssd(SArgs a, int64_t batch, int64_t headdim, hipStream_t s) {
  a.S = (int)(headdim / P);
  const size_t lds = SsdLds<N, P>::bytes();
  hipError_t e = hipFuncSetAttribute((const void*)ssd_fwd_kernel<N, P, NW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_fwd_kernel<N, P, NW>), dim3((unsigned)(batch * a.H * a.S)), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd(const SsdArgs& p, hipStream_t stream) {
  SArgs a{};
  a.x = static_cast<const uint16_t*>(p.x);
  a.dt = static_cast<const uint16_t*>(p.dt);
  a.A_log = p.A_log;
  a.B = static_cast<const uint16_t*>(p.B);
  a.C = static_cast<const uint16_t*>(p.C);
  a.D = p.D;
  a.z = static_cast<const uint16_t*>(p.z);
  a.dt_bias = p.dt_bias;
  a.h0 = p.h0;
  a.hT = p.final_state;
  a.y = static_cast<uint16_t*>(p.y);
  a.L = p.seqlen;
  a.H = (int)p.nheads;
  a.softplus = p.softplus;
  a.euler = p.euler;
  // 32-channel slices only when the head dim is an odd multiple of 32: at the
  // 64-head, batch-4 layer two 32-channel workgroups per CU (which compute
  // B C^T twice and stage B and C twice) took 0.384 ms against 0.343 ms for
  // one 64-channel workgroup per CU
  const bool p32 = p.headdim % 64 != 0;
  // (N, P) = (128, 64) in 16 waves: at the same layer 0.326 ms against 0.328 ms for 8 waves
  // without the gate, 0.362 against 0.390 ms with it
  if (p.dstate == 128)
    return p32 ? run_ssd<128, 32>(a, p.batch, p.headdim, stream) : run_ssd<128, 64, 16>(a, p.batch, p.headdim, stream);
  return p32 ? run_ssd<64, 32>(a, p.batch, p.headdim, stream) : run_ssd<64, 64>(a, p.batch, p.headdim, stream);
}

}  // namespace mscan
