// scan_fwd.hip -- forward selective scan on gfx950 (CDNA4).
//
// Method (Mamba notes, awesome.papernotes.org, 设计 1 and 设计 2; State space
// models and Mamba, jonathanding.github.io, §2 and Parallel Scan): per
// (batch, channel, state) a diagonal recurrence h = Abar h + Bbar u with the
// zero-order-hold discretization of A = -exp(A_log) at step Delta =
// softplus(delta + bias), read out as y = C.h + D u and gated by SiLU(z).
// The expanded (batch, L, channel, state) tensors are never formed: inputs are
// read from HBM once, discretized and scanned on chip, and only y (and the
// final state) are written back.
//
// Mapping.  A workgroup owns 64 channels of one batch row and all 16 states
// of each, held in VGPRs and scanned sequentially in time, tile by tile (64
// tokens): two states per lane, 8 waves (two per SIMD), described above
// scan_fwd_h2_kernel.  Three stages touch every tile:
//   stage    -- convert the tile's delta/u rows (16-byte buffer loads), compute
//               Delta*log2e = softplus(delta+bias)*log2e once per token-channel,
//               and put Delta, u and the tile's B/C values (shared by the 64
//               channels) as fp32 in LDS;
//   scan     -- per group of 4 tokens read Delta/u of the lane's channel and
//               the B/C values of the lane's two states for the four tokens
//               (four 16-byte LDS reads that every lane of a wave half shares,
//               so the values arrive as plain VGPR operands); leave a partial
//               readout over the wave's states in LDS;
//   epilogue -- sum the four partials, add D u, apply the SiLU gate, store y.
// A wave cannot hide its own stalls, so the stages are software-pipelined
// across tiles inside one instruction stream: while a wave
// scans tile k it also finishes tile k-1's epilogue and stages tile k+1, and
// the global loads of tile k+2 are in flight.  That work sits inside the
// scan's group loop, so the compiler interleaves it with the recurrence.
// Inner step per (token, state): y = Delta*log2e * A; m = 2^y - 1 (decay_m1,
// accurate for small Delta |A|); s = B u / A; h = h + m (h + s)
// (= Abar h + (Abar - 1)/A B u);  y += C h.
//
// Time chunks.  When batch x channel groups cannot fill the GPU (e.g. one
// batch row of 2048 channels and a million tokens) the sequence is cut into
// chunks scanned in parallel, each in one pass that writes its outputs: the
// first chunk from the initial state, the others from a zero state, each
// recording (sum of Delta, h_end).  A small carry kernel folds the chunks in
// order with (a1,b1) o (a2,b2) = (a2 a1, a2 b1 + b2), using the chunk decay
// exp(A * sum Delta) (exact for a diagonal, time-invariant A), and a fix-up
// kernel adds to each later chunk's outputs what its carried-in state
// contributes, C_t exp(A cumDelta_t) h_in, until that has decayed away (MAMBA
// walkthrough, x-humanoid.csdn.net, §2.2: chunks in parallel, only the state
// crosses chunk boundaries; State space models and Mamba, Parallel Scan: the
// associative operator).
#include "scan_fwd_h2.h"

namespace mscan {
namespace {

// Folds the chunk aggregates in time order.  Chunk 0 ran from the initial
// state, so its end state is exact; chunk k > 0 ran from zero and left its
// end state h_end(k) and sum Delta*log2e.  With (a1,b1) o (a2,b2) = (a2 a1,
// a2 b1 + b2) and the chunk decay exp(A sum Delta) (exact for a diagonal,
// time-invariant A), the state entering chunk k is left in carry[.., k, ..]
// and the state after the last chunk in final_state.  One thread per
// (batch, channel, state).
__global__ __launch_bounds__(256) void carry_kernel(float* __restrict__ carry, const float* __restrict__ dsum,
                                                    const float* __restrict__ A_log, float* __restrict__ final_state,
                                                    int64_t batch, int64_t dim, int dstate, int np, int64_t nchunks) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * dim * dstate) return;
  const int n = (int)(i % dstate);
  const int64_t bd = i / dstate;
  const int64_t d = bd % dim;
  const float An = -expf(A_log[d * dstate + n]);
  float h = carry[(bd * nchunks) * np + n];
  for (int64_t k = 1; k < nchunks; ++k) {
    float* slot = carry + (bd * nchunks + k) * np + n;
    const float hend = *slot;
    *slot = h;
    const float P = exp2f(An * dsum[bd * nchunks + k]);   // decay over chunk k: exp(A * sum Delta)
    h = fmaf(P, h, hend);
  }
  if (final_state) final_state[bd * dstate + n] = h;
}

// seqlen == 0: final_state = initial_state or zeros.
__global__ __launch_bounds__(256) void copy_state_kernel(const float* __restrict__ h0, float* __restrict__ fs,
                                                         int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) fs[i] = h0 ? h0[i] : 0.0f;
}

template <bool kMulti, bool kYf>
struct PickH2 {
  template <typename IoT, bool kVec, int kMode>
  struct P {
    static auto get() { return scan_fwd_h2_kernel<IoT, kVec, kMode, kMulti, false, false, kYf>; }
  };
};

template <bool kYf>
struct PickH2Conv {
  template <typename IoT, bool kVec, int kMode>
  struct P {
    static auto get() { return scan_fwd_h2_kernel<IoT, kVec, kMode, false, false, true, kYf>; }
  };
};

// the same kernel with or without the fp32 tail rows (head/tail plan)
template <bool kYf, typename IoT>
auto pick_scan_h2(const KArgs& k, bool vec) {
  if (k.conv_w != nullptr) return pick_kernel<PickH2Conv<kYf>::template P, IoT>(vec, k.mode);   // 16 states, two per lane
  if (k.acc != 0) return pick_kernel<PickH2<true, kYf>::template P, IoT>(vec, k.mode);
  return pick_kernel<PickH2<false, kYf>::template P, IoT>(vec, k.mode);
}

template <typename IoT>
hipError_t launch_scan_h2(const KArgs& k, bool vec, int64_t grid, hipStream_t s) {
  auto kern = k.yf32 != nullptr ? pick_scan_h2<true, IoT>(k, vec) : pick_scan_h2<false, IoT>(k, vec);
  const size_t lds = sizeof(float) * LdsH2::floats();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, s, k);
  return hipGetLastError();
}


template <typename IoT>
hipError_t run_fwd(const FwdArgs& a, const FwdPlan& p, hipStream_t s) {
  if (a.seqlen == 0) {
    if (a.final_state) {
      const int64_t n = a.batch * a.dim * a.dstate;
      hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.h0,
                         a.final_state, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  char* ws = static_cast<char*>(a.workspace);
  float* carry = p.nchunks > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  float* dsum = p.nchunks > 1
                    ? reinterpret_cast<float*>(ws + align256(sizeof(float) *
                                                             (size_t)(a.batch * a.dim * p.nchunks * p.np)))
                    : nullptr;
  // the sum of Delta over each range of a chunk (chunks of several ranges)
  float* rsum = (p.nchunks > 1 && p.nranges > 1)
                    ? reinterpret_cast<float*>(reinterpret_cast<char*>(dsum) +
                                               align256(sizeof(float) * (size_t)(a.batch * a.dim * p.nchunks)))
                    : nullptr;
  const size_t esz = sizeof(IoT);
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a.u) | reinterpret_cast<uintptr_t>(a.delta) |
                        reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.z) |
                        reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.C) |
                        reinterpret_cast<uintptr_t>(a.u_out);
  const bool vec = ((mis & 15) == 0) && ((a.seqlen * (int64_t)esz) % 16 == 0);
  KArgs k{};
  k.conv_w = a.conv_w; k.conv_b = a.conv_b; k.conv_state = a.conv_state; k.u_out = a.u_out;
  k.u = a.u; k.delta = a.delta; k.A_log = a.A_log; k.B = a.B; k.C = a.C; k.D = a.D; k.z = a.z; k.bias = a.bias;
  k.h0 = a.h0; k.final_state = a.final_state; k.y = a.y; k.carry = carry; k.dsum = dsum;
  k.rsum = rsum; k.nranges = p.nranges; k.range_tiles = p.range_tiles; k.head_tail = p.head_tail;
  k.range_shift = __builtin_ctz((unsigned)p.range_tiles);
  k.yf32 = p.head_tail ? reinterpret_cast<float*>(ws + p.off_yf32) : nullptr;
  k.yf32_pitch = p.tail_tiles * p.tile;
  k.dim = a.dim; k.seqlen = a.seqlen; k.chunk_len = p.chunk_len; k.nchunks = p.nchunks;
  k.chgroups = (a.dim + kCh - 1) / kCh;
  k.dstate = (int)a.dstate; k.np = p.np; k.mode = (a.softplus ? kModeSoftplus : 0) | (a.euler ? kModeEuler : 0); k.gated = a.z != nullptr;
  const int64_t groups = a.batch * k.chgroups;
  // dstate > 16: one pass per 16-state group; the readouts are summed in yacc
  const int ng = p.ngroups;
  k.yacc = ng > 1 ? reinterpret_cast<float*>(ws + p.off_yacc) : nullptr;
  // every chunk is scanned at once (chunks after the first from a zero state),
  // then the carry is folded and the fix-up adds the carried-in part to y
  k.nwork = groups * p.nchunks;
  for (int g = 0; g < ng; ++g) {
    k.n0 = 16 * g;
    k.acc = ng == 1 ? 0 : (g == 0 ? 1 : (g == ng - 1 ? 3 : 2));
    hipError_t e = launch_scan_h2<IoT>(k, vec, k.nwork, s);
    if (e != hipSuccess) return e;
  }
  if (p.nchunks > 1) {
    const int64_t n = a.batch * a.dim * a.dstate;
    hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, carry, dsum, a.A_log,
                       a.final_state, a.batch, a.dim, (int)a.dstate, p.np, p.nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    FixArgs f{};
    f.delta = a.delta; f.bias = a.bias; f.A_log = a.A_log; f.C = a.C; f.z = a.z; f.y = a.y; f.carry = carry;
    f.rsum = rsum; f.nranges = p.nranges; f.range_len = (int64_t)p.range_tiles * p.tile;
    f.yf32 = k.yf32; f.yf32_pitch = k.yf32_pitch;
    f.dim = a.dim; f.seqlen = a.seqlen; f.chunk_len = p.chunk_len; f.nchunks = p.nchunks;
    f.chgroups = (a.dim + kFixCh - 1) / kFixCh;   // the fix-up's narrower channel groups
    f.nwork = a.batch * f.chgroups * (p.nchunks - 1) * p.nranges; f.dstate = (int)a.dstate; f.np = p.np; f.softplus = a.softplus;
    launch_fix_ng<IoT, false>(f, ng, vec, s);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

constexpr int64_t kCUs = 256;   // MI355X compute units (one scan workgroup per CU, by LDS)

bool make_fwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t nchunks_req, int npw_req,
                   FwdPlan* p) {
  if (npw_req != 0 && npw_req != 2) return false;   // one layout: two states per lane
  if (nchunks_req < 0) return false;
  if (dstate < 1 || dstate > 64) return false;
  p->ngroups = (int)((dstate + 15) / 16);
  // states past dstate are padding that contributes exactly zero
  p->npw = 2;
  p->tile = 64;
  p->nsplit = 8;   // waves per workgroup
  p->np = 16 * p->ngroups;
  const int64_t T = p->tile;
  const int64_t tiles = (seqlen + T - 1) / T;
  p->lp = tiles * T;
  int64_t nch = 1;
  const int64_t groups = batch * ((dim + kCh - 1) / kCh);
  int64_t head_tiles = 0;   // > 0: a head and a tail chunk of unequal length
  p->range_tiles = kFixRangeTiles;
  if (nchunks_req > 0) {
    nch = nchunks_req;
  } else if (groups < 128 && tiles >= 16) {
    // too few workgroups to fill 256 CUs: scan time chunks in parallel (each >= 8 tiles)
    nch = std::min<int64_t>(kCUs / groups, tiles / 8);
  } else if (groups > 128 && groups < kCUs) {
    // groups on as many CUs and kCUs - groups idle: each row's head runs on its own CU while
    // the tails, `rounds` at a time, take the idle CUs; with the tail a (rounds + 1)-th of the
    // row (less a tile per extra round: a workgroup's start-up, its first prefetches and
    // staging, costs about a tile, paid by a head once and by the tails once per round), heads
    // and tails end together.  The tails' fix-up (every state still live over a tail) runs in
    // ranges of a quarter of a tail (2 or 4 tiles), spread over the whole GPU.  At most 4
    // rounds and tails of 6 to 16 tiles (measured at 7: the 130M layer; 8 and 9 tiles there
    // were slower): shorter or more tails cost more in start-up and fix-up than they save,
    // and longer ones are not measured.
    const int64_t rounds = (groups + (kCUs - groups) - 1) / (kCUs - groups);
    const int64_t tail = (tiles - (rounds - 1)) / (rounds + 1);
    if (rounds <= 4 && tail >= 6 && tail <= 16) {
      head_tiles = tiles - tail;
      nch = 2;
      p->range_tiles = tail > 8 ? 4 : 2;
    }
  }
  nch = std::max<int64_t>(1, std::min<int64_t>(nch, std::max<int64_t>(tiles, 1)));
  const int64_t tiles_per = head_tiles > 0 ? head_tiles : (tiles + nch - 1) / nch;
  p->chunk_len = std::max<int64_t>(1, tiles_per) * T;
  p->nchunks = tiles > 0 ? (tiles + tiles_per - 1) / tiles_per : 1;
  p->head_tail = head_tiles > 0 && p->nchunks == 2;
  p->tail_tiles = p->head_tail ? tiles - head_tiles : 0;
  const int64_t range_len = (int64_t)p->range_tiles * T;
  p->nranges = p->nchunks > 1 ? (p->chunk_len + range_len - 1) / range_len : 1;
  p->ws_carry = 0;
  if (p->nchunks > 1)
    p->ws_carry = align256(sizeof(float) * (size_t)(batch * dim * p->nchunks * p->np)) +
                  align256(sizeof(float) * (size_t)(batch * dim * p->nchunks)) +
                  (p->nranges > 1 ? align256(sizeof(float) * (size_t)(batch * dim * p->nchunks * p->nranges)) : 0);
  // head/tail: the tail's gated y in fp32, so its outputs are rounded to the io dtype once
  // (after the fix-up's correction), as in a one-pass scan
  p->off_yf32 = p->ws_carry;
  if (p->head_tail) p->ws_carry += align256(sizeof(float) * (size_t)(batch * dim * p->tail_tiles * T));
  p->off_yacc = p->ws_carry;
  p->ws_yacc = p->ngroups > 1 ? align256(sizeof(float) * (size_t)(batch * dim * seqlen)) : 0;
  p->ws_total = seqlen == 0 ? 0 : p->ws_carry + p->ws_yacc;
  return true;
}

hipError_t launch_fwd(const FwdArgs& a, const FwdPlan& p, hipStream_t stream) {
  return a.io_bf16 ? run_fwd<uint16_t>(a, p, stream) : run_fwd<float>(a, p, stream);
}

}  // namespace mscan
