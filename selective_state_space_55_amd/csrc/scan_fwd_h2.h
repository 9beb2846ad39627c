// scan_fwd_h2.h -- the forward scan's shared definitions and its
// two-states-per-lane kernel, included by scan_fwd.hip (fixed-length batches)
// and scan_fwd_varlen.hip (sequences packed along time).  Private to the
// library; everything is in an anonymous namespace, so each including file
// gets its own instantiations.
#pragma once

#include "internal.h"
#include "io.h"

namespace mscan {
namespace {

constexpr int kCh = 64;   // channels per workgroup, one per lane
constexpr int kPad = 4;   // LDS row padding in floats
constexpr int kModeSoftplus = 1;   // Delta = softplus(delta + bias)
constexpr int kModeEuler = 2;      // Bbar u = Delta B u instead of the zero-order hold

// A chunk's fix-up is cut into ranges (kFixRangeTiles tiles by default), one workgroup
// each: a range starts from the chunk's Delta summed over the ranges before it (recorded
// by the scan) and stops when its states have decayed, so a slowly decaying channel's
// correction runs in parallel ranges rather than as one long sequential walk.
constexpr int kFixRangeTiles = 32;

struct KArgs {
  const void* u;
  const void* delta;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const float* h0;
  float* final_state;
  void* y;
  float* carry;        // [batch][dim][nchunks][np]
  float* dsum;         // [batch][dim][nchunks]
  float* rsum;         // [batch][dim][nchunks][nranges]: sum of Delta*log2e over each range of range_tiles tiles
  int64_t nranges;     // (chunks of more than one range; else rsum is null)
  int range_tiles, range_shift;   // a power of two and its log2
  int head_tail;       // work items chunk by chunk in launch order (every head, then the tails)
  float* yacc;         // [batch][dim][seqlen] fp32 readout summed over state groups (dstate > 16)
  int64_t dim, seqlen, chunk_len, nchunks, chgroups, nwork;
  int dstate, np, mode, gated;   // mode: kModeSoftplus | kModeEuler
  const int64_t* cu;   // varlen: sequence start offsets (nseq + 1), device memory
  const int64_t* pstart;   // varlen: first piece of each sequence (nseq + 1), device memory
  int64_t nseq;            // varlen: number of sequences
  int n0;              // first state of this pass (a multiple of 16)
  int acc;             // state-group pass: 1 first (writes yacc), 2 middle (adds), 3 last (adds, writes y)
  // fused causal conv1d (K = 4) + SiLU in front of the scan: u holds the conv input x
  const float* conv_w;     // (dim, 4) taps, oldest input first
  const float* conv_b;     // (dim) or NULL
  const void* conv_state;  // (batch, dim, 3) io: the inputs before the sequence, or NULL (zeros)
  void* u_out;             // (batch, dim, seqlen) io: the conv output, or NULL
  // head/tail plan: the tail chunk's gated y in fp32, (batch, dim, yf32_pitch), rounded to
  // the io dtype once, by the fix-up, after its correction is added
  float* yf32;
  int64_t yf32_pitch;
};

// Work id with XCD-aware placement: the hardware deals consecutive workgroup
// ids round-robin over the 8 XCDs; map them so each XCD gets a contiguous
// range of work ids (same batch row -> same B/C lines in that XCD's L2).
__device__ __forceinline__ int64_t work_id(int64_t bid, int64_t nwork) {
  if ((nwork & 7) != 0) return bid;
  return (bid & 7) * (nwork >> 3) + (bid >> 3);
}

// Two-states-per-lane layout: 8 waves (two per SIMD) over 64 channels.  Wave w
// covers channels (w & 1) * 32 .. +31; its lanes l and l + 32 hold the same
// channel and different state pairs, states (w >> 1) * 4 + (l >> 5) * 2 + {0, 1}.
// The two halves' readouts are summed in the wave (v_permlane32_swap), so a
// (token, channel) again has four partial readouts, one per wave pair.  With
// two waves per SIMD one wave's LDS, memory and barrier waits overlap the
// other's arithmetic.  Tiles are 64 tokens, so the 8 threads that load a
// row's tile read one whole 128-byte line (bf16) with one instruction; staging
// and the epilogue use one 8-token piece per thread.  The partial readouts
// are single-buffered: the epilogue reads of tile k-1 finish (barrier) before
// tile k's scan writes its partials.
struct LdsH2 {
  static constexpr int kT = 64;
  static constexpr int kRow = kT + kPad;
  static constexpr int kG = kT / 4;
  static constexpr int kDU = 2 * kCh * kRow;
  static constexpr int kBC = 2 * kG * 16 * 8;
  static constexpr int kPar = 2 * kCh;
  static constexpr int kY = 4 * kCh * kRow;
  static constexpr int floats() { return 2 * kDU + kBC + kPar + kY; }
};

// kMulti: one of several 16-state passes of a dstate > 16 scan; the readout of
// the pass is summed into an fp32 buffer, and the last pass adds D u, gates
// and writes y.
// kVarlen: sequences packed along the time axis of one row per channel; a
// work item is (piece, channel group), a piece being up to chunk_len tokens of
// one sequence [cu[s], cu[s+1]): the first piece starts from the sequence's
// own initial state, later ones from the carry, as the time chunks of a row
// do.  Tiles stay aligned to 64 tokens of the row (whole-line loads); tokens of
// the first tile before the piece start are staged as Delta = 0, u = 0 (state
// unchanged) and not stored.
// kConv: u is the output of a causal depthwise conv1d (4 taps) + SiLU of the
// input in a.u, computed while staging: a piece's three inputs before its first
// token come from the neighbouring piece (cross-lane read) or, for a tile's
// first piece, from the previous tile (kept in registers), the chunk's
// preceding inputs or the conv state.  The conv output is rounded to the io
// dtype, so the result equals the conv1d launch followed by the scan.
// kYf: head/tail plan, the tail chunk's y goes to the fp32 rows a.yf32 (fixed-length rows only)
template <typename IoT, bool kVec, int kMode, bool kMulti, bool kVarlen = false, bool kConv = false, bool kYf = false>
__global__ __launch_bounds__(512) void scan_fwd_h2_kernel(KArgs a) {
  static_assert(!(kYf && kVarlen), "the fp32 tail rows exist for fixed-length rows only");
  using IO = Io<IoT>;
  using V4 = typename IO::V4;
  using V8 = typename IO::V8;
  constexpr int NT = 512;
  constexpr int T = LdsH2::kT;
  constexpr int kRow = LdsH2::kRow;
  constexpr int kG = LdsH2::kG;
  constexpr int NP = 16;
  constexpr int kPieces = kCh * T / 8;     // (channel, 8-token) pieces of Delta/u/z per tile
  static_assert(kPieces == NT, "one piece per thread");
  constexpr int kBCPieces = 2 * NP * kG;   // (B or C, state, 4-token group) pieces per tile
  static_assert(kBCPieces == NT, "one B/C piece per thread");
  constexpr int kEsz = (int)sizeof(IoT);
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;
  constexpr bool kSp = (kMode & kModeSoftplus) != 0;
  constexpr bool kEuler = (kMode & kModeEuler) != 0;

  extern __shared__ float smem[];
  float* dbuf = smem;                      // [2][64][kRow]  Delta*log2e
  float* ubuf = dbuf + LdsH2::kDU;         // [2][64][kRow]  u
  float* bcs = ubuf + LdsH2::kDU;          // [2][kG][NP/2 state pairs][4 tokens][B0, B1, C0, C1]
  float* par = bcs + LdsH2::kBC;           // [2][64]        bias, D
  float* ypart = par + LdsH2::kPar;        // [4][64][kRow]  partial readouts (output pass only)
  lds_poison(smem, (int)sizeof(float) * LdsH2::floats());

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;                // lane half: which state pair of the wave's four states
  const int chw = (w & 1) * 32 + (lane & 31);   // the lane's channel within the workgroup
  const int sp = w >> 1;                   // partial-readout slot of the wave pair
  const int pc = tid / 8;                  // this thread's staging/epilogue piece: channel
  const int pg = tid % 8;                  //   and tokens 8 pg .. 8 pg + 7

  // varlen: work items of unequal length are dealt round-robin over the XCDs as
  // launched (a contiguous range per XCD would give one XCD all of a long
  // sequence's channel groups)
  int64_t wid = (kVarlen || a.head_tail) ? (int64_t)blockIdx.x : work_id(blockIdx.x, a.nwork);
  // kc of nk: this work item's time chunk (varlen: piece pidx, the kc-th of its sequence's nk)
  int64_t kc, nk, cg, b, t_begin, t_end, sidx, pidx = 0;   // sidx: batch row or sequence of the state arrays
  if constexpr (kVarlen) {
    cg = wid % a.chgroups;
    pidx = wid / a.chgroups;
    const int64_t* ps = a.pstart;
    if (pidx >= ps[a.nseq]) return;   // the grid is an upper bound on the number of pieces
    int64_t lo = 0, hi = a.nseq - 1;  // the sequence: the last s with ps[s] <= pidx
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (ps[mid] <= pidx)
        lo = mid;
      else
        hi = mid - 1;
    }
    sidx = lo;
    kc = pidx - ps[lo];
    nk = ps[lo + 1] - ps[lo];
    b = 0;
    const int64_t s_begin = min(max(a.cu[sidx], (int64_t)0), a.seqlen);   // clamped: any offsets stay in bounds
    const int64_t s_end = min(max(a.cu[sidx + 1], s_begin), a.seqlen);
    t_begin = min(s_begin + kc * a.chunk_len, s_end);
    t_end = min(t_begin + a.chunk_len, s_end);
  } else {
    if (a.head_tail) {   // chunk-major: every head is dispatched before any tail
      const int64_t per = a.nwork / a.nchunks;
      kc = wid / per;
      wid %= per;
    } else {
      kc = wid % a.nchunks;
      wid /= a.nchunks;
    }
    cg = wid % a.chgroups;
    b = wid / a.chgroups;
    sidx = b;
    nk = a.nchunks;
    t_begin = kc * a.chunk_len;
    t_end = min(t_begin + a.chunk_len, a.seqlen);
  }
  const int64_t d0 = cg * kCh;
  const int64_t t_first = kVarlen ? (t_begin & ~(int64_t)(T - 1)) : t_begin;   // first tile
  const int64_t ntile = (t_end - t_first + T - 1) / T;

  const IoT* __restrict__ gu = static_cast<const IoT*>(a.u);
  const IoT* __restrict__ gd = static_cast<const IoT*>(a.delta);
  const IoT* __restrict__ gz = static_cast<const IoT*>(a.z);
  const IoT* __restrict__ gB = static_cast<const IoT*>(a.B);
  const IoT* __restrict__ gC = static_cast<const IoT*>(a.C);
  IoT* __restrict__ gy = static_cast<IoT*>(a.y);

  if (tid < kCh) {
    const int64_t dd = d0 + tid;
    const bool ok = dd < a.dim;
    par[tid] = (ok && a.bias) ? a.bias[dd] : 0.0f;
    par[kCh + tid] = (ok && a.D) ? a.D[dd] : 0.0f;
  }

  // ---- per-lane constants and state ----
  const int64_t d = d0 + chw;
  const bool ch_ok = d < a.dim;
  const int64_t bd = sidx * a.dim + d;   // (batch row or sequence, channel) of the state arrays
  const int64_t cslot = kVarlen ? pidx * a.dim + d : bd * a.nchunks + kc;   // chunk slot of carry and dsum
  float A[2], iA[2], h[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = a.n0 + sp * 4 + hf * 2 + j;
    const bool valid = ch_ok && n < a.dstate;
    const float An = valid ? -expf(a.A_log[d * a.dstate + n]) : 0.0f;
    A[j] = An;
    iA[j] = valid ? 1.0f / An : 0.0f;
    // the first chunk (piece of a sequence) starts from the initial state, later
    // ones from zero: their carried-in part is added to y by the fix-up kernel
    float hv = 0.0f;
    if (valid && kc == 0 && a.h0) hv = a.h0[bd * a.dstate + n];
    h[j] = hv;
  }
  // the chunk's sum of Delta*log2e over this thread's staging pieces (channel pc, tokens
  // 8 pg .. 8 pg + 7 of every tile; masked tokens are staged as 0)
  float dsum_st = 0.0f;
  float rsum_st = 0.0f;   // the same over the current range of the chunk (rsum)
  const bool gate_on = a.gated != 0;
  const float gate_off = gate_on ? 0.0f : 1.0f;

  // ---- buffer descriptors (as in the four-states layout) ----
  const int rows_ok = (int)min((int64_t)kCh, a.dim - d0);
  const int64_t row0 = (b * a.dim + d0) * a.seqlen;
  const int nrec_ch = (int)((int64_t)rows_ok * a.seqlen * kEsz);
  const int nrec_bc = (int)((int64_t)a.dstate * a.seqlen * kEsz);
  const __amdgpu_buffer_rsrc_t rs_u = make_rsrc(gu + row0, nrec_ch);
  const __amdgpu_buffer_rsrc_t rs_d = make_rsrc(gd + row0, nrec_ch);
  const __amdgpu_buffer_rsrc_t rs_z = make_rsrc(gate_on ? gz + row0 : gu + row0, gate_on ? nrec_ch : 0);
  const __amdgpu_buffer_rsrc_t rs_B = make_rsrc(gB + b * a.dstate * a.seqlen, nrec_bc);
  const __amdgpu_buffer_rsrc_t rs_C = make_rsrc(gC + b * a.dstate * a.seqlen, nrec_bc);

  // conv taps and bias of the staging piece's channel; xlast: the three inputs
  // before the next tile's first piece (meaningful on the pieces that end a tile)
  float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f, xlast[3] = {0.0f, 0.0f, 0.0f};
  if constexpr (kConv) {
    const int64_t dp = d0 + pc;
    if (dp < a.dim) {
#pragma unroll
      for (int k = 0; k < 4; ++k) cw[k] = a.conv_w[dp * 4 + k];
      cbias = a.conv_b ? a.conv_b[dp] : 0.0f;
      if (pg == 7) {
        if (t_first > 0) {
#pragma unroll
          for (int i = 0; i < 3; ++i) xlast[i] = IO::load1(gu + (b * a.dim + dp) * a.seqlen + t_first - 3 + i);
        } else if (a.conv_state) {
          const IoT* cs = static_cast<const IoT*>(a.conv_state) + (b * a.dim + dp) * 3;
#pragma unroll
          for (int i = 0; i < 3; ++i) xlast[i] = IO::load1(cs + i);
        }
      }
    }
  }
  IoT* __restrict__ guo = static_cast<IoT*>(a.u_out);

  // B/C piece: state bn, 4-token group bg; waves 0-3 load B, 4-7 load C
  const int bn = tid % NP;          // state of this thread's B/C piece within the pass's 16
  const int bg = (tid / NP) % kG;
  const bool isB = w < 4;

  struct Pf {
    V8 d, u, z;
    V4 bc;
  };
  struct Keep {
    float u[8];
    V8 z;
  };

  auto prefetch = [&](int64_t tile, Pf& p) {
    const int off = (int)(((int64_t)pc * a.seqlen + tile + pg * 8) * kEsz);
    p.d = IO::buf_load8(rs_d, off, kVec);
    p.u = IO::buf_load8(rs_u, off, kVec);
    p.z = IO::buf_load8(rs_z, off, kVec);
    const int boff = (int)(((int64_t)(a.n0 + bn) * a.seqlen + tile + bg * 4) * kEsz);   // past dstate: reads 0
    p.bc = IO::buf_load4(isB ? rs_B : rs_C, boff, kVec);
  };

  auto stage = [&](int64_t tile, const Pf& p, int buf, Keep& kp, auto full_c) {
    constexpr bool kFull = decltype(full_c)::value;
    const int nv = kFull ? 8 : (int)max((int64_t)0, min((int64_t)8, t_end - (tile + pg * 8)));
    // varlen: tokens before the sequence start (first tile only) are masked like those past the end
    const int lo = (kVarlen && !kFull) ? (int)min((int64_t)8, max((int64_t)0, t_begin - (tile + pg * 8))) : 0;
    float fd[8], fu[8];
    IO::to_f32(p.d, fd);
    IO::to_f32(p.u, fu);
    if constexpr (kConv) {
      // xx[0..2]: inputs before the piece (from the piece below, or for the
      // first piece of the tile from the previous tile's last piece), xx[3..10]: the piece
      float xx[11];
      const int src = pg == 0 ? lane + 7 : lane - 1;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const float pv = pg == 7 ? xlast[i] : fu[5 + i];
        xx[i] = __shfl(pv, src);
        xlast[i] = fu[5 + i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) xx[3 + i] = fu[i];
      float cu[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float acc = cbias;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = fmaf(cw[k], xx[i + k], acc);   // input time t - 3 + k
        cu[i] = acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * kLog2e));
      }
      const V8 cr = IO::from_f32(cu);   // rounded to the io dtype, as a stored conv output
      IO::to_f32(cr, fu);
      {
        if (guo != nullptr && d0 + pc < a.dim) {
          IoT* uo = guo + (b * a.dim + d0 + pc) * a.seqlen + tile + pg * 8;
          if (kFull && kVec)
            IO::store8(uo, cr);
          else
            IO::store_n(uo, cr, nv);
        }
      }
    }
    const float bi = par[pc];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = fd[j] + bi;
      const float dl = kSp ? softplus_log2e(x) : x * kLog2e;
      const bool ok = j >= lo && j < nv;   // masked tokens: Delta = 0, u = 0 leave h unchanged
      fd[j] = ok ? dl : 0.0f;
      fu[j] = ok ? fu[j] : 0.0f;
    }
    const float psum = ((fd[0] + fd[1]) + (fd[2] + fd[3])) + ((fd[4] + fd[5]) + (fd[6] + fd[7]));
    dsum_st += psum;
    if constexpr (!kVarlen) {
      if (a.rsum != nullptr && tile < t_end) {
        // the range's sum of Delta*log2e for the fix-up, written when the range's last tile is staged
        rsum_st += psum;
        const int64_t lt = (tile - t_begin) / T;   // the tile within the chunk
        if (((lt + 1) & (a.range_tiles - 1)) == 0 || tile + T >= t_end) {
          float rs = rsum_st;
          rs += __shfl_xor(rs, 1);
          rs += __shfl_xor(rs, 2);
          rs += __shfl_xor(rs, 4);
          if (pg == 0 && d0 + pc < a.dim)
            a.rsum[((sidx * a.dim + d0 + pc) * a.nchunks + kc) * a.nranges + (lt >> a.range_shift)] = rs;
          rsum_st = 0.0f;
        }
      }
    }
    float fs[8];   // what the scan reads per token: u, or Delta*u for the Euler input term
#pragma unroll
    for (int j = 0; j < 8; ++j) fs[j] = kEuler ? (fd[j] * kLn2) * fu[j] : fu[j];
    float* dp = dbuf + (buf * kCh + pc) * kRow + pg * 8;
    float* up = ubuf + (buf * kCh + pc) * kRow + pg * 8;
    reinterpret_cast<float4*>(dp)[0] = make_float4(fd[0], fd[1], fd[2], fd[3]);
    reinterpret_cast<float4*>(dp)[1] = make_float4(fd[4], fd[5], fd[6], fd[7]);
    reinterpret_cast<float4*>(up)[0] = make_float4(fs[0], fs[1], fs[2], fs[3]);
    reinterpret_cast<float4*>(up)[1] = make_float4(fs[4], fs[5], fs[6], fs[7]);
    {
#pragma unroll
      for (int j = 0; j < 8; ++j) kp.u[j] = fu[j];
      kp.z = p.z;
    }
    {
      const int nvb = kFull ? 4 : (int)max((int64_t)0, min((int64_t)4, t_end - (tile + bg * 4)));
      float f[4];
      IO::to_f32(p.bc, f);
      // state bn is element (bn & 1) of its pair's B (0, 1) or C (2, 3) quadruple
      float* q = bcs + buf * kG * NP * 8 + (bg * (NP / 2) + (bn >> 1)) * 16 + (isB ? 0 : 2) + (bn & 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) q[kk * 4] = (kk < nvb) ? f[kk] : 0.0f;
    }
  };

  auto epi_read = [&](float4 (&yp)[4][2]) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float4* q = reinterpret_cast<const float4*>(ypart + (s2 * kCh + pc) * kRow + pg * 8);
      yp[s2][0] = q[0];
      yp[s2][1] = q[1];
    }
  };
  // returns false when this pass only accumulates into yacc (no y store)
  auto epi_finish = [&](const float4 (&yp)[4][2], const Keep& kp, float (&yv)[8], int64_t tile) -> bool {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float* o = yv + 4 * h2;
      o[0] = yp[0][h2].x; o[1] = yp[0][h2].y; o[2] = yp[0][h2].z; o[3] = yp[0][h2].w;
#pragma unroll
      for (int s2 = 1; s2 < 4; ++s2) {
        o[0] += yp[s2][h2].x; o[1] += yp[s2][h2].y; o[2] += yp[s2][h2].z; o[3] += yp[s2][h2].w;
      }
    }
    if constexpr (kMulti) {
      // the pipelined body calls the epilogue of tile k-1 at k = 0 too, where
      // y stores are dropped by an empty buffer descriptor; yacc is a plain
      // pointer, so that call must not touch it
      if (tile < t_first) return false;
      using IOF = Io<float>;
      const int64_t t0 = tile + pg * 8;
      int nv = (int)max((int64_t)0, min((int64_t)8, t_end - t0));
      if (d0 + pc >= a.dim) nv = 0;
      float* ya = a.yacc + (b * a.dim + d0 + pc) * a.seqlen + t0;
      if (kVarlen && t0 < t_begin) {
        // piece straddling the sequence start: only its own tokens, one by one
        const int lo = (int)min((int64_t)8, t_begin - t0);
        for (int j = lo; j < nv; ++j) {
          const float v = yv[j] + (a.acc >= 2 ? ya[j] : 0.0f);
          if (a.acc < 3) ya[j] = v; else yv[j] = v;
        }
        if (a.acc < 3) return false;
      } else {
      const bool vec8 = nv == 8 && (a.seqlen & 3) == 0;
      if (a.acc >= 2) {
        float prev[8];
        IOF::to_f32(vec8 ? IOF::load8(ya) : IOF::load_n(ya, nv), prev);
#pragma unroll
        for (int j = 0; j < 8; ++j) yv[j] += prev[j];
      }
      if (a.acc < 3) {
        if (vec8)
          IOF::store8(ya, IOF::from_f32(yv));
        else
          IOF::store_n(ya, IOF::from_f32(yv), nv);
        return false;
      }
      }
    }
    const float Dd = par[kCh + pc];
    float zf[8];
    IO::to_f32(kp.z, zf);
#pragma unroll
    for (int j = 0; j < 8; ++j) yv[j] = fmaf(Dd, kp.u[j], yv[j]) * (silu(zf[j]) + gate_off);
    return true;
  };
  // head/tail plan, tail chunk: y goes to the fp32 buffer (rows padded to whole tiles, so the
  // pieces past the end are written too, into the padding).  The pipelined body's call for
  // tile k-1 at k = 0 (tile before the chunk) stores nothing: it would land in the previous row.
  const bool y_to_f32 = kYf && kc == 1;
  auto epi_store_f32 = [&](int64_t tile, const float (&yv)[8]) {
    if (tile < t_begin || d0 + pc >= a.dim) return;
    float* p = a.yf32 + (b * a.dim + d0 + pc) * a.yf32_pitch + (tile - t_begin) + pg * 8;
    reinterpret_cast<float4*>(p)[0] = make_float4(yv[0], yv[1], yv[2], yv[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(yv[4], yv[5], yv[6], yv[7]);
  };
  auto epi_store_full = [&](int64_t tile, const float (&yv)[8], __amdgpu_buffer_rsrc_t rs) {
    if (y_to_f32) {
      epi_store_f32(tile, yv);
      return;
    }
    const int off = (int)(((int64_t)pc * a.seqlen + tile + pg * 8) * kEsz);
    IO::buf_store8(rs, off, IO::from_f32(yv), kVec);
  };
  auto epi_store_tail = [&](int64_t tile, const float (&yv)[8]) {
    if (y_to_f32) {
      epi_store_f32(tile, yv);
      return;
    }
    const int64_t t0 = tile + pg * 8;
    int nv = (int)max((int64_t)0, min((int64_t)8, t_end - t0));
    if (d0 + pc >= a.dim) nv = 0;
    IO::store_n(gy + (b * a.dim + d0 + pc) * a.seqlen + t0, IO::from_f32(yv), nv);
  };
  // varlen: stores only the piece's tokens inside [t_begin, t_end), one by one
  auto epi_store_head = [&](int64_t tile, const float (&yv)[8]) {
    const int64_t t0 = tile + pg * 8;
    int nv = (int)max((int64_t)0, min((int64_t)8, t_end - t0));
    if (d0 + pc >= a.dim) nv = 0;
    const int lo = (int)min((int64_t)8, max((int64_t)0, t_begin - t0));
    IoT* p = gy + (b * a.dim + d0 + pc) * a.seqlen + t0;
    for (int j = lo; j < nv; ++j) IO::store1(p + j, yv[j]);
  };

  auto body = [&](int64_t k, auto P_c, Pf& pfCur, Pf& pfOther, Keep& kpOther) {
    constexpr int P = decltype(P_c)::value;
    const int64_t tile = t_first + k * T;
    const float* drow = dbuf + (P * kCh + chw) * kRow;
    const float* urow = ubuf + (P * kCh + chw) * kRow;
    // (B, C) of the lane's two states for the four tokens of a group: 16 floats, read as
    // four float4 (every lane of a wave half reads the same ones: an LDS broadcast)
    const float* bcl = bcs + P * kG * NP * 8 + (sp * 2 + hf) * 16;
    float* yrow = ypart + (sp * kCh + chw) * kRow + 2 * hf;

    float4 dv = *reinterpret_cast<const float4*>(drow);
    float4 uv = *reinterpret_cast<const float4*>(urow);
    // Delta of the next group: the decays a group forms are the next group's, so
    // Delta is read two groups ahead of the tokens (softplus on)
    float4 dv1 = kSp ? *reinterpret_cast<const float4*>(drow + 4) : dv;
    float4 bcv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bcv[kk] = reinterpret_cast<const float4*>(bcl)[kk];
    // varlen: tile k+2's loads at the tile start (its work items are short; issuing them in
    // group 3, as below, measured 1% slower on the 28-sequence mix)
    if constexpr (kVarlen) prefetch(tile + 2 * T, pfCur);
    float4 yp[4][2];
    {
      // tile k-1's partials must be read by every wave before tile k's are written
      epi_read(yp);
      lds_barrier();
    }
    const __amdgpu_buffer_rsrc_t rs_y = make_rsrc(gy + row0, k >= 1 ? nrec_ch : 0);

    // The update is written with the decrement m = Abar - 1 of the decay (decay_m1):
    //   zero-order hold  h_t = h + m (h + s),  s = B u / A   (= Abar h + (Abar - 1)/A B u),
    //   Euler            h_t = h + (m h + s),  s = B Delta u.
    // Rounding h + s costs eps |s| absolutely, but it is scaled by m, so the
    // step stays accurate however small Delta |A| is (the form Abar (h + s) - s
    // loses eps |B u / A| per token, without decay, when Delta |A| -> 0).  The
    // small increment is formed before it meets h, so the one rounding onto h's
    // grid varies with the input from token to token; adding a slowly varying
    // m h to an h + s already on that grid would round the same way every token
    // and drift.
    // bq = (B of state 0, B of state 1, C of state 0, C of state 1) of this token
    auto token = [&](const float (&m)[2], float uu, float4 bq) -> float {
      const float m0 = m[0], m1 = m[1];
      if constexpr (kEuler) {
        const float s0 = bq.x * uu;                                 // s = B * Delta * u
        const float s1 = bq.y * uu;
        h[0] += fmaf(m0, h[0], s0);                                 // h + (m h + s)
        h[1] += fmaf(m1, h[1], s1);
      } else {
        const float s0 = bq.x * (uu * iA[0]);                       // s = B * u / A
        const float s1 = bq.y * (uu * iA[1]);
        h[0] = fmaf(m0, h[0] + s0, h[0]);                           // h + m (h + s)
        h[1] = fmaf(m1, h[1] + s1, h[1]);
      }
      return fmaf(bq.w, h[1], bq.z * h[0]);   // C . h
    };

    // decrements of the tile's first group; each group forms the next group's
    // while it runs its own recurrence (softplus on: Delta > 0)
    float mc[4][2];
    {
      const float dls[4] = {dv.x, dv.y, dv.z, dv.w};
      decay_m1_4x2<!kSp>(dls, A, mc);
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      // next group's LDS reads first (Delta two groups ahead), then the four tokens with the
      // next group's decays issued between them, so the exp2 results and decay_m1's steps meet
      // their consumers a group later instead of stalling them (same-box A/B at the 1.4B layer:
      // 0.817 -> 0.800 ms); the epilogue and staging groups interleave with both
      float4 dn = dv, un = uv;
      float4 bcn[4] = {bcv[0], bcv[1], bcv[2], bcv[3]};
      const bool nxt = g + 1 < kG;
      float4 dn2 = dv1;
      if (kSp && g + 2 < kG) dn2 = *reinterpret_cast<const float4*>(drow + 4 * (g + 2));
      if (nxt) {
        if (!kSp) dn = *reinterpret_cast<const float4*>(drow + 4 * (g + 1));
        un = *reinterpret_cast<const float4*>(urow + 4 * (g + 1));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bcn[kk] = reinterpret_cast<const float4*>(bcl + (g + 1) * NP * 8)[kk];
      }
      float y0, y1, y2, y3;
      float mn[4][2];
      if constexpr (kSp) {
        // decay_m1 of the next group, one step between each pair of this group's tokens
        const float dln[4] = {dv1.x, dv1.y, dv1.z, dv1.w};
        float yy[4][2], ab[4][2], p1[4][2], m0[4][2], tt[4][2];
        y0 = token(mc[0], uv.x, bcv[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (nxt) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) yy[q][j] = dln[q] * A[j];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) ab[q][j] = __builtin_amdgcn_exp2f(yy[q][j]);
        }
        y1 = token(mc[1], uv.y, bcv[1]);
        __builtin_amdgcn_sched_barrier(0);
        if (nxt) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              p1[q][j] = fmaf(yy[q][j], kDecayC2, kDecayC1);
              m0[q][j] = ab[q][j] - kDecayHi;
            }
        }
        y2 = token(mc[2], uv.z, bcv[2]);
        __builtin_amdgcn_sched_barrier(0);
        if (nxt) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) tt[q][j] = __builtin_amdgcn_fmed3f(m0[q][j] - yy[q][j] * p1[q][j], 0.0f, 1.0f);
        }
        y3 = token(mc[3], uv.w, bcv[3]);
        __builtin_amdgcn_sched_barrier(0);
        if (nxt) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) mn[q][j] = m0[q][j] - tt[q][j];   // min(m0, p2), as in decay_m1
        }
      } else {
        y0 = token(mc[0], uv.x, bcv[0]);
        y1 = token(mc[1], uv.y, bcv[1]);
        y2 = token(mc[2], uv.z, bcv[2]);
        y3 = token(mc[3], uv.w, bcv[3]);
        if (nxt) {
          const float dln[4] = {dn.x, dn.y, dn.z, dn.w};
          decay_m1_4x2<true>(dln, A, mn);
        }
      }
      {
        // lanes 0-31 get tokens 0, 1 and lanes 32-63 tokens 2, 3 of their channel, over all four states
        *reinterpret_cast<float2*>(yrow + 4 * g) = make_float2(half_sum2(y0, y2), half_sum2(y1, y3));
      }
      {
        if (g == 1) {
          float yv[8];
          if (epi_finish(yp, kpOther, yv, tile - T)) {
            if constexpr (kVarlen) {
              if (k >= 1) {   // the first tile may start before the sequence
                if (tile - T < t_begin)
                  epi_store_head(tile - T, yv);
                else
                  epi_store_full(tile - T, yv, rs_y);
              }
            } else {
              epi_store_full(tile - T, yv, rs_y);
            }
          }
        }
      }
      // tile k+2's loads (pfCur was staged in the previous body), issued after the epilogue and
      // staging groups rather than beside the tile-start barrier: 0.830 -> 0.823 ms at the 1.4B layer
      if (!kVarlen && g == 3) prefetch(tile + 2 * T, pfCur);
      if (g == 2) {
        if (tile + 2 * T <= t_end)
          stage(tile + T, pfOther, 1 - P, kpOther, IntC<1>{});
        else
          stage(tile + T, pfOther, 1 - P, kpOther, IntC<0>{});
      }
      if (nxt) {
        dv = dn;
        dv1 = dn2;
        uv = un;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bcv[kk] = bcn[kk];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 2; ++j) mc[q][j] = mn[q][j];
      }
    }
    lds_barrier();
  };

  auto last_epilogue = [&](int64_t k, const Keep& kp) {
    {
      float4 yp[4][2];
      epi_read(yp);
      float yv[8];
      if (epi_finish(yp, kp, yv, t_first + k * T)) {
        if constexpr (kVarlen)
          epi_store_head(t_first + k * T, yv);
        else
          epi_store_tail(t_first + k * T, yv);
      }
    }
  };

  Pf pf0, pf1;
  Keep kp0 = {}, kp1 = {};
  prefetch(t_first, pf0);
  prefetch(t_first + T, pf1);
  __syncthreads();   // par[] visible
  stage(t_first, pf0, 0, kp0, IntC<0>{});
  lds_barrier();
  for (int64_t k = 0; k < ntile; k += 2) {
    body(k, IntC<0>{}, pf0, pf1, kp1);
    if (k + 1 >= ntile) {
      last_epilogue(k, kp0);
      break;
    }
    body(k + 1, IntC<1>{}, pf1, pf0, kp0);
    if (k + 2 >= ntile) {
      last_epilogue(k + 1, kp1);
      break;
    }
  }

  // ---- final state or chunk aggregate ----
  // rows in several chunks, and every varlen piece: each chunk leaves (h_end,
  // sum Delta) for the carry kernel, which writes the final state
  const bool chunk_out = kVarlen || a.nchunks > 1;
  if (ch_ok) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = a.n0 + sp * 4 + hf * 2 + j;
      if (chunk_out) {
        a.carry[cslot * a.np + n] = h[j];
      } else if (kc == nk - 1 && a.final_state && n < a.dstate) {
        a.final_state[bd * a.dstate + n] = h[j];
      }
    }
  }
  if (chunk_out) {
    // the 8 staging pieces of a channel are lanes 8 pc .. 8 pc + 7
    float ds = dsum_st;
    ds += __shfl_xor(ds, 1);
    ds += __shfl_xor(ds, 2);
    ds += __shfl_xor(ds, 4);
    const int64_t dp = d0 + pc;
    if (pg == 0 && dp < a.dim) a.dsum[kVarlen ? pidx * a.dim + dp : (sidx * a.dim + dp) * a.nchunks + kc] = ds;
  }
}

// Fix-up of chunks k > 0 after they were scanned from a zero state: the
// recurrence is linear in the state, so h_t = h_t(from 0) + P_t h_in with
// P_t = exp(A cumDelta_t) (cumDelta from the chunk start through token t), and
// y_t gains (sum_n C_t[n] P_t[n] h_in[n]) SiLU(z_t).  A thread owns an 8-token
// piece of one channel (the 8 threads of a channel read its 128-byte line
// segment of a tile), so the sum over states stays in registers; the pieces'
// cumDelta come from a prefix sum over the channel's 8 lanes; C of the tile is
// staged in LDS.  The correction decays with cumDelta: with softplus (Delta >=
// 0) the workgroup stops once every lane's decay is below 2^-32 at the end of
// a tile (a multiple of the state scale far below fp32 resolution of y), so
// usually only the head of a chunk is touched.  3 VALU + 1 exp per (token,
// state).
// The fix-up's workgroup: 16 channels (two waves).  A workgroup stops once the
// slowest-decaying state of its channels is below the cut-off, so narrow groups
// stop sooner (the slowest of 16 channels rather than of 64), and the small
// groups share a CU, whose other waves cover a group's barrier and memory waits.
constexpr int kFixCh = 16;
constexpr int kFixNT = kFixCh * 8;   // a thread per 8-token piece of a channel's tile

struct FixArgs {
  const int64_t* cu;       // varlen: sequence offsets (nseq + 1), device memory
  const int64_t* pstart;   // varlen: first piece of each sequence (nseq + 1), device memory
  int64_t nseq;
  const void* delta;
  const float* bias;
  const float* A_log;
  const void* C;
  const void* z;
  void* y;
  const float* carry;
  const float* rsum;       // per-range Delta sums (nranges > 1), as written by the scan
  int64_t nranges;         // ranges per chunk (1 for variable-length pieces)
  int64_t range_len;       // tokens per range (a multiple of 64)
  int64_t dim, seqlen, chunk_len, nchunks, chgroups, nwork;
  int dstate, np, softplus;
  const float* yf32;       // head/tail plan: the tail's y in fp32 (the scan's yf32), else null
  int64_t yf32_pitch;
};


// kVarlen: rows (dim, total) hold sequences back to back; a work item is
// (piece, channel group) as in the scan kernel, pieces after a sequence's first
// are fixed, and tiles stay aligned to 64 tokens of the row (the first may
// start before the piece: its earlier tokens are masked).
// kYf: the chunk's y is read from the fp32 rows a.yf32 (head/tail plan's tail) rather than from y
template <typename IoT, bool kVec, int NG, bool kVarlen, bool kYf>
__global__ __launch_bounds__(kFixNT) void fix_kernel(FixArgs a) {
  using IO = Io<IoT>;
  using V4 = typename IO::V4;
  using V8 = typename IO::V8;
  constexpr int T = 64;
  constexpr int NPS = 16 * NG;          // states, processed 16 at a time
  constexpr int kCRow = T + 4;          // LDS row of C (floats)
  constexpr int kSRow = NPS + 4;        // LDS row of a channel's A or h_in
  constexpr int kEsz = (int)sizeof(IoT);
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float cbuf[NPS * kCRow];   // [state][token]
  __shared__ float sA[kFixCh * kSRow];     // [channel][state]
  __shared__ float sH[kFixCh * kSRow];
  __shared__ float par[kFixCh];
  __shared__ unsigned long long live_w[kFixNT / 64];   // per wave: states still above the cut-off
  __shared__ unsigned long long live0;                 // states above the cut-off at the range start
  lds_poison(cbuf, (int)sizeof(cbuf));
  lds_poison(live_w, (int)sizeof(live_w));
  lds_poison(sA, (int)sizeof(sA));
  lds_poison(sH, (int)sizeof(sH));
  lds_poison(par, (int)sizeof(par));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int pc = tid / 8;               // channel within the group
  const int pg = tid % 8;               // tokens 8 pg .. 8 pg + 7 of a tile
  int64_t kc, cg, b, t_begin, t_end, slot0;   // slot0: carry slot of channel 0 of the group
  int64_t rj = 0;                              // the range of the chunk (fixed-length rows)
  int64_t c_begin0 = 0;                        // the chunk's first token (fixed-length rows)
  if constexpr (kVarlen) {
    cg = blockIdx.x % a.chgroups;
    const int64_t pidx = blockIdx.x / a.chgroups;
    const int64_t* ps = a.pstart;
    if (pidx >= ps[a.nseq]) return;   // the grid is an upper bound on the number of pieces
    int64_t lo = 0, hi = a.nseq - 1;  // the sequence: the last s with ps[s] <= pidx
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (ps[mid] <= pidx)
        lo = mid;
      else
        hi = mid - 1;
    }
    kc = pidx - ps[lo];
    if (kc == 0) return;              // a sequence's first piece ran from its initial state
    b = 0;
    const int64_t s_begin = min(max(a.cu[lo], (int64_t)0), a.seqlen);
    const int64_t s_end = min(max(a.cu[lo + 1], s_begin), a.seqlen);
    t_begin = min(s_begin + kc * a.chunk_len, s_end);
    t_end = min(t_begin + a.chunk_len, s_end);
    slot0 = pidx * a.dim;
  } else {
    // launch order: every (chunk, channel group)'s first range, then every second range, ...
    const int64_t per = a.nwork / a.nranges;
    rj = (int64_t)blockIdx.x / per;
    int64_t wid = work_id((int64_t)blockIdx.x % per, per);
    const int64_t nk1 = a.nchunks - 1;
    kc = wid % nk1 + 1;
    wid /= nk1;
    cg = wid % a.chgroups;
    b = wid / a.chgroups;
    const int64_t c_begin = kc * a.chunk_len;
    const int64_t c_end = min(c_begin + a.chunk_len, a.seqlen);
    c_begin0 = c_begin;
    t_begin = c_begin + rj * a.range_len;
    if (t_begin >= c_end) return;     // (the last chunk may be shorter)
    t_end = min(t_begin + a.range_len, c_end);
    slot0 = -1;
  }
  const int64_t d0 = cg * kFixCh;
  const int64_t d = d0 + pc;
  const bool ch_ok = d < a.dim;
  const int64_t t_first = kVarlen ? (t_begin & ~(int64_t)(T - 1)) : t_begin;
  if (tid < kFixCh) par[tid] = (d0 + tid < a.dim && a.bias) ? a.bias[d0 + tid] : 0.0f;
  if (tid == 0) live0 = 0;
  bool finite = true;
  for (int i = tid; i < kFixCh * NPS; i += kFixNT) {
    const int c = i / NPS, n = i % NPS;
    const int64_t dc = d0 + c;
    const bool valid = dc < a.dim && n < a.dstate;
    const int64_t slot = kVarlen ? slot0 + dc : (b * a.dim + dc) * a.nchunks + kc;
    const float hv = valid ? a.carry[slot * a.np + n] : 0.0f;
    sA[c * kSRow + n] = valid ? -expf(a.A_log[dc * a.dstate + n]) : 0.0f;
    sH[c * kSRow + n] = hv;
    finite = finite && (fabsf(hv) <= 3.4e38f);
  }
  // a non-finite carried-in state propagates to the chunk's end (no early stop)
  // (and with the tail's y in fp32, every token is corrected and rounded: no early stop)
  const bool all_finite = __syncthreads_and(finite ? 1 : 0) != 0;
  const bool may_stop = a.softplus != 0 && all_finite && !kYf;

  const int rows_ok = (int)min((int64_t)kFixCh, a.dim - d0);
  const int64_t row0 = (b * a.dim + d0) * a.seqlen;
  const int nrec_ch = (int)((int64_t)rows_ok * a.seqlen * kEsz);
  const bool gated = a.z != nullptr;
  const IoT* gd = static_cast<const IoT*>(a.delta);
  const __amdgpu_buffer_rsrc_t rs_d = make_rsrc(gd + row0, nrec_ch);
  const __amdgpu_buffer_rsrc_t rs_z = make_rsrc(gated ? static_cast<const IoT*>(a.z) + row0 : gd + row0,
                                                gated ? nrec_ch : 0);
  const __amdgpu_buffer_rsrc_t rs_y = make_rsrc(static_cast<IoT*>(a.y) + row0, nrec_ch);
  const __amdgpu_buffer_rsrc_t rs_C = make_rsrc(static_cast<const IoT*>(a.C) + b * a.dstate * a.seqlen,
                                                (int)((int64_t)a.dstate * a.seqlen * kEsz));
  IoT* gy = static_cast<IoT*>(a.y);
  const float bi = par[pc];
  constexpr int kCP = (NPS * 16 + kFixNT - 1) / kFixNT;   // four-token pieces of C per thread

  float base = 0.0f;   // cumDelta*log2e of the channel before the tile
  // States still corrected (bit 16 g + n).  With Delta >= 0 a state's decay only
  // shrinks, so once it is below 2^-32 at every lane's last token of a tile the
  // state's term stays under fp32 resolution of its own carried-in scale for the
  // rest of the chunk and is dropped; the workgroup stops when none is left.
  // States decay at their own rates (|A_n| spans an order of magnitude), so most
  // are dropped long before the slowest.
  uint64_t live = NPS == 64 ? ~0ull : ((1ull << NPS) - 1);
  if (!kVarlen && rj > 0) {
    // cumDelta before the range: the scan's sums over the chunk's earlier ranges, split over
    // the channel's 8 threads
    float sb = 0.0f;
    if (ch_ok) {
      const float* rs = a.rsum + ((b * a.dim + d) * a.nchunks + kc) * a.nranges;
      for (int64_t i = pg; i < rj; i += 8) sb += rs[i];
    }
    sb += __shfl_xor(sb, 1, 8);
    sb += __shfl_xor(sb, 2, 8);
    sb += __shfl_xor(sb, 4, 8);
    base = sb;
    if (may_stop) {
      // states already below the cut-off at the range start stay so (Delta >= 0): dropped,
      // and a range with none left does nothing
      unsigned long long m = 0;
      if (ch_ok)
        for (int n = pg; n < NPS; n += 8)
          if (__builtin_amdgcn_exp2f(sA[pc * kSRow + n] * base) >= 2.3283064e-10f) m |= 1ull << n;
      if (m != 0) atomicOr(&live0, m);
      __syncthreads();
      const unsigned long long l0 = live0;
      live &= ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(l0 >> 32)) << 32) |
              __builtin_amdgcn_readfirstlane((uint32_t)l0);
      if (live == 0) return;
    }
  }
  // a tile's global loads; the next tile's are issued before this tile's work,
  // so their latency overlaps it (the work per tile is small once most states
  // are dropped, and the loop would otherwise wait a memory round trip per tile;
  // two tiles ahead measured no better)
  struct Ld {
    V8 d, y, z;
    float4 yf[2];   // the tail's y in fp32 (head/tail plan)
    V4 c[kCP];
  };
  const float* const yf_row =
      (kYf && ch_ok) ? a.yf32 + (b * a.dim + d) * a.yf32_pitch + pg * 8 : nullptr;
  auto load = [&](int64_t tile, Ld& l) {
    const int off = (int)(((int64_t)pc * a.seqlen + tile + pg * 8) * kEsz);
    l.d = IO::buf_load8(rs_d, off, kVec);
    if constexpr (kYf) {
      l.yf[0] = l.yf[1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (yf_row != nullptr) {
        l.yf[0] = reinterpret_cast<const float4*>(yf_row + (tile - c_begin0))[0];
        l.yf[1] = reinterpret_cast<const float4*>(yf_row + (tile - c_begin0))[1];
      }
    } else {
      l.y = IO::buf_load8(rs_y, off, kVec);
    }
    l.z = IO::buf_load8(rs_z, off, kVec);
#pragma unroll
    for (int r = 0; r < kCP; ++r) {
      const int i = tid + r * kFixNT;
      const int n = i / 16, g4 = i % 16;
      if (i < NPS * 16) l.c[r] = IO::buf_load4(rs_C, (int)(((int64_t)n * a.seqlen + tile + 4 * g4) * kEsz), kVec);
    }
  };
  // one tile: its loads were issued a tile earlier; true once no state is left
  auto step = [&](int64_t tile, Ld& ld) -> bool {
    const int off = (int)(((int64_t)pc * a.seqlen + tile + pg * 8) * kEsz);
    const V8 vd = ld.d;
    const V8 vy = ld.y;
    const float4 yf0 = ld.yf[0], yf1 = ld.yf[1];
    const V8 vz = ld.z;
    V4 vc[kCP];
#pragma unroll
    for (int r = 0; r < kCP; ++r) vc[r] = ld.c[r];
    if (tile + T < t_end) load(tile + T, ld);   // past the row: the descriptors return 0
    __syncthreads();   // the previous tile's C reads are done
#pragma unroll
    for (int r = 0; r < kCP; ++r) {
      const int i = tid + r * kFixNT;
      const int n = i / 16, g4 = i % 16;
      if (i < NPS * 16) {
        float f[4];
        IO::to_f32(vc[r], f);
        const int64_t t4 = tile + 4 * g4;
        float4 cv;
        cv.x = (t4 >= t_begin && t4 < t_end) ? f[0] : 0.0f;
        cv.y = (t4 + 1 >= t_begin && t4 + 1 < t_end) ? f[1] : 0.0f;
        cv.z = (t4 + 2 >= t_begin && t4 + 2 < t_end) ? f[2] : 0.0f;
        cv.w = (t4 + 3 >= t_begin && t4 + 3 < t_end) ? f[3] : 0.0f;
        *reinterpret_cast<float4*>(cbuf + n * kCRow + 4 * g4) = cv;
      }
    }
    __syncthreads();
    // this thread's tokens inside [t_begin, t_end): j in [lo, nv)
    const int nv = (int)max((int64_t)0, min((int64_t)8, t_end - (tile + pg * 8)));
    const int lo = kVarlen ? (int)min((int64_t)8, max((int64_t)0, t_begin - (tile + pg * 8))) : 0;
    float fd[8], c[8];
    IO::to_f32(vd, fd);
    float run = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = fd[j] + bi;
      const float dl = a.softplus ? softplus_log2e(x) : x * kLog2e;
      run += (j >= lo && j < nv) ? dl : 0.0f;
      c[j] = run;   // inclusive within the piece
    }
    // exclusive prefix of the pieces' sums over the channel's 8 lanes
    float incl = run;
#pragma unroll
    for (int sh = 1; sh < 8; sh <<= 1) {
      const float o = __shfl_up(incl, sh, 8);
      if (pg >= sh) incl += o;
    }
    const float excl = incl - run;
    const float total = __shfl(incl, (lane & ~7) | 7);
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] += base + excl;
    base += total;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    unsigned long long alive = 0;   // this wave's lanes: states whose decay is still >= 2^-32
#pragma unroll 1
    for (int g = 0; g < NG; ++g) {
      float An[16], Hn[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 va = *reinterpret_cast<const float4*>(sA + pc * kSRow + 16 * g + 4 * q);
        const float4 vh = *reinterpret_cast<const float4*>(sH + pc * kSRow + 16 * g + 4 * q);
        An[4 * q] = va.x; An[4 * q + 1] = va.y; An[4 * q + 2] = va.z; An[4 * q + 3] = va.w;
        Hn[4 * q] = vh.x; Hn[4 * q + 1] = vh.y; Hn[4 * q + 2] = vh.z; Hn[4 * q + 3] = vh.w;
      }
#pragma unroll 4
      for (int n = 0; n < 16; ++n) {
        if (((live >> (16 * g + n)) & 1) == 0) continue;   // uniform over the workgroup
        const float* crow = cbuf + (16 * g + n) * kCRow + 8 * pg;
        const float4 c0 = *reinterpret_cast<const float4*>(crow);
        const float4 c1 = *reinterpret_cast<const float4*>(crow + 4);
        const float cn[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float P = __builtin_amdgcn_exp2f(An[n] * c[j]);   // exp(A cumDelta)
          acc[j] = fmaf(cn[j], P * Hn[n], acc[j]);
          if (j == 7) alive |= (__ballot(ch_ok && P >= 2.3283064e-10f) != 0 ? 1ull : 0ull) << (16 * g + n);
        }
      }
    }
    float fy[8], fz[8];
    if constexpr (kYf) {
      fy[0] = yf0.x; fy[1] = yf0.y; fy[2] = yf0.z; fy[3] = yf0.w;
      fy[4] = yf1.x; fy[5] = yf1.y; fy[6] = yf1.z; fy[7] = yf1.w;
    } else {
      IO::to_f32(vy, fy);
    }
    IO::to_f32(vz, fz);
#pragma unroll
    for (int j = 0; j < 8; ++j) fy[j] = fmaf(acc[j], gated ? silu(fz[j]) : 1.0f, fy[j]);
    if (nv == 8 && lo == 0) {
      IO::buf_store8(rs_y, off, IO::from_f32(fy), kVec);
    } else if (nv > lo && ch_ok) {
      IoT* py = gy + row0 + (int64_t)pc * a.seqlen + tile + pg * 8;
      if (lo == 0) {
        IO::store_n(py, IO::from_f32(fy), nv);
      } else {
        for (int j = lo; j < nv; ++j) IO::store1(py + j, fy[j]);
      }
    }
    if (may_stop) {
      // live_w is next written after the next tile's two barriers
      if (lane == 0) live_w[w] = alive;
      __syncthreads();
      unsigned long long al = 0;
#pragma unroll
      for (int i = 0; i < kFixNT / 64; ++i) al |= live_w[i];
      const uint32_t lo32 = __builtin_amdgcn_readfirstlane((uint32_t)al);
      const uint32_t hi32 = __builtin_amdgcn_readfirstlane((uint32_t)(al >> 32));
      live &= ((uint64_t)hi32 << 32) | lo32;
      if (live == 0) return true;   // no state needs correcting in the rest of the chunk
    }
    return false;
  };
  Ld ld;
  load(t_first, ld);
  for (int64_t tile = t_first; tile < t_end; tile += T)
    if (step(tile, ld)) break;
}

template <typename IoT, int NG, bool kVarlen>
void launch_fix(const FixArgs& f, bool vec, hipStream_t s) {
  if constexpr (!kVarlen) {
    if (f.yf32 != nullptr) {
      auto kern = vec ? fix_kernel<IoT, true, NG, false, true> : fix_kernel<IoT, false, NG, false, true>;
      hipLaunchKernelGGL(kern, dim3((unsigned)f.nwork), dim3(kFixNT), 0, s, f);
      return;
    }
  }
  auto kern = vec ? fix_kernel<IoT, true, NG, kVarlen, false> : fix_kernel<IoT, false, NG, kVarlen, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)f.nwork), dim3(kFixNT), 0, s, f);
}

// Fix-up launch for 16-state groups ng = 1..4.
template <typename IoT, bool kVarlen>
void launch_fix_ng(const FixArgs& f, int ng, bool vec, hipStream_t s) {
  switch (ng) {
    case 1: launch_fix<IoT, 1, kVarlen>(f, vec, s); break;
    case 2: launch_fix<IoT, 2, kVarlen>(f, vec, s); break;
    case 3: launch_fix<IoT, 3, kVarlen>(f, vec, s); break;
    default: launch_fix<IoT, 4, kVarlen>(f, vec, s); break;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Kernel pointer for a runtime (vec, mode) pair; Pick<IoT, kVec, kMode>::get() names the kernel.
template <template <typename, bool, int> class Pick, typename IoT>
auto pick_kernel(bool vec, int mode) {
  switch (mode) {
    case 1: return vec ? Pick<IoT, true, 1>::get() : Pick<IoT, false, 1>::get();
    case 2: return vec ? Pick<IoT, true, 2>::get() : Pick<IoT, false, 2>::get();
    case 3: return vec ? Pick<IoT, true, 3>::get() : Pick<IoT, false, 3>::get();
    default: return vec ? Pick<IoT, true, 0>::get() : Pick<IoT, false, 0>::get();
  }
}

}  // namespace
}  // namespace mscan
