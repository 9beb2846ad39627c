// scan_fwd_varlen.hip -- forward selective scan over a variable-length batch:
// nseq sequences packed one after another along the time axis of a single
// row per channel, sequence s on tokens [cu[s], cu[s+1]), each scanned from its
// own initial state with its own final state.  (The pages define the scan of
// one sequence -- Mamba notes, awesome.papernotes.org, 设计 1 and 设计 2; State
// space models and Mamba, jonathanding.github.io, §3 -- and packing unequal
// lengths without padding restarts the recurrence at every sequence start.)
//
// A sequence is cut into pieces of at most `piece` tokens, which are scanned
// as the time chunks of a fixed-length row are (the associative combine of
// the pages' parallel scan, applied between pieces): every piece is scanned at
// once -- a sequence's first from its initial state, the others from zero --
// leaving its end state and sum of Delta; a carry kernel folds them in order
// per sequence, and the fix-up kernel adds each later piece's carried-in part
// to its outputs.  Work items are (piece, 64-channel group), so one long
// sequence still fills the GPU.  The offsets are device memory: a
// one-workgroup kernel counts the pieces of each sequence (prefix sums) and
// the passes launch over an upper bound, with work items past the last piece
// exiting at once.  The scan kernel is the two-states-per-lane kernel of
// scan_fwd_h2.h.
#include "scan_fwd_h2.h"

namespace mscan {
namespace {

constexpr int64_t kPiece = 2048;   // tokens per piece (32 tiles)

// pstart[s] = number of pieces of sequences 0 .. s-1 (each has at least one,
// empty sequences included, so every sequence gets its final state), and
// pstart[nseq] = the total.  Offsets are clamped as the scan kernel clamps them.
__global__ __launch_bounds__(1024) void varlen_plan_kernel(const int64_t* __restrict__ cu, int64_t nseq,
                                                           int64_t total, int64_t piece, int64_t* __restrict__ pstart) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  int64_t run = 0;
  for (int64_t base = 0; base < nseq; base += 1024) {
    const int64_t s = base + tid;
    int64_t cnt = 0;
    if (s < nseq) {
      const int64_t b = min(max(cu[s], (int64_t)0), total);
      const int64_t e = min(max(cu[s + 1], b), total);
      cnt = max((int64_t)1, (e - b + piece - 1) / piece);
    }
    part[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan
      const int64_t v = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    if (s < nseq) pstart[s] = run + part[tid] - cnt;
    run += part[1023];
    __syncthreads();
  }
  if (tid == 0) pstart[nseq] = run;
}

// Per (sequence, channel, state): folds the sequence's pieces in order.  Its
// first piece ran from the initial state (its end state is exact); piece k > 0
// ran from zero and left h_end(k) and its sum of Delta*log2e.  Leaves in
// carry[piece k] the state entering piece k and writes the sequence's final
// state.  Pieces at or past maxp (possible only for offsets that are not
// non-decreasing) were not scanned and are not touched.
__global__ __launch_bounds__(256) void varlen_carry_kernel(float* __restrict__ carry, const float* __restrict__ dsum,
                                                           const float* __restrict__ A_log,
                                                           float* __restrict__ final_states,
                                                           const int64_t* __restrict__ pstart, int64_t nseq,
                                                           int64_t dim, int dstate, int np, int64_t maxp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nseq * dim * dstate) return;
  const int n = (int)(i % dstate);
  const int64_t sd = i / dstate;
  const int64_t d = sd % dim;
  const int64_t s = sd / dim;
  const int64_t p0 = pstart[s];
  const int64_t p1 = min(pstart[s + 1], maxp);
  if (p1 <= p0) return;
  const float An = -expf(A_log[d * dstate + n]);
  float h = carry[(p0 * dim + d) * np + n];
  for (int64_t k = p0 + 1; k < p1; ++k) {
    float* slot = carry + (k * dim + d) * np + n;
    const float hend = *slot;
    *slot = h;
    const float P = exp2f(An * dsum[k * dim + d]);   // decay over piece k: exp(A * sum Delta)
    h = fmaf(P, h, hend);
  }
  if (final_states) final_states[sd * dstate + n] = h;
}

template <bool kMulti>
struct PickVarlen {
  template <typename IoT, bool kVec, int kMode>
  struct P {
    static auto get() { return scan_fwd_h2_kernel<IoT, kVec, kMode, kMulti, true>; }
  };
};

template <typename IoT>
hipError_t run_varlen(const FwdArgs& a, const VarlenPlan& p, hipStream_t s) {
  const size_t esz = sizeof(IoT);
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a.u) | reinterpret_cast<uintptr_t>(a.delta) |
                        reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.z) |
                        reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.C);
  const bool vec = ((mis & 15) == 0) && ((a.seqlen * (int64_t)esz) % 16 == 0);
  char* ws = static_cast<char*>(a.workspace);
  int64_t* pstart = reinterpret_cast<int64_t*>(ws + p.off_pstart);
  KArgs k{};
  k.u = a.u; k.delta = a.delta; k.A_log = a.A_log; k.B = a.B; k.C = a.C; k.D = a.D; k.z = a.z; k.bias = a.bias;
  k.h0 = a.h0; k.final_state = a.final_state; k.y = a.y; k.cu = a.cu;
  k.pstart = pstart; k.nseq = a.nseq;
  k.carry = reinterpret_cast<float*>(ws + p.off_carry);
  k.dsum = reinterpret_cast<float*>(ws + p.off_dsum);
  k.dim = a.dim; k.seqlen = a.seqlen; k.chunk_len = p.piece; k.nchunks = 1;
  k.chgroups = (a.dim + kCh - 1) / kCh;
  k.dstate = (int)a.dstate; k.np = p.np;
  k.mode = (a.softplus ? kModeSoftplus : 0) | (a.euler ? kModeEuler : 0);
  k.gated = a.z != nullptr;
  k.nwork = p.maxp * k.chgroups;
  const int ng = p.ngroups;
  k.yacc = ng > 1 ? reinterpret_cast<float*>(ws + p.off_yacc) : nullptr;
  const size_t lds = sizeof(float) * LdsH2::floats();

  hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(1024), 0, s, a.cu, a.nseq, a.seqlen, p.piece, pstart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int g = 0; g < ng; ++g) {
    k.n0 = 16 * g;
    k.acc = ng == 1 ? 0 : (g == 0 ? 1 : (g == ng - 1 ? 3 : 2));
    auto kern = k.acc ? pick_kernel<PickVarlen<true>::template P, IoT>(vec, k.mode)
                      : pick_kernel<PickVarlen<false>::template P, IoT>(vec, k.mode);
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)k.nwork), dim3(512), lds, s, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nthr = a.nseq * a.dim * a.dstate;
  hipLaunchKernelGGL(varlen_carry_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, s, k.carry, k.dsum,
                     a.A_log, a.final_state, pstart, a.nseq, a.dim, (int)a.dstate, p.np, p.maxp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  FixArgs f{};
  f.cu = a.cu; f.pstart = pstart; f.nseq = a.nseq;
  f.delta = a.delta; f.bias = a.bias; f.A_log = a.A_log; f.C = a.C; f.z = a.z; f.y = a.y; f.carry = k.carry;
  f.dim = a.dim; f.seqlen = a.seqlen; f.chunk_len = p.piece; f.nchunks = 1;
  f.chgroups = (a.dim + kFixCh - 1) / kFixCh;   // the fix-up's narrower channel groups
  f.rsum = nullptr; f.nranges = 1;               // a piece is one range
  f.range_len = p.piece;
  f.nwork = p.maxp * f.chgroups; f.dstate = (int)a.dstate; f.np = p.np; f.softplus = a.softplus;
  launch_fix_ng<IoT, true>(f, ng, vec, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

bool make_varlen_plan(int64_t nseq, int64_t dim, int64_t dstate, int64_t total, VarlenPlan* p) {
  if (nseq < 1 || dim < 1 || dstate < 1 || dstate > 64 || total < 0) return false;
  p->piece = kPiece;
  p->maxp = nseq + (total + kPiece - 1) / kPiece;
  p->ngroups = (int)((dstate + 15) / 16);
  p->np = 16 * p->ngroups;
  size_t off = 0;
  p->off_pstart = off;
  off += align256(sizeof(int64_t) * (size_t)(nseq + 1));
  p->off_carry = off;
  off += align256(sizeof(float) * (size_t)(p->maxp * dim * p->np));
  p->off_dsum = off;
  off += align256(sizeof(float) * (size_t)(p->maxp * dim));
  p->off_yacc = off;
  if (p->ngroups > 1) off += align256(sizeof(float) * (size_t)(dim * total));
  p->ws_total = off;
  return true;
}

hipError_t launch_fwd_varlen(const FwdArgs& a, const VarlenPlan& p, hipStream_t stream) {
  return a.io_bf16 ? run_varlen<uint16_t>(a, p, stream) : run_varlen<float>(a, p, stream);
}

}  // namespace mscan
