// scan_fwd_varlen.hip -- forward selective scan over a variable-length batch:
// nseq sequences packed one after another along the time axis of a single
// row per channel, sequence s on tokens [cu[s], cu[s+1]), each scanned from its
// own initial state with its own final state.  (The pages define the scan of
// one sequence -- Mamba notes, awesome.papernotes.org, 设计 1 and 设计 2; State
// space models and Mamba, jonathanding.github.io, §3 -- and packing unequal
// lengths without padding restarts the recurrence at every sequence start.)
//
// It runs the two-states-per-lane kernel with work items (sequence, 64-channel
// group); see scan_fwd_h2.h.  No time chunking: a long sequence is one work
// item per channel group, so the parallelism is nseq x channel groups.
#include "scan_fwd_h2.h"

namespace mscan {
namespace {

template <bool kMulti>
struct PickVarlen {
  template <typename IoT, bool kAgg, bool kVec, int kMode>
  struct P {
    static auto get() { return scan_fwd_h2_kernel<IoT, false, kVec, kMode, kMulti, true>; }
  };
};

template <typename IoT>
hipError_t run_varlen(const FwdArgs& a, const FwdPlan& p, hipStream_t s) {
  const size_t esz = sizeof(IoT);
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a.u) | reinterpret_cast<uintptr_t>(a.delta) |
                        reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.z) |
                        reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.C);
  const bool vec = ((mis & 15) == 0) && ((a.seqlen * (int64_t)esz) % 16 == 0);
  KArgs k{};
  k.u = a.u; k.delta = a.delta; k.A_log = a.A_log; k.B = a.B; k.C = a.C; k.D = a.D; k.z = a.z; k.bias = a.bias;
  k.h0 = a.h0; k.final_state = a.final_state; k.y = a.y; k.cu = a.cu;
  k.dim = a.dim; k.seqlen = a.seqlen; k.chunk_len = a.seqlen; k.nchunks = 1;
  k.chgroups = (a.dim + kCh - 1) / kCh;
  k.dstate = (int)a.dstate; k.np = p.np;
  k.mode = (a.softplus ? kModeSoftplus : 0) | (a.euler ? kModeEuler : 0);
  k.gated = a.z != nullptr;
  k.nwork = a.nseq * k.chgroups;
  const int ng = p.ngroups;
  k.yacc = ng > 1 ? reinterpret_cast<float*>(static_cast<char*>(a.workspace) + p.off_yacc) : nullptr;
  const size_t lds = sizeof(float) * LdsH2::floats(false);
  for (int g = 0; g < ng; ++g) {
    k.n0 = 16 * g;
    k.acc = ng == 1 ? 0 : (g == 0 ? 1 : (g == ng - 1 ? 3 : 2));
    auto kern = k.acc ? pick_kernel<PickVarlen<true>::template P, IoT, false>(vec, k.mode)
                      : pick_kernel<PickVarlen<false>::template P, IoT, false>(vec, k.mode);
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)k.nwork), dim3(512), lds, s, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_varlen(const FwdArgs& a, const FwdPlan& p, hipStream_t stream) {
  return a.io_bf16 ? run_varlen<uint16_t>(a, p, stream) : run_varlen<float>(a, p, stream);
}

}  // namespace mscan
