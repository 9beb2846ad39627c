// api.hip -- C ABI of libmamba_scan (declared in include/mamba_scan.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime; a rejected call launches nothing and returns a status code.
#include <limits.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/mamba_scan.h"
#include "internal.h"

// ---- scratch for the allocation-free forward (mamba_scan_fwd_noalloc) ----
// One array per GPU: each device that loads the library holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory; the device address comes from hipGetSymbolAddress (see
// scratch_address), once per device with that device current, and only that
// address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MAMBA_SCAN_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// A launch of `blocks` workgroups of `threads` work-items: the dispatch's grid size
// counts work-items in 32 bits.
bool launch_ok(int64_t blocks, int64_t threads) {
  int64_t t;
  return blocks >= 0 && mul_ok(blocks, threads, &t) && t <= (int64_t)UINT32_MAX;
}

int check_common(int64_t batch, int64_t dim, int64_t dstate, int io_dtype) {
  if (io_dtype != MAMBA_SCAN_F32 && io_dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_DTYPE;
  if (batch < 1 || dim < 1 || dstate < 1) return MAMBA_SCAN_ERR_SHAPE;
  if (dstate > MAMBA_SCAN_MAX_DSTATE) return MAMBA_SCAN_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(batch, dim, &t) || !mul_ok(t, 64, &t)) return MAMBA_SCAN_ERR_SHAPE;
  return MAMBA_SCAN_OK;
}

int check_fwd_sizes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype) {
  int st = check_common(batch, dim, dstate, io_dtype);
  if (st != MAMBA_SCAN_OK) return st;
  if (seqlen < 0) return MAMBA_SCAN_ERR_SHAPE;
  // a workgroup addresses 64 rows of one tensor with 32-bit byte offsets
  const int64_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  if (seqlen > 0 && 64 * (seqlen + 8) * esz >= ((int64_t)1 << 31)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  int64_t t;
  // (batch*dim*(seqlen+64)*4 bytes must be representable)
  if (!mul_ok(batch * dim, seqlen + 64, &t) || !mul_ok(t, 16, &t)) return MAMBA_SCAN_ERR_SHAPE;
  return MAMBA_SCAN_OK;
}

// The forward's launches fit a dispatch: the scan (64-channel groups x time chunks, 512
// work-items), the chunk fix-up (16-channel groups x later chunks x ranges, 128), the carry fold and
// the state copy (one work-item per state).
bool fwd_launches_ok(int64_t batch, int64_t dim, int64_t dstate, const mscan::FwdPlan& p) {
  int64_t t;
  return mul_ok(batch, (dim + 63) / 64, &t) && mul_ok(t, p.nchunks, &t) && launch_ok(t, 512) &&
         mul_ok(batch, (dim + 15) / 16, &t) && mul_ok(t, p.nchunks - 1, &t) && mul_ok(t, p.nranges, &t) &&
         launch_ok(t, 128) &&
         mul_ok(batch * dim, dstate, &t) && launch_ok((t + 255) / 256, 256);
}

// Validation shared by the forward entry points: sizes, flags, pointers and the launch plan.
int check_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C, const float* D,
              const void* z, const float* delta_bias, const float* initial_state, const float* final_state,
              const void* y, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype, int flags,
              int64_t nchunks, int states_per_wave, mscan::FwdPlan* plan) {
  int st = check_fwd_sizes(batch, dim, dstate, seqlen, io_dtype);
  if (st != MAMBA_SCAN_OK) return st;
  if (flags & ~(MAMBA_SCAN_FLAG_SOFTPLUS | MAMBA_SCAN_FLAG_EULER)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  // tensors with a seqlen dimension are zero-sized when seqlen == 0 and may then be NULL
  if (!A_log) return MAMBA_SCAN_ERR_NULL;
  if (seqlen > 0 && (!u || !delta || !B || !C || !y)) return MAMBA_SCAN_ERR_NULL;
  const size_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  const void* io_ptrs[] = {u, delta, B, C, z, y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, esz)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {A_log, D, delta_bias, initial_state, final_state};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  if (!mscan::make_fwd_plan(batch, dim, dstate, seqlen, nchunks, states_per_wave, plan))
    return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!fwd_launches_ok(batch, dim, dstate, *plan)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  return MAMBA_SCAN_OK;
}

int run_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C, const float* D,
            const void* z, const float* delta_bias, const float* initial_state, float* final_state, void* y,
            int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype, int flags,
            const mscan::FwdPlan& plan, void* workspace, void* stream) {
  mscan::FwdArgs a{};
  a.u = u; a.delta = delta; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.h0 = initial_state; a.final_state = final_state; a.y = y;
  a.batch = batch; a.dim = dim; a.dstate = dstate; a.seqlen = seqlen;
  a.io_bf16 = io_dtype == MAMBA_SCAN_BF16;
  a.softplus = (flags & MAMBA_SCAN_FLAG_SOFTPLUS) != 0;
  a.euler = (flags & MAMBA_SCAN_FLAG_EULER) != 0;
  a.workspace = workspace;
  hipError_t e = mscan::launch_fwd(a, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

// The device address of this GPU's copy of `scratch` (below), looked up once
// per device with that device current.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr || !aligned(p, 256)) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* mamba_scan_status_str(int status) {
  switch (status) {
    case MAMBA_SCAN_OK: return "ok";
    case MAMBA_SCAN_ERR_NULL: return "a required pointer is NULL";
    case MAMBA_SCAN_ERR_SHAPE: return "a size is out of range";
    case MAMBA_SCAN_ERR_DTYPE: return "io_dtype is not MAMBA_SCAN_F32 or MAMBA_SCAN_BF16";
    case MAMBA_SCAN_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case MAMBA_SCAN_ERR_UNSUPPORTED: return "unsupported option (a size past a documented limit, an unknown flag or an invalid tuning knob)";
    case MAMBA_SCAN_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case MAMBA_SCAN_ERR_HIP: return "the HIP runtime reported an error";
    default: return "unknown status";
  }
}

int mamba_scan_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

size_t mamba_scan_fwd_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                                        int64_t nchunks, int states_per_wave) {
  if (check_fwd_sizes(batch, dim, dstate, seqlen, io_dtype) != MAMBA_SCAN_OK) return (size_t)-1;
  mscan::FwdPlan p;
  if (!mscan::make_fwd_plan(batch, dim, dstate, seqlen, nchunks, states_per_wave, &p)) return (size_t)-1;
  return p.ws_total;
}

size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype) {
  return mamba_scan_fwd_workspace_size_ex(batch, dim, dstate, seqlen, io_dtype, 0, 0);
}

int mamba_scan_fwd_ex(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                      const float* D, const void* z, const float* delta_bias, const float* initial_state,
                      float* final_state, void* y, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                      int io_dtype, int flags, int64_t nchunks, int states_per_wave, void* workspace,
                      size_t workspace_bytes, void* stream) {
  mscan::FwdPlan plan;
  int st = check_fwd(u, delta, A_log, B, C, D, z, delta_bias, initial_state, final_state, y, batch, dim, dstate,
                     seqlen, io_dtype, flags, nchunks, states_per_wave, &plan);
  if (st != MAMBA_SCAN_OK) return st;
  if (plan.ws_total > 0) {
    if (!workspace || workspace_bytes < plan.ws_total || !aligned(workspace, 256)) return MAMBA_SCAN_ERR_WORKSPACE;
  }
  return run_fwd(u, delta, A_log, B, C, D, z, delta_bias, initial_state, final_state, y, batch, dim, dstate,
                 seqlen, io_dtype, flags, plan, workspace, stream);
}

int mamba_scan_fwd_noalloc(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, const float* initial_state,
                           float* final_state, void* y, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                           int io_dtype, int flags, void* stream) {
  mscan::FwdPlan plan;
  int st = check_fwd(u, delta, A_log, B, C, D, z, delta_bias, initial_state, final_state, y, batch, dim, dstate,
                     seqlen, io_dtype, flags, 0, 0, &plan);
  if (st != MAMBA_SCAN_OK) return st;
  if (plan.ws_total > (size_t)MAMBA_SCAN_NOALLOC_SCRATCH_BYTES) return MAMBA_SCAN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_total > 0) {
    // everything in the scratch is written before it is read within one call (chunk
    // aggregates, then the carry; the first state group's readout sum), so nothing is cleared
    if (scratch_address(&ws) != hipSuccess) return MAMBA_SCAN_ERR_HIP;
  }
  return run_fwd(u, delta, A_log, B, C, D, z, delta_bias, initial_state, final_state, y, batch, dim, dstate,
                 seqlen, io_dtype, flags, plan, ws, stream);
}

int mamba_scan_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const float* initial_state,
                   float* final_state, void* y, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                   int io_dtype, int flags, void* workspace, size_t workspace_bytes, void* stream) {
  return mamba_scan_fwd_ex(u, delta, A_log, B, C, D, z, delta_bias, initial_state, final_state, y, batch, dim,
                           dstate, seqlen, io_dtype, flags, 0, 0, workspace, workspace_bytes, stream);
}

int mamba_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias, const void* conv_state_in,
                        void* conv_state_out, const void* delta, const float* A_log, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, const float* initial_state,
                        float* final_state, void* u_out, void* y, int64_t batch, int64_t dim, int64_t dstate,
                        int64_t seqlen, int io_dtype, int flags, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_fwd_sizes(batch, dim, dstate, seqlen, io_dtype);
  if (st != MAMBA_SCAN_OK) return st;
  if (dstate > 16) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (flags & ~(MAMBA_SCAN_FLAG_SOFTPLUS | MAMBA_SCAN_FLAG_EULER)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!A_log || !conv_weight) return MAMBA_SCAN_ERR_NULL;
  if (seqlen > 0 && (!x || !delta || !B || !C || !y)) return MAMBA_SCAN_ERR_NULL;
  const size_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  const void* io_ptrs[] = {x, delta, B, C, z, y, u_out, conv_state_in, conv_state_out};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, esz)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {A_log, D, delta_bias, initial_state, final_state, conv_weight, conv_bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  mscan::FwdPlan plan;
  if (!mscan::make_fwd_plan(batch, dim, dstate, seqlen, 0, 0, &plan)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!fwd_launches_ok(batch, dim, dstate, plan)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (plan.ws_total > 0) {
    if (!workspace || workspace_bytes < plan.ws_total || !aligned(workspace, 256)) return MAMBA_SCAN_ERR_WORKSPACE;
  }
  mscan::FwdArgs a{};
  a.u = x; a.delta = delta; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.h0 = initial_state; a.final_state = final_state; a.y = y;
  a.batch = batch; a.dim = dim; a.dstate = dstate; a.seqlen = seqlen;
  a.io_bf16 = io_dtype == MAMBA_SCAN_BF16;
  a.softplus = (flags & MAMBA_SCAN_FLAG_SOFTPLUS) != 0;
  a.euler = (flags & MAMBA_SCAN_FLAG_EULER) != 0;
  a.workspace = workspace;
  a.conv_w = conv_weight; a.conv_b = conv_bias; a.conv_state = conv_state_in; a.u_out = u_out;
  hipError_t e = mscan::launch_fwd(a, plan, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && conv_state_out) {
    // after the scan, which reads conv_state_in (the two may be the same buffer)
    mscan::ConvArgs c{};
    c.x = x; c.state_in = conv_state_in; c.state_out = conv_state_out;
    c.batch = batch; c.dim = dim; c.seqlen = seqlen; c.K = 4; c.io_bf16 = a.io_bf16;
    e = mscan::launch_conv_state(c, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

size_t mamba_scan_fwd_varlen_workspace_size(int64_t nseq, int64_t dim, int64_t dstate, int64_t total_len,
                                            int io_dtype) {
  if (nseq < 1) return (size_t)-1;
  if (check_fwd_sizes(1, dim, dstate, total_len, io_dtype) != MAMBA_SCAN_OK) return (size_t)-1;
  mscan::VarlenPlan p;
  if (!mscan::make_varlen_plan(nseq, dim, dstate, total_len, &p)) return (size_t)-1;
  return p.ws_total;
}

int mamba_scan_fwd_varlen(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, const int64_t* cu_seqlens,
                          const float* initial_states, float* final_states, void* y, int64_t nseq, int64_t dim,
                          int64_t dstate, int64_t total_len, int io_dtype, int flags, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (nseq < 1) return MAMBA_SCAN_ERR_SHAPE;
  int st = check_fwd_sizes(1, dim, dstate, total_len, io_dtype);
  if (st != MAMBA_SCAN_OK) return st;
  if (flags & ~(MAMBA_SCAN_FLAG_SOFTPLUS | MAMBA_SCAN_FLAG_EULER)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  mscan::VarlenPlan plan;
  if (!mscan::make_varlen_plan(nseq, dim, dstate, total_len, &plan)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  int64_t t;
  // grid sizes: the scan's (piece, 64-channel group) items of 512 work-items, the fix-up's
  // (piece, 16-channel group) items of 128
  if (!mul_ok(plan.maxp, (dim + 63) / 64, &t) || !launch_ok(t, 512)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!mul_ok(plan.maxp, (dim + 15) / 16, &t) || !launch_ok(t, 128)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!mul_ok(nseq, dim * dstate, &t) || t > INT32_MAX) return MAMBA_SCAN_ERR_UNSUPPORTED;   // carry threads
  if (!A_log || !cu_seqlens) return MAMBA_SCAN_ERR_NULL;
  if (total_len > 0 && (!u || !delta || !B || !C || !y)) return MAMBA_SCAN_ERR_NULL;
  const size_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  const void* io_ptrs[] = {u, delta, B, C, z, y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, esz)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {A_log, D, delta_bias, initial_states, final_states};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  if (!aligned(cu_seqlens, 8)) return MAMBA_SCAN_ERR_ALIGN;
  if (!workspace || workspace_bytes < plan.ws_total || !aligned(workspace, 256)) return MAMBA_SCAN_ERR_WORKSPACE;
  mscan::FwdArgs a{};
  a.u = u; a.delta = delta; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.h0 = initial_states; a.final_state = final_states; a.y = y;
  a.batch = 1; a.dim = dim; a.dstate = dstate; a.seqlen = total_len;
  a.io_bf16 = io_dtype == MAMBA_SCAN_BF16;
  a.softplus = (flags & MAMBA_SCAN_FLAG_SOFTPLUS) != 0;
  a.euler = (flags & MAMBA_SCAN_FLAG_EULER) != 0;
  a.workspace = workspace;
  a.cu = cu_seqlens;
  a.nseq = nseq;
  hipError_t e = mscan::launch_fwd_varlen(a, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

int mamba_scan_step(float* state, const void* x, const void* dt, const float* A_log, const void* B, const void* C,
                    const float* D, const void* z, const float* dt_bias, int flags, void* y, int64_t batch,
                    int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  int st = check_common(batch, dim, dstate, io_dtype);
  if (st != MAMBA_SCAN_OK) return st;
  if ((batch + 3) / 4 > 65535) return MAMBA_SCAN_ERR_UNSUPPORTED;   // grid rows of four batch rows
  // a grid row's work-items: 4, 8 or 16 lanes per channel
  if (!launch_ok((dim * (dstate <= 16 ? 4 : dstate <= 32 ? 8 : 16) + 255) / 256, 256)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (flags & ~(MAMBA_SCAN_FLAG_SOFTPLUS | MAMBA_SCAN_FLAG_EULER)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!state || !x || !dt || !A_log || !B || !C || !y) return MAMBA_SCAN_ERR_NULL;
  const size_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  const void* io_ptrs[] = {x, dt, B, C, z, y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, esz)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {state, A_log, D, dt_bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  mscan::StepArgs a{};
  a.state = state; a.x = x; a.dt = dt; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = dt_bias;
  a.y = y; a.batch = batch; a.dim = dim; a.dstate = dstate; a.io_bf16 = io_dtype == MAMBA_SCAN_BF16;
  a.softplus = (flags & MAMBA_SCAN_FLAG_SOFTPLUS) != 0;
  a.euler = (flags & MAMBA_SCAN_FLAG_EULER) != 0;
  hipError_t e = mscan::launch_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype) {
  if (check_fwd_sizes(batch, dim, dstate, seqlen, io_dtype) != MAMBA_SCAN_OK) return (size_t)-1;
  if (dstate > MAMBA_SCAN_MAX_DSTATE_BWD) return (size_t)-1;
  mscan::BwdPlan p;
  mscan::make_bwd_plan(batch, dim, dstate, seqlen, &p);
  return p.ws_total;
}

int mamba_scan_bwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const float* initial_state,
                   const void* dy, const float* d_final_state, void* du, void* ddelta, float* dA_log, void* dB,
                   void* dC, float* dD, void* dz, float* ddelta_bias, float* d_initial_state, int64_t batch,
                   int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype, int flags, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_fwd_sizes(batch, dim, dstate, seqlen, io_dtype);
  if (st != MAMBA_SCAN_OK) return st;
  if (flags & ~(MAMBA_SCAN_FLAG_SOFTPLUS | MAMBA_SCAN_FLAG_EULER)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (dstate > MAMBA_SCAN_MAX_DSTATE_BWD) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!A_log || !dA_log) return MAMBA_SCAN_ERR_NULL;
  if (seqlen > 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta || !dB || !dC)) return MAMBA_SCAN_ERR_NULL;
  if (seqlen > 0 && z && !dz) return MAMBA_SCAN_ERR_NULL;
  const size_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  const void* io_ptrs[] = {u, delta, B, C, z, dy, du, ddelta, dB, dC, dz};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, esz)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {A_log, D, delta_bias, initial_state, d_final_state, dA_log, dD, ddelta_bias, d_initial_state};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  mscan::BwdPlan plan;
  mscan::make_bwd_plan(batch, dim, dstate, seqlen, &plan);
  {
    // launches: checkpoint and gradient passes (64-channel groups, 512 work-items), the dB/dC
    // reduction (one per (batch, state, token)), the parameter reduction
    int64_t t, t2;
    if (!mul_ok(batch, (dim + 63) / 64, &t) || !launch_ok(t, 512) || !mul_ok(batch * dstate, seqlen, &t2) ||
        !launch_ok((t2 + 255) / 256, 256) || !launch_ok((dim * dstate + 255) / 256, 256))
      return MAMBA_SCAN_ERR_UNSUPPORTED;
  }
  if (plan.ws_total > 0) {
    if (!workspace || workspace_bytes < plan.ws_total || !aligned(workspace, 256)) return MAMBA_SCAN_ERR_WORKSPACE;
  }
  mscan::BwdArgs a{};
  a.u = u; a.delta = delta; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.h0 = initial_state; a.dy = dy; a.dfs = d_final_state;
  a.du = du; a.ddelta = ddelta; a.dA_log = dA_log; a.dB = dB; a.dC = dC; a.dD = dD; a.dz = dz;
  a.dbias = ddelta_bias; a.dh0 = d_initial_state;
  a.batch = batch; a.dim = dim; a.dstate = dstate; a.seqlen = seqlen;
  a.io_bf16 = io_dtype == MAMBA_SCAN_BF16;
  a.softplus = (flags & MAMBA_SCAN_FLAG_SOFTPLUS) != 0;
  a.euler = (flags & MAMBA_SCAN_FLAG_EULER) != 0;
  a.workspace = workspace;
  hipError_t e = mscan::launch_bwd(a, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

int mamba_ssd_fwd(const void* x, const void* dt, const float* A_log, const void* B, const void* C, const float* D,
                  const void* z, const float* dt_bias, const float* initial_state, float* final_state, void* y,
                  int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype,
                  int flags, void* stream) {
  if (io_dtype != MAMBA_SCAN_F32 && io_dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_DTYPE;
  if (batch < 1 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1) return MAMBA_SCAN_ERR_SHAPE;
  if (io_dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_UNSUPPORTED;              // bf16 operands only
  if (headdim % 32 != 0 || headdim > 256 || (dstate != 64 && dstate != 128)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (flags & ~(MAMBA_SCAN_FLAG_SOFTPLUS | MAMBA_SCAN_FLAG_EULER)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  int64_t t;
  // grid: at most headdim / 32 slices per head, at most 1024 work-items each
  if (!mul_ok(batch, nheads * (headdim / 32), &t) || !launch_ok(t, 1024)) return MAMBA_SCAN_ERR_UNSUPPORTED;
  // a chunk's 64 token rows of x / y (nheads * headdim bf16 each) are addressed with 32-bit offsets
  if (nheads > (1 << 24) / headdim) return MAMBA_SCAN_ERR_UNSUPPORTED;
  if (!mul_ok(t, seqlen, &t) || !mul_ok(t, headdim * 2, &t)) return MAMBA_SCAN_ERR_SHAPE;
  if (!A_log) return MAMBA_SCAN_ERR_NULL;
  if (seqlen > 0 && (!x || !dt || !B || !C || !y)) return MAMBA_SCAN_ERR_NULL;
  const void* v16[] = {x, B, C, z, y, initial_state, final_state};   // 16-byte vector accesses
  for (const void* p : v16)
    if (p && !aligned(p, 16)) return MAMBA_SCAN_ERR_ALIGN;
  if (dt && !aligned(dt, 2)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {A_log, D, dt_bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  mscan::SsdArgs a{};
  a.x = x; a.dt = dt; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z; a.dt_bias = dt_bias;
  a.h0 = initial_state; a.final_state = final_state; a.y = y;
  a.batch = batch; a.seqlen = seqlen; a.nheads = nheads; a.headdim = headdim; a.dstate = dstate;
  a.softplus = (flags & MAMBA_SCAN_FLAG_SOFTPLUS) != 0;
  a.euler = (flags & MAMBA_SCAN_FLAG_EULER) != 0;
  hipError_t e = mscan::launch_ssd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

int mamba_conv1d_fwd(const void* x, const float* weight, const float* bias, const void* conv_state_in,
                     void* conv_state_out, void* u, int64_t batch, int64_t dim, int64_t seqlen, int64_t kernel_size,
                     int io_dtype, int silu, void* stream) {
  if (io_dtype != MAMBA_SCAN_F32 && io_dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_DTYPE;
  if (batch < 1 || dim < 1 || seqlen < 0) return MAMBA_SCAN_ERR_SHAPE;
  if (kernel_size < 1 || kernel_size > 4) return MAMBA_SCAN_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(batch, dim, &t) || !mul_ok(t, seqlen + 8, &t) || !mul_ok(t, 4, &t)) return MAMBA_SCAN_ERR_SHAPE;
  if (!weight) return MAMBA_SCAN_ERR_NULL;
  if (seqlen > 0 && (!x || !u)) return MAMBA_SCAN_ERR_NULL;
  const size_t esz = io_dtype == MAMBA_SCAN_BF16 ? 2 : 4;
  const void* io_ptrs[] = {x, u, conv_state_in, conv_state_out};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, esz)) return MAMBA_SCAN_ERR_ALIGN;
  const void* f_ptrs[] = {weight, bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return MAMBA_SCAN_ERR_ALIGN;
  mscan::ConvArgs a{};
  a.x = x; a.weight = weight; a.bias = bias; a.state_in = conv_state_in; a.state_out = conv_state_out; a.u = u;
  a.batch = batch; a.dim = dim; a.seqlen = seqlen; a.K = kernel_size;
  a.io_bf16 = io_dtype == MAMBA_SCAN_BF16;
  a.silu = silu != 0;
  hipError_t e = mscan::launch_conv(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_HIP;
}

}  // extern "C"
