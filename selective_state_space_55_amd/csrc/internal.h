// internal.h -- declarations shared by the library's own source files only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mscan {

// Forward-scan launch plan, chosen on the host from the sizes.
struct FwdPlan {
  int npw;            // states per lane (per wave): 2 or 4
  int nsplit;         // waves per workgroup = padded states / npw (power of two)
  int np;             // padded state count = nsplit * npw
  int tile;           // tokens staged per workgroup iteration
  int64_t nchunks;    // time chunks scanned in parallel (1 = one pass)
  int64_t chunk_len;  // tokens per chunk, a multiple of tile
  int64_t lp;         // seqlen rounded up to a multiple of tile
  size_t ws_bc;       // bytes of packed fp32 B/C
  size_t ws_carry;    // bytes of chunk carry (h_end / h_in) + chunk Delta sums
  size_t ws_total;
};

// Returns false if the explicit knobs are invalid for these sizes.
bool make_fwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t nchunks_req,
                   int npw_req, FwdPlan* plan);

struct FwdArgs {
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
  int64_t batch, dim, dstate, seqlen;
  int io_bf16;
  int softplus;
  void* workspace;
};

hipError_t launch_fwd(const FwdArgs& a, const FwdPlan& p, hipStream_t stream);

struct StepArgs {
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
  int64_t batch, dim, dstate;
  int io_bf16;
  int softplus;
};

hipError_t launch_step(const StepArgs& a, hipStream_t stream);

}  // namespace mscan
