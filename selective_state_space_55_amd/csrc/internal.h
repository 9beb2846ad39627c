// internal.h -- declarations shared by the library's own source files only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mscan {

// Forward-scan launch plan, chosen on the host from the sizes.
struct FwdPlan {
  int npw;            // states per lane (per wave): 2
  int nsplit;         // waves per workgroup
  int np;             // padded state count (16 per state group)
  int tile;           // tokens staged per workgroup iteration
  int64_t nchunks;    // time chunks scanned in parallel (1 = one pass)
  int64_t chunk_len;  // tokens per chunk, a multiple of tile
  int64_t nranges;    // ranges of range_tiles tiles per chunk: the chunk fix-up's work items
  int range_tiles;    // a power of two
  // two chunks of unequal length (a head of chunk_len tokens and the rest), launched chunk
  // by chunk: every head first, one per CU, then the tails on the CUs left over
  int head_tail;
  int64_t tail_tiles; // head/tail: the tail's tiles (its fp32 y rows are tail_tiles * tile long)
  size_t off_yf32;    // head/tail: byte offset of the tail's fp32 y in the workspace
  int64_t lp;         // seqlen rounded up to a multiple of tile
  int ngroups;        // 16-state passes (dstate > 16 runs several)
  size_t ws_carry;    // bytes of chunk carry (h_end / h_in) + chunk Delta sums
  size_t off_yacc;    // byte offset of the fp32 readout sum over state groups
  size_t ws_yacc;     // its bytes (0 when ngroups == 1)
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
  int euler;          // Bbar = Delta B (Euler) instead of the zero-order hold
  void* workspace;
  const int64_t* cu;  // variable-length batch: sequence offsets (nseq + 1), device; rows are (dim, seqlen)
  int64_t nseq;
  // fused causal conv1d (K = 4) + SiLU: u is the conv input; conv_w non-NULL turns it on
  const float* conv_w;       // (dim, 4)
  const float* conv_b;       // (dim) or NULL
  const void* conv_state;    // (batch, dim, 3) io or NULL
  void* u_out;               // (batch, dim, seqlen) io or NULL
};

hipError_t launch_fwd(const FwdArgs& a, const FwdPlan& p, hipStream_t stream);

// Variable-length batch: each sequence is cut into pieces of at most `piece`
// tokens, scanned like the time chunks of a row (aggregate pass, carry, output
// pass).  The pieces per sequence are counted on the device (the offsets are
// device memory), so launches cover the upper bound maxp.
struct VarlenPlan {
  int64_t piece;       // tokens per piece, a multiple of 64
  int64_t maxp;        // nseq + ceil(total / piece) >= the number of pieces
  int ngroups, np;     // 16-state groups, padded states
  size_t off_pstart;   // (nseq + 1) int64: first piece of each sequence, then the total
  size_t off_carry;    // (maxp, dim, np) fp32: piece aggregates, then the state entering each piece
  size_t off_dsum;     // (maxp, dim) fp32: sum of Delta*log2e over each piece
  size_t off_yacc;     // (dim, total) fp32 readout sum when dstate > 16
  size_t ws_total;
};
bool make_varlen_plan(int64_t nseq, int64_t dim, int64_t dstate, int64_t total, VarlenPlan* p);
// h0 / final_state are (nseq, dim, dstate)
hipError_t launch_fwd_varlen(const FwdArgs& a, const VarlenPlan& p, hipStream_t stream);

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
  int euler;
};

hipError_t launch_step(const StepArgs& a, hipStream_t stream);

// Backward pass: workspace layout (byte offsets, each part 256-byte aligned).
struct BwdPlan {
  int64_t ntile;      // 32-token tiles
  int64_t nsub;       // 8-token sub-chunks
  int64_t chgroups;   // 64-channel groups
  size_t off_ckpt;    // (batch, nsub, 16, dim) fp32: state before each sub-chunk
  size_t off_dB;      // (batch, 2 chgroups, 16 ngroups, seqlen) fp32: per-32-channel-group partial dB
  size_t off_dC;      // same for dC
  size_t off_dA;      // (batch, dim, 16 ngroups) fp32: per-row partial dA_log
  size_t off_dD;      // (batch, dim) fp32: per-row partial dD
  size_t off_dbias;   // (batch, dim) fp32: per-row partial ddelta_bias
  size_t off_acc;     // dstate > 16: 3 x (batch, dim, seqlen) fp32 running sums over state groups
  int ngroups;        // passes of 16 states
  size_t ws_total;
};

void make_bwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, BwdPlan* plan);

struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const float* h0;
  const void* dy;
  const float* dfs;   // gradient of the final state, or NULL
  void* du;
  void* ddelta;
  float* dA_log;
  void* dB;
  void* dC;
  float* dD;          // NULL: not written
  void* dz;           // written iff z is given
  float* dbias;       // NULL: not written
  float* dh0;         // NULL: not written
  int64_t batch, dim, dstate, seqlen;
  int io_bf16;
  int softplus;
  int euler;          // Bbar = Delta B (Euler) instead of the zero-order hold
  void* workspace;
};

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, hipStream_t stream);

struct ConvArgs {
  const void* x;
  const float* weight;     // (dim, K)
  const float* bias;       // (dim) or NULL
  const void* state_in;    // (batch, dim, K-1) io or NULL
  void* state_out;         // (batch, dim, K-1) io or NULL; may equal state_in
  void* u;
  int64_t batch, dim, seqlen, K;
  int io_bf16;
  int silu;
};

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);
// only the conv state update of launch_conv (state_out from x and state_in)
hipError_t launch_conv_state(const ConvArgs& a, hipStream_t stream);

// Multi-head SSM with a scalar decay per head (state-space-duality form), bf16 io.
struct SsdArgs {
  const void* x;          // (batch, L, H, P) bf16
  const void* dt;         // (batch, L, H) bf16
  const float* A_log;     // (H)
  const void* B;          // (batch, L, N) bf16
  const void* C;          // (batch, L, N) bf16
  const float* D;         // (H) or NULL
  const void* z;          // (batch, L, H, P) bf16 or NULL
  const float* dt_bias;   // (H) or NULL
  const float* h0;        // (batch, H, P, N) or NULL
  float* final_state;     // (batch, H, P, N) or NULL
  void* y;                // (batch, L, H, P) bf16
  int64_t batch, seqlen, nheads, headdim, dstate;
  int softplus, euler;
};

hipError_t launch_ssd(const SsdArgs& a, hipStream_t stream);

}  // namespace mscan
