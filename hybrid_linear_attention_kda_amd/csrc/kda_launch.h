// Internal launch interface between the C ABI (kda_abi.cpp) and the kernels.
// Not part of the public ABI: the public declarations live in include/kda.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kMaxConvWidth = 8;       // conv taps supported (W - 1 <= 7 raw inputs of state)
constexpr int kRollbackBatch = 256;    // sequences per rollback launch (accepted counts ride in the args)
constexpr int kVarlenBatch = 128;      // sequences per variable-length prefill launch (their table rides in the args)
constexpr int kVarlenGroups = 64;      // sequence groups of a launch's matrix-core state pass

enum IoType { kF32 = 0, kBF16 = 1 };

// Arguments shared by the recurrent (decode / verify) kernels and the prefill kernels.
struct LayerArgs {
  int B, T, H, D, W;
  int gate;             // 0: bounded sigmoid with bound lb; 1: softplus branch (lb unused)
  float lb, l2_eps, rms_eps, scale;
  const void* qkv;      // [B, T, 3*H*D] io
  const void* f;        // [B, T, H*D] io
  const void* beta;     // [B, T, H] io
  const void* g_out;    // [B, T, H*D] io
  const void* conv_w;   // [3*H*D, W] io
  const float* A_log;   // [H]
  const float* dt_bias; // [H*D]
  const void* norm_w;   // [D] io
  const float* state_in;
  float* state_out;     // decode / prefill: [B, H, D, D] (may alias state_in); verify: snapshots [B, T, H, D, D]
  const void* conv_in;  // [B, 3*H*D, W-1] io
  void* conv_out;       // may alias conv_in; nullptr: conv state not written (verify)
  void* out;            // [B, T, H*D] out type
  int snapshots;        // 1: write the state after every token to state_out (verify)
  float* tape;          // verify with a replay tape: [B, T, H, 3, D] = (alpha, k, u) per token and
                        // head, written instead of any state (state_out unused); nullptr otherwise
};

// The sequences of one prefill launch.  n == 0: a.B sequences of a.T tokens each (sequence b at
// packed tokens b*T.., chunk blocks b*NC.., state and conv-state slot b).  n > 0: the n sequences
// of the table, each of length >= 1, packed along the token axis.
struct SeqTab {
  int n;
  int total_chunks;                // sum over the table of ceil(len / 64) (the matrix-core path's chunks)
  int tok0[kVarlenBatch + 1];      // first packed token of sequence i; tok0[n] = tokens of the launch
  int chunk0[kVarlenBatch + 1];    // first chunk block of sequence i
  int slot[kVarlenBatch];          // state / conv-state slot of sequence i
  // set by the matrix-core launch: its state pass runs one workgroup per (column block, head,
  // group of consecutive sequences), group g being sequences grp0[g] .. grp0[g + 1] - 1
  int ngroups;
  int grp0[kVarlenGroups + 1];
};

struct RollbackArgs {
  int B0, nB, T_d, H, D, W;
  const float* snaps;   // [B, T_d, H, D, D]
  const void* qkv;      // [B, T_d, 3*H*D] io
  float* state;         // [B, H, D, D]
  void* conv_state;     // [B, 3*H*D, W-1] io
  uint8_t accepted[kRollbackBatch];
};

struct CommitArgs {
  int B0, nB, T_d, H, D, W;
  const float* tape;    // [B, T_d, H, 3, D]: alpha, k, u of every draft token
  const void* qkv;      // [B, T_d, 3*H*D] io
  float* state;         // [B, H, D, D]
  void* conv_state;     // [B, 3*H*D, W-1] io
  uint8_t accepted[kRollbackBatch];
};

// The current device's compute-unit count (looked up once per device; 256 if the query fails).
int device_cus();
// Allow `bytes` of dynamic LDS for kernel `fn` on the current device (set once per device and
// kernel; the status of that first attempt is returned on every later call).
hipError_t set_lds_limit(const void* fn, int bytes);

// Per-kernel timing (kda_timing_enable): the launch functions bracket each kernel launch with
// timing_begin / timing_end; both do nothing unless timing is on for the calling thread.
void timing_begin(const char* kernel, hipStream_t s);
void timing_end(hipStream_t s);

hipError_t launch_recurrent(const LayerArgs& a, int io, int ot, hipStream_t s);
hipError_t launch_rollback(const RollbackArgs& a, int io, hipStream_t s);
hipError_t launch_commit_tape(const CommitArgs& a, int io, hipStream_t s);

// Input projection (the fused-rows matmul + the low-rank / beta kernel).  Rank r = 128; H*D a
// multiple of 128; hidden a multiple of 128; bf16 weights and hidden states; outputs bf16 or fp32.
constexpr int kProjRank = 128;
struct ProjArgs {
  int T, hidden, H, D, out_type;
  const void* x;      // [T, hidden] bf16
  const void* w_in;   // [3*H*D + 2*r + H, hidden] bf16: rows q | k | v | f_a | g_a | b
  const void* w_fb;   // [H*D, r] bf16
  const void* w_gb;   // [H*D, r] bf16
  void* qkv;          // [T, 3*H*D]
  void* f;            // [T, H*D]
  void* beta;         // [T, H]
  void* g;            // [T, H*D]
  void* ws;
  size_t ws_bytes;
};
size_t projection_workspace(int T, int H, int D);
// On failure returns an error and writes a description into err.
hipError_t launch_projection(const ProjArgs& p, hipStream_t s, char* err, size_t errlen);

// Chunked prefill, fp32 VALU form (any supported head size; internal chunk <= 4096 / D).
hipError_t launch_prefill_generic(const LayerArgs& a, const SeqTab& st, int chunk, int io, int ot, hipStream_t s);

// Chunked prefill on bf16 MFMA (D = 128, chunk 64, bf16 io, conv width <= 4; the bounded gate with
// lb <= 0, or the softplus branch).
// Workspace: chunk blocks for `chunks` chunks of H heads, o for `tokens` tokens, a scratch slot.
constexpr int kMfmaChunk = 64;
bool prefill_mfma_supported(int D, int chunk, int io, int W, float lb, int gate);
size_t prefill_mfma_workspace(long long chunks, long long tokens, int H);
hipError_t launch_prefill_mfma(const LayerArgs& a, const SeqTab& st, void* ws, size_t ws_bytes, int ot,
                               hipStream_t s);

// kda_prefill_noalloc: the matrix-core prefill's workspace from a fixed device array of the library
// (kNoallocScratchBytes per GPU, held until the process ends).  noalloc_scratch returns the
// current device's address of that array, looked up on the first call on each device.
constexpr size_t kNoallocScratchBytes = 64u << 20;
hipError_t noalloc_scratch(void** ptr);

// kda_measure_stream: a streaming copy (src == nullptr: a zero fill) of bytes / 16 16-byte words.
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace kda
