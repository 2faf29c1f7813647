/*
 * kda.h — C ABI of the MI355X-native Kimi Delta Attention (KDA) layer library.
 *
 * The layer (llama.cpp PR #27754 "model: add GLM-5-Next (GLM-5.3-Flash)",
 * KDA commit message; Splash issue #740, maintainer answer):
 *   1. one depthwise causal conv over the concatenated q|k|v channels, whose
 *      state is one contiguous block of the W-1 previous raw inputs;
 *   2. SiLU on the conv output;
 *   3. q and k L2-normalised per head as x / max(||x||, l2_eps) (l2_eps is a
 *      literal 1e-6 in the model), q then multiplied by `scale`;
 *   4. a bounded-sigmoid per-channel log-decay
 *        g = gate_lower_bound * sigmoid(exp(A_log[h]) * (f + dt_bias)),
 *      dt_bias added per channel before the reshape to heads, A per head;
 *      or, where kda.gate_lower_bound is absent, the softplus branch
 *      (metadata commit of the same PR: a different function, not a missing
 *      clamp; read here as g = -exp(A_log[h]) * softplus(f + dt_bias), no
 *      lower bound), selected by gate_kind;
 *   5. per head a d_k x d_v fp32 state S (row = key channel) that decays on
 *      the key axis and takes a beta-weighted delta-rule update per token:
 *        S <- Diag(exp(g_t)) S;  u = beta_t (v_t - S^T k_t);  S <- S + k_t u^T;
 *        o_t = S^T q_t;
 *   6. a gated output RMSNorm with a plain weight over d_v per (token, head):
 *        out = o / sqrt(mean(o^2) + rms_eps) * norm_w * sigmoid(g_out).
 * Speculative decoding needs the state to roll back to an accepted prefix of
 * a verified draft block (dflash-mlx issue #63, "What the backend needs";
 * the DFlash2 drafter proposes blocks of 8 tokens, "Context").
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *     16-byte aligned.  The library allocates no device memory and keeps no
 *     state between calls; prefill scratch comes from the caller's workspace.
 *     One exception: kda_prefill_noalloc takes its scratch from a fixed
 *     device array of the library (see there).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  The returned status covers argument validation and launch
 *     errors only.  Validation runs before any launch: a call that returns an
 *     error has touched no buffer.
 *   - The library never aborts or throws; kda_last_error() returns a
 *     thread-local description of the most recent error.
 *   - Channel order of qkv: [q head 0..H-1 | k head 0..H-1 | v head 0..H-1],
 *     each head's d channels contiguous.  f and g_out are [.., H*d] in head
 *     order; beta is [.., H].
 *   - io_dtype (KDA_F32 or KDA_BF16) is the type of qkv, f, beta, g_out,
 *     conv_w, norm_w and conv_state; out_dtype the type of out; the state,
 *     the snapshots, A_log and dt_bias are always fp32.
 *   - One call covers at most 2^31 - 1 token-heads (B * T * H, or the packed
 *     tokens times H); larger requests return KDA_ERR_UNSUPPORTED.
 *   - Supported: d_k == d_v in {16, 32, 64, 128}; conv_width 1..8;
 *     prefill chunk_size in {16, 32, 64}.  Other shapes return
 *     KDA_ERR_UNSUPPORTED.  bf16 io with d = 128, chunk 64, conv width <= 4
 *     and a decaying gate (the softplus branch, or the bounded gate with
 *     gate_lower_bound <= 0) runs the bf16 matrix-core prefill; every other
 *     prefill (fp32 io, other head sizes or chunks, conv width > 4, a positive
 *     bound, under which the state grows) runs the fp32 vector-ALU form.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad size, NaN gate bound, ... */
  KDA_ERR_UNSUPPORTED = 2,      /* valid request for a shape or dtype this build does not run */
  KDA_ERR_HIP = 3               /* a HIP launch failed */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Decay gate (step 4).  KDA_GATE_BOUNDED_SIGMOID needs a finite gate_lower_bound;
 * KDA_GATE_SOFTPLUS is the branch for a model without one, and takes
 * gate_lower_bound = NaN (absent); any other combination is an error. */
typedef enum kda_gate_kind { KDA_GATE_BOUNDED_SIGMOID = 0, KDA_GATE_SOFTPLUS = 1 } kda_gate_kind;

/* Per-layer description.  Parameter pointers are device pointers. */
typedef struct kda_layer_desc {
  int32_t num_heads;        /* H */
  int32_t head_dim_k;       /* d_k */
  int32_t head_dim_v;       /* d_v (must equal d_k) */
  int32_t conv_width;       /* W: conv taps; the conv state holds W-1 inputs */
  int32_t chunk_size;       /* prefill chunk length C */
  int32_t io_dtype;         /* kda_dtype */
  int32_t out_dtype;        /* kda_dtype */
  float gate_lower_bound;   /* kda.gate_lower_bound: finite for the bounded gate, NaN (absent) for softplus */
  float l2_eps;             /* q/k L2 clamp, > 0 (1e-6 in the model) */
  float rms_eps;            /* output RMSNorm eps, >= 0 (1e-5 in the model) */
  float scale;              /* query scale applied after the L2 norm */
  const void* conv_w;       /* [3*H*d, W] io_dtype; tap W-1 multiplies the current token */
  const float* A_log;       /* [H] fp32 */
  const float* dt_bias;     /* [H*d_k] fp32 */
  const void* norm_w;       /* [d_v] io_dtype, plain weight (not 1 + w) */
  int32_t gate_kind;        /* kda_gate_kind (0, the bounded gate, when zero-initialised) */
} kda_layer_desc;

/* Version of this ABI (KDA_ABI_VERSION). */
int32_t kda_abi_version(void);

/* Static description of a status code. */
const char* kda_status_string(kda_status status);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* kda_last_error(void);

/*
 * Workspace bytes kda_prefill needs for (desc, B, T); 0 when no workspace is
 * needed.  Returns (size_t)-1 if the arguments are invalid.
 */
size_t kda_prefill_workspace_size(const kda_layer_desc* desc, int32_t B, int32_t T);

/*
 * Chunked prefill of T tokens on each of B sequences (steps 1-6 above; the
 * recurrence in chunked WY/UT form with chunk desc->chunk_size).  It plays
 * the role of the "chunked fallback" delta net of llama.cpp PR #27754, KDA
 * commit; chained calls carrying state and conv_state equal one call, as the
 * glm53-flash-mlx README's tests require of split prefills (5 + 7 tokens).
 *   qkv        [B, T, 3*H*d]   raw pre-conv projections        (in)
 *   f          [B, T, H*d]     gate pre-activation             (in)
 *   beta       [B, T, H]       delta-rule step, in (0, 1)      (in)
 *   g_out      [B, T, H*d]     output-gate logits              (in)
 *   state      [B, H, d, d]    fp32 recurrent state            (in/out)
 *   conv_state [B, 3*H*d, W-1] previous raw inputs, oldest first (in/out)
 *   out        [B, T, H*d]     gated RMSNorm output            (out)
 *   workspace  >= kda_prefill_workspace_size(desc, B, T) bytes, 256-byte aligned
 * Any T >= 0 (T need not be a multiple of the chunk; T = 0 or B = 0 is a
 * no-op).  Calls that pass state and conv_state along equal one longer call.
 * out must not alias any input.
 */
kda_status kda_prefill(const kda_layer_desc* desc, int32_t B, int32_t T, const void* qkv, const void* f,
                       const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_prefill without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the scratch the matrix-core prefill needs comes from
 * a fixed array inside the library, 64 MiB on each GPU the call runs on (held
 * from the first such call on that GPU until the process ends).  Arguments
 * and results are those of kda_prefill; no device memory is allocated or
 * freed.  A request whose scratch, kda_prefill_workspace_size(desc, B, T),
 * exceeds 64 MiB returns KDA_ERR_UNSUPPORTED before anything runs (at H = 32,
 * B = 1 that is T up to 1472 tokens; chain calls for longer prompts).  Every
 * call on one GPU uses the same array: calls that overlap in time on one GPU
 * (on different streams, or from different threads) race and must not be
 * issued; calls in one stream's order are safe.
 */
kda_status kda_prefill_noalloc(const kda_layer_desc* desc, int32_t B, int32_t T, const void* qkv, const void* f,
                               const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                               void* stream);

/*
 * Variable-length prefill: N sequences of different lengths packed along the
 * token axis in one call, each continuing the state held in its own slot of a
 * state pool (the serving shape of a hybrid memory with one recurrent-state
 * cell per sequence, llama.cpp PR #27754, KDA commit: n_rs_seq).  Each
 * sequence gives exactly what kda_prefill gives for it alone.
 *   cu_seqlens_host [N+1] HOST int32: cu_seqlens[0] = 0, non-decreasing;
 *                   sequence i owns packed tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
 *   slots_host      [N] HOST int32, distinct, in 0..num_slots-1: the state /
 *                   conv-state slot of sequence i (NULL: slot i)
 *   qkv   [total, 3*H*d], f [total, H*d], beta [total, H], g_out [total, H*d]
 *         with total = cu_seqlens[N]                                 (in)
 *   state      [num_slots, H, d, d] fp32                             (in/out)
 *   conv_state [num_slots, 3*H*d, W-1]                               (in/out)
 *   out        [total, H*d]                                          (out)
 *   workspace  >= kda_prefill_varlen_workspace_size(desc, N, cu_seqlens_host)
 *              bytes, 256-byte aligned (0 bytes for the fp32 path)
 * Only the slots of sequences with at least one token are read or written;
 * a sequence of length 0 is a no-op.  An invalid table (decreasing offsets,
 * a slot out of range or used twice) fails before anything runs.
 * kda_prefill_varlen_workspace_size returns (size_t)-1 for invalid arguments.
 */
size_t kda_prefill_varlen_workspace_size(const kda_layer_desc* desc, int32_t N, const int32_t* cu_seqlens_host);
kda_status kda_prefill_varlen(const kda_layer_desc* desc, int32_t N, const int32_t* cu_seqlens_host,
                              const int32_t* slots_host, int32_t num_slots, const void* qkv, const void* f,
                              const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step: one new token per sequence, state and conv_state updated
 * in place.  Tensor shapes as kda_prefill with T = 1.  It plays the role of
 * build_delta_net_autoregressive (llama.cpp PR #27754, KDA commit: the
 * token-by-token path, key-axis decay); decoding token by token equals one
 * prefill over the same tokens (glm53-flash-mlx README, tests).
 */
kda_status kda_decode_step(const kda_layer_desc* desc, int32_t B, const void* qkv, const void* f,
                           const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                           void* stream);

/*
 * Verify a draft block of T_d tokens per sequence from the live state,
 * recording the state after every token, so that the state can roll back to
 * any accepted prefix (dflash-mlx issue #63, "What the backend needs": KDA
 * state rollback; "Context": the DFlash2 drafter proposes blocks of 8; the
 * conv state is one contiguous block so that it can be snapshotted, llama.cpp
 * PR #27754, KDA commit).  state and conv_state are read only.
 * 1 <= T_d <= 255 (T_d = 0 or B = 0 is a no-op; T_d > 255 returns
 * KDA_ERR_UNSUPPORTED); the same limit holds for kda_rollback,
 * kda_verify_block_tape, kda_commit_tape and kda_verify_tape_size.
 *   qkv, f, beta, g_out  [B, T_d, ...] as kda_prefill
 *   snaps  [B, T_d, H, d, d] fp32: snaps[b, t] = state after draft token t+1 (out)
 *   out    [B, T_d, H*d] (out)
 */
kda_status kda_verify_block(const kda_layer_desc* desc, int32_t B, int32_t T_d, const void* qkv, const void* f,
                            const void* beta, const void* g_out, const float* state, const void* conv_state,
                            float* snaps, void* out, void* stream);

/*
 * Commit the accepted prefix of a verified block (dflash-mlx issue #63, "What
 * the backend needs"; a rollback depth must never be silently clamped,
 * llama.cpp PR #27754, KDA commit on n_rs_seq).  accepted_host is a HOST
 * array of B counts m_b in 0..T_d (outside that range the call fails; no
 * clamping).  For each b with m_b > 0:
 *   state[b]      <- snaps[b, m_b - 1]
 *   conv_state[b] <- the last W-1 raw inputs of (conv_state[b] || qkv_block[b, :m_b])
 * Sequences with m_b = 0 are left untouched.  qkv_block is the verify call's qkv.
 */
kda_status kda_rollback(const kda_layer_desc* desc, int32_t B, int32_t T_d, const int32_t* accepted_host,
                        const float* snaps, const void* qkv_block, float* state, void* conv_state, void* stream);

/*
 * Speculative verify with a replay tape instead of snapshots.  The state after
 * draft token t is Diag(alpha_t) S_{t-1} + k_t u_t^T, where alpha_t is the
 * token's decay, k_t its normalised key and u_t = beta_t (v_t - (Diag(alpha_t)
 * S_{t-1})^T k_t) its delta-rule update; all three are known once the verify
 * pass has computed u_t.  Recording them (3*d floats per token and head)
 * instead of the d*d state lets the commit replay the accepted prefix on the
 * live state, so a block costs about three state passes (verify read, commit
 * read and write) instead of 1 + T_d + 1.
 *
 * kda_verify_tape_size: bytes of the tape for (desc, B, T_d),
 *   B * T_d * H * 3 * d * 4; (size_t)-1 if the arguments are invalid or
 *   T_d > 255.
 * kda_verify_block_tape: as kda_verify_block (same outputs, bit-identical),
 *   but writes
 *     tape [B, T_d, H, 3, d] fp32: tape[b, t, h] = (alpha, k, u) of token t
 *   and no state at all.  state and conv_state are read only.
 * kda_commit_tape: commits the accepted prefix from the tape.  accepted_host
 *   is a HOST array of B counts m_b in 0..T_d (outside that range the call
 *   fails; no clamping).  For each b with m_b > 0 it replays tokens 0..m_b-1
 *   on state[b] (the state the verify call read), which gives the verify
 *   pass's own state after token m_b bit for bit, and sets conv_state[b] to
 *   the last W-1 raw inputs of (conv_state[b] || qkv_block[b, :m_b]).
 *   Sequences with m_b = 0 are left untouched.  qkv_block is the verify call's
 *   qkv; tape the verify call's tape, unchanged.
 */
size_t kda_verify_tape_size(const kda_layer_desc* desc, int32_t B, int32_t T_d);
kda_status kda_verify_block_tape(const kda_layer_desc* desc, int32_t B, int32_t T_d, const void* qkv,
                                 const void* f, const void* beta, const void* g_out, const float* state,
                                 const void* conv_state, float* tape, void* out, void* stream);
kda_status kda_commit_tape(const kda_layer_desc* desc, int32_t B, int32_t T_d, const int32_t* accepted_host,
                           const float* tape, const void* qkv_block, float* state, void* conv_state,
                           void* stream);

/*
 * Input projection of a KDA layer: the step before the layer.  The q, k, v,
 * f_a, g_a and b projections of the hidden states are one weight matrix (the
 * runtime fuses the six KDA input projections into one matmul, glm53-flash-mlx
 * README, quantization recipe); f and the output gate are low rank,
 * f = f_b(f_a x), g_out = g_b(g_a x) (llama.cpp PR #27754, KDA commit), and
 * beta = sigmoid(b x).  Weights are Linear weights ([out, in], row-major):
 *   w_in [3*H*d + 2*rank + H, hidden] bf16, rows q | k | v | f_a | g_a | b
 *   w_fb [H*d, rank] bf16,  w_gb [H*d, rank] bf16
 * Supported: rank = 128, H*d a multiple of 128, hidden a multiple of 128.
 */
typedef struct kda_proj_desc {
  int32_t num_heads;   /* H */
  int32_t head_dim;    /* d */
  int32_t hidden;      /* model width of the hidden states */
  int32_t rank;        /* f_a / g_a width (128) */
  int32_t out_dtype;   /* KDA_BF16 or KDA_F32: type of qkv, f, beta, g_out */
  const void* w_in;
  const void* w_fb;
  const void* w_gb;
} kda_proj_desc;

/*
 * Workspace bytes kda_input_projection needs for T tokens ((size_t)-1 if the
 * arguments are invalid): 9 blocks of T * P * 4 bytes, each rounded up to 256,
 * P = 2 * rank + H rounded up to a multiple of 4: the rank / beta activations
 * in fp32 and 8 partial sums of them over pieces of the hidden dimension.
 */
size_t kda_input_projection_workspace_size(const kda_proj_desc* desc, int32_t T);

/*
 * x [T, hidden] bf16 (in) -> qkv [T, 3*H*d], f [T, H*d], beta [T, H],
 * g_out [T, H*d] (out, desc->out_dtype): exactly the token inputs of
 * kda_prefill.  workspace: >= kda_input_projection_workspace_size bytes,
 * 256-byte aligned.  Accumulation is fp32; the rank activations stay fp32
 * until the up-projections (which split them into bf16 hi + lo).
 */
kda_status kda_input_projection(const kda_proj_desc* desc, int32_t T, const void* x, void* qkv, void* f,
                                void* beta, void* g_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing, for benchmarks (not part of the layer).
 * kda_timing_enable(1) makes every later call made on this host thread record
 * a HIP event pair on the call's stream around each kernel it launches;
 * kda_timing_enable(0) stops recording.  Off by default; recording adds two
 * event records per kernel and changes no result.  Returns the previous
 * setting.
 * kda_timing_read waits for the recorded events, writes the kernel names
 * (static strings owned by the library) and durations in milliseconds of the
 * first `cap` records in launch order into names / ms (host arrays, either may
 * be NULL when cap is 0), releases every record and returns how many records
 * there were (possibly more than cap), or -1 if a HIP call failed (the records
 * are released all the same; kda_last_error() says which).
 */
int32_t kda_timing_enable(int32_t on);
int32_t kda_timing_read(const char** names, float* ms, int32_t cap);

/*
 * A streaming copy, for benchmarks (not part of the layer): the HBM ceilings the
 * layer's bandwidth-bound calls are reported against.  Copies `bytes` from src to
 * dst (device pointers, 16-byte aligned, bytes a multiple of 16, the ranges
 * disjoint), or writes zeros to dst when src is NULL, with 16-byte non-temporal
 * loads and stores, asynchronously on `stream`.  KDA_ERR_INVALID_ARGUMENT on a
 * null dst, misaligned pointers or a size that is not a multiple of 16.
 */
kda_status kda_measure_stream(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
