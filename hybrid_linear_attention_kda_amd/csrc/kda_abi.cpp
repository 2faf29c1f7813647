// C ABI of the KDA layer library: argument validation and dispatch.
//
// Every check runs before the first launch, so a call that returns an error
// has touched no buffer (refuse unsupported configurations up front rather
// than failing mid-run, as llama.cpp PR #27754 does for its indexer cache;
// a missing kda.gate_lower_bound is an error, never a silent default, as in
// its metadata commit; a rollback depth is never silently clamped, as its
// KDA commit warns).
#include "../../include/kda.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "kda_launch.h"

namespace kda {

namespace {
std::mutex g_dev_mu;
std::map<int, int> g_cus;
std::map<std::pair<int, const void*>, hipError_t> g_lds;
}  // namespace

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cus[dev] = n;
  return n;
}

hipError_t set_lds_limit(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  const auto key = std::make_pair(dev, fn);
  auto it = g_lds.find(key);
  if (it != g_lds.end()) return it->second;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  g_lds[key] = e;
  return e;
}

}  // namespace kda


namespace {

thread_local char g_last_error[512] = "";

kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

kda_status ok() {
  g_last_error[0] = '\0';
  return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kda_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is null", name);
  if (!aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return KDA_OK;
}

#define KDA_TRY(expr)                      \
  do {                                     \
    kda_status _s = (expr);                \
    if (_s != KDA_OK) return _s;           \
  } while (0)

kda_status check_desc(const kda_layer_desc* d) {
  if (d == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is null");
  if (d->num_heads < 1 || d->head_dim_k < 1 || d->head_dim_v < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_heads / head dims must be >= 1");
  if (d->num_heads > 65535) return fail(KDA_ERR_UNSUPPORTED, "num_heads > 65535");
  if (d->head_dim_k != d->head_dim_v)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim_k (%d) != head_dim_v (%d)", d->head_dim_k, d->head_dim_v);
  const int D = d->head_dim_k;
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(KDA_ERR_UNSUPPORTED, "head dim %d not in {16, 32, 64, 128}", D);
  if (d->conv_width < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "conv_width must be >= 1");
  if (d->conv_width > kda::kMaxConvWidth)
    return fail(KDA_ERR_UNSUPPORTED, "conv_width %d > %d", d->conv_width, kda::kMaxConvWidth);
  if ((d->io_dtype != KDA_F32 && d->io_dtype != KDA_BF16) || (d->out_dtype != KDA_F32 && d->out_dtype != KDA_BF16))
    return fail(KDA_ERR_INVALID_ARGUMENT, "io_dtype / out_dtype must be KDA_F32 or KDA_BF16");
  if (d->gate_kind == KDA_GATE_BOUNDED_SIGMOID) {
    if (std::isnan(d->gate_lower_bound))
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "gate_lower_bound is absent (NaN); the bounded gate requires it (the softplus branch is "
                  "gate_kind KDA_GATE_SOFTPLUS)");
    if (!std::isfinite(d->gate_lower_bound)) return fail(KDA_ERR_INVALID_ARGUMENT, "gate_lower_bound is not finite");
  } else if (d->gate_kind == KDA_GATE_SOFTPLUS) {
    if (!std::isnan(d->gate_lower_bound))
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "gate_kind KDA_GATE_SOFTPLUS is the branch without a lower bound: gate_lower_bound must be NaN");
  } else {
    return fail(KDA_ERR_INVALID_ARGUMENT, "gate_kind %d is not a kda_gate_kind", d->gate_kind);
  }
  if (!std::isfinite(d->l2_eps) || !(d->l2_eps > 0.f)) return fail(KDA_ERR_INVALID_ARGUMENT, "l2_eps must be > 0");
  if (!std::isfinite(d->rms_eps) || d->rms_eps < 0.f) return fail(KDA_ERR_INVALID_ARGUMENT, "rms_eps must be >= 0");
  if (!std::isfinite(d->scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
  KDA_TRY(check_ptr(d->conv_w, "desc.conv_w"));
  KDA_TRY(check_ptr(d->A_log, "desc.A_log"));
  KDA_TRY(check_ptr(d->dt_bias, "desc.dt_bias"));
  KDA_TRY(check_ptr(d->norm_w, "desc.norm_w"));
  return KDA_OK;
}

// B sequences of T tokens over H heads; the launches index token-heads (and their 64-token
// chunks) with 32-bit integers, so one call covers at most 2^31 - 1 token-heads.
kda_status check_batch(int32_t B, int32_t T, int32_t H) {
  if (B < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B and T must be >= 0");
  if (B > 65535) return fail(KDA_ERR_UNSUPPORTED, "B > 65535");
  if ((long long)B * T * H > 0x7fffffffLL)
    return fail(KDA_ERR_UNSUPPORTED, "B * T * H = %lld token-heads exceeds 2^31 - 1 per call", (long long)B * T * H);
  return KDA_OK;
}

kda_status check_chunk(const kda_layer_desc* d) {
  if (d->chunk_size < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "chunk_size must be >= 1");
  if (d->chunk_size != 16 && d->chunk_size != 32 && d->chunk_size != 64)
    return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d not in {16, 32, 64}", d->chunk_size);
  return KDA_OK;
}

kda::LayerArgs make_args(const kda_layer_desc* d, int B, int T) {
  kda::LayerArgs a{};
  a.B = B;
  a.T = T;
  a.H = d->num_heads;
  a.D = d->head_dim_k;
  a.W = d->conv_width;
  a.gate = d->gate_kind;
  a.lb = d->gate_kind == KDA_GATE_SOFTPLUS ? 0.f : d->gate_lower_bound;
  a.l2_eps = d->l2_eps;
  a.rms_eps = d->rms_eps;
  a.scale = d->scale;
  a.conv_w = d->conv_w;
  a.A_log = d->A_log;
  a.dt_bias = d->dt_bias;
  a.norm_w = d->norm_w;
  return a;
}

// bf16 io at the model's head size runs the matrix-core prefill; everything else the fp32 form.
bool mfma_path(const kda_layer_desc* d) {
  return kda::prefill_mfma_supported(d->head_dim_k, d->chunk_size, d->io_dtype, d->conv_width, d->gate_lower_bound,
                                     d->gate_kind);
}

kda_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// One launch of a variable-length prefill: up to kVarlenBatch sequences of length >= 1, packed from
// token t0 of the call on (the table's token offsets are relative to t0).
struct Launch {
  long long t0;
  kda::SeqTab tab;
};

// Validate a variable-length call and cut it into launches.  cu_seqlens[0] = 0 and non-decreasing;
// slots (NULL: sequence i uses slot i) in 0..num_slots-1 and distinct.  Sequences of length 0 are
// no-ops and get no table entry.
kda_status plan_varlen(int32_t N, const int32_t* cu, const int32_t* slots, int32_t num_slots, int32_t H,
                       std::vector<Launch>& plan) {
  plan.clear();
  if (N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "N must be >= 0");
  if (N == 0) return KDA_OK;
  if (cu == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host is null");
  if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d, must be 0", cu[0]);
  if (num_slots < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "num_slots must be >= 1");
  std::vector<char> used((size_t)num_slots, 0);
  Launch cur{};
  for (int32_t i = 0; i < N; ++i) {
    if (cu[i + 1] < cu[i])
      return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d (%d -> %d)", i, cu[i], cu[i + 1]);
    const int32_t slot = slots != nullptr ? slots[i] : i;
    if (slot < 0 || slot >= num_slots)
      return fail(KDA_ERR_INVALID_ARGUMENT, "slot of sequence %d = %d outside 0..%d", i, slot, num_slots - 1);
    if (used[(size_t)slot]) return fail(KDA_ERR_INVALID_ARGUMENT, "slot %d is used by two sequences", slot);
    used[(size_t)slot] = 1;
    const int32_t len = cu[i + 1] - cu[i];
    if (len == 0) continue;
    if (cur.tab.n == kda::kVarlenBatch) {
      plan.push_back(cur);
      cur = Launch{};
    }
    kda::SeqTab& t = cur.tab;
    if (t.n == 0) {
      cur.t0 = cu[i];
      t.tok0[0] = 0;
      t.chunk0[0] = 0;
    }
    t.slot[t.n] = slot;
    t.tok0[t.n + 1] = cu[i + 1] - (int32_t)cur.t0;
    t.chunk0[t.n + 1] = t.chunk0[t.n] + (len + kda::kMfmaChunk - 1) / kda::kMfmaChunk;
    t.total_chunks = t.chunk0[t.n + 1];
    ++t.n;
  }
  if (cur.tab.n > 0) plan.push_back(cur);
  if ((long long)cu[N] * H > 0x7fffffffLL)
    return fail(KDA_ERR_UNSUPPORTED, "%d packed tokens x %d heads exceeds 2^31 - 1 token-heads per call", cu[N], H);
  return KDA_OK;
}

size_t varlen_workspace(const std::vector<Launch>& plan, int H) {
  size_t need = 0;
  for (const Launch& l : plan) {
    const size_t n = kda::prefill_mfma_workspace(l.tab.total_chunks, l.tab.tok0[l.tab.n], H);
    if (n > need) need = n;
  }
  return need;
}

kda_status check_proj(const kda_proj_desc* d) {
  if (d == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is null");
  if (d->num_heads < 1 || d->head_dim < 1 || d->hidden < 1 || d->rank < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_heads, head_dim, hidden and rank must be >= 1");
  if (d->rank != kda::kProjRank) return fail(KDA_ERR_UNSUPPORTED, "rank %d != %d", d->rank, kda::kProjRank);
  if ((long long)d->num_heads * d->head_dim > 65536 || d->hidden > 65536)
    return fail(KDA_ERR_UNSUPPORTED, "H*d and hidden must be <= 65536");
  if ((d->num_heads * d->head_dim) % 128 != 0)
    return fail(KDA_ERR_UNSUPPORTED, "H*d = %d is not a multiple of 128", d->num_heads * d->head_dim);
  if (d->hidden % 128 != 0) return fail(KDA_ERR_UNSUPPORTED, "hidden = %d is not a multiple of 128", d->hidden);
  if (d->out_dtype != KDA_F32 && d->out_dtype != KDA_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "out_dtype must be KDA_F32 or KDA_BF16");
  KDA_TRY(check_ptr(d->w_in, "desc.w_in"));
  KDA_TRY(check_ptr(d->w_fb, "desc.w_fb"));
  KDA_TRY(check_ptr(d->w_gb, "desc.w_gb"));
  return KDA_OK;
}

kda_status check_token_tensors(const void* qkv, const void* f, const void* beta, const void* g_out) {
  KDA_TRY(check_ptr(qkv, "qkv"));
  KDA_TRY(check_ptr(f, "f"));
  KDA_TRY(check_ptr(beta, "beta"));
  KDA_TRY(check_ptr(g_out, "g_out"));
  return KDA_OK;
}

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* kda_last_error(void) { return g_last_error; }

size_t kda_prefill_workspace_size(const kda_layer_desc* desc, int32_t B, int32_t T) {
  if (check_desc(desc) != KDA_OK || check_batch(B, T, desc->num_heads) != KDA_OK || check_chunk(desc) != KDA_OK) return (size_t)-1;
  if (!mfma_path(desc)) return 0;
  const long long nc = ((long long)T + kda::kMfmaChunk - 1) / kda::kMfmaChunk;
  return kda::prefill_mfma_workspace((long long)B * nc, (long long)B * T, desc->num_heads);
}

kda_status kda_prefill(const kda_layer_desc* desc, int32_t B, int32_t T, const void* qkv, const void* f,
                       const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, T, desc->num_heads));
  KDA_TRY(check_chunk(desc));
  if (B == 0 || T == 0) return ok();
  KDA_TRY(check_token_tensors(qkv, f, beta, g_out));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  KDA_TRY(check_ptr(out, "out"));
  kda::LayerArgs a = make_args(desc, B, T);
  a.qkv = qkv;
  a.f = f;
  a.beta = beta;
  a.g_out = g_out;
  a.state_in = state;
  a.state_out = state;
  a.conv_in = conv_state;
  a.conv_out = desc->conv_width > 1 ? conv_state : nullptr;
  a.out = out;
  a.snapshots = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma_path(desc)) {
    const size_t need = kda_prefill_workspace_size(desc, B, T);
    if (need > 0) {
      if (workspace == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is null (%zu bytes needed)", need);
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
      if (workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    }
    return launched(kda::launch_prefill_mfma(a, kda::SeqTab{}, workspace, workspace_bytes, desc->out_dtype, s),
                    "kda_prefill");
  }
  return launched(kda::launch_prefill_generic(a, kda::SeqTab{}, desc->chunk_size, desc->io_dtype, desc->out_dtype, s),
                  "kda_prefill");
}

kda_status kda_prefill_noalloc(const kda_layer_desc* desc, int32_t B, int32_t T, const void* qkv, const void* f,
                               const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                               void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, T, desc->num_heads));
  KDA_TRY(check_chunk(desc));
  if (B == 0 || T == 0) return ok();
  const size_t need = kda_prefill_workspace_size(desc, B, T);
  if (need > kda::kNoallocScratchBytes)
    return fail(KDA_ERR_UNSUPPORTED,
                "kda_prefill_noalloc: B = %d, T = %d, H = %d needs %zu scratch bytes, more than the library's fixed "
                "%zu; use kda_prefill with a workspace, or fewer tokens per call",
                B, T, desc->num_heads, need, kda::kNoallocScratchBytes);
  KDA_TRY(check_token_tensors(qkv, f, beta, g_out));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  KDA_TRY(check_ptr(out, "out"));
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = kda::noalloc_scratch(&scratch);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_prefill_noalloc: scratch lookup: %s", hipGetErrorString(e));
  }
  return kda_prefill(desc, B, T, qkv, f, beta, g_out, state, conv_state, out, scratch, need, stream);
}

size_t kda_prefill_varlen_workspace_size(const kda_layer_desc* desc, int32_t N, const int32_t* cu_seqlens_host) {
  if (check_desc(desc) != KDA_OK || check_chunk(desc) != KDA_OK) return (size_t)-1;
  std::vector<Launch> plan;
  // slots do not change the size: check the offsets with slot i for sequence i
  if (plan_varlen(N, cu_seqlens_host, nullptr, N > 0 ? N : 1, desc->num_heads, plan) != KDA_OK) return (size_t)-1;
  if (!mfma_path(desc)) return 0;
  return varlen_workspace(plan, desc->num_heads);
}

kda_status kda_prefill_varlen(const kda_layer_desc* desc, int32_t N, const int32_t* cu_seqlens_host,
                              const int32_t* slots_host, int32_t num_slots, const void* qkv, const void* f,
                              const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_chunk(desc));
  std::vector<Launch> plan;
  KDA_TRY(plan_varlen(N, cu_seqlens_host, slots_host, num_slots, desc->num_heads, plan));
  if (plan.empty()) return ok();  // no sequence has a token
  KDA_TRY(check_token_tensors(qkv, f, beta, g_out));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  KDA_TRY(check_ptr(out, "out"));
  const bool mfma = mfma_path(desc);
  if (mfma) {
    const size_t need = varlen_workspace(plan, desc->num_heads);
    if (workspace == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is null (%zu bytes needed)", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(KDA_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t io = desc->io_dtype == KDA_BF16 ? 2 : 4, ob = desc->out_dtype == KDA_BF16 ? 2 : 4;
  const long long H = desc->num_heads, HD = H * desc->head_dim_k;
  for (const Launch& l : plan) {
    // each launch sees its tokens from its first one on; slots stay absolute
    kda::LayerArgs a = make_args(desc, l.tab.n, 0);
    a.qkv = static_cast<const char*>(qkv) + l.t0 * 3 * HD * io;
    a.f = static_cast<const char*>(f) + l.t0 * HD * io;
    a.beta = static_cast<const char*>(beta) + l.t0 * H * io;
    a.g_out = static_cast<const char*>(g_out) + l.t0 * HD * io;
    a.out = static_cast<char*>(out) + l.t0 * HD * ob;
    a.state_in = state;
    a.state_out = state;
    a.conv_in = conv_state;
    a.conv_out = desc->conv_width > 1 ? conv_state : nullptr;
    a.snapshots = 0;
    const hipError_t e = mfma ? kda::launch_prefill_mfma(a, l.tab, workspace, workspace_bytes, desc->out_dtype, s)
                              : kda::launch_prefill_generic(a, l.tab, desc->chunk_size, desc->io_dtype,
                                                            desc->out_dtype, s);
    KDA_TRY(launched(e, "kda_prefill_varlen"));
  }
  return ok();
}

kda_status kda_decode_step(const kda_layer_desc* desc, int32_t B, const void* qkv, const void* f,
                           const void* beta, const void* g_out, float* state, void* conv_state, void* out,
                           void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, 1, desc->num_heads));
  if (B == 0) return ok();
  KDA_TRY(check_token_tensors(qkv, f, beta, g_out));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  KDA_TRY(check_ptr(out, "out"));
  kda::LayerArgs a = make_args(desc, B, 1);
  a.qkv = qkv;
  a.f = f;
  a.beta = beta;
  a.g_out = g_out;
  a.state_in = state;
  a.state_out = state;
  a.conv_in = conv_state;
  a.conv_out = desc->conv_width > 1 ? conv_state : nullptr;
  a.out = out;
  a.snapshots = 0;
  return launched(kda::launch_recurrent(a, desc->io_dtype, desc->out_dtype, static_cast<hipStream_t>(stream)),
                  "kda_decode_step");
}

kda_status kda_verify_block(const kda_layer_desc* desc, int32_t B, int32_t T_d, const void* qkv, const void* f,
                            const void* beta, const void* g_out, const float* state, const void* conv_state,
                            float* snaps, void* out, void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, T_d, desc->num_heads));
  if (T_d > 255) return fail(KDA_ERR_UNSUPPORTED, "draft block T_d = %d > 255", T_d);
  if (B == 0 || T_d == 0) return ok();
  KDA_TRY(check_token_tensors(qkv, f, beta, g_out));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  KDA_TRY(check_ptr(snaps, "snaps"));
  KDA_TRY(check_ptr(out, "out"));
  kda::LayerArgs a = make_args(desc, B, T_d);
  a.qkv = qkv;
  a.f = f;
  a.beta = beta;
  a.g_out = g_out;
  a.state_in = state;
  a.state_out = snaps;
  a.conv_in = conv_state;
  a.conv_out = nullptr;
  a.out = out;
  a.snapshots = 1;
  return launched(kda::launch_recurrent(a, desc->io_dtype, desc->out_dtype, static_cast<hipStream_t>(stream)),
                  "kda_verify_block");
}

kda_status kda_rollback(const kda_layer_desc* desc, int32_t B, int32_t T_d, const int32_t* accepted_host,
                        const float* snaps, const void* qkv_block, float* state, void* conv_state, void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, T_d, desc->num_heads));
  if (T_d > 255) return fail(KDA_ERR_UNSUPPORTED, "draft block T_d = %d > 255", T_d);
  if (B == 0) return ok();
  if (accepted_host == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "accepted_host is null");
  bool any = false;
  for (int32_t b = 0; b < B; ++b) {
    if (accepted_host[b] < 0 || accepted_host[b] > T_d)
      return fail(KDA_ERR_INVALID_ARGUMENT, "accepted[%d] = %d outside 0..%d", b, accepted_host[b], T_d);
    any = any || accepted_host[b] > 0;
  }
  if (!any) return ok();
  KDA_TRY(check_ptr(snaps, "snaps"));
  KDA_TRY(check_ptr(qkv_block, "qkv_block"));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t b0 = 0; b0 < B; b0 += kda::kRollbackBatch) {
    kda::RollbackArgs r{};
    r.B0 = b0;
    r.nB = (B - b0) < kda::kRollbackBatch ? (B - b0) : kda::kRollbackBatch;
    r.T_d = T_d;
    r.H = desc->num_heads;
    r.D = desc->head_dim_k;
    r.W = desc->conv_width;
    r.snaps = snaps;
    r.qkv = qkv_block;
    r.state = state;
    r.conv_state = conv_state;
    for (int i = 0; i < r.nB; ++i) r.accepted[i] = (uint8_t)accepted_host[b0 + i];
    kda_status st = launched(kda::launch_rollback(r, desc->io_dtype, s), "kda_rollback");
    if (st != KDA_OK) return st;
  }
  return ok();
}

size_t kda_verify_tape_size(const kda_layer_desc* desc, int32_t B, int32_t T_d) {
  if (check_desc(desc) != KDA_OK || check_batch(B, T_d, desc->num_heads) != KDA_OK) return (size_t)-1;
  if (T_d > 255) {
    fail(KDA_ERR_UNSUPPORTED, "draft block T_d = %d > 255", T_d);
    return (size_t)-1;
  }
  return (size_t)B * (size_t)T_d * (size_t)desc->num_heads * 3u * (size_t)desc->head_dim_k * sizeof(float);
}

kda_status kda_verify_block_tape(const kda_layer_desc* desc, int32_t B, int32_t T_d, const void* qkv,
                                 const void* f, const void* beta, const void* g_out, const float* state,
                                 const void* conv_state, float* tape, void* out, void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, T_d, desc->num_heads));
  if (T_d > 255) return fail(KDA_ERR_UNSUPPORTED, "draft block T_d = %d > 255", T_d);
  if (B == 0 || T_d == 0) return ok();
  KDA_TRY(check_token_tensors(qkv, f, beta, g_out));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  KDA_TRY(check_ptr(tape, "tape"));
  KDA_TRY(check_ptr(out, "out"));
  kda::LayerArgs a = make_args(desc, B, T_d);
  a.qkv = qkv;
  a.f = f;
  a.beta = beta;
  a.g_out = g_out;
  a.state_in = state;
  a.state_out = nullptr;
  a.conv_in = conv_state;
  a.conv_out = nullptr;
  a.out = out;
  a.snapshots = 0;
  a.tape = tape;
  return launched(kda::launch_recurrent(a, desc->io_dtype, desc->out_dtype, static_cast<hipStream_t>(stream)),
                  "kda_verify_block_tape");
}

kda_status kda_commit_tape(const kda_layer_desc* desc, int32_t B, int32_t T_d, const int32_t* accepted_host,
                           const float* tape, const void* qkv_block, float* state, void* conv_state,
                           void* stream) {
  KDA_TRY(check_desc(desc));
  KDA_TRY(check_batch(B, T_d, desc->num_heads));
  if (T_d > 255) return fail(KDA_ERR_UNSUPPORTED, "draft block T_d = %d > 255", T_d);
  if (B == 0) return ok();
  if (accepted_host == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "accepted_host is null");
  bool any = false;
  for (int32_t b = 0; b < B; ++b) {
    if (accepted_host[b] < 0 || accepted_host[b] > T_d)
      return fail(KDA_ERR_INVALID_ARGUMENT, "accepted[%d] = %d outside 0..%d", b, accepted_host[b], T_d);
    any = any || accepted_host[b] > 0;
  }
  if (!any) return ok();
  KDA_TRY(check_ptr(tape, "tape"));
  KDA_TRY(check_ptr(qkv_block, "qkv_block"));
  KDA_TRY(check_ptr(state, "state"));
  if (desc->conv_width > 1) KDA_TRY(check_ptr(conv_state, "conv_state"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t b0 = 0; b0 < B; b0 += kda::kRollbackBatch) {
    kda::CommitArgs c{};
    c.B0 = b0;
    c.nB = (B - b0) < kda::kRollbackBatch ? (B - b0) : kda::kRollbackBatch;
    c.T_d = T_d;
    c.H = desc->num_heads;
    c.D = desc->head_dim_k;
    c.W = desc->conv_width;
    c.tape = tape;
    c.qkv = qkv_block;
    c.state = state;
    c.conv_state = conv_state;
    for (int i = 0; i < c.nB; ++i) c.accepted[i] = (uint8_t)accepted_host[b0 + i];
    kda_status st = launched(kda::launch_commit_tape(c, desc->io_dtype, s), "kda_commit_tape");
    if (st != KDA_OK) return st;
  }
  return ok();
}

size_t kda_input_projection_workspace_size(const kda_proj_desc* desc, int32_t T) {
  if (check_proj(desc) != KDA_OK || check_batch(1, T, desc->num_heads) != KDA_OK) return (size_t)-1;
  return kda::projection_workspace(T, desc->num_heads, desc->head_dim);
}

kda_status kda_input_projection(const kda_proj_desc* desc, int32_t T, const void* x, void* qkv, void* f,
                                void* beta, void* g_out, void* workspace, size_t workspace_bytes, void* stream) {
  KDA_TRY(check_proj(desc));
  KDA_TRY(check_batch(1, T, desc->num_heads));
  if (T == 0) return ok();
  KDA_TRY(check_ptr(x, "x"));
  KDA_TRY(check_ptr(qkv, "qkv"));
  KDA_TRY(check_ptr(f, "f"));
  KDA_TRY(check_ptr(beta, "beta"));
  KDA_TRY(check_ptr(g_out, "g_out"));
  const size_t need = kda::projection_workspace(T, desc->num_heads, desc->head_dim);
  if (workspace == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is null (%zu bytes needed)", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(KDA_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  kda::ProjArgs p{};
  p.T = T;
  p.hidden = desc->hidden;
  p.H = desc->num_heads;
  p.D = desc->head_dim;
  p.out_type = desc->out_dtype;
  p.x = x;
  p.w_in = desc->w_in;
  p.w_fb = desc->w_fb;
  p.w_gb = desc->w_gb;
  p.qkv = qkv;
  p.f = f;
  p.beta = beta;
  p.g = g_out;
  p.ws = workspace;
  p.ws_bytes = workspace_bytes;
  char err[256] = "";
  const hipError_t e = kda::launch_projection(p, static_cast<hipStream_t>(stream), err, sizeof(err));
  if (e != hipSuccess) {
    if (err[0] != '\0') return fail(KDA_ERR_HIP, "kda_input_projection: %s", err);
    return fail(KDA_ERR_HIP, "kda_input_projection: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // extern "C"

// ---- per-kernel timing ------------------------------------------------------------------------

namespace {
struct TimingRecord {
  const char* kernel;
  hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<TimingRecord> g_records;
thread_local std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

namespace kda {
void timing_begin(const char* kernel, hipStream_t s) {
  if (!g_timing) return;
  TimingRecord r{kernel, pooled_event(), pooled_event()};
  if (r.start != nullptr) (void)hipEventRecord(r.start, s);
  g_records.push_back(r);
}
void timing_end(hipStream_t s) {
  if (!g_timing || g_records.empty()) return;
  if (g_records.back().stop != nullptr) (void)hipEventRecord(g_records.back().stop, s);
}
}  // namespace kda

extern "C" {

int32_t kda_timing_enable(int32_t on) {
  const int32_t prev = g_timing ? 1 : 0;
  g_timing = on != 0;
  return prev;
}

int32_t kda_timing_read(const char** names, float* ms, int32_t cap) {
  int32_t n = 0;
  bool failed = false;
  for (const TimingRecord& r : g_records) {
    float t = -1.0f;
    if (r.start == nullptr || r.stop == nullptr || hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) {
      failed = true;
    }
    if (n < cap) {
      if (names != nullptr) names[n] = r.kernel;
      if (ms != nullptr) ms[n] = t;
    }
    ++n;
    if (r.start != nullptr) g_event_pool.push_back(r.start);
    if (r.stop != nullptr) g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  if (failed) {
    fail(KDA_ERR_HIP, "kda_timing_read: a timing event could not be created, recorded or read");
    return -1;
  }
  return n;
}

kda_status kda_measure_stream(void* dst, const void* src, size_t bytes, void* stream) {
  KDA_TRY(check_ptr(dst, "dst"));
  if (src != nullptr && !aligned16(src)) return fail(KDA_ERR_INVALID_ARGUMENT, "src is not 16-byte aligned");
  if (bytes % 16 != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes = %zu is not a multiple of 16", bytes);
  const hipError_t e = kda::launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_measure_stream: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
