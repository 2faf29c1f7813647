// KDA input projection: the q, k, v, f_a, g_a and b projections of the hidden states as one
// weight matrix (one matmul over the concatenated output rows, glm53-flash-mlx README,
// quantization recipe: the runtime fuses the six KDA input projections into one matmul), then
// the low-rank up-projections f = f_b(f_a x) and g = g_b(g_a x) (the output gate is low rank,
// llama.cpp PR #27754, KDA commit) and beta = sigmoid(b x) in one kernel of our own.
//
// The big matmul is a plain bf16 GEMM with fp32 accumulation and runs on hipBLASLt: the q|k|v
// rows write straight into the layer's qkv input, the 2r + H rank / beta rows into an fp32
// workspace.  The low-rank kernel splits the fp32 rank-r activations into bf16 hi + lo (two
// matrix-core products per k-step, ~16 mantissa bits) so the only bf16 rounding an output sees is
// its own.
#include <hipblaslt/hipblaslt.h>

#include <cstdio>
#include <map>
#include <tuple>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int PJ_ROWS = 64;    // token rows per workgroup (16 per wave)
constexpr int PJ_COLS = 128;   // output columns per workgroup
constexpr int PJ_NT = 256;
constexpr int PJ_PB = kProjRank + 8;    // LDS pitch of a weight row (bf16), spreads the banks
constexpr int PJ_PO = PJ_COLS + 4;      // LDS pitch of an output row (fp32)

__device__ __forceinline__ f32x4 pj_mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void pj_store(float* p, float v) { *p = v; }
__device__ __forceinline__ void pj_store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void pj_store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void pj_store8(bf16_t* p, const float* v) {
  uint4 u;
  u.x = f32_to_bf16(v[0]) | (uint32_t)f32_to_bf16(v[1]) << 16;
  u.y = f32_to_bf16(v[2]) | (uint32_t)f32_to_bf16(v[3]) << 16;
  u.z = f32_to_bf16(v[4]) | (uint32_t)f32_to_bf16(v[5]) << 16;
  u.w = f32_to_bf16(v[6]) | (uint32_t)f32_to_bf16(v[7]) << 16;
  *reinterpret_cast<uint4*>(p) = u;
}

// out[T, HD] = act[T, R] . W^T for W [HD, R] (a Linear weight), act the fp32 rank activations
// (columns act_col .. act_col + R - 1 of the workspace rows, leading dimension ld).  blockIdx.z
// selects f (0) or g (1); the z = 0 workgroups of column block 0 also write beta.
template <typename OT>
__global__ __launch_bounds__(PJ_NT) void kda_proj_lowrank_kernel(const float* __restrict__ act, int ld, int T,
                                                                 int HD, int H, const bf16_t* __restrict__ w_fb,
                                                                 const bf16_t* __restrict__ w_gb, OT* __restrict__ f,
                                                                 OT* __restrict__ g, OT* __restrict__ beta) {
  constexpr int R = kProjRank;
  // the weight block, then (after every read of it) the output rows
  static_assert(PJ_ROWS * PJ_PO * 4 <= PJ_COLS * PJ_PB * 2, "output rows fit in the weight block");
  __shared__ __align__(16) __bf16 sW[PJ_COLS * PJ_PB];
  float* sO = reinterpret_cast<float*>(sW);
  const int which = blockIdx.z;
  const int r0 = blockIdx.y * PJ_ROWS, c0 = blockIdx.x * PJ_COLS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const bf16_t* W = which == 0 ? w_fb : w_gb;
  OT* out = which == 0 ? f : g;
  const int acol = which * R;

  // the weight rows of this column block into LDS: 16-byte pieces, 16 per row
  for (int i = tid; i < PJ_COLS * (R / 8); i += PJ_NT) {
    const int row = i / (R / 8), seg = i % (R / 8);
    *reinterpret_cast<uint4*>(sW + row * PJ_PB + seg * 8) =
        *reinterpret_cast<const uint4*>(W + (long long)(c0 + row) * R + seg * 8);
  }
  // this wave's 16 activation rows as split A operands (rows past T read row T-1; not stored)
  const int arow = min(r0 + 16 * wave + l16, T - 1);
  const float* ap = act + (long long)arow * ld + acol + 8 * lg;
  bf16x8 ahi[R / 32], alo[R / 32];
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    const float4 x0 = *reinterpret_cast<const float4*>(ap + 32 * s);
    const float4 x1 = *reinterpret_cast<const float4*>(ap + 32 * s + 4);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 hi = (__bf16)x[e];
      ahi[s][e] = hi;
      alo[s][e] = (__bf16)(x[e] - (float)hi);
    }
  }
  __syncthreads();
  f32x4 acc[PJ_COLS / 16];
#pragma unroll
  for (int ct = 0; ct < PJ_COLS / 16; ++ct) {
    acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < R / 32; ++s) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sW + (16 * ct + l16) * PJ_PB + 32 * s + 8 * lg);
      acc[ct] = pj_mfma(alo[s], b, acc[ct]);
      acc[ct] = pj_mfma(ahi[s], b, acc[ct]);
    }
  }
  // accumulator tiles (lane: rows 4 lg .. 4 lg + 3 of column l16) -> LDS rows -> 16-byte stores
  __syncthreads();  // every read of the weight block is done
#pragma unroll
  for (int ct = 0; ct < PJ_COLS / 16; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[(16 * wave + 4 * lg + r) * PJ_PO + 16 * ct + l16] = acc[ct][r];
  __syncthreads();
  for (int i = tid; i < PJ_ROWS * (PJ_COLS / 8); i += PJ_NT) {
    const int row = i / (PJ_COLS / 8), c8 = (i % (PJ_COLS / 8)) * 8;
    if (r0 + row >= T) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = sO[row * PJ_PO + c8 + e];
    pj_store8(out + (long long)(r0 + row) * HD + c0 + c8, v);
  }
  if (which == 0 && blockIdx.x == 0) {
    for (int i = tid; i < PJ_ROWS * H; i += PJ_NT) {
      const int row = i / H, hh = i % H;
      if (r0 + row >= T) continue;
      const float z = act[(long long)(r0 + row) * ld + 2 * R + hh];
      pj_store(beta + (long long)(r0 + row) * H + hh, 1.0f / (1.0f + __expf(-z)));
    }
  }
}

struct GemmKey {
  int m, n, k, ldd, dtype;
  bool operator<(const GemmKey& o) const {
    return std::tie(m, n, k, ldd, dtype) < std::tie(o.m, o.n, o.k, o.ldd, o.dtype);
  }
};

struct LtState {
  int device = -1;
  hipblasLtHandle_t handle = nullptr;
  std::map<GemmKey, hipblasLtMatmulAlgo_t> algos;
};
thread_local LtState g_lt;

#define LT_TRY(expr, what)                                                                 \
  do {                                                                                     \
    const hipblasStatus_t _st = (expr);                                                    \
    if (_st != HIPBLAS_STATUS_SUCCESS) {                                                   \
      snprintf(err, errlen, "hipBLASLt %s failed (status %d)", what, (int)_st);            \
      ok = false;                                                                          \
    }                                                                                      \
  } while (0)

// D [T, m] (row-major, leading dimension ldd) = X [T, k] . Wr^T, Wr the m rows of a row-major [*, k]
// bf16 weight starting at Wr.  Column-major view: D^T (m x T) = op_T(Wr as k x m) . (X as k x T).
bool gemm_xwt(int T, int k, int m, const void* X, const void* Wr, hipDataType dtype, void* D, int ldd, void* ws,
              size_t wsb, hipStream_t s, const char* name, char* err, size_t errlen) {
  bool ok = true;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    snprintf(err, errlen, "hipGetDevice failed");
    return false;
  }
  if (g_lt.handle == nullptr || g_lt.device != dev) {
    if (g_lt.handle != nullptr) hipblasLtDestroy(g_lt.handle);
    g_lt = LtState{};
    LT_TRY(hipblasLtCreate(&g_lt.handle), "create");
    if (!ok) return false;
    g_lt.device = dev;
  }
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  LT_TRY(hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F), "desc");
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  if (ok) LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)), "transa");
  if (ok) LT_TRY(hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)), "transb");
  if (ok) LT_TRY(hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, k, m, k), "layout A");
  if (ok) LT_TRY(hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, k, T, k), "layout B");
  if (ok) LT_TRY(hipblasLtMatrixLayoutCreate(&ld, dtype, m, T, ldd), "layout D");
  hipblasLtMatmulAlgo_t algo{};
  if (ok) {
    const GemmKey key{m, T, k, ldd, (int)dtype};
    auto it = g_lt.algos.find(key);
    if (it != g_lt.algos.end()) {
      algo = it->second;
    } else {
      LT_TRY(hipblasLtMatmulPreferenceCreate(&pref), "preference");
      const uint64_t cap = wsb;
      if (ok)
        LT_TRY(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap)),
               "workspace preference");
      hipblasLtMatmulHeuristicResult_t res{};
      int nres = 0;
      if (ok) LT_TRY(hipblasLtMatmulAlgoGetHeuristic(g_lt.handle, op, la, lb, ld, ld, pref, 1, &res, &nres), "heuristic");
      if (ok && (nres < 1 || res.state != HIPBLAS_STATUS_SUCCESS || res.workspaceSize > wsb)) {
        snprintf(err, errlen, "hipBLASLt has no algorithm for this GEMM within %zu workspace bytes", wsb);
        ok = false;
      }
      if (ok) {
        algo = res.algo;
        g_lt.algos[key] = algo;
      }
    }
  }
  if (ok) {
    const float one = 1.f, zero = 0.f;
    timing_begin(name, s);
    LT_TRY(hipblasLtMatmul(g_lt.handle, op, &one, Wr, la, X, lb, &zero, D, ld, D, ld, &algo, ws, wsb, s), "matmul");
    timing_end(s);
  }
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (op) hipblasLtMatmulDescDestroy(op);
  return ok;
}

}  // namespace

size_t projection_workspace(int T, int H, int D) {
  const size_t act = ((size_t)T * (2 * kProjRank + H) * sizeof(float) + 255) / 256 * 256;
  return act + kProjGemmWorkspace;
}

hipError_t launch_projection(const ProjArgs& p, hipStream_t s, char* err, size_t errlen) {
  const int HD = p.H * p.D, N3 = 3 * HD, NS = 2 * kProjRank + p.H;
  float* act = static_cast<float*>(p.ws);
  const size_t act_bytes = ((size_t)p.T * NS * sizeof(float) + 255) / 256 * 256;
  void* gws = static_cast<char*>(p.ws) + act_bytes;
  const size_t gwsb = p.ws_bytes - act_bytes;
  const bf16_t* w = static_cast<const bf16_t*>(p.w_in);
  const hipDataType dt = p.out_type == kBF16 ? HIP_R_16BF : HIP_R_32F;
  if (!gemm_xwt(p.T, p.hidden, N3, p.x, w, dt, p.qkv, N3, gws, gwsb, s, "hipblaslt_gemm[qkv]", err, errlen))
    return hipErrorUnknown;
  if (!gemm_xwt(p.T, p.hidden, NS, p.x, w + (long long)N3 * p.hidden, HIP_R_32F, act, NS, gws, gwsb, s,
                "hipblaslt_gemm[rank|beta]", err, errlen))
    return hipErrorUnknown;
  const dim3 grid(HD / PJ_COLS, (p.T + PJ_ROWS - 1) / PJ_ROWS, 2);
  timing_begin("kda_proj_lowrank_kernel", s);
  if (p.out_type == kBF16)
    kda_proj_lowrank_kernel<bf16_t><<<grid, PJ_NT, 0, s>>>(
        act, NS, p.T, HD, p.H, static_cast<const bf16_t*>(p.w_fb), static_cast<const bf16_t*>(p.w_gb),
        static_cast<bf16_t*>(p.f), static_cast<bf16_t*>(p.g), static_cast<bf16_t*>(p.beta));
  else
    kda_proj_lowrank_kernel<float><<<grid, PJ_NT, 0, s>>>(
        act, NS, p.T, HD, p.H, static_cast<const bf16_t*>(p.w_fb), static_cast<const bf16_t*>(p.w_gb),
        static_cast<float*>(p.f), static_cast<float*>(p.g), static_cast<float*>(p.beta));
  timing_end(s);
  return hipGetLastError();
}

}  // namespace kda
