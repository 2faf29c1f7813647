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
constexpr int PJ_XCD = 8;               // L2 domains the workgroups are dealt over, round robin

__device__ __forceinline__ f32x4 pj_mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void pj_store(float* p, float v) { *p = v; }
__device__ __forceinline__ void pj_store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
// four consecutive outputs of one token
__device__ __forceinline__ void pj_store4(float* p, f32x4 v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void pj_store4(bf16_t* p, f32x4 v) {
  uint2 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = u;
}

// out[T, HD] = act[T, R] . W^T for W [HD, R] (a Linear weight), act the fp32 rank activations
// (columns which*R .. which*R + R - 1 of the workspace rows, leading dimension ld), f for which = 0
// and g for which = 1.  A workgroup multiplies one 64-token tile by one 128-column block of W held
// in LDS.  The product is taken transposed (out^T tile = W tile . act^T) so that each lane ends
// with four consecutive output columns of one token and stores them directly.
//
// Workgroup b runs on L2 domain b % 8 and takes a row tile = b % 8 modulo 8, so one domain's L2
// holds the activations of its own row tiles only, beside the 2 MB of weights; within a domain
// the (column block, which) pairs run fastest.  The workgroups of column block 0 of f also write
// beta = sigmoid(b x) for their tile.
template <typename OT>
__global__ __launch_bounds__(PJ_NT) void kda_proj_lowrank_kernel(const float* __restrict__ act, int ld, int T,
                                                                 int HD, int H, const bf16_t* __restrict__ w_fb,
                                                                 const bf16_t* __restrict__ w_gb, OT* __restrict__ f,
                                                                 OT* __restrict__ g, OT* __restrict__ beta) {
  constexpr int R = kProjRank;
  __shared__ __align__(16) __bf16 sW[PJ_COLS * PJ_PB];
  const int ncb2 = 2 * (HD / PJ_COLS);
  const int xcd = blockIdx.x % PJ_XCD, k = blockIdx.x / PJ_XCD;
  const int r0 = ((k / ncb2) * PJ_XCD + xcd) * PJ_ROWS;
  if (r0 >= T) return;  // the spare workgroups of the last domains
  const int which = k % 2, c0 = ((k % ncb2) / 2) * PJ_COLS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const bf16_t* W = which == 0 ? w_fb : w_gb;
  OT* out = which == 0 ? f : g;

  // the weight rows of this column block, 16-byte pieces (16 per row): all loads, then the LDS writes
  constexpr int NW = PJ_COLS * (R / 8) / PJ_NT;
  uint4 wv[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int i = tid + j * PJ_NT, row = i / (R / 8), seg = i % (R / 8);
    wv[j] = *reinterpret_cast<const uint4*>(W + (long long)(c0 + row) * R + seg * 8);
  }
  // this wave's 16 activation rows (rows past T read row T-1 and are not stored)
  const int trow = r0 + 16 * wave + l16;
  const float* ap = act + (long long)min(trow, T - 1) * ld + which * R + 8 * lg;
  float4 xv[R / 32][2];
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    xv[s][0] = *reinterpret_cast<const float4*>(ap + 32 * s);
    xv[s][1] = *reinterpret_cast<const float4*>(ap + 32 * s + 4);
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int i = tid + j * PJ_NT, row = i / (R / 8), seg = i % (R / 8);
    *reinterpret_cast<uint4*>(sW + row * PJ_PB + seg * 8) = wv[j];
  }
  // split B operands: fp32 activations as bf16 hi + lo
  bf16x8 xhi[R / 32], xlo[R / 32];
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    const float x[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w,
                        xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 hi = (__bf16)x[e];
      xhi[s][e] = hi;
      xlo[s][e] = (__bf16)(x[e] - (float)hi);
    }
  }
  __syncthreads();
  f32x4 acc[PJ_COLS / 16];
#pragma unroll
  for (int ct = 0; ct < PJ_COLS / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < R / 32; ++s)
#pragma unroll
    for (int ct = 0; ct < PJ_COLS / 16; ++ct) {
      const bf16x8 w = *reinterpret_cast<const bf16x8*>(sW + (16 * ct + l16) * PJ_PB + 32 * s + 8 * lg);
      acc[ct] = pj_mfma(w, xlo[s], acc[ct]);
      acc[ct] = pj_mfma(w, xhi[s], acc[ct]);
    }
  // lane: output columns 16 ct + 4 lg .. + 3 of token trow
  if (trow < T) {
    OT* orow = out + (long long)trow * HD + c0 + 4 * lg;
#pragma unroll
    for (int ct = 0; ct < PJ_COLS / 16; ++ct) pj_store4(orow + 16 * ct, acc[ct]);
  }
  if (which == 0 && c0 == 0) {
    for (int i0 = 0; i0 < PJ_ROWS * H; i0 += 4 * PJ_NT) {
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + tid + e * PJ_NT, row = r0 + i / H;
        z[e] = (i < PJ_ROWS * H && row < T) ? act[(long long)row * ld + 2 * R + i % H] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + tid + e * PJ_NT, row = r0 + i / H;
        if (i < PJ_ROWS * H && row < T) pj_store(beta + (long long)row * H + i % H, 1.0f / (1.0f + __expf(-z[e])));
      }
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
// A GEMM is resolved (descriptors and algorithm) before anything is launched, so that a call whose
// second GEMM has no algorithm fails with no buffer touched.  The algorithm is chosen within
// kProjGemmWorkspace bytes, the library's share of every valid workspace, so an algorithm cached
// under one call fits every later call of the same shape.
struct Gemm {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  Gemm() = default;
  Gemm(const Gemm&) = delete;
  Gemm& operator=(const Gemm&) = delete;
  ~Gemm() {
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

bool lt_handle(char* err, size_t errlen) {
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
  return true;
}

bool gemm_resolve(Gemm& g, int T, int k, int m, hipDataType dtype, int ldd, char* err, size_t errlen) {
  bool ok = true;
  LT_TRY(hipblasLtMatmulDescCreate(&g.op, HIPBLAS_COMPUTE_32F, HIP_R_32F), "desc");
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  if (ok) LT_TRY(hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)), "transa");
  if (ok) LT_TRY(hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)), "transb");
  if (ok) LT_TRY(hipblasLtMatrixLayoutCreate(&g.la, HIP_R_16BF, k, m, k), "layout A");
  if (ok) LT_TRY(hipblasLtMatrixLayoutCreate(&g.lb, HIP_R_16BF, k, T, k), "layout B");
  if (ok) LT_TRY(hipblasLtMatrixLayoutCreate(&g.ld, dtype, m, T, ldd), "layout D");
  if (!ok) return false;
  const GemmKey key{m, T, k, ldd, (int)dtype};
  auto it = g_lt.algos.find(key);
  if (it != g_lt.algos.end()) {
    g.algo = it->second;
    return true;
  }
  hipblasLtMatmulPreference_t pref = nullptr;
  LT_TRY(hipblasLtMatmulPreferenceCreate(&pref), "preference");
  const uint64_t cap = kProjGemmWorkspace;
  if (ok)
    LT_TRY(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap)),
           "workspace preference");
  hipblasLtMatmulHeuristicResult_t res{};
  int nres = 0;
  if (ok) LT_TRY(hipblasLtMatmulAlgoGetHeuristic(g_lt.handle, g.op, g.la, g.lb, g.ld, g.ld, pref, 1, &res, &nres),
                 "heuristic");
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ok && (nres < 1 || res.state != HIPBLAS_STATUS_SUCCESS || res.workspaceSize > kProjGemmWorkspace)) {
    snprintf(err, errlen, "hipBLASLt has no algorithm for this GEMM within %zu workspace bytes", kProjGemmWorkspace);
    ok = false;
  }
  if (ok) {
    g.algo = res.algo;
    g_lt.algos[key] = g.algo;
  }
  return ok;
}

bool gemm_run(const Gemm& g, const void* X, const void* Wr, void* D, void* ws, hipStream_t s, const char* name,
              char* err, size_t errlen) {
  bool ok = true;
  const float one = 1.f, zero = 0.f;
  timing_begin(name, s);
  LT_TRY(hipblasLtMatmul(g_lt.handle, g.op, &one, Wr, g.la, X, g.lb, &zero, D, g.ld, D, g.ld, &g.algo, ws,
                         kProjGemmWorkspace, s),
         "matmul");
  timing_end(s);
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
  const bf16_t* w = static_cast<const bf16_t*>(p.w_in);
  const hipDataType dt = p.out_type == kBF16 ? HIP_R_16BF : HIP_R_32F;
  // both GEMMs are resolved before the first launch
  if (!lt_handle(err, errlen)) return hipErrorUnknown;
  Gemm g_qkv, g_rank;
  if (!gemm_resolve(g_qkv, p.T, p.hidden, N3, dt, N3, err, errlen)) return hipErrorUnknown;
  if (!gemm_resolve(g_rank, p.T, p.hidden, NS, HIP_R_32F, NS, err, errlen)) return hipErrorUnknown;
  if (!gemm_run(g_qkv, p.x, w, p.qkv, gws, s, "hipblaslt_gemm[qkv]", err, errlen)) return hipErrorUnknown;
  if (!gemm_run(g_rank, p.x, w + (long long)N3 * p.hidden, act, gws, s, "hipblaslt_gemm[rank|beta]", err, errlen))
    return hipErrorUnknown;
  // per domain ceil(tiles / 8) row tiles, times the (column block, which) pairs
  const int tiles = (p.T + PJ_ROWS - 1) / PJ_ROWS;
  const dim3 grid(((tiles + PJ_XCD - 1) / PJ_XCD) * PJ_XCD * 2 * (HD / PJ_COLS));
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
