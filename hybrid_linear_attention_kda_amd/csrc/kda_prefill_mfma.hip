// Chunked KDA prefill on bf16 MFMA for d_k = d_v = 128, chunk 64, bf16 io (gfx950).
//
// The recurrence in chunked WY/UT form (chunk of C = 64 tokens, Gam = inclusive
// cumulative log-decay per key channel, S = chunk-start state):
//   A_kk[i,j] = beta_i sum_c k_i k_j e^(Gam_i - Gam_j)   (j < i)
//   A_qk[i,j] =        sum_c q_i k_j e^(Gam_i - Gam_j)   (j <= i)
//   T = (I + A_kk)^-1,   W = T (beta K e^Gam),   Ut = T (beta V)
//   U = Ut - W S,   O = (Q e^Gam) S + A_qk U,   S <- e^(Gam_C) S + (K e^(Gam_C - Gam))^T U
// The layer around it follows llama.cpp PR #27754 "model: add GLM-5-Next
// (GLM-5.3-Flash)", KDA commit (depthwise conv over q|k|v, SiLU, L2 with
// max(||x||, eps), bounded-sigmoid per-channel decay on the key axis, gated
// output RMSNorm with a plain weight).
//
// O is taken as written, Q~ S + A_qk U: U is formed in the sequential part anyway, so the
// chunk-parallel part needs no product with A_qk beyond A_qk itself.
//
// Two phases.
//  A (chunk-parallel: persistent workgroups, one per CU, looping over the
//    (sequence, head, chunk) tasks chunk-major from the last chunk down, so that
//    the tiles B reads first were written last and are still in the last-level
//    cache): conv + SiLU,
//    L2 norms, gate and its cumulative sum, A_kk, T, A_qk, W and Ut = T (beta V),
//    with Q~ = Q e^Gam and K~ = K e^(Gam_C - Gam).  Everything that does not
//    depend on the state is written to the workspace once per chunk: Q~, W, K~^T
//    (transposed), Ut and A_qk as fp16, e^Gam_C as fp32, each in the order the
//    matrix cores consume it.
//  B (sequential over chunks, one workgroup per (sequence, head, 16-column
//    block of d_v); with a sequence table, per group of consecutive sequences,
//    whose chunks it runs as one stream): per chunk
//      U = Ut - W S,  O = Q~ S + A_qk U,  S <- e^Gam_C S + K~^T U,
//    with the 128 x 16 state block in MFMA accumulators and the operands of
//    chunk c+1 loaded into registers while chunk c is computed.  blockIdx.x =
//    vb * H + h, so with H a multiple of 8 the eight workgroups of a head run on
//    one XCD and share its L2 for the operand tiles.
//
// Per-channel decay inside MFMA tiles (phase A).  The chunk is cut into four
// 16-token sub-chunks anchored at their first token n(I).  Operands carry
// e^(Gam_i - Gam_n(I)) (<= 1) on rows and e^(Gam_n(J) - Gam_j) (<= e^(15|lb|))
// on columns, and block (I, J) of A multiplies the row operand by the
// per-channel factor e^(Gam_n(I) - Gam_n(J)) (<= 1).  With the bounded gate
// (|lb| <= 5.5) every factor stays a finite fp32 / bf16 number.  The softplus decay
// branch (llama.cpp PR #27754, metadata commit: the function taken without a lower
// bound) has no such bound; its instance anchors the columns at the end of their
// sub-chunk instead, which keeps every off-diagonal factor <= 1, and sums the four
// diagonal blocks exactly per channel (see kda_chunk_prep_kernel).
//
// Precision.  bf16 operands round to 8 bits; A_qk is formed on split bf16 (x = hi
// + lo, three MFMAs: hi.hi + hi.lo + lo.hi), A_kk in plain bf16, and T in fp32.
// The products of phase A that use them (W = T X, Ut = T (beta V)) take T as fp16
// (11 significant bits) and the other operand split into fp16 hi + lo (~22 bits),
// two MFMAs each, as phase B does.  Phase B's products (W S, Q~ S, A_qk U, K~^T U) take
// W, Q~, A_qk and K~^T as fp16 (11 significant bits, half the bytes of a split bf16 pair
// on the per-chunk operand path) and S or U split into fp16 hi + lo (~22 bits),
// two MFMAs each.  fp16's range holds these values: |q| and |k| are at most
// 1 after the L2 norm, and the delta rule keeps every state entry within the
// value vectors' scale (the largest |S| over the 4096- and 32768-token workloads
// is below 2).
//
// The output RMSNorm needs all 128 columns of o, which live in eight
// workgroups, so o goes to the workspace as fp16 (11 significant bits; |o| stays far inside
// fp16's range) and a third, bandwidth-bound kernel applies the norm,
// weight and gate.  Phase B's loader waves also write the new conv state.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int D = 128;       // head size (d_k = d_v)
constexpr int C = 64;        // chunk
constexpr int NVB = 16;      // d_v columns per phase-B workgroup
constexpr int NBLK = D / NVB; // phase-B workgroups per head
constexpr int NT = 512;      // lanes
constexpr int HALO = 3;      // staged rows before the chunk (conv width <= 4)

constexpr int PQ = 132;      // fp32 pitch of [64][128] arrays
constexpr int PKB = 136;     // bf16 pitch of [64][128] arrays
constexpr int PA = 68;       // fp32 pitch of [64][64] arrays
constexpr int PTB = 72;      // fp16 pitch of the [64][64] T and A_qk planes (row r starts 36 r banks on)
constexpr int PXT = 68;      // bf16 pitch of the transposed [128][64] X planes (8-byte aligned rows)
constexpr int PR = 280;      // bf16 pitch of the raw staging rows: q 128 | k 128 | v 16 | pad
constexpr int RROWS = C + HALO;

// Phase A LDS layout (bytes)
constexpr int OFF_Q = 0;                              // q^ -> QR = q e^(Gam - Gam_n) -> P
constexpr int OFF_KB = OFF_Q + C * PQ * 4;            // KR (bf16) -> W (bf16)
constexpr int OFF_G = OFF_KB + C * PKB * 2;           // KC = k e^(Gam_n - Gam) as bf16 hi | lo [2][64][PKB] -> raw v rows
constexpr int OFF_STG = OFF_G + 2 * C * PKB * 2;      // raw q|k staging | A_kk + T (-> T split planes)
constexpr int STG_BYTES = RROWS * PR * 2;             // 37520 >= 2 * C * PA * 4 and >= C * PQ * 4
constexpr int OFF_TMP = OFF_STG + STG_BYTES;          // scratch while forming T [1024]
constexpr int OFF_GN = OFF_TMP + 1024 * 4;            // log-decay of each sub-chunk's first token [4][128] (+ spare)
constexpr int OFF_EN = OFF_GN + 5 * D * 4;            // e^(Gam_n(I)) [4][128]
constexpr int OFF_E = OFF_EN + 4 * D * 4;             // e^(Gam_n(I) - Gam_n(J)), I > J [6][128]
constexpr int OFF_FAC = OFF_E + 6 * D * 4;            // spare [4][128]
constexpr int OFF_GC = OFF_FAC + 4 * D * 4;           // e^(Gam_C) [128]
constexpr int OFF_BETA = OFF_GC + D * 4;              // [64]
constexpr int OFF_NRM = OFF_BETA + C * 4;             // spare [2][64]
constexpr int OFF_SEG = OFF_NRM + 2 * C * 4;          // cumulative-sum segment totals [4][128]
constexpr int OFF_AQK = OFF_SEG + 4 * D * 4;           // f [64][PKB] bf16 -> A_qk [64][PTB] fp16 (formed while T is)
constexpr int OFF_GA = OFF_AQK + C * PA * 4;           // per-wave squared-norm sums, then normalisers [2][8][32]
constexpr int LDS_A = OFF_GA + 4 * D * 4;
static_assert(STG_BYTES >= 2 * C * PA * 4, "staging aliases");
static_assert(C * PTB * 2 <= C * PA * 4, "the fp16 T and A_qk planes fit their regions");
static_assert(D * PXT * 2 <= C * PKB * 2 && D * PXT * 2 <= 2 * C * PKB * 2, "X planes alias KR and the KC planes");
static_assert(C * PKB * 2 <= C * PA * 4 && (RROWS) * PKB * 2 <= 2 * C * PKB * 2, "W aliases the fp32 T, the v rows the KC planes");
static_assert(LDS_A <= 160 * 1024, "LDS budget");

// Workspace tile block per (sequence, head, chunk), written by phase A and read by phase B.
// Every fp16 matrix is stored in MFMA fragment order: fragment f = (row / 16) * (K / 32) + k / 32
// of a [rows][K] operand holds, for lane l, the 8 elements (row 16*(f / (K/32)) + l % 16,
// k = 32*(f % (K/32)) + 8*(l / 16) + 0..7), so a wave loads one fragment as 1 KB contiguous.
// The fp32 [64][128] matrices are stored as 16 x 16 accumulator tiles (I, j), tile-major
// (I * 8 + j), lane l holding rows 16 I + 4 (l / 16) + 0..3 of column 16 j + l % 16.
constexpr int W_QT = 0;                    // Q~ = Q e^Gam [64][128] fp16 (16 fragments)
constexpr int W_KTHI = W_QT + C * D * 2;   // K~^T [128][64] fp16
constexpr int W_W = W_KTHI + D * C * 2;    // W [64][128] fp16
constexpr int W_UT = W_W + C * D * 2;      // Ut = T (beta V) [64][128] fp16, accumulator-fragment order,
                                           // column tile major (a column tile's 4 row tiles are 2 KB)
constexpr int W_AQK = W_UT + C * D * 2;    // A_qk [64][64] fp16 (8 fragments; (0, 1) and (1, 1), above
                                           // the diagonal, hold zeros)
constexpr int W_GC = W_AQK + C * C * 2;    // e^Gam_C [128] fp32
constexpr int CH_BYTES = W_GC + D * 4;     // 74240
static_assert(CH_BYTES % 256 == 0, "tile blocks stay 256-byte aligned");

// Phase B: 8 compute waves and 4 loader waves per workgroup.
constexpr int NTB = 768;
constexpr int PVT = 72;                    // fp16 pitch of the [16][64] token-major U operand
constexpr int PST = 136;                   // fp16 pitch of the [16][128] state operand
// Phase B LDS layout (bytes): U and S operands (fp16 hi / lo), a scratch line for cache-warming
// loads, then the buffers of the tiles the loader waves bring in (W, this block's Ut, K~^T,
// e^Gam_C), each byte-for-byte as in the workspace (1 KB fragments).
constexpr int B_UHI = 0;
constexpr int B_ULO = B_UHI + NVB * PVT * 2;
constexpr int B_SHI = B_ULO + NVB * PVT * 2;
constexpr int B_SLO = B_SHI + NVB * PST * 2;
constexpr int B_TRASH = B_SLO + NVB * PST * 2;   // 256 B, written by warming loads, never read
// W and Ut are read before barrier (b), K~^T and e^Gam_C after it, so they sit in separate
// buffers: two of W | Ut (each copied a chunk and a half ahead) and two of K~^T | e^Gam_C.
constexpr int WU_W = 0;
constexpr int WU_UT = WU_W + C * D * 2;
constexpr int WU_BYTES = WU_UT + 4 * 512;        // 18432
constexpr int KB_KHI = 0;
constexpr int KB_GC = KB_KHI + D * C * 2;
constexpr int KB_BYTES = KB_GC + D * 4;          // 16896
constexpr int B_WU0 = B_TRASH + 256;
constexpr int B_KB0 = B_WU0 + 2 * WU_BYTES;
constexpr int LDS_B = B_KB0 + 2 * KB_BYTES;
static_assert(NVB == 16, "one accumulator column tile per phase-B workgroup");
static_assert(B_WU0 % 16 == 0 && WU_BYTES % 16 == 0 && KB_BYTES % 16 == 0, "16-byte aligned tile buffers");
static_assert(LDS_B <= 160 * 1024, "LDS budget");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// The depthwise conv on bf16 pairs: a.x * b.x + a.y * b.y + c (products exact in fp32).
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
// a.x * b.x + a.y * b.y with the zero addend as an inline constant (the accumulating form would
// first have to move a zero into its destination)
__device__ __forceinline__ float dot2z(bf16x2 a, bf16x2 b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// (x.y, y.x): the pair between two consecutive pairs of a column
__device__ __forceinline__ bf16x2 mid_pair(bf16x2 x, bf16x2 y) {
  return __builtin_bit_cast(bf16x2, __builtin_amdgcn_alignbit(__builtin_bit_cast(uint32_t, y),
                                                               __builtin_bit_cast(uint32_t, x), 16));
}

struct Split8 {
  bf16x8 hi, lo;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp16 operands (the phase-B products): 11 significant bits, with the state-side operand split
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 to_f16x8(const float (&x)[8]) {
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
  return h;
}
// hi.hi + hi.lo + lo.hi: about 16 significant bits per operand
__device__ __forceinline__ f32x4 mfma3(const Split8& a, const Split8& b, f32x4 c) {
  c = mfma(a.lo, b.hi, c);
  c = mfma(a.hi, b.lo, c);
  return mfma(a.hi, b.hi, c);
}
__device__ __forceinline__ Split8 split(const float (&x)[8]) {
  Split8 s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)x[e];
    s.hi[e] = h;
    s.lo[e] = (__bf16)(x[e] - (float)h);
  }
  return s;
}
// fp16 hi + lo of 8 values (~22 significant bits): the B operands of the products with an fp16 A
struct Half8 {
  f16x8 hi, lo;
};
__device__ __forceinline__ Half8 split16(const float (&x)[8]) {
  Half8 s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 h = (_Float16)x[e];
    s.hi[e] = h;
    s.lo[e] = (_Float16)(x[e] - (float)h);
  }
  return s;
}
// A (fp16) times B (fp16 hi + lo): the small term first
__device__ __forceinline__ f32x4 mfma2h(f16x8 a, const Half8& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b.lo, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b.hi, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 round8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// 8 bf16 at p and at p + off2 (4 + 4 elements), rows of 8-byte alignment
__device__ __forceinline__ bf16x8 ld4x2(const __bf16* p, int off2) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + off2);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f16x8 ld4x2(const _Float16* p, int off2) {
  const f16x4 a = *reinterpret_cast<const f16x4*>(p);
  const f16x4 b = *reinterpret_cast<const f16x4*>(p + off2);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// fp32 matrix core step: D += A[16 x 4] B[4 x 16]; lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Orders this wave's LDS writes before its later LDS reads (other waves are not waited for).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Cross-lane steps of the wave reduce-scatter below.
__device__ __forceinline__ float dpp_ror8(float x) {  // lane l <- lane l ^ 8 (rotation by 8 in a row of 16)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {  // quad_perm [2, 3, 0, 1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_xor1(float x) {  // quad_perm [1, 0, 3, 2]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float swz_xor4(float x) {  // ds_swizzle bit mode, xor mask 4
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1f));
}
// Reduce-scatter over the wave: every lane holds v[0..63]; lane l returns the sum over the 64
// lanes of v[l].  Each step halves the values a lane holds: the lanes whose step bit is set keep
// the upper half, and add the partner's copy of it (permlane32 / permlane16 swaps exchange two
// registers' halves at once; the steps inside a row of 16 use DPP and swizzle).
__device__ __forceinline__ float reduce_scatter64(float (&v)[64], int lane) {
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 32]), false, false);
    v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 16]), false, false);
    v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
#pragma unroll
  for (int m = 0; m < 8; ++m) v[m] = (b3 ? v[m + 8] : v[m]) + dpp_ror8(b3 ? v[m] : v[m + 8]);
#pragma unroll
  for (int m = 0; m < 4; ++m) v[m] = (b2 ? v[m + 4] : v[m]) + swz_xor4(b2 ? v[m] : v[m + 4]);
#pragma unroll
  for (int m = 0; m < 2; ++m) v[m] = (b1 ? v[m + 2] : v[m]) + dpp_xor2(b1 ? v[m] : v[m + 2]);
  return (b0 ? v[1] : v[0]) + dpp_xor1(b0 ? v[0] : v[1]);
}

// The same over 32 values: lane l returns the sum over the 64 lanes of v[l / 2] (lanes 2m and 2m + 1
// hold the same sum; the last step adds the partner's copy of the one value left).
__device__ __forceinline__ float reduce_scatter32(float (&v)[32], int lane) {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 16]), false, false);
    v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 8]), false, false);
    v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
  for (int m = 0; m < 4; ++m) v[m] = (b3 ? v[m + 4] : v[m]) + dpp_ror8(b3 ? v[m] : v[m + 4]);
#pragma unroll
  for (int m = 0; m < 2; ++m) v[m] = (b2 ? v[m + 2] : v[m]) + swz_xor4(b2 ? v[m] : v[m + 2]);
  const float x = (b1 ? v[1] : v[0]) + dpp_xor2(b1 ? v[0] : v[1]);
  return x + dpp_xor1(x);
}

// Softplus branch, exact diagonal sub-chunk blocks: the values of one 16-token sub-chunk are
// enumerated column by column, n = 0..255: for column j, A_qk(j, j), then for each row i > j
// A_kk(i, j) and A_qk(i, j).  Column j starts at n = 32 j - j^2.
__device__ __forceinline__ void diag_entry(int n, bool& qk, int& i, int& j) {
  j = 0;
#pragma unroll
  for (int jj = 1; jj < 16; ++jj) j += (32 * jj - jj * jj <= n) ? 1 : 0;
  const int r = n - (32 * j - j * j);
  i = r == 0 ? j : j + 1 + ((r - 1) >> 1);
  qk = r == 0 || ((r - 1) & 1);
}

// Element offset of (row, k .. k+7) (k a multiple of 8) in the fragment-order layout of a
// [rows][K] operand.
__device__ __forceinline__ int frag_offset(int row, int k, int K) {
  const int f = (row >> 4) * (K >> 5) + (k >> 5);
  const int lane = (row & 15) + 16 * ((k & 31) >> 3);
  return (f * 64 + lane) * 8;
}

// (I, J) of the ten lower sub-chunk blocks, and the index of the factor table for I > J.
__device__ __forceinline__ void block_ij(int bi, int& I, int& J) {
  I = bi < 1 ? 0 : bi < 3 ? 1 : bi < 6 ? 2 : 3;
  J = bi - I * (I + 1) / 2;
}
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

__device__ __forceinline__ float silu_fast(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// 2^x on v_exp_f32 (the decay factors of phase A are formed from base-2 log-decays)
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }


// ---------------------------------------------------------------------------------------------
// Phase A: persistent workgroups (one per CU) loop over the tasks (chunk, head, sequence); the
// global inputs of the next task are loaded into registers while the current one is computed.
// ---------------------------------------------------------------------------------------------
constexpr int NRAW = (RROWS * 16 + NT - 1) / NT;  // raw q and k row-segment loads per lane
constexpr int NRV = (RROWS * 16 + NT - 1) / NT;   // raw v row loads per lane

struct PrepTask {
  int h, b, ci;
};
// Tasks run head-fastest and chunk-major from the last chunk down (within each sequence of a
// uniform batch; over the whole launch with a table), so that the tiles phase B reads first were
// written last and are still in the last-level cache.
template <bool VL>
__device__ __forceinline__ PrepTask prep_task(int task, int H, int NC, const SeqTab& st) {
  PrepTask k;
  k.h = task % H;
  const int r = task / H;
  if (!VL) {
    k.ci = NC - 1 - r % NC;
    k.b = r / NC;
  } else {
    // the launch's chunks from its last one down: the sequence holding chunk gc is the last i
    // with chunk0[i] <= gc (the state pass reads each group of sequences from its first chunk up)
    const int gc = st.total_chunks - 1 - r;
    int lo = 0, hi = st.n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (st.chunk0[mid] <= gc)
        lo = mid;
      else
        hi = mid - 1;
    }
    k.b = lo;
    k.ci = gc - st.chunk0[lo];
  }
  return k;
}

// The global inputs of one task, as loaded: 16-byte loads only (addresses clamped into the
// sequence and into the parameter blocks; rows outside the sequence are replaced when staged).
struct PrepIn {
  uint4 raw[NRAW][2];  // raw rows c0-3 .. c0+63: lane task (row, 8-channel segment), q then k
  uint4 rawv[NRV];   // raw v rows, the same way
  uint4 f[2];        // gate inputs of tokens c0 .. c0+63: lane task (token, 8-channel segment)
  uint4 par;         // 16 bytes of the head's parameter block (q, k, v conv taps, dt_bias)
  bf16_t beta;       // beta of token tid % 64
  float alog;        // A_log of the head
};

// Parameter block of a head in LDS: q taps [128][W], k taps, v taps (bf16), dt_bias [128] (fp32).
__device__ __forceinline__ int par_segments(int W) { return 48 * W + 32; }

// The loads of one task, in three groups (0: q|k rows, 1: v rows, 2: the rest) that the kernel
// issues at different points of the previous task, so that no phase carries all of them.
template <bool VL>
__device__ __forceinline__ void prep_issue(const LayerArgs& a, const SeqTab& st, const PrepTask& k, int tid, PrepIn& in,
                                           int part) {
  const SeqView sv = seq_view<VL>(st, k.b, a.T, 0);
  const int H = a.H, T = sv.len, W = a.W, HD = H * D, Cq = 3 * HD;
  const int h = k.h, c0 = k.ci * C;
  const bf16_t* __restrict__ qkv = static_cast<const bf16_t*>(a.qkv) + sv.tok0 * Cq;
  if (part == 0) {
#pragma unroll
    for (int s = 0; s < NRAW; ++s) {
      const int r = min((tid + s * NT) >> 4, RROWS - 1), sg = tid & 15;
      const int tt = min(max(c0 - HALO + r, 0), T - 1);
      const bf16_t* row = qkv + (long long)tt * Cq + h * D + sg * 8;
      in.raw[s][0] = *reinterpret_cast<const uint4*>(row);
      in.raw[s][1] = *reinterpret_cast<const uint4*>(row + HD);
    }
  } else if (part == 1) {
#pragma unroll
    for (int s = 0; s < NRV; ++s) {
      const int r = min((tid + s * NT) >> 4, RROWS - 1), sg = tid & 15;
      const int tt = min(max(c0 - HALO + r, 0), T - 1);
      in.rawv[s] = *reinterpret_cast<const uint4*>(qkv + (long long)tt * Cq + 2LL * HD + h * D + sg * 8);
    }
  } else {
    const bf16_t* __restrict__ fin = static_cast<const bf16_t*>(a.f) + sv.tok0 * HD + h * D;
    const bf16_t* __restrict__ bin = static_cast<const bf16_t*>(a.beta) + sv.tok0 * H + h;
    const bf16_t* __restrict__ cw = static_cast<const bf16_t*>(a.conv_w);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int t = (tid + s * NT) >> 4, sg = tid & 15;
      in.f[s] = *reinterpret_cast<const uint4*>(fin + (long long)min(c0 + t, T - 1) * HD + sg * 8);
    }
    {
      // segment p of the parameter block: 16 W segments per tap block, then 32 of dt_bias
      const int p = min(tid, par_segments(W) - 1);
      const int blkw = 16 * W;
      const uint4* src;
      if (p < 3 * blkw) {
        const int which = p / blkw, o = p - which * blkw;
        src = reinterpret_cast<const uint4*>(cw + ((long long)which * HD + h * D) * W) + o;
      } else {
        src = reinterpret_cast<const uint4*>(a.dt_bias + h * D) + (p - 3 * blkw);
      }
      in.par = *src;
    }
    in.beta = bin[(long long)min(c0 + (tid & 63), T - 1) * H];
    in.alog = a.A_log[h];
  }
}

// VL: the launch carries a sequence table (variable-length call); otherwise a.B sequences of a.T.
// GK: the gate and its factoring.  0: the bounded sigmoid with -5.5 <= lb <= 0, start-anchored
// sub-chunks.  1: the softplus decay branch (no lower bound).  2: the bounded sigmoid with lb < -5.5.
// Under kinds 1 and 2 a 16-token sub-chunk can decay past the range of fp32 (e^-88), so the
// factoring changes: key columns are anchored at the END of their sub-chunk (every off-diagonal
// factor is then <= 1, whatever the gate), and the four diagonal 16 x 16 blocks of A_kk and A_qk,
// which no single anchor keeps finite, are summed exactly per channel (pairwise decay as running
// products of the per-token decays) and reduced across the channels' lanes.
template <bool VL, int GK>
__global__ __launch_bounds__(NT) void kda_chunk_prep_kernel(LayerArgs a, SeqTab st, unsigned char* __restrict__ ws) {
  constexpr bool SP = GK != 0;  // end-anchored columns, exact diagonal blocks
  extern __shared__ __align__(16) unsigned char smem[];
  float* sQ = reinterpret_cast<float*>(smem + OFF_Q);
  __bf16* sKb = reinterpret_cast<__bf16*>(smem + OFF_KB);
  __bf16* sKChi = reinterpret_cast<__bf16*>(smem + OFF_G);  // KC split planes [64][PKB]
  __bf16* sKClo = sKChi + C * PKB;
  __bf16* sRaw = reinterpret_cast<__bf16*>(smem + OFF_STG);
  float* sAkk = reinterpret_cast<float*>(smem + OFF_STG);
  float* sT = reinterpret_cast<float*>(smem + OFF_STG + C * PA * 4);
  _Float16* sA16 = reinterpret_cast<_Float16*>(smem + OFF_AQK);  // A_qk [64][PTB] fp16
  _Float16* sT16 = reinterpret_cast<_Float16*>(smem + OFF_STG);  // T [64][PTB] fp16, in place of A_kk
  float* sTmp = reinterpret_cast<float*>(smem + OFF_TMP);
  float* sEn = reinterpret_cast<float*>(smem + OFF_EN);
  float* sE = reinterpret_cast<float*>(smem + OFF_E);
  float* sGC = reinterpret_cast<float*>(smem + OFF_GC);
  float* sBeta = reinterpret_cast<float*>(smem + OFF_BETA);
  float* sSeg = reinterpret_cast<float*>(smem + OFF_SEG);

  const int H = a.H, W = a.W;
  const int NC = (a.T + C - 1) / C;  // chunks per sequence of a uniform launch
  const int ntask = (VL ? st.total_chunks : a.B * NC) * H;
  const int HD = H * D, Cq = 3 * HD;

  PrepIn cur;
  {
    const PrepTask k0 = prep_task<VL>(min((int)blockIdx.x, ntask - 1), H, NC, st);
    prep_issue<VL>(a, st, k0, (int)threadIdx.x, cur, 0);
    prep_issue<VL>(a, st, k0, (int)threadIdx.x, cur, 1);
    prep_issue<VL>(a, st, k0, (int)threadIdx.x, cur, 2);
    // the first task's inputs are awaited here, so that inside the loop the waits for a task's
    // inputs count only the loads and stores issued after them in the previous task (without
    // it the loop entry would force a wait for every outstanding access, the previous task's
    // tile stores included)
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  }
  for (int tk = blockIdx.x; tk < ntask; tk += gridDim.x) {
    // lane indices are re-derived per task from an opaque copy, so that the address arithmetic
    // built on them is not hoisted out of the loop and held in registers across it
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;  // MFMA row/column index and k-group
    const PrepTask ktask = prep_task<VL>(tk, H, NC, st);
    const int h = ktask.h, ci = ktask.ci;
    const SeqView sv = seq_view<VL>(st, ktask.b, a.T, NC);
    const int T = sv.len;  // this sequence's tokens
    const int c0 = ci * C;
    const int L = min(C, T - c0);
    const bf16_t* __restrict__ cin = static_cast<const bf16_t*>(a.conv_in) + (long long)sv.slot * Cq * (W - 1);
    // chunk blocks of a sequence: head-major, then chunk
    unsigned char* __restrict__ blk =
        ws + ((long long)sv.chunk0 * H + (long long)h * ((T + C - 1) / C) + ci) * (long long)CH_BYTES;

    // ---- P1: stage this task's raw q | k rows for tokens c0-3 .. c0+63 with q and k of each
    //      channel side by side (one 32-bit word per channel: q low, k high), its gate inputs and
    //      its head's parameter block (bf16) from the registers loaded during the previous task ----
    __bf16* sF = reinterpret_cast<__bf16*>(smem + OFF_AQK);  // f [64][PKB] until A_qk is formed
    unsigned char* sPar = smem + OFF_TMP;                    // parameter block until T is formed
    float* sFirst = reinterpret_cast<float*>(smem + OFF_GN);  // log-decay of each sub-chunk's first token [4][128]
    float* sPart = reinterpret_cast<float*>(smem + OFF_GA);   // per-wave squared-norm sums [8][32], then normalisers [8][32]
    const float alog = cur.alog;
    // 8 q and 8 k values of one row as 8 (q, k) words
    auto stage_pairs = [&](__bf16* dst, uint4 q, uint4 k) __attribute__((always_inline)) {
      const uint32_t qw[4] = {q.x, q.y, q.z, q.w}, kw[4] = {k.x, k.y, k.z, k.w};
      uint32_t o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __builtin_amdgcn_perm(kw[e], qw[e], 0x05040100u);
        o[2 * e + 1] = __builtin_amdgcn_perm(kw[e], qw[e], 0x07060302u);
      }
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    };
#pragma unroll
    for (int s = 0; s < NRAW; ++s) {
      const int idx = tid + s * NT;
      if (idx < RROWS * 16) {
        const int r = idx >> 4, sg = idx & 15;
        const int tt = c0 - HALO + r;
        const bool in_seq = tt >= 0 && tt < T;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        stage_pairs(sRaw + r * PR + sg * 16, in_seq ? cur.raw[s][0] : z, in_seq ? cur.raw[s][1] : z);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int t = (tid + s * NT) >> 4, sg = tid & 15;
      *reinterpret_cast<uint4*>(sF + t * PKB + sg * 8) = cur.f[s];
    }
    if (tid < par_segments(W)) reinterpret_cast<uint4*>(sPar)[tid] = cur.par;
    if (ci == 0 && tid < HALO * 16) {
      // rows before the sequence start come from the conv state (the same lane wrote them as zeros)
      const int r = tid >> 4, sg = tid & 15;
      const int tt = r - HALO;
      if ((W - 1) + tt >= 0) {
        const long long ch = (long long)h * D + sg * 8;
        uint16_t eq[8], ek[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          eq[e] = cin[(ch + e) * (W - 1) + (W - 1) + tt];
          ek[e] = cin[(HD + ch + e) * (W - 1) + (W - 1) + tt];
        }
        stage_pairs(sRaw + r * PR + sg * 16,
                    make_uint4(eq[0] | (uint32_t)eq[1] << 16, eq[2] | (uint32_t)eq[3] << 16,
                               eq[4] | (uint32_t)eq[5] << 16, eq[6] | (uint32_t)eq[7] << 16),
                    make_uint4(ek[0] | (uint32_t)ek[1] << 16, ek[2] | (uint32_t)ek[3] << 16,
                               ek[4] | (uint32_t)ek[5] << 16, ek[6] | (uint32_t)ek[7] << 16));
      }
    }
    if (tid < C) sBeta[tid] = tid < L ? to_f32(cur.beta) : 0.f;
    __syncthreads();

    // From here to the A_kk blocks a lane owns key channel c = tid % 128 of q and k and the 16
    // tokens of segment seg = tid / 128 (sub-chunk seg), which is also the channel of the gate.
    const int c = tid & 127, seg = tid >> 7;
    // conv taps of this lane's q and k channels and of the v channel it converts in P9
    // (16 * wave + lane % 16), zero-padded on the left to 4 taps; read before T reuses the block;
    // taps as bf16 pairs (tap of the older token first): {t0, t1}, {t2, t3}
    bf16x2 ta01, ta23, tb01, tb23, tv01, tv23;
    {
      const __bf16* taps = reinterpret_cast<const __bf16*>(sPar);  // rows: q channels, k channels, v channels
      __bf16 ta[4], tb[4], tv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = max(j - (4 - W), 0);
        ta[j] = j >= 4 - W ? taps[c * W + w] : (__bf16)0.f;
        tb[j] = j >= 4 - W ? taps[(D + c) * W + w] : (__bf16)0.f;
        tv[j] = j >= 4 - W ? taps[(2 * D + 16 * wave + l16) * W + w] : (__bf16)0.f;
      }
      ta01 = bf16x2{ta[0], ta[1]};
      ta23 = bf16x2{ta[2], ta[3]};
      tb01 = bf16x2{tb[0], tb[1]};
      tb23 = bf16x2{tb[2], tb[3]};
      tv01 = bf16x2{tv[0], tv[1]};
      tv23 = bf16x2{tv[2], tv[3]};
    }
    const float* sDtb = reinterpret_cast<const float*>(sPar + 3 * D * W * 2);

    // ---- P2: causal conv + SiLU of q and k of channel c over the segment's 16 tokens, kept in
    //      registers.  Tokens past the sequence's end are not masked: beta is 0 there, so their
    //      rows of W and Ut, and with them their share of the state update, are exactly 0, and
    //      their outputs are not stored ----
    float qx[16], kx[16];
    {
      const int tb = 16 * seg;
      const uint32_t* col = reinterpret_cast<const uint32_t*>(sRaw + 2 * c);  // (q, k) of a row
      // the lane's 19 raw rows are read before any arithmetic, then regrouped per channel as
      // pairs pe[m] = (row 2m, row 2m+1) and, between them, po[m] = (row 2m+1, row 2m+2); output
      // row i takes pairs i and i+2
      uint32_t w[20];
#pragma unroll
      for (int r = 0; r < 19; ++r) w[r] = col[(tb + r) * (PR / 2)];
      w[19] = 0u;
      bf16x2 pa[10], pb[10], qa[9], qb[9];
#pragma unroll
      for (int m = 0; m < 10; ++m) {
        pa[m] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(w[2 * m + 1], w[2 * m], 0x05040100u));
        pb[m] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(w[2 * m + 1], w[2 * m], 0x07060302u));
      }
#pragma unroll
      for (int m = 0; m < 9; ++m) {
        qa[m] = mid_pair(pa[m], pa[m + 1]);
        qb[m] = mid_pair(pb[m], pb[m + 1]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = i >> 1;
        const float ya = (i & 1) ? dot2(ta23, qa[m + 1], dot2z(ta01, qa[m])) : dot2(ta23, pa[m + 1], dot2z(ta01, pa[m]));
        const float yb = (i & 1) ? dot2(tb23, qb[m + 1], dot2z(tb01, qb[m])) : dot2(tb23, pb[m + 1], dot2z(tb01, pb[m]));
        qx[i] = silu_fast(ya);
        kx[i] = silu_fast(yb);
      }
    }

    // ---- P3: bounded-sigmoid gate of channel c and its cumulative sum over the segment;
    //      gl[k] = Gam(16 seg + k) - Gam(16 seg - 1).  From here on every log-decay is held in
    //      base-2 units (Gam log2 e), so each decay factor is one v_exp_f32 ----
    float gl[16];
    float graw[16];  // softplus branch: this token's own log-decay, for the exact diagonal blocks
    {
      const float Ah = __expf(alog);
      const float dtb = sDtb[c];
      const float Ah2 = Ah * kLog2e, lb2 = a.lb * kLog2e;
      // the sigmoid's exponent -A (f + dt_bias) in base 2 as one fma of the raw f
      const float k1 = -Ah2, k2 = k1 * dtb;
      float acc = 0.f;
      // tokens past the sequence's end (a partial last chunk only) take no decay
      auto gate = [&](bool full) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float fr = (float)sF[(16 * seg + k) * PKB + c];
          const float fv = fr + dtb;
          // bounded sigmoid or softplus; under the end-anchored factoring floored at -100 (a decay
          // below e^-100 is zero at fp32 precision either way), which keeps the 16-token sums of
          // the log-decay well scaled
          const float gb = lb2 * __builtin_amdgcn_rcpf(1.0f + exp2f_(fmaf(fr, k1, k2)));
          const float g = GK == 1 ? fmaxf(-Ah2 * (fmaxf(fv, 0.f) + __logf(1.0f + __expf(-fabsf(fv)))), -100.f * kLog2e)
                        : GK == 2 ? fmaxf(gb, -100.f * kLog2e)
                                  : gb;
          const float gv = (full || 16 * seg + k < L) ? g : 0.f;
          acc += gv;
          gl[k] = acc;
          graw[k] = gv;
        }
      };
      if (L == C)
        gate(true);
      else
        gate(false);
      sSeg[seg * D + c] = acc;
      sFirst[seg * D + c] = gl[0];
    }
    // ---- P4 (same phase): squared norms of q and k per token, summed over this wave's 64
    //      channels (value m of the reduce-scatter: q of token m, k of token m - 16); lanes 2m and
    //      2m + 1 end with the sum m ----
    {
      float v[32];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[k] = qx[k] * qx[k];
        v[16 + k] = kx[k] * kx[k];
      }
      const float tot = reduce_scatter32(v, lane);
      if ((lane & 1) == 0) sPart[wave * 32 + (lane >> 1)] = tot;
    }
    __syncthreads();

    // the next task's inputs (the last task loads its own again: the loads stay unconditional),
    // issued in three groups spread over this task
    const PrepTask knext = prep_task<VL>(min(tk + (int)gridDim.x, ntask - 1), H, NC, st);
    PrepIn nxt;
    prep_issue<VL>(a, st, knext, tid, nxt, 0);

    // ---- P5: the segment offsets of the cumulative log-decay and the L2 normalisers, then the
    //      anchored operands QR, KR (bf16), KC (Gam_t - Gam_n(I) = gl[k] - gl[0]) and this
    //      lane's row of the per-channel factor tables ----
    float dpart[4];  // softplus branch: this lane's share of its wave's diagonal-block sums
    // X = beta K e^Gam (Gam from the chunk start) of this lane's channel and 16 tokens, in fp32: the
    // right-hand side of W = T X, kept in registers until T is formed
    float xk[16];
    {
      // Gam at each sub-chunk's first token (gn), at its last token (ga) and at the chunk end
      float off = 0.f, gn[4], ga[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const float segt = sSeg[J * D + c];
        gn[J] = sFirst[J * D + c] + off;
        ga[J] = segt + off;
        off += segt;
      }
      const float GC = ga[3];
      const float gn0 = gn[seg];
      const float egn = exp2f_(gn0);
      // 1 / max(||x||, eps) = min(1 / ||x||, 1 / eps) (rsq(0) is +inf): the two waves of the
      // segment hold channels 0-63 and 64-127; lanes 2m and 2m + 1 form normaliser m (q of token
      // m, k of token m - 16) into this wave's own slot, which every lane then reads with 16-byte
      // broadcast reads
      float nqv[16], nkv[16], bev[16];
      {
        const int m = lane >> 1;
        const float ss = sPart[(2 * seg) * 32 + m] + sPart[(2 * seg + 1) * 32 + m];
        const float nrm = fminf(__builtin_amdgcn_rsqf(ss), 1.0f / a.l2_eps) * (m < 16 ? a.scale : 1.0f);
        float* mine = sPart + 256 + wave * 32;
        if ((lane & 1) == 0) mine[m] = nrm;
        wave_lds_sync();
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 q4 = reinterpret_cast<const float4*>(mine)[g];
          const float4 k4 = reinterpret_cast<const float4*>(mine)[4 + g];
          const float4 b4 = reinterpret_cast<const float4*>(sBeta + 16 * seg)[g];
          nqv[4 * g] = q4.x; nqv[4 * g + 1] = q4.y; nqv[4 * g + 2] = q4.z; nqv[4 * g + 3] = q4.w;
          nkv[4 * g] = k4.x; nkv[4 * g + 1] = k4.y; nkv[4 * g + 2] = k4.z; nkv[4 * g + 3] = k4.w;
          bev[4 * g] = b4.x; bev[4 * g + 1] = b4.y; bev[4 * g + 2] = b4.z; bev[4 * g + 3] = b4.w;
        }
      }
      float* qp = sQ + 16 * seg * PQ + c;
      __bf16* khp = sKChi + 16 * seg * PKB + c;
      __bf16* klp = sKClo + 16 * seg * PKB + c;
      __bf16* rp = sKb + 16 * seg * PKB + c;
      // KC = K e^(Gam_n - Gam) goes to LDS split into bf16 hi + lo (the column operand of A_kk and
      // A_qk), and K~ = KC e^(Gam_C - Gam_n) straight to the workspace: K~^T [128][64] in fragment
      // order, this lane's 16 tokens as two 8-token pieces
      const float fac = exp2f_(GC - (SP ? ga[seg] : gn0));
      float kt[16];
      auto put_kc = [&](int k, float kcv) __attribute__((always_inline)) {
        const __bf16 kh = (__bf16)kcv;
        khp[k * PKB] = kh;
        klp[k * PKB] = (__bf16)(kcv - (float)kh);
        kt[k] = kcv * fac;
      };
      if (!SP) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float d = gl[k] - gl[0];
          const float e1 = exp2f_(d);   // <= 1
          const float e2 = exp2f_(-d);  // in [1, e^(15|lb|)]
          const float q = qx[k] * nqv[k];
          const float kv = kx[k] * nkv[k];
          qp[k * PQ] = q * e1;
          rp[k * PKB] = (__bf16)(kv * e1);
          put_kc(k, kv * e2);
          xk[k] = bev[k] * (kv * e1) * egn;
        }
      } else {
        float qn[16], kn[16], al[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          qn[k] = qx[k] * nqv[k];
          kn[k] = kx[k] * nkv[k];
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float e1 = exp2f_(gl[k] - gl[0]);   // <= 1
          const float e2 = exp2f_(gl[15] - gl[k]);  // <= 1: key columns anchored at the sub-chunk's end
          qp[k * PQ] = qn[k] * e1;
          rp[k * PKB] = (__bf16)(kn[k] * e1);
          put_kc(k, kn[k] * e2);
          xk[k] = bev[k] * (kn[k] * e1) * egn;
          al[k] = exp2f_(graw[k]);  // this token's decay
        }
        // the diagonal block entries of this channel (enumerated as in diag_entry), 64 at a time,
        // each batch summed over the wave's 64 channels; the pairwise decay e^(Gam_i - Gam_j) is
        // the running product of the decays of tokens j+1 .. i
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v[64];
          int n = 0;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float w = kn[j];
            if (n >= 64 * b && n < 64 * b + 64) v[n - 64 * b] = qn[j] * kn[j];
            ++n;
#pragma unroll
            for (int ii = j + 1; ii < 16; ++ii) {
              w *= al[ii];
              if (n >= 64 * b && n < 64 * b + 64) v[n - 64 * b] = kn[ii] * w;
              ++n;
              if (n >= 64 * b && n < 64 * b + 64) v[n - 64 * b] = qn[ii] * w;
              ++n;
            }
          }
          dpart[b] = reduce_scatter64(v, lane);
        }
        // the first wave of each sub-chunk (channels 0..63) hands its sums to the second
        if ((wave & 1) == 0) {
#pragma unroll
          for (int b = 0; b < 4; ++b) sTmp[seg * 256 + 64 * b + lane] = dpart[b];
        }
      }
      {
        _Float16* kthi = reinterpret_cast<_Float16*>(blk + W_KTHI);
        float a8[8], b8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a8[e] = kt[e];
          b8[e] = kt[8 + e];
        }
        *reinterpret_cast<f16x8*>(kthi + frag_offset(c, 16 * seg, C)) = to_f16x8(a8);
        *reinterpret_cast<f16x8*>(kthi + frag_offset(c, 16 * seg + 8, C)) = to_f16x8(b8);
      }
      // factor tables, row I = seg of channel c; column anchors: the sub-chunk's first token, or
      // its last one for the softplus branch
      const int I = seg;
      const float GI = gn0;
      sEn[I * D + c] = exp2f_(GI);
#pragma unroll
      for (int J = 0; J < 3; ++J)
        if (J < I) sE[pair_index(I, J) * D + c] = exp2f_(GI - (SP ? ga[J] : gn[J]));
      if (I == 0) sGC[c] = exp2f_(GC);
    }
    __syncthreads();

    prep_issue<VL>(a, st, knext, tid, nxt, 1);

    // ---- P6a: A_kk = beta_i * KR_I E_IJ . KC_J^T (plain bf16), strictly lower: one 16 x 16 block.
    //      The diagonal blocks and four below them here, one per wave; blocks (3,1) and (3,2),
    //      which only the off-diagonal T chains read, during the diagonal solve ----
    auto akk_block = [&](int bi) {
      int I, J;
      block_ij(bi, I, J);
      if (SP && I == J) return;  // formed exactly from the per-channel sums
      // two accumulators (even and odd k-steps): independent products overlap on the matrix core
      f32x4 acc2[2] = {zero4(), zero4()};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 32 * s + 8 * lg;
        bf16x8 av = *reinterpret_cast<const bf16x8*>(sKb + (16 * I + l16) * PKB + c);
        if (I > J) {
          const float* ef = sE + pair_index(I, J) * D + c;
#pragma unroll
          for (int e = 0; e < 8; ++e) av[e] = (__bf16)((float)av[e] * ef[e]);
        }
        acc2[s & 1] = mfma(av, *reinterpret_cast<const bf16x8*>(sKChi + (16 * J + l16) * PKB + c), acc2[s & 1]);
      }
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = acc2[0][r] + acc2[1][r];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * lg + r, j = 16 * J + l16;
        sAkk[i * PA + j] = j < i ? sBeta[i] * acc[r] : 0.f;
      }
    };
    akk_block(wave < 7 ? wave : 9);
    if (SP && (wave & 1)) {
      // diagonal block of sub-chunk seg: this wave's sums plus the partner wave's, as A_kk (times
      // beta, strictly lower) and A_qk (split planes, lower with the diagonal); then the upper
      // triangles, lane -> row l16, columns 4 lg .. 4 lg + 3
      const int base = 16 * (wave >> 1);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float tot = dpart[b] + sTmp[(wave >> 1) * 256 + 64 * b + lane];
        bool qk;
        int i, j;
        diag_entry(64 * b + lane, qk, i, j);
        const int R = base + i, Cc = base + j;
        if (qk) {
          sA16[R * PTB + Cc] = (_Float16)tot;
        } else {
          sAkk[R * PA + Cc] = sBeta[R] * tot;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * lg + e, R = base + l16, Cc = base + j;
        if (j >= l16) sAkk[R * PA + Cc] = 0.f;
        if (j > l16) sA16[R * PTB + Cc] = (_Float16)0.f;
      }
    }
    __syncthreads();

    // ---- P6b: A_qk = QR_I E_IJ . KC_J^T (split bf16), lower incl. diagonal: one 16 x 16 block ----
    auto aqk_block = [&](int bi) {
      int I, J;
      block_ij(bi, I, J);
      if (SP && I == J) return;  // formed exactly from the per-channel sums
      // the three split products (lo.hi, hi.lo, hi.hi) in three accumulators: three independent
      // chains on the matrix core instead of one of twelve dependent products
      f32x4 acc3[3] = {zero4(), zero4(), zero4()};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 32 * s + 8 * lg;
        float qv[8];
        ld8(sQ + (16 * I + l16) * PQ + c, qv);
        if (I > J) {
          const float* ef = sE + pair_index(I, J) * D + c;
#pragma unroll
          for (int e = 0; e < 8; ++e) qv[e] *= ef[e];
        }
        const int ko = (16 * J + l16) * PKB + c;
        const Split8 qs = split(qv);
        const Split8 ks{*reinterpret_cast<const bf16x8*>(sKChi + ko), *reinterpret_cast<const bf16x8*>(sKClo + ko)};
        acc3[0] = mfma(qs.lo, ks.hi, acc3[0]);
        acc3[1] = mfma(qs.hi, ks.lo, acc3[1]);
        acc3[2] = mfma(qs.hi, ks.hi, acc3[2]);
      }
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (acc3[0][r] + acc3[1][r]) + acc3[2][r];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * lg + r, j = 16 * J + l16;
        sA16[i * PTB + j] = (_Float16)(j <= i ? acc[r] : 0.f);  // zero above the diagonal
      }
    };

    // ---- P7: T = (I + A_kk)^-1 in fp32: diagonal 16x16 blocks by forward substitution on wave 0,
    //      while waves 1-7 clear T's strictly-upper blocks, waves 1-2 form A_kk blocks (3,1) and
    //      (3,2) and waves 3-7 A_qk blocks 0..4 ----
    if (wave == 0) {
      // lane: column cc of diagonal block I.  Column-oriented: once x[j] is final it is folded
      // into every row below at once, so the dependent chain is 16 steps long; each x[i] still
      // accumulates its terms in the order j = 0, 1, ...
      const int I = lg, cc = l16;
      const float* aI = sAkk + 16 * I * PA + 16 * I;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == cc) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < 15; ++j)
#pragma unroll
        for (int i = j + 1; i < 16; ++i) x[i] -= aI[i * PA + j] * x[j];
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[(16 * I + i) * PA + 16 * I + cc] = x[i];
    } else {
      // zero the strictly-upper blocks: W = T X reads blocks (0,1) and (2,3) inside its 32-token k-steps
      for (int idx = tid - 64; idx < 6 * 256; idx += NT - 64) {
        const int blk6 = idx >> 8, e = idx & 255;
        const int I = blk6 < 3 ? 0 : blk6 < 5 ? 1 : 2;
        const int J = blk6 < 3 ? blk6 + 1 : blk6 < 5 ? blk6 - 1 : 3;
        sT[(16 * I + (e >> 4)) * PA + 16 * J + (e & 15)] = 0.f;
      }
      // A_qk blocks (0,1) and (2,3) lie inside the 32-token k-steps that P9 reads
      for (int idx = tid - 64; idx < 2 * 256; idx += NT - 64) {
        const int I = 2 * (idx >> 8), e = idx & 255;
        const int o = (16 * I + (e >> 4)) * PTB + 16 * (I + 1) + (e & 15);
        sA16[o] = (_Float16)0.f;
      }
      if (wave < 3)
        akk_block(wave + 6);
      else
        aqk_block(wave - 3);
    }
    __syncthreads();
    // Off-diagonal blocks, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, column block J = wave (0..2)
    // top to bottom on the fp32 matrix cores, while waves 3-7 form A_qk blocks 5..9.
    // The sums M_I = sum_K A_IK T_KJ of every block below are started at once with their K = J
    // terms, and each gains its K term as soon as T_KJ is formed (the terms in the order K = J, J+1,
    // ...), so independent products overlap on the matrix core.
    if (wave < 3) {
      const int J = wave;
      float* sM = sTmp + wave * 16 * 17;
      auto add_term = [&](f32x4& m, int I, int K) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          m = mfma_f32(sAkk[(16 * I + l16) * PA + 16 * K + 4 * s + lg], sT[(16 * K + 4 * s + lg) * PA + 16 * J + l16], m);
      };
      f32x4 m[3] = {zero4(), zero4(), zero4()};
#pragma unroll
      for (int I = 1; I < 4; ++I)
        if (I > J) add_term(m[I - 1], I, J);
#pragma unroll
      for (int I = 1; I < 4; ++I) {
        if (I <= J) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) sM[(4 * lg + r) * 17 + l16] = m[I - 1][r];
        wave_lds_sync();
        f32x4 tij = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s)
          tij = mfma_f32(sT[(16 * I + l16) * PA + 16 * I + 4 * s + lg], sM[(4 * s + lg) * 17 + l16], tij);
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * lg + r) * PA + 16 * J + l16] = -tij[r];
        wave_lds_sync();
#pragma unroll
        for (int I2 = I + 1; I2 < 4; ++I2) add_term(m[I2 - 1], I2, I);
      }
    } else {
      aqk_block(wave + 2);
    }
    __syncthreads();
    // T as fp16 in place of A_kk: eight elements per lane
    {
      const int t = tid >> 3, j8 = (tid & 7) * 8;
      float v[8];
      ld8(sT + t * PA + j8, v);
      *reinterpret_cast<f16x4*>(sT16 + t * PTB + j8) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      *reinterpret_cast<f16x4*>(sT16 + t * PTB + j8 + 4) = f16x4{(_Float16)v[4], (_Float16)v[5], (_Float16)v[6], (_Float16)v[7]};
    }
    // ---- P8 (from the same phase): W = T X with T in fp16 and X split into fp16 hi + lo (T.X lo +
    //      T.X hi).  X goes to LDS transposed, [channel][token], as two planes in place of KR and
    //      of the KC planes (both last read by the A blocks): a lane writes its 16 tokens of one
    //      channel, and a B-operand fragment (8 tokens of one channel) is two 8-byte reads;
    //      wave -> 16 key channels ----
    _Float16* sXhi = reinterpret_cast<_Float16*>(sKb);           // [128][PXT]
    _Float16* sXlo = reinterpret_cast<_Float16*>(smem + OFF_G);  // [128][PXT]
    {
      const int i = tid & 127, seg = tid >> 7;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f16x4 h4, l4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = xk[4 * g + e];
          h4[e] = (_Float16)x;
          l4[e] = (_Float16)(x - (float)h4[e]);
        }
        *reinterpret_cast<f16x4*>(sXhi + i * PXT + 16 * seg + 4 * g) = h4;
        *reinterpret_cast<f16x4*>(sXlo + i * PXT + 16 * seg + 4 * g) = l4;
      }
    }
    __syncthreads();

    prep_issue<VL>(a, st, knext, tid, nxt, 2);

    f32x4 wacc[4] = {zero4(), zero4(), zero4(), zero4()};
    {
      const int c = 16 * wave + l16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tb = 32 * s + 8 * lg;
        const Half8 x{ld4x2(sXhi + c * PXT + tb, 4), ld4x2(sXlo + c * PXT + tb, 4)};
        // the lo products of every row block, then the hi ones: consecutive products independent
        f16x8 tI[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (32 * s > 16 * I + 15) continue;  // T is lower triangular
          tI[I] = ld4x2(sT16 + (16 * I + l16) * PTB + 32 * s + 8 * lg, 4);
          wacc[I] = mfma16(tI[I], x.lo, wacc[I]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (32 * s > 16 * I + 15) continue;
          wacc[I] = mfma16(tI[I], x.hi, wacc[I]);
        }
      }
    }
    // W (fp16) in place of the fp32 T (converted above); each wave stores its own 16 columns in
    // fragment order (64 rows x 2 pieces of 8 channels) from there, after a wave-local sync
    _Float16* sW = reinterpret_cast<_Float16*>(smem + OFF_STG + C * PA * 4);  // [64][PKB]
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) sW[(16 * I + 4 * lg + r) * PKB + 16 * wave + l16] = (_Float16)wacc[I][r];
    wave_lds_sync();
    {
      _Float16* wdst = reinterpret_cast<_Float16*>(blk + W_W);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int sl = lane + 64 * q, t = sl >> 1, c8 = 16 * wave + 8 * (sl & 1);
        *reinterpret_cast<f16x8*>(wdst + frag_offset(t, c8, D)) = *reinterpret_cast<const f16x8*>(sW + t * PKB + c8);
      }
    }
    __syncthreads();  // every read of X is done: the raw v rows take X lo's place

    // every lane stores (four lanes per value, the same value) so that the number of stores is fixed
    reinterpret_cast<float*>(blk + W_GC)[tid & 127] = sGC[tid & 127];

    // ---- stage raw v rows for tokens c0-3 .. c0+63 (bf16, pitch PKB) ----
    __bf16* sRv = reinterpret_cast<__bf16*>(smem + OFF_G);
#pragma unroll
    for (int s = 0; s < NRV; ++s) {
      const int idx = tid + s * NT;
      if (idx < RROWS * 16) {
        const int r = idx >> 4, sg = idx & 15;
        const int tt = c0 - HALO + r;
        *reinterpret_cast<uint4*>(sRv + r * PKB + sg * 8) = (tt >= 0 && tt < T) ? cur.rawv[s] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (ci == 0 && tid < HALO * 16) {
      // rows before the sequence start come from the conv state (the same lane wrote them as zeros)
      const int r = tid >> 4, sg = tid & 15;
      const int tt = r - HALO;
      if ((W - 1) + tt >= 0) {
        const long long ch = 2LL * HD + h * D + sg * 8;
        uint16_t e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = cin[(ch + e) * (W - 1) + (W - 1) + tt];
        *reinterpret_cast<uint4*>(sRv + r * PKB + sg * 8) =
            make_uint4(e8[0] | (uint32_t)e8[1] << 16, e8[2] | (uint32_t)e8[3] << 16, e8[4] | (uint32_t)e8[5] << 16,
                       e8[6] | (uint32_t)e8[7] << 16);
      }
    }
    __syncthreads();

    // ---- P9: the operands of O = Q~ S + A_qk U for phase B, both fp16 in fragment order:
    //      Q~ = QR e^Gam_n (each wave its own 16 columns: 64 rows x 2 pieces of 8 channels) and
    //      the six A_qk fragments on or below the diagonal (one per wave 0-5); then per wave,
    //      column tile j = wave of the value axis, Ut = T (beta V) (T fp16, beta V fp16 hi + lo) ----
    {
      _Float16* qdst = reinterpret_cast<_Float16*>(blk + W_QT);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int sl = lane + 64 * q, t = sl >> 1, c8 = 16 * wave + 8 * (sl & 1);
        float v[8], e[8];
        ld8(sQ + t * PQ + c8, v);
        ld8(sEn + (t >> 4) * D + c8, e);
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] *= e[x];
        *reinterpret_cast<f16x8*>(qdst + frag_offset(t, c8, D)) = to_f16x8(v);
      }
      {
        // fragment f = 2 I + s of [64][64]: wave 0 -> (0, 0), 1 -> (1, 0), 2.. 5 -> (2, 0) .. (3, 1);
        // waves 6 and 7 write (0, 1) and (1, 1), which lie above the diagonal, as zeros (phase B reads
        // only fragment (I, 0) for I < 2; the fixed store count keeps this phase free of a branch)
        const int f = wave < 2 ? 2 * wave : wave < 6 ? wave + 2 : 2 * (wave - 6) + 1;
        const int t = 16 * (f >> 1) + l16, k = 32 * (f & 1) + 8 * lg;
        const f16x8 z = {};
        reinterpret_cast<f16x8*>(blk + W_AQK)[f * 64 + lane] = wave < 6 ? ld4x2(sA16 + t * PTB + k, 4) : z;
      }
    }
    {
      const int vc = 16 * wave + l16;
      // beta V for tokens 32 s + 8 lg + 0..7 of channel vc: the B operand of Ut
      Half8 bv[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int tb = 32 * st + 8 * lg;
        // rows tb .. tb+10 of channel vc as pairs, as in the q|k conv
        bf16x2 pe[6], po[5];
#pragma unroll
        for (int m = 0; m < 5; ++m) pe[m] = bf16x2{sRv[(tb + 2 * m) * PKB + vc], sRv[(tb + 2 * m + 1) * PKB + vc]};
        pe[5] = bf16x2{sRv[(tb + 10) * PKB + vc], (__bf16)0.f};
#pragma unroll
        for (int m = 0; m < 5; ++m) po[m] = mid_pair(pe[m], pe[m + 1]);
        float xv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = e >> 1;
          const float y = (e & 1) ? dot2(tv23, po[m + 1], dot2z(tv01, po[m])) : dot2(tv23, pe[m + 1], dot2z(tv01, pe[m]));
          xv[e] = sBeta[tb + e] * silu_fast(y);
        }
        bv[st] = split16(xv);
      }
      f32x4 ut[4];
      f16x4* utd = reinterpret_cast<f16x4*>(blk + W_UT);
#pragma unroll
      for (int I = 0; I < 4; ++I) ut[I] = zero4();
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // the lo products of every row block, then the hi ones (T is lower triangular)
        f16x8 tI[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (32 * st > 16 * I + 15) continue;
          tI[I] = ld4x2(sT16 + (16 * I + l16) * PTB + 32 * st + 8 * lg, 4);
          ut[I] = mfma16(tI[I], bv[st].lo, ut[I]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (32 * st > 16 * I + 15) continue;
          ut[I] = mfma16(tI[I], bv[st].hi, ut[I]);
        }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
        utd[(wave * 4 + I) * 64 + lane] = f16x4{(_Float16)ut[I][0], (_Float16)ut[I][1], (_Float16)ut[I][2], (_Float16)ut[I][3]};
    }
    __syncthreads();  // the next task overwrites the staging rows and tables
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------------------------
// Phase B: one workgroup per (16-column block of d_v, head, sequence or group of sequences),
// sequential over chunks.
// Waves 0-3 form U = Ut - W S for row tile I = wave and then update state row tiles wave and
// wave + 4; waves 4-7 form O = Q~ S + A_qk U for row tile I = wave - 4, store it and load their
// Q~ and A_qk of two chunks later into registers.  Waves 8-11 only
// move data: they copy the tiles that waves 0-3 read (W, Ut, K~^T, e^Gam_C) straight into LDS
// ahead of use and touch later chunks so that they are in L2.
// ---------------------------------------------------------------------------------------------
// Operands the output waves (4-7) keep in registers: their row tile of Q~ and of A_qk.
struct OpTiles {
  f16x8 x0[4];  // Q~ (fp16), row tile I = wave - 4 (4 k-steps over the key channels)
  f16x8 aq[2];  // A_qk (fp16), row tile I (2 k-steps over the tokens; 1 for I < 2)
};

// Direct global -> LDS copies (gfx950 global_load_lds): lane l's bytes land at lds + l * size.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
// Workgroup barrier for LDS only: this wave's LDS operations complete, then s_barrier; the asm is
// a compiler memory barrier.  Unlike __syncthreads it does not wait for outstanding global loads
// (phase B shares no global memory between waves), so copies into LDS may stay in flight across
// it; their issuing waves wait for them explicitly before the barrier that publishes them.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
#define KDA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

template <bool VL>
__global__ __launch_bounds__(NTB) void kda_chunk_state_kernel(LayerArgs a, SeqTab st, const unsigned char* __restrict__ ws,
                                                           _Float16* __restrict__ ows) {
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* sUhi = reinterpret_cast<_Float16*>(smem + B_UHI);
  _Float16* sUlo = reinterpret_cast<_Float16*>(smem + B_ULO);
  _Float16* sShi = reinterpret_cast<_Float16*>(smem + B_SHI);
  _Float16* sSlo = reinterpret_cast<_Float16*>(smem + B_SLO);

  const int H = a.H;
  const int h = blockIdx.x % H;
  const int vb = blockIdx.x / H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: role branches are uniform
  const int l16 = lane & 15, lg = lane >> 4;
  const int HD = H * D;
  // The workgroup's sequences: group blockIdx.y of the table (consecutive sequences, whose chunks
  // it runs as one stream, so the tile pipeline stays full across sequence boundaries), or
  // sequence blockIdx.y of a uniform batch.  Chunk g of the stream is chunk ci of sequence s.
  const int s_first = VL ? st.grp0[blockIdx.y] : (int)blockIdx.y;
  const int s_end = VL ? st.grp0[blockIdx.y + 1] : (int)blockIdx.y + 1;
  const int NCu = (a.T + C - 1) / C;  // chunks per sequence of a uniform batch
  const int g0 = VL ? st.chunk0[s_first] : 0;
  const int NG = VL ? st.chunk0[s_end] - g0 : NCu;
  struct ChunkRef {
    int s, ci, nc, base;  // sequence, chunk in it, its chunk count, its first chunk in the launch
    long long tok0;       // the sequence's first packed token
    int len;              // and its length
  };
  // Each call site walks the stream forward through its own cursor: the sequence it reached with
  // its chunk range and tokens, so the table is read only when a sequence boundary is crossed.
  struct Cursor {
    int s, base, next, len;
    long long tok0;
    int nn, nt;  // chunk0 and tok0 of sequence s + 2 (the end of s + 1), loaded one step ahead
  };
  auto cursor0 = [&]() {
    const int s2 = min(s_first + 2, s_end);
    return VL ? Cursor{s_first, st.chunk0[s_first], st.chunk0[s_first + 1], st.tok0[s_first + 1] - st.tok0[s_first],
                       (long long)st.tok0[s_first], st.chunk0[s2], st.tok0[s2]}
              : Cursor{s_first, 0, NCu, a.T, (long long)s_first * a.T, 0, 0};
  };
  // Every sequence of the table has at least one chunk (the host leaves empty sequences out), so a
  // cursor that moves one chunk at a time crosses at most one sequence boundary per step: the
  // advance is one select over values the previous step loaded (the next sequence starts where this
  // one ends), with no loop or branch, which keeps the compiler's memory-counter waits in the role
  // loops per load, and no step waits for its own table reads.
  auto locate = [&](Cursor& cu, int g) -> ChunkRef {
    if (!VL) return ChunkRef{s_first, g, NCu, s_first * NCu, (long long)s_first * a.T, a.T};
    const int gc = g0 + g;
    const bool adv = gc >= cu.next && cu.s + 1 < s_end;
    const long long t0 = cu.tok0 + cu.len;
    cu.s = adv ? cu.s + 1 : cu.s;
    cu.base = adv ? cu.next : cu.base;
    cu.len = adv ? (int)(cu.nt - t0) : cu.len;
    cu.tok0 = adv ? t0 : cu.tok0;
    cu.next = adv ? cu.nn : cu.next;
    const int s2 = min(cu.s + 2, s_end);
    cu.nn = st.chunk0[s2];
    cu.nt = st.tok0[s2];
    return ChunkRef{cu.s, gc - cu.base, cu.next - cu.base, cu.base, cu.tok0, cu.len};
  };
  // tile block of a chunk: sequence-major, then head, then chunk
  auto chunk_ptr = [&](Cursor& cu, int g) -> const unsigned char* {
    const ChunkRef r = locate(cu, g);
    return ws + (((long long)r.base * H + (long long)h * r.nc) + r.ci) * CH_BYTES;
  };
  auto seq_tok0 = [&](int sq) -> long long { return VL ? (long long)st.tok0[sq] : (long long)sq * a.T; };
  auto seq_len = [&](int sq) -> int { return VL ? st.tok0[sq + 1] - st.tok0[sq] : a.T; };
  auto seq_slot = [&](int sq) -> long long { return VL ? st.slot[sq] : sq; };
  auto wubuf = [&](int c) { return smem + B_WU0 + (c & 1) * WU_BYTES; };
  auto kbuf = [&](int c) { return smem + B_KB0 + (c & 1) * KB_BYTES; };

  // ---- loader waves (lw = 0..3): each copies 4 of the 16 W fragments, row tile lw of this block's
  //      Ut (512 B, half the lanes) and 4 of the 16 K~^T fragments of a chunk (wave 3 also e^Gam_C);
  //      cache lines of later chunks touched ----
  const int lw = wave - 8;
  constexpr int N_WU = 5, N_K = 4;
  Cursor cur_wu = cursor0(), cur_k = cursor0(), cur_t = cursor0();
  auto issue_wu = [&](int cn) {
    const unsigned char* blk = chunk_ptr(cur_wu, cn);
    unsigned char* wb = wubuf(cn);
#pragma unroll
    for (int q = 0; q < N_WU - 1; ++q) {
      const int f = lw * (N_WU - 1) + q;  // W fragment f
      dma16(blk + W_W + f * 1024 + lane * 16, wb + WU_W + f * 1024);
    }
    if (lane < 32) dma16(blk + W_UT + (vb * 4 + lw) * 512 + lane * 16, wb + WU_UT + lw * 512);
  };
  auto issue_k = [&](int cn) {
    const unsigned char* blk = chunk_ptr(cur_k, cn);
    unsigned char* kb = kbuf(cn);
#pragma unroll
    for (int q = 0; q < N_K; ++q) {
      const int f = lw * N_K + q;  // K~^T fragment f
      dma16(blk + W_KTHI + f * 1024 + lane * 16, kb + KB_KHI + f * 1024);
    }
    if (lw == 3) {
#pragma unroll
      for (int q = 0; q < 2; ++q) dma4(blk + W_GC + q * 256 + lane * 4, kb + KB_GC + q * 256);
    }
  };
  // the 8 workgroups of a head touch one eighth each of a chunk's 128-byte lines (one 4-byte copy
  // per line), so that the chunk is in L2 when its tiles are fetched a chunk later
  constexpr int LINES = CH_BYTES / 128;
  constexpr int LINES_PER_WG = (LINES + NBLK - 1) / NBLK;
  constexpr int TOUCH_PER_WAVE = (LINES_PER_WG + 4 * 64 - 1) / (4 * 64);
  auto touch_chunk = [&](int cw) {
    const unsigned char* blk = chunk_ptr(cur_t, cw);
#pragma unroll
    for (int q = 0; q < TOUCH_PER_WAVE; ++q) {
      const int line = min(vb * LINES_PER_WG + min((q * 4 + lw) * 64 + lane, LINES_PER_WG - 1), LINES - 1);
      dma4(blk + line * 128, smem + B_TRASH);
    }
  };

  if (wave >= 8) {
    // Loader waves: their own loop, with the same two barriers per chunk as the compute waves.
    // W | Ut of chunk c goes to buffer c & 1, whose last reader (chunk c-2's U waves) is done at
    // barrier (b) of chunk c-2: it is copied right after that barrier.  K~^T of chunk c goes to
    // buffer c & 1 after barrier (a) of chunk c-1 (its last reader, chunk c-2's state update, is done
    // by then), and chunk c+3 is touched into L2 then too.  Before barrier (a) of chunk c this wave
    // waits for its W | Ut copies of c, before barrier (b) for its K~^T copies of c; each wait counts
    // the copies issued after the awaited ones, and near the end waits for everything.
    issue_wu(0);
    issue_k(0);
    if (NG > 1) issue_wu(1);
    if (NG > 2) {
      (void)locate(cur_t, 1);  // the touch cursor starts at chunk 2: step it through chunk 1 first
      touch_chunk(2);
    }
    KDA_WAIT_VMCNT(0);
    for (int ci = 0; ci < NG; ++ci) {
      if (ci >= 2) {
        // after W | Ut(ci): K~^T(ci) and the touch of ci+2 (chunk ci-1, after (a)), W | Ut(ci+1) (after (b))
        if (ci + 2 < NG) {
          if (lw == 3)
            KDA_WAIT_VMCNT(N_K + 2 + TOUCH_PER_WAVE + N_WU);
          else
            KDA_WAIT_VMCNT(N_K + TOUCH_PER_WAVE + N_WU);
        } else {
          KDA_WAIT_VMCNT(0);
        }
      }
      lds_barrier();  // (a)
      if (ci + 1 < NG) issue_k(ci + 1);
      if (ci + 3 < NG) touch_chunk(ci + 3);
      if (ci >= 1) {
        // after K~^T(ci): the touch of ci+2, W | Ut(ci+1), K~^T(ci+1) and the touch of ci+3
        if (ci + 3 < NG) {
          if (lw == 3)
            KDA_WAIT_VMCNT(TOUCH_PER_WAVE + N_WU + N_K + 2 + TOUCH_PER_WAVE);
          else
            KDA_WAIT_VMCNT(TOUCH_PER_WAVE + N_WU + N_K + TOUCH_PER_WAVE);
        } else {
          KDA_WAIT_VMCNT(0);
        }
      }
      lds_barrier();  // (b)
      if (ci + 2 < NG) issue_wu(ci + 2);
    }
    // The new conv state of this workgroup's 48 channels (16 each of q, k and v) for each of its
    // sequences: the last W-1 raw inputs, from the conv state passed in where a sequence is shorter.
    // The 256 loader lanes take (sequence, channel) pairs, four at a time with every load issued
    // before the first store, so a group of sequences costs about one memory round trip.
    if (a.W > 1 && a.conv_out != nullptr) {
      const int W = a.W, Cq = 3 * HD;
      const int npairs = (s_end - s_first) * 48;
      const bf16_t* x = static_cast<const bf16_t*>(a.qkv);
      for (int p0 = tid - 8 * 64; p0 < npairs; p0 += 4 * 256) {
        bf16_t win[4][3];
        long long dst[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = p0 + q * 256;
          dst[q] = -1;
          if (p < npairs) {
            const int sq = s_first + p / 48, j = p % 48;
            const long long slot = seq_slot(sq), tok0 = seq_tok0(sq);
            const int T = seq_len(sq);
            const long long c = (long long)(j >> 4) * HD + h * D + vb * NVB + (j & 15);
            const bf16_t* cin = static_cast<const bf16_t*>(a.conv_in) + (slot * Cq + c) * (W - 1);
            dst[q] = (slot * Cq + c) * (W - 1);
#pragma unroll
            for (int w = 0; w < 3; ++w) {
              const int tt = T - (W - 1) + w;
              if (w < W - 1) win[q][w] = tt >= 0 ? x[(tok0 + tt) * Cq + c] : cin[(W - 1) + tt];
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (dst[q] < 0) continue;
          bf16_t* cout = static_cast<bf16_t*>(a.conv_out) + dst[q];
#pragma unroll
          for (int w = 0; w < 3; ++w)
            if (w < W - 1) cout[w] = win[q][w];
        }
      }
    }
    return;
  }

  // ---- state waves (0-3): wave w owns state row tiles w and w + 4 (channels 16t..16t+15); the
  //      lane holds rows 16t+4lg+r of column vb*16 + l16 ----
  f32x4 Sacc[2];
  auto s_in = [&](int sq) { return a.state_in + (seq_slot(sq) * H + h) * D * D + vb * NVB + l16; };
  auto s_out = [&](int sq) { return a.state_out + (seq_slot(sq) * H + h) * D * D + vb * NVB + l16; };
  // S^T as the split fp16 B operand [column][channel] (hi + lo: ~22 significant bits); the lane's
  // four rows are contiguous
  auto write_state_operand = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = wave + 4 * u;
      f16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = (_Float16)Sacc[u][r];
        lo[r] = (_Float16)(Sacc[u][r] - (float)hi[r]);
      }
      *reinterpret_cast<f16x4*>(sShi + l16 * PST + 16 * t + 4 * lg) = hi;
      *reinterpret_cast<f16x4*>(sSlo + l16 * PST + 16 * t + 4 * lg) = lo;
    }
  };

  // S <- e^Gam_C S + K~^T U from chunk ci's buffer, then the state operand for the next chunk
  // (every read of the old one came before barrier (b)).
  auto state_update = [&](const unsigned char* kb) {
    f32x4 sa[2], sb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = wave + 4 * u;
      const float4 gc = *reinterpret_cast<const float4*>(kb + KB_GC + (16 * t + 4 * lg) * 4);
      sa[u][0] = gc.x * Sacc[u][0];
      sa[u][1] = gc.y * Sacc[u][1];
      sa[u][2] = gc.z * Sacc[u][2];
      sa[u][3] = gc.w * Sacc[u][3];
      sb[u] = zero4();
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f16x8 uh = *reinterpret_cast<const f16x8*>(sUhi + l16 * PVT + 32 * s + 8 * lg);
      const f16x8 ul = *reinterpret_cast<const f16x8*>(sUlo + l16 * PVT + 32 * s + 8 * lg);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = wave + 4 * u;
        const f16x8 k0 = *reinterpret_cast<const f16x8*>(kb + KB_KHI + ((t * 2 + s) * 64 + lane) * 16);
        sa[u] = mfma16(k0, uh, sa[u]);
        sb[u] = mfma16(k0, ul, sb[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) Sacc[u][r] = sa[u][r] + sb[u][r];
    write_state_operand();
  };

  // Each role runs its own loop (so that no wave's waits are derived from another role's loads),
  // with the same two barriers per chunk: (a) the state operand and chunk ci's W | Ut are in
  // LDS; (b) U and chunk ci's K~^T are in LDS and every read of the state operand is done.
  if (wave < 4) {
    {
      const float* si = s_in(s_first);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[u][r] = si[(16 * (wave + 4 * u) + 4 * lg + r) * D];
    }
    write_state_operand();
    // U = Ut - W S for row tile I = wave, as the split B operand [column][token]
    const int I = wave;
    Cursor cur_s = cursor0();
    f32x4 Snext[2];  // the next sequence's state, loaded during the current one's first chunk
    for (int ci = 0; ci < NG; ++ci) {
      const ChunkRef rc = locate(cur_s, ci);
      const bool seq_last = rc.ci == rc.nc - 1, more = ci + 1 < NG;
      if (rc.ci == 0 && rc.s + 1 < s_end) {
        const float* si = s_in(rc.s + 1);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) Snext[u][r] = si[(16 * (wave + 4 * u) + 4 * lg + r) * D];
      }
      const unsigned char* wb = wubuf(ci);
      lds_barrier();  // (a)
      f32x4 pa = zero4(), pb = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 w = *reinterpret_cast<const f16x8*>(wb + WU_W + ((I * 4 + s) * 64 + lane) * 16);
        const f16x8 sh = *reinterpret_cast<const f16x8*>(sShi + l16 * PST + 32 * s + 8 * lg);
        const f16x8 sl = *reinterpret_cast<const f16x8*>(sSlo + l16 * PST + 32 * s + 8 * lg);
        pa = mfma16(w, sh, pa);
        pb = mfma16(w, sl, pb);
      }
      const f16x4 ut = *reinterpret_cast<const f16x4*>(wb + WU_UT + (I * 64 + lane) * 8);
      f16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = (float)ut[r] - (pa[r] + pb[r]);
        hi[r] = (_Float16)u;
        lo[r] = (_Float16)(u - (float)hi[r]);
      }
      *reinterpret_cast<f16x4*>(sUhi + l16 * PVT + 16 * I + 4 * lg) = hi;
      *reinterpret_cast<f16x4*>(sUlo + l16 * PVT + 16 * I + 4 * lg) = lo;
      lds_barrier();  // (b)
      state_update(kbuf(ci));
      if (seq_last) {
        // the sequence's final state; the next sequence starts from its own slot's state (its
        // operand replaces the one state_update just wrote, before barrier (a) publishes it).  The
        // swap comes before the stores, so that waiting for the prefetched state never waits for them.
        const f32x4 fin[2] = {Sacc[0], Sacc[1]};
        if (more) {
          Sacc[0] = Snext[0];
          Sacc[1] = Snext[1];
          write_state_operand();
        }
        float* so = s_out(rc.s);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) so[(16 * (wave + 4 * u) + 4 * lg + r) * D] = fin[u][r];
      }
    }
  } else {
    // O = Q~ S + A_qk U for row tile I = wave - 4, with Q~ and A_qk in registers: Q~ S between
    // barriers (a) and (b) (the state operand is replaced after (b)), A_qk U after (b), where U
    // is in LDS until the U waves replace it after the next barrier (a), so the matrix-core work of
    // the output waves is split between the two halves of the chunk.  Then the rows are stored and
    // the register set is refilled with the tiles of chunk ci + 2 (two sets alternate, so no
    // loaded value is copied, and a load has two chunks to arrive).  The loop body has no branch,
    // which keeps the compiler's memory-counter waits per load (a branch there made it wait for
    // every outstanding load and store at the top of each chunk).  Rows past the end of the
    // sequence go to a scratch slot after o, so that every lane issues the same stores; the last
    // chunk's tiles are loaded again in place of chunks past the end.
    const int I = wave - 4;
    _Float16* scratch = ows + (VL ? (long long)st.tok0[st.n] : (long long)a.B * a.T) * HD + lane * 4;
    Cursor cur_o = cursor0(), cur_l = cursor0();
    // Row tiles 0 and 1 see tokens 0-31 only (A_qk's second k-step is zero for them): the loop is
    // instantiated for them with one k-step of A_qk U, chosen once, outside the loop
    auto run = [&](auto low) __attribute__((always_inline)) {
      constexpr int NKA = decltype(low)::value ? 1 : 2;  // k-steps of A_qk U
      auto load_tiles = [&](int c, OpTiles& o) __attribute__((always_inline)) {
        const unsigned char* blk = chunk_ptr(cur_l, c);
        const f16x8* x0p = reinterpret_cast<const f16x8*>(blk + W_QT) + (I * 4) * 64 + lane;
#pragma unroll
        for (int s = 0; s < 4; ++s) o.x0[s] = x0p[s * 64];
        const f16x8* ap = reinterpret_cast<const f16x8*>(blk + W_AQK) + (I * 2) * 64 + lane;
#pragma unroll
        for (int s = 0; s < NKA; ++s) o.aq[s] = ap[s * 64];
      };
      auto chunk_o = [&](int ci, OpTiles& cur) __attribute__((always_inline)) {
        const ChunkRef rc = locate(cur_o, ci);
        lds_barrier();  // (a)
        // the state's fp16 hi part only: O is not fed back into the state, so its rounding does not
        // accumulate over chunks, and Q~ itself is fp16
        f32x4 oa = zero4(), ob = zero4();
#pragma unroll
        for (int s = 0; s < 4; s += 2) {
          const f16x8 s0 = *reinterpret_cast<const f16x8*>(sShi + l16 * PST + 32 * s + 8 * lg);
          const f16x8 s1 = *reinterpret_cast<const f16x8*>(sShi + l16 * PST + 32 * (s + 1) + 8 * lg);
          oa = mfma16(cur.x0[s], s0, oa);
          ob = mfma16(cur.x0[s + 1], s1, ob);
        }
        asm volatile("" : "+v"(oa), "+v"(ob));  // both products ahead of barrier (b)
        lds_barrier();  // (b)
        // A_qk U with U split into fp16 hi + lo
        f32x4 oc = zero4(), od = zero4();
#pragma unroll
        for (int s = 0; s < NKA; ++s) {
          const f16x8 uh = *reinterpret_cast<const f16x8*>(sUhi + l16 * PVT + 32 * s + 8 * lg);
          const f16x8 ul = *reinterpret_cast<const f16x8*>(sUlo + l16 * PVT + 32 * s + 8 * lg);
          oc = mfma16(cur.aq[s], uh, oc);
          od = mfma16(cur.aq[s], ul, od);
        }
        const int c0 = rc.ci * C, L = min(C, rc.len - c0);
        _Float16* op = ows + ((rc.tok0 + c0) * H + h) * D + vb * NVB + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * I + 4 * lg + r;
          *(t < L ? op + (long long)t * HD : scratch + r) = (_Float16)((oa[r] + ob[r]) + (oc[r] + od[r]));
        }
        load_tiles(min(ci + 2, NG - 1), cur);
      };
      OpTiles ta, tb2;
      load_tiles(0, ta);
      load_tiles(min(1, NG - 1), tb2);
      int ci = 0;
      for (; ci + 1 < NG; ci += 2) {
        chunk_o(ci, ta);
        chunk_o(ci + 1, tb2);
      }
      if (ci < NG) chunk_o(ci, ta);
    };
    if (I < 2)
      run(std::true_type());
    else
      run(std::false_type());
  }
}

// Gated output RMSNorm over the 128 columns of each (token, head) row of o: 16 lanes per row,
// 8 columns per lane, 16-byte loads and stores.
__device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void unpack8(const uint4 u, float (&v)[8]) {
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
  v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}

template <typename OT>
__global__ __launch_bounds__(256) void kda_out_norm_kernel(const _Float16* __restrict__ ows, const bf16_t* __restrict__ gout,
                                                        const bf16_t* __restrict__ nw, OT* __restrict__ out,
                                                        long long rows, float eps) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c8 = (threadIdx.x & 15) * 8;
  if (row >= rows) return;  // the 16 lanes of a row leave together
  // o and the gate are read once: non-temporal loads keep them from displacing cached lines
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const f16x8 ov = __builtin_bit_cast(f16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ows + row * D + c8)));
  const u32x4 gq = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gout + row * D + c8));
  const uint4 g = make_uint4(gq.x, gq.y, gq.z, gq.w);
  const uint4 w = *reinterpret_cast<const uint4*>(nw + c8);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)ov[e];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += o[e] * o[e];
  ss = group_sum<16>(ss);
  const float rr = rsqrtf(ss / (float)D + eps);
  float gv[8], wv[8], r[8];
  unpack8(g, gv);
  unpack8(w, wv);
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = o[e] * rr * wv[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[e]));
  store8(out + row * D + c8, r);
}

}  // namespace

// The staging halo covers conv widths up to 4.  Every gate whose log-decay is <= 0 runs here: the
// bounded gate with -5.5 <= lb <= 0 on start-anchored sub-chunks (its factors stay finite while
// 15 |lb| < 87), with lb < -5.5 and the softplus branch on end-anchored ones with exact diagonal
// blocks.  W and Ut keep ~11 bits through phase B (fp16), so weak decay (lb near 0, or
// pre-activations that keep the gate near 0) keeps the state within the tolerance.  A positive bound (log-decay above
// 0, a growing state) takes the fp32 path.
bool prefill_mfma_supported(int Dh, int chunk, int io, int W, float lb, int gate) {
  if (!(Dh == D && chunk == C && io == kBF16 && W >= 1 && W <= HALO + 1)) return false;
  return gate == 1 || lb <= 0.f;
}

size_t prefill_mfma_workspace(long long chunks, long long tokens, int H) {
  return (size_t)chunks * H * CH_BYTES + (size_t)tokens * H * D * sizeof(_Float16) + 64 * 4 * sizeof(_Float16);
}

template <bool VL>
static hipError_t launch_mfma_t(const LayerArgs& a, const SeqTab& st, void* ws, int ot, hipStream_t s) {
  unsigned char* tiles = static_cast<unsigned char*>(ws);
  const int NC = (a.T + C - 1) / C;
  const long long chunks = VL ? st.total_chunks : (long long)a.B * NC;
  const long long tokens = VL ? st.tok0[st.n] : (long long)a.B * a.T;
  _Float16* ows = reinterpret_cast<_Float16*>(tiles + (size_t)chunks * a.H * CH_BYTES);
  {
    hipError_t e0 = set_lds_limit(reinterpret_cast<const void*>(kda_chunk_prep_kernel<VL, 0>), LDS_A);
    if (e0 == hipSuccess) e0 = set_lds_limit(reinterpret_cast<const void*>(kda_chunk_prep_kernel<VL, 1>), LDS_A);
    if (e0 == hipSuccess) e0 = set_lds_limit(reinterpret_cast<const void*>(kda_chunk_prep_kernel<VL, 2>), LDS_A);
    if (e0 == hipSuccess) e0 = set_lds_limit(reinterpret_cast<const void*>(kda_chunk_state_kernel<VL>), LDS_B);
    if (e0 != hipSuccess) return e0;
  }
  // persistent: one workgroup per CU (the LDS use admits one), each looping over tasks
  const int ncu = device_cus();
  const int ntask = (int)(chunks * a.H);
  // the gate's phase-A instance: 0 bounded with -5.5 <= lb <= 0, 1 softplus, 2 bounded with lb < -5.5
  const int gk = a.gate != 0 ? 1 : (a.lb < -5.5f ? 2 : 0);
  // timing names (kept apart per call kind: [varlen] table mode, [softplus] decay branch, [strong]
  // the bounded gate below -5.5)
  static const char* const kname[3][6] = {
      {"kda_chunk_prep_kernel", "kda_chunk_prep_kernel[softplus]", "kda_chunk_prep_kernel[strong]",
       "kda_chunk_prep_kernel[varlen]", "kda_chunk_prep_kernel[varlen][softplus]",
       "kda_chunk_prep_kernel[varlen][strong]"},
      {"kda_chunk_state_kernel", "kda_chunk_state_kernel[softplus]", "kda_chunk_state_kernel[strong]",
       "kda_chunk_state_kernel[varlen]", "kda_chunk_state_kernel[varlen][softplus]",
       "kda_chunk_state_kernel[varlen][strong]"},
      {"kda_out_norm_kernel", "kda_out_norm_kernel[softplus]", "kda_out_norm_kernel[strong]",
       "kda_out_norm_kernel[varlen]", "kda_out_norm_kernel[varlen][softplus]", "kda_out_norm_kernel[varlen][strong]"}};
  const int kn = (VL ? 3 : 0) + gk;
  const dim3 grid_a(ntask < ncu ? ntask : ncu);
  timing_begin(kname[0][kn], s);
  if (gk == 0)
    kda_chunk_prep_kernel<VL, 0><<<grid_a, NT, LDS_A, s>>>(a, st, tiles);
  else if (gk == 1)
    kda_chunk_prep_kernel<VL, 1><<<grid_a, NT, LDS_A, s>>>(a, st, tiles);
  else
    kda_chunk_prep_kernel<VL, 2><<<grid_a, NT, LDS_A, s>>>(a, st, tiles);
  timing_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // table mode: the sequences split into groups of consecutive sequences with about equal chunk
  // counts, as many groups as keep every CU busy with one (column block, head, group) workgroup
  SeqTab stb = st;
  if (VL) {
    int G = (ncu + NBLK * a.H - 1) / (NBLK * a.H);
    G = G < 1 ? 1 : G > kVarlenGroups ? kVarlenGroups : G;
    G = G > st.n ? st.n : G;
    stb.grp0[0] = 0;
    for (int g = 1; g < G; ++g) {
      const long long target = (long long)st.total_chunks * g / G;
      int e = stb.grp0[g - 1] + 1;  // every group keeps at least one sequence
      while (e < st.n - (G - g) && st.chunk0[e] < target) ++e;
      stb.grp0[g] = e;
    }
    stb.grp0[G] = st.n;
    stb.ngroups = G;
  }
  const dim3 grid_b(NBLK * a.H, VL ? stb.ngroups : a.B);
  timing_begin(kname[1][kn], s);
  kda_chunk_state_kernel<VL><<<grid_b, NTB, LDS_B, s>>>(a, stb, tiles, ows);
  timing_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long rows = tokens * a.H;
  const dim3 ng((unsigned)((rows + 15) / 16));
  timing_begin(kname[2][kn], s);
  if (ot == kBF16)
    kda_out_norm_kernel<bf16_t><<<ng, 256, 0, s>>>(ows, static_cast<const bf16_t*>(a.g_out),
                                                   static_cast<const bf16_t*>(a.norm_w), static_cast<bf16_t*>(a.out),
                                                   rows, a.rms_eps);
  else
    kda_out_norm_kernel<float><<<ng, 256, 0, s>>>(ows, static_cast<const bf16_t*>(a.g_out),
                                                  static_cast<const bf16_t*>(a.norm_w), static_cast<float*>(a.out), rows,
                                                  a.rms_eps);
  timing_end(s);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const LayerArgs& a, const SeqTab& st, void* ws, size_t, int ot, hipStream_t s) {
  static_assert(C == kMfmaChunk, "chunk of the sequence tables");
  return st.n > 0 ? launch_mfma_t<true>(a, st, ws, ot, s) : launch_mfma_t<false>(a, st, ws, ot, s);
}

}  // namespace kda
