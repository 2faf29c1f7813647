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
// Work split.  The columns of S are independent (decay acts on rows, u is per
// column), so one workgroup owns (sequence, head, 16-column block of d_v):
// grid = 8 column blocks x H heads x B, 512 lanes, ~150 KB of LDS.  Each
// workgroup walks its head's chunks in order, recomputes the d_v-independent
// chunk quantities (conv, norms, gate, A_kk, T, W, A_qk) and carries its
// 128 x 16 fp32 state block in MFMA accumulators.  blockIdx.x = vb * H + h,
// so with H a multiple of 8 the eight workgroups of a head land on the same
// XCD and share its L2 for the chunk inputs.
//
// Per-channel decay inside MFMA tiles.  The chunk is cut into four 16-token
// sub-chunks anchored at their first token n(I).  Operands carry
// e^(Gam_i - Gam_n(I)) (<= 1) on rows and e^(Gam_n(J) - Gam_j) (<= e^(15|lb|))
// on columns, and block (I, J) of A multiplies the row operand by the
// per-channel factor e^(Gam_n(I) - Gam_n(J)) (<= 1).  With the bounded gate
// (|lb| <= 5.5) every factor stays a finite fp32 / bf16 number.
//
// Precision.  bf16 operands round to 8 bits; contractions that feed the
// output or the state directly use split bf16 (x = hi + lo, three MFMAs:
// hi.hi + hi.lo + lo.hi): A_qk, Ut, Q~ S, A_qk U, K~^T U.  A_kk and W run
// in plain bf16 and W S splits only S.  T is formed in fp32.
//
// The output RMSNorm needs all 128 columns of o, which live in eight
// workgroups, so o (fp32) goes to the workspace and a second, bandwidth-bound
// kernel applies the norm, weight and gate; it also writes the new conv state.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int D = 128;       // head size (d_k = d_v)
constexpr int C = 64;        // chunk
constexpr int NV = 16;       // d_v columns per workgroup
constexpr int NBLK = D / NV; // workgroups per head
constexpr int NT = 512;      // lanes
constexpr int HALO = 3;      // staged rows before the chunk (conv width <= 4)

constexpr int PQ = 132;      // fp32 pitch of [64][128] arrays
constexpr int PKB = 136;     // bf16 pitch of [64][128] arrays
constexpr int PA = 68;       // fp32 pitch of [64][64] arrays
constexpr int PT = 68;       // fp32 pitch of [16][64] (transposed token-major) arrays
constexpr int PS = 132;      // fp32 pitch of the transposed state block [16][128]
constexpr int PR = 280;      // bf16 pitch of the raw staging rows: q 128 | k 128 | v 16 | pad
constexpr int RROWS = C + HALO;

// LDS layout (bytes)
constexpr int OFF_Q = 0;                              // q^ -> QR = q e^(Gam - Gam_n)
constexpr int OFF_KB = OFF_Q + C * PQ * 4;            // KR (bf16) -> W (bf16)
constexpr int OFF_G = OFF_KB + C * PKB * 2;           // k^ -> KC = k e^(Gam_n - Gam)
constexpr int OFF_STG = OFF_G + C * PQ * 4;           // raw staging | Gam | A_kk + T | A_qk
constexpr int STG_BYTES = RROWS * PR * 2;             // 37520 >= 2 * C * PA * 4 and >= C * PQ * 4
constexpr int OFF_VT = OFF_STG + STG_BYTES;           // beta v, transposed [16][64]
constexpr int OFF_UT = OFF_VT + NV * PT * 4;          // U transposed [16][64]; scratch while forming T
constexpr int OFF_ST = OFF_UT + NV * PT * 4;          // state block transposed [16][128]
constexpr int OFF_GN = OFF_ST + NV * PS * 4;          // Gam at the four anchors + Gam_C [5][128]
constexpr int OFF_EN = OFF_GN + 5 * D * 4;            // e^(Gam_n(I)) [4][128]
constexpr int OFF_E = OFF_EN + 4 * D * 4;             // e^(Gam_n(I) - Gam_n(J)), I > J [6][128]
constexpr int OFF_FAC = OFF_E + 6 * D * 4;            // e^(Gam_C - Gam_n(J)) [4][128]
constexpr int OFF_GC = OFF_FAC + 4 * D * 4;           // e^(Gam_C) [128]
constexpr int OFF_BETA = OFF_GC + D * 4;              // [64]
constexpr int OFF_NRM = OFF_BETA + C * 4;             // q / k normalisers [2][64]
constexpr int OFF_SEG = OFF_NRM + 2 * C * 4;          // cumulative-sum segment totals [4][128]
constexpr int LDS_BYTES = OFF_SEG + 4 * D * 4;
static_assert(STG_BYTES >= 2 * C * PA * 4 && STG_BYTES >= C * PQ * 4, "staging aliases");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Split8 {
  bf16x8 hi, lo;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// (I, J) of the ten lower sub-chunk blocks, and the index of the factor table for I > J.
__device__ __forceinline__ void block_ij(int bi, int& I, int& J) {
  I = bi < 1 ? 0 : bi < 3 ? 1 : bi < 6 ? 2 : 3;
  J = bi - I * (I + 1) / 2;
}
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

template <typename OT>
__global__ __launch_bounds__(NT) void kda_prefill_mfma_kernel(LayerArgs a, float* __restrict__ ows) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sQ = reinterpret_cast<float*>(smem + OFF_Q);
  __bf16* sKb = reinterpret_cast<__bf16*>(smem + OFF_KB);
  float* sG = reinterpret_cast<float*>(smem + OFF_G);
  __bf16* sRaw = reinterpret_cast<__bf16*>(smem + OFF_STG);
  float* sGam = reinterpret_cast<float*>(smem + OFF_STG);
  float* sAkk = reinterpret_cast<float*>(smem + OFF_STG);
  float* sT = reinterpret_cast<float*>(smem + OFF_STG + C * PA * 4);
  float* sAqk = sAkk;  // A_kk is dead once T is formed
  float* sVT = reinterpret_cast<float*>(smem + OFF_VT);
  float* sUT = reinterpret_cast<float*>(smem + OFF_UT);
  float* sST = reinterpret_cast<float*>(smem + OFF_ST);
  float* sGn = reinterpret_cast<float*>(smem + OFF_GN);
  float* sEn = reinterpret_cast<float*>(smem + OFF_EN);
  float* sE = reinterpret_cast<float*>(smem + OFF_E);
  float* sFac = reinterpret_cast<float*>(smem + OFF_FAC);
  float* sGC = reinterpret_cast<float*>(smem + OFF_GC);
  float* sBeta = reinterpret_cast<float*>(smem + OFF_BETA);
  float* sNrm = reinterpret_cast<float*>(smem + OFF_NRM);
  float* sSeg = reinterpret_cast<float*>(smem + OFF_SEG);

  const int H = a.H, T = a.T, W = a.W;
  const int h = blockIdx.x % H;
  const int vb = blockIdx.x / H;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;  // MFMA row/column index and k-group
  const int HD = H * D, Cq = 3 * HD;

  const bf16_t* __restrict__ qkv = static_cast<const bf16_t*>(a.qkv) + (long long)b * T * Cq;
  const bf16_t* __restrict__ fin = static_cast<const bf16_t*>(a.f) + (long long)b * T * HD + h * D;
  const bf16_t* __restrict__ bin = static_cast<const bf16_t*>(a.beta) + (long long)b * T * H + h;
  const bf16_t* __restrict__ cw = static_cast<const bf16_t*>(a.conv_w);
  const bf16_t* __restrict__ cin = static_cast<const bf16_t*>(a.conv_in) + (long long)b * Cq * (W - 1);

  // State block: wave w owns channel rows 16w..16w+15; lane holds rows 16w+4lg+r, column l16.
  f32x4 Sacc;
  {
    const float* sp = a.state_in + ((long long)b * H + h) * D * D + vb * NV + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) Sacc[r] = sp[(16 * wave + 4 * lg + r) * D];
#pragma unroll
    for (int r = 0; r < 4; ++r) sST[l16 * PS + 16 * wave + 4 * lg + r] = Sacc[r];
  }
  const float Ah = __expf(a.A_log[h]);
  const float lb = a.lb;

  // conv taps of this lane's q/k channel (P2) and v column, zero-padded on the left to 4 taps
  const int cq = tid & 255;
  const long long gqk = cq < D ? (long long)h * D + cq : (long long)HD + h * D + (cq - D);
  float tq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = j - (4 - W);
    tq[j] = w >= 0 ? to_f32(cw[gqk * W + w]) : 0.f;
  }
  const int vj = tid & 15;
  const long long gv = 2LL * HD + (long long)h * D + vb * NV + vj;
  float tv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = j - (4 - W);
    tv[j] = w >= 0 ? to_f32(cw[gv * W + w]) : 0.f;
  }
  const float dtb = a.dt_bias[h * D + (tid & 127)];

  for (int c0 = 0; c0 < T; c0 += C) {
    const int L = min(C, T - c0);
    __syncthreads();  // the previous chunk is done with every aliased buffer

    // ---- P1: stage raw q | k | v-block rows for tokens c0-3 .. c0+63 (bf16) ----
    for (int idx = tid; idx < RROWS * 34; idx += NT) {
      const int r = idx / 34, sg = idx % 34;
      const int tt = c0 - HALO + r;
      long long ch;
      int col;
      if (sg < 16) {
        ch = (long long)h * D + sg * 8;
        col = sg * 8;
      } else if (sg < 32) {
        ch = (long long)HD + h * D + (sg - 16) * 8;
        col = D + (sg - 16) * 8;
      } else {
        ch = 2LL * HD + h * D + vb * NV + (sg - 32) * 8;
        col = 2 * D + (sg - 32) * 8;
      }
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (tt >= 0 && tt < T) {
        v = *reinterpret_cast<const uint4*>(qkv + (long long)tt * Cq + ch);
      } else if (tt < 0 && (W - 1) + tt >= 0) {
        uint16_t e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = cin[(ch + e) * (W - 1) + (W - 1) + tt];
        v = make_uint4(e8[0] | (uint32_t)e8[1] << 16, e8[2] | (uint32_t)e8[3] << 16, e8[4] | (uint32_t)e8[5] << 16,
                       e8[6] | (uint32_t)e8[7] << 16);
      }
      *reinterpret_cast<uint4*>(sRaw + r * PR + col) = v;
    }
    if (tid < C) sBeta[tid] = tid < L ? to_f32(bin[(long long)(c0 + tid) * H]) : 0.f;
    __syncthreads();

    // ---- P2: causal conv + SiLU.  q|k: lane -> channel cq, 32 tokens; v block: 2 tokens per lane ----
    {
      const int tb = 32 * (tid >> 8);
      const __bf16* col = sRaw + cq;
      float r0 = (float)col[(tb + 0) * PR], r1 = (float)col[(tb + 1) * PR], r2 = (float)col[(tb + 2) * PR];
      float* dst = cq < D ? sQ + cq : sG + (cq - D);
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int t = tb + i;
        const float r3 = (float)col[(t + 3) * PR];
        const float y = tq[0] * r0 + tq[1] * r1 + tq[2] * r2 + tq[3] * r3;
        dst[t * PQ] = t < L ? y / (1.0f + __expf(-y)) : 0.f;
        r0 = r1; r1 = r2; r2 = r3;
      }
      const int tg = tid >> 4;  // 0..31
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = 2 * tg + i;
        const __bf16* vc = sRaw + 2 * D + vj;
        const float y = tv[0] * (float)vc[t * PR] + tv[1] * (float)vc[(t + 1) * PR] + tv[2] * (float)vc[(t + 2) * PR] +
                        tv[3] * (float)vc[(t + 3) * PR];
        sVT[vj * PT + t] = t < L ? sBeta[t] * (y / (1.0f + __expf(-y))) : 0.f;
      }
    }
    __syncthreads();

    // ---- P3: bounded-sigmoid gate and its cumulative sum (lane -> channel, 16-token segment) ----
    {
      const int i = tid & 127, seg = tid >> 7;
      float gl[16];
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int t = 16 * seg + k;
        float g = 0.f;
        if (t < L) {
          const float fv = to_f32(fin[(long long)(c0 + t) * HD + i]) + dtb;
          g = lb / (1.0f + __expf(-Ah * fv));
        }
        acc += g;
        gl[k] = acc;
      }
      sSeg[seg * D + i] = acc;
      // ---- P4 (same phase): q / k L2 normalisers, one wave per 8 tokens ----
      for (int t = wave * 8; t < wave * 8 + 8; ++t) {
        const float q0 = sQ[t * PQ + lane], q1 = sQ[t * PQ + lane + 64];
        const float k0 = sG[t * PQ + lane], k1 = sG[t * PQ + lane + 64];
        const float qq = wave_sum(q0 * q0 + q1 * q1);
        const float kk = wave_sum(k0 * k0 + k1 * k1);
        if (lane == 0) {
          sNrm[t] = a.scale / fmaxf(sqrtf(qq), a.l2_eps);
          sNrm[C + t] = 1.0f / fmaxf(sqrtf(kk), a.l2_eps);
        }
      }
      __syncthreads();
      float off = 0.f;
      for (int s = 0; s < seg; ++s) off += sSeg[s * D + i];
#pragma unroll
      for (int k = 0; k < 16; ++k) sGam[(16 * seg + k) * PQ + i] = gl[k] + off;
      sGn[seg * D + i] = gl[0] + off;
      if (seg == 3) sGn[4 * D + i] = gl[15] + off;
    }
    __syncthreads();

    // ---- P5: anchored operands QR, KR (bf16), KC and the per-channel factor tables ----
    for (int idx = tid; idx < C * D; idx += NT) {
      const int t = idx >> 7, c = idx & 127;
      const float G = sGam[t * PQ + c];
      const float Gn = sGn[(t >> 4) * D + c];
      const float e1 = __expf(G - Gn);  // <= 1
      const float e2 = __expf(Gn - G);  // in [1, e^(15|lb|)]
      const float q = sQ[t * PQ + c] * sNrm[t];
      const float k = sG[t * PQ + c] * sNrm[C + t];
      sQ[t * PQ + c] = q * e1;
      sKb[t * PKB + c] = (__bf16)(k * e1);
      sG[t * PQ + c] = k * e2;
    }
    if (tid < D) {
      const int c = tid;
      const float GC = sGn[4 * D + c];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const float GI = sGn[I * D + c];
        sEn[I * D + c] = __expf(GI);
        sFac[I * D + c] = __expf(GC - GI);
#pragma unroll
        for (int J = 0; J < I; ++J) sE[pair_index(I, J) * D + c] = __expf(GI - sGn[J * D + c]);
      }
      sGC[c] = __expf(GC);
    }
    __syncthreads();

    // ---- P6a: A_kk = beta_i * KR_I E_IJ . KC_J^T (plain bf16), strictly lower ----
    for (int bi = wave; bi < 10; bi += 8) {
      int I, J;
      block_ij(bi, I, J);
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 32 * s + 8 * lg;
        bf16x8 av = *reinterpret_cast<const bf16x8*>(sKb + (16 * I + l16) * PKB + c);
        if (I > J) {
          const float* ef = sE + pair_index(I, J) * D + c;
#pragma unroll
          for (int e = 0; e < 8; ++e) av[e] = (__bf16)((float)av[e] * ef[e]);
        }
        float kc[8];
        ld8(sG + (16 * J + l16) * PQ + c, kc);
        acc = mfma(av, round8(kc), acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * lg + r, j = 16 * J + l16;
        sAkk[i * PA + j] = j < i ? sBeta[i] * acc[r] : 0.f;
      }
    }
    __syncthreads();

    // ---- P7: T = (I + A_kk)^-1 in fp32: diagonal 16x16 blocks by forward substitution ----
    if (wave == 0) {
      const int I = lg, cc = l16;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = (i == cc) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) v -= sAkk[(16 * I + i) * PA + 16 * I + j] * x[j];
        x[i] = v;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[(16 * I + i) * PA + 16 * I + cc] = x[i];
    } else {
      // zero the strictly-upper blocks of T
      for (int idx = tid - 64; idx < 6 * 256; idx += NT - 64) {
        const int blk = idx >> 8, e = idx & 255;
        const int I = blk < 3 ? 0 : blk < 5 ? 1 : 2;
        const int J = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
        sT[(16 * I + (e >> 4)) * PA + 16 * J + (e & 15)] = 0.f;
      }
    }
    __syncthreads();
    // off-diagonal blocks by distance d: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
    for (int d = 1; d < 4; ++d) {
      const int nb = 4 - d;
      for (int idx = tid; idx < nb * 256; idx += NT) {
        const int J = idx >> 8, i = (idx >> 4) & 15, jj = idx & 15, I = J + d;
        float m = 0.f;
        for (int K = J; K < I; ++K)
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) m += sAkk[(16 * I + i) * PA + 16 * K + kk] * sT[(16 * K + kk) * PA + 16 * J + jj];
        sUT[idx] = m;
      }
      __syncthreads();
      for (int idx = tid; idx < nb * 256; idx += NT) {
        const int J = idx >> 8, i = (idx >> 4) & 15, jj = idx & 15, I = J + d;
        float m = 0.f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
          if (kk <= i) m += sT[(16 * I + i) * PA + 16 * I + kk] * sUT[(J << 8) + (kk << 4) + jj];
        sT[(16 * I + i) * PA + 16 * J + jj] = -m;
      }
      __syncthreads();
    }

    // ---- P6b: A_qk = QR_I E_IJ . KC_J^T (split bf16), lower incl. diagonal; zero upper blocks read later ----
    for (int bi = wave; bi < 10; bi += 8) {
      int I, J;
      block_ij(bi, I, J);
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 32 * s + 8 * lg;
        float qv[8], kc[8];
        ld8(sQ + (16 * I + l16) * PQ + c, qv);
        if (I > J) {
          const float* ef = sE + pair_index(I, J) * D + c;
#pragma unroll
          for (int e = 0; e < 8; ++e) qv[e] *= ef[e];
        }
        ld8(sG + (16 * J + l16) * PQ + c, kc);
        acc = mfma3(split(qv), split(kc), acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * lg + r, j = 16 * J + l16;
        sAqk[i * PA + j] = j <= i ? acc[r] : 0.f;
      }
    }
    if (wave >= 6) {  // blocks (0,1) and (2,3) fall inside the 32-token k-steps of A_qk . U
      const int e = tid - 6 * 64;  // 0..127
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = e + 128 * k, blk = idx >> 8, ee = idx & 255;
        const int I = blk == 0 ? 0 : 2, J = I + 1;
        sAqk[(16 * I + (ee >> 4)) * PA + 16 * J + (ee & 15)] = 0.f;
      }
    }

    // ---- P8: W = T . (beta KR e^Gam_n) (plain bf16); wave -> 16 key channels ----
    f32x4 wacc[4] = {zero4(), zero4(), zero4(), zero4()};
    {
      const int c = 16 * wave + l16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tb = 32 * s + 8 * lg;
        const float fac = sEn[(tb >> 4) * D + c];
        float xv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = sBeta[tb + e] * (float)sKb[(tb + e) * PKB + c] * fac;
        const bf16x8 bx = round8(xv);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (32 * s > 16 * I + 15) continue;  // T is lower triangular
          float tvv[8];
          ld8(sT + (16 * I + l16) * PA + 32 * s + 8 * lg, tvv);
          wacc[I] = mfma(round8(tvv), bx, wacc[I]);
        }
      }
    }
    // ---- P9: Ut = T . (beta V) (split), waves 0..3 own row tile I = wave ----
    f32x4 uacc = zero4();
    if (wave < 4) {
      const int I = wave;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (32 * s > 16 * I + 15) continue;
        float tvv[8], vv[8];
        ld8(sT + (16 * I + l16) * PA + 32 * s + 8 * lg, tvv);
        ld8(sVT + l16 * PT + 32 * s + 8 * lg, vv);
        uacc = mfma3(split(tvv), split(vv), uacc);
      }
    }
    __syncthreads();  // every read of KR is done: W takes its place
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) sKb[(16 * I + 4 * lg + r) * PKB + 16 * wave + l16] = (__bf16)wacc[I][r];
    __syncthreads();

    // ---- S1: U = Ut - W S (waves 0..3, row tile I = wave) -> sUT ----
    if (wave < 4) {
      const int I = wave;
      f32x4 pacc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 32 * s + 8 * lg;
        const bf16x8 aw = *reinterpret_cast<const bf16x8*>(sKb + (16 * I + l16) * PKB + c);
        float sv[8];
        ld8(sST + l16 * PS + c, sv);
        const Split8 bs = split(sv);
        pacc = mfma(aw, bs.lo, pacc);
        pacc = mfma(aw, bs.hi, pacc);
      }
      float4 u4;
      u4.x = uacc[0] - pacc[0];
      u4.y = uacc[1] - pacc[1];
      u4.z = uacc[2] - pacc[2];
      u4.w = uacc[3] - pacc[3];
      *reinterpret_cast<float4*>(sUT + l16 * PT + 16 * I + 4 * lg) = u4;
    }
    __syncthreads();

    // ---- S3: O = (QR e^Gam_n) S + A_qk U (waves 4..7, row tile I = wave - 4) -> workspace ----
    if (wave >= 4) {
      const int I = wave - 4;
      f32x4 oacc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 32 * s + 8 * lg;
        float qv[8], sv[8];
        ld8(sQ + (16 * I + l16) * PQ + c, qv);
        const float* en = sEn + I * D + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] *= en[e];
        ld8(sST + l16 * PS + c, sv);
        oacc = mfma3(split(qv), split(sv), oacc);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (32 * s > 16 * I + 15) continue;
        float av[8], uv[8];
        ld8(sAqk + (16 * I + l16) * PA + 32 * s + 8 * lg, av);
        ld8(sUT + l16 * PT + 32 * s + 8 * lg, uv);
        oacc = mfma3(split(av), split(uv), oacc);
      }
      float* op = ows + (((long long)b * T + c0) * H + h) * D + vb * NV + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * I + 4 * lg + r;
        if (t < L) op[(long long)t * HD] = oacc[r];
      }
    }
    // ---- S4: S <- e^Gam_C S + (KC e^(Gam_C - Gam_n))^T U (all waves, channel tile = wave) ----
    {
      f32x4 sn;
#pragma unroll
      for (int r = 0; r < 4; ++r) sn[r] = sGC[16 * wave + 4 * lg + r] * Sacc[r];
      const int c = 16 * wave + l16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tb = 32 * s + 8 * lg;
        const float fac = sFac[(tb >> 4) * D + c];
        float kv[8], uv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = sG[(tb + e) * PQ + c] * fac;
        ld8(sUT + l16 * PT + tb, uv);
        sn = mfma3(split(kv), split(uv), sn);
      }
      Sacc = sn;
    }
    __syncthreads();  // the old state block has been read by S1 and S3
#pragma unroll
    for (int r = 0; r < 4; ++r) sST[l16 * PS + 16 * wave + 4 * lg + r] = Sacc[r];
  }

  {
    float* sp = a.state_out + ((long long)b * H + h) * D * D + vb * NV + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) sp[(16 * wave + 4 * lg + r) * D] = Sacc[r];
  }
}

// out = o / sqrt(mean(o^2) + eps) * w * sigmoid(g_out), one wave per (token, head) row of 128.
template <typename OT>
__global__ __launch_bounds__(256) void kda_out_norm_kernel(const float* __restrict__ ows, const bf16_t* __restrict__ gout,
                                                        const bf16_t* __restrict__ nw, OT* __restrict__ out,
                                                        long long rows, float eps) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float2 o = *reinterpret_cast<const float2*>(ows + row * D + 2 * lane);
  const float ss = wave_sum(o.x * o.x + o.y * o.y);
  const float rr = rsqrtf(ss / (float)D + eps);
  const uint32_t g2 = *reinterpret_cast<const uint32_t*>(gout + row * D + 2 * lane);
  const uint32_t w2 = *reinterpret_cast<const uint32_t*>(nw + 2 * lane);
  const float g0 = __uint_as_float(g2 << 16), g1 = __uint_as_float(g2 & 0xffff0000u);
  const float w0 = __uint_as_float(w2 << 16), w1 = __uint_as_float(w2 & 0xffff0000u);
  store_as(out + row * D + 2 * lane, o.x * rr * w0 / (1.0f + __expf(-g0)));
  store_as(out + row * D + 2 * lane + 1, o.y * rr * w1 / (1.0f + __expf(-g1)));
}

// New conv state: the last W-1 raw inputs of (conv state || this call's tokens), per channel.
__global__ __launch_bounds__(256) void kda_conv_state_kernel(LayerArgs a) {
  const int Cq = 3 * a.H * a.D;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= Cq) return;
  const int W = a.W, T = a.T;
  const bf16_t* x = static_cast<const bf16_t*>(a.qkv);
  bf16_t* cs = static_cast<bf16_t*>(a.conv_out);
  const bf16_t* ci = static_cast<const bf16_t*>(a.conv_in);
  bf16_t win[3];
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (w < W - 1) {
      const int tt = T - (W - 1) + w;
      win[w] = tt >= 0 ? x[((long long)b * T + tt) * Cq + c] : ci[((long long)b * Cq + c) * (W - 1) + (W - 1) + tt];
    }
  }
#pragma unroll
  for (int w = 0; w < 3; ++w)
    if (w < W - 1) cs[((long long)b * Cq + c) * (W - 1) + w] = win[w];
}

}  // namespace

// The anchored decay factors stay finite only for a bounded gate (15 |lb| < 87), and the
// staging halo covers conv widths up to 4.
bool prefill_mfma_supported(int Dh, int chunk, int io, int W, float lb) {
  return Dh == D && chunk == C && io == kBF16 && W >= 1 && W <= HALO + 1 && lb <= 0.f && lb >= -5.5f;
}

size_t prefill_mfma_workspace(int B, int T, int H, int Dh, int) {
  return (size_t)B * T * H * Dh * sizeof(float);
}

hipError_t launch_prefill_mfma(const LayerArgs& a, void* ws, size_t, int ot, hipStream_t s) {
  float* ows = static_cast<float*>(ws);
  const dim3 grid(NBLK * a.H, a.B), block(NT);
  hipError_t e;
  if (ot == kBF16) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kda_prefill_mfma_kernel<bf16_t>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
    kda_prefill_mfma_kernel<bf16_t><<<grid, block, LDS_BYTES, s>>>(a, ows);
  } else {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kda_prefill_mfma_kernel<float>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
    kda_prefill_mfma_kernel<float><<<grid, block, LDS_BYTES, s>>>(a, ows);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long rows = (long long)a.B * a.T * a.H;
  const dim3 ng((unsigned)((rows + 3) / 4));
  if (ot == kBF16)
    kda_out_norm_kernel<bf16_t><<<ng, 256, 0, s>>>(ows, static_cast<const bf16_t*>(a.g_out),
                                                   static_cast<const bf16_t*>(a.norm_w), static_cast<bf16_t*>(a.out),
                                                   rows, a.rms_eps);
  else
    kda_out_norm_kernel<float><<<ng, 256, 0, s>>>(ows, static_cast<const bf16_t*>(a.g_out),
                                                  static_cast<const bf16_t*>(a.norm_w), static_cast<float*>(a.out), rows,
                                                  a.rms_eps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.W > 1 && a.conv_out != nullptr) {
    const int Cq = 3 * a.H * a.D;
    kda_conv_state_kernel<<<dim3((Cq + 255) / 256, a.B), 256, 0, s>>>(a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kda
