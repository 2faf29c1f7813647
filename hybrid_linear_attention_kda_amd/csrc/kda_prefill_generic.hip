// Chunked KDA prefill in fp32 on the vector ALUs (fp32 io, small heads).
//
// One workgroup owns one (sequence, head) and walks its chunks in order with
// the fp32 state resident in LDS.  Per chunk of L tokens (Gam = inclusive
// cumulative log-decay per key channel, S = chunk-start state):
//   A_kk[i,j] = beta_i sum_c k_i k_j exp(Gam_i - Gam_j)   (j < i)
//   A_qk[i,j] =        sum_c q_i k_j exp(Gam_i - Gam_j)   (j <= i)
//   W  = (I + A_kk)^-1 (beta K exp(Gam)),  Ut = (I + A_kk)^-1 (beta V)
//   U  = Ut - W S
//   O  = (Q exp(Gam)) S + A_qk U
//   S <- Diag(exp(Gam_L)) S + (K exp(Gam_L - Gam))^T U
// The pairwise factors exp(Gam_i - Gam_j) (<= 1) are formed per channel, so
// nothing overflows whatever the decay.  Every contraction is fp32 FMA: this
// is the path that holds the fp32 tolerance.  The conv / SiLU / L2 / gate
// prologue and the gated RMSNorm epilogue are fused in.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kGenericThreads = 1024;  // four waves per SIMD: the loops below are chains of LDS reads and FMAs
constexpr int kGenericChunkElems = 4096;  // internal chunk <= 4096 / D keeps LDS within 160 KB

__host__ __device__ constexpr int generic_chunk(int D, int chunk) {
  return chunk < kGenericChunkElems / D ? chunk : kGenericChunkElems / D;
}

__host__ __device__ constexpr size_t generic_lds_floats(int D, int Cc) {
  return (size_t)4 * Cc * (D + 1) + (size_t)D * D + (size_t)2 * Cc * (Cc + 1) + Cc + D + 2 * Cc;
}

template <int D, typename IO, typename OT>
__global__ __launch_bounds__(kGenericThreads) void kda_prefill_generic_kernel(LayerArgs a, SeqTab st, int Cc) {
  constexpr int NT = kGenericThreads;
  constexpr int NW = NT / 64;
  constexpr int LP = D + 1;
  const int AP = Cc + 1;
  extern __shared__ float smem[];
  float* sq = smem;                 // [Cc][LP]  q, then Q exp(Gam)
  float* sk = sq + Cc * LP;         // [Cc][LP]  k, then K exp(Gam_L - Gam)
  float* sv = sk + Cc * LP;         // [Cc][LP]  v, then beta V, Ut, U
  float* sg = sv + Cc * LP;         // [Cc][LP]  g, Gam, beta K exp(Gam), W, O
  float* sS = sg + Cc * LP;         // [D][D]    state
  float* sAkk = sS + D * D;         // [Cc][AP]
  float* sAqk = sAkk + Cc * AP;     // [Cc][AP]
  float* sbeta = sAqk + Cc * AP;    // [Cc]
  float* sgl = sbeta + Cc;          // [D]       Gam at the chunk's last token
  float* snrm = sgl + D;            // [2*Cc]    per-token q / k normalisers

  const int h = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const SeqView sq0 = st.n > 0 ? seq_view<true>(st, blockIdx.y, a.T, 0) : seq_view<false>(st, blockIdx.y, a.T, 0);
  const long long tok0 = sq0.tok0;  // packed token of the sequence's first token
  const long long b = sq0.slot;     // state and conv-state slot
  const int H = a.H, W = a.W, T = sq0.len;
  const long long Cqkv = 3LL * H * D;
  const long long bh = b * H + h;
  const IO* qkv = static_cast<const IO*>(a.qkv);
  const IO* fin = static_cast<const IO*>(a.f);
  const IO* bin = static_cast<const IO*>(a.beta);
  const IO* gin = static_cast<const IO*>(a.g_out);
  const IO* cw = static_cast<const IO*>(a.conv_w);
  const IO* nw = static_cast<const IO*>(a.norm_w);
  const IO* cin = static_cast<const IO*>(a.conv_in);
  OT* out = static_cast<OT*>(a.out);

  for (int e = tid; e < D * D; e += NT) sS[e] = a.state_in[bh * D * D + e];
  const float Ah = expf(a.A_log[h]);

  for (int c0 = 0; c0 < T; c0 += Cc) {
    const int L = min(Cc, T - c0);
    // -- prologue: conv (halo from earlier tokens or the conv state), SiLU, gate, beta
    for (int idx = tid; idx < L * 3 * D; idx += NT) {
      const int t = idx / (3 * D), c = idx % (3 * D);
      const int part = c / D, i = c % D;
      const long long gc = (long long)part * H * D + (long long)h * D + i;
      float y = 0.f;
      for (int w = 0; w < W; ++w) {
        const int tt = c0 + t - (W - 1) + w;
        const float x = tt >= 0 ? to_f32(qkv[(tok0 + tt) * Cqkv + gc])
                                : to_f32(cin[(b * Cqkv + gc) * (W - 1) + (W - 1) + tt]);
        y += to_f32(cw[gc * W + w]) * x;
      }
      (part == 0 ? sq : part == 1 ? sk : sv)[t * LP + i] = y / (1.0f + expf(-y));
    }
    for (int idx = tid; idx < L * D; idx += NT) {
      const int t = idx / D, i = idx % D;
      const float fv = to_f32(fin[(tok0 + c0 + t) * H * D + (long long)h * D + i]) +
                       a.dt_bias[(long long)h * D + i];
      sg[t * LP + i] = log_decay(a.gate, a.lb, Ah, fv);
    }
    for (int t = tid; t < L; t += NT) sbeta[t] = to_f32(bin[(tok0 + c0 + t) * H + h]);
    __syncthreads();
    // -- q/k L2 normalisation (one wave per token), q scale
    for (int t = wave; t < L; t += NW) {
      float qq = 0.f, kk = 0.f;
      for (int i = lane; i < D; i += 64) {
        qq += sq[t * LP + i] * sq[t * LP + i];
        kk += sk[t * LP + i] * sk[t * LP + i];
      }
      qq = wave_sum(qq);
      kk = wave_sum(kk);
      if (lane == 0) {
        snrm[t] = a.scale / fmaxf(sqrtf(qq), a.l2_eps);
        snrm[Cc + t] = 1.0f / fmaxf(sqrtf(kk), a.l2_eps);
      }
    }
    __syncthreads();
    for (int idx = tid; idx < L * D; idx += NT) {
      const int t = idx / D, i = idx % D;
      sq[t * LP + i] *= snrm[t];
      sk[t * LP + i] *= snrm[Cc + t];
    }
    // -- inclusive cumulative log-decay within the chunk
    for (int i = tid; i < D; i += NT) {
      float acc = 0.f;
      for (int t = 0; t < L; ++t) {
        acc += sg[t * LP + i];
        sg[t * LP + i] = acc;
      }
    }
    __syncthreads();
    // -- intra-chunk A_kk, A_qk with pairwise decay factors
    for (int p = tid; p < L * L; p += NT) {
      const int i = p / L, j = p % L;
      if (j > i) continue;
      float akk = 0.f, aqk = 0.f;
      for (int c = 0; c < D; ++c) {
        const float kj = sk[j * LP + c] * expf(sg[i * LP + c] - sg[j * LP + c]);
        akk += sk[i * LP + c] * kj;
        aqk += sq[i * LP + c] * kj;
      }
      sAkk[i * AP + j] = (j < i) ? sbeta[i] * akk : 0.f;
      sAqk[i * AP + j] = aqk;
    }
    for (int i = tid; i < D; i += NT) sgl[i] = sg[(L - 1) * LP + i];
    __syncthreads();
    // -- decay the operands: Q exp(Gam), K exp(Gam_L - Gam), rhs beta K exp(Gam) and beta V
    for (int idx = tid; idx < L * D; idx += NT) {
      const int t = idx / D, i = idx % D;
      const float G = sg[t * LP + i];
      const float e = expf(G);
      const float kv = sk[t * LP + i];
      sg[t * LP + i] = sbeta[t] * kv * e;
      sk[t * LP + i] = kv * expf(sgl[i] - G);
      sq[t * LP + i] *= e;
      sv[t * LP + i] *= sbeta[t];
    }
    __syncthreads();
    // -- UT solve by forward substitution: X[i] -= sum_{j<i} A_kk[i,j] X[j]  (X = W | Ut)
    for (int i = 1; i < L; ++i) {
      for (int col = tid; col < 2 * D; col += NT) {
        float* X = col < D ? sg : sv;
        const int cc = col < D ? col : col - D;
        float acc = X[i * LP + cc];
        for (int j = 0; j < i; ++j) acc -= sAkk[i * AP + j] * X[j * LP + cc];
        X[i * LP + cc] = acc;
      }
      __syncthreads();
    }
    // -- U = Ut - W S
    for (int idx = tid; idx < L * D; idx += NT) {
      const int i = idx / D, j = idx % D;
      float acc = sv[i * LP + j];
      for (int c = 0; c < D; ++c) acc -= sg[i * LP + c] * sS[c * D + j];
      sv[i * LP + j] = acc;
    }
    __syncthreads();
    // -- O = Q exp(Gam) S + A_qk U   (into sg; W is no longer needed)
    for (int idx = tid; idx < L * D; idx += NT) {
      const int i = idx / D, j = idx % D;
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc += sq[i * LP + c] * sS[c * D + j];
      for (int m = 0; m <= i; ++m) acc += sAqk[i * AP + m] * sv[m * LP + j];
      sg[i * LP + j] = acc;
    }
    __syncthreads();
    // -- S <- Diag(exp(Gam_L)) S + (K exp(Gam_L - Gam))^T U
    for (int idx = tid; idx < D * D; idx += NT) {
      const int c = idx / D, j = idx % D;
      float acc = expf(sgl[c]) * sS[c * D + j];
      for (int i = 0; i < L; ++i) acc += sk[i * LP + c] * sv[i * LP + j];
      sS[c * D + j] = acc;
    }
    // -- gated RMSNorm epilogue (one wave per token)
    for (int t = wave; t < L; t += NW) {
      float oo = 0.f;
      for (int i = lane; i < D; i += 64) oo += sg[t * LP + i] * sg[t * LP + i];
      oo = wave_sum(oo);
      const float rr = rsqrtf(oo / (float)D + a.rms_eps);
      const long long ob = (tok0 + c0 + t) * H * D + (long long)h * D;
      for (int i = lane; i < D; i += 64) {
        const float gv = to_f32(gin[ob + i]);
        store_as(&out[ob + i], sg[t * LP + i] * rr * to_f32(nw[i]) / (1.0f + expf(-gv)));
      }
    }
    __syncthreads();
  }

  for (int e = tid; e < D * D; e += NT) a.state_out[bh * D * D + e] = sS[e];
  // new conv state: the last W-1 raw inputs of (conv state || this call's tokens)
  if (a.conv_out != nullptr) {
    IO* cs = static_cast<IO*>(a.conv_out);
    for (int c = tid; c < 3 * D; c += NT) {
      const long long gc = (long long)(c / D) * H * D + (long long)h * D + (c % D);
      IO win[kMaxConvWidth - 1];
      for (int w = 0; w < W - 1; ++w) {
        const int tt = T - (W - 1) + w;
        win[w] = tt >= 0 ? qkv[(tok0 + tt) * Cqkv + gc] : cin[(b * Cqkv + gc) * (W - 1) + (W - 1) + tt];
      }
      for (int w = 0; w < W - 1; ++w) cs[(b * Cqkv + gc) * (W - 1) + w] = win[w];
    }
  }
}

template <int D, typename IO, typename OT>
static hipError_t launch_generic_t(const LayerArgs& a, const SeqTab& st, int Cc, hipStream_t s) {
  const size_t lds = generic_lds_floats(D, Cc) * sizeof(float);
  auto kern = kda_prefill_generic_kernel<D, IO, OT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  timing_begin("kda_prefill_generic_kernel", s);
  kern<<<dim3(a.H, st.n > 0 ? st.n : a.B), dim3(kGenericThreads), lds, s>>>(a, st, Cc);
  timing_end(s);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_generic_d(const LayerArgs& a, const SeqTab& st, int Cc, int io, int ot, hipStream_t s) {
  if (io == kBF16)
    return ot == kBF16 ? launch_generic_t<D, bf16_t, bf16_t>(a, st, Cc, s) : launch_generic_t<D, bf16_t, float>(a, st, Cc, s);
  return ot == kBF16 ? launch_generic_t<D, float, bf16_t>(a, st, Cc, s) : launch_generic_t<D, float, float>(a, st, Cc, s);
}

hipError_t launch_prefill_generic(const LayerArgs& a, const SeqTab& st, int chunk, int io, int ot, hipStream_t s) {
  const int Cc = generic_chunk(a.D, chunk);
  switch (a.D) {
    case 16: return launch_generic_d<16>(a, st, Cc, io, ot, s);
    case 32: return launch_generic_d<32>(a, st, Cc, io, ot, s);
    case 64: return launch_generic_d<64>(a, st, Cc, io, ot, s);
    case 128: return launch_generic_d<128>(a, st, Cc, io, ot, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
