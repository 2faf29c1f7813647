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
//
// Where (sequence, head) pairs alone would leave most CUs idle and out is fp32, the value columns
// are split over nvb workgroups per pair (grid.z): each one forms the key side (conv, norms, gate,
// A_kk, A_qk, W) in full and Ut, U, O and the state for its own D / nvb columns, writes O un-normed
// into out, and kda_prefill_generic_norm_kernel then applies the gated RMSNorm in place (it needs
// whole rows of O) and writes the new conv state: conv_state is updated in place, so it is written
// only once every column block has read the old one.
#include "kda_device.h"
#include "kda_launch.h"

#include <algorithm>
#include <type_traits>

namespace kda {

constexpr int kGenericThreads = 1024;  // four waves per SIMD: the loops below are chains of LDS reads and FMAs
constexpr int kGenericChunkElems = 4096;  // internal chunk <= 4096 / D keeps LDS within 160 KB
static_assert(kGenericChunkElems <= 4 * kGenericThreads, "the prologue loads a chunk's gate inputs in one batch of four");

__host__ __device__ constexpr int generic_chunk(int D, int chunk) {
  return chunk < kGenericChunkElems / D ? chunk : kGenericChunkElems / D;
}

__host__ __device__ constexpr size_t generic_lds_floats(int D, int Cc) {
  return (size_t)4 * Cc * (D + 1) + (size_t)D * D + (size_t)2 * Cc * (Cc + 1) + Cc + D + 2 * Cc;
}

// New conv state of head h of one sequence: the last W-1 raw inputs of (conv state || its tokens).
template <int D, typename IO>
__device__ void generic_conv_state(const LayerArgs& a, const SeqView& sv, int h, int tid, int nt) {
  const int H = a.H, W = a.W, T = sv.len;
  const long long Cqkv = 3LL * H * D, b = sv.slot, tok0 = sv.tok0;
  const IO* qkv = static_cast<const IO*>(a.qkv);
  const IO* cin = static_cast<const IO*>(a.conv_in);
  IO* cs = static_cast<IO*>(a.conv_out);
  for (int c = tid; c < 3 * D; c += nt) {
    const long long gc = (long long)(c / D) * H * D + (long long)h * D + (c % D);
    IO win[kMaxConvWidth - 1];
    for (int w = 0; w < W - 1; ++w) {
      const int tt = T - (W - 1) + w;
      win[w] = tt >= 0 ? qkv[(tok0 + tt) * Cqkv + gc] : cin[(b * Cqkv + gc) * (W - 1) + (W - 1) + tt];
    }
    for (int w = 0; w < W - 1; ++w) cs[(b * Cqkv + gc) * (W - 1) + w] = win[w];
  }
}

template <int D, typename IO, typename OT>
__global__ __launch_bounds__(kGenericThreads) void kda_prefill_generic_kernel(LayerArgs a, SeqTab st, int Cc, int nvb) {
  constexpr int NT = kGenericThreads;
  constexpr int NW = NT / 64;
  constexpr int LP = D + 1;
  const int AP = Cc + 1;
  extern __shared__ float smem[];
  float* sq = smem;                 // [Cc][LP]  q, then Q exp(Gam)
  float* sk = sq + Cc * LP;         // [Cc][LP]  k, then K exp(Gam_L - Gam)
  float* sv = sk + Cc * LP;         // [Cc][LP]  v, then beta V, Ut, U
  float* sg = sv + Cc * LP;         // [Cc][LP]  g, Gam, beta K exp(Gam), W, O
  float* sS = sg + Cc * LP;         // [D][DV]   this workgroup's state columns
  float* sAkk = sS + D * D;         // [Cc][AP]
  float* sAqk = sAkk + Cc * AP;     // [Cc][AP]
  float* sbeta = sAqk + Cc * AP;    // [Cc]
  float* sgl = sbeta + Cc;          // [D]       Gam at the chunk's last token
  float* snrm = sgl + D;            // [2*Cc]    per-token q / k normalisers

  const int h = blockIdx.x, tid = threadIdx.x;
  const int DV = D / nvb, v0 = blockIdx.z * DV;  // this workgroup's value columns v0 .. v0 + DV - 1
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

  for (int e = tid; e < D * DV; e += NT) sS[e] = a.state_in[bh * D * D + (long long)(e / DV) * D + v0 + e % DV];
  const float Ah = expf(a.A_log[h]);

  for (int c0 = 0; c0 < T; c0 += Cc) {
    const int L = min(Cc, T - c0);
    // -- prologue.  Every load below has a valid (clamped) address and its value is selected
    //    afterwards, so a thread issues all of a batch before its first use: the chunk costs a few
    //    memory round trips, not one per token.
    // gate and beta inputs first (L * D <= 4 * NT: one batch of four per thread)
    float fv[4], bv;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = min(tid + u * NT, L * D - 1), t = idx / D, i = idx % D;
      fv[u] = to_f32(fin[(tok0 + c0 + t) * H * D + (long long)h * D + i]) + a.dt_bias[(long long)h * D + i];
    }
    bv = to_f32(bin[(tok0 + c0 + min(tid, L - 1)) * H + h]);
    // conv (halo from earlier tokens or the conv state) and SiLU: a thread takes one of the 3D
    // channels and a run of tpg consecutive tokens, with its taps and an 8 + 7 value window in
    // registers; tap k of the eight multiplies token t - 7 + k (taps below 8 - W are zero)
    {
      constexpr int KW = kMaxConvWidth;
      const int G = NT / (3 * D), tpg = (L + G - 1) / G;
      const int c = tid % (3 * D), grp = tid / (3 * D);
      const int part = c / D, i = c % D;
      const long long gc = (long long)part * H * D + (long long)h * D + i;
      float* dst = part == 0 ? sq : part == 1 ? sk : sv;
      const int ts = grp * tpg, te = min(ts + tpg, L);
      if (grp < G && ts < te) {
        float wk[KW];
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          const int w = k - (KW - W);
          const float v = to_f32(cw[gc * W + max(w, 0)]);
          wk[k] = w >= 0 ? v : 0.f;
        }
        // raw input of token tt of this sequence (tt < -(W-1) meets only zero taps)
        auto raw = [&](int tt) {
          const bool from_state = tt < 0 && tt >= -(W - 1);
          const IO* p = from_state ? cin + (b * Cqkv + gc) * (W - 1) + (W - 1) + tt
                                   : qkv + (tok0 + min(max(tt, 0), T - 1)) * Cqkv + gc;
          const float v = to_f32(*p);
          return tt >= -(W - 1) ? v : 0.f;
        };
        float win[KW - 1 + 8];
#pragma unroll
        for (int k = 0; k < KW - 1; ++k) win[k] = raw(c0 + ts - (KW - 1) + k);
        for (int t0 = ts; t0 < te; t0 += 8) {
#pragma unroll
          for (int k = 0; k < 8; ++k) win[KW - 1 + k] = raw(c0 + t0 + k);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            float y = 0.f;
#pragma unroll
            for (int w = 0; w < KW; ++w) y += wk[w] * win[k + w];
            if (t0 + k < te) dst[(t0 + k) * LP + i] = y / (1.0f + expf(-y));
          }
#pragma unroll
          for (int k = 0; k < KW - 1; ++k) win[k] = win[8 + k];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + u * NT;
      if (idx < L * D) sg[(idx / D) * LP + idx % D] = log_decay(a.gate, a.lb, Ah, fv[u]);
    }
    if (tid < L) sbeta[tid] = bv;
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
    // -- UT solve by forward substitution: X[i] -= sum_{j<i} A_kk[i,j] X[j]  (X = W | this
    //    workgroup's columns of Ut).  A column's rows depend only on that column, and one thread
    //    owns each column (D + DV <= NT), so the rows need no barrier between them.
    //    Where a chunk has at most 32 rows the column sits in registers and the rows are unrolled,
    //    so the A_kk reads are independent of the running sums and all in flight together.
    static_assert(2 * D <= NT, "one thread per column of W | Ut");
    if (tid < D + DV) {
      float* X = tid < D ? sg : sv;
      const int cc = tid < D ? tid : v0 + tid - D;
      constexpr int R = kGenericChunkElems / D;  // rows of the largest chunk
      if constexpr (R <= 32) {
        float x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = X[min(r, L - 1) * LP + cc];
#pragma unroll
        for (int i = 1; i < R; ++i) {
          if (i < L) {
            float acc = x[i];
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= sAkk[i * AP + j] * x[j];
            x[i] = acc;
          }
        }
#pragma unroll
        for (int r = 1; r < R; ++r)
          if (r < L) X[r * LP + cc] = x[r];
      } else {
        for (int i = 1; i < L; ++i) {
          float acc = X[i * LP + cc];
#pragma unroll 8
          for (int j = 0; j < i; ++j) acc -= sAkk[i * AP + j] * X[j * LP + cc];
          X[i * LP + cc] = acc;
        }
      }
    }
    __syncthreads();
    // -- U = Ut - W S
    for (int idx = tid; idx < L * DV; idx += NT) {
      const int i = idx / DV, jj = idx % DV, j = v0 + jj;
      float acc = sv[i * LP + j];
      for (int c = 0; c < D; ++c) acc -= sg[i * LP + c] * sS[c * DV + jj];
      sv[i * LP + j] = acc;
    }
    __syncthreads();
    // -- O = Q exp(Gam) S + A_qk U   (into sg; W is no longer needed)
    for (int idx = tid; idx < L * DV; idx += NT) {
      const int i = idx / DV, jj = idx % DV, j = v0 + jj;
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc += sq[i * LP + c] * sS[c * DV + jj];
      for (int m = 0; m <= i; ++m) acc += sAqk[i * AP + m] * sv[m * LP + j];
      sg[i * LP + j] = acc;
    }
    __syncthreads();
    // -- S <- Diag(exp(Gam_L)) S + (K exp(Gam_L - Gam))^T U
    for (int idx = tid; idx < D * DV; idx += NT) {
      const int c = idx / DV, jj = idx % DV;
      float acc = expf(sgl[c]) * sS[c * DV + jj];
      for (int i = 0; i < L; ++i) acc += sk[i * LP + c] * sv[i * LP + v0 + jj];
      sS[c * DV + jj] = acc;
    }
    if (nvb > 1) {
      // split columns (out is fp32): O un-normed; the norm kernel finishes the rows
      for (int idx = tid; idx < L * DV; idx += NT) {
        const int t = idx / DV, j = v0 + idx % DV;
        store_as(&out[(tok0 + c0 + t) * H * D + (long long)h * D + j], sg[t * LP + j]);
      }
    } else
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

  for (int e = tid; e < D * DV; e += NT) a.state_out[bh * D * D + (long long)(e / DV) * D + v0 + e % DV] = sS[e];
  // with split columns the norm kernel writes the conv state (the other blocks still read it)
  if (a.conv_out != nullptr && nvb == 1) generic_conv_state<D, IO>(a, sq0, h, tid, NT);
}

// Gated RMSNorm of the un-normed fp32 O rows the split-column kernel left in out, in place, one wave
// per token row; grid (H, sequences, token slices).  Slice 0 also writes the new conv state.
constexpr int kGenericNormThreads = 256;

template <int D, typename IO>
__global__ __launch_bounds__(kGenericNormThreads) void kda_prefill_generic_norm_kernel(LayerArgs a, SeqTab st) {
  constexpr int NW = kGenericNormThreads / 64;
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SeqView sv = st.n > 0 ? seq_view<true>(st, blockIdx.y, a.T, 0) : seq_view<false>(st, blockIdx.y, a.T, 0);
  const int H = a.H;
  const IO* gin = static_cast<const IO*>(a.g_out);
  const IO* nw = static_cast<const IO*>(a.norm_w);
  float* out = static_cast<float*>(a.out);
  for (int t = blockIdx.z * NW + wave; t < sv.len; t += gridDim.z * NW) {
    const long long ob = (sv.tok0 + t) * H * D + (long long)h * D;
    float o[(D + 63) / 64];
    float oo = 0.f;
#pragma unroll
    for (int r = 0; r < (D + 63) / 64; ++r) {
      const int i = lane + 64 * r;
      o[r] = i < D ? out[ob + i] : 0.f;
      oo += o[r] * o[r];
    }
    oo = wave_sum(oo);
    const float rr = rsqrtf(oo / (float)D + a.rms_eps);
#pragma unroll
    for (int r = 0; r < (D + 63) / 64; ++r) {
      const int i = lane + 64 * r;
      if (i < D) {
        const float gv = to_f32(gin[ob + i]);
        out[ob + i] = o[r] * rr * to_f32(nw[i]) / (1.0f + expf(-gv));
      }
    }
  }
  if (a.conv_out != nullptr && blockIdx.z == 0) generic_conv_state<D, IO>(a, sv, h, tid, kGenericNormThreads);
}

// Column blocks per (sequence, head): enough workgroups for the 256 CUs where the pairs alone are
// too few, and only for fp32 out (it holds the un-normed O); each block keeps at least
// kGenericThreads / Cc columns so that its (token, column) loops still occupy every lane.
int generic_column_blocks(int D, int Cc, long long pairs, bool fp32_out) {
  int nvb = 1;
  if (!fp32_out) return nvb;
  while (pairs * nvb < 256 && D % (2 * nvb) == 0 && (D / (2 * nvb)) * Cc >= kGenericThreads) nvb *= 2;
  return nvb;
}

template <int D, typename IO, typename OT>
static hipError_t launch_generic_t(const LayerArgs& a, const SeqTab& st, int Cc, hipStream_t s) {
  const size_t lds = generic_lds_floats(D, Cc) * sizeof(float);
  auto kern = kda_prefill_generic_kernel<D, IO, OT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nseq = st.n > 0 ? st.n : a.B;
  const int nvb = generic_column_blocks(D, Cc, (long long)a.H * nseq, std::is_same<OT, float>::value);
  timing_begin("kda_prefill_generic_kernel", s);
  kern<<<dim3(a.H, nseq, nvb), dim3(kGenericThreads), lds, s>>>(a, st, Cc, nvb);
  timing_end(s);
  e = hipGetLastError();
  if (e != hipSuccess || nvb == 1) return e;
  // the norm pass: about 1024 workgroups, each slice at least 16 token rows per wave
  const long long pairs = (long long)a.H * nseq;
  int maxlen = a.T;
  if (st.n > 0) {
    maxlen = 0;
    for (int i = 0; i < st.n; ++i) maxlen = std::max(maxlen, st.tok0[i + 1] - st.tok0[i]);
  }
  int slices = (int)((1024 + pairs - 1) / pairs);
  slices = std::max(1, std::min(slices, (maxlen + 16 * 4 - 1) / (16 * 4)));
  timing_begin("kda_prefill_generic_norm_kernel", s);
  kda_prefill_generic_norm_kernel<D, IO><<<dim3(a.H, nseq, slices), dim3(kGenericNormThreads), 0, s>>>(a, st);
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
