// Token-recurrent KDA kernels: decode step, speculative verify block, rollback.
//
// One workgroup owns one (sequence, head).  Its d_k x d_v fp32 state is read
// from HBM once into registers (float4 per lane, coalesced along d_v), kept
// there across the tokens of the call, and written once per token (verify:
// one snapshot per token) or once at the end (decode).  There is no
// contraction worth a matrix core here: every state element takes part in
// three multiply-adds per token, so these kernels are HBM-bound and the
// design goal is one streaming read plus one streaming write of the state.
//
// Per token (the layer as described in llama.cpp PR #27754, KDA commit):
//   conv over this head's q|k|v channels from the rolling conv window, SiLU,
//   q/k L2 normalisation with max(||x||, eps), q scale, bounded-sigmoid decay
//   alpha = exp(lb * sigmoid(exp(A_log[h]) * (f + dt_bias))),
//   S' = Diag(alpha) S  (key axis = rows),  u = beta (v - S'^T k),
//   o = S'^T q + (q.k) u  (= (S' + k u^T)^T q, so S is swept only once),
//   S = S' + k u^T,  out = o / sqrt(mean(o^2) + eps) * w * sigmoid(g_out).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int D>
struct RecLayout {
  static constexpr int NT = (D >= 64) ? 256 : (D == 32 ? 128 : 64);
  static constexpr int CG = D / 4;     // float4 column groups of a state row
  static constexpr int RG = NT / CG;   // row groups
  static constexpr int RPT = D / RG;   // state rows held per lane
  static_assert(RG * CG == NT && RPT * RG == D, "layout");
};

template <int D, typename IO, typename OT>
__global__ __launch_bounds__(RecLayout<D>::NT) void kda_recurrent_kernel(LayerArgs a) {
  using L = RecLayout<D>;
  constexpr int NT = L::NT;
  constexpr int C3 = 3 * D;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int H = a.H, W = a.W, T = a.T;
  const long long Cqkv = 3LL * H * D;

  __shared__ float s_win[C3][kMaxConvWidth - 1];
  __shared__ float s_q[D], s_k[D], s_v[D], s_alpha[D], s_u[D], s_o[D];
  __shared__ float s_part[2][L::RG][D];
  __shared__ float s_red[4];

  const IO* qkv = static_cast<const IO*>(a.qkv);
  const IO* fin = static_cast<const IO*>(a.f);
  const IO* bin = static_cast<const IO*>(a.beta);
  const IO* gin = static_cast<const IO*>(a.g_out);
  const IO* cw = static_cast<const IO*>(a.conv_w);
  const IO* nw = static_cast<const IO*>(a.norm_w);
  const IO* cin = static_cast<const IO*>(a.conv_in);
  OT* out = static_cast<OT*>(a.out);

  // 1. Issue the state loads first so the prologue below overlaps them.
  const int cg = tid % L::CG;
  const int rg = tid / L::CG;
  const long long bh = (long long)b * H + h;
  float4 S[L::RPT];
  {
    const float* src = a.state_in + bh * D * D + 4 * cg;
#pragma unroll
    for (int r = 0; r < L::RPT; ++r)
      S[r] = *reinterpret_cast<const float4*>(src + (long long)(rg + r * L::RG) * D);
  }

  // 2. Conv window: the W-1 raw inputs before the first token, oldest first.
  for (int c = tid; c < C3; c += NT) {
    const long long gc = (long long)(c / D) * H * D + (long long)h * D + (c % D);
    for (int w = 0; w < W - 1; ++w) s_win[c][w] = to_f32(cin[(b * Cqkv + gc) * (W - 1) + w]);
  }
  const float Ah = __expf(a.A_log[h]);

  for (int t = 0; t < T; ++t) {
    const long long tok = (long long)b * T + t;
    __syncthreads();  // window ready; previous token's shared values consumed
    // conv + SiLU over this head's q|k|v channels; advance the window
    for (int c = tid; c < C3; c += NT) {
      const int part = c / D, i = c % D;
      const long long gc = (long long)part * H * D + (long long)h * D + i;
      const float x = to_f32(qkv[tok * Cqkv + gc]);
      float y = to_f32(cw[gc * W + (W - 1)]) * x;
      for (int w = 0; w < W - 1; ++w) y += to_f32(cw[gc * W + w]) * s_win[c][w];
      for (int w = 0; w + 1 < W - 1; ++w) s_win[c][w] = s_win[c][w + 1];
      if (W > 1) s_win[c][W - 2] = x;
      const float z = y / (1.0f + expf(-y));
      (part == 0 ? s_q : part == 1 ? s_k : s_v)[i] = z;
    }
    // bounded-sigmoid decay gate (log-decay in (lb, 0)), per key channel
    for (int i = tid; i < D; i += NT) {
      const float fv = to_f32(fin[tok * H * D + (long long)h * D + i]) + a.dt_bias[(long long)h * D + i];
      s_alpha[i] = expf(a.lb / (1.0f + expf(-Ah * fv)));
    }
    __syncthreads();
    if (tid < 64) {
      float qq = 0.f, kk = 0.f, qk = 0.f;
      for (int i = tid; i < D; i += 64) {
        qq += s_q[i] * s_q[i];
        kk += s_k[i] * s_k[i];
        qk += s_q[i] * s_k[i];
      }
      qq = wave_sum(qq);
      kk = wave_sum(kk);
      qk = wave_sum(qk);
      if (tid == 0) {
        const float rq = a.scale / fmaxf(sqrtf(qq), a.l2_eps);
        const float rk = 1.0f / fmaxf(sqrtf(kk), a.l2_eps);
        s_red[0] = rq;
        s_red[1] = rk;
        s_red[2] = qk * rq * rk;
      }
    }
    __syncthreads();
    const float rq = s_red[0], rk = s_red[1], qkn = s_red[2];

    // 3. One sweep over this lane's rows: decay, then partial S'^T k and S'^T q.
    float4 kS = make_float4(0.f, 0.f, 0.f, 0.f), qS = kS;
#pragma unroll
    for (int r = 0; r < L::RPT; ++r) {
      const int i = rg + r * L::RG;
      const float al = s_alpha[i], ki = s_k[i] * rk, qi = s_q[i] * rq;
      S[r].x *= al; S[r].y *= al; S[r].z *= al; S[r].w *= al;
      kS.x += ki * S[r].x; kS.y += ki * S[r].y; kS.z += ki * S[r].z; kS.w += ki * S[r].w;
      qS.x += qi * S[r].x; qS.y += qi * S[r].y; qS.z += qi * S[r].z; qS.w += qi * S[r].w;
    }
    *reinterpret_cast<float4*>(&s_part[0][rg][4 * cg]) = kS;
    *reinterpret_cast<float4*>(&s_part[1][rg][4 * cg]) = qS;
    __syncthreads();
    const float bt = to_f32(bin[tok * H + h]);
    for (int j = tid; j < D; j += NT) {
      float ks = 0.f, qs = 0.f;
#pragma unroll
      for (int g = 0; g < L::RG; ++g) {
        ks += s_part[0][g][j];
        qs += s_part[1][g][j];
      }
      const float u = bt * (s_v[j] - ks);
      s_u[j] = u;
      s_o[j] = qs + qkn * u;
    }
    __syncthreads();

    // 4. Rank-1 update in registers; verify streams a snapshot per token.
    {
      const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
      for (int r = 0; r < L::RPT; ++r) {
        const float ki = s_k[rg + r * L::RG] * rk;
        S[r].x += ki * u4.x; S[r].y += ki * u4.y; S[r].z += ki * u4.z; S[r].w += ki * u4.w;
      }
      if (a.snapshots) {
        float* dst = a.state_out + (tok * H + h) * D * D + 4 * cg;
#pragma unroll
        for (int r = 0; r < L::RPT; ++r)
          store_nt(dst + (long long)(rg + r * L::RG) * D, S[r]);
      }
    }

    // 5. Gated RMSNorm over d_v.
    if (tid < 64) {
      float oo = 0.f;
      for (int j = tid; j < D; j += 64) oo += s_o[j] * s_o[j];
      oo = wave_sum(oo);
      if (tid == 0) s_red[3] = rsqrtf(oo / (float)D + a.rms_eps);
    }
    __syncthreads();
    const float rr = s_red[3];
    for (int j = tid; j < D; j += NT) {
      const float gv = to_f32(gin[tok * H * D + (long long)h * D + j]);
      const float y = s_o[j] * rr * to_f32(nw[j]) / (1.0f + expf(-gv));
      store_as(&out[tok * H * D + (long long)h * D + j], y);
    }
  }

  if (!a.snapshots) {
    float* dst = a.state_out + bh * D * D + 4 * cg;
#pragma unroll
    for (int r = 0; r < L::RPT; ++r)
      *reinterpret_cast<float4*>(dst + (long long)(rg + r * L::RG) * D) = S[r];
  }
  if (a.conv_out != nullptr) {
    IO* cout_ = static_cast<IO*>(a.conv_out);
    __syncthreads();
    for (int c = tid; c < C3; c += NT) {
      const long long gc = (long long)(c / D) * H * D + (long long)h * D + (c % D);
      for (int w = 0; w < W - 1; ++w) store_as(&cout_[(b * Cqkv + gc) * (W - 1) + w], s_win[c][w]);
    }
  }
}

// Commit the accepted prefix of a verified draft block.
//   state[b]      <- snaps[b, m-1]                      (untouched when m == 0)
//   conv_state[b] <- last W-1 rows of (conv_state[b] || qkv[b, :m])
// grid.x splits a sequence's state into float4 ranges, grid.y = sequence.
template <typename IO>
__global__ __launch_bounds__(256) void kda_rollback_kernel(RollbackArgs a) {
  const int lb = blockIdx.y;
  const int m = a.accepted[lb];
  if (m == 0) return;
  const int b = a.B0 + lb;
  const long long HDD = (long long)a.H * a.D * a.D;
  const long long n4 = HDD / 4;
  const float4* src = reinterpret_cast<const float4*>(a.snaps + ((long long)b * a.T_d + (m - 1)) * HDD);
  float4* dst = reinterpret_cast<float4*>(a.state + (long long)b * HDD);
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) dst[i] = src[i];

  const long long Cqkv = 3LL * a.H * a.D;
  const int Wm1 = a.W - 1;
  IO* cs = static_cast<IO*>(a.conv_state);
  const IO* x = static_cast<const IO*>(a.qkv);
  for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < Cqkv; c += stride) {
    IO win[kMaxConvWidth - 1];
    // position p of (old window || accepted tokens), length Wm1 + m; keep p = m .. m + Wm1 - 1
    for (int w = 0; w < Wm1; ++w) {
      const int p = m + w;
      win[w] = (p < Wm1) ? cs[(b * Cqkv + c) * Wm1 + p] : x[((long long)b * a.T_d + (p - Wm1)) * Cqkv + c];
    }
    for (int w = 0; w < Wm1; ++w) cs[(b * Cqkv + c) * Wm1 + w] = win[w];
  }
}

template <int D>
static hipError_t launch_rec_d(const LayerArgs& a, int io, int ot, hipStream_t s) {
  dim3 grid(a.H, a.B), block(RecLayout<D>::NT);
  if (io == kBF16) {
    if (ot == kBF16)
      kda_recurrent_kernel<D, bf16_t, bf16_t><<<grid, block, 0, s>>>(a);
    else
      kda_recurrent_kernel<D, bf16_t, float><<<grid, block, 0, s>>>(a);
  } else {
    if (ot == kBF16)
      kda_recurrent_kernel<D, float, bf16_t><<<grid, block, 0, s>>>(a);
    else
      kda_recurrent_kernel<D, float, float><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_recurrent(const LayerArgs& a, int io, int ot, hipStream_t s) {
  switch (a.D) {
    case 16: return launch_rec_d<16>(a, io, ot, s);
    case 32: return launch_rec_d<32>(a, io, ot, s);
    case 64: return launch_rec_d<64>(a, io, ot, s);
    case 128: return launch_rec_d<128>(a, io, ot, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rollback(const RollbackArgs& a, int io, hipStream_t s) {
  const long long n4 = (long long)a.H * a.D * a.D / 4;
  int gx = (int)((n4 + 256 * 8 - 1) / (256 * 8));  // 8 float4 per lane
  if (gx < 1) gx = 1;
  dim3 grid(gx, a.nB), block(256);
  if (io == kBF16)
    kda_rollback_kernel<bf16_t><<<grid, block, 0, s>>>(a);
  else
    kda_rollback_kernel<float><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kda
