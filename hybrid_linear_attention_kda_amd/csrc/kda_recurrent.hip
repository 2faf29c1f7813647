// Token-recurrent KDA kernels: decode step, speculative verify block, rollback,
// and the replay-tape commit.
//
// One workgroup owns one (sequence, head).  Its d_k x d_v fp32 state is read
// from HBM once into registers (float4 per lane, coalesced along d_v), kept
// there across the tokens of the call, and written once per token (verify:
// one snapshot per token), once at the end (decode), or not at all (verify
// with a replay tape: per token only alpha, k and u, 3 x d floats).  There is no
// contraction worth a matrix core here: every state element takes part in
// three multiply-adds per token, so these kernels are HBM-bound and the
// design goal is one streaming read plus one streaming write of the state.
//
// Per token (the layer as described in llama.cpp PR #27754, KDA commit):
//   conv over this head's q|k|v channels from the rolling conv window, SiLU,
//   q/k L2 normalisation with max(||x||, eps), q scale, decay
//   alpha = exp(lb * sigmoid(exp(A_log[h]) * (f + dt_bias))) (bounded gate) or
//   alpha = exp(-exp(A_log[h]) * softplus(f + dt_bias)) (softplus branch),
//   S' = Diag(alpha) S  (key axis = rows),  u = beta (v - S'^T k),
//   o = S'^T q + (q.k) u  (= (S' + k u^T)^T q, so S is swept only once),
//   S = S' + k u^T,  out = o / sqrt(mean(o^2) + eps) * w * sigmoid(g_out).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int D>
struct RecLayout {
#ifndef KDA_REC_NT128
#define KDA_REC_NT128 512
#endif
  static constexpr int NT = (D == 128) ? KDA_REC_NT128 : (D == 64 ? 256 : (D == 32 ? 128 : 64));
  static constexpr int CG = D / 4;     // float4 column groups of a state row
  static constexpr int RG = NT / CG;   // row groups
  static constexpr int RPT = D / RG;   // consecutive state rows held per lane
  static constexpr int NCH = (3 * D + NT - 1) / NT;  // conv channels per lane
  static_assert(RG * CG == NT && RPT * RG == D, "layout");
};

// MULTI: the call carries several tokens (verify); otherwise exactly one (decode).
// TAPE: verify that records the replay tape and writes no state.
// WMAX: compile-time bound on the conv width, so taps and window stay in registers.
template <int D, int WMAX, bool MULTI, bool TAPE, typename IO, typename OT>
__global__ __launch_bounds__(RecLayout<D>::NT) void kda_recurrent_kernel(LayerArgs a) {
  using L = RecLayout<D>;
  constexpr int NT = L::NT;
  constexpr int C3 = 3 * D;
  constexpr int NCH = L::NCH;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int H = a.H, W = a.W, T = MULTI ? a.T : 1;
  const int HD = H * D;
  const int Cqkv = 3 * HD;

  // q, k, v and alpha alternate between two buffers by token parity, so that the next token's
  // conv can write them while this token's update still reads k (no end-of-token barrier)
  __shared__ float s_q[2][D], s_k[2][D], s_v[2][D], s_alpha[2][D], s_u[D], s_o[D];
  __shared__ float s_part[2][L::RG][D];
  __shared__ float s_nrm[3][L::RG];  // per row group: sum q^2, sum k^2, sum q k (raw q, k)
  __shared__ float s_rk;

  // Uniform (per-workgroup) base pointers; lanes add 32-bit offsets.
  const long long bh = (long long)b * H + h;
  const IO* __restrict__ xq = static_cast<const IO*>(a.qkv) + (long long)b * T * Cqkv + h * D;
  const IO* __restrict__ xf = static_cast<const IO*>(a.f) + (long long)b * T * HD + h * D;
  const IO* __restrict__ xg = static_cast<const IO*>(a.g_out) + (long long)b * T * HD + h * D;
  const IO* __restrict__ xb = static_cast<const IO*>(a.beta) + (long long)b * T * H + h;
  OT* __restrict__ out = static_cast<OT*>(a.out) + (long long)b * T * HD + h * D;

  // 1. Small per-token and per-channel inputs first.  Loads retire in order, so issuing them
  //    ahead of the state lets the prologue below run while the state is still in flight.
  //    Conv taps are held right-aligned (tapr[0] multiplies the current token) and the window
  //    newest-first (win[j] = input j tokens back), so no register is indexed at run time.
  //    A snapshot verify loads the inputs of PF tokens ahead (a whole draft block of 8 at
  //    once), so no token waits on the latency of its own loads.  The tape verify, which has
  //    no state stores to hide them behind, keeps the registers for occupancy instead (two
  //    workgroups per CU) and loads one token ahead.
  constexpr int PF = (MULTI && !TAPE) ? 8 : 1;
  int choff[NCH];
  float tapr[NCH][WMAX], win[NCH][WMAX];
  float xs[PF][NCH], fs[PF], gs[PF], bs[PF];
#pragma unroll
  for (int n = 0; n < NCH; ++n) {
    const int c = tid + n * NT;
    const int cc = c < C3 ? c : 0;
    choff[n] = (cc / D) * HD + (cc % D);  // offset of the channel inside a token row (head h base)
    const IO* cwp = static_cast<const IO*>(a.conv_w) + ((long long)h * D + (long long)(cc / D) * HD + (cc % D)) * W;
    const IO* csp = static_cast<const IO*>(a.conv_in) +
                    ((long long)b * Cqkv + (long long)h * D + (long long)(cc / D) * HD + (cc % D)) * (W - 1);
#pragma unroll
    for (int j = 0; j < WMAX; ++j) {
      tapr[n][j] = (j < W) ? to_f32(cwp[W - 1 - j]) : 0.f;
      win[n][j] = (j >= 1 && j < W) ? to_f32(csp[W - 1 - j]) : 0.f;
    }
  }
  const int ci = tid < D ? tid : 0;
  // token tl's inputs into slot j (j is a compile-time index wherever this is called)
  auto load_token = [&](int j, int tl) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) xs[j][n] = to_f32(xq[(long long)tl * Cqkv + choff[n]]);
    fs[j] = to_f32(xf[(long long)tl * HD + ci]);
    gs[j] = to_f32(xg[(long long)tl * HD + ci]);
    bs[j] = to_f32(xb[(long long)tl * H]);
  };
  // tokens past the end re-read the last one: the loads stay unconditional
#pragma unroll
  for (int j = 0; j < PF; ++j) load_token(j, min(j, T - 1));
  const float dtb = a.dt_bias[h * D + ci];
  const float nwj = to_f32(static_cast<const IO*>(a.norm_w)[ci]);
  const float Ah = __expf(a.A_log[h]);

  // 2. The state: read once (streaming), kept in registers for the whole call.
  const int cg = tid % L::CG;
  const int rg = tid / L::CG;
  const int soff = rg * L::RPT * D + 4 * cg;
  float4 S[L::RPT];
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.state_in + bh * D * D + soff);
#pragma unroll
    for (int r = 0; r < L::RPT; ++r) {
      const f32x4 v = __builtin_nontemporal_load(src + r * (D / 4));
      S[r] = make_float4(v.x, v.y, v.z, v.w);
    }
  }

  for (int t0 = 0; t0 < T; t0 += PF) {
#pragma unroll
  for (int pj = 0; pj < PF; ++pj) {
    const int t = t0 + pj;
    if (t >= T) break;
    const int pb = t & 1;
    // conv + SiLU over this lane's channels; advance the window
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int c = tid + n * NT;
      float y = tapr[n][0] * xs[pj][n];
#pragma unroll
      for (int j = 1; j < WMAX; ++j) y += tapr[n][j] * win[n][j];
#pragma unroll
      for (int j = WMAX - 1; j >= 2; --j) win[n][j] = win[n][j - 1];
      win[n][1 % WMAX] = (WMAX > 1) ? xs[pj][n] : win[n][0];
      if (c < C3) {
        const float z = y / (1.0f + expf(-y));
        const int part = c / D, i = c % D;
        (part == 0 ? s_q[pb] : part == 1 ? s_k[pb] : s_v[pb])[i] = z;
      }
    }
    // decay gate (bounded sigmoid or the softplus branch), per key channel
    if (tid < D) s_alpha[pb][tid] = expf(log_decay(a.gate, a.lb, Ah, fs[pj] + dtb));
    const float bt = bs[pj], gcur = gs[pj];
    if (MULTI && t + PF < T) load_token(pj, t + PF);  // refill the slot: issued before this token's stores
    __syncthreads();

    // 3. One sweep over this lane's rows with the raw (unnormalised) q and k: decay, partial
    //    S'^T k and S'^T q, and the row group's share of |q|^2, |k|^2 and q.k.  The L2 scales
    //    are applied to the reduced sums, so no reduction stands between the conv and the sweep.
    float4 kS = make_float4(0.f, 0.f, 0.f, 0.f), qS = kS;
    float nq = 0.f, nk = 0.f, nqk = 0.f;
#pragma unroll
    for (int r = 0; r < L::RPT; ++r) {
      const int i = rg * L::RPT + r;
      const float al = s_alpha[pb][i], ki = s_k[pb][i], qi = s_q[pb][i];
      S[r].x *= al; S[r].y *= al; S[r].z *= al; S[r].w *= al;
      kS.x += ki * S[r].x; kS.y += ki * S[r].y; kS.z += ki * S[r].z; kS.w += ki * S[r].w;
      qS.x += qi * S[r].x; qS.y += qi * S[r].y; qS.z += qi * S[r].z; qS.w += qi * S[r].w;
      nq += qi * qi; nk += ki * ki; nqk += qi * ki;
    }
    *reinterpret_cast<float4*>(&s_part[0][rg][4 * cg]) = kS;
    *reinterpret_cast<float4*>(&s_part[1][rg][4 * cg]) = qS;
    if (cg == 0) {
      s_nrm[0][rg] = nq;
      s_nrm[1][rg] = nk;
      s_nrm[2][rg] = nqk;
    }
    __syncthreads();
    if (tid < D) {
      float ks = 0.f, qs = 0.f, qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
      for (int g = 0; g < L::RG; ++g) {
        ks += s_part[0][g][tid];
        qs += s_part[1][g][tid];
        qq += s_nrm[0][g];
        kk += s_nrm[1][g];
        qk += s_nrm[2][g];
      }
      const float rq = a.scale / fmaxf(sqrtf(qq), a.l2_eps);
      const float rk = 1.0f / fmaxf(sqrtf(kk), a.l2_eps);
      const float u = bt * (s_v[pb][tid] - rk * ks);
      s_u[tid] = u;
      s_o[tid] = rq * qs + (qk * rq * rk) * u;
      if (tid == 0) s_rk = rk;
    }
    __syncthreads();
    const float rk = s_rk;

    // 4. Rank-1 update in registers (one fused multiply-add per element, as the tape replay does);
    //    verify streams a snapshot per token, or the token's replay tape, decode the final state.
    {
      const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
      for (int r = 0; r < L::RPT; ++r) {
        const float ki = s_k[pb][rg * L::RPT + r] * rk;
        S[r].x = __builtin_fmaf(ki, u4.x, S[r].x);
        S[r].y = __builtin_fmaf(ki, u4.y, S[r].y);
        S[r].z = __builtin_fmaf(ki, u4.z, S[r].z);
        S[r].w = __builtin_fmaf(ki, u4.w, S[r].w);
      }
      if (TAPE) {
        if (tid < D) {
          float* tp = a.tape + (((long long)b * T + t) * H + h) * 3 * D;
          tp[tid] = s_alpha[pb][tid];
          tp[D + tid] = s_k[pb][tid] * rk;
          tp[2 * D + tid] = s_u[tid];
        }
      } else {
        float* dst = a.snapshots ? a.state_out + (((long long)b * T + t) * H + h) * D * D
                                 : a.state_out + bh * D * D;
        if (a.snapshots || t + 1 == T) {
#pragma unroll
          for (int r = 0; r < L::RPT; ++r) store_nt(dst + soff + r * D, S[r]);
        }
      }
    }

    // 5. Gated RMSNorm over d_v (the waves holding lanes < D reduce and write).  s_o and s_u
    //    are rewritten only after the next token's second barrier, which every lane reaches
    //    after this point.
    if (tid < ((D + 63) / 64) * 64) {
      float oo = 0.f;
      for (int j = lane; j < D; j += 64) oo += s_o[j] * s_o[j];
      oo = wave_sum(oo);
      if (tid < D) {
        const float rr = rsqrtf(oo / (float)D + a.rms_eps);
        store_as(&out[(long long)t * HD + tid], s_o[tid] * rr * nwj / (1.0f + expf(-gcur)));
      }
    }
  }
  }

  if (a.conv_out != nullptr) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int c = tid + n * NT;
      if (c < C3) {
        IO* csp = static_cast<IO*>(a.conv_out) + ((long long)b * Cqkv + (long long)h * D + (long long)(c / D) * HD + (c % D)) * (W - 1);
#pragma unroll
        for (int j = 1; j < WMAX; ++j)
          if (j < W) store_as(&csp[W - 1 - j], win[n][j]);
      }
    }
  }
}

// Commit the accepted prefix of a verified draft block.
//   state[b]      <- snaps[b, m-1]                      (untouched when m == 0)
//   conv_state[b] <- last W-1 rows of (conv_state[b] || qkv[b, :m])
// grid.x splits a sequence's state into float4 ranges, grid.y = sequence.
constexpr int kRollbackPer = 8;  // 16-byte pieces of the state copy per lane
template <typename IO>
__global__ __launch_bounds__(256) void kda_rollback_kernel(RollbackArgs a) {
  const int lb = blockIdx.y;
  const int m = a.accepted[lb];
  if (m == 0) return;
  const int b = a.B0 + lb;
  const long long HDD = (long long)a.H * a.D * a.D;
  const long long n4 = HDD / 4;
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v* __restrict__ src = reinterpret_cast<const f32x4v*>(a.snaps + ((long long)b * a.T_d + (m - 1)) * HDD);
  f32x4v* __restrict__ dst = reinterpret_cast<f32x4v*>(a.state + (long long)b * HDD);
  const long long stride = (long long)gridDim.x * blockDim.x;
  // the launch gives every lane at most kRollbackPer 16-byte pieces: all loads in flight before the
  // first store (the snapshot is read once, the state written once: non-temporal both ways)
  const long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  f32x4v v[kRollbackPer];
#pragma unroll
  for (int k = 0; k < kRollbackPer; ++k) v[k] = __builtin_nontemporal_load(src + min(i0 + k * stride, n4 - 1));
#pragma unroll
  for (int k = 0; k < kRollbackPer; ++k) {
    const long long i = i0 + k * stride;
    if (i < n4) __builtin_nontemporal_store(v[k], dst + i);
  }

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

// Commit the accepted prefix of a draft block verified with a replay tape: for t < m,
//   S <- Diag(alpha_t) S + k_t u_t^T
// with the (alpha, k, u) the verify call recorded.  The verify call computed u_t from exactly the
// state this replay reaches before token t, and performs the same multiply and fused multiply-add
// per element, so the committed state is bit-identical to its state after token m.  The conv
// state takes the last W-1 raw inputs, as in the rollback.  grid = (head x row block, sequence):
// a d = 128 state is split into four blocks of 32 rows, so that enough workgroups stream at once.
constexpr int kCommitNT = 256;
constexpr int kCommitTok = 8;  // tape tokens staged in LDS at a time
template <int D>
struct CommitLayout {
  static constexpr int NS = D == 128 ? 4 : 1;  // row blocks per head
  static constexpr int RW = D / NS;            // rows per workgroup
};
template <int D, typename IO>
__global__ __launch_bounds__(kCommitNT) void kda_commit_tape_kernel(CommitArgs a) {
  constexpr int NT = kCommitNT;
  constexpr int NS = CommitLayout<D>::NS;
  constexpr int CG = D / 4;                          // float4 per state row
  constexpr int NV = CommitLayout<D>::RW * D / 4;    // float4 in this workgroup's rows
  constexpr int PER = (NV + NT - 1) / NT;            // float4 per lane
  __shared__ float s_tp[kCommitTok * 3 * D];
  const int h = blockIdx.x / NS;
  const int part = blockIdx.x % NS;
  const int lbi = blockIdx.y;
  const int m = a.accepted[lbi];
  if (m == 0) return;
  const int b = a.B0 + lbi;
  const int tid = threadIdx.x;
  const int H = a.H;
  const int r0 = part * CommitLayout<D>::RW;
  float* S = a.state + ((long long)b * H + h) * D * D + (long long)r0 * D;
  float4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * NT;
    if (NV % NT == 0 || i < NV) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S) + i);
      v[k] = make_float4(x.x, x.y, x.z, x.w);
    }
  }
  const float* tp = a.tape + ((long long)b * a.T_d * H + h) * 3 * D;  // token t at tp + t * H * 3 * D
  for (int t0 = 0; t0 < m; t0 += kCommitTok) {
    const int nt = min(kCommitTok, m - t0);
    __syncthreads();  // the previous tokens' reads are done
    for (int i = tid; i < nt * 3 * D; i += NT) s_tp[i] = tp[(long long)(t0 + i / (3 * D)) * H * 3 * D + i % (3 * D)];
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const float* al = s_tp + t * 3 * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = tid + k * NT;
        if (NV % NT == 0 || i < NV) {
          const int row = r0 + i / CG, c4 = i % CG;
          const float alr = al[row], kr = al[D + row];
          const float4 u4 = *reinterpret_cast<const float4*>(al + 2 * D + 4 * c4);
          v[k].x *= alr; v[k].y *= alr; v[k].z *= alr; v[k].w *= alr;
          v[k].x = __builtin_fmaf(kr, u4.x, v[k].x);
          v[k].y = __builtin_fmaf(kr, u4.y, v[k].y);
          v[k].z = __builtin_fmaf(kr, u4.z, v[k].z);
          v[k].w = __builtin_fmaf(kr, u4.w, v[k].w);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * NT;
    if (NV % NT == 0 || i < NV) store_nt(S + 4 * i, v[k]);
  }

  // conv window of this head's q, k and v channels
  const long long HD = (long long)H * D, Cqkv = 3 * HD;
  const int Wm1 = a.W - 1;
  IO* cs = static_cast<IO*>(a.conv_state);
  const IO* x = static_cast<const IO*>(a.qkv);
  for (int j = part * NT + tid; Wm1 > 0 && j < 3 * D; j += NS * NT) {
    const long long c = (long long)(j / D) * HD + (long long)h * D + (j % D);
    IO win[kMaxConvWidth - 1];
    // position p of (old window || accepted tokens), length Wm1 + m; keep p = m .. m + Wm1 - 1
    for (int w = 0; w < Wm1; ++w) {
      const int p = m + w;
      win[w] = (p < Wm1) ? cs[(b * Cqkv + c) * Wm1 + p] : x[((long long)b * a.T_d + (p - Wm1)) * Cqkv + c];
    }
    for (int w = 0; w < Wm1; ++w) cs[(b * Cqkv + c) * Wm1 + w] = win[w];
  }
}

template <int D, int WMAX, bool MULTI, bool TAPE>
static hipError_t launch_rec_t(const LayerArgs& a, int io, int ot, hipStream_t s) {
  dim3 grid(a.H, a.B), block(RecLayout<D>::NT);
  // timing names per call kind, [softplus] for the decay branch without a bound
  static const char* const kname[2][3] = {
      {"kda_recurrent_kernel[decode]", "kda_recurrent_kernel[verify]", "kda_recurrent_kernel[verify_tape]"},
      {"kda_recurrent_kernel[decode][softplus]", "kda_recurrent_kernel[verify][softplus]",
       "kda_recurrent_kernel[verify_tape][softplus]"}};
  timing_begin(kname[a.gate != 0][TAPE ? 2 : a.snapshots ? 1 : 0], s);
  if (io == kBF16) {
    if (ot == kBF16)
      kda_recurrent_kernel<D, WMAX, MULTI, TAPE, bf16_t, bf16_t><<<grid, block, 0, s>>>(a);
    else
      kda_recurrent_kernel<D, WMAX, MULTI, TAPE, bf16_t, float><<<grid, block, 0, s>>>(a);
  } else {
    if (ot == kBF16)
      kda_recurrent_kernel<D, WMAX, MULTI, TAPE, float, bf16_t><<<grid, block, 0, s>>>(a);
    else
      kda_recurrent_kernel<D, WMAX, MULTI, TAPE, float, float><<<grid, block, 0, s>>>(a);
  }
  timing_end(s);
  return hipGetLastError();
}

// A one-token tape call runs the multi-token instance (its loop covers T = 1).
template <int D, int WMAX>
static hipError_t launch_rec_w(const LayerArgs& a, int io, int ot, hipStream_t s) {
  if (a.tape != nullptr) return launch_rec_t<D, WMAX, true, true>(a, io, ot, s);
  return a.T > 1 ? launch_rec_t<D, WMAX, true, false>(a, io, ot, s) : launch_rec_t<D, WMAX, false, false>(a, io, ot, s);
}

template <int D>
static hipError_t launch_rec_d(const LayerArgs& a, int io, int ot, hipStream_t s) {
  return a.W <= 4 ? launch_rec_w<D, 4>(a, io, ot, s) : launch_rec_w<D, kMaxConvWidth>(a, io, ot, s);
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
  int gx = (int)((n4 + 256 * kRollbackPer - 1) / (256 * kRollbackPer));  // kRollbackPer float4 per lane
  if (gx < 1) gx = 1;
  dim3 grid(gx, a.nB), block(256);
  timing_begin("kda_rollback_kernel", s);
  if (io == kBF16)
    kda_rollback_kernel<bf16_t><<<grid, block, 0, s>>>(a);
  else
    kda_rollback_kernel<float><<<grid, block, 0, s>>>(a);
  timing_end(s);
  return hipGetLastError();
}

template <int D>
static void commit_d(const CommitArgs& a, int io, hipStream_t s) {
  dim3 grid(a.H * CommitLayout<D>::NS, a.nB), block(kCommitNT);
  if (io == kBF16)
    kda_commit_tape_kernel<D, bf16_t><<<grid, block, 0, s>>>(a);
  else
    kda_commit_tape_kernel<D, float><<<grid, block, 0, s>>>(a);
}

hipError_t launch_commit_tape(const CommitArgs& a, int io, hipStream_t s) {
  timing_begin("kda_commit_tape_kernel", s);
  switch (a.D) {
    case 16: commit_d<16>(a, io, s); break;
    case 32: commit_d<32>(a, io, s); break;
    case 64: commit_d<64>(a, io, s); break;
    case 128: commit_d<128>(a, io, s); break;
    default: timing_end(s); return hipErrorInvalidValue;
  }
  timing_end(s);
  return hipGetLastError();
}

}  // namespace kda
