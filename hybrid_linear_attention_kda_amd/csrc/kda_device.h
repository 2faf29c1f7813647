// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_launch.h"

namespace kda {

// bf16 values travel as raw 16-bit patterns; fp32 as float.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// Round to nearest even on the hardware conversion (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }

// Two values rounded as above into one 32-bit word, a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void store_as(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_as(bf16_t* p, float v) { *p = f32_to_bf16(v); }

template <typename T>
__device__ __forceinline__ float load_f32(const T* p) { return to_f32(*p); }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte store: data written once and not re-read by this kernel.
__device__ __forceinline__ void store_nt(float* p, float4 v) {
  f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Per-channel log-decay from x = f + dt_bias and A = exp(A_log[h]) (llama.cpp PR #27754, KDA and
// metadata commits): gate 0, the bounded sigmoid lb * sigmoid(A x) in (lb, 0); gate 1, the softplus
// branch -A * softplus(x) in (-inf, 0), softplus(x) = max(x, 0) + log(1 + e^-|x|).
__device__ __forceinline__ float log_decay(int gate, float lb, float A, float x) {
  if (gate == 0) return lb / (1.0f + expf(-A * x));
  return -A * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sequence b of a prefill launch: first packed token, length, first chunk block, state slot.
struct SeqView {
  long long tok0;
  int len, chunk0, slot;
};
// TABLE: the launch carries a sequence table (st.n >= 1); otherwise the uniform layout.
template <bool TABLE>
__device__ __forceinline__ SeqView seq_view(const SeqTab& st, int b, int T, int NC) {
  SeqView v;
  if (!TABLE) {
    v.tok0 = (long long)b * T;
    v.len = T;
    v.chunk0 = b * NC;
    v.slot = b;
  } else {
    v.tok0 = st.tok0[b];
    v.len = st.tok0[b + 1] - st.tok0[b];
    v.chunk0 = st.chunk0[b];
    v.slot = st.slot[b];
  }
  return v;
}

}  // namespace kda
