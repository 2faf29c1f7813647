// KDA input projection: the q, k, v, f_a, g_a and b projections of the hidden states as one
// weight matrix and one matmul over the concatenated output rows (glm53-flash-mlx README,
// quantization recipe: the runtime fuses the six KDA input projections into one matmul), then the
// low-rank up-projections f = f_b(f_a x) and g = g_b(g_a x) (the output gate is low rank,
// llama.cpp PR #27754, KDA commit) and beta = sigmoid(b x).
//
// Both steps are kernels of this library on the bf16 matrix cores with fp32 accumulation.  The
// fused matmul (kda_proj_gemm_kernel) writes the q|k|v columns straight into the layer's qkv input
// and the 2r + H rank / beta columns in fp32 into the workspace.  The low-rank kernel splits those
// fp32 rank-r activations into bf16 hi + lo (two matrix-core products per k-step, ~16 mantissa
// bits) so the only bf16 rounding an output sees is its own.
#include <algorithm>
#include <cstdio>

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
constexpr int PJ_CB = 8;                // 128-column blocks one low-rank workgroup walks
constexpr int PJ_OUT_POLICY = 2;        // cache policy of the low-rank outputs' stores: non-temporal

__device__ __forceinline__ f32x4 pj_mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void pj_store(float* p, float v) { *p = v; }
__device__ __forceinline__ void pj_store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
// four consecutive outputs of one token through a buffer resource (byte offset; out of range: dropped)
template <typename OT>
__device__ __forceinline__ void pj_buffer_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v);
template <>
__device__ __forceinline__ void pj_buffer_store4<float>(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, off, 0, PJ_OUT_POLICY);
}
template <>
__device__ __forceinline__ void pj_buffer_store4<bf16_t>(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  const __attribute__((ext_vector_type(2))) unsigned u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
}
// eight consecutive outputs of one token, a then b, through a buffer resource (as above)
template <typename OT>
__device__ __forceinline__ void pj_buffer_store8(__amdgpu_buffer_rsrc_t r, int off, f32x4 a, f32x4 b);
template <>
__device__ __forceinline__ void pj_buffer_store8<float>(__amdgpu_buffer_rsrc_t r, int off, f32x4 a, f32x4 b) {
  pj_buffer_store4<float>(r, off, a);
  pj_buffer_store4<float>(r, off + 16, b);
}
template <>
__device__ __forceinline__ void pj_buffer_store8<bf16_t>(__amdgpu_buffer_rsrc_t r, int off, f32x4 a, f32x4 b) {
  const __attribute__((ext_vector_type(4))) unsigned u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                          pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, PJ_OUT_POLICY);
}
// LDS row of weight row n within its 128-row block: n = 32 p + 8 a + 4 h + i goes to row
// 16 (2 p + h) + 4 a + i, so that product tile 2 p + h gives lane group a (accumulator rows
// 4 a .. 4 a + 3) the columns 32 p + 8 a + 4 h + 0..3, and the lane holds eight consecutive
// columns of its token over tiles 2 p and 2 p + 1
__device__ __forceinline__ int pj_lds_row(int n) {
  return 16 * (2 * (n >> 5) + ((n >> 2) & 1)) + 4 * ((n >> 3) & 3) + (n & 3);
}
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
// and g for which = 1.  A workgroup keeps one 64-token tile of activations in registers (split into
// bf16 hi + lo once) and walks up to PJ_CB consecutive 128-column blocks of W: block j + 1 is loaded
// into registers while block j is multiplied from LDS, then written into the other of two LDS
// buffers.  The product is taken transposed (out^T tile = W tile . act^T), with the weight rows
// placed in LDS in the order pj_lds_row gives, so that each lane ends with eight consecutive output
// columns of one token over two tiles and writes them as one 16-byte store (bf16; two for fp32),
// 64 contiguous bytes per token row and store; the stores go through a buffer resource that
// ends at row T, so rows past the end are dropped by the hardware and the loop has no branch.
//
// Workgroup b runs on L2 domain b % 8 and takes a row tile = b % 8 modulo 8, so one domain's L2
// holds the activations of its own row tiles only, beside the 2 MB of weights; within a domain
// the (column group, which) pairs run fastest.  The workgroups of column group 0 of f also write
// beta = sigmoid(b x) for their tile.
// two workgroups per CU by LDS (two weight buffers), so two waves per SIMD: the register budget
// that leaves keeps the next block's weights in registers without spilling them
template <typename OT>
__global__ __launch_bounds__(PJ_NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void kda_proj_lowrank_kernel(const float* __restrict__ act, int ld, int T,
                                                                 int HD, int H, const bf16_t* __restrict__ w_fb,
                                                                 const bf16_t* __restrict__ w_gb, OT* __restrict__ f,
                                                                 OT* __restrict__ g, OT* __restrict__ beta) {
  constexpr int R = kProjRank;
  __shared__ __align__(16) __bf16 sW[2][PJ_COLS * PJ_PB];
  const int ncb = HD / PJ_COLS, ncg = (ncb + PJ_CB - 1) / PJ_CB;
  const int xcd = blockIdx.x % PJ_XCD, k = blockIdx.x / PJ_XCD;
  const int r0 = ((k / (2 * ncg)) * PJ_XCD + xcd) * PJ_ROWS;
  if (r0 >= T) return;  // the spare workgroups of the last domains
  const int which = k % 2, cb0 = ((k % (2 * ncg)) / 2) * PJ_CB;
  const int nb = min(PJ_CB, ncb - cb0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const bf16_t* W = which == 0 ? w_fb : w_gb;
  OT* out = which == 0 ? f : g;

  // the weight rows of a column block, 16-byte pieces (16 per row)
  constexpr int NW = PJ_COLS * (R / 8) / PJ_NT;
  const bf16_t* wsrc = W + (long long)(tid / (R / 8)) * R + (tid % (R / 8)) * 8;  // piece j: + j * (PJ_NT / 16) rows
  constexpr int WROWS = PJ_NT / (R / 8);
  // LDS position of piece j (weight row tid / 16 + j WROWS of the block, permuted by pj_lds_row)
  auto wdst = [&](int j) __attribute__((always_inline)) {
    return pj_lds_row(tid / (R / 8) + j * WROWS) * PJ_PB + (tid % (R / 8)) * 8;
  };
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 wv[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) wv[j] = *reinterpret_cast<const u32x4*>(wsrc + ((long long)cb0 * PJ_COLS + j * WROWS) * R);
  // this wave's 16 activation rows (rows past T read row T-1; their outputs are dropped)
  const int trow = r0 + 16 * wave + l16;
  const float* ap = act + (long long)min(trow, T - 1) * ld + which * R + 8 * lg;
  float4 xv[R / 32][2];
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    xv[s][0] = *reinterpret_cast<const float4*>(ap + 32 * s);
    xv[s][1] = *reinterpret_cast<const float4*>(ap + 32 * s + 4);
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) *reinterpret_cast<u32x4*>(&sW[0][wdst(j)]) = wv[j];
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
  // output rows r0 .. T-1 of this workgroup's tile; lane: columns 32 p + 8 lg .. + 7 of token trow
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      out + (long long)r0 * HD, 0, (int)((long long)min(PJ_ROWS, T - r0) * HD * (int)sizeof(OT)), 0x00020000);
  const int obase = ((16 * wave + l16) * HD + 8 * lg) * (int)sizeof(OT);
  __syncthreads();
  for (int j = 0; j < nb; ++j) {
    // the next block (the last one again at the end)
    u32x4 wn[NW];
    const long long nrow = (long long)(cb0 + min(j + 1, nb - 1)) * PJ_COLS;
#pragma unroll
    for (int q = 0; q < NW; ++q) wn[q] = *reinterpret_cast<const u32x4*>(wsrc + (nrow + q * WROWS) * R);
    f32x4 acc[PJ_COLS / 16];
#pragma unroll
    for (int ct = 0; ct < PJ_COLS / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const __bf16* sb = sW[j & 1];
#pragma unroll
    for (int s = 0; s < R / 32; ++s)
#pragma unroll
      for (int ct = 0; ct < PJ_COLS / 16; ++ct) {
        const bf16x8 w = *reinterpret_cast<const bf16x8*>(sb + (16 * ct + l16) * PJ_PB + 32 * s + 8 * lg);
        acc[ct] = pj_mfma(w, xlo[s], acc[ct]);
        acc[ct] = pj_mfma(w, xhi[s], acc[ct]);
      }
    const int ob = obase + (cb0 + j) * PJ_COLS * (int)sizeof(OT);
#pragma unroll
    for (int p = 0; p < PJ_COLS / 32; ++p)
      pj_buffer_store8<OT>(orsrc, ob + 32 * p * (int)sizeof(OT), acc[2 * p], acc[2 * p + 1]);
    // buffer (j + 1) & 1 was last read in block j - 1, before the previous barrier
    __bf16* sn = sW[(j + 1) & 1];
#pragma unroll
    for (int q = 0; q < NW; ++q) *reinterpret_cast<u32x4*>(sn + wdst(q)) = wn[q];
    __syncthreads();
  }
  if (which == 0 && cb0 == 0) {
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

// ---------------------------------------------------------------------------------------------
// The fused projection matmul: D [T, N] = X [T, hidden] . W^T for the N = 3Hd + 2r + H rows of the
// fused weight.  It is taken transposed, D^T tile = W tile . X tile^T, so that each lane's
// accumulator holds four consecutive output columns of one token and stores them at once.
//
// One workgroup computes a 256-column x 256-token tile with 4 waves, one per SIMD, in a 2 x 2
// arrangement: each wave owns 128 columns x 128 tokens, 8 x 8 accumulator tiles of 16 x 16 (256
// fp32 per lane, pinned in the accumulation registers).  K advances in stages of 64 through two
// LDS slots of 64 KiB: stage s + 1 is copied global -> LDS (global_load_lds, 16 bytes a lane) while
// stage s is multiplied.  Each copy instruction moves 8 whole 128-byte rows (64 k) of one operand,
// so every request is a full cache line; within a row the eight 16-byte chunks are stored in an
// XOR-permuted order chosen so that an MFMA fragment read (16 rows x 32 k, lane l reading row
// l % 16, k 8 (l / 16) .. + 7) hits 16 different 16-byte bank groups per 16 lanes (and 8 per 8
// lanes): conflict-free 16-byte LDS reads.  Each wave reads the next half-stage's fragments into a
// second register set while the matrix cores work on the current one.
//
// Tiles are dealt to the 8 L2 domains (XCDs) so that the 32 tiles a domain runs at once are a
// compact block (4 token tiles x 8 column tiles sharing their operand rows in that L2).
// ---------------------------------------------------------------------------------------------
constexpr int GM = 256;                        // tokens per tile (X rows)
constexpr int GN = 256;                        // output columns per tile (W rows)
constexpr int GK = 64;                         // K per stage: one 128-byte row segment
constexpr int G_NT = 256;                      // 4 waves
constexpr int G_BLOCKS = (GM + GN) / 8;        // 64 copy blocks (8 rows x 128 bytes) per stage: W then X
constexpr int G_CPW = G_BLOCKS / (G_NT / 64);  // 16 copies per wave per stage
constexpr int G_STAGE = G_BLOCKS * 1024;       // 64 KiB
constexpr int G_XOFF = (GN / 8) * 1024;        // X blocks after the W blocks
constexpr int G_LDS = 2 * G_STAGE;             // 128 KiB
constexpr int G_MGROUP = 4;                    // token tiles per group of the tile order
constexpr int G_KSPLIT = 8;                    // K pieces of a rank / beta tile
static_assert(G_LDS <= 160 * 1024, "LDS budget");
static_assert(G_CPW == 16, "the wait counts below assume 16 copies per wave per stage");

__device__ __forceinline__ void g_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void g_store4(float* p, f32x4 v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void g_store4(bf16_t* p, f32x4 v) {
  uint2 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = u;
}

// acc += a . b^T on the matrix cores with the accumulator pinned in the accumulation registers:
// 256 fp32 per lane live across the K loop, which the register allocator otherwise splits between
// the two register files and shuffles every trip.
__device__ __forceinline__ void g_mfma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// the first product of an accumulator: acc = a . b^T (a zero constant for the addend, so no
// register is read before it is written)
__device__ __forceinline__ void g_mfma0(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// Wait until this wave's copies have all landed and its LDS reads have returned, then meet the
// other waves.  (The LDS wait repeated as a builtin tells the compiler that the operand registers
// have arrived, so it adds no wait of its own before the products, which would also wait on reads
// of the next half-stage issued in between.)
__device__ __forceinline__ void g_meet() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt not waited on
}

// position of 16-byte chunk c of row r (0..15 within a 16-row fragment) inside its 128-byte row
__device__ __forceinline__ int g_pos(int r, int c) { return c ^ (r & 7) ^ (r >> 3); }

// Work items of one launch (g_items): first the q|k|v tiles, full K each, dealt to the 8 L2 domains
// (block % 8) in 8 * ceil(tiles / 8) blocks; then the tiles of the 2r + H rank / beta columns, each
// split into `ksplit` K pieces that write fp32 partial sums to part[piece] [T, g_pitch(N - N3)],
// summed by kda_proj_act_reduce_kernel.  The rank / beta columns are 2.3% of the work at the layer's sizes:
// as whole tiles they would be the only work of a fourth round of tiles (768 q|k|v tiles fill three
// rounds of 256 CUs exactly); as pieces they add an eighth of one.
// row pitch of a partial-sum block: a multiple of 4 floats, so each lane stores its four columns
// as one 16-byte store (4-byte stores of the 37 MB of partial sums left partly written lines that
// took ~25 us more to write back when the launch ends)
__host__ __device__ inline int g_pitch(int ns) { return (ns + 3) & ~3; }

struct GItems {
  int MT, NQ, NA, ksplit, qblocks, nblocks;
};
__host__ __device__ inline GItems g_items(int T, int K, int N, int N3) {
  GItems g;
  g.MT = (T + GM - 1) / GM;
  g.NQ = (N3 + GN - 1) / GN;
  g.NA = (N - N3 + GN - 1) / GN;
  g.ksplit = min(G_KSPLIT, K / GK);
  g.qblocks = 8 * ((g.MT * g.NQ + 7) / 8);
  g.nblocks = g.qblocks + g.MT * g.NA * g.ksplit;
  return g;
}

// X [T, K] bf16, W [N, K] bf16 (rows of the fused weight), K a multiple of 128, N3 a multiple of 16.
// Columns n < N3 go to qkv [T, N3] (OT); columns N3 <= n < N go, as partial sums over K piece p, to
// part + p * T * P ([T, P] fp32 each, P = g_pitch(N - N3), columns past N - N3 unused).
template <typename OT>
__global__ __launch_bounds__(G_NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void kda_proj_gemm_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ Wt, int T, int K, int N, int N3, OT* __restrict__ qkv,
    float* __restrict__ part) {
  extern __shared__ __align__(16) unsigned char smem[];
  const GItems gi = g_items(T, K, N, N3);
  const int KS = K / GK;  // >= 2
  int m0, n0, s0, s1, piece = -1;
  if ((int)blockIdx.x < gi.qblocks) {
    const int G = gi.MT * gi.NQ;
    // logical tile: the blocks of one L2 domain (block % 8) take consecutive logical tiles
    const int per = gi.qblocks / 8;
    const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
    if (L >= G) return;
    // logical tiles run in groups of G_MGROUP token tiles x all column tiles, the token tile
    // fastest within a group, so a domain's 32 concurrent (consecutive) logical tiles span 4 x 8
    const int gsz = G_MGROUP * gi.NQ;
    const int grp = L / gsz, r = L % gsz;
    const int mrows = min(G_MGROUP, gi.MT - grp * G_MGROUP);
    m0 = (grp * G_MGROUP + r % mrows) * GM;
    n0 = (r / mrows) * GN;
    s0 = 0;
    s1 = KS;
  } else {
    // rank / beta piece: the K piece fastest, so one tile's pieces run side by side
    const int a = blockIdx.x - gi.qblocks;
    piece = a % gi.ksplit;
    const int t = a / gi.ksplit;
    m0 = (t / gi.NA) * GM;
    n0 = N3 + (t % gi.NA) * GN;
    s0 = KS * piece / gi.ksplit;
    s1 = KS * (piece + 1) / gi.ksplit;
  }
  const int nst = s1 - s0;  // >= 1 stages of this item

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;  // columns 128 wn .., tokens 128 wm ..

  // copies: this wave moves blocks q = wave + 4 i (q < 32: W rows n0 + 8 q .., else X rows
  // m0 + 8 (q - 32) ..); lane l takes row 8 q + l / 8 and stores at position l % 8 of it the chunk
  // that belongs there.  Byte offsets from the matrix base (both matrices are under 4 GiB); rows
  // past the end are clamped (computed, never stored).
  unsigned ofs[G_CPW];
  {
    const int rr = lane >> 3, p = lane & 7;
#pragma unroll
    for (int i = 0; i < G_CPW; ++i) {
      const int q = wave + 4 * i;
      const int c = p ^ rr ^ (q & 1);  // g_pos(8 (q & 1) + rr, c) == p
      const int row = q < GN / 8 ? min(n0 + 8 * q + rr, N - 1) : min(m0 + 8 * (q - GN / 8) + rr, T - 1);
      ofs[i] = (unsigned)row * (unsigned)(2 * K) + 16u * c;
    }
  }
  const unsigned char* wbase = reinterpret_cast<const unsigned char*>(Wt);
  const unsigned char* xbase = reinterpret_cast<const unsigned char*>(X);
  // copy i of the item's stage s (stages past its last re-copy the last one into a slot no later
  // read uses)
  auto dma = [&](int s, int slot, int i) __attribute__((always_inline)) {
    const int sk = (s0 + min(s, nst - 1)) * (2 * GK);
    g_dma16((i < G_CPW / 2 ? wbase : xbase) + sk + ofs[i], smem + slot * G_STAGE + (wave + 4 * i) * 1024);
  };
  // fragment reads: lane l reads row l % 16 of a fragment, chunk 4 h + l / 16 of half h
  const int fr = lane & 15;
  const unsigned char* rb0 = smem + (fr >> 3) * 1024 + 128 * (fr & 7) + 16 * g_pos(fr, lane >> 4);
  const unsigned char* rb1 = smem + (fr >> 3) * 1024 + 128 * (fr & 7) + 16 * g_pos(fr, 4 + (lane >> 4));
  // read r of a half-stage: r < 8 the W fragment 8 wn + r, else the X fragment 8 wm + r - 8
  auto rd = [&](int slot, int h, int r) __attribute__((always_inline)) -> bf16x8 {
    const unsigned char* b = (h ? rb1 : rb0) + slot * G_STAGE;
    const int off = r < 8 ? (8 * wn + r) * 2048 : G_XOFF + (8 * wm + r - 8) * 2048;
    return *reinterpret_cast<const bf16x8*>(b + off);
  };

  f32x4 acc[8][8];

  // one half-stage: the 64 products of register set (ca, cb), with the 16 reads of the next
  // half-stage (slot rs, half rh) into (na, nb) and (do_copy) the 16 copies of stage ds into slot
  // dsl spread evenly between them, one read or copy after every second product; the order is
  // kept as written.  (Copies any denser than one per four products stall the products: bunched
  // into the first half of the products, the same 16 copies cost 15% more cycles per tile.)
  auto half = [&](const bf16x8 (&ca)[8], const bf16x8 (&cb)[8], bf16x8 (&na)[8], bf16x8 (&nb)[8], int rs, int rh,
                  bool do_read, bool do_copy, int ds, int dsl, bool first = false) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      if (first)
        g_mfma0(acc[k >> 3][k & 7], ca[k >> 3], cb[k & 7]);
      else
        g_mfma(acc[k >> 3][k & 7], ca[k >> 3], cb[k & 7]);
      if (do_read && k % 4 == 0) {
        const int r = k / 4;
        if (r < 8)
          na[r] = rd(rs, rh, r);
        else
          nb[r - 8] = rd(rs, rh, r);
      }
      if (do_copy && k % 4 == 2) dma(ds, dsl, k / 4);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  bf16x8 a0[8], b0[8], a1[8], b1[8];
  // stage 0 -> slot 0, stage 1 -> slot 1 (stages counted from the item's first)
#pragma unroll
  for (int i = 0; i < G_CPW; ++i) dma(0, 0, i);
#pragma unroll
  for (int i = 0; i < G_CPW; ++i) dma(1, 1, i);
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int r = 0; r < 8; ++r) a0[r] = rd(0, 0, r);
#pragma unroll
  for (int r = 0; r < 8; ++r) b0[r] = rd(0, 0, 8 + r);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  half(a0, b0, a1, b1, 0, 1, true, false, 0, 0, true);  // stage 0 half 0, reading stage 0 half 1
  // Stage s (slot s % 2): its half 1 is in (a1, b1).  The meeting: every wave's copies of stage
  // s + 1 have landed and every wave's reads of stage s have returned, so slot s % 2 takes stage
  // s + 2 while half 1 of stage s is multiplied and half 0 of stage s + 1 read, then half 0 of
  // stage s + 1 is multiplied while its half 1 is read.
  auto stage = [&](int s, int sl) __attribute__((always_inline)) {
    g_meet();
    half(a1, b1, a0, b0, sl ^ 1, 0, true, true, s + 2, sl);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    half(a0, b0, a1, b1, sl ^ 1, 1, true, false, 0, 0);
  };
  int j = 0;
  for (; j + 1 <= nst - 2; j += 2) {
    stage(j, 0);
    stage(j + 1, 1);
  }
  if (j == nst - 2) stage(j, 0);  // its copies re-copy the last stage into slot 0
  g_meet();
  half(a1, b1, a0, b0, 0, 0, false, false, 0, 0);  // the last stage's half 1
  // the no-ops cover the matrix cores' result latency before the accumulators are read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // acc[i][j]: columns n0 + 16 (8 wn + i) + 4 lg .. + 3 of token m0 + 16 (8 wm + j) + l16
  const int l16 = lane & 15, lg = lane >> 4;
  const int NP = g_pitch(N - N3);
  float* pp = piece >= 0 ? part + (long long)piece * T * NP : nullptr;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int m = m0 + 16 * (8 * wm + jj) + l16;
    if (m >= T) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + 16 * (8 * wn + i) + 4 * lg;
      if (piece < 0) {
        if (n < N3) g_store4(qkv + (long long)m * N3 + n, acc[i][jj]);  // N3 a multiple of 16: n + 3 < N3
      } else if (n < N) {
        // the four columns n .. n + 3 lie inside the pitch (n - N3 < N - N3 <= P, P a multiple of 4)
        *reinterpret_cast<float4*>(pp + (long long)m * NP + (n - N3)) =
            make_float4(acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]);
      }
    }
  }
}

// act [T, ns] = sum over the K pieces of part [p] [T, np] (np = g_pitch(ns)): a wave per row, four
// consecutive columns per lane (16-byte loads; every piece's load issued before the sums)
__global__ __launch_bounds__(256) void kda_proj_act_reduce_kernel(const float* __restrict__ part, int pieces,
                                                                 int T, int ns, float* __restrict__ act) {
  const int np = g_pitch(ns), nq = np / 4;
  const long long pstride = (long long)T * np;
  const int lane = threadIdx.x & 63;
  for (long long t = blockIdx.x * 4LL + (threadIdx.x >> 6); t < T; t += gridDim.x * 4LL) {
    for (int c4 = lane; c4 < nq; c4 += 64) {
      const float* src = part + t * np + 4 * c4;
      float4 x[G_KSPLIT];
#pragma unroll
      for (int p = 0; p < G_KSPLIT; ++p)
        x[p] = *reinterpret_cast<const float4*>(src + min(p, pieces - 1) * pstride);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int p = 0; p < G_KSPLIT; ++p) {
        if (p < pieces) {
          v.x += x[p].x;
          v.y += x[p].y;
          v.z += x[p].z;
          v.w += x[p].w;
        }
      }
      float* dst = act + t * ns + 4 * c4;
      if ((ns & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = v;  // 4 c4 < np = ns
      } else {
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * c4 + j < ns) dst[j] = vv[j];
      }
    }
  }
}

}  // namespace

// workspace: the rank / beta activations act [T, 2r + H] fp32, then room for G_KSPLIT partial sums
// of them at a row pitch of g_pitch(2r + H) (the launch uses min(G_KSPLIT, hidden / 64) of them)
static size_t proj_act_bytes(int T, int H) {
  return ((size_t)T * g_pitch(2 * kProjRank + H) * sizeof(float) + 255) / 256 * 256;
}
size_t projection_workspace(int T, int H, int D) {
  (void)D;
  return (1 + G_KSPLIT) * proj_act_bytes(T, H);
}

hipError_t launch_projection(const ProjArgs& p, hipStream_t s, char* err, size_t errlen) {
  (void)err;
  (void)errlen;
  const int HD = p.H * p.D, N3 = 3 * HD, NS = 2 * kProjRank + p.H, N = N3 + NS;
  const size_t one = proj_act_bytes(p.T, p.H);
  float* act = static_cast<float*>(p.ws);
  float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(p.ws) + one);
  {
    hipError_t e0 = set_lds_limit(reinterpret_cast<const void*>(kda_proj_gemm_kernel<float>), G_LDS);
    if (e0 == hipSuccess) e0 = set_lds_limit(reinterpret_cast<const void*>(kda_proj_gemm_kernel<bf16_t>), G_LDS);
    if (e0 != hipSuccess) return e0;
  }
  const GItems gi = g_items(p.T, p.hidden, N, N3);
  {
    timing_begin("kda_proj_gemm_kernel", s);
    if (p.out_type == kBF16)
      kda_proj_gemm_kernel<bf16_t><<<gi.nblocks, G_NT, G_LDS, s>>>(static_cast<const bf16_t*>(p.x),
                                                                   static_cast<const bf16_t*>(p.w_in), p.T, p.hidden,
                                                                   N, N3, static_cast<bf16_t*>(p.qkv), part);
    else
      kda_proj_gemm_kernel<float><<<gi.nblocks, G_NT, G_LDS, s>>>(static_cast<const bf16_t*>(p.x),
                                                                  static_cast<const bf16_t*>(p.w_in), p.T, p.hidden,
                                                                  N, N3, static_cast<float*>(p.qkv), part);
    timing_end(s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    timing_begin("kda_proj_act_reduce_kernel", s);
    kda_proj_act_reduce_kernel<<<(unsigned)std::min<long long>((p.T + 3) / 4, 4096), 256, 0, s>>>(part, gi.ksplit,
                                                                                                 p.T, NS, act);
    timing_end(s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // per domain ceil(tiles / 8) row tiles, times the (column group, which) pairs
  const int tiles = (p.T + PJ_ROWS - 1) / PJ_ROWS;
  const dim3 grid(((tiles + PJ_XCD - 1) / PJ_XCD) * PJ_XCD * 2 * ((HD / PJ_COLS + PJ_CB - 1) / PJ_CB));
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
