// HIP kernels for gfx950 (MI355X): multi-axis RoPE and packed varlen
// flash-attention forward.
//
// The operation: every token of a packed video+audio sequence attends to
// every token of its own segment ("Day 0 Support for MiniMax-H3 on AMD
// Instinct GPUs", "The diffusion transformer (DiT)"; vLLM-Omni "MiniMax-H3"
// recipe, "Step execution and continuous batching"), with queries and keys
// turned by a rotary embedding of their (t, h, w) position.
//
// Three kernels:
//   rope_apply_kernel   y = rope(x): one 16-byte chunk (8 dims) per thread.
//   kv_prologue_kernel  rotates K once per call and packs it, with V
//                       transposed, into 64-key tiles that start on a 64-key
//                       boundary for every segment.  HBM-bound.
//   attn_fwd_kernel     one workgroup per (query tile, segment, head).  It
//                       rotates its queries while loading them, then streams
//                       the segment's key tiles through LDS and runs an online
//                       softmax between two bf16 MFMA contractions.
//
// MFMA orientation.  The score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims (from LDS), B = 16 dims x
// 32 queries (held in registers for the whole kernel).  In the 32x32
// accumulator, lane L owns query column L % 32 and the 16 key rows
// 8*(r/4) + 4*(L/32) + r%4, r = 0..15; the other 16 keys of that query sit in
// lane L ^ 32.  So a row maximum or row sum is an in-lane reduction plus one
// v_permlane32_swap.  The probabilities then serve directly as the B operand
// of O^T += V^T P^T (keys are the contraction index), with no data movement:
// registers 8*hh .. 8*hh+7 of a sub-block hold 8 keys of one 16-key group.
// The prologue stores V^T with its keys permuted inside each 16-key group so
// that the matching A operand (8 keys of one value dim) is one contiguous
// 16-byte LDS read.
//
// Operand precision.  The rotated queries and keys feed the score contraction
// as fp16 with power-of-two block scales: each query row and each 64-key tile
// is scaled so its largest magnitude lands in [2^14, 2^15) before rounding.
// That keeps bf16's range with fp16's 11-bit significand (8x finer rounding
// than bf16; bf16 operands alone put the log-sum-exp off by up to ~1.1e-3 on
// short sequences).  The two scales multiply into the one coefficient that
// already turns raw scores into base-2 logits, so the inner loop pays nothing
// for them.  P and V stay bf16 for the second contraction.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace h3attn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr int D = kHeadDim;
constexpr int BK = kKeyTile;                    // keys per tile
constexpr int CHUNKS_PER_ROW = D / 8;           // 16-byte chunks per 128-dim row
constexpr int TILE_CHUNKS = BK * CHUNKS_PER_ROW;  // 1024 chunks = 16 KiB per tile
constexpr int VT = 32;                           // keys per transposed value tile

__device__ __forceinline__ float bf_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even), low half first.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(unsigned, v);
}

// Two floats -> two fp16 (round to nearest even), low half first.
__device__ __forceinline__ unsigned pack_f16x2(float a, float b) {
  f16x2 v;
  v[0] = static_cast<_Float16>(a);
  v[1] = static_cast<_Float16>(b);
  return __builtin_bit_cast(unsigned, v);
}

// 8 floats times a power of two -> 8 fp16.
__device__ __forceinline__ u32x4 pack8_f16(const float (&f)[8], float mul) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_f16x2(f[2 * i] * mul, f[2 * i + 1] * mul);
  return v;
}

// Power-of-two block scale: with amax = max |x| over a block, returns
// down = 2^-e and up = 2^e such that amax * down lies in [2^14, 2^15), with
// e >= -110 so that both factors stay normal floats.  amax = 0 (or not
// finite) gives 1 and 1.
__device__ __forceinline__ void block_scale(float amax, float& down, float& up) {
  if (!(amax > 0.0f) || !__builtin_isfinite(amax)) {
    down = 1.0f;
    up = 1.0f;
    return;
  }
  int E;
  (void)frexpf(amax, &E);  // amax = f * 2^E, f in [0.5, 1)
  const int e = max(E - 15, -110);
  down = ldexpf(1.0f, -e);
  up = ldexpf(1.0f, e);
}

__device__ __forceinline__ float amax8(const float (&f)[8], float m) {
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  return m;
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(v[i]);
    f[2 * i + 1] = bf_hi(v[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// Rotate 4 consecutive pairs (dims 2*pair0 .. 2*pair0+7) in fp32.  Pair p
// turns by phi = pos[axis(p)] * omega(p); (x0, x1) -> (x0 cos - x1 sin,
// x0 sin + x1 cos).  Every caller goes through this one function, so the
// standalone RoPE and the rotation fused into the attention loads round
// identically.
__device__ __forceinline__ void rope8(float (&x)[8], int pair0, const float* s_omega, const int* s_axis,
                                      float pt, float ph, float pw) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = pair0 + i;
    const int ax = s_axis[p];
    const float ps = ax == 0 ? pt : (ax == 1 ? ph : pw);
    const float phi = ps * s_omega[p];
    float sn, cs;
    sincosf(phi, &sn, &cs);
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = fmaf(x0, cs, -(x1 * sn));
    x[2 * i + 1] = fmaf(x0, sn, x1 * cs);
  }
}

__device__ __forceinline__ void stage_rope_table(const RopeTable& tab, float* s_omega, int* s_axis) {
  if (threadIdx.x < kPairs) {
    s_omega[threadIdx.x] = tab.omega[threadIdx.x];
    s_axis[threadIdx.x] = tab.axis[threadIdx.x];
  }
}

// ---------------------------------------------------------------------------
// Standalone RoPE.  x and y may be the same buffer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_apply_kernel(const u32x4* x, u32x4* y, const float* __restrict__ pos,
                                                         int64_t n_chunks, int32_t chunks_per_token, RopeTable tab) {
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];
  stage_rope_table(tab, s_omega, s_axis);
  __syncthreads();
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
    const int64_t tok = c / chunks_per_token;
    const int pair0 = int(c % CHUNKS_PER_ROW) * 4;
    float f[8];
    unpack8(x[c], f);
    rope8(f, pair0, s_omega, s_axis, pos[3 * tok], pos[3 * tok + 1], pos[3 * tok + 2]);
    y[c] = pack8(f);
  }
}

// Row of the packed workspace where segment s's first key lives.
__device__ __forceinline__ int64_t packed_start(int32_t seg_begin, int32_t s) {
  return int64_t(BK) * ((int64_t(seg_begin) + BK - 1) / BK + s);
}

// ---------------------------------------------------------------------------
// K/V prologue.  grid = (key tiles of the longest segment, segments, heads).
// k_ws: [H][rows][128] rotated keys as fp16, each 64-key tile scaled by a
//       power of two (rows past a segment's end are zero).
// k_scale: [H][rows/64] the factor that undoes each tile's scaling.
// v_ws: [H][rows/32][128][32] transposed 32-key value tiles; inside each 16-key
//       group the 4-key runs are stored in the order 0, 2, 1, 3.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_prologue_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                          const int32_t* __restrict__ cu,
                                                          const float* __restrict__ pos, int32_t n_heads,
                                                          RopeTable tab, u32x4* __restrict__ k_ws,
                                                          u32x2* __restrict__ v_ws, float* __restrict__ k_scale,
                                                          int64_t rows_per_head) {
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];
  __shared__ float s_red[4];
  const int tile = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t seg_a = cu[s];
  const int32_t S = cu[s + 1] - seg_a;
  if (tile * BK >= S) return;  // whole block leaves together
  stage_rope_table(tab, s_omega, s_axis);
  __syncthreads();
  const int tid = threadIdx.x;
  const int64_t prow = packed_start(seg_a, s) + int64_t(tile) * BK;  // packed row of this tile's key 0

  // Keys: 1024 chunks, 4 per thread; chunk c is row c / 16, dims 8 * (c % 16) ..
  // Rotate in fp32, find the tile's largest magnitude, then store fp16 scaled
  // by the tile's power-of-two factor (and the factor itself).
  float kf[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 4, cc = c & 15;
    const int key = tile * BK + r;
    if (key < S) {
      const int64_t tok = int64_t(seg_a) + key;
      unpack8(k[(tok * n_heads + h) * CHUNKS_PER_ROW + cc], kf[i]);
      rope8(kf[i], cc * 4, s_omega, s_axis, pos[3 * tok], pos[3 * tok + 1], pos[3 * tok + 2]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[i][e] = 0.0f;
    }
    amax = amax8(kf[i], amax);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float down, up;
  block_scale(amax, down, up);
  if (tid == 0) k_scale[int64_t(h) * (rows_per_head / BK) + prow / BK] = up;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    k_ws[(int64_t(h) * rows_per_head + prow + (c >> 4)) * CHUNKS_PER_ROW + (c & 15)] = pack8_f16(kf[i], down);
  }

  // Values: thread owns keys 4*k4 .. 4*k4+3 and dims 8*dc .. 8*dc+7.
  {
    const int k4 = tid & 15, dc = tid >> 4;
    unsigned w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = tile * BK + 4 * k4 + i;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (key < S) val = v[((int64_t(seg_a) + key) * n_heads + h) * CHUNKS_PER_ROW + dc];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[i][j] = val[j];
    }
    // 32-key value tile this run falls in, and the stored position of the
    // 4-key run inside its 16-key group
    const int half = k4 >> 3, run = k4 & 3;
    const int kpos = 16 * ((k4 & 7) >> 2) + 4 * (((run & 1) << 1) | (run >> 1));
    u32x2* vt = v_ws + (int64_t(h) * (rows_per_head / VT) + prow / VT + half) * (D * VT / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // dims 8*dc + 2j (low halves) and 8*dc + 2j + 1 (high halves)
      u32x2 lo, hi;
      lo[0] = (w[0][j] & 0xffffu) | (w[1][j] << 16);
      lo[1] = (w[2][j] & 0xffffu) | (w[3][j] << 16);
      hi[0] = (w[0][j] >> 16) | (w[1][j] & 0xffff0000u);
      hi[1] = (w[2][j] >> 16) | (w[3][j] & 0xffff0000u);
      const int d = 8 * dc + 2 * j;
      vt[(d * VT + kpos) / 4] = lo;
      vt[((d + 1) * VT + kpos) / 4] = hi;
    }
  }
}

// Max / sum with the partner lane (L ^ 32) that holds the other 16 keys.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Attention forward.  Eight waves per workgroup, one 32-row query block per
// wave; BQ = 256 query rows per workgroup.
// grid = (query tiles of the longest segment, segments, heads).
//
// Ping-pong schedule.  Waves 0-3 (group A) and waves 4-7 (group B) land one
// of each on every SIMD and work through the same 64-key tiles half a phase
// apart.  Between two barriers, for tile t:
//   group A:  S(t) = K(t) Q^T  |  softmax(t)    |  O += V(t) P(t)
//   group B:  softmax(t-1)     |  O += V(t-1) P(t-1)  |  S(t) = K(t) Q^T
// so while one wave of a SIMD runs its softmax (VALU) the other issues MFMAs.
// Each wave's own code stays in plain order; the overlap comes from the two
// waves.  Group B finishes its last tile after the loop.
//
// LDS: a ring of two key tiles (16 KiB each) and three value tiles (group B
// reads value tile t-1 while tile t+1 is being filled), filled by direct
// global->LDS loads one tile ahead.  Rows are not padded; 16-byte chunks are
// XOR-swizzled so that every fragment read (16 lanes on 16 different rows,
// same logical chunk) touches each bank once:
//   key tile         64 rows x 16 chunks: chunk c of row r at r*256 + 16*(c ^ (r & 15))
//   value sub-tile  128 rows x  4 chunks: chunk c of row d at d*64 + 16*(c ^ ((d >> 2) & 3))
// (a 64-key value tile is two 32-key sub-tiles, as in the workspace).
// ---------------------------------------------------------------------------
constexpr int KT_BYTES = BK * D * 2;    // 16 KiB key tile
constexpr int VT_BYTES = BK * D * 2;    // 16 KiB value tile (two sub-tiles of 8 KiB)
constexpr int KSLOTS = 2, VSLOTS = 3;
constexpr float RESCALE_SLACK = 8.0f;  // base-2 logit units the running max may lag behind

__device__ __forceinline__ int k_lds_offset(int r, int c) { return r * 256 + 16 * (c ^ (r & 15)); }
__device__ __forceinline__ int v_lds_offset(int d, int c) { return d * 64 + 16 * (c ^ ((d >> 2) & 3)); }

typedef __attribute__((address_space(3))) void lds_void;

constexpr int ATTN_NW = 8;
constexpr int ATTN_BQ = 32 * ATTN_NW;
constexpr size_t ATTN_SMEM = KSLOTS * KT_BYTES + VSLOTS * VT_BYTES;

__global__ __launch_bounds__(ATTN_NW * 64, 1) void attn_fwd_kernel(
    const u32x4* __restrict__ q, const int32_t* __restrict__ cu, const float* __restrict__ pos,
    u32x2* __restrict__ out, float* __restrict__ lse, int32_t n_tokens, int32_t n_heads, float scale_log2,
    RopeTable tab, const u32x4* __restrict__ k_ws, const u32x4* __restrict__ v_ws, const float* __restrict__ k_scale,
    int64_t rows_per_head) {
  constexpr int NW = ATTN_NW;
  constexpr int NT = NW * 64;
  constexpr int BQ = ATTN_BQ;
  constexpr int LOADS = TILE_CHUNKS / NT;  // direct-load instructions per wave per tile and tensor
  static_assert(TILE_CHUNKS % NT == 0, "tile must split evenly over the workgroup");

  extern __shared__ __attribute__((aligned(16))) char smem[];  // key slots, then value slots
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];

  const int qt = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t seg_a = cu[s];
  const int32_t S = cu[s + 1] - seg_a;
  if (qt * BQ >= S) return;  // whole block leaves together

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  stage_rope_table(tab, s_omega, s_axis);

  const int n_kt = (S + BK - 1) / BK;
  const int64_t prow = packed_start(seg_a, s);
  const u32x4* kg = k_ws + (int64_t(h) * rows_per_head + prow) * CHUNKS_PER_ROW;
  const u32x4* vg = v_ws + (int64_t(h) * rows_per_head + prow) * CHUNKS_PER_ROW;
  const float* ksc = k_scale + int64_t(h) * (rows_per_head / BK) + prow / BK;

  // Lane L of load instruction i fills LDS chunk p = (i*NW + wave)*64 + L of
  // the tile, so it fetches the logical chunk the swizzle puts there.
  auto load_tiles = [&](int t) {
    const u32x4* ksrc = kg + int64_t(t) * TILE_CHUNKS;
    const u32x4* vsrc = vg + int64_t(t) * TILE_CHUNKS;
    char* kdst = smem + (t % KSLOTS) * KT_BYTES;
    char* vdst = smem + KSLOTS * KT_BYTES + (t % VSLOTS) * VT_BYTES;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = (i * NW + wave) * 64 + lane;
      const int r = p >> 4, c = (p & 15) ^ (r & 15);
      __builtin_amdgcn_global_load_lds(ksrc + r * CHUNKS_PER_ROW + c, (lds_void*)(kdst + (i * NW + wave) * 1024), 16,
                                       0, 0);
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = (i * NW + wave) * 64 + lane;
      const int sub = p >> 9, qq = p & 511;
      const int d = qq >> 2, c = (qq & 3) ^ ((d >> 2) & 3);
      __builtin_amdgcn_global_load_lds(vsrc + sub * 512 + d * 4 + c, (lds_void*)(vdst + (i * NW + wave) * 1024), 16,
                                       0, 0);
    }
  };

  load_tiles(0);  // first tile loads while the queries are rotated
  __syncthreads();  // rope table staged

  // Queries: B operand of S^T = K Q^T.  Lane holds query row l32 of its block
  // and dims 16*ks + 8*g .. +7, rotated in fp32, scaled by the row's
  // power-of-two factor and rounded to fp16; cq folds the undoing factor into
  // the base-2 logit coefficient.
  f16x8 qf[8];
  float cq;
  const int qrow = qt * BQ + wave * 32 + l32;
  {
    float f[8][8];
    if (qrow < S) {
      const int64_t tok = int64_t(seg_a) + qrow;
      const float pt = pos[3 * tok], ph = pos[3 * tok + 1], pw = pos[3 * tok + 2];
      const u32x4* qp = q + (tok * n_heads + h) * CHUNKS_PER_ROW;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        unpack8(qp[2 * ks + g], f[ks]);
        rope8(f[ks], ks * 8 + g * 4, s_omega, s_axis, pt, ph, pw);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[ks][e] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) amax = amax8(f[ks], amax);
    amax = pair_max(amax);  // the row's other 64 dims sit in lane L ^ 32
    float down, up;
    block_scale(amax, down, up);
    cq = scale_log2 * up;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(f16x8, pack8_f16(f[ks], down));
  }

  // Per-lane fragment offsets within a slot (the sub-block / value-dim
  // block / sub-tile parts are immediate offsets on top).
  int koff[8], voff[2];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = k_lds_offset(l32, 2 * ks + g);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) voff[hh] = KSLOTS * KT_BYTES + v_lds_offset(l32, 2 * hh + g);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  f32x16 sc[2];       // S^T of one 64-key tile (two 32-key sub-blocks)
  bf16x8 pf[2][2];    // its probabilities, [sub-block][key half]

  // Fragment prefetch: LDS reads take longer than an MFMA, so each chain's
  // operands are read eight ahead and a register is refilled as soon as its
  // MFMA has been issued.
  bf16x8 fr[8];
  auto k_frag = [&](const char* kb, int sb, int ks) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kb + sb * 32 * 256 + koff[ks]));
  };
  auto v_frag = [&](const char* vb, int sb, int hh, int db) {
    return *reinterpret_cast<const bf16x8*>(vb + sb * (VT_BYTES / 2) + db * 32 * 64 + voff[hh]);
  };
  // S^T for tile t: 2 sub-blocks x 8 MFMAs over the head dim.
  auto qk = [&](int t) {
    const char* kb = smem + (t % KSLOTS) * KT_BYTES;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) fr[ks] = k_frag(kb, 0, ks);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[sb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fr[ks]), qf[ks], sc[sb], 0, 0, 0);
        if (sb == 0) fr[ks] = k_frag(kb, 1, ks);
      }
    }
  };
  // First eight value fragments of tile t (sub-block 0), read ahead of the
  // softmax so they arrive while it runs.
  auto pv_prefetch = [&](int t) {
    const char* vb = smem + (t % VSLOTS) * VT_BYTES;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < 4; ++db) fr[4 * hh + db] = v_frag(vb, 0, hh, db);
  };
  // O^T += V^T P^T for tile t (after pv_prefetch): 2 sub-blocks x 2 key
  // halves x 4 value-dim blocks.
  auto pv = [&](int t) {
    const char* vb = smem + (t % VSLOTS) * VT_BYTES;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[4 * hh + db], pf[sb][hh], o[db], 0, 0, 0);
          if (sb == 0) fr[4 * hh + db] = v_frag(vb, 1, hh, db);
        }
  };
  // Online softmax of tile t (its scores in sc): mask the segment tail on the
  // last tile, find the tile max, move the running max if needed, then form
  // the bf16 probabilities and add their row sums to l.
  //
  // The running max m only moves when a tile's max exceeds it by more than
  // RESCALE_SLACK; until then probabilities are exp2(t - m) <= 2^RESCALE_SLACK,
  // which bf16 and fp32 hold without loss, and O and l need no rescaling.
  // Exact either way: the final normalisation divides by an l built with the
  // same m.  Every PV product issued so far used the old m, so rescaling O
  // here keeps it consistent.
  auto softmax = [&](int t) {
    if (t == n_kt - 1 && (S % BK) != 0) {
      const int kbase = t * BK;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3) >= S) sc[sb][r] = -INFINITY;
    }
    // c turns a raw score of this tile into a base-2 logit (softmax scale,
    // log2 e and both block scales).
    const float c = cq * ksc[t];
    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    const float tmax = pair_max(mx) * c;
    const bool grow = tmax > m + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform; rare after the first tile
      const float m_new = grow ? tmax : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 1 where m stays, 0 from -inf
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    float rs = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[sb][8 * hh + 2 * i], c, -m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[sb][8 * hh + 2 * i + 1], c, -m));
          w[i] = pack_bf16x2(p0, p1);
          rs += p0 + p1;
        }
        pf[sb][hh] = __builtin_bit_cast(bf16x8, w);
      }
    l += rs;
  };

  __syncthreads();  // tile 0 has landed
  const bool group_b = wave >= NW / 2;
  if (!group_b) {
    for (int t = 0; t < n_kt; ++t) {
      if (t + 1 < n_kt) load_tiles(t + 1);
      qk(t);
      pv_prefetch(t);
      softmax(t);
      pv(t);
      __syncthreads();  // tile t+1 has landed; reads of the slots refilled next are done
    }
  } else {
    for (int t = 0; t < n_kt; ++t) {
      if (t + 1 < n_kt) load_tiles(t + 1);
      if (t > 0) {
        pv_prefetch(t - 1);
        softmax(t - 1);
        pv(t - 1);
      }
      qk(t);
      __syncthreads();
    }
    pv_prefetch(n_kt - 1);
    softmax(n_kt - 1);
    pv(n_kt - 1);
  }

  // Epilogue: O = O / l, lse = (m + log2 l) * ln 2.
  const float lt = pair_sum(l);
  const float inv = 1.0f / lt;
  if (qrow < S) {
    const int64_t tok = int64_t(seg_a) + qrow;
    u32x2* orow = out + (tok * n_heads + h) * (D / 4);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][4 * k4] * inv, o[db][4 * k4 + 1] * inv);
        w[1] = pack_bf16x2(o[db][4 * k4 + 2] * inv, o[db][4 * k4 + 3] * inv);
        orow[db * 8 + 2 * k4 + g] = w;
      }
    if (g == 0) lse[int64_t(h) * n_tokens + tok] = (m + log2f(lt)) * 0.69314718055994531f;
  }
}

}  // namespace

const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

int launch_rope_apply(const void* x, void* y, const float* pos, int64_t n_tokens, int32_t n_heads,
                      const RopeTable& table, void* stream) {
  const int64_t n_chunks = n_tokens * n_heads * CHUNKS_PER_ROW;
  int64_t blocks = (n_chunks + 255) / 256;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
  hipLaunchKernelGGL(rope_apply_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(x), static_cast<u32x4*>(y), pos, n_chunks,
                     int32_t(n_heads * CHUNKS_PER_ROW), table);
  return int(hipGetLastError());
}

int launch_kv_prologue(const void* k, const void* v, const int32_t* cu, const float* pos, int64_t /*n_tokens*/,
                       int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, const RopeTable& table, void* k_ws,
                       void* v_ws, float* k_scale, int64_t rows_per_head, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + BK - 1) / BK);
  if (tiles == 0) return 0;
  hipLaunchKernelGGL(kv_prologue_kernel, dim3(tiles, unsigned(n_seqs), unsigned(n_heads)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), cu,
                     pos, n_heads, table, static_cast<u32x4*>(k_ws), static_cast<u32x2*>(v_ws), k_scale,
                     rows_per_head);
  return int(hipGetLastError());
}

int launch_attention(const void* q, const int32_t* cu, const float* pos, void* out, float* lse, int64_t n_tokens,
                     int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, float scale, const RopeTable& table,
                     const void* k_ws, const void* v_ws, const float* k_scale, int64_t rows_per_head, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + ATTN_BQ - 1) / ATTN_BQ);
  if (tiles == 0) return 0;
  // The dynamic LDS limit is raised once per device.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  static std::atomic<uint64_t> attr_set{0};
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit == 0 || (attr_set.load(std::memory_order_acquire) & bit) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(ATTN_SMEM));
    if (e != hipSuccess) return int(e);
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(tiles, unsigned(n_seqs), unsigned(n_heads)),
                     dim3(ATTN_NW * 64), ATTN_SMEM, static_cast<hipStream_t>(stream), static_cast<const u32x4*>(q), cu,
                     pos, static_cast<u32x2*>(out), lse, int32_t(n_tokens), n_heads, scale_log2, table,
                     static_cast<const u32x4*>(k_ws), static_cast<const u32x4*>(v_ws), k_scale, rows_per_head);
  return int(hipGetLastError());
}

}  // namespace h3attn
