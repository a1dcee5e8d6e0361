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
//   rope_apply_kernel   y = rope(x): one 16-byte chunk position (8 dims) per
//                       thread, applied to every head of the token.
//   kv_prologue_kernel  rotates K once per call and packs it, with V
//                       transposed, into 64-key tiles that start on a 64-key
//                       boundary for every segment.  HBM-bound.
//   attn_fwd_kernel     one workgroup per (256-query tile, head, segment
//                       rank), longest segments first (the prologue ranks
//                       them).  It rotates its queries while loading them, then
//                       streams the segment's 32-key tiles through LDS and
//                       runs an online softmax between two MFMA contractions,
//                       software-pipelined inside each wave.
//
// MFMA orientation.  The score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims (from LDS), B = 16 dims x
// 32 queries (held in registers for the whole kernel).  In the 32x32
// accumulator, lane L owns query column L % 32 and the 16 key rows
// 8*(r/4) + 4*(L/32) + r%4, r = 0..15; the other 16 keys of that query sit in
// lane L ^ 32.  So a row maximum or row sum is an in-lane reduction plus one
// v_permlane32_swap.  The probabilities then serve directly as the B operand
// of O^T += V^T P^T (keys are the contraction index), with no data movement:
// registers 8*hh .. 8*hh+7 of a 32-key tile hold 8 keys of one 16-key group.
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

#include <atomic>
#include <cmath>
#include <mutex>

#include "device_common.h"

namespace h3attn {
namespace {

using namespace dev;

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

constexpr int BK = kKeyTile;  // keys per packed workspace tile
constexpr int VT = 32;        // keys per transposed value tile

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

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// ---------------------------------------------------------------------------
// Standalone RoPE.  x and y may be the same buffer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_apply_kernel(const u32x4* x, u32x4* y, const float* __restrict__ pos,
                                                         int64_t n_tokens, int32_t n_heads, RopeTable tab) {
  // Thread (token, c): chunk c (dims 8c .. 8c+7) of every head of the token.
  // The four angles are computed once and applied to all heads.
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];
  stage_rope_table(tab, s_omega, s_axis);
  __syncthreads();
  const int64_t n_items = n_tokens * CHUNKS_PER_ROW;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t it = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; it < n_items; it += stride) {
    const int64_t tok = it / CHUNKS_PER_ROW;
    const int c = int(it % CHUNKS_PER_ROW);
    const float pt = pos[3 * tok], ph = pos[3 * tok + 1], pw = pos[3 * tok + 2];
    const int64_t base = tok * n_heads * CHUNKS_PER_ROW + c;
    // At the origin every angle is +0, whose sine and cosine are exactly +0
    // and 1: that Rot4 is written out instead of computed, bit for bit the same.
    Rot4 r;
    if (at_origin(pt, ph, pw)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) r.sn[i] = 0.0f, r.cs[i] = 1.0f;
    } else {
      r = rope_angles4(c * 4, s_omega, s_axis, pt, ph, pw);
    }
    int h = 0;
    for (; h + 4 <= n_heads; h += 4) {  // four loads in flight before any use
      u32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = x[base + int64_t(h + j) * CHUNKS_PER_ROW];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f[8];
        unpack8(v[j], f);
        rope_turn4(f, r);
        y[base + int64_t(h + j) * CHUNKS_PER_ROW] = pack8(f);
      }
    }
    for (; h < n_heads; ++h) {
      float f[8];
      unpack8(x[base + int64_t(h) * CHUNKS_PER_ROW], f);
      rope_turn4(f, r);
      y[base + int64_t(h) * CHUNKS_PER_ROW] = pack8(f);
    }
  }
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
                                                          int32_t* __restrict__ order, int64_t rows_per_head,
                                                          int32_t max_seqlen) {
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];
  __shared__ float s_red[4];
  const int tile = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  if (tile == 0 && h == 0) write_segment_rank(cu, int(gridDim.y), s, order);  // before any early exit
  const int32_t seg_a = cu[s];
  const int32_t S = min(cu[s + 1] - seg_a, max_seqlen);  // a longer segment counts as its first max_seqlen tokens
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

// ---------------------------------------------------------------------------
// Attention forward, software-pipelined inside each wave.
//
// Eight waves per workgroup, two per SIMD, one 32-row query block per wave:
// BQ = 256 query rows per workgroup.  Keys arrive in 32-key tiles.  Iteration
// t of the main loop issues, in one branch-free block of 16 slots,
//     S(t+1) = K(t+1) Q^T     8 MFMAs (f16)
//     O     += V(t-1) P(t-1)  8 MFMAs (bf16)
// and, between them, the exponentials of tile t, so that the matrix core and
// the vector ALU of the SIMD work at the same time (and the second wave of
// the SIMD fills what one wave leaves idle).
//
// Online softmax in base 2 with a lazily moved running max m: the
// probabilities of tile t are formed as exp2(s*c - m) with the current m.
// A lane whose row sum for the tile exceeds 2^LAZY_LOG2 (or is not finite,
// as on the first tile where m = -inf) sends the wave down a rare path that
// takes the exact tile max, moves m, rescales l and O and recomputes the
// tile's probabilities.  Until then every probability is at most
// 2^LAZY_LOG2, well inside bf16 and fp32 range, and nothing is rescaled.
// The result is exact softmax either way: O and l always share one m.
//
// LDS: rings of eight key slots and eight value slots of 8 KiB.  Iteration t
// reads K(t+1) and V(t-1) and issues direct buffer->LDS loads of K(t+5) and
// V(t+3), four iterations ahead.  Iterations pair up into epochs that end
// with one barrier, which waits only for loads issued before the epoch.  The
// loop is unrolled by eight so that every slot offset is an immediate.
// (Buffer rather than global loads: the compiler counts a global->LDS load
// as touching both memory counters and would then wait for every LDS read in
// full while one is in flight.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int k_lds_offset(int r, int c) { return r * 256 + 16 * (c ^ (r & 15)); }
__device__ __forceinline__ int v_lds_offset(int d, int c) { return d * 64 + 16 * (c ^ ((d >> 2) & 3)); }

constexpr int PK = 32;                              // keys per tile
constexpr int P_NW = 8;                             // waves per workgroup
constexpr int ATTN_BQ = 32 * P_NW;                  // 256 query rows per workgroup
constexpr int P_TILE_BYTES = PK * D * 2;            // 8 KiB
constexpr int P_TILE_CHUNKS = PK * CHUNKS_PER_ROW;  // 512 16-byte chunks
constexpr int P_NS = 8;                             // slots per ring
constexpr int P_VBASE = P_NS * P_TILE_BYTES;        // value ring after the key ring
constexpr size_t ATTN_SMEM = 2 * P_NS * P_TILE_BYTES;  // 128 KiB
constexpr float LAZY_LOG2 = 16.0f;                  // log2 of the largest row sum left unrescaled

__global__ __launch_bounds__(P_NW * 64, 1) void attn_fwd_kernel(
    const u32x4* __restrict__ q, const int32_t* __restrict__ cu, const float* __restrict__ pos,
    u32x2* __restrict__ out, float* __restrict__ lse, int32_t n_tokens, int32_t n_heads, float scale_log2,
    RopeTable tab, const u32x4* __restrict__ k_ws, const u32x4* __restrict__ v_ws, const float* __restrict__ k_scale,
    const int32_t* __restrict__ order, int64_t rows_per_head, int32_t max_seqlen) {
  static_assert(P_TILE_CHUNKS == P_NW * 64, "one direct load per wave, tile and tensor");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];

  // The segment comes from the rank order the K/V prologue wrote.
  const int qt = blockIdx.x, h = blockIdx.y;
  const int s = gridDim.z == 1 ? 0 : order[blockIdx.z];
  const int32_t seg_a = cu[s];
  const int32_t S = min(cu[s + 1] - seg_a, max_seqlen);  // a longer segment counts as its first max_seqlen tokens
  if (qt * ATTN_BQ >= S) return;  // whole block leaves together

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  stage_rope_table(tab, s_omega, s_axis);

  const int n_kt = (S + PK - 1) / PK;
  const int last_t = n_kt - 1;
  const bool ragged = (S % PK) != 0;
  const int64_t prow = packed_start(seg_a, s);
  const char* kg = reinterpret_cast<const char*>(k_ws + (int64_t(h) * rows_per_head + prow) * CHUNKS_PER_ROW);
  const char* vg = reinterpret_cast<const char*>(v_ws + (int64_t(h) * rows_per_head + prow) * CHUNKS_PER_ROW);
  const float* ksc = k_scale + int64_t(h) * (rows_per_head / 64) + prow / 64;  // one factor per 64 keys

  // Direct loads: lane L of wave w fills LDS chunk p = 64*w + L of a slot, so
  // it fetches the logical chunk that the swizzle puts there.  The per-lane
  // source offsets are the same for every tile.
  unsigned ksrc_off, vsrc_off;
  {
    const int p = wave * 64 + lane;
    const int r = p >> 4, c = (p & 15) ^ (r & 15);
    ksrc_off = unsigned(r * CHUNKS_PER_ROW + c) * 16u;
    const int d = p >> 2, cv = (p & 3) ^ ((d >> 2) & 3);
    vsrc_off = unsigned(d * 4 + cv) * 16u;
  }
  // Buffer resources over this head's segment of the key and value planes
  // (tiles 0 .. n_kt-1); loads past the end read zeros.
  const int seg_bytes = n_kt * P_TILE_BYTES;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, seg_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, seg_bytes, 0x00020000);
  auto load_k = [&](int t, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(smem + slot * P_TILE_BYTES + wave * 1024), 16, ksrc_off,
                                             t * P_TILE_BYTES, 0, 0);
  };
  auto load_v = [&](int t, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(smem + P_VBASE + slot * P_TILE_BYTES + wave * 1024), 16,
                                             vsrc_off, t * P_TILE_BYTES, 0, 0);
  };

  load_k(0, ic<0>());
  load_k(min(1, last_t), ic<1>());
  __syncthreads();  // rope table staged; K(0) and K(1) have landed
  // The loads iterations -2 and -1 would have issued, in the same order.
  load_k(min(2, last_t), ic<2>());
  load_v(0, ic<0>());
  load_k(min(3, last_t), ic<3>());
  load_v(min(1, last_t), ic<1>());
  load_k(min(4, last_t), ic<4>());
  load_v(min(2, last_t), ic<2>());

  // Queries: B operand of S^T = K Q^T.  The lane holds query row l32 and dims
  // 16*ks + 8*g .. +7, rotated in fp32, scaled by the row's power-of-two
  // factor and rounded to fp16; cq folds the undoing factor into the base-2
  // logit coefficient.
  const int qrow = qt * ATTN_BQ + wave * 32 + l32;
  f16x8 qf[8];
  float cq;
  {
    float f[8][8];
    if (qrow < S) {
      const int64_t tok = int64_t(seg_a) + qrow;
      const float pt = pos[3 * tok], ph = pos[3 * tok + 1], pw = pos[3 * tok + 2];
      const u32x4* qp = q + (tok * n_heads + h) * CHUNKS_PER_ROW;
      // The test reads only the positions, so a turning wave computes its
      // angles while the query chunks are still in flight.
      if (wave_at_origin(pt, ph, pw)) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) unpack8(qp[2 * ks + g], f[ks]);
      } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          unpack8(qp[2 * ks + g], f[ks]);
          rope_turn4(f[ks], rope_angles4(ks * 8 + g * 4, s_omega, s_axis, pt, ph, pw));
        }
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

  // Per-lane fragment offsets inside a slot; slot and sub-block parts are
  // immediates.
  int koff[8], voff[2];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = k_lds_offset(l32, 2 * ks + g);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) voff[hh] = v_lds_offset(l32, 2 * hh + g);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  float ct = cq * ksc[0];   // base-2 logit coefficient of the tile whose exponentials come next
  f32x16 sc[2];             // S^T of one tile, double-buffered by tile parity
  bf16x8 pf[2][2];          // its probabilities, [buffer][key half]

  auto kfrag = [&](auto SLOT, int ks) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    return *reinterpret_cast<const u32x4*>(smem + slot * P_TILE_BYTES + koff[ks]);
  };
  auto vfrag = [&](auto SLOT, int f) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    return *reinterpret_cast<const bf16x8*>(smem + P_VBASE + slot * P_TILE_BYTES + (f & 3) * 32 * 64 + voff[f >> 2]);
  };
  auto mfma_qk = [&](f32x16 acc, u32x4 kf, int ks) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf), qf[ks], acc, 0, 0, 0);
  };

  // S^T(t) into buffer B, alone (pipeline fill).
  auto qk_alone = [&](auto B, auto SLOT) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma_qk(acc, kfrag(SLOT, ks), ks);
    sc[b] = acc;
  };
  // O^T += V^T(t) P^T(t) from buffer B, alone (pipeline drain).
  auto pv_alone = [&](auto B, auto SLOT) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int f = 0; f < 8; ++f)
      o[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(SLOT, f), pf[b][f >> 2], o[f & 3], 0, 0, 0);
  };
  // Keys of tile t at or past the segment end get score -inf.
  auto mask_tail = [&](auto B, int t) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const int kbase = t * PK;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kbase + 8 * (r >> 2) + 4 * g + (r & 3) >= S) sc[b][r] = -INFINITY;
  };
  // Probabilities of the scores in buffer B at the current m, in units u of
  // two (registers 2u and 2u+1, key half u >> 2), each split in two halves:
  // the exponentials, then the bf16 packing and the row-sum update.
  auto exp_half_a = [&](auto B, int u, float& p0, float& p1) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    p0 = __builtin_amdgcn_exp2f(fmaf(sc[b][2 * u], ct, -m));
    p1 = __builtin_amdgcn_exp2f(fmaf(sc[b][2 * u + 1], ct, -m));
    pin(p0);
    pin(p1);
  };
  auto exp_half_b = [&](int u, float p0, float p1, u32x4 (&pw)[2], float& rs) __attribute__((always_inline)) {
    unsigned w = pack_bf16x2(p0, p1);
    float r = u == 0 ? p0 + p1 : rs + (p0 + p1);
    pin(w);
    pin(r);
    pw[u >> 2][u & 3] = w;
    rs = r;
  };
  // After the exponentials of tile t (scores in buffer B, products of tile
  // t-1 issued): the rare path that moves m, then the row sums and the
  // probabilities for the next products.
  auto settle = [&](auto B, u32x4 (&pw)[2], float rs) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const bool over = !(rs <= exp2f(LAZY_LOG2));  // also true for inf and NaN
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      float mx = sc[b][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[b][r]);
      const float tmax = pair_max(mx) * ct;
      const float m_new = fmaxf(m, tmax);
      const float a = __builtin_amdgcn_exp2f(m - m_new);  // 0 from m = -inf
      m = m_new;
      l *= a;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= a;
      rs = 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[b][2 * u], ct, -m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[b][2 * u + 1], ct, -m));
        pw[u >> 2][u & 3] = pack_bf16x2(p0, p1);
        rs += p0 + p1;
      }
    }
    l += rs;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) pf[b][hh] = __builtin_bit_cast(bf16x8, pw[hh]);
  };

  // The main block of iteration t for T4 = t mod 4 (S(t) in sc[t & 1]):
  // 16 issue slots.  Slots 0..7 issue the S(t+1) MFMAs (when QK) as one
  // accumulation chain, slots 8..15 the O += V(t-1) P(t-1) MFMAs (when PV)
  // with the four of each key half back to back, so that consecutive MFMAs
  // share an operand or an accumulator (less switching, less energy on a
  // power-limited chip).  The first half of an exponential unit follows every
  // even slot and its second half every odd slot; fragment reads run two to
  // four slots ahead.  A scheduling fence after every slot keeps this order.
  auto region = [&](auto T4, auto QK, auto PV, u32x4 (&pw)[2], float& rs) __attribute__((always_inline)) {
    constexpr int t4 = decltype(T4)::value;
    constexpr int b = t4 & 1;
    constexpr bool do_qk = decltype(QK)::value != 0;
    constexpr bool do_pv = decltype(PV)::value != 0;
    constexpr ic<(t4 + 1) & 7> kslot{};  // K(t+1)
    constexpr ic<(t4 + 7) & 7> vslot{};  // V(t-1)
    u32x4 kf[8];
    bf16x8 vf[8];
    float ep0 = 0.0f, ep1 = 0.0f;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    // Value MFMA k (k = 0..7) uses key half k >> 2 and value-dim block k & 3.
    if (do_qk) {
      kf[0] = kfrag(kslot, 0);
      kf[1] = kfrag(kslot, 1);
    }
    if (do_pv) {
#pragma unroll
      for (int k = 0; k < 4; ++k) vf[k] = vfrag(vslot, k);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = j >> 1;
      if (j < 8) {
        if (do_qk) {
          acc = mfma_qk(acc, kf[j], j);
          if (j + 2 < 8) kf[j + 2] = kfrag(kslot, j + 2);
        }
        if (do_pv && j >= 4) vf[j] = vfrag(vslot, j);
      } else if (do_pv) {
        const int k = j - 8, hh = k >> 2, db = k & 3;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[k], pf[1 - b][hh], o[db], 0, 0, 0);
      }
      if ((j & 1) == 0)
        exp_half_a(ic<b>(), i, ep0, ep1);
      else
        exp_half_b(i, ep0, ep1, pw, rs);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (do_qk) sc[1 - b] = acc;
  };

  // Steady iteration t (1 <= t <= last_t - 1), T8 = t mod 8.  Loads K(t+5)
  // and V(t+3).  Iterations pair up into epochs (t odd, t+1) that end with
  // one barrier: within an epoch no slot that is read is also written, and
  // everything an epoch reads was issued at least two epochs earlier.  Past
  // the last tile the index is clamped: the duplicate goes to a slot that is
  // not read again, and every iteration keeps issuing the same loads, which
  // the ring barrier counts.
  auto step = [&](auto T8, int t) __attribute__((always_inline)) {
    constexpr int t8 = decltype(T8)::value;
    u32x4 pw[2];
    float rs;
    region(T8, ic<1>(), ic<1>(), pw, rs);
    load_k(min(t + 5, last_t), ic<(t8 + 5) & 7>());
    load_v(min(t + 3, last_t), ic<(t8 + 3) & 7>());
    settle(ic<t8 & 1>(), pw, rs);
    ct = cq * ksc[(t + 1) >> 1];
    if ((t8 & 1) == 0) ring_barrier<4>();  // end of an epoch: its loads may stay in flight
  };
  // Last iteration t = last_t >= 1: exponentials of tile t and products of
  // tile t-1, then the products of tile t.
  auto last = [&](auto T8) __attribute__((always_inline)) {
    constexpr int t8 = decltype(T8)::value;
    if (ragged) mask_tail(ic<t8 & 1>(), last_t);
    u32x4 pw[2];
    float rs;
    region(T8, ic<0>(), ic<1>(), pw, rs);
    settle(ic<t8 & 1>(), pw, rs);
    ring_barrier<0>();  // V(t) has landed
    pv_alone(ic<t8 & 1>(), ic<t8>());
  };
  qk_alone(ic<0>(), ic<0>());
  if (n_kt == 1) {
    if (ragged) mask_tail(ic<0>(), 0);
    u32x4 pw[2];
    float rs;
    region(ic<0>(), ic<0>(), ic<0>(), pw, rs);
    settle(ic<0>(), pw, rs);
    ring_barrier<0>();
    pv_alone(ic<0>(), ic<0>());
  } else {
    ring_barrier<6>();  // every wave is done with K(0) before its slot is refilled
    {
      // t = 0: no products of an earlier tile yet; an epoch of its own.
      u32x4 pw[2];
      float rs;
      region(ic<0>(), ic<1>(), ic<0>(), pw, rs);
      load_k(min(5, last_t), ic<5>());
      load_v(min(3, last_t), ic<3>());
      settle(ic<0>(), pw, rs);
      ct = cq * ksc[1 >> 1];
      ring_barrier<4>();
    }
    int t = 1;
    for (; t + 7 <= last_t - 1; t += 8) {
      step(ic<1>(), t);
      step(ic<2>(), t + 1);
      step(ic<3>(), t + 2);
      step(ic<4>(), t + 3);
      step(ic<5>(), t + 4);
      step(ic<6>(), t + 5);
      step(ic<7>(), t + 6);
      step(ic<0>(), t + 7);
    }
    // Up to seven more steps, continuing the t mod 8 sequence 1, 2, ..., 7.
    if (t <= last_t - 1) { step(ic<1>(), t); ++t;
    if (t <= last_t - 1) { step(ic<2>(), t); ++t;
    if (t <= last_t - 1) { step(ic<3>(), t); ++t;
    if (t <= last_t - 1) { step(ic<4>(), t); ++t;
    if (t <= last_t - 1) { step(ic<5>(), t); ++t;
    if (t <= last_t - 1) { step(ic<6>(), t); ++t;
    if (t <= last_t - 1) { step(ic<7>(), t); ++t; } } } } } } }
    // The last iteration starts a new epoch when t is odd; when t is even
    // its epoch partner (t - 1) ended without a barrier, and the one in
    // last() closes it.
    switch (last_t & 7) {
      case 0: last(ic<0>()); break;
      case 1: last(ic<1>()); break;
      case 2: last(ic<2>()); break;
      case 3: last(ic<3>()); break;
      case 4: last(ic<4>()); break;
      case 5: last(ic<5>()); break;
      case 6: last(ic<6>()); break;
      default: last(ic<7>()); break;
    }
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
// Workspace of the no-allocation entry point: one array per GPU, held from the
// code object's load until the process ends.  Host code never uses this name
// as an address: it takes the device address from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

}  // namespace

const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

int noalloc_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  // The address is looked up once per device, with that device current, and kept.
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    if (p == nullptr) return int(hipErrorInvalidSymbol);
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_rope_apply(const void* x, void* y, const float* pos, int64_t n_tokens, int32_t n_heads,
                      const RopeTable& table, void* stream) {
  const int64_t n_items = n_tokens * CHUNKS_PER_ROW;
  int64_t blocks = (n_items + 255) / 256;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
  hipLaunchKernelGGL(rope_apply_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(x), static_cast<u32x4*>(y), pos, n_tokens, n_heads, table);
  return int(hipGetLastError());
}

int launch_kv_prologue(const void* k, const void* v, const int32_t* cu, const float* pos, int64_t /*n_tokens*/,
                       int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, const RopeTable& table, void* k_ws,
                       void* v_ws, float* k_scale, int32_t* order, int64_t rows_per_head, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + BK - 1) / BK);
  if (tiles == 0) return 0;
  hipLaunchKernelGGL(kv_prologue_kernel, dim3(tiles, unsigned(n_seqs), unsigned(n_heads)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), cu,
                     pos, n_heads, table, static_cast<u32x4*>(k_ws), static_cast<u32x2*>(v_ws), k_scale, order,
                     rows_per_head, max_seqlen);
  return int(hipGetLastError());
}

int launch_attention(const void* q, const int32_t* cu, const float* pos, void* out, float* lse, int64_t n_tokens,
                     int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, float scale, const RopeTable& table,
                     const void* k_ws, const void* v_ws, const float* k_scale, const int32_t* order,
                     int64_t rows_per_head, void* stream) {
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
  // Grid (query tile, head, segment rank): the longest segments go first.
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(tiles, unsigned(n_heads), unsigned(n_seqs)),
                     dim3(P_NW * 64), ATTN_SMEM, static_cast<hipStream_t>(stream), static_cast<const u32x4*>(q), cu,
                     pos, static_cast<u32x2*>(out), lse, int32_t(n_tokens), n_heads, scale_log2, table,
                     static_cast<const u32x4*>(k_ws), static_cast<const u32x4*>(v_ws), k_scale, order,
                     rows_per_head, max_seqlen);
  return int(hipGetLastError());
}

}  // namespace h3attn
