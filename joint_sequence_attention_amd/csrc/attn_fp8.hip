// HIP kernels for gfx950 (MI355X): the lossy FP8 mode of packed varlen
// attention.
//
// The mode: SAGE-style quantization of the long main DiT attention (vLLM-Omni
// "MiniMax-H3" recipe, "Attention Backends"): queries and keys in FP8 e4m3
// with one scale per query token and one scale per 16 keys, probabilities and
// values in FP8 too, and optionally Skip-Softmax tile skipping.  The
// attention itself is the one the exact path computes ("Day 0 Support for
// MiniMax-H3 on AMD Instinct GPUs", "The diffusion transformer (DiT)"): every
// token of a packed segment attends to every token of its segment, after the
// multi-axis rotation of queries and keys.
//
// What is quantized how (the page gives only the block sizes):
//   * every scale is a power of two 2^e, e the smallest integer that brings the
//     block's largest magnitude to at most 448 (the largest finite e4m3 value);
//   * Q: one block per (token, head) row of 128 rotated dims; K: 16 keys of one
//     head counted from the segment's first key; V: one scale per value
//     channel over all keys of the segment (a scale constant along the keys
//     factors out of the sum over keys); P: the same rule applied to its bound
//     1 relative to the row maximum, i.e. e4m3(256 p);
//   * the softmax scale multiplies the product of the quantized Q and K.
//
// Kernels:
//   fp8_clear_kernel        zeroes the per-channel value maxima.
//   v_amax_fp8_kernel       takes each value channel's largest magnitude over
//                           its segment: a reduction over 1024 keys per
//                           workgroup, then one atomic max per channel.
//   kv_prologue_fp8_kernel  rotates K, quantizes it in 16-key blocks and packs
//                           it into 64-key tiles.
//   v_quant_fp8_kernel      quantizes V with the channel scales and packs it,
//                           transposed, into 64-key tiles.  All HBM-bound.
//   attn_fwd_fp8_kernel     one workgroup per (256-query tile, head, segment
//                           rank), longest segments first; eight waves, 32
//                           queries per wave; 64-key tiles through LDS rings;
//                           both contractions on v_mfma_scale_f32_32x32x64_f8f6f4.
//
// MFMA orientation.  As in the bf16 kernel, scores are computed transposed,
// S^T = K Q^T: A = 32 keys x 64 dims (LDS), B = 64 dims x 32 queries
// (registers).  A 64-key tile is two 32-key subtiles u; in the accumulator of
// subtile u, lane L owns query L % 32 and keys 32u + 8(r/4) + 4(L/32) + r%4,
// r = 0..15.  Lane L's 32 probabilities of the tile (byte b = 16u + r) are the
// B operand of O^T += V^T P^T over the tile's 64 keys as they stand; the
// prologue stores each value-dim row of V^T with its keys in the matching
// order: byte 32g + b holds key 32(b/16) + 8((b%16)/4) + 4g + b%4.  The
// hardware pairs byte b of lane group g in A with byte b of lane group g in
// B, so any order works as long as both sides use the same one.
//
// Scales.  The matrix core applies every block scale as an 8-bit exponent:
// per query row the B scale of the score products (each lane carries its
// row's), per 16 keys the A scale (the scale of lanes L and L + 32 covers key
// L % 32), and per value channel the A scale of the value products (lane L of
// value-dim block db carries channel 32 db + L % 32's).  So a score MFMA
// returns q8 . k8 itself and a value MFMA sum_j p'_j v8_jd.

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>

#include "device_common.h"

namespace h3attn {
namespace {

using namespace dev;

constexpr int KT = 64;                   // keys per tile
constexpr int F8_TILE_BYTES = KT * D;    // 8 KiB: K 64 x 128 B, V^T 128 x 64 B
constexpr int F8_NW = 8;                 // waves per workgroup
constexpr int F8_BQ = 32 * F8_NW;        // 256 query rows per workgroup
constexpr int F8_NS = 8;                 // slots per ring
constexpr int F8_VBASE = F8_NS * F8_TILE_BYTES;
constexpr size_t F8_SMEM = 2 * F8_NS * F8_TILE_BYTES;  // 128 KiB
constexpr float P_SHIFT = 8.0f;          // probabilities are stored as p * 2^8, p relative to the row maximum
// A stored probability p' = 2^(z - mm) with z the base-2 logit and mm the
// running reference minus 8; it must not exceed 448 (the largest finite e4m3
// value), i.e. z - mm <= log2 448.
// The reference is moved when that could fail; 8.75 < log2 448 = 8.807 leaves
// room for the rounding of the exponent's argument.
constexpr float P_ROOM_LOG2 = 8.75f;
constexpr int E8M0_ONE = 127;            // 8-bit exponent scale of 2^0
// The dense instance moves its reference in one of two ways (see the kernel):
// early, from each tile's maximum taken before its exponentials, or late,
// after a test of the packed probabilities.  On N(0, 1)-like logits the
// reference of some row of a wave moves on about 26 % of tiles at 8K keys
// and 3 % at 130K keys; the late form is cheaper per tile and dearer per
// move, and wins from about this many keys per segment.
constexpr int32_t F8_LATE_MIN_KEYS = 65536;

// LDS layouts, XOR-swizzled so that the 16-byte fragment reads of a wave hit
// distinct banks (SQ_LDS_BANK_CONFLICT reads 0 for both access patterns on
// gfx950; a value-row swizzle of ((d >> 1) ^ (d >> 3)) & 3 measured conflicts).
__device__ __forceinline__ int k8_swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }
__device__ __forceinline__ int v8_swz(int d) { return (d >> 2) & 3; }
__device__ __forceinline__ int k8_lds_offset(int r, int c) { return r * 128 + 16 * (c ^ k8_swz(r)); }
__device__ __forceinline__ int v8_lds_offset(int d, int c) { return d * 64 + 16 * (c ^ v8_swz(d)); }

// Byte position of key kk (0..63) of a tile inside a value-dim row of V^T.
__device__ __forceinline__ int v8_key_byte(int kk) {
  const int u = kk >> 5, w = kk & 31;
  const int g = (w & 7) >> 2;
  return 32 * g + 16 * u + 4 * (w >> 3) + (w & 3);
}

// ---------------------------------------------------------------------------
// Per-channel value maxima start at 0 (bit pattern of +0.0f).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_clear_kernel(unsigned* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Value channel maxima.  grid = (VA_KEYS-key chunks of the longest segment,
// segments, heads), 256 threads.
// v_amax: [H][n_seqs][128] per value channel, the largest magnitude over the
//         segment (float bit patterns, which order like the values since they
//         are >= 0); raised here with atomic max from 0.  One atomic per
//         channel and chunk: the atomics of a segment all land on four cache
//         lines per head, so their number, not the bytes read, sets the time
//         when a chunk is small.
// ---------------------------------------------------------------------------
constexpr int VA_KEYS = 1024;
__global__ __launch_bounds__(256) void v_amax_fp8_kernel(const u32x4* __restrict__ v, const int32_t* __restrict__ cu,
                                                         int32_t n_heads, unsigned* __restrict__ v_amax,
                                                         int32_t max_seqlen) {
  __shared__ float s_red[4][D];
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t seg_a = cu[s];
  const int32_t S = min(cu[s + 1] - seg_a, max_seqlen);
  const int32_t k0 = c * VA_KEYS;
  if (k0 >= S) return;  // whole block leaves together
  const int32_t k1 = min(S, k0 + VA_KEYS);
  // Thread reads chunk cc (dims 8 cc .. 8 cc + 7) of keys k0 + r, + 16, ...:
  // sixteen consecutive threads cover one key's 256 bytes.
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, cc = tid & 15, r = tid >> 4;
  float vm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vm[j] = 0.0f;
  for (int32_t key = k0 + r; key < k1; key += 128) {
    u32x4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t kk = key + 16 * i;
      x[i] = u32x4{0u, 0u, 0u, 0u};
      if (kk < k1) x[i] = v[((int64_t(seg_a) + kk) * n_heads + h) * CHUNKS_PER_ROW + cc];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float f[8];
      unpack8(x[i], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) vm[j] = fmaxf(vm[j], fabsf(f[j]));
    }
  }
  // Over the four threads of the wave with the same chunk, then over the waves.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    vm[j] = fmaxf(vm[j], __shfl_xor(vm[j], 16));
    vm[j] = fmaxf(vm[j], __shfl_xor(vm[j], 32));
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_red[wv][8 * cc + j] = vm[j];
  }
  __syncthreads();
  if (tid < D) {
    const float m = fmaxf(fmaxf(s_red[0][tid], s_red[1][tid]), fmaxf(s_red[2][tid], s_red[3][tid]));
    if (m > 0.0f) atomicMax(v_amax + (int64_t(h) * gridDim.y + s) * D + tid, __float_as_uint(m));
  }
}

// ---------------------------------------------------------------------------
// FP8 K/V prologue, keys.  grid = (64-key tiles of the longest segment,
// segments, heads), 256 threads.
// k_ws:   [H][rows][128] e4m3 rotated keys, rows past a segment's end zero.
// k_sc:   [H][rows/64] one word per tile: byte i = 8-bit exponent scale of
//         keys 16i .. 16i+15.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_prologue_fp8_kernel(const u32x4* __restrict__ k,
                                                              const int32_t* __restrict__ cu,
                                                              const float* __restrict__ pos, int32_t n_heads,
                                                              RopeTable tab, u32x2* __restrict__ k_ws,
                                                              unsigned* __restrict__ k_sc,
                                                              int32_t* __restrict__ order, int64_t rows_per_head,
                                                              int32_t max_seqlen) {
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];
  __shared__ float s_red[4][4];
  const int tile = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  if (tile == 0 && h == 0) write_segment_rank(cu, int(gridDim.y), s, order);  // before any early exit
  const int32_t seg_a = cu[s];
  const int32_t S = min(cu[s + 1] - seg_a, max_seqlen);  // a longer segment counts as its first max_seqlen tokens
  if (tile * KT >= S) return;  // whole block leaves together
  stage_rope_table(tab, s_omega, s_axis);
  __syncthreads();
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t prow = packed_start(seg_a, s) + int64_t(tile) * KT;  // packed row of this tile's key 0
  const int64_t tiles_per_head = rows_per_head / KT;

  // Keys: 1024 chunks of 8 dims, 4 per thread; chunk i of the thread is key
  // (tid >> 4) + 16 i, dims 8 (tid & 15) ..; so chunk i lies in 16-key block i.
  float kf[4][8];
  float amax[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i, cc = tid & 15;
    const int key = tile * KT + r;
    if (key < S) {
      const int64_t tok = int64_t(seg_a) + key;
      unpack8(k[(tok * n_heads + h) * CHUNKS_PER_ROW + cc], kf[i]);
      rope8(kf[i], cc * 4, s_omega, s_axis, pos[3 * tok], pos[3 * tok + 1], pos[3 * tok + 2]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[i][e] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(kf[i][e]));
    amax[i] = m;
  }

  // Key block maxima over the workgroup.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], off));
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s_red[wv][j] = amax[j];
  }
  __syncthreads();
  int ex[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ex[j] = e4m3_scale_exponent(fmaxf(fmaxf(s_red[0][j], s_red[1][j]), fmaxf(s_red[2][j], s_red[3][j])));
  if (tid == 0) {
    unsigned w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= unsigned(ex[j] + E8M0_ONE) << (8 * j);
    k_sc[int64_t(h) * tiles_per_head + prow / KT] = w;
  }

  // Quantized keys: 8 bytes per chunk.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float down = ldexpf(1.0f, -ex[i]);
    const int r = (tid >> 4) + 16 * i, cc = tid & 15;
    u32x2 w;
    w[0] = pack_e4m3x4(kf[i][0] * down, kf[i][1] * down, kf[i][2] * down, kf[i][3] * down);
    w[1] = pack_e4m3x4(kf[i][4] * down, kf[i][5] * down, kf[i][6] * down, kf[i][7] * down);
    k_ws[((int64_t(h) * rows_per_head + prow + r) * D) / 8 + cc] = w;
  }
}

// ---------------------------------------------------------------------------
// FP8 K/V prologue, values.  grid = (64-key tiles, segments, heads), 256
// threads, after v_amax_fp8_kernel has finished.
// v_ws:   [H][rows/64][128][64] e4m3 values, transposed per tile, keys in the
//         order v8_key_byte gives, each channel scaled by its segment's
//         power of two (the exponent e4m3_scale_exponent gives for v_amax).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void v_quant_fp8_kernel(const u32x4* __restrict__ v, const int32_t* __restrict__ cu,
                                                          int32_t n_heads, unsigned* __restrict__ v_ws,
                                                          const unsigned* __restrict__ v_amax,
                                                          int64_t rows_per_head, int32_t max_seqlen) {
  const int tile = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t seg_a = cu[s];
  const int32_t S = min(cu[s + 1] - seg_a, max_seqlen);
  if (tile * KT >= S) return;
  const int tid = threadIdx.x;
  const int64_t prow = packed_start(seg_a, s) + int64_t(tile) * KT;
  const int64_t tiles_per_head = rows_per_head / KT;
  // Thread owns keys 4 k4 .. 4 k4 + 3 and dims 8 dc .. 8 dc + 7; for each of
  // its 8 dims, its 4 keys are 4 consecutive bytes of that dim's row.
  const int k4 = tid & 15, dc = tid >> 4;
  const unsigned* am = v_amax + (int64_t(h) * gridDim.y + s) * D + 8 * dc;
  float down[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) down[j] = ldexpf(1.0f, -e4m3_scale_exponent(__uint_as_float(am[j])));
  float vf[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = tile * KT + 4 * k4 + i;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < S) val = v[((int64_t(seg_a) + key) * n_heads + h) * CHUNKS_PER_ROW + dc];
    unpack8(val, vf[i]);
  }
  const int pos0 = v8_key_byte(4 * k4);
  unsigned* vt = v_ws + ((int64_t(h) * tiles_per_head + prow / KT) * D * KT) / 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = 8 * dc + j;
    vt[(d * KT + pos0) / 4] =
        pack_e4m3x4(vf[0][j] * down[j], vf[1][j] * down[j], vf[2][j] * down[j], vf[3][j] * down[j]);
  }
}

// ---------------------------------------------------------------------------
// FP8 attention forward, software-pipelined inside each wave.
//
// Iteration t issues, in one block of 8 MFMA slots,
//     S(t+1) = K(t+1) Q^T      4 MFMAs (two subtiles x two 64-dim halves)
//     O     += V(t-1) P(t-1)   4 MFMAs (one per 32-dim block of O^T)
// and, after every slot, the exponentials of 4 of the 32 probabilities each
// lane forms for tile t.  Consecutive score MFMAs share their query operand
// and the four value MFMAs share the probabilities.
//
// Online softmax in base 2.  A score MFMA returns s = q8 . k8; the base-2
// logit is z = cl * s with cl = scale * log2 e, and a probability is stored
// as p' = exp2(cl * s - mm) = 256 p, where mm is the running reference minus
// 8 (one multiply-add and one exp2 per element).  Dense instance: the
// reference moves lazily, only where some p' could pass 448 (the tile's
// largest logit more than P_ROOM_LOG2 above mm), to that logit, in one of two
// forms chosen per launch by the longest segment.  Early (shorter segments,
// where moves are frequent): every tile's maximum is taken before its
// exponentials, the lane's part while the previous tile's exponentials run,
// and O and l follow after the previous tile's products.  Late (long
// segments): a tile none of whose packed probabilities reached 448 needs
// nothing; otherwise the wave takes the tile's exact maximum, moves the
// reference where needed, rescales O and l and recomputes the tile.
// Skip-Softmax instance: every tile's maximum is taken for the skip rule
// anyway, so the reference is the exact running maximum of the kept tiles.
// Either way O and l share one reference, so the result is softmax over the
// kept keys with P rounded relative to a reference within a factor 1.75 of
// the running maximum.
//
// LDS: rings of eight key slots and eight value slots of 8 KiB.  Iteration t
// reads K(t+1) and V(t-1) and issues direct buffer->LDS loads of K(t+5) and
// V(t+3); iterations pair up into epochs that end with one barrier, exactly
// as in the bf16 kernel.
// ---------------------------------------------------------------------------
template <bool SKIP, bool LATE>
__global__ __launch_bounds__(F8_NW * 64, 1) void attn_fwd_fp8_kernel(
    const u32x4* __restrict__ q, const int32_t* __restrict__ cu, const float* __restrict__ pos,
    u32x2* __restrict__ out, float* __restrict__ lse, int32_t n_tokens, int32_t n_heads, float scale_log2,
    RopeTable tab, const char* __restrict__ k_ws, const char* __restrict__ v_ws,
    const unsigned* __restrict__ k_sc, const unsigned* __restrict__ v_amax, const int32_t* __restrict__ order,
    int64_t rows_per_head, int32_t max_seqlen, float skip_log2, unsigned long long* __restrict__ skip_stats) {
  static_assert(F8_TILE_BYTES / 16 == F8_NW * 64, "one direct load per lane, tile and tensor");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];

  // The segment comes from the rank order the K/V prologue wrote.
  const int qt = blockIdx.x, h = blockIdx.y;
  const int s = gridDim.z == 1 ? 0 : order[blockIdx.z];
  const int32_t seg_a = cu[s];
  const int32_t S = min(cu[s + 1] - seg_a, max_seqlen);  // a longer segment counts as its first max_seqlen tokens
  if (qt * F8_BQ >= S) return;  // whole block leaves together

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  stage_rope_table(tab, s_omega, s_axis);

  const int n_kt = (S + KT - 1) / KT;
  const int last_t = n_kt - 1;
  const int64_t prow = packed_start(seg_a, s);
  const int64_t tiles_per_head = rows_per_head / KT;
  const char* kg = k_ws + (int64_t(h) * rows_per_head + prow) * D;
  const char* vg = v_ws + (int64_t(h) * rows_per_head + prow) * D;
  const unsigned* ksp = k_sc + int64_t(h) * tiles_per_head + prow / KT;

  // Direct loads: lane L of wave w fills LDS chunk p = 64 w + L of a slot
  // with the logical chunk the swizzle puts there.
  unsigned ksrc_off, vsrc_off;
  {
    const int p = wave * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ k8_swz(r);
    ksrc_off = unsigned(r * 128 + 16 * c);
    const int d = p >> 2, cv = (p & 3) ^ v8_swz(d);
    vsrc_off = unsigned(d * 64 + 16 * cv);
  }
  const int seg_bytes = n_kt * F8_TILE_BYTES;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, seg_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, seg_bytes, 0x00020000);
  auto load_k = [&](int t, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(smem + slot * F8_TILE_BYTES + wave * 1024), 16,
                                             ksrc_off, t * F8_TILE_BYTES, 0, 0);
  };
  auto load_v = [&](int t, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(smem + F8_VBASE + slot * F8_TILE_BYTES + wave * 1024),
                                             16, vsrc_off, t * F8_TILE_BYTES, 0, 0);
  };

  load_k(0, ic<0>());
  load_k(min(1, last_t), ic<1>());
  __syncthreads();  // rope table staged; K(0) and K(1) have landed
  load_k(min(2, last_t), ic<2>());
  load_v(0, ic<0>());
  load_k(min(3, last_t), ic<3>());
  load_v(min(1, last_t), ic<1>());
  load_k(min(4, last_t), ic<4>());
  load_v(min(2, last_t), ic<2>());

  // Value scales: lane L of value-dim block db carries the exponent scale of
  // channel 32 db + L % 32 over this segment, for both 32-key halves.
  unsigned vsc[4];
  {
    const unsigned* am = v_amax + (int64_t(h) * gridDim.z + s) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      vsc[db] = unsigned(e4m3_scale_exponent(__uint_as_float(am[32 * db + l32])) + E8M0_ONE);
  }

  // Queries: B operand of S^T = K Q^T.  Lane holds query row l32 and, for
  // half ks, dims 64 ks + 32 g .. + 31, rotated in fp32, scaled by the row's
  // power-of-two factor and rounded to e4m3; qsc is that factor's 8-bit
  // exponent scale, which the score MFMAs apply.
  const int qrow = qt * F8_BQ + wave * 32 + l32;
  i32x8 qf[2];
  unsigned qsc;
  {
    float f[2][4][8];
    if (qrow < S) {
      const int64_t tok = int64_t(seg_a) + qrow;
      const float pt = pos[3 * tok], ph = pos[3 * tok + 1], pw = pos[3 * tok + 2];
      const u32x4* qp = q + (tok * n_heads + h) * CHUNKS_PER_ROW;
      // The test reads only the positions, so a turning wave computes its
      // angles while the query chunks are still in flight.
      if (wave_at_origin(pt, ph, pw)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 4; ++j) unpack8(qp[8 * ks + 4 * g + j], f[ks][j]);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = 8 * ks + 4 * g + j;
            unpack8(qp[c], f[ks][j]);
            rope_turn4(f[ks][j], rope_angles4(c * 4, s_omega, s_axis, pt, ph, pw));
          }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) f[ks][j][e] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[ks][j][e]));
    amax = pair_max(amax);  // the row's other 64 dims sit in lane L ^ 32
    const int eq = e4m3_scale_exponent(amax);
    const float down = ldexpf(1.0f, -eq);
    qsc = unsigned(eq + E8M0_ONE);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float* x = &f[ks][w >> 1][4 * (w & 1)];
        qf[ks][w] = int(pack_e4m3x4(x[0] * down, x[1] * down, x[2] * down, x[3] * down));
      }
  }
  const float cl = scale_log2;  // base-2 logit per unit of q8 . k8

  // Per-lane fragment offsets inside a slot (subtile, slot and 32-dim block
  // parts are immediates): K rows 32u + l32, chunks 4 ks + 2 g + hf; V^T rows
  // 32 db + l32, chunks 2 g + hf.
  int koff[2][2], voff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) koff[ks][hf] = k8_lds_offset(l32, 4 * ks + 2 * g + hf);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) voff[hf] = F8_VBASE + v8_lds_offset(l32, 2 * g + hf);
  // The 16-key block of the keys this lane feeds, per subtile: 2u + (l32 >= 16).
  const unsigned ksh0 = l32 >= 16 ? 8u : 0u;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float mm = -INFINITY, l = 0.0f;   // reference minus 8, and the row sum of p' = exp2(z - mm)
  // The factor that takes O and l to this tile's reference, and whether some
  // row of the wave moved it (wave-uniform): Skip-Softmax and the early dense
  // form.
  float resc = 1.0f;
  bool rescale = false;
  // Early dense form: the lane's largest raw score of the tile whose
  // exponentials come next.
  float tmx = -INFINITY;
  // Skip-Softmax: the row's largest base-2 logit over the tiles seen so far, the
  // exponent offset of the current tile (mm, or +inf where the row leaves the
  // tile out), and the row's counts.
  float mt = -INFINITY, moff = 0.0f;
  unsigned n_seen = 0, n_skipped = 0;
  bool prev_kept = true;       // Skip-Softmax: the wave kept the previous tile (wave-uniform)
  f32x16 sc[2][2];          // S^T of one tile [buffer by tile parity][subtile]
  i32x8 pf[2];              // its e4m3 probabilities, by tile parity

  // Slots are compile-time constants (ic<>) in the unrolled loop and run-time
  // values in the last iteration; int(SLOT) covers both.
  auto kfrag = [&](auto SLOT, int u, int ks) __attribute__((always_inline)) {
    const int slot = int(SLOT);
    const char* base = smem + slot * F8_TILE_BYTES + u * 4096;
    const u32x4 a = *reinterpret_cast<const u32x4*>(base + koff[ks][0]);
    const u32x4 b = *reinterpret_cast<const u32x4*>(base + koff[ks][1]);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto vfrag = [&](auto SLOT, int db) __attribute__((always_inline)) {
    const int slot = int(SLOT);
    const char* base = smem + slot * F8_TILE_BYTES + db * 2048;  // voff holds the value ring's base
    const u32x4 a = *reinterpret_cast<const u32x4*>(base + voff[0]);
    const u32x4 b = *reinterpret_cast<const u32x4*>(base + voff[1]);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // ksw holds the lane's key scales of subtiles 0 and 1 in bytes 0 and 2; the
  // instruction's scale byte select picks one, so no per-subtile extraction.
  auto mfma_qk = [&](f32x16 acc, i32x8 kf, int ks, int u, unsigned ksw) __attribute__((always_inline)) {
    if (u == 0) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[ks], acc, 0, 0, 0, int(ksw), 0, int(qsc));
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[ks], acc, 0, 0, 2, int(ksw), 0, int(qsc));
  };
  // Value products: per-lane channel scales on V^T, p' unscaled.
  auto mfma_pv = [&](f32x16 acc, i32x8 vf, const i32x8& p, int db) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, p, acc, 0, 0, 0, int(vsc[db]), 0, E8M0_ONE);
  };
  // Per-lane exponent scales of K tile t (subtile 0 in byte 0, subtile 1 in
  // byte 2, both in k0; k1 carries the same word).
  auto kscales = [&](int t, unsigned& k0, unsigned& k1) __attribute__((always_inline)) {
    k0 = ksp[t] >> ksh0;
    k1 = k0;
  };

  // S^T(t) into buffer B, alone (pipeline fill).
  auto qk_alone = [&](auto B, auto SLOT, unsigned k0, unsigned k1) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma_qk(acc, kfrag(SLOT, u, ks), ks, u, u ? k1 : k0);
      sc[b][u] = acc;
    }
  };
  // O^T += V^T(t) P^T(t) from buffer B, alone (pipeline drain).
  auto pv_alone = [&](auto B, auto SLOT) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_pv(o[db], vfrag(SLOT, db), pf[b], db);
  };
  // Keys of tile t at or past the segment end get score -inf.  Key (u, r) of
  // this lane is t*64 + 32u + 8(r/4) + 4g + r%4: compare the constant part
  // with the lane's limit.
  auto mask_tail = [&](auto B, int t) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const int lim = S - t * KT - 4 * g;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = sc[b][u][r];
        sc[b][u][r] = 32 * u + 8 * (r >> 2) + (r & 3) < lim ? x : -INFINITY;
      }
  };
  // The lane's largest raw score of subtile u of the tile in buffer B, of the
  // whole tile, and of the tile with its partner's (the row's).
  // Chains of three-operand maxima from a seed (a seed that is itself a
  // maximum, or -inf, spares the compiler's canonicalizing of raw scores).
  auto subtile_max = [&](auto B, int u, float seed) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    float mx = seed;
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sc[b][u][r]), sc[b][u][r + 1]);
    return mx;
  };
  auto lane_max = [&](auto B) __attribute__((always_inline)) {
    return subtile_max(B, 1, subtile_max(B, 0, -INFINITY));
  };
  auto tile_max = [&](auto B) __attribute__((always_inline)) { return pair_max(lane_max(B)); };
  // Unit j (0..7) of tile t's probabilities (scores in buffer B): word j of
  // the lane's 32 bytes, i.e. subtile j / 4, registers 4 (j % 4) .. + 3.
  auto exp_unit = [&](auto B, int j, float (&p)[4]) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const float off = SKIP ? moff : mm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sc[b][j >> 2][4 * (j & 3) + i], cl, -off));
      pin(p[i]);
    }
  };
  auto pack_unit = [&](int j, const float (&p)[4], i32x8& pw, float& rs) __attribute__((always_inline)) {
    // both halves of the word are written, so its previous contents may seed the conversion
    unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], unsigned(pw[j]), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
    float r = j == 0 ? (p[0] + p[1]) + (p[2] + p[3]) : rs + ((p[0] + p[1]) + (p[2] + p[3]));
    pin(w);
    pin(r);
    pw[j] = int(w);
    rs = r;
  };
  // After the exponentials of tile t (buffer B, products of tile t-1 issued),
  // with chk the OR over the lane's packed words of (word + 0x02020202).
  // Late dense form: every p' <= 448 rounds to at most 0x7e and an overflow
  // gives 0x7f (an e4m3 NaN), so a byte at 0x7e or above, i.e. bit 7 set in
  // chk, flags a p' that reached 448; a NaN gives 0xff, whose carry spoils the
  // test, but then the row sum is NaN or infinite too.  Only a flagged wave
  // takes the tile's exact maximum, and only where some p' could pass 448
  // (the tile's largest logit more than P_ROOM_LOG2 above mm) does it move the
  // reference to that maximum, rescale O and l and recompute the tile.  The
  // first tile always takes this path (mm is still -inf there).  Skip-Softmax
  // instance and early dense form: the reference was set before the
  // exponentials (decide, prepare); here O and l are rescaled to it (after
  // the products of tile t-1, which used the old one).
  auto settle = [&](auto B, i32x8& pw, float rs, unsigned chk) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    if constexpr (SKIP || !LATE) {
      (void)chk;
      if (rescale) {
        l *= resc;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= resc;
      }
      l += rs;
    } else {
      const bool over = (chk & 0x80808080u) != 0u || !(rs <= FLT_MAX);
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        const float tmax = tile_max(ic<b>()) * cl;
        const bool move = !(tmax - mm <= P_ROOM_LOG2);  // some p' could pass 448 (or mm = -inf)
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          const float m_new = move ? fmaxf(mm, tmax - P_SHIFT) : mm;
          const float a = __builtin_amdgcn_exp2f(mm - m_new);  // 0 from mm = -inf, 1 where unmoved
          mm = m_new;
          l *= a;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= a;
          rs = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              p[i] = __builtin_amdgcn_exp2f(fmaf(sc[b][j >> 2][4 * (j & 3) + i], cl, -mm));
            pw[j] = int(pack_e4m3x4(p[0], p[1], p[2], p[3]));
            rs += (p[0] + p[1]) + (p[2] + p[3]);
          }
        }
      }
      l += rs;
    }
  };

  // Early dense form, before the exponentials of a tile: move the reference of
  // the rows where some p' could pass 448 (the tile's largest logit more than
  // P_ROOM_LOG2 above mm, or mm = -inf on the first tile) to that logit minus
  // 8.  tmx holds the lane's largest raw score of the tile, taken while the
  // previous tile's exponentials ran.  O and l follow in settle.
  auto prepare = [&]() __attribute__((always_inline)) {
    const float tmax = pair_max(tmx) * cl;
    const bool move = !(tmax - mm <= P_ROOM_LOG2);
    rescale = __builtin_amdgcn_ballot_w64(move) != 0;
    if (rescale) {
      const float m_new = move ? fmaxf(mm, tmax - P_SHIFT) : mm;
      resc = __builtin_amdgcn_exp2f(mm - m_new);  // 0 from mm = -inf, 1 where unmoved
      mm = m_new;
    }
  };

  // Iteration t, B = t mod 2 (S(t) in sc[B], P(t-1) in pf[1 - B]), reading
  // K(t+1) from kslot and V(t-1) from vslot: 8 MFMA slots.  Slots 0..3 issue
  // S(t+1) in the order (subtile, half) = (0,0), (1,0), (0,1), (1,1), straight
  // into sc[1 - B] (consecutive pairs share the query operand); slots 4..7
  // issue O += V(t-1) P(t-1), one MFMA per 32-dim block of O^T (all four
  // share the probabilities).  Exponential unit j of tile t follows slot j,
  // then tile t settles; the early dense form moves the reference for tile t
  // first (prepare) and takes the lane's maximum of S(t+1) in slots 5 and 6.
  // Two fragment registers alternate, each read one or
  // two slots ahead of its MFMA (the first two at the start).  A scheduling
  // fence after every slot keeps this order.  The Skip-Softmax instance keeps
  // the MFMA order but groups the exponentials: units 0..3 after the score
  // MFMAs and units 4..7 after the value MFMAs, each group under one
  // wave-uniform branch, the value MFMAs under a third (a left-out tile then
  // skips three branches, where interleaving needed twelve).
  auto region = [&](auto B, auto QK, auto PV, bool do_exp, bool pv_live, auto kslot, auto vslot, unsigned k0,
                    unsigned k1) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    constexpr bool do_qk = decltype(QK)::value != 0;
    constexpr bool do_pv = decltype(PV)::value != 0;
    i32x8 fr[2], pw;
    asm volatile("" : "=v"(pw));  // every word is written below; no need to clear it first
    float rs = 0.0f;
    if (do_qk) {
      fr[0] = kfrag(kslot, 0, 0);
      fr[1] = kfrag(kslot, 1, 0);
    } else if (do_pv) {
      fr[0] = vfrag(vslot, 0);
      fr[1] = vfrag(vslot, 1);
    }
    if constexpr (!SKIP && !LATE) {
      if (do_exp) prepare();
    }
    if constexpr (SKIP) {
      // Skip-Softmax instance: the MFMAs of each half, then its exponentials
      // under one wave-uniform branch.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (do_qk) {
          const int u = j & 1, ks = j >> 1;
          f32x16 acc;
          if (ks == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
          } else {
            acc = sc[1 - b][u];
          }
          sc[1 - b][u] = mfma_qk(acc, fr[u], ks, u, u ? k1 : k0);
          if (j < 2)
            fr[u] = kfrag(kslot, u, 1);
          else if (do_pv)
            fr[u] = vfrag(vslot, j - 2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_exp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p[4];
          exp_unit(ic<b>(), j, p);
          pack_unit(j, p, pw, rs);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_pv) {
        if (pv_live) {
#pragma unroll
          for (int j = 4; j < 8; ++j) {
            o[j - 4] = mfma_pv(o[j - 4], fr[j & 1], pf[1 - b], j - 4);
            if (j < 6) fr[j & 1] = vfrag(vslot, j - 2);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_exp) {
#pragma unroll
        for (int j = 4; j < 8; ++j) {
          float p[4];
          exp_unit(ic<b>(), j, p);
          pack_unit(j, p, pw, rs);
        }
      }
    } else {
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (do_qk) {
          const int u = j & 1, ks = j >> 1;
          f32x16 acc;
          if (ks == 0) {
  #pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
          } else {
            acc = sc[1 - b][u];
          }
          sc[1 - b][u] = mfma_qk(acc, fr[u], ks, u, u ? k1 : k0);
          // next fragment into the register this MFMA has read
          if (j < 2)
            fr[u] = kfrag(kslot, u, 1);
          else if (do_pv)
            fr[u] = vfrag(vslot, j - 2);
        }
        if (do_exp) {
          float p[4];
          exp_unit(ic<b>(), j, p);
          pack_unit(j, p, pw, rs);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float tn = -INFINITY;
  #pragma unroll
      for (int j = 4; j < 8; ++j) {
        if (do_pv) {
          if (pv_live) o[j - 4] = mfma_pv(o[j - 4], fr[j & 1], pf[1 - b], j - 4);
          if (j < 6) fr[j & 1] = vfrag(vslot, j - 2);
        }
        if (do_exp) {
          float p[4];
          exp_unit(ic<b>(), j, p);
          pack_unit(j, p, pw, rs);
        }
        // Early form: the next tile's maximum, subtile 0 then 1, once their
        // score MFMAs (slots 2 and 3) are done.
        if constexpr (!LATE) {
          if (do_qk && (j == 5 || j == 6)) {
            tn = subtile_max(ic<1 - b>(), j - 5, tn);
            pin(tn);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // A use of S(t+1) in this block (the early form's maximum, the late
      // form's empty asm) keeps its MFMAs here, between the exponentials they
      // overlap: otherwise the compiler sinks them past the settle branch,
      // next to the next tile's exponentials, where they run back to back and
      // the exponentials wait for them.  They are done by now, so the use
      // waits for nothing.
      if constexpr (LATE) {
        if (do_qk) asm volatile("" ::"v"(sc[1 - b][0]), "v"(sc[1 - b][1]));
      } else {
        if (do_qk) tmx = tn;
      }
    }
    if (do_exp) {
      unsigned chk = 0u;
      if constexpr (!SKIP && LATE) {
#pragma unroll
        for (int j = 0; j < 8; ++j) chk |= unsigned(pw[j]) + 0x02020202u;
      }
      settle(ic<b>(), pw, rs, chk);
      pf[b] = pw;
    }
  };

  // Skip-Softmax decision for tile t (scores in buffer B), per row: the row
  // leaves the tile out when its largest logit in the tile is below its
  // largest logit over the earlier tiles plus log2 of the threshold; rows past
  // the segment end leave every tile out.  Sets the row's exponent offset and
  // its reference (the running maximum, which only a kept tile can raise) and
  // the rescale factor settle applies; counts the row's decisions.  Returns
  // whether the whole wave leaves the tile out.
  auto decide = [&](auto B) __attribute__((always_inline)) {
    const float tm = tile_max(B) * cl;
    const bool valid = qrow < S;
    const bool lets_go = !valid || tm < mt + skip_log2;
    mt = fmaxf(mt, tm);
    const float m_new = fmaxf(mm, mt - P_SHIFT);
    resc = __builtin_amdgcn_exp2f(mm - m_new);  // 1 where unmoved, 0 from -inf
    rescale = __builtin_amdgcn_ballot_w64(m_new != mm) != 0;
    mm = m_new;
    moff = lets_go ? INFINITY : mm;
    n_seen += valid ? 1u : 0u;
    n_skipped += (valid && lets_go) ? 1u : 0u;
    return __builtin_amdgcn_ballot_w64(!lets_go) == 0;
  };
  // Iteration t under Skip-Softmax: the exponentials of tile t only if some
  // row of the wave keeps it, the products of tile t-1 only if some row kept
  // that one.
  auto region_skip = [&](auto B, auto QK, auto kslot, auto vslot, unsigned k0, unsigned k1, bool skip)
      __attribute__((always_inline)) {
    region(B, QK, ic<1>(), !skip, prev_kept, kslot, vslot, k0, k1);
    prev_kept = !skip;
  };

  // Scales for the products iteration t issues: K(t+1).
  unsigned kq0, kq1;
  // Steady iteration t (1 <= t <= last_t - 1), T8 = t mod 8.  Loads K(t+5) and
  // V(t+3).  Iterations pair up into epochs (t odd, t+1) that end with one
  // barrier: within an epoch no slot that is read is also written, and
  // everything an epoch reads was issued at least two epochs earlier.  Past
  // the last tile the index is clamped: the duplicate goes to a slot that is
  // not read again, and every iteration keeps issuing the same loads, which
  // the ring barrier counts.
  auto step = [&](auto T8, int t) __attribute__((always_inline)) {
    constexpr int t8 = decltype(T8)::value;
    if constexpr (SKIP)
      region_skip(ic<t8 & 1>(), ic<1>(), ic<(t8 + 1) & 7>(), ic<(t8 + 7) & 7>(), kq0, kq1, decide(ic<t8 & 1>()));
    else
      region(ic<t8 & 1>(), ic<1>(), ic<1>(), true, true, ic<(t8 + 1) & 7>(), ic<(t8 + 7) & 7>(), kq0, kq1);
    load_k(min(t + 5, last_t), ic<(t8 + 5) & 7>());
    load_v(min(t + 3, last_t), ic<(t8 + 3) & 7>());
    kscales(min(t + 2, last_t), kq0, kq1);
    if ((t8 & 1) == 0) ring_barrier<4>();  // end of an epoch: its loads may stay in flight
  };
  // Last iteration t = last_t >= 1, B = t mod 2: exponentials of tile t and
  // products of tile t-1, then the products of tile t.  It runs once, so its
  // slots are run-time values.
  auto last = [&](auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    mask_tail(ic<b>(), last_t);
    if constexpr (!SKIP && !LATE) tmx = lane_max(ic<b>());  // of the masked scores
    if constexpr (SKIP)
      region_skip(ic<b>(), ic<0>(), 0, (last_t - 1) & 7, kq0, kq1, decide(ic<b>()));
    else
      region(ic<b>(), ic<0>(), ic<1>(), true, true, 0, (last_t - 1) & 7, kq0, kq1);
    ring_barrier<0>();  // V(t) has landed
    __builtin_amdgcn_sched_barrier(0);
    if (prev_kept) pv_alone(ic<b>(), last_t & 7);
  };
  {
    unsigned k0, k1;
    kscales(0, k0, k1);
    qk_alone(ic<0>(), ic<0>(), k0, k1);
  }
  if (n_kt == 1) {
    mask_tail(ic<0>(), 0);
    if constexpr (!SKIP && !LATE) tmx = lane_max(ic<0>());  // of the masked scores
    if constexpr (SKIP) (void)decide(ic<0>());  // the first tile is always kept: this sets the reference
    region(ic<0>(), ic<0>(), ic<0>(), true, true, ic<1>(), ic<7>(), 0u, 0u);
    ring_barrier<0>();
    pv_alone(ic<0>(), ic<0>());
  } else {
    ring_barrier<6>();  // every wave is done with K(0) before its slot is refilled
    kscales(1, kq0, kq1);
    if constexpr (!SKIP && !LATE) tmx = lane_max(ic<0>());
    // t = 0: no products of an earlier tile yet; an epoch of its own.
    if constexpr (SKIP) (void)decide(ic<0>());  // the first tile is always kept: this sets the reference
    region(ic<0>(), ic<1>(), ic<0>(), true, true, ic<1>(), ic<7>(), kq0, kq1);
    load_k(min(5, last_t), ic<5>());
    load_v(min(3, last_t), ic<3>());
    kscales(min(2, last_t), kq0, kq1);
    ring_barrier<4>();
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
    if (last_t & 1)
      last(ic<1>());
    else
      last(ic<0>());
  }

  // Epilogue: O = O / l, lse = (mm + log2 l) * ln 2 (the 2^8 of the stored
  // probabilities cancels: mm and l carry it with opposite signs).
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
    if (g == 0) lse[int64_t(h) * n_tokens + tok] = (mm + log2f(lt)) * 0.69314718055994531f;
  }
  if constexpr (SKIP) {
    // (row, tile) pairs seen and left out by this wave's rows, for callers that ask; lane L and
    // L + 32 hold the same row, so only the lower half counts
    if (skip_stats != nullptr) {
      unsigned long long seen = g == 0 ? n_seen : 0u, left = g == 0 ? n_skipped : 0u;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        seen += __shfl_xor(seen, off);
        left += __shfl_xor(left, off);
      }
      if (lane == 0 && seen != 0) {
        atomicAdd(&skip_stats[0], seen);
        atomicAdd(&skip_stats[1], left);
      }
    }
  }
}
}  // namespace

int launch_kv_prologue_fp8(const void* k, const void* v, const int32_t* cu, const float* pos, int32_t n_heads,
                           int32_t n_seqs, int32_t max_seqlen, const RopeTable& table, void* k_ws, void* v_ws,
                           unsigned* k_sc, unsigned* v_amax, int32_t* order, int64_t rows_per_head, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + KT - 1) / KT);
  if (tiles == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The channel maxima are raised from 0 by atomic max: clear them first (a fill kernel, so that the
  // sequence may be captured in a graph).
  const int64_t n_amax = int64_t(n_heads) * n_seqs * D;
  const unsigned clear_blocks = unsigned(std::min<int64_t>((n_amax + 255) / 256, 4096));
  hipLaunchKernelGGL(fp8_clear_kernel, dim3(clear_blocks), dim3(256), 0, st, v_amax, n_amax);
  const unsigned chunks = unsigned((int64_t(max_seqlen) + VA_KEYS - 1) / VA_KEYS);
  hipLaunchKernelGGL(v_amax_fp8_kernel, dim3(chunks, unsigned(n_seqs), unsigned(n_heads)), dim3(256), 0, st,
                     static_cast<const u32x4*>(v), cu, n_heads, v_amax, max_seqlen);
  const dim3 grid(tiles, unsigned(n_seqs), unsigned(n_heads));
  hipLaunchKernelGGL(kv_prologue_fp8_kernel, grid, dim3(256), 0, st, static_cast<const u32x4*>(k), cu, pos,
                     n_heads, table, static_cast<u32x2*>(k_ws), k_sc, order, rows_per_head, max_seqlen);
  hipLaunchKernelGGL(v_quant_fp8_kernel, grid, dim3(256), 0, st, static_cast<const u32x4*>(v), cu, n_heads,
                     static_cast<unsigned*>(v_ws), static_cast<const unsigned*>(v_amax), rows_per_head, max_seqlen);
  return int(hipGetLastError());
}

int launch_attention_fp8(const void* q, const int32_t* cu, const float* pos, void* out, float* lse,
                         int64_t n_tokens, int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, float scale,
                         float skip_threshold, const RopeTable& table, const void* k_ws, const void* v_ws,
                         const unsigned* k_sc, const unsigned* v_amax, const int32_t* order, int64_t rows_per_head,
                         unsigned long long* skip_stats, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + F8_BQ - 1) / F8_BQ);
  if (tiles == 0) return 0;
  const bool skip = skip_threshold > 0.0f;
  const bool late = !skip && max_seqlen >= F8_LATE_MIN_KEYS;
  const int inst = skip ? 2 : late ? 1 : 0;
  const void* fn = skip   ? reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<true, false>)
                   : late ? reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<false, true>)
                          : reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<false, false>);
  // The dynamic LDS limit is raised once per device and kernel instance.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  static std::atomic<uint64_t> attr_set[3] = {0, 0, 0};
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit == 0 || (attr_set[inst].load(std::memory_order_acquire) & bit) == 0) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(F8_SMEM));
    if (e != hipSuccess) return int(e);
    attr_set[inst].fetch_or(bit, std::memory_order_acq_rel);
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const float skip_log2 = skip ? std::log2(skip_threshold) : 0.0f;
  // Grid (query tile, head, segment rank): the longest segments go first.
  const dim3 grid(tiles, unsigned(n_heads), unsigned(n_seqs));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* q4 = static_cast<const u32x4*>(q);
  u32x2* o2 = static_cast<u32x2*>(out);
  const char* kc = static_cast<const char*>(k_ws);
  const char* vc = static_cast<const char*>(v_ws);
  if (skip)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, false>), grid, dim3(F8_NW * 64), F8_SMEM, st, q4, cu, pos, o2, lse,
                       int32_t(n_tokens), n_heads, scale_log2, table, kc, vc, k_sc, v_amax, order, rows_per_head,
                       max_seqlen, skip_log2, skip_stats);
  else if (late)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, true>), grid, dim3(F8_NW * 64), F8_SMEM, st, q4, cu, pos, o2, lse,
                       int32_t(n_tokens), n_heads, scale_log2, table, kc, vc, k_sc, v_amax, order, rows_per_head,
                       max_seqlen, 0.0f, nullptr);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, false>), grid, dim3(F8_NW * 64), F8_SMEM, st, q4, cu, pos, o2, lse,
                       int32_t(n_tokens), n_heads, scale_log2, table, kc, vc, k_sc, v_amax, order, rows_per_head,
                       max_seqlen, 0.0f, nullptr);
  return int(hipGetLastError());
}

}  // namespace h3attn
