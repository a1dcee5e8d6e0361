// HIP kernels for gfx950 (MI355X): the lossy FP8 mode of packed varlen
// attention.
//
// The mode: SAGE-style quantization of the long main DiT attention (vLLM-Omni
// "MiniMax-H3" recipe, "Attention Backends"): queries and keys in FP8 e4m3
// with one scale per query token and one scale per 16 keys, probabilities and
// values in FP8 too.  The attention itself is the one the exact path computes
// ("Day 0 Support for MiniMax-H3 on AMD Instinct GPUs", "The diffusion
// transformer (DiT)"): every token of a packed segment attends to every token
// of its segment, after the multi-axis rotation of queries and keys.
//
// Two kernels:
//   kv_prologue_fp8_kernel  rotates K, quantizes it in 16-key blocks and V in
//                           64-key blocks (power-of-two scales), and packs
//                           both into 64-key tiles, V transposed.  HBM-bound.
//   attn_fwd_fp8_kernel     one workgroup per (256-query tile, head, segment
//                           rank), longest segments first; eight waves, 32
//                           queries per wave; 64-key tiles
//                           through LDS rings; both contractions on
//                           v_mfma_scale_f32_32x32x64_f8f6f4.
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
// Scales.  Per query row: a power-of-two factor folded into the base-2 logit
// coefficient.  Per 16 keys: the 8-bit exponent scale of the A operand (the
// matrix core applies it; the scale of lanes L and L + 32 covers key L % 32).
// Per 64 keys of V: the same, one value for all lanes.  Probabilities are
// formed as p * 2^4 (the shift is folded into the running maximum) so that
// values down to 2^-10 of the maximum stay normal e4m3; row sums add the
// unrounded fp32 probabilities.

#include <atomic>
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
constexpr float P_SHIFT = 4.0f;          // probabilities are stored as p * 2^4
constexpr float LAZY_SUM = 256.0f;       // largest row sum of a tile's scaled probabilities left unrescaled
constexpr int E8M0_ONE = 127;            // 8-bit exponent scale of 2^0

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
// FP8 K/V prologue.  grid = (64-key tiles of the longest segment, segments,
// heads), 256 threads.
// k_ws:   [H][rows][128] e4m3 rotated keys, rows past a segment's end zero.
// v_ws:   [H][rows/64][128][64] e4m3 values, transposed per tile, keys in the
//         order v8_key_byte gives.
// k_sc:   [H][rows/64] one word per tile: byte i = 8-bit exponent scale of
//         keys 16i .. 16i+15.
// v_sc:   [H][rows/64] one word per tile: the exponent scale of its values.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_prologue_fp8_kernel(const u32x4* __restrict__ k,
                                                              const u32x4* __restrict__ v,
                                                              const int32_t* __restrict__ cu,
                                                              const float* __restrict__ pos, int32_t n_heads,
                                                              RopeTable tab, u32x2* __restrict__ k_ws,
                                                              unsigned* __restrict__ v_ws,
                                                              unsigned* __restrict__ k_sc, unsigned* __restrict__ v_sc,
                                                              int32_t* __restrict__ order, int64_t rows_per_head) {
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];
  __shared__ float s_red[4][5];
  const int tile = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  if (tile == 0 && h == 0) write_segment_rank(cu, int(gridDim.y), s, order);  // before any early exit
  const int32_t seg_a = cu[s];
  const int32_t S = cu[s + 1] - seg_a;
  if (tile * KT >= S) return;  // whole block leaves together
  stage_rope_table(tab, s_omega, s_axis);
  __syncthreads();
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t prow = packed_start(seg_a, s) + int64_t(tile) * KT;  // packed row of this tile's key 0
  const int64_t tiles_per_head = rows_per_head / KT;

  // Keys: 1024 chunks of 8 dims, 4 per thread; chunk i of the thread is key
  // (tid >> 4) + 16 i, dims 8 (tid & 15) ..; so chunk i lies in 16-key block i.
  float kf[4][8];
  float amax[5];
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

  // Values: thread owns keys 4 k4 .. 4 k4 + 3 and dims 8 dc .. 8 dc + 7.
  const int k4 = tid & 15, dc = tid >> 4;
  float vf[4][8];
  {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = tile * KT + 4 * k4 + i;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (key < S) val = v[((int64_t(seg_a) + key) * n_heads + h) * CHUNKS_PER_ROW + dc];
      unpack8(val, vf[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(vf[i][e]));
    }
    amax[4] = m;
  }

  // Block maxima: four key blocks and the value tile.
#pragma unroll
  for (int j = 0; j < 5; ++j) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], off));
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 5; ++j) s_red[wv][j] = amax[j];
  }
  __syncthreads();
  int ex[5];
#pragma unroll
  for (int j = 0; j < 5; ++j)
    ex[j] = e4m3_scale_exponent(fmaxf(fmaxf(s_red[0][j], s_red[1][j]), fmaxf(s_red[2][j], s_red[3][j])));
  if (tid == 0) {
    unsigned w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= unsigned(ex[j] + E8M0_ONE) << (8 * j);
    k_sc[int64_t(h) * tiles_per_head + prow / KT] = w;
    v_sc[int64_t(h) * tiles_per_head + prow / KT] = unsigned(ex[4] + E8M0_ONE);
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

  // Quantized values: for each of the thread's 8 dims, its 4 keys are 4
  // consecutive bytes of that dim's row.
  {
    const float down = ldexpf(1.0f, -ex[4]);
    const int pos0 = v8_key_byte(4 * k4);
    unsigned* vt = v_ws + ((int64_t(h) * tiles_per_head + prow / KT) * D * KT) / 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = 8 * dc + j;
      vt[(d * KT + pos0) / 4] =
          pack_e4m3x4(vf[0][j] * down, vf[1][j] * down, vf[2][j] * down, vf[3][j] * down);
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 attention forward, software-pipelined inside each wave.
//
// Iteration t issues, in one branch-free block of 8 MFMA slots,
//     S(t+1) = K(t+1) Q^T      4 MFMAs (two subtiles x two 64-dim halves)
//     O     += V(t-1) P(t-1)   4 MFMAs (one per 32-dim block of O^T)
// and, after every slot, the exponentials of 4 of the 32 probabilities each
// lane forms for tile t.  Consecutive score MFMAs share their query operand
// and the four value MFMAs share the probabilities.
//
// Online softmax in base 2 with a lazily moved running maximum, as in the
// bf16 kernel, here with the probabilities stored as p * 2^4: the running
// value mm is the maximum minus 4, a tile's probabilities stay at most
// 2^4 after a move and are rescaled once a lane's row sum for a tile
// exceeds 256, so every stored probability is below 448.  The queries carry
// the base-2 logit coefficient (scale * log2 e) into their quantization and
// their power-of-two row scale rides on the matrix core's B scale, so a
// score MFMA yields base-2 logits; its accumulator starts at -mm, so a
// probability is one exp2 of the accumulator (no multiply-add per element).
//
// LDS: rings of eight key slots and eight value slots of 8 KiB.  Iteration t
// reads K(t+1) and V(t-1) and issues direct buffer->LDS loads of K(t+5) and
// V(t+3); iterations pair up into epochs that end with one barrier, exactly
// as in the bf16 kernel.
// ---------------------------------------------------------------------------
template <bool SKIP>
__global__ __launch_bounds__(F8_NW * 64, 1) void attn_fwd_fp8_kernel(
    const u32x4* __restrict__ q, const int32_t* __restrict__ cu, const float* __restrict__ pos,
    u32x2* __restrict__ out, float* __restrict__ lse, int32_t n_tokens, int32_t n_heads, float scale_log2,
    RopeTable tab, const char* __restrict__ k_ws, const char* __restrict__ v_ws,
    const unsigned* __restrict__ k_sc, const unsigned* __restrict__ v_sc, const int32_t* __restrict__ order,
    int64_t rows_per_head, float skip_log2, unsigned long long* __restrict__ skip_stats) {
  static_assert(F8_TILE_BYTES / 16 == F8_NW * 64, "one direct load per lane, tile and tensor");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_omega[kPairs];
  __shared__ int s_axis[kPairs];

  // The segment comes from the rank order the K/V prologue wrote.
  const int qt = blockIdx.x, h = blockIdx.y;
  const int s = gridDim.z == 1 ? 0 : order[blockIdx.z];
  const int32_t seg_a = cu[s];
  const int32_t S = cu[s + 1] - seg_a;
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
  const unsigned* vsp = v_sc + int64_t(h) * tiles_per_head + prow / KT;

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

  // Queries: B operand of S^T = K Q^T.  Lane holds query row l32 and, for
  // half ks, dims 64 ks + 32 g .. + 31, rotated in fp32 and multiplied by
  // the base-2 logit coefficient, then scaled by the row's power-of-two
  // factor and rounded to e4m3; qsc is that factor's 8-bit exponent scale,
  // which the score MFMAs apply.
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
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) f[ks][j][e] *= scale_log2;
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
  float mm = -INFINITY, l = 0.0f;
  // Dense instance: score accumulators start at -moff (0 until mm is finite,
  // then mm), so the exponentials need no subtraction.  The Skip-Softmax
  // instance starts them at 0 and subtracts mm in the exponent: the start
  // tuple's sixteen registers would push its loop into scratch reloads.
  constexpr bool START_AT_M = !SKIP;
  float moff = 0.0f;
  float mt = -INFINITY;        // Skip-Softmax: largest base-2 logit of the tiles seen so far
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
  auto mfma_pv = [&](f32x16 acc, i32x8 vf, const i32x8& p, unsigned vsc) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, p, acc, 0, 0, 0, int(vsc), 0, E8M0_ONE);
  };
  // Per-lane exponent scales of K tile t (subtile 0 in byte 0, subtile 1 in
  // byte 2, both in k0; k1 carries the same word), and V tile t's.
  auto kscales = [&](int t, unsigned& k0, unsigned& k1) __attribute__((always_inline)) {
    k0 = ksp[t] >> ksh0;
    k1 = k0;
  };
  auto vscale = [&](int t) __attribute__((always_inline)) { return vsp[t]; };

  // S^T(t) into buffer B, alone (pipeline fill).
  auto qk_alone = [&](auto B, auto SLOT, unsigned k0, unsigned k1) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = START_AT_M ? -moff : 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma_qk(acc, kfrag(SLOT, u, ks), ks, u, u ? k1 : k0);
      sc[b][u] = acc;
    }
  };
  // O^T += V^T(t) P^T(t) from buffer B, alone (pipeline drain).
  auto pv_alone = [&](auto B, auto SLOT, unsigned vsc) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_pv(o[db], vfrag(SLOT, db), pf[b], vsc);
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
  // Unit j (0..7) of tile t's probabilities (scores in buffer B): word j of
  // the lane's 32 bytes, i.e. subtile j / 4, registers 4 (j % 4) .. + 3.
  auto exp_unit = [&](auto B, int j, float (&p)[4]) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sc[b][j >> 2][4 * (j & 3) + i];
      p[i] = __builtin_amdgcn_exp2f(START_AT_M ? x : x - mm);
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
  // After the exponentials of tile t (buffer B): the rare path that moves the
  // running maximum (rescaling O and l, recomputing the tile's probabilities
  // and, when the scores of tile t+1 are already under way (PENDING), moving
  // them to the new start), then the row sum.  The first tile always takes
  // it: mm is still -inf there.
  auto settle = [&](auto B, auto PENDING, i32x8& pw, float rs) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const bool over = !(rs <= LAZY_SUM) || mm == -INFINITY;  // also true for inf and NaN
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      float mx = sc[b][0][0];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[b][u][r]);
      const float tmax = pair_max(mx) + moff;
      const float m_new = fmaxf(mm, tmax - P_SHIFT);
      const float a = __builtin_amdgcn_exp2f(mm - m_new);  // 0 from mm = -inf
      const float shift = moff - m_new;
      mm = m_new;
      if constexpr (START_AT_M) moff = m_new;
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
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[b][j >> 2][4 * (j & 3) + i] + shift);
        pw[j] = int(pack_e4m3x4(p[0], p[1], p[2], p[3]));
        rs += (p[0] + p[1]) + (p[2] + p[3]);
      }
      if constexpr (START_AT_M && decltype(PENDING)::value != 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[1 - b][u][r] += shift;
      }
    }
    l += rs;
  };

  // Iteration t, B = t mod 2 (S(t) in sc[B], P(t-1) in pf[1 - B]), reading
  // K(t+1) from kslot and V(t-1) from vslot: 8 MFMA slots.  Slots 0..3 issue
  // S(t+1) in the order (subtile, half) = (0,0), (1,0), (0,1), (1,1), straight
  // into sc[1 - B] (consecutive pairs share the query operand); slots 4..7
  // issue O += V(t-1) P(t-1), one MFMA per 32-dim block of O^T (all four
  // share the probabilities).  Exponential unit j of tile t follows slot j,
  // then tile t settles.  Two fragment registers alternate, each read one or
  // two slots ahead of its MFMA (the first two at the start).  A scheduling
  // fence after every slot keeps this order.  The Skip-Softmax instance keeps
  // the MFMA order but groups the exponentials: units 0..3 after the score
  // MFMAs and units 4..7 after the value MFMAs, each group under one
  // wave-uniform branch, the value MFMAs under a third (a left-out tile then
  // skips three branches, where interleaving needed twelve).
  auto region = [&](auto B, auto QK, auto PV, bool do_exp, bool pv_live, auto kslot, auto vslot, unsigned k0,
                    unsigned k1, unsigned vsc) __attribute__((always_inline)) {
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
            o[j - 4] = mfma_pv(o[j - 4], fr[j & 1], pf[1 - b], vsc);
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
            if constexpr (START_AT_M) {
              acc = splat16(-moff);  // the first half starts the chain at -moff
            } else {
  #pragma unroll
              for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            }
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
  #pragma unroll
      for (int j = 4; j < 8; ++j) {
        if (do_pv) {
          if (pv_live) o[j - 4] = mfma_pv(o[j - 4], fr[j & 1], pf[1 - b], vsc);
          if (j < 6) fr[j & 1] = vfrag(vslot, j - 2);
        }
        if (do_exp) {
          float p[4];
          exp_unit(ic<b>(), j, p);
          pack_unit(j, p, pw, rs);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (do_exp) {
      settle(ic<b>(), QK, pw, rs);
      pf[b] = pw;
    }
  };

  // Skip-Softmax decision for tile t (scores in buffer B): the wave leaves the
  // tile out when each of its rows has a tile maximum below its running
  // maximum of earlier tiles times the threshold (rows past the segment end
  // do not vote).  Updates the running maximum; returns the uniform decision.
  auto decide = [&](auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    float mx = sc[b][0][0];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[b][u][r]);
    const float tm = pair_max(mx) + moff;
    const bool lets_go = qrow >= S || tm < mt + skip_log2;
    mt = fmaxf(mt, tm);
    return __builtin_amdgcn_ballot_w64(!lets_go) == 0;
  };
  // Iteration t under Skip-Softmax: the exponentials of tile t only if the
  // wave keeps it, the products of tile t-1 only if it kept that one.
  auto region_skip = [&](auto B, auto QK, auto kslot, auto vslot, unsigned k0, unsigned k1, unsigned vsc, bool skip)
      __attribute__((always_inline)) {
    region(B, QK, ic<1>(), !skip, prev_kept, kslot, vslot, k0, k1, vsc);
    prev_kept = !skip;
    ++n_seen;
    n_skipped += skip ? 1u : 0u;
  };

  // Scales for the products iteration t issues: K(t+1) and V(t-1).
  unsigned kq0, kq1, vq;
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
      region_skip(ic<t8 & 1>(), ic<1>(), ic<(t8 + 1) & 7>(), ic<(t8 + 7) & 7>(), kq0, kq1, vq, decide(ic<t8 & 1>()));
    else
      region(ic<t8 & 1>(), ic<1>(), ic<1>(), true, true, ic<(t8 + 1) & 7>(), ic<(t8 + 7) & 7>(), kq0, kq1, vq);
    load_k(min(t + 5, last_t), ic<(t8 + 5) & 7>());
    load_v(min(t + 3, last_t), ic<(t8 + 3) & 7>());
    kscales(min(t + 2, last_t), kq0, kq1);
    vq = vscale(t);
    if ((t8 & 1) == 0) ring_barrier<4>();  // end of an epoch: its loads may stay in flight
  };
  // Last iteration t = last_t >= 1, B = t mod 2: exponentials of tile t and
  // products of tile t-1, then the products of tile t.  It runs once, so its
  // slots are run-time values.
  auto last = [&](auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    mask_tail(ic<b>(), last_t);
    if constexpr (SKIP)
      region_skip(ic<b>(), ic<0>(), 0, (last_t - 1) & 7, kq0, kq1, vq, decide(ic<b>()));
    else
      region(ic<b>(), ic<0>(), ic<1>(), true, true, 0, (last_t - 1) & 7, kq0, kq1, vq);
    const unsigned vl = vscale(last_t);
    ring_barrier<0>();  // V(t) has landed
    __builtin_amdgcn_sched_barrier(0);
    if (prev_kept) pv_alone(ic<b>(), last_t & 7, vl);
  };
  {
    unsigned k0, k1;
    kscales(0, k0, k1);
    qk_alone(ic<0>(), ic<0>(), k0, k1);
  }
  if (n_kt == 1) {
    mask_tail(ic<0>(), 0);
    if constexpr (SKIP) (void)decide(ic<0>());  // the first tile is always kept; this seeds the running maximum
    region(ic<0>(), ic<0>(), ic<0>(), true, true, ic<1>(), ic<7>(), 0u, 0u, 0u);
    const unsigned vl = vscale(0);
    ring_barrier<0>();
    pv_alone(ic<0>(), ic<0>(), vl);
  } else {
    ring_barrier<6>();  // every wave is done with K(0) before its slot is refilled
    kscales(1, kq0, kq1);
    // t = 0: no products of an earlier tile yet; an epoch of its own.
    if constexpr (SKIP) {
      (void)decide(ic<0>());  // the first tile is always kept; this seeds the running maximum
      ++n_seen;
    }
    region(ic<0>(), ic<1>(), ic<0>(), true, true, ic<1>(), ic<7>(), kq0, kq1, 0u);
    load_k(min(5, last_t), ic<5>());
    load_v(min(3, last_t), ic<3>());
    kscales(min(2, last_t), kq0, kq1);
    vq = vscale(0);
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

  // Epilogue: O = O / l, lse = (mm + log2 l) * ln 2 (the 2^4 of the stored
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
    // tiles seen and left out by this wave (if any of its rows exists), for callers that ask
    if (skip_stats != nullptr && lane == 0 && qt * F8_BQ + wave * 32 < S) {
      atomicAdd(&skip_stats[0], (unsigned long long)(n_kt == 1 ? 1u : n_seen));
      atomicAdd(&skip_stats[1], (unsigned long long)n_skipped);
    }
  }
}
}  // namespace

int launch_kv_prologue_fp8(const void* k, const void* v, const int32_t* cu, const float* pos, int32_t n_heads,
                           int32_t n_seqs, int32_t max_seqlen, const RopeTable& table, void* k_ws, void* v_ws,
                           unsigned* k_sc, unsigned* v_sc, int32_t* order, int64_t rows_per_head, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + KT - 1) / KT);
  if (tiles == 0) return 0;
  hipLaunchKernelGGL(kv_prologue_fp8_kernel, dim3(tiles, unsigned(n_seqs), unsigned(n_heads)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
                     cu, pos, n_heads, table, static_cast<u32x2*>(k_ws), static_cast<unsigned*>(v_ws), k_sc, v_sc,
                     order, rows_per_head);
  return int(hipGetLastError());
}

int launch_attention_fp8(const void* q, const int32_t* cu, const float* pos, void* out, float* lse,
                         int64_t n_tokens, int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, float scale,
                         float skip_threshold, const RopeTable& table, const void* k_ws, const void* v_ws,
                         const unsigned* k_sc, const unsigned* v_sc, const int32_t* order, int64_t rows_per_head,
                         unsigned long long* skip_stats, void* stream) {
  const unsigned tiles = unsigned((int64_t(max_seqlen) + F8_BQ - 1) / F8_BQ);
  if (tiles == 0) return 0;
  const bool skip = skip_threshold > 0.0f;
  const void* fn = skip ? reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<true>)
                        : reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<false>);
  // The dynamic LDS limit is raised once per device and kernel instance.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  static std::atomic<uint64_t> attr_set[2] = {0, 0};
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit == 0 || (attr_set[skip].load(std::memory_order_acquire) & bit) == 0) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(F8_SMEM));
    if (e != hipSuccess) return int(e);
    attr_set[skip].fetch_or(bit, std::memory_order_acq_rel);
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const float skip_log2 = skip ? std::log2(skip_threshold) : 0.0f;
  // Grid (query tile, head, segment rank): the longest segments go first.
  const dim3 grid(tiles, unsigned(n_heads), unsigned(n_seqs));
  if (skip)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<true>, grid, dim3(F8_NW * 64), F8_SMEM, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(q), cu, pos, static_cast<u32x2*>(out), lse, int32_t(n_tokens),
                       n_heads, scale_log2, table, static_cast<const char*>(k_ws), static_cast<const char*>(v_ws),
                       k_sc, v_sc, order, rows_per_head, skip_log2, skip_stats);
  else
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<false>, grid, dim3(F8_NW * 64), F8_SMEM,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(q), cu, pos,
                       static_cast<u32x2*>(out), lse, int32_t(n_tokens), n_heads, scale_log2, table,
                       static_cast<const char*>(k_ws), static_cast<const char*>(v_ws), k_sc, v_sc, order,
                       rows_per_head, 0.0f, nullptr);
  return int(hipGetLastError());
}

}  // namespace h3attn
