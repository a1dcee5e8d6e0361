// Device-side helpers shared by the gfx950 kernels of libh3attn: vector
// types, bf16 / fp16 / fp8 packing, the multi-axis rotation, wave-pair
// reductions and the LDS-ring barrier.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace h3attn {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int D = kHeadDim;
constexpr int CHUNKS_PER_ROW = D / 8;  // 16-byte bf16 chunks per 128-dim row

template <int N>
using ic = std::integral_constant<int, N>;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float bf_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even), low half first.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(v[i]);
    f[2 * i + 1] = bf_hi(v[i]);
  }
}

// Four floats -> four e4m3 bytes (OCP "fn" encoding, round to nearest even),
// first value in the lowest byte.  Every input must be finite with magnitude
// below 464; larger values have no finite e4m3 encoding.
__device__ __forceinline__ unsigned pack_e4m3x4(float a, float b, float c, float d) {
  unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Power-of-two block scale for e4m3: the smallest e with amax * 2^-e <= 448
// (the largest finite e4m3 value), limited to [-127, 127]; 0 when amax is 0
// or not finite.  Returns e; down = 2^-e is the factor applied before
// rounding.
__device__ __forceinline__ int e4m3_scale_exponent(float amax) {
  if (!(amax > 0.0f) || !__builtin_isfinite(amax)) return 0;
  int E;
  const float f = frexpf(amax, &E);  // amax = f * 2^E, f in [0.5, 1)
  const int e = f <= 0.875f ? E - 9 : E - 8;  // f * 512 <= 448, else f * 256 in (224, 256)
  return max(-127, min(127, e));
}

// Sixteen copies of x, built from 64-bit halves so that the compiler can
// materialize them with 64-bit moves.
__device__ __forceinline__ f32x16 splat16(float x) {
  typedef __attribute__((__vector_size__(8 * sizeof(unsigned long long)))) unsigned long long u64x8;
  const unsigned long long w = (unsigned long long)__float_as_uint(x) * 0x100000001ull;
  u64x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = w;
  return __builtin_bit_cast(f32x16, z);
}

// Max / sum with the partner lane (L ^ 32).
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

// Rotation of 4 consecutive pairs (dims 2*pair0 .. 2*pair0+7) in fp32.  Pair
// p turns by phi = pos[axis(p)] * omega(p); (x0, x1) -> (x0 cos - x1 sin,
// x0 sin + x1 cos).
struct Rot4 {
  float sn[4], cs[4];
};

__device__ __forceinline__ Rot4 rope_angles4(int pair0, const float* s_omega, const int* s_axis, float pt, float ph,
                                             float pw) {
  Rot4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = pair0 + i;
    const int ax = s_axis[p];
    const float ps = ax == 0 ? pt : (ax == 1 ? ph : pw);
    const float phi = ps * s_omega[p];
    sincosf(phi, &r.sn[i], &r.cs[i]);
  }
  return r;
}

__device__ __forceinline__ void rope_turn4(float (&x)[8], const Rot4& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = fmaf(x0, r.cs[i], -(x1 * r.sn[i]));
    x[2 * i + 1] = fmaf(x0, r.sn[i], x1 * r.cs[i]);
  }
}

// A token at position (0, 0, 0) turns every pair by angle 0, the identity
// (sin 0 = 0 and cos 0 = 1 are exact), so its rows may be left as they are.
// The test is taken per wave: when every active lane holds such a token (a
// wave of text rows) the angles are skipped with one scalar branch; a wave
// with any other token turns all its lanes, which changes no value of a
// lane at the origin except the sign of a zero.
__device__ __forceinline__ bool at_origin(float pt, float ph, float pw) {
  return pt == 0.0f && ph == 0.0f && pw == 0.0f;
}

__device__ __forceinline__ bool wave_at_origin(float pt, float ph, float pw) {
  return __builtin_amdgcn_ballot_w64(!at_origin(pt, ph, pw)) == 0;
}

__device__ __forceinline__ void rope8(float (&x)[8], int pair0, const float* s_omega, const int* s_axis,
                                      float pt, float ph, float pw) {
  if (wave_at_origin(pt, ph, pw)) return;
  rope_turn4(x, rope_angles4(pair0, s_omega, s_axis, pt, ph, pw));
}

__device__ __forceinline__ void stage_rope_table(const RopeTable& tab, float* s_omega, int* s_axis) {
  if (threadIdx.x < kPairs) {
    s_omega[threadIdx.x] = tab.omega[threadIdx.x];
    s_axis[threadIdx.x] = tab.axis[threadIdx.x];
  }
}

// Called by every thread of one workgroup per segment s (a block-uniform
// condition): writes order[rank] = s, where segments rank by length, longest
// first, equal lengths by index.  That key is a strict total order, so order
// becomes a permutation of 0 .. n_seqs-1 whatever cu holds.  The attention
// grid walks it so that the longest segments' workgroups start first and the
// grid ends on short ones.
__device__ __forceinline__ void write_segment_rank(const int32_t* cu, int n_seqs, int s, int32_t* order) {
  __shared__ int s_before;
  if (threadIdx.x == 0) s_before = 0;
  __syncthreads();
  const int32_t len = cu[s + 1] - cu[s];
  int before = 0;
  for (int j = threadIdx.x; j < n_seqs; j += blockDim.x) {
    const int32_t lj = cu[j + 1] - cu[j];
    before += (lj > len || (lj == len && j < s)) ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) before += __shfl_xor(before, off);
  if ((threadIdx.x & 63) == 0 && before != 0) atomicAdd(&s_before, before);
  __syncthreads();
  if (threadIdx.x == 0) order[s_before] = s;
}

// Row of the packed workspace where segment s's first key lives: every
// segment starts on a 64-key boundary.
__device__ __forceinline__ int64_t packed_start(int32_t seg_begin, int32_t s) {
  return int64_t(kKeyTile) * ((int64_t(seg_begin) + kKeyTile - 1) / kKeyTile + s);
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then meet the other waves.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Pins a value to the point where this is called: the compiler may neither
// compute it later nor fold it into later code.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(unsigned& x) { asm volatile("" : "+v"(x)); }

}  // namespace dev
}  // namespace h3attn
