// Internal declarations shared by the host-side translation units of libh3attn.
#pragma once

#include <cstddef>
#include <cstdint>

#include "h3attn.h"

namespace h3attn {

// Thread-local error detail for h3attn_last_error().
void clear_error();
h3attn_status fail(h3attn_status s, const char* msg);

constexpr int kHeadDim = 128;
constexpr int kPairs = kHeadDim / 2;
constexpr int kKeyTile = 64;  // keys per packed workspace tile

// Longest segment the attention kernels take.  A head's keys (and values) of
// one segment occupy 256 bytes per key of the packed workspace and are read
// through one buffer resource with 32-bit signed offsets; 2^22 keys (1 GiB)
// keeps every offset and the resource's byte count below 2^31 in both modes.
constexpr int32_t kMaxSeqlen = int32_t(1) << 22;

// Rotary table for one call: per rotation pair p (dims 2p, 2p+1), the axis it
// turns with (0 = t, 1 = h, 2 = w) and its angular frequency in float.
struct RopeTable {
  float omega[kPairs];
  int32_t axis[kPairs];
};

// Validates a rotary config for head_dim and fills the table (frequencies
// formed in double, rounded to float).
h3attn_status make_rope_table(const h3attn_rope_cfg* cfg, int32_t head_dim, RopeTable* out);

// Rows of the packed key workspace per head: each segment starts on a
// 64-key boundary, at 64 * (ceil(cu[s] / 64) + s).
inline int64_t packed_rows(int64_t n_tokens, int32_t n_seqs) {
  return int64_t(kKeyTile) * ((n_tokens + kKeyTile - 1) / kKeyTile + n_seqs);
}

// Workspace layout, in this order:
//   keys    fp16 [H][rows][128]     rotated, each 64-key tile block-scaled
//   values  bf16 [H][rows/32][128][32]  transposed 32-key tiles
//   scales  fp32 [H][rows/64]       per-tile factor that undoes the key scaling
//   order   i32  [n_seqs]           segments by length, longest first (256-byte aligned)
struct WorkspaceLayout {
  size_t keys_offset, values_offset, scales_offset, order_offset, total;
};
inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }
inline WorkspaceLayout workspace_layout(int64_t n_tokens, int32_t n_heads, int32_t n_seqs) {
  const size_t rows = size_t(packed_rows(n_tokens, n_seqs));
  const size_t plane = size_t(n_heads) * rows * kHeadDim * 2;
  WorkspaceLayout w;
  w.keys_offset = 0;
  w.values_offset = plane;
  w.scales_offset = 2 * plane;
  w.order_offset = align256(2 * plane + size_t(n_heads) * (rows / kKeyTile) * 4);
  w.total = w.order_offset + size_t(n_seqs) * 4;
  return w;
}

// FP8 workspace layout, in this order (every part 256-byte aligned):
//   keys    e4m3 [H][rows][128]            rotated keys
//   values  e4m3 [H][rows/64][128][64]     transposed 64-key tiles
//   kscale  u32  [H][rows/64]              per tile: 4 exponent scales of 16 keys
//   vamax   u32  [H][n_seqs][128]          per value channel, the largest magnitude over the segment
//   order   i32  [n_seqs]                  segments by length, longest first
struct WorkspaceLayoutFp8 {
  size_t keys_offset, values_offset, kscale_offset, vamax_offset, order_offset, total;
};
inline WorkspaceLayoutFp8 workspace_layout_fp8(int64_t n_tokens, int32_t n_heads, int32_t n_seqs) {
  const size_t rows = size_t(packed_rows(n_tokens, n_seqs));
  const size_t plane = size_t(n_heads) * rows * kHeadDim;
  const size_t kscales = align256(size_t(n_heads) * (rows / kKeyTile) * 4);
  const size_t vamax = align256(size_t(n_heads) * size_t(n_seqs) * kHeadDim * 4);
  WorkspaceLayoutFp8 w;
  w.keys_offset = 0;
  w.values_offset = plane;
  w.kscale_offset = 2 * plane;
  w.vamax_offset = 2 * plane + kscales;
  w.order_offset = 2 * plane + kscales + vamax;
  w.total = w.order_offset + size_t(n_seqs) * 4;
  return w;
}

// Workspace of h3attn_varlen_fwd_noalloc: a file-scope device array of this
// size on each GPU (attn_kernels.hip).  noalloc_workspace() returns its device
// address on the current device (looked up once per device) or a HIP error.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
int noalloc_workspace(void** ptr);

// Kernel launchers (attn_kernels.hip, attn_fp8.hip).  They only enqueue; the caller has
// validated every argument.  Return hipSuccess or the launch error.
int launch_rope_apply(const void* x, void* y, const float* pos, int64_t n_tokens, int32_t n_heads,
                      const RopeTable& table, void* stream);
int launch_kv_prologue(const void* k, const void* v, const int32_t* cu, const float* pos, int64_t n_tokens,
                       int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, const RopeTable& table, void* k_ws,
                       void* v_ws, float* k_scale, int32_t* order, int64_t rows_per_head, void* stream);
int launch_attention(const void* q, const int32_t* cu, const float* pos, void* out, float* lse, int64_t n_tokens,
                     int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, float scale, const RopeTable& table,
                     const void* k_ws, const void* v_ws, const float* k_scale, const int32_t* order,
                     int64_t rows_per_head, void* stream);
int launch_kv_prologue_fp8(const void* k, const void* v, const int32_t* cu, const float* pos, int32_t n_heads,
                           int32_t n_seqs, int32_t max_seqlen, const RopeTable& table, void* k_ws, void* v_ws,
                           unsigned* k_sc, unsigned* v_amax, int32_t* order, int64_t rows_per_head, void* stream);
int launch_attention_fp8(const void* q, const int32_t* cu, const float* pos, void* out, float* lse,
                         int64_t n_tokens, int32_t n_heads, int32_t n_seqs, int32_t max_seqlen, float scale,
                         float skip_threshold, const RopeTable& table, const void* k_ws, const void* v_ws,
                         const unsigned* k_sc, const unsigned* v_amax, const int32_t* order, int64_t rows_per_head,
                         unsigned long long* skip_stats, void* stream);
const char* hip_error_string(int err);

}  // namespace h3attn
