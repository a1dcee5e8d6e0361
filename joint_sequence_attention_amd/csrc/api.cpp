// C ABI of libh3attn: argument checks, status strings, and dispatch to the
// kernel launchers.  Nothing here allocates device memory or synchronizes.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "h3attn.h"
#include "internal.h"

namespace h3attn {

namespace {
thread_local std::string g_last_error;
}

void clear_error() { g_last_error.clear(); }

h3attn_status fail(h3attn_status s, const char* msg) {
  try {
    g_last_error = msg ? msg : "";
  } catch (...) {
  }
  return s;
}

h3attn_status make_rope_table(const h3attn_rope_cfg* cfg, int32_t head_dim, RopeTable* out) {
  if (!cfg) return fail(H3ATTN_ERR_INVALID_ARG, "rope config is NULL");
  if (!(std::isfinite(cfg->theta) && cfg->theta > 0.0)) return fail(H3ATTN_ERR_INVALID_ARG, "rope theta must be finite and > 0");
  const int32_t w[3] = {cfg->dim_t, cfg->dim_h, cfg->dim_w};
  int64_t sum = 0;
  for (int a = 0; a < 3; ++a) {
    if (w[a] < 0 || (w[a] & 1)) return fail(H3ATTN_ERR_UNSUPPORTED, "rope axis widths must be even and >= 0");
    sum += w[a];
  }
  if (sum != head_dim) return fail(H3ATTN_ERR_UNSUPPORTED, "rope axis widths must add up to head_dim");
  int p = 0;
  for (int a = 0; a < 3; ++a) {
    for (int j = 0; j < w[a] / 2; ++j, ++p) {
      out->axis[p] = a;
      out->omega[p] = static_cast<float>(std::pow(cfg->theta, -2.0 * j / double(w[a])));
    }
  }
  return H3ATTN_OK;
}

namespace {

h3attn_status check_common(int64_t n_tokens, int32_t n_heads, int32_t head_dim) {
  if (n_tokens < 0) return fail(H3ATTN_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens > INT32_MAX) return fail(H3ATTN_ERR_UNSUPPORTED, "n_tokens above INT32_MAX");
  if (n_heads < 1) return fail(H3ATTN_ERR_INVALID_ARG, "n_heads must be >= 1");
  if (n_heads > 65535) return fail(H3ATTN_ERR_UNSUPPORTED, "n_heads above 65535");
  if (head_dim != kHeadDim) return fail(H3ATTN_ERR_UNSUPPORTED, "only head_dim = 128 is supported");
  return H3ATTN_OK;
}

h3attn_status check_varlen(int64_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_seqs, int32_t max_seqlen) {
  h3attn_status st = check_common(n_tokens, n_heads, head_dim);
  if (st != H3ATTN_OK) return st;
  if (n_seqs < 1) return fail(H3ATTN_ERR_INVALID_ARG, "n_seqs must be >= 1");
  if (n_seqs > 65535) return fail(H3ATTN_ERR_UNSUPPORTED, "n_seqs above 65535");
  if (max_seqlen < 0) return fail(H3ATTN_ERR_INVALID_ARG, "max_seqlen must be >= 0");
  if (max_seqlen > n_tokens) return fail(H3ATTN_ERR_INVALID_ARG, "max_seqlen exceeds n_tokens");
  if (max_seqlen > kMaxSeqlen) return fail(H3ATTN_ERR_UNSUPPORTED, "max_seqlen above 4,194,304 (2^22) tokens");
  return H3ATTN_OK;
}

size_t workspace_bytes_for(int64_t n_tokens, int32_t n_heads, int32_t n_seqs) {
  return workspace_layout(n_tokens, n_heads, n_seqs).total;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

h3attn_status check_workspace_size(const void* ws, size_t bytes, size_t need, const char* too_small) {
  if (!ws) return fail(H3ATTN_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(H3ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < need) return fail(H3ATTN_ERR_WORKSPACE, too_small);
  return H3ATTN_OK;
}

h3attn_status check_workspace(const void* ws, size_t bytes, int64_t n_tokens, int32_t n_heads, int32_t n_seqs) {
  return check_workspace_size(ws, bytes, workspace_bytes_for(n_tokens, n_heads, n_seqs),
                              "workspace smaller than h3attn_varlen_fwd_workspace_size");
}

h3attn_status check_workspace_fp8(const void* ws, size_t bytes, int64_t n_tokens, int32_t n_heads, int32_t n_seqs) {
  return check_workspace_size(ws, bytes, workspace_layout_fp8(n_tokens, n_heads, n_seqs).total,
                              "workspace smaller than h3attn_varlen_fwd_fp8_workspace_size");
}

// out and lse against q (and k, v when given), each other and the workspace.
h3attn_status check_outputs(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* ws, size_t ws_bytes, int64_t n_tokens, int32_t n_heads, int32_t head_dim) {
  const size_t nb = size_t(n_tokens) * n_heads * head_dim * 2;
  const size_t nl = size_t(n_tokens) * n_heads * 4;
  const void* ins[3] = {q, k, v};
  for (const void* in : ins) {
    if (!in) continue;
    if (overlaps(out, nb, in, nb) || overlaps(lse, nl, in, nb) || overlaps(ws, ws_bytes, in, nb))
      return fail(H3ATTN_ERR_INVALID_ARG, "out, lse and workspace must not overlap the inputs");
  }
  if (overlaps(out, nb, lse, nl) || overlaps(out, nb, ws, ws_bytes) || overlaps(lse, nl, ws, ws_bytes))
    return fail(H3ATTN_ERR_INVALID_ARG, "out, lse and workspace must not overlap each other");
  return H3ATTN_OK;
}

h3attn_status hip_status(int err) {
  if (err == 0) return H3ATTN_OK;
  return fail(H3ATTN_ERR_HIP, hip_error_string(err));
}

}  // namespace
}  // namespace h3attn

using namespace h3attn;

extern "C" {

const char* h3attn_status_string(h3attn_status s) {
  switch (s) {
    case H3ATTN_OK: return "H3ATTN_OK";
    case H3ATTN_ERR_INVALID_ARG: return "H3ATTN_ERR_INVALID_ARG";
    case H3ATTN_ERR_UNSUPPORTED: return "H3ATTN_ERR_UNSUPPORTED";
    case H3ATTN_ERR_WORKSPACE: return "H3ATTN_ERR_WORKSPACE";
    case H3ATTN_ERR_HIP: return "H3ATTN_ERR_HIP";
  }
  return "H3ATTN_UNKNOWN_STATUS";
}

const char* h3attn_last_error(void) { return g_last_error.c_str(); }

int32_t h3attn_abi_version(void) { return H3ATTN_ABI_VERSION; }

size_t h3attn_varlen_fwd_workspace_size(int64_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_seqs) {
  if (n_tokens < 0 || n_heads < 1 || head_dim != kHeadDim || n_seqs < 1) return 0;
  return workspace_bytes_for(n_tokens, n_heads, n_seqs);
}

h3attn_status h3attn_rope_apply(const void* x, void* y, const float* pos_thw, int64_t n_tokens, int32_t n_heads,
                                int32_t head_dim, const h3attn_rope_cfg* rope, void* stream) {
  try {
    clear_error();
    h3attn_status st = check_common(n_tokens, n_heads, head_dim);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (n_tokens == 0) return H3ATTN_OK;
    if (!x || !y || !pos_thw) return fail(H3ATTN_ERR_INVALID_ARG, "x, y and pos_thw must be non-NULL");
    const size_t nb = size_t(n_tokens) * n_heads * head_dim * 2;
    if (x != y && overlaps(x, nb, y, nb)) return fail(H3ATTN_ERR_INVALID_ARG, "y must equal x or not overlap it");
    if (overlaps(pos_thw, size_t(n_tokens) * 12, y, nb)) return fail(H3ATTN_ERR_INVALID_ARG, "y overlaps pos_thw");
    return hip_status(launch_rope_apply(x, y, pos_thw, n_tokens, n_heads, table, stream));
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_rope_apply");
  }
}

h3attn_status h3attn_varlen_kv_prologue(const void* k, const void* v, const int32_t* cu_seqlens,
                                        const float* pos_thw, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                        int32_t n_seqs, int32_t max_seqlen, const h3attn_rope_cfg* rope,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  try {
    clear_error();
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (n_tokens == 0) return H3ATTN_OK;
    if (!k || !v || !cu_seqlens || !pos_thw) return fail(H3ATTN_ERR_INVALID_ARG, "k, v, cu_seqlens and pos_thw must be non-NULL");
    st = check_workspace(workspace, workspace_bytes, n_tokens, n_heads, n_seqs);
    if (st != H3ATTN_OK) return st;
    const int64_t rows = packed_rows(n_tokens, n_seqs);
    const WorkspaceLayout wl = workspace_layout(n_tokens, n_heads, n_seqs);
    char* ws = static_cast<char*>(workspace);
    return hip_status(launch_kv_prologue(k, v, cu_seqlens, pos_thw, n_tokens, n_heads, n_seqs, max_seqlen, table,
                                         ws + wl.keys_offset, ws + wl.values_offset,
                                         reinterpret_cast<float*>(ws + wl.scales_offset),
                                         reinterpret_cast<int32_t*>(ws + wl.order_offset), rows, stream));
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_kv_prologue");
  }
}

h3attn_status h3attn_varlen_attention(const void* q, const int32_t* cu_seqlens, const float* pos_thw, void* out,
                                      float* lse, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                      int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                      const h3attn_rope_cfg* rope, const void* workspace, size_t workspace_bytes,
                                      void* stream) {
  try {
    clear_error();
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (!std::isfinite(softmax_scale)) return fail(H3ATTN_ERR_INVALID_ARG, "softmax_scale must be finite");
    if (n_tokens == 0) return H3ATTN_OK;
    if (!q || !cu_seqlens || !pos_thw || !out || !lse)
      return fail(H3ATTN_ERR_INVALID_ARG, "q, cu_seqlens, pos_thw, out and lse must be non-NULL");
    st = check_workspace(workspace, workspace_bytes, n_tokens, n_heads, n_seqs);
    if (st != H3ATTN_OK) return st;
    const size_t nb = size_t(n_tokens) * n_heads * head_dim * 2;
    const size_t nl = size_t(n_tokens) * n_heads * 4;
    if (overlaps(out, nb, q, nb) || overlaps(lse, nl, q, nb) || overlaps(out, nb, lse, nl) ||
        overlaps(out, nb, workspace, workspace_bytes) || overlaps(lse, nl, workspace, workspace_bytes))
      return fail(H3ATTN_ERR_INVALID_ARG, "out and lse must not overlap q, each other or the workspace");
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(float(head_dim));
    const int64_t rows = packed_rows(n_tokens, n_seqs);
    const WorkspaceLayout wl = workspace_layout(n_tokens, n_heads, n_seqs);
    const char* ws = static_cast<const char*>(workspace);
    return hip_status(launch_attention(q, cu_seqlens, pos_thw, out, lse, n_tokens, n_heads, n_seqs, max_seqlen, scale,
                                       table, ws + wl.keys_offset, ws + wl.values_offset,
                                       reinterpret_cast<const float*>(ws + wl.scales_offset),
                                       reinterpret_cast<const int32_t*>(ws + wl.order_offset), rows, stream));
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_attention");
  }
}

h3attn_status h3attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                const float* pos_thw, void* out, float* lse, int64_t n_tokens, int32_t n_heads,
                                int32_t head_dim, int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                const h3attn_rope_cfg* rope, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    clear_error();
    // Check everything both stages need before launching the first one.
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (!std::isfinite(softmax_scale)) return fail(H3ATTN_ERR_INVALID_ARG, "softmax_scale must be finite");
    if (n_tokens == 0) return H3ATTN_OK;
    if (!q || !k || !v || !cu_seqlens || !pos_thw || !out || !lse)
      return fail(H3ATTN_ERR_INVALID_ARG, "q, k, v, cu_seqlens, pos_thw, out and lse must be non-NULL");
    st = check_workspace(workspace, workspace_bytes, n_tokens, n_heads, n_seqs);
    if (st != H3ATTN_OK) return st;
    const size_t nb = size_t(n_tokens) * n_heads * head_dim * 2;
    const size_t nl = size_t(n_tokens) * n_heads * 4;
    const void* ins[3] = {q, k, v};
    for (const void* in : ins) {
      if (overlaps(out, nb, in, nb) || overlaps(lse, nl, in, nb) || overlaps(workspace, workspace_bytes, in, nb))
        return fail(H3ATTN_ERR_INVALID_ARG, "out, lse and workspace must not overlap q, k or v");
    }
    if (overlaps(out, nb, lse, nl) || overlaps(out, nb, workspace, workspace_bytes) ||
        overlaps(lse, nl, workspace, workspace_bytes))
      return fail(H3ATTN_ERR_INVALID_ARG, "out, lse and workspace must not overlap each other");
    st = h3attn_varlen_kv_prologue(k, v, cu_seqlens, pos_thw, n_tokens, n_heads, head_dim, n_seqs, max_seqlen, rope,
                                   workspace, workspace_bytes, stream);
    if (st != H3ATTN_OK) return st;
    return h3attn_varlen_attention(q, cu_seqlens, pos_thw, out, lse, n_tokens, n_heads, head_dim, n_seqs, max_seqlen,
                                   softmax_scale, rope, workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_fwd");
  }
}

h3attn_status h3attn_varlen_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                        const float* pos_thw, void* out, float* lse, int64_t n_tokens,
                                        int32_t n_heads, int32_t head_dim, int32_t n_seqs, int32_t max_seqlen,
                                        float softmax_scale, const h3attn_rope_cfg* rope, void* stream) {
  try {
    clear_error();
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (!std::isfinite(softmax_scale)) return fail(H3ATTN_ERR_INVALID_ARG, "softmax_scale must be finite");
    if (n_tokens == 0) return H3ATTN_OK;
    if (workspace_bytes_for(n_tokens, n_heads, n_seqs) > kNoAllocScratchBytes)
      return fail(H3ATTN_ERR_UNSUPPORTED,
                  "the call needs more workspace than the library's 128 MiB array "
                  "(h3attn_varlen_fwd_workspace_size > 134217728): use h3attn_varlen_fwd");
    void* ws = nullptr;
    const int e = noalloc_workspace(&ws);
    if (e != 0) return hip_status(e);
    return h3attn_varlen_fwd(q, k, v, cu_seqlens, pos_thw, out, lse, n_tokens, n_heads, head_dim, n_seqs, max_seqlen,
                             softmax_scale, rope, ws, kNoAllocScratchBytes, stream);
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_fwd_noalloc");
  }
}

size_t h3attn_varlen_fwd_fp8_workspace_size(int64_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_seqs) {
  if (n_tokens < 0 || n_heads < 1 || head_dim != kHeadDim || n_seqs < 1) return 0;
  return workspace_layout_fp8(n_tokens, n_heads, n_seqs).total;
}

h3attn_status h3attn_varlen_kv_prologue_fp8(const void* k, const void* v, const int32_t* cu_seqlens,
                                            const float* pos_thw, int64_t n_tokens, int32_t n_heads,
                                            int32_t head_dim, int32_t n_seqs, int32_t max_seqlen,
                                            const h3attn_rope_cfg* rope, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  try {
    clear_error();
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (n_tokens == 0) return H3ATTN_OK;
    if (!k || !v || !cu_seqlens || !pos_thw) return fail(H3ATTN_ERR_INVALID_ARG, "k, v, cu_seqlens and pos_thw must be non-NULL");
    st = check_workspace_fp8(workspace, workspace_bytes, n_tokens, n_heads, n_seqs);
    if (st != H3ATTN_OK) return st;
    const size_t nb = size_t(n_tokens) * n_heads * head_dim * 2;
    if (overlaps(workspace, workspace_bytes, k, nb) || overlaps(workspace, workspace_bytes, v, nb))
      return fail(H3ATTN_ERR_INVALID_ARG, "workspace must not overlap k or v");
    const int64_t rows = packed_rows(n_tokens, n_seqs);
    const WorkspaceLayoutFp8 wl = workspace_layout_fp8(n_tokens, n_heads, n_seqs);
    char* ws = static_cast<char*>(workspace);
    return hip_status(launch_kv_prologue_fp8(k, v, cu_seqlens, pos_thw, n_heads, n_seqs, max_seqlen, table,
                                             ws + wl.keys_offset, ws + wl.values_offset,
                                             reinterpret_cast<unsigned*>(ws + wl.kscale_offset),
                                             reinterpret_cast<unsigned*>(ws + wl.vamax_offset),
                                             reinterpret_cast<int32_t*>(ws + wl.order_offset), rows, stream));
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_kv_prologue_fp8");
  }
}

h3attn_status h3attn_varlen_attention_fp8(const void* q, const int32_t* cu_seqlens, const float* pos_thw, void* out,
                                          float* lse, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                          int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                          float skip_threshold, const h3attn_rope_cfg* rope, const void* workspace,
                                          size_t workspace_bytes, uint64_t* skip_stats, void* stream) {
  try {
    clear_error();
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (!std::isfinite(softmax_scale)) return fail(H3ATTN_ERR_INVALID_ARG, "softmax_scale must be finite");
    if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f))
      return fail(H3ATTN_ERR_INVALID_ARG, "skip_threshold must lie in [0, 1)");
    if (n_tokens == 0) return H3ATTN_OK;
    if (!q || !cu_seqlens || !pos_thw || !out || !lse)
      return fail(H3ATTN_ERR_INVALID_ARG, "q, cu_seqlens, pos_thw, out and lse must be non-NULL");
    st = check_workspace_fp8(workspace, workspace_bytes, n_tokens, n_heads, n_seqs);
    if (st != H3ATTN_OK) return st;
    st = check_outputs(q, nullptr, nullptr, out, lse, workspace, workspace_bytes, n_tokens, n_heads, head_dim);
    if (st != H3ATTN_OK) return st;
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(float(head_dim));
    const int64_t rows = packed_rows(n_tokens, n_seqs);
    const WorkspaceLayoutFp8 wl = workspace_layout_fp8(n_tokens, n_heads, n_seqs);
    const char* ws = static_cast<const char*>(workspace);
    return hip_status(launch_attention_fp8(q, cu_seqlens, pos_thw, out, lse, n_tokens, n_heads, n_seqs, max_seqlen,
                                           scale, skip_threshold, table, ws + wl.keys_offset, ws + wl.values_offset,
                                           reinterpret_cast<const unsigned*>(ws + wl.kscale_offset),
                                           reinterpret_cast<const unsigned*>(ws + wl.vamax_offset),
                                           reinterpret_cast<const int32_t*>(ws + wl.order_offset), rows,
                                           reinterpret_cast<unsigned long long*>(skip_stats), stream));
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_attention_fp8");
  }
}

h3attn_status h3attn_varlen_fwd_fp8(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                    const float* pos_thw, void* out, float* lse, int64_t n_tokens, int32_t n_heads,
                                    int32_t head_dim, int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                    float skip_threshold, const h3attn_rope_cfg* rope, void* workspace,
                                    size_t workspace_bytes, uint64_t* skip_stats, void* stream) {
  try {
    clear_error();
    // Check everything both stages need before launching the first one.
    h3attn_status st = check_varlen(n_tokens, n_heads, head_dim, n_seqs, max_seqlen);
    if (st != H3ATTN_OK) return st;
    RopeTable table;
    st = make_rope_table(rope, head_dim, &table);
    if (st != H3ATTN_OK) return st;
    if (!std::isfinite(softmax_scale)) return fail(H3ATTN_ERR_INVALID_ARG, "softmax_scale must be finite");
    if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f))
      return fail(H3ATTN_ERR_INVALID_ARG, "skip_threshold must lie in [0, 1)");
    if (n_tokens == 0) return H3ATTN_OK;
    if (!q || !k || !v || !cu_seqlens || !pos_thw || !out || !lse)
      return fail(H3ATTN_ERR_INVALID_ARG, "q, k, v, cu_seqlens, pos_thw, out and lse must be non-NULL");
    st = check_workspace_fp8(workspace, workspace_bytes, n_tokens, n_heads, n_seqs);
    if (st != H3ATTN_OK) return st;
    st = check_outputs(q, k, v, out, lse, workspace, workspace_bytes, n_tokens, n_heads, head_dim);
    if (st != H3ATTN_OK) return st;
    st = h3attn_varlen_kv_prologue_fp8(k, v, cu_seqlens, pos_thw, n_tokens, n_heads, head_dim, n_seqs, max_seqlen,
                                       rope, workspace, workspace_bytes, stream);
    if (st != H3ATTN_OK) return st;
    return h3attn_varlen_attention_fp8(q, cu_seqlens, pos_thw, out, lse, n_tokens, n_heads, head_dim, n_seqs,
                                       max_seqlen, softmax_scale, skip_threshold, rope, workspace, workspace_bytes,
                                       skip_stats, stream);
  } catch (...) {
    return fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_varlen_fwd_fp8");
  }
}

h3attn_status h3attn_skip_gate(float skip_threshold, float disabled_until_timestep, float sigma,
                               float* threshold_out) {
  clear_error();
  if (!threshold_out) return fail(H3ATTN_ERR_INVALID_ARG, "threshold_out is NULL");
  if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f))
    return fail(H3ATTN_ERR_INVALID_ARG, "skip_threshold must lie in [0, 1)");
  if (std::isnan(disabled_until_timestep)) return fail(H3ATTN_ERR_INVALID_ARG, "disabled_until_timestep is NaN");
  if (std::isnan(sigma)) return fail(H3ATTN_ERR_INVALID_ARG, "sigma is NaN");
  // dense while the step's noise level is above the cutoff
  *threshold_out = sigma > disabled_until_timestep ? 0.0f : skip_threshold;
  return H3ATTN_OK;
}

}  // extern "C"
