// Host layout builder: items in reference order -> cu_seqlens + (t, h, w) positions.
//
// Positions follow the shared audio/video rotary clock: references are read
// in order and each advances the clock ("minimax-h3-reference" README,
// "References"); each packed request is its own attention document with its
// own clock (vLLM-Omni "MiniMax-H3" recipe, "Step execution and continuous
// batching"); positions are formed in double and rounded to float for device
// arithmetic ("MiniMax H3 on Moore Threads MUSA", "MUSA validation").  A clock
// item moves the clock with no tokens, which places a long video's
// continuation chunk at its global time (same recipe, "Long video and driving
// audio"); a text item is a run of rows at position 0, the token refiner's
// short attention path (same recipe, "Attention Backends").

#include <cmath>
#include <cstdint>
#include <limits>

#include "h3attn.h"
#include "internal.h"

namespace {

// Nearest integer, ties to even (IEEE default): nearbyint under the default
// rounding mode does exactly this.
double round_half_even(double x) { return std::nearbyint(x); }

h3attn_status check_item(const h3attn_item& it) {
  if (it.kind == H3ATTN_ITEM_VISUAL) {
    if (it.T < 1 || it.H < 1 || it.W < 1) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "visual item needs T, H, W >= 1");
    return H3ATTN_OK;
  }
  if (it.kind == H3ATTN_ITEM_AUDIO) {
    if (it.n_audio < 0) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "audio item needs n_audio >= 0");
    if (!(std::isfinite(it.span) && it.span >= 0.0))
      return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "audio span must be finite and >= 0");
    if (it.rule != H3ATTN_AUDIO_LINEAR && it.rule != H3ATTN_AUDIO_ROUND_HALF_EVEN)
      return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "unknown audio position rule");
    if (it.attached != 0 && it.attached != 1) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "attached must be 0 or 1");
    return H3ATTN_OK;
  }
  if (it.kind == H3ATTN_ITEM_CLOCK) {
    if (!(std::isfinite(it.span) && it.span >= 0.0))
      return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "clock span must be finite and >= 0");
    return H3ATTN_OK;
  }
  if (it.kind == H3ATTN_ITEM_TEXT) {
    if (it.n_audio < 0) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "text item needs n_audio (its rows) >= 0");
    return H3ATTN_OK;
  }
  return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "unknown item kind");
}

int64_t item_rows(const h3attn_item& it) {
  if (it.kind == H3ATTN_ITEM_VISUAL) return int64_t(it.T) * it.H * it.W;
  if (it.kind == H3ATTN_ITEM_CLOCK) return 0;
  return it.n_audio;  // audio and text rows
}

}  // namespace

extern "C" h3attn_status h3attn_build_layout(const h3attn_item* items, const int32_t* items_per_seq, int32_t n_seqs,
                                             int32_t* cu_seqlens, float* pos_thw, int64_t pos_capacity,
                                             int64_t* n_tokens) {
  try {
    h3attn::clear_error();
    if (!n_tokens) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "n_tokens is NULL");
    if (n_seqs < 1) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "n_seqs must be >= 1");
    if (!items_per_seq) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "items_per_seq is NULL");
    int64_t n_items = 0;
    for (int32_t s = 0; s < n_seqs; ++s) {
      if (items_per_seq[s] < 0) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "items_per_seq entries must be >= 0");
      n_items += items_per_seq[s];
    }
    if (n_items > 0 && !items) return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "items is NULL");

    // Pass 1: validate and count.
    int64_t total = 0;
    {
      int64_t idx = 0;
      for (int32_t s = 0; s < n_seqs; ++s) {
        bool have_visual = false;
        for (int32_t i = 0; i < items_per_seq[s]; ++i, ++idx) {
          const h3attn_item& it = items[idx];
          h3attn_status st = check_item(it);
          if (st != H3ATTN_OK) return st;
          if (it.kind == H3ATTN_ITEM_AUDIO && it.attached && !have_visual)
            return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "attached audio needs a visual item before it in its segment");
          if (it.kind == H3ATTN_ITEM_VISUAL) have_visual = true;
          total += item_rows(it);
          if (total > std::numeric_limits<int32_t>::max())
            return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "layout exceeds INT32_MAX tokens");
        }
      }
    }
    *n_tokens = total;
    if (pos_thw && pos_capacity < total)
      return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "pos_capacity is smaller than the token count");

    // Pass 2: prefix sums and positions.
    int64_t row = 0, idx = 0;
    if (cu_seqlens) cu_seqlens[0] = 0;
    for (int32_t s = 0; s < n_seqs; ++s) {
      double clock = 0.0, last_visual_start = 0.0;
      for (int32_t i = 0; i < items_per_seq[s]; ++i, ++idx) {
        const h3attn_item& it = items[idx];
        if (it.kind == H3ATTN_ITEM_VISUAL) {
          if (pos_thw) {
            for (int32_t t = 0; t < it.T; ++t)
              for (int32_t h = 0; h < it.H; ++h)
                for (int32_t w = 0; w < it.W; ++w) {
                  float* p = pos_thw + 3 * (row + (int64_t(t) * it.H + h) * it.W + w);
                  p[0] = static_cast<float>(clock + t);
                  p[1] = static_cast<float>(h);
                  p[2] = static_cast<float>(w);
                }
          }
          last_visual_start = clock;
          clock += it.T;
        } else if (it.kind == H3ATTN_ITEM_CLOCK) {
          clock += it.span;
        } else if (it.kind == H3ATTN_ITEM_TEXT) {
          if (pos_thw)
            for (int64_t k = 0; k < 3 * int64_t(it.n_audio); ++k) pos_thw[3 * row + k] = 0.0f;
        } else {
          const double start = it.attached ? last_visual_start : clock;
          if (pos_thw) {
            for (int32_t a = 0; a < it.n_audio; ++a) {
              double off = double(a) * it.span / double(it.n_audio);
              if (it.rule == H3ATTN_AUDIO_ROUND_HALF_EVEN) off = round_half_even(off);
              float* p = pos_thw + 3 * (row + a);
              p[0] = static_cast<float>(start + off);
              p[1] = 0.0f;
              p[2] = 0.0f;
            }
          }
          if (!it.attached) clock += it.span;
        }
        row += item_rows(it);
      }
      if (cu_seqlens) cu_seqlens[s + 1] = static_cast<int32_t>(row);
    }
    return H3ATTN_OK;
  } catch (...) {
    return h3attn::fail(H3ATTN_ERR_INVALID_ARG, "unexpected host exception in h3attn_build_layout");
  }
}
