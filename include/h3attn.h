/*
 * h3attn -- joint audio/video attention for MI355X (gfx950).
 *
 * One hot path: multi-axis rotary position embedding on one shared
 * audio/video clock, followed by packed variable-length flash-attention
 * forward (bf16 in, fp32 accumulate), as computed inside the MiniMax-H3
 * flow-matching DiT for every block.
 *
 * Where the operation is defined:
 *   - The DiT flattens the video latent and the audio latent into one long
 *     token sequence and attends over all of it, with rotary (RoPE) position
 *     encoding and 56 heads of width 128 ("Day 0 Support for MiniMax-H3 on
 *     AMD Instinct GPUs", section "The diffusion transformer (DiT)" and its
 *     property table).
 *   - Co-batched requests are packed into one sequence that keeps one
 *     attention document per request; the backend that serves this is
 *     packed variable-length attention (vLLM-Omni "MiniMax-H3" recipe,
 *     sections "Step execution and continuous batching" and "AMD ROCm
 *     (gfx942 / gfx950)").
 *   - References are read in a fixed order that advances the shared
 *     audio/video rotary clock, and they are packed in front of the
 *     generated rows ("minimax-h3-reference" Space README, sections
 *     "References" and "AoTI-compiled blocks").
 *   - Position metadata is formed in FP64 on the host and cast to FP32
 *     before device arithmetic; attention must return finite BF16 output
 *     ("MiniMax H3 on Moore Threads MUSA", section "MUSA validation").
 *
 * Conventions shared by every entry point:
 *   - Device pointers are plain HIP device addresses; the caller allocates
 *     and owns every buffer, including the workspace.  The library never
 *     allocates, frees or synchronizes; all work is enqueued on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream).
 *   - q, k, v, out, rope_apply's x and y: bf16, token-major [N][H][D],
 *     contiguous.  pos_thw: fp32 [N][3] as (t, h, w).  lse: fp32 [H][N],
 *     natural log.  cu_seqlens: int32 [n_seqs + 1], rising from 0 to N.
 *   - Only D = 128 is supported.  The rotary split (dim_t, dim_h, dim_w)
 *     must be even widths adding up to D.
 *   - Arguments that the host can check are checked before anything is
 *     launched; a failed check returns a status and launches nothing.
 *     Device-resident cu_seqlens and pos_thw are trusted (h3attn_build_layout
 *     is the checked producer).  No entry point aborts, exits or prints, and
 *     no C++ exception crosses this interface.  h3attn_last_error() gives a
 *     human-readable reason for the last failure on the calling thread.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3ATTN_ABI_VERSION 1

typedef enum h3attn_status {
  H3ATTN_OK = 0,
  H3ATTN_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad layout item ... */
  H3ATTN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement (D != 128 ...) */
  H3ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size function asks for */
  H3ATTN_ERR_HIP = 4          /* the HIP runtime refused a launch */
} h3attn_status;

/* Multi-axis rotary configuration.  The head is split into consecutive
 * chunks t | h | w of widths dim_t, dim_h, dim_w; inside a chunk of width d,
 * dims (2j, 2j+1) form pair j, which turns by pos * theta^(-2j/d) radians.
 * The workloads here use theta = 10000 and (32, 48, 48). */
typedef struct h3attn_rope_cfg {
  double theta;
  int32_t dim_t;
  int32_t dim_h;
  int32_t dim_w;
  int32_t reserved; /* set to 0 */
} h3attn_rope_cfg;

/* ---------------------------------------------------------------------
 * Layout: items (visual grids and audio runs, in reference order) ->
 * cu_seqlens and per-token (t, h, w) positions.  Host only.
 *
 * Each segment is one attention document and starts its clock at 0.  A
 * visual item (T, H, W) emits T*H*W tokens, w fastest, at (clock + t, h, w),
 * then advances the clock by T.  An audio item emits n_audio tokens at
 * (start + a(i), 0, 0) with a(i) = i * span / n_audio (rule LINEAR) or that
 * value rounded half to even (rule ROUND_HALF_EVEN); attached audio starts
 * where the preceding visual item started and leaves the clock alone, a
 * standalone audio item starts at the clock and advances it by span.
 * A clock item emits no tokens and advances the clock by span: a long
 * video's continuation chunk keeps its global temporal positions by putting
 * one in front of its latents (vLLM-Omni "MiniMax-H3" recipe, "Long video
 * and driving audio").  A text item emits n_audio tokens at (0, 0, 0) and
 * leaves the clock alone: with every position 0 the rotation is the identity
 * and the attention is plain softmax attention, the token refiner's short
 * path (same recipe, "Attention Backends").
 * Positions are formed in double and rounded to float.
 * ------------------------------------------------------------------- */
enum { H3ATTN_ITEM_VISUAL = 0, H3ATTN_ITEM_AUDIO = 1, H3ATTN_ITEM_CLOCK = 2, H3ATTN_ITEM_TEXT = 3 };
enum { H3ATTN_AUDIO_LINEAR = 0, H3ATTN_AUDIO_ROUND_HALF_EVEN = 1 };

typedef struct h3attn_item {
  int32_t kind;     /* H3ATTN_ITEM_VISUAL, _AUDIO, _CLOCK or _TEXT */
  int32_t T, H, W;  /* visual grid (each >= 1); ignored otherwise */
  int32_t n_audio;  /* audio or text rows (>= 0); ignored otherwise */
  int32_t attached; /* audio: 1 = soundtrack of the preceding visual item */
  int32_t rule;     /* audio: H3ATTN_AUDIO_LINEAR or H3ATTN_AUDIO_ROUND_HALF_EVEN */
  int32_t reserved; /* set to 0 */
  double span;      /* audio: latent frames covered; clock: the advance (finite, >= 0) */
} h3attn_item;

/* items: host [sum(items_per_seq)]; items_per_seq: host [n_seqs] (>= 0 each);
 * n_seqs >= 1.  cu_seqlens: host [n_seqs + 1] or NULL.  pos_thw: host
 * [pos_capacity * 3] floats, or NULL to only count.  n_tokens (required)
 * receives N.  Fails with INVALID_ARG on a malformed item, on a total above
 * INT32_MAX tokens, or when pos_capacity < N while pos_thw is not NULL. */
h3attn_status h3attn_build_layout(const h3attn_item* items, const int32_t* items_per_seq, int32_t n_seqs,
                                  int32_t* cu_seqlens, float* pos_thw, int64_t pos_capacity,
                                  int64_t* n_tokens);

/* ---------------------------------------------------------------------
 * Standalone RoPE: y = rope(x, pos_thw), bf16 -> bf16 (fp32 arithmetic,
 * rounded to nearest even).  x, y: device [N][H][D]; y may equal x (in
 * place) but must not otherwise overlap it.  N = 0 is a no-op.
 * ------------------------------------------------------------------- */
h3attn_status h3attn_rope_apply(const void* x, void* y, const float* pos_thw, int64_t n_tokens, int32_t n_heads,
                                int32_t head_dim, const h3attn_rope_cfg* rope, void* stream);

/* ---------------------------------------------------------------------
 * Packed varlen attention forward.
 *
 *   out[i, h] = sum_j softmax_j(scale * <rope(q)[i,h], rope(k)[j,h]>) v[j, h]
 *   lse[h, i] = ln sum_j exp(scale * <rope(q)[i,h], rope(k)[j,h]>)
 *
 * with i, j ranging over the same segment [cu[s], cu[s+1]) and no causal
 * order.  scale <= 0 selects 1/sqrt(D).  max_seqlen is the longest segment
 * length the call computes, at most 2^22 = 4,194,304 (UNSUPPORTED above) and
 * at most N: a segment longer than max_seqlen is computed as its first
 * max_seqlen tokens alone, so its later rows of out and lse are not written
 * and its later keys are not attended.  Empty segments produce no rows; N = 0
 * is a no-op.  out and lse must not overlap any input.
 *
 * The workspace (device, >= h3attn_varlen_fwd_workspace_size bytes, 256-byte
 * aligned) holds the rotated keys (fp16, each 64-key tile scaled by a power
 * of two), the transposed values, the per-tile key scales and the segments'
 * order by length (the attention grid starts the longest first), in the
 * layout the attention kernel reads; its contents on return are unspecified.
 *
 * Precision: the rotated queries and keys enter the score contraction as
 * fp16 with power-of-two block scales (one per query row, one per 64-key
 * tile), which keeps bf16's range; probabilities and values enter the second
 * contraction as bf16; all accumulation is fp32.
 *
 * Inputs are not scanned.  A NaN or infinity in q makes that row's out and
 * lse undefined, in k or v those of the rows of its segment (of one head);
 * other segments and heads come out exactly as without it, and so, up to the
 * rounding of their shared softmax reference, do the other rows of the
 * segment.  The same holds for the FP8 mode below.
 * ------------------------------------------------------------------- */
size_t h3attn_varlen_fwd_workspace_size(int64_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_seqs);

h3attn_status h3attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                const float* pos_thw, void* out, float* lse, int64_t n_tokens, int32_t n_heads,
                                int32_t head_dim, int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                const h3attn_rope_cfg* rope, void* workspace, size_t workspace_bytes, void* stream);

/* The two stages h3attn_varlen_fwd runs, exported so that a caller can time
 * or overlap them separately.  Calling h3attn_varlen_kv_prologue and then
 * h3attn_varlen_attention on the same stream, with the same arguments,
 * computes exactly what h3attn_varlen_fwd computes.
 *
 * kv_prologue: rotates k and packs it, with v transposed, into the workspace,
 *              and ranks the segments by length there.
 * attention:   rotates q as it loads it and runs the attention kernel on the
 *              packed keys and values; it reads k and v only through the
 *              workspace, and takes its segment order from it. */
h3attn_status h3attn_varlen_kv_prologue(const void* k, const void* v, const int32_t* cu_seqlens,
                                        const float* pos_thw, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                        int32_t n_seqs, int32_t max_seqlen, const h3attn_rope_cfg* rope,
                                        void* workspace, size_t workspace_bytes, void* stream);

h3attn_status h3attn_varlen_attention(const void* q, const int32_t* cu_seqlens, const float* pos_thw, void* out,
                                      float* lse, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                      int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                      const h3attn_rope_cfg* rope, const void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ---------------------------------------------------------------------
 * h3attn_varlen_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and checks are
 * h3attn_varlen_fwd's minus the workspace: the library uses a 128 MiB array
 * of its own on each GPU instead, held from the library's load until the
 * process ends, and allocates nothing.  Fails with UNSUPPORTED, before any
 * launch, when h3attn_varlen_fwd_workspace_size(n_tokens, n_heads, head_dim,
 * n_seqs) exceeds 134,217,728 bytes (about 250,000 (token, head) pairs: the
 * 480p-shaped workload fits, the 1344x768-shaped one does not).  All calls on
 * one GPU share its array and find it as the last call left it; every call
 * rewrites all of it that it reads, so calls in order on one stream are safe,
 * while calls that overlap in time on one GPU (other streams or threads) race
 * and give wrong results.
 * ------------------------------------------------------------------- */
h3attn_status h3attn_varlen_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                        const float* pos_thw, void* out, float* lse, int64_t n_tokens,
                                        int32_t n_heads, int32_t head_dim, int32_t n_seqs, int32_t max_seqlen,
                                        float softmax_scale, const h3attn_rope_cfg* rope, void* stream);

/* ---------------------------------------------------------------------
 * Lossy FP8 mode of the same attention ("SAGE" quantization).
 *
 * Defined by the vLLM-Omni "MiniMax-H3" recipe, section "Attention
 * Backends": for the long main DiT attention, queries and keys are quantized
 * to FP8 e4m3 with one scale per query token and one scale per 16 keys, and
 * probabilities and values are FP8 as well.  The recipe marks it lossy and
 * asks for a comparison against dense output before use.
 *
 * Here: every scale is a power of two, the smallest that brings its block's
 * largest magnitude to <= 448, and every value is rounded to nearest e4m3
 * (OCP E4M3).  Blocks: a (token, head) row of rotated q (fp32); 16
 * consecutive rotated keys of one head counted from the segment's first key;
 * one value channel (one of the 128 dims) of one head over all keys of the
 * segment.  The logits are softmax_scale times the product of the quantized
 * q and k.  Softmax itself is exact (fp32 running maximum and row sums of the
 * unrounded probabilities); probabilities enter the product with V as
 * e4m3(256 p) with p relative to a running maximum; all accumulation is fp32;
 * out is bf16 and lse fp32 exactly as for h3attn_varlen_fwd, whose argument
 * meanings, layout, ownership and error rules apply unchanged.  Only the
 * workspace differs: it must hold h3attn_varlen_fwd_fp8_workspace_size bytes
 * (256-byte aligned) and its contents on return are unspecified.
 *
 * Skip-Softmax (same recipe section: an optional lossy "sparse attention"
 * with a direct threshold, 0.05 there).  skip_threshold in [0, 1); 0 computes
 * every key.  Otherwise keys go in tiles of 64 counted from the segment
 * start, and each query row decides alone: it leaves a tile out when its
 * largest logit in the tile is below ln(skip_threshold) plus its largest
 * logit over the earlier tiles (the first tile is always kept); out and lse
 * are then softmax over the kept tiles.  Whether to use it for a given
 * denoising step (the recipe keeps the early, high-noise steps dense) is the
 * caller's choice.  skip_stats: NULL, or device uint64[2] to which the call
 * adds the (row, tile) pairs its rows saw and those they left out (nothing
 * when skip_threshold is 0); the caller clears it.  Fails with INVALID_ARG for
 * a threshold outside [0, 1).
 * ------------------------------------------------------------------- */
size_t h3attn_varlen_fwd_fp8_workspace_size(int64_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_seqs);

h3attn_status h3attn_varlen_fwd_fp8(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                    const float* pos_thw, void* out, float* lse, int64_t n_tokens, int32_t n_heads,
                                    int32_t head_dim, int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                    float skip_threshold, const h3attn_rope_cfg* rope, void* workspace,
                                    size_t workspace_bytes, uint64_t* skip_stats, void* stream);

/* The two stages of h3attn_varlen_fwd_fp8, with the same contract as the
 * exact mode's pair: kv_prologue_fp8 rotates k, quantizes k and v and packs
 * them into the workspace; attention_fp8 rotates and quantizes q as it loads
 * it and reads k and v only through the workspace. */
h3attn_status h3attn_varlen_kv_prologue_fp8(const void* k, const void* v, const int32_t* cu_seqlens,
                                            const float* pos_thw, int64_t n_tokens, int32_t n_heads,
                                            int32_t head_dim, int32_t n_seqs, int32_t max_seqlen,
                                            const h3attn_rope_cfg* rope, void* workspace, size_t workspace_bytes,
                                            void* stream);

h3attn_status h3attn_varlen_attention_fp8(const void* q, const int32_t* cu_seqlens, const float* pos_thw, void* out,
                                          float* lse, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                                          int32_t n_seqs, int32_t max_seqlen, float softmax_scale,
                                          float skip_threshold, const h3attn_rope_cfg* rope, const void* workspace,
                                          size_t workspace_bytes, uint64_t* skip_stats, void* stream);

/* Skip-Softmax timestep gate (vLLM-Omni "MiniMax-H3" recipe, section
 * "Attention Backends": disabled_until_timestep keeps the early, high-noise
 * denoising steps dense by comparing a cutoff with the step's video sigma).
 * Host only, no device work.  Writes to *threshold_out the skip_threshold to
 * pass to the FP8 calls for a step at noise level sigma: 0 (dense) while
 * sigma > disabled_until_timestep, else skip_threshold.  With the recipe's
 * flow shift of 12 and 50 steps, cutoffs 0.99, 0.97 and 0.95 keep the first
 * 6, 14 and 19 of the 49 forwards dense.  Fails with INVALID_ARG for a NULL
 * threshold_out, a skip_threshold outside [0, 1) or a NaN cutoff or sigma. */
h3attn_status h3attn_skip_gate(float skip_threshold, float disabled_until_timestep, float sigma,
                               float* threshold_out);

/* Status name ("H3ATTN_OK", ...); never NULL. */
const char* h3attn_status_string(h3attn_status s);
/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* h3attn_last_error(void);
/* H3ATTN_ABI_VERSION of the built library. */
int32_t h3attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
