/*
 * svga.h - block-sparse spatio-temporal attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libsvga.so. Every entry point takes plain pointers and sizes; the
 * caller owns every buffer and stream. Device pointers point to GPU memory,
 * host pointers to CPU memory, as each parameter says.
 *
 * Source cited as ASTA: "Accelerating Spatio-Temporal Attention for Video
 * Diffusion on TPUs" (Google Developers Blog). Sections are named by heading,
 * figures by number.
 *
 * Common conventions
 * ------------------
 * - Tensors Q, K, V, O are bfloat16, contiguous [B, n_heads, N, head_dim],
 *   N = F*H*W tokens per head: the head-local layout of ASTA section
 *   "Perform layout transformations on local heads" (every head holds its
 *   whole sequence). Byte offsets are 64-bit.
 * - Token t of frame-major (F, H, W) order has frame f = t / (H*W) and
 *   flattened spatial index s = t % (H*W) = h*W + w (ASTA Figure 9).
 * - Flags are uint8 [B, n_heads] in device memory, one per (batch, head):
 *   0 = spatial head, nonzero = temporal head (ASTA section "Support dynamic
 *   routing with fixed tensor shapes"). Flags are read on the device; no
 *   entry point copies them to the host, and tensor shapes never depend on them.
 * - Every device entry point only enqueues work on `stream` (a hipStream_t;
 *   NULL = the null stream) and returns without synchronising. Arguments are
 *   checked on the host before anything is enqueued: a nonzero status means
 *   nothing was launched. Device-resident values (flags, sample ids, the tile
 *   map's contents) cannot be checked on the host; the kernels keep every
 *   access in bounds whatever they hold.
 * - The library allocates no device memory, frees none, and keeps no state
 *   except a per-thread copy of the last error message.
 */
#ifndef SVGA_H
#define SVGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */

typedef int32_t svga_status;
#define SVGA_OK 0
#define SVGA_EINVAL (-1)        /* null pointer, size out of range, N != F*H*W, aliasing */
#define SVGA_EUNSUPPORTED (-2)  /* head_dim / tile sizes / sample count with no compiled kernel */
#define SVGA_ECAPACITY (-3)     /* a caller buffer is smaller than the size query returns */
#define SVGA_EHIP (-4)          /* the HIP runtime reported an error when launching */

/* Static text for a status code. */
const char* svga_status_string(svga_status status);
/* Message of the last failing call on this thread ("" if none). Owned by the library. */
const char* svga_last_error(void);
/* ABI version, major*100 + minor. */
int32_t svga_version(void);

/* ---------------------------------------------------------------- geometry and masks */

/* Video latent: F frames of H x W tokens. N = F*H*W must be below 2^30. */
typedef struct svga_geom {
    int32_t F, H, W;
} svga_geom;

enum { SVGA_KIND_SPATIAL = 0, SVGA_KIND_TEMPORAL = 1 };
/* Temporal-head token order (ASTA section "Arrange tokens for efficient
 * temporal access", Figure 9). SINK_FIRST: tokens of the sink frames keep
 * their frame-major places at the front; every other token follows, ordered
 * by spatial index s, then frame. LITERAL: all tokens ordered by (s, frame). */
enum { SVGA_TL_SINK_FIRST = 0, SVGA_TL_LITERAL = 1 };

/* Masks of ASTA section "Speeding up attention" and Figure 3. Query token q
 * keeps key token k iff
 *   f_k < sink_frames                      (first-frame attention sink), or
 *   spatial head:  |f_k - f_q| <= spatial_band     (local frame band), or
 *   temporal head: |s_k - s_q| <= temporal_band    (spatial window, every frame).
 * 0 <= sink_frames <= F; bands >= 0. */
typedef struct svga_mask {
    int32_t sink_frames;
    int32_t spatial_band;
    int32_t temporal_band;
    int32_t temporal_layout;
} svga_mask;

/* Mask for target kept fractions: the sparsity knob of ASTA section
 * "End-to-end results and takeaways" (Table 3 compares schedules that keep
 * progressively fewer attention pairs; a schedule picks, per denoising step
 * and layer, how many pairs each head kind keeps).
 * Fills *out with sink_frames, temporal_layout and, for each kind, the
 * smallest band whose kept pairs of one head, counted in closed form from
 * the mask definitions above (spatial: frames; temporal: flattened
 * positions), reach target * N^2. The comparison is exact: a double target
 * is a dyadic rational, and the count it needs is formed in 128-bit integer
 * arithmetic. Bands run from 0 up to the first that keeps every pair
 * (F - 1, resp. H*W - 1), so a target at or below a kind's band-0 fraction
 * gives band 0 and a target of 1 gives the dense mask.
 * spatial_target, temporal_target: in [0, 1] (SVGA_EINVAL otherwise, NaN
 * included). kept_pairs: host int64[2] receiving the chosen masks' kept pairs
 * per head (spatial, temporal), or NULL. Host only; no device work. */
svga_status svga_mask_for_kept_fraction(const svga_geom* geom, int32_t sink_frames, int32_t temporal_layout,
                                        double spatial_target, double temporal_target,
                                        svga_mask* out, int64_t* kept_pairs);

/* ---------------------------------------------------------------- tile map */

/* Traversals of ASTA Figure 4 / Table 2.
 * DENSE   (B0): every tile visited; only the last key tile, if it holds padding, is masked.
 * NAIVE   (B1): tiles with no kept pair skipped; the exact mask applied on every visited tile.
 * EXACT   (B2): tiles whose pairs are all kept run unmasked; the exact mask only on
 *               boundary tiles (ASTA section "Avoid intra-tile masking ...").
 * ROUNDED (B3): each tile kept whole iff it has a kept pair and at least half its
 *               valid area is kept; only tiles holding padding are masked (ASTA
 *               section "Align the sparse mask with final execution"). This changes
 *               the mask. */
enum { SVGA_MAP_DENSE = 0, SVGA_MAP_NAIVE = 1, SVGA_MAP_EXACT = 2, SVGA_MAP_ROUNDED = 3 };
/* Tile classes of ASTA section "Logical sparsity is not physical sparsity", Figure 5. */
enum { SVGA_TILE_SKIP = 0, SVGA_TILE_FULL = 1, SVGA_TILE_BOUNDARY = 2 };

#define SVGA_TILEMAP_MAGIC 0x4d475653u /* "SVGM" */
#define SVGA_TILEMAP_VERSION 1

/* A tile map is one byte blob holding both head kinds (the map depends on
 * the kind, never on which heads carry it). Layout:
 *   svga_tilemap_header (64 bytes)
 *   int32 n_full[2][tq]        full tiles per (kind, query tile)
 *   int32 n_bnd [2][tq]        boundary tiles per (kind, query tile)
 *   int32 kv    [2][tq][tk]    key-tile lists: full tiles ascending, then boundary
 *                              tiles ascending, then -1
 *   int8  cls   [2][tq][tk]    SVGA_TILE_* of every tile
 * Kind 0 is spatial, kind 1 temporal. Tiles are in each kind's executed token
 * order (temporal heads: the permuted order). tq = ceil(N/bq), tk = ceil(N/bkv).
 * Query rows past N never decide a class; a key tile holding positions past N
 * is never FULL. Use svga_tilemap_layout() for the byte offsets. */
typedef struct svga_tilemap_header {
    uint32_t magic;
    int32_t version;
    int32_t F, H, W;
    int32_t sink_frames, spatial_band, temporal_band, temporal_layout;
    int32_t bq, bkv, tq, tk, mode;
    int32_t reserved[2];
} svga_tilemap_header;

typedef struct svga_tilemap_offsets {
    size_t n_full, n_bnd, kv, cls; /* byte offsets from the start of the blob */
    size_t total;                  /* blob size in bytes */
    int32_t tq, tk;
} svga_tilemap_offsets;

/* Byte layout of the tile map for this geometry and tile shape.
 * bq, bkv: query / key tile sizes, 1..4096. tq*tk must stay below 2^28. */
svga_status svga_tilemap_layout(const svga_geom* geom, int32_t bq, int32_t bkv,
                                svga_tilemap_offsets* out);

/* Build a tile map in HOST memory `h_map` (map_bytes >= layout total).
 * Counts every tile's kept pairs from each row's key ranges (exact integer
 * arithmetic), classifies per `mode`, writes the canonical lists. */
svga_status svga_build_tilemap_host(const svga_geom* geom, const svga_mask* mask,
                                    int32_t bq, int32_t bkv, int32_t mode,
                                    void* h_map, size_t map_bytes);

/* Same map, built by GPU kernels into DEVICE memory `d_map`, enqueued on `stream`.
 * Bit-identical to svga_build_tilemap_host. Needs tk <= 8000 (the per-workgroup
 * counters then fit 64 KB of LDS); SVGA_EUNSUPPORTED above that. */
svga_status svga_build_tilemap(const svga_geom* geom, const svga_mask* mask,
                               int32_t bq, int32_t bkv, int32_t mode,
                               void* d_map, size_t map_bytes, void* stream);

/* ---------------------------------------------------------------- token permutation */

/* ASTA sections "Support dynamic routing with fixed tensor shapes" and
 * "Arrange tokens for efficient temporal access": for every (b, h) whose flag
 * is nonzero, out[b,h,p(t),:] = in[b,h,t,:] with p the temporal order of
 * `mask->temporal_layout`; heads with flag 0 are copied unchanged. Out of
 * place: d_in and d_out are distinct device buffers of B*n_heads*N*head_dim
 * bf16. head_dim: a multiple of 8, at most 512; N * head_dim / 8 (16-byte
 * vectors per head) must stay below 2^31, else SVGA_EINVAL. */
svga_status svga_permute(const void* d_in, void* d_out, const uint8_t* d_flags,
                         int32_t B, int32_t n_heads, const svga_geom* geom,
                         const svga_mask* mask, int32_t head_dim, void* stream);

/* Inverse of svga_permute: out[b,h,t,:] = in[b,h,p(t),:] for flagged heads,
 * a copy for the others, so later layers see frame-major order again. */
svga_status svga_unpermute(const void* d_in, void* d_out, const uint8_t* d_flags,
                           int32_t B, int32_t n_heads, const svga_geom* geom,
                           const svga_mask* mask, int32_t head_dim, void* stream);

/* ---------------------------------------------------------------- head routing */

/* Device workspace bytes svga_route_heads needs for these sizes. */
svga_status svga_route_workspace_bytes(int32_t B, int32_t n_heads, const svga_geom* geom,
                                       int32_t head_dim, int32_t n_samples, size_t* bytes);

/* ASTA section "Speeding up attention": for each (b, h), the queries
 * d_sample_idx[0..n_samples) (frame-major token ids, device int32) attend to
 * all N keys three times: unmasked, under the spatial mask and under the
 * temporal mask (exact masks, frame-major order, no tiling). With
 * err_x = sum over samples of ||o_x - o_dense||^2, the head's flag is 1
 * (temporal) iff err_temporal < err_spatial, else 0.
 * Inputs d_q, d_k, d_v: frame-major bf16 [B, n_heads, N, head_dim].
 * d_flags_out: device uint8 [B, n_heads]. d_err_out: device float
 * [B, n_heads, 2] = (err_spatial, err_temporal), or NULL.
 * softmax_scale: usually 1/sqrt(head_dim). n_samples: 1..64. head_dim: 64 or 128.
 * Sample ids outside [0, N) are clamped into range. */
svga_status svga_route_heads(const void* d_q, const void* d_k, const void* d_v,
                             int32_t B, int32_t n_heads, const svga_geom* geom,
                             const svga_mask* mask, int32_t head_dim,
                             const int32_t* d_sample_idx, int32_t n_samples,
                             float softmax_scale, void* d_workspace, size_t workspace_bytes,
                             uint8_t* d_flags_out, float* d_err_out, void* stream);

/* ---------------------------------------------------------------- sparse attention */

/* Block-sparse flash attention forward: O = SoftMax(Q K^T * softmax_scale) V
 * over each query's kept keys (ASTA section "Logical sparsity is not physical
 * sparsity"). For each (b, h, query tile) the kernel walks that head kind's
 * FULL list without any mask, then its BOUNDARY list with the mask, carrying
 * one running max / sum / output through both (ASTA section "Avoid intra-tile
 * masking ..."). Masked and padded pairs get exactly zero weight.
 *
 * d_map: device tile map built with these geom/mask/bq/bkv/mode (both host
 *   and device builders give the same blob); map_bytes its size.
 * mode: the map's SVGA_MAP_*; NAIVE and EXACT apply the exact mask on
 *   boundary tiles, DENSE and ROUNDED only the padding mask.
 * gather_temporal = 0: Q, K, V, O of temporal heads are already in the
 *   permuted order (svga_permute before, svga_unpermute after).
 * gather_temporal = 1: Q, K, V, O are all frame-major; temporal heads load
 *   and store rows through the permutation inside the kernel (ASTA section
 *   "Arrange tokens ..." compares this against permuting). Both settings give
 *   bit-identical outputs.
 * d_lse: device float [B, n_heads, N] log-sum-exp of each row's scaled
 *   scores (natural log; -inf for a row with no kept key), rows in O's
 *   order; or NULL.
 * Rows with no kept key get O = 0.
 * Supported: head_dim 64 or 128; bq in {32, 64, 128, 256, 512}; bkv a
 * multiple of 32 from 32 to 512. One head of
 * K or V (N * head_dim * 2 bytes) must stay below 2^31 bytes, which the
 * tile-count limit (tq * tk below 2^28) already implies for these tiles.
 * d_o must not alias d_q, d_k or d_v. */
svga_status svga_sparse_attn_fwd(const void* d_q, const void* d_k, const void* d_v,
                                 void* d_o, float* d_lse,
                                 int32_t B, int32_t n_heads, const svga_geom* geom,
                                 const svga_mask* mask, int32_t head_dim, float softmax_scale,
                                 const uint8_t* d_flags, const void* d_map, size_t map_bytes,
                                 int32_t bq, int32_t bkv, int32_t mode,
                                 int32_t gather_temporal, void* stream);

/* Device workspace bytes that svga_sparse_attn_fwd_ws needs (a work counter). */
svga_status svga_attn_workspace_bytes(size_t* bytes);

/* Device workspace bytes with which svga_sparse_attn_fwd_ws also splits the
 * tail of its work (ASTA section "Avoid intra-tile masking when there is
 * nothing to mask": partial results over disjoint key sets combine through
 * their softmax statistics). For bq 256 and 512: the last query tiles (256-row
 * parts of a 512-row tile), as many as the device holds workgroups at once
 * and at most 256, each run as 4 pieces over contiguous quarters of their key
 * tile lists; each piece stores its normalised output O_p (bf16) and its
 * log-sum-exp L_p in the workspace, and a second kernel on the same stream
 * writes, with m = max_p L_p and w_p = e^(L_p - m),
 * O = sum_p w_p O_p / sum_p w_p and LSE = m + ln sum_p w_p. About 68 MB at
 * head_dim 128. Smaller bq do not split: svga_attn_workspace_bytes' size.
 * Depends on head_dim and bq only.
 * SVGA_EUNSUPPORTED for a head_dim / bq without an attention kernel,
 * SVGA_EINVAL if bytes is NULL. */
svga_status svga_attn_split_workspace_bytes(int32_t head_dim, int32_t bq, size_t* bytes);

/* The operation of svga_sparse_attn_fwd (ASTA section "Logical sparsity is
 * not physical sparsity": the tile walk over each query tile's FULL, then
 * BOUNDARY key tiles), launched as persistent workgroups: as many workgroups
 * as the device holds at once, each taking the next (batch, head, query tile) from a
 * counter in d_workspace until none is left (no workgroup launch between
 * query tiles, and no CU idles while the in-order dispatcher waits on a busy
 * one). Same arguments, plus:
 * d_workspace: caller-owned device memory, at least svga_attn_workspace_bytes
 *   bytes, 16-byte aligned; its content on entry does not matter (the call
 *   clears what it needs on the stream first) and is undefined afterwards.
 *   SVGA_EINVAL if NULL or misaligned, SVGA_ECAPACITY if too small.
 * Below svga_attn_split_workspace_bytes(head_dim, bq) bytes, and for bq
 * below 256, the results are those of svga_sparse_attn_fwd bit for bit; from
 * there on the last query tiles run split (see
 * svga_attn_split_workspace_bytes) and their rows equal svga_sparse_attn_fwd's
 * up to the bf16 rounding of the pieces' outputs.
 * Calls that share one workspace must not overlap (one stream, or ordered). */
svga_status svga_sparse_attn_fwd_ws(const void* d_q, const void* d_k, const void* d_v,
                                    void* d_o, float* d_lse,
                                    int32_t B, int32_t n_heads, const svga_geom* geom,
                                    const svga_mask* mask, int32_t head_dim, float softmax_scale,
                                    const uint8_t* d_flags, const void* d_map, size_t map_bytes,
                                    int32_t bq, int32_t bkv, int32_t mode,
                                    int32_t gather_temporal, void* d_workspace,
                                    size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The operation
 * and launch of svga_sparse_attn_fwd_ws with a split-tail workspace (same
 * kernels, same bits), with the library's own scratch memory in place of the
 * workspace: one file-scope device array of 68,157,696 bytes per GPU (the
 * work counter plus the split tail of the largest supported case, head_dim
 * 128 and 256-row workgroups), which that GPU holds from the first call on it
 * until the process ends. The call allocates and frees nothing; the scratch
 * address is looked up once per device, on the first call with that device
 * current. Every call on one GPU uses the same scratch, and the call clears
 * what must start at zero (the work counter) on `stream` itself: calls on one
 * GPU that may overlap (different streams without ordering, several host
 * threads) race on it and must be serialised by the caller. Arguments and
 * errors as svga_sparse_attn_fwd; SVGA_ECAPACITY if a configuration would
 * need more scratch than the array holds (none of the supported head_dim and
 * bq values does); SVGA_EHIP if the scratch address cannot be found. */
svga_status svga_sparse_attn_fwd_noalloc(const void* d_q, const void* d_k, const void* d_v,
                                         void* d_o, float* d_lse,
                                         int32_t B, int32_t n_heads, const svga_geom* geom,
                                         const svga_mask* mask, int32_t head_dim, float softmax_scale,
                                         const uint8_t* d_flags, const void* d_map, size_t map_bytes,
                                         int32_t bq, int32_t bkv, int32_t mode,
                                         int32_t gather_temporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVGA_H */
