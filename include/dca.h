/*
 * dca.h -- C ABI of libdca: causal GQA prefill attention under Dual Chunk
 * Attention (DCA) on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages):
 *   [mizuki] "Qwen2.5-1M 不重训外推 1M", mizuki-eaf.pages.dev: sections
 *            "核心思想" (the L x L attention matrix split into intra-chunk,
 *            successive-chunk and inter-chunk parts), "Intra-Chunk Attention",
 *            "Successive-Chunk Attention" (local window W), "Inter-Chunk
 *            Attention" (query pinned at a large fixed index, key positions
 *            repeating periodically), "DCA + YaRN" (temperature on the
 *            logits), and the MInference vertical-slash sections.
 *   [yudong] "Qwen-2.5 explained", yudonglee.me, section 3: GQA at every
 *            size, RoPE base 1e7.
 *
 * What the library computes, for query head h, batch b, row i and every key
 * j <= i (and only keys in active tiles when a vertical-slash mask is given):
 *
 *   c(i) = i / C, r(i) = i mod C, P = C + W - 1 (pinned query index)
 *   key position        Pk(j)       = j mod C
 *   intra  (c(i)=c(j))  Pq(i)       = r(i)
 *   succ   (c(i)=c(j)+1) Pq(i)      = min(C + r(i), P)
 *   inter  (otherwise)  Pq(i)       = P
 *   s_ij  = yarn_scale * softmax_scale * < R(Pq(i)) q_i , R(Pk(j)) k_j >
 *   out_i = sum_j softmax_j(s_i.) v_j          lse_i = ln sum_j exp(s_ij)
 *
 * R(p) is half-split RoPE: pairs (m, m + d/2) rotated by p * base^(-2m/d);
 * cos and sin are taken in float64 and rounded to float32. KV head of query
 * head h is h / (n_q_heads / n_kv_heads).
 *
 * Conventions for every entry point:
 *   - Return value: a dca_status. On DCA_E_INVALID, DCA_E_UNSUPPORTED or
 *     DCA_E_WORKSPACE nothing is enqueued and no output is touched; the
 *     reason is in dca_last_error() (thread-local, valid until the next call
 *     on the same thread). Nothing is thrown or aborted across the ABI.
 *   - Device entry points enqueue on `stream` (a hipStream_t; NULL = the
 *     null stream) and return without synchronizing. Results are valid
 *     after the stream is synchronized. Launch failures return DCA_E_DEVICE.
 *     They enqueue kernel launches only (no allocation, memset, copy or
 *     synchronization), so a call may be captured into a HIP graph.
 *   - Pointers marked "device" are caller-owned device memory; the library
 *     allocates and frees nothing.
 *   - Tensors are contiguous row-major; q, out: [batch, n_q_heads, seq,
 *     head_dim]; k, v: [batch, n_kv_heads, seq, head_dim]; all four share one
 *     dtype. lse: [batch, n_q_heads, seq] float32.
 *   - q, k, v and out must be 16-byte aligned, lse and mask lists 4-byte.
 *   - Supported domain: head_dim 64 or 128; n_q_heads % n_kv_heads == 0;
 *     seq >= 1 (ragged tails are handled); C >= 64 and C % 64 == 0;
 *     0 <= W <= C; rope_base > 1; yarn_scale > 0; seq and C + W below 2^31.
 *   - Calls are deterministic (bit-identical results for identical inputs)
 *     and re-entrant; calls that share a workspace must not overlap.
 */
#ifndef DCA_H
#define DCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DCA_OK = 0,
    DCA_E_INVALID = 1,      /* a null pointer, a bad size, aliasing outputs */
    DCA_E_UNSUPPORTED = 2,  /* valid but outside the supported domain */
    DCA_E_WORKSPACE = 3,    /* workspace smaller than dca_workspace_size */
    DCA_E_DEVICE = 4        /* HIP runtime or launch failure, or no GPU */
} dca_status;

typedef enum { DCA_F32 = 0, DCA_BF16 = 1 } dca_dtype;

typedef struct {
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t dtype;          /* dca_dtype */
    float softmax_scale;    /* 0 => 1 / sqrt(head_dim) */
} dca_shape;

/* MInference-style vertical-slash mask [mizuki, sparse-attention sections],
 * read tile-granular on 64 x 64 (query, key) tiles: tile (t, kt), kt <= t, is
 * active for query head h iff some vertical column of h lies in
 * [64 kt, 64 kt + 63] or some slash offset of h lies in
 * [max(0, 64 (t - kt) - 63), 64 (t - kt) + 63]. Columns and offsets are true
 * indices (key j, distance i - j), not remapped positions. Every causal pair
 * inside an active tile is attended; none in an inactive tile. The same mask
 * applies to every batch entry. Entries outside [0, seq) are ignored; order
 * and duplicates do not matter. */
typedef struct {
    const int32_t *vertical;  /* device [n_q_heads][n_vertical] */
    const int32_t *slash;     /* device [n_q_heads][n_slash]    */
    int32_t n_vertical;       /* >= 0 */
    int32_t n_slash;          /* >= 0 */
} dca_vs_mask;

/* Text for a status code (static storage). */
const char *dca_status_str(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char *dca_last_error(void);

/* Host-only position-index map [mizuki, Intra-/Successive-/Inter-Chunk]:
 * pq_intra[i] = i mod C, pq_succ[i] = min(C + i mod C, C + W - 1),
 * *pq_inter = C + W - 1, pk[j] = j mod C, for i, j in [0, seq). Host arrays
 * of seq int32 each (pq_inter: one int32), caller-owned; any of them may be
 * NULL to skip it. */
int dca_remap_positions(int64_t seq, int64_t C, int64_t W,
                        int32_t *pq_intra, int32_t *pq_succ, int32_t *pq_inter,
                        int32_t *pk);

/* Bytes of device workspace dca_prefill needs for these arguments (mask may
 * be NULL for dense causal). Written to *bytes. The workspace holds the
 * float32 cos/sin table for positions [0, C + W), the three rotated query
 * variants, the rotated keys and the re-laid-out values in the attention
 * kernel's operand order, and (with a mask) the per-head tile lists. */
int dca_workspace_size(int64_t seq, int64_t C, int64_t W, const dca_shape *shape,
                       const dca_vs_mask *mask, size_t *bytes);

/* The whole path [mizuki, 核心思想 through DCA + YaRN]: remap pre-pass
 * (cos/sin table, rotated Q variants, rotated K, value re-layout), the
 * vertical-slash tile index when mask != NULL, and the
 * attention kernel. q, k, v: device, read-only. out: device, written for
 * every (b, h, i < seq, d). lse: device float32 or NULL (skip). workspace:
 * device, at least dca_workspace_size bytes, 256-byte aligned. out and lse
 * must not overlap q, k, v, the workspace or each other; q, k and v must not
 * overlap the workspace; the mask lists must not overlap the workspace, out
 * or lse (each DCA_E_INVALID). */
int dca_prefill(const void *q, const void *k, const void *v, void *out, float *lse,
                int64_t seq, int64_t C, int64_t W, double rope_base, float yarn_scale,
                const dca_vs_mask *mask, const dca_shape *shape,
                void *workspace, size_t workspace_bytes, void *stream);

/* Chunked prefill [mizuki, Chunked Prefill]: the sequence of seq tokens is
 * prefilled a block of rows at a time, in order, on one workspace.
 *
 * dca_chunk_workspace_size: bytes of workspace for calls on this sequence
 * with up to max_rows rows each (1 <= max_rows <= seq). The rotated keys and
 * re-laid-out values of all seq positions stay in the workspace between
 * calls; the query variants of one call come after them.
 *
 * dca_prefill_chunk: computes the query rows [q_offset, q_offset + n_rows)
 * against the keys [0, q_offset + n_rows). q is [batch][n_q_heads][n_rows]
 * [head_dim], k and v are [batch][n_kv_heads][n_rows][head_dim]: the rows and
 * keys of this block only (device, read-only). out is [batch][n_q_heads]
 * [n_rows][head_dim], lse [batch][n_q_heads][n_rows] float32 or NULL. The
 * call rotates and stores this block's keys and values in the workspace, so
 * the blocks before it (rows [0, q_offset)) must have been passed to earlier
 * calls on the same workspace, with the same seq, C, W, rope_base,
 * yarn_scale and shape (the keys are stored scaled by yarn_scale); calls on
 * one workspace must not overlap in time. q_offset must be a multiple of 64
 * (DCA_E_UNSUPPORTED) and the rows must lie inside [0, seq) (DCA_E_INVALID).
 * The outputs are identical to the rows [q_offset, q_offset + n_rows) of one
 * dca_prefill over the whole sequence. Other arguments and errors are as for
 * dca_prefill. */
int dca_chunk_workspace_size(int64_t seq, int64_t max_rows, int64_t C, int64_t W,
                             const dca_shape *shape, const dca_vs_mask *mask, size_t *bytes);
int dca_prefill_chunk(const void *q, const void *k, const void *v, void *out, float *lse,
                      int64_t q_offset, int64_t n_rows, int64_t seq, int64_t C, int64_t W,
                      double rope_base, float yarn_scale, const dca_vs_mask *mask,
                      const dca_shape *shape, void *workspace, size_t workspace_bytes,
                      void *stream);

/* The whole path with the query rotation fused into the attention kernel
 * [mizuki, Inter-Chunk Attention: only position indices change]: the pre-pass
 * rotates and stores only the keys (and re-lays out the values); each wave
 * reads its rows of q and turns them to the region's query position when it
 * enters a region (three times per row block at most), with the same cos/sin
 * table entries and the same arithmetic as the pre-pass, so out and lse are
 * identical to dca_prefill's. The workspace (dca_fused_workspace_size) holds
 * no query variants: 3 n_q_heads / (3 n_q_heads + 2 n_kv_heads) of the
 * dca_prefill workspace less. q must stay unchanged until the call's work on
 * the stream has finished. Arguments, layouts and errors are as for
 * dca_prefill. */
int dca_fused_workspace_size(int64_t seq, int64_t C, int64_t W, const dca_shape *shape,
                             const dca_vs_mask *mask, size_t *bytes);
int dca_prefill_fused(const void *q, const void *k, const void *v, void *out, float *lse,
                      int64_t seq, int64_t C, int64_t W, double rope_base, float yarn_scale,
                      const dca_vs_mask *mask, const dca_shape *shape,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Online vertical-slash estimation with continuous positions [mizuki,
 * 稀疏注意力 + 核优化: key tokens are selected with the continuous relative
 * positions restored; 跟 NSA / 其他稀疏注意力的区别: vertical-slash pattern].
 * The last n_last (1..64) query rows of the sequence attend to every key with
 * RoPE at the true indices i and j (not the DCA map) and the logit scale
 * yarn_scale * softmax_scale; per query head, key column j scores the sum of
 * its softmax weights over those rows and diagonal o = i - j the sum along
 * it. Each head keeps columns [0, n_forced) plus the n_vertical - n_forced
 * best other columns, and offsets [0, n_forced) plus the n_slash - n_forced
 * best other offsets, ties to the smaller index. Batch must be 1
 * (DCA_E_UNSUPPORTED). q: device [1][n_q_heads][seq][head_dim]; k: device
 * [1][n_kv_heads][seq][head_dim]. vertical: device int32 [n_q_heads]
 * [n_vertical], slash: device int32 [n_q_heads][n_slash], written ascending:
 * ready to be a dca_vs_mask. vertical_score / slash_score: device float32
 * [n_q_heads][seq] or NULL (then kept in the workspace). 1 <= n_vertical,
 * n_slash <= seq and 0 <= n_forced <= both (DCA_E_INVALID). workspace: at
 * least dca_vs_estimate_workspace_size bytes, 256-byte aligned; it holds the
 * keys rotated at their own index and the reduction scratch. The four outputs
 * must not overlap each other, the workspace, q or k, and q and k must not
 * overlap the workspace (DCA_E_INVALID). */
int dca_vs_estimate_workspace_size(int64_t seq, const dca_shape *shape, size_t *bytes);
int dca_vs_estimate(const void *q, const void *k, int64_t seq, int32_t n_last, double rope_base,
                    float yarn_scale, int32_t n_vertical, int32_t n_slash, int32_t n_forced,
                    const dca_shape *shape, int32_t *vertical, int32_t *slash,
                    float *vertical_score, float *slash_score, void *workspace,
                    size_t workspace_bytes, void *stream);

/* DCA decode of one new token per sequence [mizuki, Intra-/Successive-/
 * Inter-Chunk Attention, DCA + YaRN]: the token at sequence index pos (the
 * same for every batch entry) attends to the keys [0, pos] with the DCA
 * position map of row pos; the result equals row pos of a prefill over the
 * first pos + 1 tokens. q is [batch][n_q_heads][head_dim], k and v are
 * [batch][n_kv_heads][head_dim]: the new token's query, key and value
 * (device, read-only). The call first stores the rotated key and the value at
 * index pos of the workspace's key/value cache, so the keys [0, pos) must
 * have been stored by earlier dca_prefill, dca_prefill_chunk or dca_decode
 * calls on the same workspace with the same seq, C, W, rope_base, yarn_scale
 * and shape; seq is the capacity the workspace was sized for
 * (dca_workspace_size or dca_chunk_workspace_size with any max_rows) and
 * 0 <= pos < seq (DCA_E_INVALID). n_q_heads / n_kv_heads must be <= 32
 * (DCA_E_UNSUPPORTED); the vertical-slash mask is a prefill feature and is
 * not taken here. out: device [batch][n_q_heads][head_dim]; lse: device
 * float32 [batch][n_q_heads] or NULL. The scratch of the split-key reduction
 * lives in the workspace's query section. Errors are as for dca_prefill. */
int dca_decode(const void *q, const void *k, const void *v, void *out, float *lse,
               int64_t pos, int64_t seq, int64_t C, int64_t W, double rope_base,
               float yarn_scale, const dca_shape *shape, void *workspace,
               size_t workspace_bytes, void *stream);

/* dca_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments and errors as dca_decode, and outputs
 * identical to it, but the scratch of the split-key reduction (the rotated
 * query variants and the per-split partial results: batch * n_q_heads *
 * (3 * head_dim * element size, rounded up to 256 bytes, + 256 *
 * (head_dim + 2) * 4) bytes) lives in a static device array of
 * DCA_DECODE_STATIC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends, instead of in the workspace. The
 * workspace then only needs the key/value cache: any workspace for this
 * sequence from dca_fused_workspace_size, dca_workspace_size or
 * dca_chunk_workspace_size (mask NULL). A call whose scratch exceeds the
 * array returns DCA_E_UNSUPPORTED and enqueues nothing. The stream's device
 * must be the current device (the array's copy on that device is the one
 * the kernels use); otherwise DCA_E_INVALID, nothing enqueued. The first
 * call on a device looks up the array's address there (a HIP call, no
 * allocation); no call allocates or frees memory. Every call on one GPU shares that GPU's
 * array, whose contents the last call left (nothing in it needs to start at
 * zero): calls that overlap in time on one GPU -- on different streams or
 * host threads -- race on it and must not be made. */
#define DCA_DECODE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int dca_decode_static(const void *q, const void *k, const void *v, void *out, float *lse,
                      int64_t pos, int64_t seq, int64_t C, int64_t W, double rope_base,
                      float yarn_scale, const dca_shape *shape, void *workspace,
                      size_t workspace_bytes, void *stream);

/* The three stages of dca_prefill, callable one at a time on the same
 * workspace (for per-stage timing and checks):
 *   dca_remap      -- the RoPE/DCA pre-pass: writes the cos/sin table, the
 *                     three rotated query variants, the rotated keys (scaled
 *                     by yarn_scale * softmax_scale * log2(e), so that scores
 *                     come out of the matrix cores in base-2 exponent units)
 *                     and the value re-layout into the workspace [mizuki,
 *                     Inter-Chunk: only position indices change].
 *   dca_vs_index   -- mask -> per-head sorted key-tile list VT_h (tiles
 *                     holding a vertical column) and tile-distance list D_h
 *                     (distances delta < ceil(seq/64) whose slash interval
 *                     [max(0, 64 delta - 63), 64 delta + 63] holds an offset);
 *                     tile (t, kt) is active iff kt in VT_h or t - kt in D_h.
 *   dca_attention  -- the flash-style kernel over the workspace written by
 *                     dca_remap (and dca_vs_index when mask != NULL).
 * Arguments have the meaning they have in dca_prefill; each stage validates
 * them the same way. dca_attention needs the same seq, C, W, shape and mask
 * as the dca_remap / dca_vs_index calls that filled the workspace (the YaRN
 * temperature is applied by dca_remap). */
int dca_remap(const void *q, const void *k, const void *v,
              int64_t seq, int64_t C, int64_t W, double rope_base, float yarn_scale,
              const dca_shape *shape, void *workspace, size_t workspace_bytes,
              void *stream);
int dca_vs_index(int64_t seq, int64_t C, int64_t W, const dca_vs_mask *mask,
                 const dca_shape *shape, void *workspace, size_t workspace_bytes,
                 void *stream);
int dca_attention(void *out, float *lse, int64_t seq, int64_t C, int64_t W,
                  const dca_vs_mask *mask, const dca_shape *shape,
                  const void *workspace, size_t workspace_bytes, void *stream);

/* Checks (device): read back what the GPU stages computed.
 *
 * dca_debug_positions -- the device's own position map (the integer code the
 *   pre-pass runs) into device int32 arrays of seq entries each:
 *   pq_intra, pq_succ, pk; *pq_inter (device, one int32). All non-NULL.
 * dca_debug_tile_regions -- the device's classification of every 64 x 64
 *   (query tile, key tile) pair: out[t * n + kt] (device uint8, n =
 *   ceil(seq/64), n * n entries) = 0 intra, 1 successive, 2 inter, 255 for
 *   kt > t (not causal).
 * dca_debug_unpack -- copy one pre-pass array out of a workspace filled by
 *   dca_remap, in plain row-major [batch, heads, seq, head_dim] order and the
 *   shape's dtype: which = 0 Q intra, 1 Q successive, 2 Q inter (n_q_heads),
 *   3 rotated K (scaled as dca_remap states), 4 V (n_kv_heads). dst: device.
 * dca_debug_vs_lists -- copy the tile lists dca_vs_index wrote: vt and dl
 *   are device int32 [n_q_heads][n_tiles] (n_tiles = ceil(seq/64)), counts
 *   device int32 [n_q_heads] each.
 * dca_debug_vs_tiles -- the key tiles the attention kernel visits for one
 *   group of `group` (1 or 2) 64-row query tiles starting at query tile
 *   q_tile (a multiple of group) of head `head`, merged from the lists
 *   dca_vs_index wrote by the kernel's own iterator [mizuki, MInference
 *   sections: a 64x64 block is computed when a vertical column or a slash
 *   diagonal crosses it]: kt_out[i] ascending, mask_out[i] bit q set when
 *   tile kt_out[i] is active for query tile q_tile + q (device int32 /
 *   uint32 [cap]); *n_out (device int32) receives the full count, of which
 *   at most cap entries are written. Group 2 is the vertical-slash
 *   workgroup. The workspace must hold the lists of a dca_vs_index call with
 *   the same arguments. */
int dca_debug_positions(int64_t seq, int64_t C, int64_t W, int32_t *pq_intra,
                        int32_t *pq_succ, int32_t *pq_inter, int32_t *pk, void *stream);
int dca_debug_tile_regions(int64_t seq, int64_t C, uint8_t *out, void *stream);
int dca_debug_unpack(const void *workspace, size_t workspace_bytes, int which,
                     int64_t seq, int64_t C, int64_t W, const dca_shape *shape,
                     void *dst, void *stream);
int dca_debug_vs_lists(const void *workspace, size_t workspace_bytes, int64_t seq,
                       int64_t C, int64_t W, const dca_vs_mask *mask, const dca_shape *shape,
                       int32_t *vt, int32_t *vt_count, int32_t *dl, int32_t *dl_count,
                       void *stream);
int dca_debug_vs_tiles(const void *workspace, size_t workspace_bytes, int64_t seq,
                       int64_t C, int64_t W, const dca_vs_mask *mask, const dca_shape *shape,
                       int32_t head, int64_t q_tile, int32_t group, int32_t *kt_out,
                       uint32_t *mask_out, int32_t cap, int32_t *n_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DCA_H */
