/*
 * kvring.h -- C ABI of libkvring.so: write-time RoPE + FP8 ring KV cache,
 * delta rebase and FP8 window attention for one AMD MI355X (gfx950).
 *
 * The method (page references, cited by title and section):
 *   [AI-cache]   ai.info, "Characters funziona in tempo reale su quattro H100,
 *                afferma Runway", section "La gestione della cache spostata al
 *                momento della scrittura": the cache is a circular buffer so the
 *                window advances without copies; rotary position encoding and
 *                FP8 quantisation are applied once, when a frame enters the
 *                cache; positions reset every 42 steps and each reset applies a
 *                single delta rotation to the stored window.
 *   [NC-cache]   neurocartel.com blog "Runway Characters ... 4 H100", section
 *                "Кэш: 240 attention calls и работа на запись": 240 attention
 *                calls per step, each over 5788 slots of which 757 are new.
 *   [WC]         wechild.cn news item 1943: the original implementation
 *                re-applied RoPE, re-quantised and shifted the window on every
 *                call.
 *   [AI-latency] same ai.info page, section "Latenza dei turni e altre
 *                configurazioni GPU": FP8 attention that accepts per-head scales.
 *
 * Conventions shared by every entry point
 *   - All device pointers are caller-owned device memory (hipMalloc or a
 *     framework allocator); the library never allocates or frees.  Host
 *     pointers are marked "host".
 *   - Every launch is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Nothing synchronises; outputs are ready when the
 *     stream reaches that point.
 *   - No global mutable state: calls are re-entrant and thread-safe, except
 *     that calls writing the same buffers must be ordered by the caller.
 *   - Arguments are validated on the host before any launch; on error nothing
 *     is launched and a negative status is returned, with a message available
 *     from kvr_last_error() (thread-local).
 *   - Cache layout (one K and one V buffer pair per cache):
 *       codes  uint8  [n_layers][n_heads][window][head_dim]   OCP E4M3 bytes
 *       scales float  [n_layers][n_heads][window]             dequant factor
 *     A stored element decodes to e4m3(code) * scale, scale = row absmax / 448.
 *   - head_dim is 64 or 128; window and n_new are >= 1 and < 2^24.
 */
#ifndef KVRING_H
#define KVRING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define KVR_OK            0
#define KVR_EINVAL       -1   /* null pointer, size or range out of bounds        */
#define KVR_EALIGN       -2   /* pointer not 16-byte aligned                      */
#define KVR_EUNSUPPORTED -3   /* head_dim not in {64,128}, unknown dtype          */
#define KVR_ELAUNCH      -4   /* a HIP launch failed (text in kvr_last_error)     */

typedef enum { KVR_F32 = 0, KVR_BF16 = 1 } kvr_dtype;

/* Device cache buffers and their shape.  [AI-cache]
 * n_prefix (0 for a pure ring): slots [0, n_prefix) of every head hold a
 * fixed prefix written once with kv_write_prefix_rows and never moved; the
 * ring is slots [n_prefix, window), capacity window - n_prefix.  Ring state
 * (kvr_ring) and the ring arguments of every call (head, slot_start,
 * n_valid) are relative to the ring: ring slot s is cache slot n_prefix + s,
 * and the kvr_ring_* functions take the ring capacity as their window. */
typedef struct {
    uint8_t *k_codes;   /* [L][H][W][D] */
    uint8_t *v_codes;   /* [L][H][W][D] */
    float   *k_scales;  /* [L][H][W]    */
    float   *v_scales;  /* [L][H][W]    */
    int32_t  n_layers, n_heads, head_dim, window;
    int32_t  n_prefix;  /* 0 <= n_prefix < window */
} kvr_cache;

/* Ring state, a host POD shared by all layers of a cache.  [AI-cache]
 *   head     : slot the next new token goes to
 *   n_valid  : number of valid slots (<= window); the valid slots, oldest
 *              first, are (head - n_valid + i) mod window, i < n_valid
 *   pos_next : rotary position of the next new token                      */
typedef struct {
    int32_t head;
    int32_t n_valid;
    int64_t pos_next;
} kvr_ring;

/* Device table of fp32 (cos, sin) pairs of the rotary angles of a range of
 * positions: cs[(p - pos0) * head_dim/2 + i] = (cos, sin)(p * theta_i) with
 * theta_i = base^(-2i/head_dim), the angle formed in fp64 and cos/sin
 * evaluated in fp64 then rounded to fp32.  Filled by kv_rope_table_fill (the
 * base is that call's argument; the entry points reading a table only read
 * its rows). */
typedef struct {
    const float *cs;    /* device, [n_pos][head_dim/2][2] */
    int64_t      pos0;  /* first position held */
    int32_t      n_pos; /* number of positions held */
    int32_t      head_dim;
} kvr_rope_table;

/* ---- (a1) ring bookkeeping: pure host integer code, no GPU ----------------
 * [AI-cache]: a circular buffer; new token j of a chunk goes to slot
 * (head + j) mod window; after a chunk of n_new tokens the head advances by
 * n_new (mod window), n_valid grows to at most window and pos_next grows by
 * n_new; a position reset by delta lowers pos_next by delta. */
void    kvr_ring_init(kvr_ring *r);                                  /* all zero */
/* Slot of new token j (0 <= j < window) of the next chunk; -1 on bad input. */
int32_t kvr_ring_slot(const kvr_ring *r, int32_t window, int32_t j);
/* Slot of the oldest valid token, (head - n_valid) mod window; -1 on bad input. */
int32_t kvr_ring_logical_start(const kvr_ring *r, int32_t window);
/* Advance the ring past a written chunk.  KVR_EINVAL if n_new not in [1, window]
 * or the state is out of range. */
int32_t kvr_ring_after_write(kvr_ring *r, int32_t window, int32_t n_new);
/* Record a position reset by delta (pos_next -= delta); head and n_valid keep. */
int32_t kvr_ring_after_rebase(kvr_ring *r, int64_t delta);

/* ---- rotary table --------------------------------------------------------
 * Fills `cs` (device, n_pos * head_dim/2 float pairs) for positions
 * pos0 .. pos0 + n_pos - 1 (see kvr_rope_table).  [AI-cache] */
int32_t kv_rope_table_fill(float *cs, int64_t pos0, int32_t n_pos, int32_t head_dim,
                           double base, void *stream);

/* ---- (a2) write-time RoPE + FP8 ------------------------------------------
 * [AI-cache] [NC-cache] [WC].  For layers layer0 .. layer0+n_layers-1 and new
 * tokens j < n_new: K row (j, h) is rotated at position before->pos_next + j
 * (pairs (x[2i], x[2i+1]) by angle p * theta_i, fp32, no FMA), then K and V
 * rows are quantised (a = row absmax; scale = a / 448; code = E4M3 RNE of
 * y * (448 / a); a == 0 gives scale 0 and zero codes; when a < 2^-64 the
 * inverse and the products are formed from a and y times 2^64, exact, since
 * 448 / a alone can overflow fp32) and stored at slot
 * (before->head + j) mod window.  The ring itself is not modified: call
 * kvr_ring_after_write afterwards.
 *   k_new, v_new : device, per layer [n_new][n_heads][head_dim] of `dtype`,
 *                  layer l at element offset (l - layer0) * layer_stride_elems;
 *                  16-byte aligned; layer_stride_elems a multiple of 8.
 *   rope         : device table covering positions pos_next .. pos_next+n_new-1.
 * Errors: KVR_EINVAL (null, n_new not in [1, window], layer range, table range,
 * table shape), KVR_EALIGN, KVR_EUNSUPPORTED (head_dim, dtype; also more than
 * 32767 layers in one call, or n_layers * n_new of 2^31 or more: the kernel's
 * grid). */
int32_t kv_write_rope_quant(const kvr_cache *cache, const kvr_ring *before,
                            int32_t layer0, int32_t n_layers,
                            const void *k_new, const void *v_new, kvr_dtype dtype,
                            int64_t layer_stride_elems, int32_t n_new,
                            const kvr_rope_table *rope, void *stream);

/* ---- (a4) delta rebase on a position reset -------------------------------
 * [AI-cache].  Every valid K row of layers layer0 .. layer0+n_layers-1 (the
 * ring's n_valid slots) is dequantised (e4m3(code) * scale, fp32), rotated by
 * -delta (cos/sin of -delta * theta_i formed in fp64, rounded to fp32; fp32
 * rotation, no FMA) and re-quantised as in kv_write_rope_quant.  V rows are
 * not touched (V carries no rotation).  Afterwards call kvr_ring_after_rebase.
 * Errors: KVR_EINVAL (also |delta| > 2^53, where the fp64 angle stops being
 * exact), KVR_EUNSUPPORTED. */
int32_t kv_delta_rebase(const kvr_cache *cache, const kvr_ring *ring, int32_t layer0,
                        int32_t n_layers, int64_t delta, double rope_base, void *stream);

/* ---- (a3) FP8 window attention -------------------------------------------
 * [AI-cache] [NC-cache] [AI-latency].  For every head h and query i < n_q:
 *   O[i][h] = sum_j softmax_j(softmax_scale * q_i . k^_j) v^_j
 * over the n_valid cached keys of `layer` at slots (slot_start + j) mod window
 * (non-causal; every query sees every valid key; with a prefix, the n_prefix
 * prefix rows come first and the ring's keys are at cache slots n_prefix +
 * (slot_start + j) mod (window - n_prefix)), q_i rotated at position
 * q_pos_start + i with frequencies rope_base^(-2i/head_dim), k^ / v^ the
 * dequantised cache rows.  Keys are visited in
 * this logical order, so a linear window (slot_start = 0) holding the same
 * rows gives a bit-identical result.
 * On the GPU, Q goes into the FP8 matrix cores as two E4M3 terms (hi + lo)
 * with one power-of-two scale per query row; the softmax weights and the
 * dequantised V rows go into bf16 matrix products; accumulation is fp32 with
 * an online softmax.
 *   softmax_scale: > 0, or 0 for the default 1/sqrt(head_dim).
 *   q       : device [n_q][n_heads][head_dim] of `dtype`, 16-byte aligned.
 *   out     : device bf16 [n_q][n_heads][head_dim] (uint16 storage).
 *   n_splits: key-range splits per (head, query block); 0 picks one for the
 *             shape.  With more than one split, partial results go to `ws`
 *             and a second kernel combines them in a fixed order.
 *   ws      : device workspace of attn_fp8_window_workspace_bytes(...) bytes
 *             (may be NULL when that is 0), 256-byte aligned.
 * Errors: KVR_EINVAL (null, n_valid not in [1, window], slot_start out of
 * range, rope_base <= 1, softmax_scale negative or not finite, workspace too
 * small, out overlapping q, the query rotary rows or the workspace), KVR_EALIGN, KVR_EUNSUPPORTED (head_dim or dtype, or more than
 * 2^31 - 1 workgroups: ceil(n_q / 256) x n_heads x splits).
 * Range: the fp32 accumulators hold sums of up to window weights below 2^16
 * times the dequantised V values, so |V| must stay below about 2^99. */
size_t  attn_fp8_window_workspace_bytes(const kvr_cache *cache, int32_t n_q, int32_t n_valid,
                                        int32_t n_splits);
int32_t attn_fp8_window(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                        int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                        int64_t q_pos_start, float softmax_scale, double rope_base,
                        uint16_t *out, int32_t n_splits, void *ws, size_t ws_bytes,
                        void *stream);
/* The two launches of attn_fp8_window, callable one by one (same arguments,
 * same validation and errors): _partial runs the attention kernel, which
 * writes `out` itself when the effective split count is 1 and the split
 * partials to `ws` otherwise; _merge then combines the partials into `out`
 * (it launches nothing for one split).  attn_fp8_window == _partial followed
 * by _merge on the same stream, bit for bit.  [AI-cache] [AI-latency] */
int32_t attn_fp8_window_partial(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                                int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                                int64_t q_pos_start, float softmax_scale, double rope_base,
                                uint16_t *out, int32_t n_splits, void *ws, size_t ws_bytes,
                                void *stream);
int32_t attn_fp8_window_merge(const kvr_cache *cache, int32_t n_q, int32_t n_valid, int32_t n_splits,
                              uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* ---- the chunk's write fused into the call that first reads it -----------
 * [AI-cache] [NC-cache]: every call of a step reads a window whose newest
 * n_new rows are the step's chunk, rotated and quantised when written.  One
 * call that writes the chunk of `layer` and attends over the window holding
 * it, with the chunk's tokens as the queries (the step's first call of the
 * layer):
 *   - the write is kv_write_rope_quant of this one layer with state `before`
 *     (K row j rotated at position before->pos_next + j, stored at ring slot
 *     (before->head + j) mod capacity), the same bits;
 *   - the attention is attn_fp8_window over the window after that write
 *     (slot_start = kvr_ring_logical_start and n_valid of `before` advanced by
 *     n_new), query i at position before->pos_next + i, the same bits.
 * The ring is not modified: call kvr_ring_after_write afterwards.
 * The new keys are the last n_new in logical order; the key tiles are dealt
 * to the splits in turn (split s takes tiles s, s + S, ...), so they sit at
 * the end of every split.  When all of the launch's workgroups can be
 * resident on the GPU at once, it is one launch: every workgroup issues its
 * first tiles of old keys, stores its share of the chunk's rows with stores
 * that write through to memory, waits for them and counts itself done in the
 * control block; a workgroup whose split holds new keys waits for every
 * share (a bounded wait) before it loads its first tile holding new keys, and
 * loads those past stale cached copies.  When the workgroups could not all be
 * resident at once (a waiting workgroup could then hold a writer back), the
 * write kernel and then the plain attention call are launched instead, with
 * the same results.
 *   k_new, v_new, q : device [n_new][n_heads][head_dim] of `dtype`, 16-byte
 *               aligned.
 *   rope      : device table covering positions pos_next .. pos_next+n_new-1
 *               (the K rows' rotation); rope_base: the queries' rotary base;
 *               softmax_scale, out, n_splits: as attn_fp8_window.
 *   ws        : device workspace of at least
 *               attn_fp8_window_write_workspace_bytes(...) bytes, 256-byte
 *               aligned.  Its control block is the 256 bytes at offset
 *               ws_bytes - 256 rounded down to a multiple of 64 (the last 256
 *               bytes when ws_bytes is a multiple of 64) whatever the call's
 *               shape, so a workspace reused by calls of several shapes keeps
 *               it in one place.  uint32 words: [0] writers done, [1] waiting
 *               workgroups through, [2] waits that gave up, [3] a poll limit
 *               (0: the library's, 2^18 polls of about a microsecond each).
 *               Words 0..2 must be zero before the first call with this
 *               workspace (allocate it zeroed); every call leaves words 0 and
 *               1 zero.  A wait that gives up adds one to word 2 and turns
 *               that workgroup's output rows into NaN; the control block must
 *               then be zeroed again.  Calls sharing a workspace must be
 *               ordered (one stream).
 * Errors: those of kv_write_rope_quant (one layer) and of attn_fp8_window;
 * KVR_EINVAL for a missing or too small workspace, KVR_EALIGN for one not
 * 256-byte aligned. */
size_t  attn_fp8_window_write_workspace_bytes(const kvr_cache *cache, const kvr_ring *before,
                                              int32_t n_new, int32_t n_splits);
int32_t attn_fp8_window_write(const kvr_cache *cache, const kvr_ring *before, int32_t layer,
                              const void *k_new, const void *v_new, const void *q, kvr_dtype dtype,
                              int32_t n_new, const kvr_rope_table *rope, float softmax_scale,
                              double rope_base, uint16_t *out, int32_t n_splits, void *ws,
                              size_t ws_bytes, void *stream);

/* ---- allocation-free attention -------------------------------------------
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): attn_fp8_window
 * without the caller's workspace.  The split partials go to a scratch array
 * of KVR_NOALLOC_SCRATCH_BYTES that the library holds in device memory on
 * every GPU it runs on, until the process ends; its device address on a GPU
 * is looked up once, on the first call there.  This entry point calls no
 * allocator (no hipMalloc, no allocating library routine).  Nothing in the
 * scratch needs clearing between calls: every partial row the merge reads is
 * written earlier in the same call.  All calls on one GPU share that GPU's
 * scratch, so calls that overlap on one GPU (on two streams, or from two
 * threads without ordering) race: issue them on one stream.  This is the one
 * exception to "no global mutable state" above.
 * Arguments, results and errors as attn_fp8_window, less ws and ws_bytes;
 * also KVR_EINVAL when the call's partials (attn_fp8_window_workspace_bytes
 * for the same shape and split count) exceed KVR_NOALLOC_SCRATCH_BYTES (the
 * production shape, 12 heads x 757 queries in 7 splits, needs 17.3 MB), and
 * KVR_ELAUNCH when the scratch address cannot be obtained. */
#define KVR_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int32_t attn_fp8_window_noalloc(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                                int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                                int64_t q_pos_start, float softmax_scale, double rope_base,
                                uint16_t *out, int32_t n_splits, void *stream);

/* ---- (a5) naive per-call upkeep (the original implementation) ------------
 * [WC] [AI-cache] [NC-cache].  Shift the linear, un-rotated window: the new
 * window is src rows [drop, n_valid_before) followed by the n_new new rows,
 * drop = max(0, n_valid_before + n_new - window); write it to lin_*_dst, then
 * rotate every K row at its absolute position (row i at
 * pos_next_before + n_new - n_after + i, n_after = min(n_valid_before + n_new,
 * window)) and quantise every K and V row exactly as kv_write_rope_quant does,
 * into linear codes [n_heads][window][head_dim] and scales [n_heads][window].
 *   lin_*_src, lin_*_dst : device [n_heads][window][head_dim] of `dtype`;
 *                          src and dst must not overlap (ping-pong buffers).
 *   k_new, v_new         : device [n_new][n_heads][head_dim] of `dtype`.
 *   rope                 : table covering the n_after positions.
 * No output (lin_*_dst, codes, scales) may overlap an input or another
 * output; the inputs may alias each other.
 * Errors: KVR_EINVAL (also overlapping buffers), KVR_EALIGN, KVR_EUNSUPPORTED. */
int32_t naive_upkeep(const void *lin_k_src, const void *lin_v_src,
                     const void *k_new, const void *v_new, kvr_dtype dtype, int32_t n_new,
                     int32_t n_valid_before, int64_t pos_next_before,
                     int32_t n_heads, int32_t head_dim, int32_t window,
                     const kvr_rope_table *rope,
                     void *lin_k_dst, void *lin_v_dst,
                     uint8_t *k_codes, uint8_t *v_codes, float *k_scales, float *v_scales,
                     void *stream);

/* ---- 3-D (frame, row, column) rotary encoding ------------------------------
 * The pages describe a video diffusion transformer and do not spell out its
 * rotary encoding; this is the 3-D reading.  A token carries integer
 * coordinates (t, y, x): frame index, row and column.  The head_dim/2
 * interleaved pairs are cut into axis_pairs[0] frame pairs, then axis_pairs[1]
 * row pairs, then axis_pairs[2] column pairs (axis_pairs[0] >= 1, the sum
 * = head_dim/2); pair k of axis a's group turns by coord[a] * theta with
 * theta = base^(-k / axis_pairs[a]) -- the 1-D rule of that group's slice.
 * axis_pairs = (head_dim/2, 0, 0) is exactly the 1-D encoding at t.
 * A position reset moves the frame index only: kv_delta_rebase_axes with
 * delta = (d, 0, 0) rotates only the frame pairs.  [AI-cache] [NC-cache] */

/* Fills cs (device, n_tok * head_dim/2 float pairs, 16-byte aligned) with the
 * (cos, sin) of every pair of tokens 0 .. n_tok-1 at coords (device int32
 * [n_tok][3]); angle and trig in fp64, rounded to fp32.
 * Errors: KVR_EINVAL (null, n_tok < 1, bad axis_pairs, base <= 1), KVR_EALIGN,
 * KVR_EUNSUPPORTED (head_dim). */
int32_t kv_rope3d_table_fill(float *cs, const int32_t *coords, int32_t n_tok, int32_t head_dim,
                             const int32_t axis_pairs[3], double base, void *stream);

/* kv_write_rope_quant with the rotation of new token j taken from row j of
 * cs_rows (device [n_new][head_dim/2][2] fp32, 16-byte aligned; e.g. from
 * kv_rope3d_table_fill) instead of a position.  Slots, quantisation,
 * arguments and errors are those of kv_write_rope_quant. */
int32_t kv_write_rope_quant_rows(const kvr_cache *cache, const kvr_ring *before,
                                 int32_t layer0, int32_t n_layers,
                                 const void *k_new, const void *v_new, kvr_dtype dtype,
                                 int64_t layer_stride_elems, int32_t n_new,
                                 const float *cs_rows, void *stream);

/* kv_delta_rebase with one shift per axis (host int64[3]): every valid K row is
 * dequantised, rotated by -delta[a] on the pairs of axis a (cos/sin of
 * -delta[a] * theta formed in fp64, rounded to fp32) and re-quantised.
 * delta = (d, 0, 0) is the frame-only reset; with axis_pairs = (head_dim/2, 0,
 * 0) this is kv_delta_rebase(d) bit for bit.  Errors as kv_delta_rebase, plus
 * KVR_EINVAL for a null delta or bad axis_pairs. */
int32_t kv_delta_rebase_axes(const kvr_cache *cache, const kvr_ring *ring, int32_t layer0,
                             int32_t n_layers, const int64_t delta[3], const int32_t axis_pairs[3],
                             double rope_base, void *stream);

/* attn_fp8_window with query i rotated by row i of q_cs_rows (device
 * [n_q][head_dim/2][2] fp32, 16-byte aligned; the chunk's own rows when the
 * queries are the chunk's new tokens) instead of a position.  Everything else
 * -- keys, splits, workspace, output, errors -- as attn_fp8_window. */
int32_t attn_fp8_window_rows(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                             int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                             const float *q_cs_rows, float softmax_scale, uint16_t *out,
                             int32_t n_splits, void *ws, size_t ws_bytes, void *stream);

/* The queries' (cos, sin) rows in the layout the attention kernel loads
 * them in (each of its loads then reads whole lines): kv_rope_query_lanes
 * rearranges rows [n_q][head_dim/2][2] (e.g. the chunk's rows from
 * kv_rope3d_table_fill) into `lanes` (device, 16-byte aligned, of
 * kv_rope_query_lanes_bytes(n_q, head_dim) bytes; an opaque layout that only
 * attn_fp8_window_lanes reads), once for every call that uses the same rows
 * (e.g. all layers and passes of a step: the queries are the chunk's tokens,
 * at the chunk's positions, in every call).  attn_fp8_window_lanes is
 * attn_fp8_window_rows taking that buffer: same results bit for bit.  The
 * rows may equally be those of the 1-D rotary table at the chunk's positions
 * (a slice of a kvr_rope_table): the attention kernel then loads the cos/sin
 * it would otherwise form itself.
 * Errors: KVR_EINVAL (null, n_q out of range), KVR_EALIGN, KVR_EUNSUPPORTED;
 * the bytes function returns 0 for bad input.  [AI-cache] */
size_t  kv_rope_query_lanes_bytes(int32_t n_q, int32_t head_dim);
int32_t kv_rope_query_lanes(const float *cs_rows, int32_t n_q, int32_t head_dim, float *lanes,
                            void *stream);
int32_t attn_fp8_window_lanes(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                              int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                              const float *q_lanes, float softmax_scale, uint16_t *out,
                              int32_t n_splits, void *ws, size_t ws_bytes, void *stream);
/* The first of attn_fp8_window_lanes's two launches (the attention kernel),
 * as attn_fp8_window_partial is for attn_fp8_window; attn_fp8_window_merge
 * completes it. */
int32_t attn_fp8_window_lanes_partial(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                                      int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                                      const float *q_lanes, float softmax_scale, uint16_t *out,
                                      int32_t n_splits, void *ws, size_t ws_bytes, void *stream);

/* Writes n_tok prefix tokens (rotation of token j from row j of cs_rows,
 * device [n_tok][head_dim/2][2] fp32) to prefix slots slot0 .. slot0+n_tok-1
 * of layers layer0 .. layer0+n_layers-1, quantised as in kv_write_rope_quant.
 * The prefix is the reading taken for the window's fixed, non-rolling part:
 * its rows keep their own coordinates, so no rebase touches them; attention
 * sees them before the ring's keys.  Errors: KVR_EINVAL (null, slot range not
 * inside [0, n_prefix), layer range), KVR_EALIGN, KVR_EUNSUPPORTED.
 * [AI-cache] [NC-cache] */
int32_t kv_write_prefix_rows(const kvr_cache *cache, int32_t slot0, int32_t layer0, int32_t n_layers,
                             const void *k_new, const void *v_new, kvr_dtype dtype,
                             int64_t layer_stride_elems, int32_t n_tok, const float *cs_rows,
                             void *stream);

/* Text of the last error on this thread ("" if none). */
const char *kvr_last_error(void);

/* Library version, e.g. "0.1.0". */
const char *kvr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVRING_H */
