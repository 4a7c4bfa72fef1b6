// kvring_host.cpp -- host side of libkvring: ring bookkeeping, argument
// validation and kernel launches for the entry points of include/kvring.h.
//
// Page references (cited by title and section):
//   [AI-cache] ai.info, "Characters funziona in tempo reale su quattro H100,
//              afferma Runway", section "La gestione della cache spostata al
//              momento della scrittura" (circular buffer, write-time RoPE and
//              FP8, one delta rotation per position reset).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kvr_internal.h"
#include "kvring.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int32_t ok() {
    g_err[0] = '\0';
    return KVR_OK;
}

int32_t launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KVR_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int32_t kMaxExtent = 1 << 24;
// rotary shifts must be exact in the fp64 angle product
constexpr int64_t kMaxDelta = (int64_t)1 << 53;

int32_t check_head_dim(int32_t D) {
    if (D != 64 && D != 128) return fail(KVR_EUNSUPPORTED, "head_dim %d not in {64,128}", D);
    return KVR_OK;
}

int32_t check_cache(const kvr_cache *c) {
    if (!c) return fail(KVR_EINVAL, "cache is NULL");
    if (int32_t r = check_head_dim(c->head_dim)) return r;
    if (!c->k_codes || !c->v_codes || !c->k_scales || !c->v_scales)
        return fail(KVR_EINVAL, "cache buffer pointer is NULL");
    if (!aligned16(c->k_codes) || !aligned16(c->v_codes) || !aligned16(c->k_scales) ||
        !aligned16(c->v_scales))
        return fail(KVR_EALIGN, "cache buffers must be 16-byte aligned");
    if (c->n_layers < 1 || c->n_heads < 1 || c->window < 1 || c->window >= kMaxExtent ||
        c->n_heads >= kMaxExtent || c->n_layers >= kMaxExtent)
        return fail(KVR_EINVAL, "cache shape out of range (L=%d H=%d W=%d)", c->n_layers,
                    c->n_heads, c->window);
    if (c->n_prefix < 0 || c->n_prefix >= c->window)
        return fail(KVR_EINVAL, "n_prefix %d not in [0,%d)", c->n_prefix, c->window);
    return KVR_OK;
}

// Ring capacity of a cache: the slots after the fixed prefix.
int32_t ring_cap(const kvr_cache *c) { return c->window - c->n_prefix; }

int32_t check_ring(const kvr_ring *r, int32_t W) {
    if (!r) return fail(KVR_EINVAL, "ring is NULL");
    if (r->head < 0 || r->head >= W) return fail(KVR_EINVAL, "ring head %d not in [0,%d)", r->head, W);
    if (r->n_valid < 0 || r->n_valid > W)
        return fail(KVR_EINVAL, "ring n_valid %d not in [0,%d]", r->n_valid, W);
    return KVR_OK;
}

int32_t check_dtype(kvr_dtype dt) {
    if (dt != KVR_F32 && dt != KVR_BF16) return fail(KVR_EUNSUPPORTED, "unknown dtype %d", (int)dt);
    return KVR_OK;
}

// Table rows for positions [p0, p0 + n) must exist; returns the row pointer.
int32_t table_rows(const kvr_rope_table *t, int32_t D, int64_t p0, int64_t n, const float **row) {
    if (!t || !t->cs) return fail(KVR_EINVAL, "rotary table is NULL");
    if (t->head_dim != D)
        return fail(KVR_EINVAL, "rotary table head_dim %d != %d", t->head_dim, D);
    if (!aligned16(t->cs)) return fail(KVR_EALIGN, "rotary table must be 16-byte aligned");
    if (p0 < t->pos0 || p0 + n > t->pos0 + (int64_t)t->n_pos)
        return fail(KVR_EINVAL, "positions [%lld,%lld) outside rotary table [%lld,%lld)",
                    (long long)p0, (long long)(p0 + n), (long long)t->pos0,
                    (long long)(t->pos0 + t->n_pos));
    *row = t->cs + (p0 - t->pos0) * D;
    return KVR_OK;
}

kvr::ThetaTable make_theta(int32_t D, double base) {
    kvr::ThetaTable th{};
    for (int i = 0; i < D / 2; ++i) th.t[i] = pow(base, -2.0 * (double)i / (double)D);
    return th;
}

// Number of key-range splits actually used: the requested count (0 = the
// shape's default) clamped to the number of 64-key tiles, then reduced to the
// fewest splits whose largest share is still ceil(tiles / requested) tiles
// (the same longest split, fewer partials to merge).  *tps receives that
// largest share; the tiles are dealt to the splits in turn.
int32_t effective_splits(int32_t n_heads, int32_t n_q, int32_t n_valid, int32_t requested,
                         int32_t *tps) {
    const int32_t tiles = (n_valid + 63) / 64;
    int32_t s = requested > 0 ? requested : kvr::attn_default_splits(n_heads, n_q, n_valid);
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    *tps = (tiles + s - 1) / s;
    return (tiles + *tps - 1) / *tps;
}

// The write kernel's grid: one workgroup per two new tokens of each (layer,
// K/V), numbered with 32-bit block indices; the second extent is 2 n_layers.
int32_t check_write_grid(int32_t n_layers, int32_t n_new) {
    const int64_t gy = 2 * (int64_t)n_layers, gx = ((int64_t)n_new + 1) / 2;
    if (gy > 65535 || gx * gy >= (int64_t{1} << 31))
        return fail(KVR_EUNSUPPORTED, "a write of %d layers x %d tokens exceeds the kernel's grid", n_layers,
                    n_new);
    return KVR_OK;
}

int32_t mod_w(int64_t x, int32_t W) {
    int64_t r = x % W;
    return (int32_t)(r < 0 ? r + W : r);
}

}  // namespace

extern "C" {

const char *kvr_last_error(void) { return g_err; }

const char *kvr_version(void) { return "0.1.0"; }

// ---- (a1) ring bookkeeping [AI-cache] -----------------------------------
void kvr_ring_init(kvr_ring *r) {
    if (r) {
        r->head = 0;
        r->n_valid = 0;
        r->pos_next = 0;
    }
}

int32_t kvr_ring_slot(const kvr_ring *r, int32_t window, int32_t j) {
    if (!r || window < 1 || j < 0 || j >= window || r->head < 0 || r->head >= window) return -1;
    return mod_w((int64_t)r->head + j, window);
}

int32_t kvr_ring_logical_start(const kvr_ring *r, int32_t window) {
    if (!r || window < 1 || r->head < 0 || r->head >= window || r->n_valid < 0 ||
        r->n_valid > window)
        return -1;
    return mod_w((int64_t)r->head - r->n_valid, window);
}

int32_t kvr_ring_after_write(kvr_ring *r, int32_t window, int32_t n_new) {
    if (window < 1) return fail(KVR_EINVAL, "window %d < 1", window);
    if (int32_t e = check_ring(r, window)) return e;
    if (n_new < 1 || n_new > window) return fail(KVR_EINVAL, "n_new %d not in [1,%d]", n_new, window);
    r->head = mod_w((int64_t)r->head + n_new, window);
    r->n_valid = r->n_valid + n_new < window ? r->n_valid + n_new : window;
    r->pos_next += n_new;
    return ok();
}

int32_t kvr_ring_after_rebase(kvr_ring *r, int64_t delta) {
    if (!r) return fail(KVR_EINVAL, "ring is NULL");
    r->pos_next -= delta;
    return ok();
}

// ---- rotary table -------------------------------------------------------
int32_t kv_rope_table_fill(float *cs, int64_t pos0, int32_t n_pos, int32_t head_dim, double base,
                           void *stream) {
    if (int32_t e = check_head_dim(head_dim)) return e;
    if (!cs) return fail(KVR_EINVAL, "table pointer is NULL");
    if (!aligned16(cs)) return fail(KVR_EALIGN, "table must be 16-byte aligned");
    if (n_pos < 1) return fail(KVR_EINVAL, "n_pos %d < 1", n_pos);
    if (!(base > 1.0) || !isfinite(base)) return fail(KVR_EINVAL, "rotary base must be > 1");
    return launch_status(kvr::launch_rope_table(cs, pos0, n_pos, head_dim,
                                                make_theta(head_dim, base),
                                                static_cast<hipStream_t>(stream)),
                         "rope table");
}

// ---- (a2) write-time RoPE + FP8 [AI-cache] -------------------------------
int32_t kv_write_rope_quant(const kvr_cache *cache, const kvr_ring *before, int32_t layer0,
                            int32_t n_layers, const void *k_new, const void *v_new,
                            kvr_dtype dtype, int64_t layer_stride_elems, int32_t n_new,
                            const kvr_rope_table *rope, void *stream) {
    if (int32_t e = check_cache(cache)) return e;
    const int32_t W = ring_cap(cache), D = cache->head_dim;
    if (int32_t e = check_ring(before, W)) return e;
    if (int32_t e = check_dtype(dtype)) return e;
    if (!k_new || !v_new) return fail(KVR_EINVAL, "k_new/v_new is NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(KVR_EALIGN, "k_new/v_new not 16-byte aligned");
    if (n_new < 1 || n_new > W) return fail(KVR_EINVAL, "n_new %d not in [1,%d]", n_new, W);
    if (layer0 < 0 || n_layers < 1 || layer0 + n_layers > cache->n_layers)
        return fail(KVR_EINVAL, "layers [%d,%d) outside cache of %d", layer0, layer0 + n_layers,
                    cache->n_layers);
    if (int32_t e = check_write_grid(n_layers, n_new)) return e;
    const int64_t per_layer = (int64_t)n_new * cache->n_heads * D;
    if (n_layers > 1 && (layer_stride_elems < per_layer || layer_stride_elems % 8 != 0))
        return fail(KVR_EINVAL, "layer_stride_elems %lld must be >= %lld and a multiple of 8",
                    (long long)layer_stride_elems, (long long)per_layer);
    const float *cs;
    if (int32_t e = table_rows(rope, D, before->pos_next, n_new, &cs)) return e;
    kvr::WriteArgs a{};
    a.k_codes = cache->k_codes;
    a.v_codes = cache->v_codes;
    a.k_scales = cache->k_scales;
    a.v_scales = cache->v_scales;
    a.k_new = k_new;
    a.v_new = v_new;
    a.layer_stride = n_layers > 1 ? layer_stride_elems : 0;
    a.cs = cs;
    a.n_heads = cache->n_heads;
    a.window = cache->window;
    a.prefix = cache->n_prefix;
    a.cap = W;
    a.head = before->head;
    a.n_new = n_new;
    a.layer0 = layer0;
    a.n_layers = n_layers;
    a.dtype = dtype;
    return launch_status(kvr::launch_write(a, D, static_cast<hipStream_t>(stream)), "write");
}

// ---- (a4) delta rebase [AI-cache] ---------------------------------------
int32_t kv_delta_rebase(const kvr_cache *cache, const kvr_ring *ring, int32_t layer0,
                        int32_t n_layers, int64_t delta, double rope_base, void *stream) {
    if (int32_t e = check_cache(cache)) return e;
    const int32_t W = ring_cap(cache), D = cache->head_dim;
    if (int32_t e = check_ring(ring, W)) return e;
    if (layer0 < 0 || n_layers < 1 || layer0 + n_layers > cache->n_layers)
        return fail(KVR_EINVAL, "layers [%d,%d) outside cache of %d", layer0, layer0 + n_layers,
                    cache->n_layers);
    if (!(rope_base > 1.0) || !isfinite(rope_base)) return fail(KVR_EINVAL, "rotary base must be > 1");
    if (delta < -kMaxDelta || delta > kMaxDelta)
        return fail(KVR_EINVAL, "delta %lld outside [-2^53, 2^53]", (long long)delta);
    if (ring->n_valid == 0) return ok();
    // cos/sin of -delta * theta_i: fp64 angle and trig, rounded to fp32
    kvr::CosSinTable rot{};
    const kvr::ThetaTable th = make_theta(D, rope_base);
    for (int i = 0; i < D / 2; ++i) {
        const double ang = (double)(-delta) * th.t[i];
        rot.cs[2 * i] = (float)cos(ang);
        rot.cs[2 * i + 1] = (float)sin(ang);
    }
    kvr::RebaseArgs a{};
    a.k_codes = cache->k_codes;
    a.k_scales = cache->k_scales;
    a.n_heads = cache->n_heads;
    a.window = cache->window;
    a.prefix = cache->n_prefix;
    a.cap = W;
    a.start = kvr_ring_logical_start(ring, W);
    a.n_valid = ring->n_valid;
    a.layer0 = layer0;
    a.n_layers = n_layers;
    return launch_status(kvr::launch_rebase(a, rot, D, static_cast<hipStream_t>(stream)), "rebase");
}

// ---- (a3) FP8 window attention --------------------------------------------
size_t attn_fp8_window_workspace_bytes(const kvr_cache *cache, int32_t n_q, int32_t n_valid,
                                       int32_t n_splits) {
    if (!cache || n_q < 1 || n_valid < 0 || n_splits < 0 || n_valid + cache->n_prefix < 1) return 0;
    int32_t tps;
    n_splits = effective_splits(cache->n_heads, n_q, n_valid + cache->n_prefix, n_splits, &tps);
    return kvr::attn_workspace_bytes(cache->n_heads, cache->head_dim, n_q, n_splits);
}

namespace {

// Workspace of a call with n_splits > 1: fp16 partial rows, then (max, sum).
int32_t check_workspace(size_t need, const void *ws, size_t ws_bytes) {
    if (need == 0) return KVR_OK;
    if (!ws) return fail(KVR_EINVAL, "workspace of %zu bytes required", need);
    if (ws_bytes < need) return fail(KVR_EINVAL, "workspace %zu < %zu bytes", ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(KVR_EALIGN, "workspace must be 256-byte aligned");
    return KVR_OK;
}

void set_partials(kvr::AttnArgs &a, void *ws, int32_t n_heads, int32_t D, int32_t n_q, int32_t n_splits) {
    if (n_splits <= 1) return;
    const size_t rows = (size_t)n_splits * n_q * n_heads;
    const size_t o_bytes = (rows * D * sizeof(uint16_t) + 255) / 256 * 256;
    a.part_o = static_cast<uint16_t *>(ws);
    a.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + o_bytes);
}

// Validation and kernel arguments shared by attn_fp8_window and its two parts.
// rope_base: the rotary base of the position form (the kernel forms the
// queries' angles from it); NULL for the row and lane forms, which take the
// queries' (cos, sin) from q_cs instead.
int32_t attn_setup(kvr::AttnArgs &a, const kvr_cache *cache, int32_t layer, int32_t slot_start,
                   int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                   int64_t q_pos_start, float softmax_scale, const double *rope_base, uint16_t *out,
                   int32_t n_splits, void *ws, size_t ws_bytes, const float *q_cs = nullptr,
                   bool q_cs_lanes = false) {
    if (int32_t e = check_cache(cache)) return e;
    const int32_t W = ring_cap(cache), D = cache->head_dim;
    if (int32_t e = check_dtype(dtype)) return e;
    if (layer < 0 || layer >= cache->n_layers)
        return fail(KVR_EINVAL, "layer %d outside cache of %d", layer, cache->n_layers);
    if (n_valid < (cache->n_prefix > 0 ? 0 : 1) || n_valid > W)
        return fail(KVR_EINVAL, "n_valid %d not in [%d,%d]", n_valid, cache->n_prefix > 0 ? 0 : 1, W);
    if (slot_start < 0 || slot_start >= W)
        return fail(KVR_EINVAL, "slot_start %d not in [0,%d)", slot_start, W);
    const int32_t n_keys = n_valid + cache->n_prefix;
    if (n_q < 1 || n_q >= kMaxExtent) return fail(KVR_EINVAL, "n_q %d out of range", n_q);
    if (!q || !out) return fail(KVR_EINVAL, "q/out is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(KVR_EALIGN, "q/out not 16-byte aligned");
    if (softmax_scale == 0.0f) softmax_scale = (float)(1.0 / sqrt((double)D));   // the default 1/sqrt(D)
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale))
        return fail(KVR_EINVAL, "softmax_scale must be 0 (default) or positive and finite");
    if (rope_base && (!(*rope_base > 1.0) || !isfinite(*rope_base)))
        return fail(KVR_EINVAL, "rotary base must be > 1");
    if (!rope_base && !q_cs) return fail(KVR_EINVAL, "query rotary rows pointer is NULL");
    if (n_splits < 0) return fail(KVR_EINVAL, "n_splits %d < 0", n_splits);
    int32_t tps;
    n_splits = effective_splits(cache->n_heads, n_q, n_keys, n_splits, &tps);
    // one workgroup per (query block, head, split), numbered with 32-bit indices
    if ((int64_t)kvr::attn_query_blocks(n_q) * cache->n_heads * n_splits >= (int64_t{1} << 31))
        return fail(KVR_EUNSUPPORTED, "%d queries x %d heads x %d splits exceed the attention kernel's grid", n_q,
                    cache->n_heads, n_splits);
    if (int32_t e = check_workspace(kvr::attn_workspace_bytes(cache->n_heads, D, n_q, n_splits), ws, ws_bytes))
        return e;
    if (q_cs && !aligned16(q_cs)) return fail(KVR_EALIGN, "query rotary rows not 16-byte aligned");
    {
        // out is written while other workgroups still read q, the rotary rows
        // and the partials: it may overlap none of them
        const size_t rows = (size_t)n_q * cache->n_heads;
        const char *o = reinterpret_cast<const char *>(out);
        const size_t ob = rows * D * 2;
        auto overlaps = [&](const void *p, size_t n) {
            const char *x = static_cast<const char *>(p);
            return p && n && o < x + n && x < o + ob;
        };
        if (overlaps(q, rows * D * (dtype == KVR_BF16 ? 2 : 4))) return fail(KVR_EINVAL, "out overlaps q");
        // the position form has no rows; the row form [n_q][D/2][2] fp32, the lane form
        // its padded load order
        const size_t cs_bytes = !q_cs ? 0 : q_cs_lanes ? kvr::query_lanes_bytes(n_q, D) : (size_t)n_q * D * 4;
        if (overlaps(q_cs, cs_bytes)) return fail(KVR_EINVAL, "out overlaps the query rotary rows");
        if (overlaps(ws, kvr::attn_workspace_bytes(cache->n_heads, D, n_q, n_splits)))
            return fail(KVR_EINVAL, "out overlaps the workspace");
    }
    a = kvr::AttnArgs{};
    a.q_cs = q_cs;
    a.q_cs_lanes = q_cs_lanes ? 1 : 0;
    const int64_t lay = (int64_t)layer * cache->n_heads * W;
    a.k_codes = cache->k_codes + lay * D;
    a.v_codes = cache->v_codes + lay * D;
    a.k_scales = cache->k_scales + lay;
    a.v_scales = cache->v_scales + lay;
    a.q = q;
    if (rope_base) {
        a.rev = make_theta(D, *rope_base);
        for (int i = 0; i < D / 2; ++i) a.rev.t[i] *= 0.15915494309189535;   // 1 / (2 pi)
        a.rev_step = pow(*rope_base, -32.0 / (double)D);
        a.q_pos0 = q_pos_start;
    }
    a.out = out;
    a.n_heads = cache->n_heads;
    a.window = cache->window;
    a.prefix = cache->n_prefix;
    a.cap = W;
    a.slot_start = slot_start;
    a.n_valid = n_keys;
    a.n_q = n_q;
    a.dtype = dtype;
    a.n_splits = n_splits;
    a.softmax_scale = softmax_scale;
    set_partials(a, ws, cache->n_heads, D, n_q, n_splits);
    return KVR_OK;
}

// Validation and kernel arguments of the merge alone: the partials' layout
// follows from the cache shape, n_q and the effective split count.
int32_t merge_setup(kvr::AttnArgs &a, const kvr_cache *cache, int32_t n_q, int32_t n_valid,
                    int32_t n_splits, uint16_t *out, void *ws, size_t ws_bytes) {
    if (int32_t e = check_cache(cache)) return e;
    const int32_t W = ring_cap(cache), D = cache->head_dim;
    if (n_valid < (cache->n_prefix > 0 ? 0 : 1) || n_valid > W)
        return fail(KVR_EINVAL, "n_valid %d not in [%d,%d]", n_valid, cache->n_prefix > 0 ? 0 : 1, W);
    n_valid += cache->n_prefix;
    if (n_q < 1 || n_q >= kMaxExtent) return fail(KVR_EINVAL, "n_q %d out of range", n_q);
    if (!out) return fail(KVR_EINVAL, "out is NULL");
    if (!aligned16(out)) return fail(KVR_EALIGN, "out not 16-byte aligned");
    if (n_splits < 0) return fail(KVR_EINVAL, "n_splits %d < 0", n_splits);
    int32_t tps;
    n_splits = effective_splits(cache->n_heads, n_q, n_valid, n_splits, &tps);
    a = kvr::AttnArgs{};
    a.out = out;
    a.n_heads = cache->n_heads;
    a.window = cache->window;
    a.n_valid = n_valid;
    a.n_q = n_q;
    a.n_splits = n_splits;
    if (int32_t e = check_workspace(kvr::attn_workspace_bytes(cache->n_heads, D, n_q, n_splits), ws, ws_bytes))
        return e;
    set_partials(a, ws, cache->n_heads, D, n_q, n_splits);
    return KVR_OK;
}

}  // namespace

int32_t attn_fp8_window(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                        int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                        int64_t q_pos_start, float softmax_scale, double rope_base,
                        uint16_t *out, int32_t n_splits, void *ws, size_t ws_bytes,
                        void *stream) {
    kvr::AttnArgs a;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, n_valid, q, dtype, n_q, q_pos_start,
                               softmax_scale, &rope_base, out, n_splits, ws, ws_bytes))
        return e;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int32_t e = launch_status(kvr::launch_attention_main(a, cache->head_dim, s), "attention"))
        return e;
    return launch_status(kvr::launch_attention_merge(a, cache->head_dim, s), "attention merge");
}

int32_t attn_fp8_window_partial(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                                int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                                int64_t q_pos_start, float softmax_scale, double rope_base,
                                uint16_t *out, int32_t n_splits, void *ws, size_t ws_bytes,
                                void *stream) {
    kvr::AttnArgs a;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, n_valid, q, dtype, n_q, q_pos_start,
                               softmax_scale, &rope_base, out, n_splits, ws, ws_bytes))
        return e;
    return launch_status(kvr::launch_attention_main(a, cache->head_dim, static_cast<hipStream_t>(stream)),
                         "attention");
}

int32_t attn_fp8_window_merge(const kvr_cache *cache, int32_t n_q, int32_t n_valid, int32_t n_splits,
                              uint16_t *out, void *ws, size_t ws_bytes, void *stream) {
    kvr::AttnArgs a;
    if (int32_t e = merge_setup(a, cache, n_q, n_valid, n_splits, out, ws, ws_bytes)) return e;
    return launch_status(kvr::launch_attention_merge(a, cache->head_dim, static_cast<hipStream_t>(stream)),
                         "attention merge");
}

// ---- the chunk's write fused into the call that first reads it -------------
// [AI-cache] [NC-cache]: every call reads a window whose newest n_new rows are
// the chunk; the step's first call of a layer writes them on the way.
namespace {

constexpr size_t kSyncBytes = 256;     // control block after the partials

size_t fused_sync_offset(size_t partial_bytes) { return (partial_bytes + 255) / 256 * 256; }

}  // namespace

size_t attn_fp8_window_write_workspace_bytes(const kvr_cache *cache, const kvr_ring *before,
                                             int32_t n_new, int32_t n_splits) {
    if (!cache || !before || n_new < 1 || n_splits < 0) return 0;
    const int32_t W = cache->window - cache->n_prefix;
    if (W < 1 || n_new > W || before->n_valid < 0 || before->n_valid > W) return 0;
    const int32_t n_valid = before->n_valid + n_new < W ? before->n_valid + n_new : W;
    return fused_sync_offset(attn_fp8_window_workspace_bytes(cache, n_new, n_valid, n_splits)) + kSyncBytes;
}

int32_t attn_fp8_window_write(const kvr_cache *cache, const kvr_ring *before, int32_t layer,
                              const void *k_new, const void *v_new, const void *q, kvr_dtype dtype,
                              int32_t n_new, const kvr_rope_table *rope, float softmax_scale,
                              double rope_base, uint16_t *out, int32_t n_splits, void *ws,
                              size_t ws_bytes, void *stream) {
    // the write's arguments, validated as kv_write_rope_quant validates them
    if (int32_t e = check_cache(cache)) return e;
    const int32_t W = ring_cap(cache), D = cache->head_dim;
    if (int32_t e = check_ring(before, W)) return e;
    if (int32_t e = check_dtype(dtype)) return e;
    if (!k_new || !v_new) return fail(KVR_EINVAL, "k_new/v_new is NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(KVR_EALIGN, "k_new/v_new not 16-byte aligned");
    if (n_new < 1 || n_new > W) return fail(KVR_EINVAL, "n_new %d not in [1,%d]", n_new, W);
    if (layer < 0 || layer >= cache->n_layers)
        return fail(KVR_EINVAL, "layer %d outside cache of %d", layer, cache->n_layers);
    const float *cs;
    if (int32_t e = table_rows(rope, D, before->pos_next, n_new, &cs)) return e;
    // the window after the write, and the chunk's tokens as the queries
    kvr_ring after = *before;
    if (int32_t e = kvr_ring_after_write(&after, W, n_new)) return e;
    const int32_t slot_start = kvr_ring_logical_start(&after, W);
    const size_t part = attn_fp8_window_workspace_bytes(cache, n_new, after.n_valid, n_splits);
    const size_t need = fused_sync_offset(part) + kSyncBytes;
    if (!ws) return fail(KVR_EINVAL, "workspace of %zu bytes required", need);
    if (ws_bytes < need) return fail(KVR_EINVAL, "workspace %zu < %zu bytes", ws_bytes, need);
    kvr::AttnArgs a;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, after.n_valid, q, dtype, n_new,
                               before->pos_next, softmax_scale, &rope_base, out, n_splits, ws, ws_bytes))
        return e;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(KVR_EALIGN, "workspace must be 256-byte aligned");
    {
        // nor the control block at the workspace's end (the partials are checked above)
        const char *o = reinterpret_cast<const char *>(out), *w = static_cast<const char *>(ws);
        if (o < w + ws_bytes && w < o + (size_t)n_new * cache->n_heads * D * 2)
            return fail(KVR_EINVAL, "out overlaps the workspace");
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // every workgroup writes a share of the chunk; a workgroup whose split
    // holds new keys (the last n_new in logical order: with the tiles dealt
    // to the splits in turn, the end of a split) waits for all of them
    const int32_t first_new = a.n_valid - n_new;
    const int64_t lay = (int64_t)layer * cache->n_heads * cache->window;
    const int32_t n_tiles = (a.n_valid + 63) / 64, S = a.n_splits;
    int32_t splits_new = 0;                          // splits whose last tile holds a new key
    for (int32_t sp = 0; sp < S; ++sp) {
        const int32_t n_s = (n_tiles - sp + S - 1) / S;
        if ((int64_t)(sp + (int64_t)(n_s - 1) * S) * 64 + 63 >= first_new) ++splits_new;
    }
    const int64_t grid = (int64_t)kvr::attn_query_blocks(n_new) * cache->n_heads * S;
    // the waiting workgroups need every writer to run, whatever order the
    // hardware dispatches them in: the fused launch only when all of its
    // workgroups fit on the GPU at once
    bool resident = false;
    {
        int dev = -1, max_blocks = 0;
        hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
        if (e == hipSuccess)
            e = kvr::attention_fused_resident(D, dtype, cache->n_prefix > 0, dev, &max_blocks);
        if (e != hipSuccess) return launch_status(e, "fused write and attention: resident workgroups");
        resident = grid <= max_blocks;
    }
    if (!resident) {
        // the launch would not be resident at once: the write kernel, then
        // the plain call
        kvr::WriteArgs w{};
        w.k_codes = cache->k_codes;
        w.v_codes = cache->v_codes;
        w.k_scales = cache->k_scales;
        w.v_scales = cache->v_scales;
        w.k_new = k_new;
        w.v_new = v_new;
        w.cs = cs;
        w.n_heads = cache->n_heads;
        w.window = cache->window;
        w.prefix = cache->n_prefix;
        w.cap = W;
        w.head = before->head;
        w.n_new = n_new;
        w.layer0 = layer;
        w.n_layers = 1;
        w.dtype = dtype;
        if (int32_t e = launch_status(kvr::launch_write(w, D, s), "write")) return e;
        if (int32_t e = launch_status(kvr::launch_attention_main(a, D, s), "attention")) return e;
        return launch_status(kvr::launch_attention_merge(a, D, s), "attention merge");
    }
    a.w_k = k_new;
    a.w_v = v_new;
    a.w_cs = cs;
    a.w_k_codes = cache->k_codes + lay * D;
    a.w_v_codes = cache->v_codes + lay * D;
    a.w_k_scales = cache->k_scales + lay;
    a.w_v_scales = cache->v_scales + lay;
    a.w_head = before->head;
    a.w_n_new = n_new;
    a.first_new = first_new;
    a.n_writers = (int32_t)grid;
    a.n_waiters = splits_new * cache->n_heads * kvr::attn_query_blocks(n_new);
    // the control block is the workspace's last 256 bytes (64-byte aligned),
    // wherever this call's partials end: a buffer reused by calls of other
    // shapes keeps its counters in one place
    a.sync = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + ((ws_bytes - kSyncBytes) & ~size_t{63}));
    if (int32_t e = launch_status(kvr::launch_attention_fused(a, D, s), "fused write and attention")) return e;
    return launch_status(kvr::launch_attention_merge(a, D, s), "attention merge");
}

// ---- allocation-free attention ------------------------------------------------
// The split partials of attn_fp8_window_noalloc live in `scratch`, a device
// array of the library's own (each GPU the library runs on holds one copy
// until the process ends).  In host code `scratch` names a host-side stand-in,
// not device memory: its device address on a GPU comes from
// hipGetSymbolAddress with that GPU current, taken once per GPU on the first
// call there and kept in g_scratch; only that address is ever passed on.
namespace {

__device__ __align__(256) uint8_t scratch[KVR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];          // device address of `scratch` per GPU, once known

// Device address of the scratch array on the GPU `stream` runs on.
int32_t scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVR_ELAUNCH, "device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KVR_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(KVR_ELAUNCH, "current device: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(KVR_ELAUNCH, "select device %d: %s", dev, hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess && e2 != hipSuccess)
                return fail(KVR_ELAUNCH, "restore device %d: %s", cur, hipGetErrorString(e2));
        }
        if (e != hipSuccess || !p)
            return fail(KVR_ELAUNCH, "scratch address on device %d: %s", dev, hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KVR_OK;
}

}  // namespace

int32_t attn_fp8_window_noalloc(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                                int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                                int64_t q_pos_start, float softmax_scale, double rope_base,
                                uint16_t *out, int32_t n_splits, void *stream) {
    // the partials this call needs (0 for one split, or for arguments that
    // attn_setup rejects below)
    const size_t need = attn_fp8_window_workspace_bytes(cache, n_q, n_valid, n_splits);
    if (need > KVR_NOALLOC_SCRATCH_BYTES)
        return fail(KVR_EINVAL, "split partials of %zu bytes exceed the %zu-byte scratch", need,
                    (size_t)KVR_NOALLOC_SCRATCH_BYTES);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // every argument is validated as attn_fp8_window validates it, with an
    // aligned stand-in for the workspace, before the device is touched; the
    // partials then point into the scratch
    kvr::AttnArgs a;
    void *const stand_in = need > 0 ? reinterpret_cast<void *>(uintptr_t{256}) : nullptr;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, n_valid, q, dtype, n_q, q_pos_start,
                               softmax_scale, &rope_base, out, n_splits, stand_in, need))
        return e;
    if (need > 0) {
        void *ws = nullptr;
        if (int32_t e = scratch_address(s, &ws)) return e;
        set_partials(a, ws, cache->n_heads, cache->head_dim, n_q, a.n_splits);
    }
    if (int32_t e = launch_status(kvr::launch_attention_main(a, cache->head_dim, s), "attention"))
        return e;
    return launch_status(kvr::launch_attention_merge(a, cache->head_dim, s), "attention merge");
}

// ---- 3-D (frame, row, column) rotary encoding -------------------------------
// The D/2 pairs are cut into n_t, n_y, n_x contiguous groups, one per axis;
// group a is the 1-D rule of its slice at that axis's coordinate (pair k of
// the group: theta = base^(-k / n_a)).
namespace {

int32_t check_axis_pairs(const int32_t *np, int32_t D) {
    if (!np) return fail(KVR_EINVAL, "axis_pairs is NULL");
    if (np[0] < 1 || np[1] < 0 || np[2] < 0 || np[0] + np[1] + np[2] != D / 2)
        return fail(KVR_EINVAL, "axis_pairs (%d, %d, %d) must be >= (1, 0, 0) and sum to %d", np[0], np[1],
                    np[2], D / 2);
    return KVR_OK;
}

kvr::AxisTheta make_axis_theta(const int32_t *np, double base) {
    kvr::AxisTheta th{};
    int i = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int k = 0; k < np[ax]; ++k, ++i) {
            th.t[i] = pow(base, -(double)k / (double)np[ax]);
            th.axis[i] = ax;
        }
    return th;
}

}  // namespace

int32_t kv_rope3d_table_fill(float *cs, const int32_t *coords, int32_t n_tok, int32_t head_dim,
                             const int32_t *axis_pairs, double base, void *stream) {
    if (int32_t e = check_head_dim(head_dim)) return e;
    if (int32_t e = check_axis_pairs(axis_pairs, head_dim)) return e;
    if (!cs || !coords) return fail(KVR_EINVAL, "table or coordinates pointer is NULL");
    if (!aligned16(cs)) return fail(KVR_EALIGN, "table must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(coords) & 3u) != 0) return fail(KVR_EALIGN, "coordinates not 4-byte aligned");
    if (n_tok < 1 || n_tok >= kMaxExtent) return fail(KVR_EINVAL, "n_tok %d out of range", n_tok);
    if (!(base > 1.0) || !isfinite(base)) return fail(KVR_EINVAL, "rotary base must be > 1");
    return launch_status(kvr::launch_rope3d_table(cs, coords, n_tok, head_dim, make_axis_theta(axis_pairs, base),
                                                  static_cast<hipStream_t>(stream)),
                         "3-D rope table");
}

int32_t kv_write_rope_quant_rows(const kvr_cache *cache, const kvr_ring *before, int32_t layer0,
                                 int32_t n_layers, const void *k_new, const void *v_new,
                                 kvr_dtype dtype, int64_t layer_stride_elems, int32_t n_new,
                                 const float *cs_rows, void *stream) {
    if (!cs_rows) return fail(KVR_EINVAL, "rotary rows pointer is NULL");
    if (!aligned16(cs_rows)) return fail(KVR_EALIGN, "rotary rows not 16-byte aligned");
    if (!cache) return fail(KVR_EINVAL, "cache is NULL");
    // the position form's validation, against a one-off table descriptor that
    // holds exactly the chunk's rows at the ring's next positions
    kvr_rope_table t{};
    t.cs = const_cast<float *>(cs_rows);
    t.pos0 = before ? before->pos_next : 0;
    t.n_pos = n_new;
    t.head_dim = cache->head_dim;
    return kv_write_rope_quant(cache, before, layer0, n_layers, k_new, v_new, dtype, layer_stride_elems,
                               n_new, &t, stream);
}

int32_t kv_write_prefix_rows(const kvr_cache *cache, int32_t slot0, int32_t layer0, int32_t n_layers,
                             const void *k_new, const void *v_new, kvr_dtype dtype,
                             int64_t layer_stride_elems, int32_t n_tok, const float *cs_rows,
                             void *stream) {
    if (int32_t e = check_cache(cache)) return e;
    const int32_t D = cache->head_dim;
    if (int32_t e = check_dtype(dtype)) return e;
    if (!cs_rows || !k_new || !v_new) return fail(KVR_EINVAL, "rotary rows or new rows pointer is NULL");
    if (!aligned16(cs_rows) || !aligned16(k_new) || !aligned16(v_new))
        return fail(KVR_EALIGN, "rotary rows or new rows not 16-byte aligned");
    if (n_tok < 1 || slot0 < 0 || (int64_t)slot0 + n_tok > cache->n_prefix)
        return fail(KVR_EINVAL, "prefix slots [%d,%d) not inside [0,%d)", slot0, slot0 + n_tok,
                    cache->n_prefix);
    if (layer0 < 0 || n_layers < 1 || layer0 + n_layers > cache->n_layers)
        return fail(KVR_EINVAL, "layers [%d,%d) outside cache of %d", layer0, layer0 + n_layers,
                    cache->n_layers);
    if (int32_t e = check_write_grid(n_layers, n_tok)) return e;
    const int64_t per_layer = (int64_t)n_tok * cache->n_heads * D;
    if (n_layers > 1 && (layer_stride_elems < per_layer || layer_stride_elems % 8 != 0))
        return fail(KVR_EINVAL, "layer_stride_elems %lld must be >= %lld and a multiple of 8",
                    (long long)layer_stride_elems, (long long)per_layer);
    // the write kernel with a ring of the whole window starting at slot0: the
    // tokens land in slots slot0 .. slot0 + n_tok - 1 without wrapping
    kvr::WriteArgs a{};
    a.k_codes = cache->k_codes;
    a.v_codes = cache->v_codes;
    a.k_scales = cache->k_scales;
    a.v_scales = cache->v_scales;
    a.k_new = k_new;
    a.v_new = v_new;
    a.layer_stride = n_layers > 1 ? layer_stride_elems : 0;
    a.cs = cs_rows;
    a.n_heads = cache->n_heads;
    a.window = cache->window;
    a.prefix = 0;
    a.cap = cache->window;
    a.head = slot0;
    a.n_new = n_tok;
    a.layer0 = layer0;
    a.n_layers = n_layers;
    a.dtype = dtype;
    return launch_status(kvr::launch_write(a, D, static_cast<hipStream_t>(stream)), "prefix write");
}

int32_t kv_delta_rebase_axes(const kvr_cache *cache, const kvr_ring *ring, int32_t layer0,
                             int32_t n_layers, const int64_t *delta, const int32_t *axis_pairs,
                             double rope_base, void *stream) {
    if (int32_t e = check_cache(cache)) return e;
    const int32_t W = ring_cap(cache), D = cache->head_dim;
    if (int32_t e = check_ring(ring, W)) return e;
    if (int32_t e = check_axis_pairs(axis_pairs, D)) return e;
    if (!delta) return fail(KVR_EINVAL, "delta is NULL");
    for (int ax = 0; ax < 3; ++ax)
        if (delta[ax] < -kMaxDelta || delta[ax] > kMaxDelta)
            return fail(KVR_EINVAL, "delta[%d] = %lld outside [-2^53, 2^53]", ax, (long long)delta[ax]);
    if (layer0 < 0 || n_layers < 1 || layer0 + n_layers > cache->n_layers)
        return fail(KVR_EINVAL, "layers [%d,%d) outside cache of %d", layer0, layer0 + n_layers,
                    cache->n_layers);
    if (!(rope_base > 1.0) || !isfinite(rope_base)) return fail(KVR_EINVAL, "rotary base must be > 1");
    if (ring->n_valid == 0) return ok();
    // cos/sin of -delta[axis] * theta per pair: fp64 angle and trig, rounded to fp32
    kvr::CosSinTable rot{};
    const kvr::AxisTheta th = make_axis_theta(axis_pairs, rope_base);
    for (int i = 0; i < D / 2; ++i) {
        const double ang = (double)(-delta[th.axis[i]]) * th.t[i];
        rot.cs[2 * i] = (float)cos(ang);
        rot.cs[2 * i + 1] = (float)sin(ang);
    }
    kvr::RebaseArgs a{};
    a.k_codes = cache->k_codes;
    a.k_scales = cache->k_scales;
    a.n_heads = cache->n_heads;
    a.window = cache->window;
    a.prefix = cache->n_prefix;
    a.cap = W;
    a.start = kvr_ring_logical_start(ring, W);
    a.n_valid = ring->n_valid;
    a.layer0 = layer0;
    a.n_layers = n_layers;
    return launch_status(kvr::launch_rebase(a, rot, D, static_cast<hipStream_t>(stream)), "rebase");
}

int32_t attn_fp8_window_rows(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                             int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                             const float *q_cs_rows, float softmax_scale, uint16_t *out,
                             int32_t n_splits, void *ws, size_t ws_bytes, void *stream) {
    kvr::AttnArgs a;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, n_valid, q, dtype, n_q, 0, softmax_scale,
                               nullptr, out, n_splits, ws, ws_bytes, q_cs_rows))
        return e;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int32_t e = launch_status(kvr::launch_attention_main(a, cache->head_dim, s), "attention"))
        return e;
    return launch_status(kvr::launch_attention_merge(a, cache->head_dim, s), "attention merge");
}

size_t kv_rope_query_lanes_bytes(int32_t n_q, int32_t head_dim) {
    if (n_q < 1 || n_q >= kMaxExtent || (head_dim != 64 && head_dim != 128)) return 0;
    return kvr::query_lanes_bytes(n_q, head_dim);
}

int32_t kv_rope_query_lanes(const float *cs_rows, int32_t n_q, int32_t head_dim, float *lanes, void *stream) {
    if (int32_t e = check_head_dim(head_dim)) return e;
    if (!cs_rows || !lanes) return fail(KVR_EINVAL, "rows or lanes pointer is NULL");
    if (!aligned16(cs_rows) || !aligned16(lanes)) return fail(KVR_EALIGN, "rows or lanes not 16-byte aligned");
    if (n_q < 1 || n_q >= kMaxExtent) return fail(KVR_EINVAL, "n_q %d out of range", n_q);
    return launch_status(kvr::launch_query_lanes(cs_rows, n_q, head_dim, lanes, static_cast<hipStream_t>(stream)),
                         "query lanes");
}

int32_t attn_fp8_window_lanes_partial(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                                      int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                                      const float *q_lanes, float softmax_scale, uint16_t *out,
                                      int32_t n_splits, void *ws, size_t ws_bytes, void *stream) {
    kvr::AttnArgs a;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, n_valid, q, dtype, n_q, 0, softmax_scale,
                               nullptr, out, n_splits, ws, ws_bytes, q_lanes, true))
        return e;
    return launch_status(kvr::launch_attention_main(a, cache->head_dim, static_cast<hipStream_t>(stream)),
                         "attention");
}

int32_t attn_fp8_window_lanes(const kvr_cache *cache, int32_t layer, int32_t slot_start,
                              int32_t n_valid, const void *q, kvr_dtype dtype, int32_t n_q,
                              const float *q_lanes, float softmax_scale, uint16_t *out,
                              int32_t n_splits, void *ws, size_t ws_bytes, void *stream) {
    kvr::AttnArgs a;
    if (int32_t e = attn_setup(a, cache, layer, slot_start, n_valid, q, dtype, n_q, 0, softmax_scale,
                               nullptr, out, n_splits, ws, ws_bytes, q_lanes, true))
        return e;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int32_t e = launch_status(kvr::launch_attention_main(a, cache->head_dim, s), "attention"))
        return e;
    return launch_status(kvr::launch_attention_merge(a, cache->head_dim, s), "attention merge");
}

// ---- (a5) naive per-call upkeep -------------------------------------------
int32_t naive_upkeep(const void *lin_k_src, const void *lin_v_src, const void *k_new,
                     const void *v_new, kvr_dtype dtype, int32_t n_new, int32_t n_valid_before,
                     int64_t pos_next_before, int32_t n_heads, int32_t head_dim, int32_t window,
                     const kvr_rope_table *rope, void *lin_k_dst, void *lin_v_dst,
                     uint8_t *k_codes, uint8_t *v_codes, float *k_scales, float *v_scales,
                     void *stream) {
    if (int32_t e = check_head_dim(head_dim)) return e;
    if (int32_t e = check_dtype(dtype)) return e;
    if (window < 1 || window >= kMaxExtent || n_heads < 1 || n_heads >= kMaxExtent)
        return fail(KVR_EINVAL, "shape out of range (H=%d W=%d)", n_heads, window);
    if (n_new < 1 || n_new > window) return fail(KVR_EINVAL, "n_new %d not in [1,%d]", n_new, window);
    if (n_valid_before < 0 || n_valid_before > window)
        return fail(KVR_EINVAL, "n_valid_before %d not in [0,%d]", n_valid_before, window);
    const void *ptrs[] = {lin_k_src, lin_v_src, k_new, v_new, lin_k_dst, lin_v_dst,
                          k_codes, v_codes, k_scales, v_scales};
    for (const void *p : ptrs) {
        if (!p) return fail(KVR_EINVAL, "naive_upkeep: NULL buffer");
        if (!aligned16(p)) return fail(KVR_EALIGN, "naive_upkeep: buffer not 16-byte aligned");
    }
    // no output may overlap an input or another output (the inputs are only read)
    const size_t esz = dtype == KVR_BF16 ? 2 : 4;
    const size_t win_bytes = (size_t)n_heads * window * head_dim * esz;
    const size_t new_bytes = (size_t)n_new * n_heads * head_dim * esz;
    const size_t code_bytes = (size_t)n_heads * window * head_dim, scale_bytes = (size_t)n_heads * window * 4;
    struct Span {
        const void *p;
        size_t n;
        const char *name;
    };
    const Span ins[] = {{lin_k_src, win_bytes, "lin_k_src"}, {lin_v_src, win_bytes, "lin_v_src"},
                        {k_new, new_bytes, "k_new"}, {v_new, new_bytes, "v_new"}};
    const Span outs[] = {{lin_k_dst, win_bytes, "lin_k_dst"}, {lin_v_dst, win_bytes, "lin_v_dst"},
                         {k_codes, code_bytes, "k_codes"},     {v_codes, code_bytes, "v_codes"},
                         {k_scales, scale_bytes, "k_scales"},  {v_scales, scale_bytes, "v_scales"}};
    auto overlap = [](const Span &a, const Span &b) {
        const char *x = static_cast<const char *>(a.p), *y = static_cast<const char *>(b.p);
        return x < y + b.n && y < x + a.n;
    };
    for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
        for (const Span &in : ins)
            if (overlap(outs[i], in))
                return fail(KVR_EINVAL, "naive_upkeep: %s overlaps the input %s", outs[i].name, in.name);
        for (size_t j = i + 1; j < sizeof outs / sizeof outs[0]; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(KVR_EINVAL, "naive_upkeep: outputs %s and %s overlap", outs[i].name, outs[j].name);
    }
    const int32_t n_after = n_valid_before + n_new < window ? n_valid_before + n_new : window;
    const int32_t drop = n_valid_before + n_new - n_after;
    const float *cs;
    if (int32_t e = table_rows(rope, head_dim, pos_next_before + n_new - n_after, n_after, &cs))
        return e;
    kvr::NaiveArgs a{};
    a.k_src = lin_k_src;
    a.v_src = lin_v_src;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_dst = lin_k_dst;
    a.v_dst = lin_v_dst;
    a.k_codes = k_codes;
    a.v_codes = v_codes;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.cs = cs;
    a.n_heads = n_heads;
    a.window = window;
    a.n_new = n_new;
    a.n_after = n_after;
    a.kept = n_valid_before - drop;
    a.drop = drop;
    a.dtype = dtype;
    return launch_status(kvr::launch_naive(a, head_dim, static_cast<hipStream_t>(stream)), "naive");
}

}  // extern "C"
