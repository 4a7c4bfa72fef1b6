// kvr_internal.h -- launch helpers shared by the host entry points and the
// HIP kernels of libkvring.  Not part of the public ABI (include/kvring.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvring.h"

namespace kvr {

constexpr int kMaxHalfDim = 64;      // head_dim <= 128

struct ThetaTable {                  // theta_i = base^(-2i/D), fp64, formed on the host
    double t[kMaxHalfDim];
};

struct CosSinTable {                 // (cos, sin) pairs of one rotation, fp32
    float cs[2 * kMaxHalfDim];
};

struct AxisTheta {                   // 3-D form: theta and coordinate axis (0 t, 1 y, 2 x) per pair
    double t[kMaxHalfDim];
    int32_t axis[kMaxHalfDim];
};

// ---- upkeep.hip ----------------------------------------------------------
hipError_t launch_rope_table(float *cs, int64_t pos0, int32_t n_pos, int32_t head_dim,
                             const ThetaTable &theta, hipStream_t s);
hipError_t launch_rope3d_table(float *cs, const int32_t *coords, int32_t n_tok, int32_t head_dim,
                               const AxisTheta &theta, hipStream_t s);

struct WriteArgs {
    uint8_t *k_codes, *v_codes;
    float *k_scales, *v_scales;
    const void *k_new, *v_new;
    int64_t layer_stride;            // elements between consecutive layers of k_new/v_new
    const float *cs;                 // rotary table row of position pos_next (pair-major)
    int32_t n_heads, window, head, n_new, layer0, n_layers;
    int32_t prefix, cap;             // ring slot s is cache slot prefix + s, s < cap
    int32_t dtype;
};
hipError_t launch_write(const WriteArgs &a, int head_dim, hipStream_t s);

struct RebaseArgs {
    uint8_t *k_codes;
    float *k_scales;
    int32_t n_heads, window, start, n_valid, layer0, n_layers;
    int32_t prefix, cap;             // ring slot s is cache slot prefix + s, s < cap
};
hipError_t launch_rebase(const RebaseArgs &a, const CosSinTable &rot, int head_dim, hipStream_t s);

struct NaiveArgs {
    const void *k_src, *v_src, *k_new, *v_new;
    void *k_dst, *v_dst;
    uint8_t *k_codes, *v_codes;
    float *k_scales, *v_scales;
    const float *cs;                 // rotary table row of the window's first position
    int32_t n_heads, window, n_new, n_after, kept, drop;
    int32_t dtype;
};
hipError_t launch_naive(const NaiveArgs &a, int head_dim, hipStream_t s);

// ---- attention.hip -------------------------------------------------------
struct AttnArgs {
    const uint8_t *k_codes, *v_codes; // this layer: [H][W][D]
    const float *k_scales, *v_scales; // this layer: [H][W]
    const void *q;                    // [n_q][H][D]
    ThetaTable rev;                   // theta_i / (2 pi): rotary frequencies in revolutions (fp64)
    double rev_step;                  // base^(-32/D) = theta_{i+16} / theta_i
    int64_t q_pos0;                   // rotary position of query 0
    const float *q_cs;                // or (cos, sin) rows of the queries [n_q][D/2][2] (then q_pos0 unused)
    int32_t q_cs_lanes;               // 1: q_cs is in the lane layout of launch_query_lanes
    uint16_t *out;                    // [n_q][H][D] bf16
    uint16_t *part_o;                 // [splits][n_q][H][D] fp16, normalised rows
    float *part_ml;                   // [splits][n_q][H][4]: running max, sum, row exponent, 0
    int32_t n_heads, window, slot_start, n_valid, n_q, dtype;   // n_valid: prefix + ring keys
    int32_t prefix, cap;              // key i < prefix: slot i; else prefix + (slot_start + i - prefix) mod cap
    int32_t n_splits;                 // key tiles dealt to the splits in turn
    float softmax_scale;
    // The chunk's write carried by the attention launch (fused form only):
    // every workgroup stores its share of the n_new new rows of this layer,
    // then counts itself done in sync[0]; a workgroup whose key range holds
    // new keys waits for n_writers before streaming its first such tile.
    const void *w_k, *w_v;            // [n_new][H][D] of `dtype`
    const float *w_cs;                // rotary table row of the chunk's first position (pair-major)
    uint8_t *w_k_codes, *w_v_codes;   // this layer's codes and scales (written)
    float *w_k_scales, *w_v_scales;
    int32_t w_head, w_n_new;          // ring slot of new token 0, tokens in the chunk
    int32_t n_writers, n_waiters;     // workgroups that write (the grid); that wait
    int32_t first_new;                // logical index of the chunk's first key (n_valid - n_new)
    uint32_t *sync;                   // control block: writers done, waiters through, timeouts, spin limit
};
int attn_default_splits(int n_heads, int n_q, int n_valid);
int attn_query_blocks(int n_q);      // query blocks (workgroups per head and split)
// (cos, sin) rows [n_q][D/2][2] rearranged so that the attention kernel's load
// c of lane l of wave w of query block b reads 16 bytes at
// ((b * 8 + w) * (D / 8) + c) * 64 + l (units of 16 bytes)
size_t query_lanes_bytes(int n_q, int head_dim);
hipError_t launch_query_lanes(const float *cs_rows, int n_q, int head_dim, float *lanes, hipStream_t s);
size_t attn_workspace_bytes(int n_heads, int head_dim, int n_q, int n_splits);
// the attention kernel (output rows when n_splits == 1, split partials else)
hipError_t launch_attention_main(const AttnArgs &a, int head_dim, hipStream_t s);
// the same kernel carrying the chunk's write (a.n_writers > 0, position form)
hipError_t launch_attention_fused(const AttnArgs &a, int head_dim, hipStream_t s);
// how many workgroups of that kernel can be resident on `device` at once
hipError_t attention_fused_resident(int head_dim, int dtype, bool prefix, int device, int *max_blocks);
constexpr uint32_t kFusedSpinLimit = 1u << 18;   // polls (each ~1 us: an atomic round trip and a short sleep) before a wait gives up
// the merge of the split partials into the output rows (nothing for one split)
hipError_t launch_attention_merge(const AttnArgs &a, int head_dim, hipStream_t s);

}  // namespace kvr
