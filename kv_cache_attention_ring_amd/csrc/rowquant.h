// rowquant.h -- the row arithmetic of every cache write: a lane's slice of a
// source row, the rotation of its interleaved pairs and the row quantisation
// to OCP E4M3 with an fp32 row scale.  Shared by the upkeep kernels
// (upkeep.hip) and the write the attention kernel can carry (attention.hip),
// so every path stores the same bits for the same row.
//
// Page reference: ai.info, "Characters funziona in tempo reale su quattro
// H100, afferma Runway", section "La gestione della cache spostata al momento
// della scrittura" (rotary encoding and FP8 applied once, when a frame enters
// the cache).
//
// Every row of head_dim elements is handled by kRowLanes = 8 consecutive
// lanes, each owning head_dim/8 contiguous elements (16-byte loads and
// stores); the row absmax is a 3-step butterfly across those 8 lanes.  The
// arithmetic order of one element is fixed (rotation: x0*c - x1*s, x0*s +
// x1*c, each product and sum rounded to fp32; quantisation: y * (448 /
// absmax) rounded to fp32, then E4M3 round-to-nearest-even via
// v_cvt_pk_fp8_f32), and the functions below turn floating-point contraction
// off for their own bodies, whatever the including file's setting, so no FMA
// merges those roundings.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvr {
namespace rowq {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

constexpr int kRowLanes = 8;          // lanes per row

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// A lane's chunk of EPT elements in its storage type, as 16-byte vectors.
template <int EPT, bool BF16>
struct RawChunk {
    static constexpr int kVecs = EPT * (BF16 ? 2 : 4) / 16;
    uint4 v[kVecs];

    __device__ __forceinline__ void load(const void *base, int64_t elem_off) {
        const uint4 *p = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const char *>(base) + elem_off * (BF16 ? 2 : 4));
#pragma unroll
        for (int k = 0; k < kVecs; ++k) v[k] = p[k];
    }
    __device__ __forceinline__ void store(void *base, int64_t elem_off) const {
        uint4 *p = reinterpret_cast<uint4 *>(reinterpret_cast<char *>(base) +
                                             elem_off * (BF16 ? 2 : 4));
        // (used by the naive rebuild for the shifted window, which the next
        // call reads from HBM again: nontemporal)
#pragma unroll
        for (int k = 0; k < kVecs; ++k)
            __builtin_nontemporal_store(u32x4v{v[k].x, v[k].y, v[k].z, v[k].w}, reinterpret_cast<u32x4v *>(p + k));
    }
    __device__ __forceinline__ void to_f32(float (&x)[EPT]) const {
#pragma unroll
        for (int k = 0; k < kVecs; ++k) {
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
            if constexpr (BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x[8 * k + 2 * q] = bf16_to_f32(w[q] & 0xFFFFu);
                    x[8 * k + 2 * q + 1] = bf16_to_f32(w[q] >> 16);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) x[4 * k + q] = __uint_as_float(w[q]);
            }
        }
    }
};

// y = R(angle) x on the EPT/2 interleaved pairs; cs holds (cos, sin) per pair.
template <int EPT>
__device__ __forceinline__ void rotate_pairs(float (&x)[EPT], const float *cs) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < EPT / 2; ++i) {
        const float c = cs[2 * i], s = cs[2 * i + 1];
        const float x0 = x[2 * i], x1 = x[2 * i + 1];
        const float a = x0 * c;
        const float b = x1 * s;
        const float e = x0 * s;
        const float f = x1 * c;
        x[2 * i] = a - b;
        x[2 * i + 1] = e + f;
    }
}

// Rows whose absmax lies below 2^-64 are lifted by 2^64 (exact) before the
// inverse is formed: 448 / a itself overflows fp32 once a < 448 / FLT_MAX, and
// y 2^64 * fl(448 / (a 2^64)) is the same real number as y * fl(448 / a)
// wherever that inverse is finite, so no other row changes.
constexpr float kTinyRow = 0x1p-64f;
constexpr float kTinyLift = 0x1p64f;

// Stores that write through to memory (system-coherent: sc0 sc1), for rows
// that workgroups on other XCDs read later in the same launch.  A vector
// store of more than 8 bytes needs one wait state before a VALU instruction
// may overwrite its data registers; the compiler inserts it for its own
// stores but cannot see into an asm statement, so the 16-byte form carries it.
__device__ __forceinline__ void store_wt(void *p, u32x4v v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 0" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_wt(void *p, u32x2v v) {
    asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_wt(void *p, float v) {
    asm volatile("global_store_dword %0, %1, off sc0 sc1" : : "v"(p), "v"(v) : "memory");
}

// Row quantisation: absmax over the 8 lanes of the row, scale = a / 448,
// codes = E4M3_RNE(y * (448 / a)).  Writes EPT codes and (lane 0) the scale;
// y is lifted in place for tiny rows.
template <int EPT, bool WT = false>
__device__ __forceinline__ void quantize_store(float (&y)[EPT], uint8_t *codes_dst,
                                               float *scale_dst, bool lane0) {
#pragma clang fp contract(off)
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) a = fmaxf(a, fabsf(y[e]));
    a = fmaxf(a, __shfl_xor(a, 1, kRowLanes));
    a = fmaxf(a, __shfl_xor(a, 2, kRowLanes));
    a = fmaxf(a, __shfl_xor(a, 4, kRowLanes));
    uint32_t w[EPT / 4];
    float scale;
    if (a == 0.0f) {
        scale = 0.0f;
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) w[k] = 0u;
    } else {
        scale = a / 448.0f;
        float inv;
        if (a < kTinyRow) {                 // rare: the row is lifted first
#pragma unroll
            for (int e = 0; e < EPT; ++e) y[e] = y[e] * kTinyLift;
            inv = 448.0f / (a * kTinyLift);
        } else {
            inv = 448.0f / a;
        }
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            const float t0 = y[4 * k] * inv, t1 = y[4 * k + 1] * inv;
            const float t2 = y[4 * k + 2] * inv, t3 = y[4 * k + 3] * inv;
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, pk, true);
            w[k] = (uint32_t)pk;
        }
    }
    // the codes are written once and not read again by this launch, a whole
    // 128-byte row per 8 lanes: nontemporal stores.  The 4-byte scales of
    // consecutive rows come from different waves: ordinary stores, so they
    // merge into whole lines in L2 before going to HBM (nontemporal scale
    // stores measured ~5% slower for the write and the rebase)
    if constexpr (WT) {
        if constexpr (EPT == 16) store_wt(codes_dst, u32x4v{w[0], w[1], w[2], w[3]});
        else store_wt(codes_dst, u32x2v{w[0], w[1]});
        if (lane0) store_wt(scale_dst, scale);
    } else {
        if constexpr (EPT == 16) {
            __builtin_nontemporal_store(u32x4v{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4v *>(codes_dst));
        } else {
            __builtin_nontemporal_store(u32x2v{w[0], w[1]}, reinterpret_cast<u32x2v *>(codes_dst));
        }
        if (lane0) *scale_dst = scale;
    }
}

}  // namespace rowq
}  // namespace kvr
