// upkeep.hip -- memory-bound cache upkeep kernels for gfx950 (CDNA4):
//   rotary (cos, sin) table, write-time RoPE + FP8 of a new chunk, the delta
//   rebase of the stored K window, and the naive per-call window rebuild.
//
// Page references (cited by title and section):
//   [AI-cache] ai.info, "Characters funziona in tempo reale su quattro H100,
//              afferma Runway", section "La gestione della cache spostata al
//              momento della scrittura".
//   [WC]       wechild.cn news item 1943 (original per-call upkeep).
//
// Every row of head_dim elements is handled by 8 consecutive lanes, each lane
// owning head_dim/8 contiguous elements (16-byte loads and stores); the row
// absmax is a 3-step butterfly across those 8 lanes.  Decoding a stored row
// is the exact E4M3 value times the fp32 row scale (one fp32 product).  The arithmetic order
// of one element is fixed (rotation: x0*c - x1*s, x0*s + x1*c, each product
// and sum rounded to fp32; quantisation: y * (448 / absmax) rounded to fp32,
// then E4M3 round-to-nearest-even via v_cvt_pk_fp8_f32), and this file is
// built with -ffp-contract=off so no FMA merges those roundings.  The write,
// rebase and naive kernels share these device helpers, so the ring cache and
// the naive linear window are bit-identical.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvr_internal.h"

#pragma clang fp contract(off)

namespace kvr {
namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

constexpr int kRowLanes = 8;          // lanes per row
constexpr int kBlock = 256;           // threads per workgroup
constexpr int kRowsPerIter = kBlock / kRowLanes;

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

// Row quantisation: absmax over the 8 lanes of the row, scale = a / 448,
// codes = E4M3_RNE(y * (448 / a)).  Writes EPT codes and (lane 0) the scale;
// y is lifted in place for tiny rows.
template <int EPT>
__device__ __forceinline__ void quantize_store(float (&y)[EPT], uint8_t *codes_dst,
                                               float *scale_dst, bool lane0) {
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
    if constexpr (EPT == 16) {
        __builtin_nontemporal_store(u32x4v{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4v *>(codes_dst));
    } else {
        __builtin_nontemporal_store(u32x2v{w[0], w[1]}, reinterpret_cast<u32x2v *>(codes_dst));
    }
    if (lane0) *scale_dst = scale;
}

// ---------------------------------------------------------------------------
// Rotary table: cs[p][i] = (cos, sin)(p * theta_i), fp64 angle and trig.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) rope_table_kernel(float2 *cs, int64_t pos0,
                                                            int32_t n_pos, int32_t half,
                                                            ThetaTable th) {
    const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (idx >= (int64_t)n_pos * half) return;
    const int64_t p = idx / half;
    const int i = (int)(idx - p * half);
    const double ang = (double)(pos0 + p) * th.t[i];
    double s, c;
    sincos(ang, &s, &c);
    cs[idx] = make_float2((float)c, (float)s);
}

// ---------------------------------------------------------------------------
// 3-D rotary rows: cs[tok][i] = (cos, sin)(coords[tok][axis_i] * theta_i), the
// pair's own axis coordinate (frame, row, column) times its frequency; fp64
// angle and trig, rounded to fp32.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) rope3d_table_kernel(float2 *cs, const int32_t *coords,
                                                              int32_t n_tok, int32_t half,
                                                              AxisTheta th) {
    const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (idx >= (int64_t)n_tok * half) return;
    const int64_t tok = idx / half;
    const int i = (int)(idx - tok * half);
    const double ang = (double)coords[3 * tok + th.axis[i]] * th.t[i];
    double s, c;
    sincos(ang, &s, &c);
    cs[idx] = make_float2((float)c, (float)s);
}

// The three row kernels below take a 2-D grid, and each 8-lane row group
// handles kUnroll rows, issuing all of their loads before any arithmetic, so a
// wave keeps kUnroll rows of data in flight (the kernels are bound by HBM
// bandwidth, which needs many bytes in flight per CU).  Rebase and naive:
// blockIdx.y picks a (layer, head) or (kv, head) row sequence, blockIdx.x a run
// of kUnroll * 32 rows of it, a group's rows 32 apart.  Write: see below.
constexpr int kUnroll = 4;
constexpr int kRunRows = kUnroll * kRowsPerIter;

// ---------------------------------------------------------------------------
// Write-time RoPE + FP8 [AI-cache].  grid = (ceil(n_new / 32),
// n_layers * 2 * ceil(n_heads / kUnroll)); y = (layer, kv, group of kUnroll
// consecutive heads), x = a run of 32 new tokens.  A row group takes one token
// and the kUnroll heads of its group: its source rows are contiguous in the
// [n_new][n_heads][D] input and its slice of the (cos, sin) row of that
// position is loaded once for all of them.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ void __launch_bounds__(kBlock) write_kernel(WriteArgs a) {
    constexpr int EPT = D / kRowLanes;
    const int lane8 = threadIdx.x % kRowLanes;
    const int n_hg = (a.n_heads + kUnroll - 1) / kUnroll;      // head groups
    const int hg = blockIdx.y % n_hg;
    const int kv = (blockIdx.y / n_hg) % 2;
    const int lrel = blockIdx.y / (2 * n_hg);
    const int jr = blockIdx.x * kRowsPerIter + threadIdx.x / kRowLanes;
    const int j = min(jr, a.n_new - 1);                         // position of the group's rows
    const void *src = kv ? a.v_new : a.k_new;
    const int64_t lay_in = (int64_t)lrel * a.layer_stride;
    RawChunk<EPT, BF16> raw[kUnroll];
    float4 csv[EPT / 4];
    if (kv == 0) {
        const float4 *t = reinterpret_cast<const float4 *>(a.cs + (int64_t)j * D + lane8 * EPT);
#pragma unroll
        for (int v = 0; v < EPT / 4; ++v) csv[v] = t[v];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int h = min(kUnroll * hg + u, a.n_heads - 1);
        raw[u].load(src, lay_in + ((int64_t)j * a.n_heads + h) * D + lane8 * EPT);
    }
    if (jr >= a.n_new) return;
    const int64_t lay_cache = (int64_t)(a.layer0 + lrel) * a.n_heads * a.window;
    uint8_t *codes = kv ? a.v_codes : a.k_codes;
    float *scales = kv ? a.v_scales : a.k_scales;
    int slot = a.head + j;
    if (slot >= a.cap) slot -= a.cap;
    slot += a.prefix;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int h = kUnroll * hg + u;
        if (h >= a.n_heads) break;
        float x[EPT];
        raw[u].to_f32(x);
        if (kv == 0) rotate_pairs<EPT>(x, reinterpret_cast<const float *>(csv));
        const int64_t row = lay_cache + (int64_t)h * a.window + slot;
        quantize_store<EPT>(x, codes + row * D + lane8 * EPT, scales + row, lane8 == 0);
    }
}

// ---------------------------------------------------------------------------
// Delta rebase [AI-cache]: every valid K row dequantised, rotated by -delta,
// re-quantised.  grid = (ceil(n_valid / kRunRows), n_layers * n_heads).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kBlock) rebase_kernel(RebaseArgs a, CosSinTable rot) {
    constexpr int EPT = D / kRowLanes;
    const int lane8 = threadIdx.x % kRowLanes;
    float cs[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) cs[e] = rot.cs[lane8 * EPT + e];
    const int64_t lh = (int64_t)a.layer0 * a.n_heads + blockIdx.y;
    const int i0 = blockIdx.x * kRunRows + threadIdx.x / kRowLanes;
    int64_t rows[kUnroll];
    uint32_t w[kUnroll][EPT / 4];
    float sc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int i = min(i0 + u * kRowsPerIter, a.n_valid - 1);
        int slot = a.start + i;
        if (slot >= a.cap) slot -= a.cap;
        rows[u] = lh * a.window + a.prefix + slot;
        const uint8_t *src = a.k_codes + rows[u] * D + lane8 * EPT;
        if constexpr (EPT == 16) {
            const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(src));
            w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
        } else {
            const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v *>(src));
            w[u][0] = v[0]; w[u][1] = v[1];
        }
        sc[u] = a.k_scales[rows[u]];          // 4 bytes of a line shared by 32 rows: ordinary load
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (i0 + u * kRowsPerIter >= a.n_valid) break;
        float x[EPT];
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[u][k], false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[u][k], true);
            x[4 * k] = lo[0] * sc[u];
            x[4 * k + 1] = lo[1] * sc[u];
            x[4 * k + 2] = hi[0] * sc[u];
            x[4 * k + 3] = hi[1] * sc[u];
        }
        rotate_pairs<EPT>(x, cs);
        quantize_store<EPT>(x, a.k_codes + rows[u] * D + lane8 * EPT, a.k_scales + rows[u], lane8 == 0);
    }
}

// ---------------------------------------------------------------------------
// Naive per-call upkeep [WC]: rebuild the shifted linear window and
// re-rotate / re-quantise all of it.  grid = (ceil(n_after / kRunRows),
// 2 * n_heads); y = (kv, head), rows = window positions.
// ---------------------------------------------------------------------------
// Two rows per lane group here (the write and rebase use kUnroll = 4): this
// kernel has only 2 x n_heads row sequences, and the extra workgroups measured
// faster (23.3 -> 22.9 us per call at the production shape).
constexpr int kNaiveUnroll = 2;

template <int D, bool BF16>
__global__ void __launch_bounds__(kBlock) naive_kernel(NaiveArgs a) {
    constexpr int kUnroll = kNaiveUnroll;
    constexpr int kRunRows = kUnroll * kRowsPerIter;
    constexpr int EPT = D / kRowLanes;
    const int lane8 = threadIdx.x % kRowLanes;
    const int h = blockIdx.y % a.n_heads;
    const int kv = blockIdx.y / a.n_heads;
    const int i0 = blockIdx.x * kRunRows + threadIdx.x / kRowLanes;
    RawChunk<EPT, BF16> raw[kUnroll];
    float4 csv[kUnroll][EPT / 4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int i = min(i0 + u * kRowsPerIter, a.n_after - 1);
        if (i < a.kept)
            raw[u].load(kv ? a.v_src : a.k_src, ((int64_t)h * a.window + i + a.drop) * D + lane8 * EPT);
        else
            raw[u].load(kv ? a.v_new : a.k_new, ((int64_t)(i - a.kept) * a.n_heads + h) * D + lane8 * EPT);
        if (kv == 0) {
            const float4 *t = reinterpret_cast<const float4 *>(a.cs + (int64_t)i * D + lane8 * EPT);
#pragma unroll
            for (int v = 0; v < EPT / 4; ++v) csv[u][v] = t[v];
        }
    }
    uint8_t *codes = kv ? a.v_codes : a.k_codes;
    float *scales = kv ? a.v_scales : a.k_scales;
    void *dst = kv ? a.v_dst : a.k_dst;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int i = i0 + u * kRowsPerIter;
        if (i >= a.n_after) break;
        const int64_t row = (int64_t)h * a.window + i;
        raw[u].store(dst, row * D + lane8 * EPT);
        float x[EPT];
        raw[u].to_f32(x);
        if (kv == 0) rotate_pairs<EPT>(x, reinterpret_cast<const float *>(csv[u]));
        quantize_store<EPT>(x, codes + row * D + lane8 * EPT, scales + row, lane8 == 0);
    }
}

}  // namespace

hipError_t launch_rope_table(float *cs, int64_t pos0, int32_t n_pos, int32_t head_dim,
                             const ThetaTable &theta, hipStream_t s) {
    const int half = head_dim / 2;
    const int64_t n = (int64_t)n_pos * half;
    const int grid = (int)((n + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(kBlock), 0, s,
                       reinterpret_cast<float2 *>(cs), pos0, n_pos, half, theta);
    return hipGetLastError();
}

hipError_t launch_rope3d_table(float *cs, const int32_t *coords, int32_t n_tok, int32_t head_dim,
                               const AxisTheta &theta, hipStream_t s) {
    const int half = head_dim / 2;
    const int64_t n = (int64_t)n_tok * half;
    const int grid = (int)((n + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(rope3d_table_kernel, dim3(grid), dim3(kBlock), 0, s,
                       reinterpret_cast<float2 *>(cs), coords, n_tok, half, theta);
    return hipGetLastError();
}

hipError_t launch_write(const WriteArgs &a, int head_dim, hipStream_t s) {
    dim3 grid((a.n_new + kRowsPerIter - 1) / kRowsPerIter,
              a.n_layers * 2 * ((a.n_heads + kUnroll - 1) / kUnroll));
    const bool bf = a.dtype == KVR_BF16;
    if (head_dim == 128 && bf)
        hipLaunchKernelGGL((write_kernel<128, true>), grid, dim3(kBlock), 0, s, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL((write_kernel<128, false>), grid, dim3(kBlock), 0, s, a);
    else if (bf)
        hipLaunchKernelGGL((write_kernel<64, true>), grid, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL((write_kernel<64, false>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_rebase(const RebaseArgs &a, const CosSinTable &rot, int head_dim,
                         hipStream_t s) {
    dim3 grid((a.n_valid + kRunRows - 1) / kRunRows, a.n_layers * a.n_heads);
    if (head_dim == 128)
        hipLaunchKernelGGL(rebase_kernel<128>, grid, dim3(kBlock), 0, s, a, rot);
    else
        hipLaunchKernelGGL(rebase_kernel<64>, grid, dim3(kBlock), 0, s, a, rot);
    return hipGetLastError();
}

hipError_t launch_naive(const NaiveArgs &a, int head_dim, hipStream_t s) {
    constexpr int kNaiveRun = kNaiveUnroll * kRowsPerIter;
    dim3 grid((a.n_after + kNaiveRun - 1) / kNaiveRun, 2 * a.n_heads);
    const bool bf = a.dtype == KVR_BF16;
    if (head_dim == 128 && bf)
        hipLaunchKernelGGL((naive_kernel<128, true>), grid, dim3(kBlock), 0, s, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL((naive_kernel<128, false>), grid, dim3(kBlock), 0, s, a);
    else if (bf)
        hipLaunchKernelGGL((naive_kernel<64, true>), grid, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL((naive_kernel<64, false>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvr
