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
// owning head_dim/8 contiguous elements; the row arithmetic (rotation of the
// interleaved pairs, row quantisation) is rowquant.h's, shared by the write,
// rebase and naive kernels here and by the write the attention kernel can
// carry, so the ring cache and the naive linear window are bit-identical.
// Decoding a stored row is the exact E4M3 value times the fp32 row scale (one
// fp32 product).  This file is also built with -ffp-contract=off, so no FMA
// merges the roundings of the rebase's dequantisation either.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvr_internal.h"
#include "rowquant.h"

#pragma clang fp contract(off)

namespace kvr {
namespace {

using namespace rowq;

constexpr int kBlock = 256;           // threads per workgroup
constexpr int kRowsPerIter = kBlock / kRowLanes;

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

// The row kernels below take a 2-D grid.  Rebase and naive: blockIdx.y picks
// a (layer, head) or (kv, head) row sequence, blockIdx.x a run of kUnroll * 32
// rows of it, a group's rows 32 apart, and each 8-lane row group issues the
// loads of its kUnroll rows before any arithmetic, so a wave keeps kUnroll
// rows of data in flight (the kernels are bound by HBM bandwidth, which needs
// many bytes in flight per CU).  Write: see below.
constexpr int kUnroll = 4;
constexpr int kRunRows = kUnroll * kRowsPerIter;

// ---------------------------------------------------------------------------
// Write-time RoPE + FP8 [AI-cache].  grid = (ceil(n_new / kWriteTokens),
// n_layers * 2): a workgroup takes kWriteTokens consecutive new tokens of one
// (layer, K/V) and all their heads, so its source rows are one contiguous run
// of the token-major [n_new][n_heads][D] input and consecutive workgroups
// stream the input in order; the tokens' (cos, sin) rows are staged in LDS
// once.  One row per 8-lane group (with 12 heads, 24 of the 32 groups work).
// Two tokens per workgroup measured fastest (75.9-76.2 us for 60 layers at the
// production shape, against 81-82 us for 32 tokens x 4 heads per workgroup:
// the source was then read in 1 KB pieces of 3 KB token rows, three passes
// over each region); the XCD runs below took it to 72.4-74.3 us.
// ---------------------------------------------------------------------------
constexpr int kWriteTokens = 2;
constexpr int kWriteRun = 16;      // token pairs per XCD run (write_kernel's numbering)

template <int D, bool BF16>
__global__ void __launch_bounds__(kBlock) write_kernel(WriteArgs a) {
    constexpr int EPT = D / kRowLanes;
    constexpr int T = kWriteTokens;
    __shared__ float4 cs_lds[T * D / 4];
    const int lane8 = threadIdx.x % kRowLanes, grp = threadIdx.x / kRowLanes;
    // Workgroups are dealt round-robin over the 8 XCDs (linear block b runs
    // on XCD b % 8).  Renumber them so that each XCD takes runs of
    // kWriteRun consecutive blocks of the (layer, K/V, token pair) order --
    // 32 tokens, as many slots as share a 128-byte line of row scales -- the
    // runs of the 8 XCDs interleaved: a line of scales then leaves the L2s in
    // at most two parts rather than in pieces from every XCD.  The last
    // G mod (8 kWriteRun) blocks keep their own numbers.
    const int GX = gridDim.x, G = GX * gridDim.y;
    const int b = blockIdx.y * GX + blockIdx.x;
    int u = b;
    if (b < G / (8 * kWriteRun) * (8 * kWriteRun)) {
        const int xcd = b % 8, k = b / 8;
        u = ((k / kWriteRun) * 8 + xcd) * kWriteRun + k % kWriteRun;
    }
    const int j0 = (u % GX) * T;
    const int nt = min(T, a.n_new - j0);
    const int kv = (u / GX) % 2;
    const int lrel = (u / GX) / 2;
    if (kv == 0) {
        // the run's (cos, sin) rows (pair-major, D floats per token)
        for (int i = threadIdx.x; i < T * D / 4; i += kBlock) {
            const int jj = min(i / (D / 4), nt - 1);
            cs_lds[i] = reinterpret_cast<const float4 *>(a.cs + (int64_t)(j0 + jj) * D)[i % (D / 4)];
        }
        __syncthreads();
    }
    const void *src = kv ? a.v_new : a.k_new;
    const int64_t lay_in = (int64_t)lrel * a.layer_stride;
    const int64_t lay_cache = (int64_t)(a.layer0 + lrel) * a.n_heads * a.window;
    uint8_t *codes = kv ? a.v_codes : a.k_codes;
    float *scales = kv ? a.v_scales : a.k_scales;
    const int rows = nt * a.n_heads;                    // token-major: row = token * n_heads + head
    for (int r = grp; r < rows; r += kRowsPerIter) {
        RawChunk<EPT, BF16> raw;
        raw.load(src, lay_in + ((int64_t)j0 * a.n_heads + r) * D + lane8 * EPT);
        const int jj = r / a.n_heads, h = r - jj * a.n_heads;
        float x[EPT];
        raw.to_f32(x);
        if (kv == 0) {
            float4 csv[EPT / 4];
#pragma unroll
            for (int v = 0; v < EPT / 4; ++v) csv[v] = cs_lds[jj * (D / 4) + lane8 * (EPT / 4) + v];
            rotate_pairs<EPT>(x, reinterpret_cast<const float *>(csv));
        }
        int slot = a.head + j0 + jj;
        if (slot >= a.cap) slot -= a.cap;
        slot += a.prefix;
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
    dim3 grid((a.n_new + kWriteTokens - 1) / kWriteTokens, a.n_layers * 2);
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
