// attention.hip -- FP8 window attention over the ring cache for gfx950 (CDNA4).
//
// Page references (cited by title and section):
//   [AI-cache]   ai.info, "Characters funziona in tempo reale su quattro H100,
//                afferma Runway", section "La gestione della cache spostata al
//                momento della scrittura": every attention call reads the whole
//                cached window (5788 slots, 757 of them new) that was rotated and
//                quantised to FP8 when written.
//   [AI-latency] same page, section "Latenza dei turni e altre configurazioni
//                GPU": the FP8 attention kernel has to accept per-head scales.
//
// What one call computes, per head h and query i (the n_q new tokens):
//   O[i] = sum_j softmax_j(scale * q_i . k^_j) v^_j,  j over the n_valid slots
// (q_i rotated at position q_pos0 + i: fp64 angle reduced to revolutions, then
// the hardware sine and cosine; the result goes into E4M3 hi/lo terms, so the
// rotation only needs fp32 accuracy)
// with k^_j = e4m3(code) * sk_j and v^_j = e4m3(code) * sv_j (one fp32 scale per
// cached row).  Keys are visited in logical window order (slot_start + j) mod W.
//
// Work decomposition.  A workgroup owns one head, a block of 256 queries and a
// contiguous range of 64-key tiles (a "split"); each of its 8 waves (two per
// SIMD) owns 32 queries.  Key tiles go global -> LDS with direct loads
// (global_load_lds, 16 bytes a lane, no VGPR staging), triple buffered, one
// barrier per tile.
//   S^T[key][query] = K . Q^T   on v_mfma_f32_32x32x64_f8f6f4: A = FP8 K rows
//                               from LDS, B = Q as two E4M3 terms (hi + lo)
//   O^T[d][query]  += V^T . P^T on v_mfma_f32_32x32x16_bf16: A = V^T in bf16,
//                               B = the softmax weights in bf16
// Each V tile is dequantised once per workgroup (E4M3 code times its row
// scale, rounded to bf16) into a transposed LDS copy while the previous tile
// is consumed; the FP8 rows are read for that with the 8x16-byte LDS
// transpose (ds_read_b64_tr_b8), so a lane gets 8 keys of one d column.
// The K rows feeding A-row i of the first product are permuted,
//   row i = 8q + 4g + r  ->  key 16g + 4q + r  (within each 32-key block),
// so that accumulator register r of lane (query, g) holds key 16g + r: eight
// consecutive registers are then the eight consecutive keys that lane
// supplies to one bf16 MFMA of the second product.  LDS tiles are
// XOR-swizzled in 16-byte chunks so the row gathers, the transpose reads and
// the V^T reads and writes are free of bank conflicts.
//
// Precision: E4M3 has 3 mantissa bits, so Q goes in as two E4M3 terms (hi +
// lo, lo = e4m3(x - hi)), about 8 significant bits and two MFMAs per 64-wide
// slice.  The per-key K scale and the Q block scale fold into one fp32 factor
// per key (a_j).  The weights and V^T are bf16 (8 significant bits), so the
// second product needs no split.  Softmax runs in the log2 domain with a
// lazily updated running max (rescale only when a score passes it by more
// than 16, so weights stay below 2^16 and the fp32 sums cannot overflow).  Splits of one (head, query block) are merged by a second kernel
// in split order, so a call is deterministic and a linear window gives the
// same bits as the ring.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "kvr_internal.h"

namespace kvr {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kKT = 64;           // keys per tile
constexpr int kQW = 32;           // queries per wave
constexpr int kNW = 8;            // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kNW;
constexpr int kQB = kQW * kNW;    // queries per workgroup
constexpr float kTau = 16.0f;     // lazy-rescale threshold (log2 units)
constexpr float kShift = 0.0f;    // weights are 2^(x - m + kShift) <= 2^(kShift + kTau)
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Lds {
    static constexpr int CH = D / 16;            // 16-byte chunks per row
    static constexpr int K_BYTES = kKT * D;
    static constexpr int V_BYTES = kKT * D;
    static constexpr int F_OFF = K_BYTES + V_BYTES;
    static constexpr int BUF = F_OFF + 2 * kKT * 4;
    // dequantised V^T of one tile: [d][64 keys] bf16, 128-byte rows
    static constexpr int VT_BYTES = D * kKT * 2;
    static constexpr int VT_OFF = 3 * BUF;       // FP8 tiles are triple buffered
    // Q operands of one wave: [slice][hi/lo][16-byte part][lane] x 16 bytes
    static constexpr int Q_WAVE = (D / 64) * 2 * 2 * 64 * 16;
    static constexpr int Q_OFF = VT_OFF + 2 * VT_BYTES;   // V^T double buffered
    static constexpr int TOTAL = Q_OFF + kNW * Q_WAVE;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Chunk swizzles: K rows are gathered 8 at a time in the pattern
// {0..3, 16..19} + 4k, V rows are read 8 consecutive rows at a time.
__device__ __forceinline__ int swz_k(int row) { return row + 4 * (row >> 4); }
__device__ __forceinline__ int swz_v(int row) { return row; }
// V^T rows (one per d, 8 chunks of 8 keys): chunk c of row d sits at
// c ^ ((d >> 1) & 7), so 16 consecutive rows hit 16 distinct 16-byte bank
// groups for both the transposing writes and the MFMA operand reads.
__device__ __forceinline__ int vt_pos(int d, int c) { return d * (2 * kKT) + 16 * (c ^ ((d >> 1) & 7)); }

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two floats -> packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf2));
}

__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, pk, true);
    return (uint32_t)pk;
}

// hi = e4m3(x), lo = e4m3(x - hi) for four values.
__device__ __forceinline__ void split4(float a, float b, float c, float d, uint32_t &hi,
                                       uint32_t &lo) {
    hi = pack4_fp8(a, b, c, d);
    auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    lo = pack4_fp8(a - h01[0], b - h01[1], c - h23[0], d - h23[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int slot_of(const AttnArgs &a, int idx) {
    idx = idx < a.n_valid ? idx : a.n_valid - 1;       // keys past the window: any valid row
    const int s = a.slot_start + idx;
    return s >= a.window ? s - a.window : s;
}

// Issue the direct global -> LDS loads of one K and one V tile; the four
// waves 0..3 load it (1 KB blocks, 16 bytes a lane).  LDS chunk position p
// (row p / CH) receives global chunk (p % CH) ^ swizzle(row).
constexpr int kLoadWaves = 4;
template <int D>
__device__ __forceinline__ void issue_tile(const AttnArgs &a, int head, int tile, uint8_t *buf,
                                           int wave) {
    using L = Lds<D>;
    constexpr int CH = L::CH;
    constexpr int BLOCKS = kKT * CH / 64;            // 1 KB blocks per K (or V) tile
    static_assert(BLOCKS % kLoadWaves == 0, "whole blocks per loading wave");
    const int lane = threadIdx.x % 64;
#pragma unroll
    for (int i = 0; i < BLOCKS / kLoadWaves; ++i) {
        const int p0 = 64 * (wave + kLoadWaves * i);  // first position of this block
        const int p = p0 + lane;
        const int row = p / CH, pos = p % CH;
        const int64_t rbase = ((int64_t)head * a.window + slot_of(a, tile * kKT + row)) * D;
        const uint8_t *gk = a.k_codes + rbase + 16 * (pos ^ (swz_k(row) & (CH - 1)));
        const uint8_t *gv = a.v_codes + rbase + 16 * (pos ^ (swz_v(row) & (CH - 1)));
        __builtin_amdgcn_global_load_lds(gk, (LDS_AS void *)(buf + 16 * p0), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(gv, (LDS_AS void *)(buf + L::K_BYTES + 16 * p0), 16, 0, 0);
    }
}

// Per-key scales of a tile: wave 0 loads sk_j, wave 1 sv_j from `scales`
// (chosen once per wave); raw, so the load is not waited for until the
// scale is stored.
__device__ __forceinline__ float load_factor(const AttnArgs &a, const float *scales, int head,
                                             int tile) {
    const int idx = tile * kKT + (int)(threadIdx.x % 64);
    if (idx >= a.n_valid) return 0.0f;
    return scales[(int64_t)head * a.window + slot_of(a, idx)];
}

// Stores the factors of a tile: a_j = sk_j * qfac (threads 0..63), sv_j (64..127).
template <int D>
__device__ __forceinline__ void store_factor(uint8_t *buf, float f, float qfac) {
    if (threadIdx.x < 2 * kKT)
        reinterpret_cast<float *>(buf + Lds<D>::F_OFF)[threadIdx.x] = threadIdx.x < kKT ? f * qfac : f;
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_kernel(AttnArgs a) {
    using L = Lds<D>;
    constexpr int CH = L::CH;
    constexpr int NH = D / 64;          // 64-wide d slices of the QK^T contraction
    constexpr int ND = D / 32;          // 32-row d blocks of O^T
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[kNW];

    // ---- (head, split, query block); a (head, split) key range stays on one
    //      XCD (workgroups are dealt round-robin over the 8 XCDs) --------------
    const int n_qb = (a.n_q + kQB - 1) / kQB;
    const int units = a.n_heads * a.n_splits;
    int unit, qb;
    const int b = blockIdx.x;
    if (units % 8 == 0) {
        const int xcd = b % 8, k = b / 8;
        unit = (k / n_qb) * 8 + xcd;
        qb = k % n_qb;
    } else {
        unit = b / n_qb;
        qb = b % n_qb;
    }
    const int head = unit / a.n_splits;
    const int split = unit % a.n_splits;
    const int n_tiles = (a.n_valid + kKT - 1) / kKT;
    const int t0 = split * a.tiles_per_split;
    const int t1 = min(n_tiles, t0 + a.tiles_per_split);

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int g = lane / 32, col = lane % 32;
    const int qi = qb * kQB + wave * kQW + col;         // this lane's query
    const bool q_ok = qi < a.n_q;

    // start streaming the first two tiles while Q is prepared
    const bool lead = wave < kLoadWaves;
    const float *my_scales = wave == 0 ? a.k_scales : a.v_scales;   // used by waves 0, 1
    if (lead) {
        issue_tile<D>(a, head, t0, smem, wave);
        if (t0 + 1 < t1) issue_tile<D>(a, head, t0 + 1, smem + L::BUF, wave);
    }

    // ---- Q: coalesced load, rotate (fp32), block absmax -----------------------
    // The wave's 32 query rows are read in chunks of 8 elements: lane L takes
    // chunk L % (D/8) of row (64i + L) / (D/8), so every load instruction reads
    // whole rows of Q and of the rotary table.
    constexpr int QCH = D / 8;                            // 8-element chunks per row
    constexpr int QIT = 32 * QCH / 64;                    // chunks per lane
    float qv[QIT][8];
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
        const int r = (i * 64 + lane) / QCH, c = (i * 64 + lane) % QCH;
        const int qr = qb * kQB + wave * kQW + r;
        if (qr < a.n_q) {
            const int64_t off = ((int64_t)qr * a.n_heads + head) * D + 8 * c;
            if (a.dtype == KVR_BF16) {
                const u32x4 u = *reinterpret_cast<const u32x4 *>(
                    reinterpret_cast<const uint16_t *>(a.q) + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qv[i][2 * e] = __uint_as_float(u[e] << 16);
                    qv[i][2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
                }
            } else {
                const f32x4 *p = reinterpret_cast<const f32x4 *>(
                    reinterpret_cast<const float *>(a.q) + off);
                const f32x4 f0 = p[0], f1 = p[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qv[i][e] = f0[e];
                    qv[i][4 + e] = f1[e];
                }
            }
            // rotation angle p * theta_i in fp64, reduced to [-1/2, 1/2]
            // revolutions, then the hardware sin/cos (revolution input)
            const double pos = (double)(a.q_pos0 + qr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double rev = pos * a.theta.t[4 * c + e] * 0.15915494309189535;
                const float fr = (float)(rev - __builtin_rint(rev));
                const float cc = __builtin_amdgcn_cosf(fr), ss = __builtin_amdgcn_sinf(fr);
                const float x0 = qv[i][2 * e], x1 = qv[i][2 * e + 1];
                qv[i][2 * e] = x0 * cc - x1 * ss;
                qv[i][2 * e + 1] = x0 * ss + x1 * cc;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[i][e] = 0.0f;
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < QIT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(qv[i][e]));
    am = wave_max(am);

    if (lane == 0) red[wave] = am;
    __syncthreads();
    float qmax = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) qmax = fmaxf(qmax, red[w]);
    const float qscale = qmax > 0.0f ? 448.0f / qmax : 1.0f;
    const float qfac = (qmax > 0.0f ? qmax / 448.0f : 1.0f) * a.softmax_scale * kLog2e;

    // ---- Q -> hi/lo E4M3 B operands, kept in this wave's LDS area ------------
    // Layout [slice h][hi/lo][16-byte part][lane' = 32g + row] x 16 bytes: lane'
    // of the MFMA B operand holds d in [64h + 32g, +32) of query row (lane' % 32).
    uint8_t *qbase = smem + L::Q_OFF + wave * L::Q_WAVE;
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
        const int r = (i * 64 + lane) / QCH, c = (i * 64 + lane) % QCH;
        const int h = c / 8, gg = (c / 4) % 2, part = (c / 2) % 2;
        uint32_t hi0, lo0, hi1, lo1;
        split4(qv[i][0] * qscale, qv[i][1] * qscale, qv[i][2] * qscale, qv[i][3] * qscale, hi0, lo0);
        split4(qv[i][4] * qscale, qv[i][5] * qscale, qv[i][6] * qscale, qv[i][7] * qscale, hi1, lo1);
        const int pos = (32 * gg + r) * 16 + 8 * (c % 2);
        *reinterpret_cast<v2i *>(qbase + (4 * h + part) * 1024 + pos) = v2i{(int)hi0, (int)hi1};
        *reinterpret_cast<v2i *>(qbase + (4 * h + 2 + part) * 1024 + pos) = v2i{(int)lo0, (int)lo1};
    }

    // Lane-constant LDS offsets.  K A-operand: A-row i (= col) of block kb is
    // key 32kb + kk with kk = 16((i>>2)&1) + 4(i>>3) + (i&3); this lane reads
    // the d chunks 4h + 2g and 4h + 2g + 1 (h = 64-wide slice).
    const int kk = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    int koff[2][NH][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + kk;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                koff[kb][h][e] = row * D + 16 * ((4 * h + 2 * g + e) ^ (swz_k(row) & (CH - 1)));
    }
    // V dequantisation: 8-key x 16-column blocks of the FP8 V tile, read with
    // the 8x16-byte transpose.  16-lane group G of wave w takes blocks
    // 4w + G (+ 32); lane j points at row 8kg + j/2, byte 8(j%2) of d chunk dc
    // and receives keys 8kg .. 8kg+7 of column d = 16dc + j.
    constexpr int NBLK = (kKT / 8) * CH;
    constexpr int NCV = (NBLK + 4 * kNW - 1) / (4 * kNW);
    const int G = lane / 16, j = lane % 16;
    int cv_src[NCV], cv_dst[NCV], cv_kg[NCV];
#pragma unroll
    for (int i = 0; i < NCV; ++i) {
        const int blk = 4 * wave + G + 4 * kNW * i;
        const int kg = blk % 8, dc = blk / 8;
        const int row = 8 * kg + j / 2;
        cv_src[i] = L::K_BYTES + row * D + 16 * (dc ^ (swz_v(row) & (CH - 1))) + 8 * (j % 2);
        cv_dst[i] = vt_pos(16 * dc + j, kg);
        cv_kg[i] = kg;
    }
    static_assert(NBLK % (4 * kNW) == 0, "whole dequantisation rounds");
    auto convert_v = [&](const uint8_t *buf, uint8_t *vt) {
        const float *fv = reinterpret_cast<const float *>(buf + L::F_OFF) + kKT;
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const v2i u = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i *)(buf + cv_src[i]));
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(fv + 8 * cv_kg[i]);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(fv + 8 * cv_kg[i] + 4);
            const auto x0 = __builtin_amdgcn_cvt_pk_f32_fp8(u[0], false);
            const auto x1 = __builtin_amdgcn_cvt_pk_f32_fp8(u[0], true);
            const auto x2 = __builtin_amdgcn_cvt_pk_f32_fp8(u[1], false);
            const auto x3 = __builtin_amdgcn_cvt_pk_f32_fp8(u[1], true);
            const u32x4 w = {pack_bf16(x0[0] * s0[0], x0[1] * s0[1]), pack_bf16(x1[0] * s0[2], x1[1] * s0[3]),
                             pack_bf16(x2[0] * s1[0], x2[1] * s1[1]), pack_bf16(x3[0] * s1[2], x3[1] * s1[3])};
            *reinterpret_cast<u32x4 *>(vt + cv_dst[i]) = w;
        }
    };
    uint8_t *vt_base = smem + L::VT_OFF;

    // ---- main loop: two wave groups in ping-pong --------------------------------
    // Per tile t a wave runs two half-steps:
    //   V(t): scores, running max, weights p = 2^x and their sum -> bf16 B operands
    //   M(t): O^T += V^T(t) . P^T(t); S^T(t+1) = K(t+1) . Q^T; dequantise V(t+1)
    // in the order M(t0-1) V(t0) M(t0) V(t0+1) ... M(t1-1), where M(t0-1) only
    // holds the tile-t0 parts.  The group of waves 0..3 runs one half-step
    // ahead of waves 4..7, and half-steps are separated by workgroup barriers,
    // so at any time the two waves sharing a SIMD are in different half-steps:
    // one keeps the matrix core busy while the other uses the VALU.
    // Buffers: FP8 tile t+2 is loaded in the odd interval 2(t-t0)+1 and is
    // waited for at the end of the next one; FP8 tiles are triple buffered
    // (the lead group reads a tile's K and V in M(t-1), the trailing group
    // reads its K factors in V(t), two intervals later); V^T is double
    // buffered (written in M(t-1), read in M(t)).
    v16f o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = v16f{};
    float lsum = 0.0f;      // this lane's share of the softmax denominator
    float cofs = 0.0f;      // kShift - running max (log2 units)
    v16f s[2];              // S^T of the tile of the next V half-step
    v8bf pb[2][2];          // P of the tile of the next M half-step

    auto half_v = [&](int t) {
        const int r0 = t - t0;
        const float *fa = reinterpret_cast<const float *>(smem + (r0 % 3) * L::BUF + L::F_OFF);
        // scores (log2 units, shifted by cofs); register r of block kb is key
        // 32kb + 16g + r of the tile
        float mx = -INFINITY;
        const int lim = a.n_valid - t * kKT;              // valid keys of this tile
        auto scores = [&](bool masked) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 f = *reinterpret_cast<const f32x4 *>(fa + 32 * kb + 16 * g + 4 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = s[kb][4 * q + r] * f[r] + cofs;
                        if (masked) v = (32 * kb + 16 * g + 4 * q + r < lim) ? v : -INFINITY;
                        s[kb][4 * q + r] = v;
                        mx = fmaxf(mx, v);
                    }
                }
        };
        if (lim >= kKT) scores(false);
        else scores(true);
        {
            // max with the other half of the wave (lanes l and l ^ 32 hold the
            // same query): swap the halves across two copies
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const bool first = t == t0;
        const bool over = mx > kShift + kTau;
        if (__any(first || over)) {
            float shift = 0.0f;                  // new cofs = cofs - shift
            if (first) {
                shift = mx - kShift;
            } else if (over) {
                shift = mx - kShift;
                const float alpha = __builtin_amdgcn_exp2f(-shift);
                lsum *= alpha;
#pragma unroll
                for (int d = 0; d < ND; ++d) o[d] *= alpha;
            }
            cofs -= shift;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] -= shift;
        }
        // weights p = 2^x, rounded to bf16; the sum is taken of the rounded
        // values (dot with (1, 1)), i.e. of exactly what the MFMA multiplies
        const bf2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w[e] = pack_bf16(__builtin_amdgcn_exp2f(s[kb][8 * ks + 2 * e]),
                                     __builtin_amdgcn_exp2f(s[kb][8 * ks + 2 * e + 1]));
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, (uint32_t)w[e]), one2,
                                                           lsum, false);
                }
                // keep the weights computed in this half-step (not sunk
                // into the matrix half-step that consumes them)
                asm volatile("" : "+v"(w));
                pb[kb][ks] = __builtin_bit_cast(v8bf, w);
            }
    };

    // Q operands of QK^T stay in VGPRs for the whole loop: lane (query, g)
    // holds d in [64h + 32g, +32) of its query, hi and lo terms.
    v8i qop[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
            const u32x4 u0 = *reinterpret_cast<const u32x4 *>(qbase + ((4 * h + 2 * hl) * 64 + lane) * 16);
            const u32x4 u1 = *reinterpret_cast<const u32x4 *>(qbase + ((4 * h + 2 * hl + 1) * 64 + lane) * 16);
            qop[h][hl] = v8i{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                             (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
        }

    // M half-step.  PV and PREP select the parts (both in the steady state).
    // Operands are read one MFMA group ahead: the PV products go in four
    // groups (kb, ks) of ND MFMAs, then QK^T of tile t+1 in NH groups of four.
    auto half_m = [&](int t, auto PV, auto PREP_) {
        const bool PREP_on = decltype(PREP_)::value && t + 1 < t1;
        using PREP = decltype(PREP_);
        const int r0 = t - t0;
        const uint8_t *vt = vt_base + (r0 % 2) * L::VT_BYTES;
        const uint8_t *buf1 = smem + ((r0 + 1) % 3) * L::BUF;
        auto read_v = [&](int grp, u32x4 (&va)[ND]) {
            const int kb = grp / 2, ks = grp % 2;
#pragma unroll
            for (int d = 0; d < ND; ++d)
                va[d] = *reinterpret_cast<const u32x4 *>(vt + vt_pos(32 * d + col, 4 * kb + 2 * g + ks));
        };
        // K operands of slice h (both 32-key blocks)
        auto read_k = [&](int h, v8i (&ka)[2]) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 u0 = *reinterpret_cast<const u32x4 *>(buf1 + koff[kb][h][0]);
                const u32x4 u1 = *reinterpret_cast<const u32x4 *>(buf1 + koff[kb][h][1]);
                ka[kb] = v8i{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                             (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
            }
        };
        if constexpr (decltype(PV)::value) {
            // O^T += V^T . P^T; A-operand lane (d, g) holds keys 32kb + 16g + 8ks + 0..7
            u32x4 va[4][ND];
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) read_v(grp, va[grp]);
#pragma unroll
            for (int grp = 0; grp < 4; ++grp)
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    o[d] = mfma_bf16(__builtin_bit_cast(v8bf, va[grp][d]), pb[grp / 2][grp % 2], o[d]);
            // reads run one MFMA group ahead
            __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
#pragma unroll
            for (int i = 0; i < 3 * ND; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, ND, 0);
        }
        if (PREP_on) {
            // S^T of tile t+1 = K . Q^T (Q hi and lo terms), both 32-key blocks
            v8i ka[NH][2];
#pragma unroll
            for (int h = 0; h < NH; ++h) read_k(h, ka[h]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = v16f{};
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma(ka[h][kb], qop[h][hl], s[kb]);
            convert_v(buf1, vt_base + ((r0 + 1) % 2) * L::VT_BYTES);
            // slice-0 operands first, slice-1 reads behind the slice-0 MFMAs,
            // the dequantisation (LDS reads, VALU, LDS writes) behind the rest
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 4 * NH - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
        }
    };
    using yes = std::true_type;
    using no = std::false_type;

    {
        const float f0 = wave < 2 ? load_factor(a, my_scales, head, t0) : 0.0f;
        const float f1 = wave < 2 && t0 + 1 < t1 ? load_factor(a, my_scales, head, t0 + 1) : 0.0f;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        store_factor<D>(smem, f0, qfac);
        if (t0 + 1 < t1) store_factor<D>(smem + L::BUF, f1, qfac);
    }
    __syncthreads();

    // Both groups run the same loop; the trailing group enters it one
    // interval late (an extra barrier first), the lead group leaves it with an
    // extra barrier, so both pass the same 2n+1 barriers.  The lead group
    // streams the tiles: tile t0+u+2 is issued in interval 2u+1 and landed
    // (waited for, factors stored) at the end of interval 2u+2.
    float nf = 0.0f;
    const int n = t1 - t0;
    half_m(t0 - 1, no{}, yes{});
    if (!lead) __syncthreads();
    for (int u = 0; u < n; ++u) {
        half_v(t0 + u);
        if (lead && u >= 1 && t0 + u + 1 < t1) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            store_factor<D>(smem + ((u + 1) % 3) * L::BUF, nf, qfac);
        }
        __syncthreads();
        if (lead && t0 + u + 2 < t1) {
            issue_tile<D>(a, head, t0 + u + 2, smem + ((u + 2) % 3) * L::BUF, wave);
            if (wave < 2) nf = load_factor(a, my_scales, head, t0 + u + 2);
        }
        half_m(t0 + u, yes{}, yes{});
        __syncthreads();
    }
    if (lead) __syncthreads();

    // ---- epilogue ------------------------------------------------------------
    // Normalised rows o = O / l go through this wave's LDS area (the Q
    // operands are no longer needed), rows of 2*D bytes whose 8-byte units are
    // XOR-swizzled by an even function of the row, then out to HBM in whole
    // 16-byte chunks:
    // bf16 outputs when there is one split, fp16 partials plus (max, sum) else.
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float f = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    const bool to_out = a.n_splits == 1;
    uint8_t *ob = qbase;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = 8 * d + 2 * q + g;              // 8-byte unit of d = 4u .. 4u+3
            const float x0 = o[d][4 * q] * f, x1 = o[d][4 * q + 1] * f;
            const float x2 = o[d][4 * q + 2] * f, x3 = o[d][4 * q + 3] * f;
            uint32_t w0, w1;
            if (to_out) {
                w0 = f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
                w1 = f32_to_bf16_rne(x2) | ((uint32_t)f32_to_bf16_rne(x3) << 16);
            } else {
                w0 = __builtin_bit_cast(uint32_t, h2{(_Float16)x0, (_Float16)x1});
                w1 = __builtin_bit_cast(uint32_t, h2{(_Float16)x2, (_Float16)x3});
            }
            *reinterpret_cast<v2i *>(ob + col * (2 * D) + 8 * (u ^ ((2 * col) & (D / 4 - 2)))) =
                v2i{(int)w0, (int)w1};
        }
    if (!to_out && g == 0 && q_ok) {
        const int64_t row = ((int64_t)split * a.n_q + qi) * a.n_heads + head;
        a.part_ml[2 * row] = kShift - cofs;             // running max, log2 units
        a.part_ml[2 * row + 1] = ltot;
    }
    // the rows were written by other lanes of this wave: wait for the LDS
    // writes and keep the compiler from moving the reads above them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int RCH = D / 8;                            // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < 32 * RCH / 64; ++i) {
        const int r = (i * 64 + lane) / RCH, k = (i * 64 + lane) % RCH;
        const int qr = qb * kQB + wave * kQW + r;
        if (qr >= a.n_q) continue;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ob + r * (2 * D) + 8 * ((2 * k) ^ ((2 * r) & (D / 4 - 2))));
        uint16_t *dst = to_out ? a.out + ((int64_t)qr * a.n_heads + head) * D
                               : a.part_o + (((int64_t)split * a.n_q + qr) * a.n_heads + head) * D;
        *reinterpret_cast<u32x4 *>(dst + 8 * k) = v;
    }
}

// Merge the split partials of (query, head) rows in split order: each split
// s holds a normalised row o_s (fp16) with its running max m_s (log2 units)
// and denominator l_s; out = sum_s w_s o_s / sum_s w_s, w_s = l_s 2^(m_s - M).
// D/8 lanes per row, eight elements per lane.
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a) {
    constexpr int LPR = D / 8;                       // lanes per row
    constexpr int RPB = 256 / LPR;                   // rows per workgroup
    const int64_t rows = (int64_t)a.n_q * a.n_heads;
    const int64_t qh = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (qh >= rows) return;
    const int e = 8 * (threadIdx.x % LPR);
    float m = -INFINITY;
    for (int s = 0; s < a.n_splits; ++s) m = fmaxf(m, a.part_ml[2 * (s * rows + qh)]);
    float l = 0.0f;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < a.n_splits; ++s) {
        const int64_t row = s * rows + qh;
        const float ls = a.part_ml[2 * row + 1];
        const float wgt = ls > 0.0f ? ls * __builtin_amdgcn_exp2f(a.part_ml[2 * row] - m) : 0.0f;
        l += wgt;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(a.part_o + row * D + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t word = v[k];                  // (bit_cast of a vector element
            const h2 x = __builtin_bit_cast(h2, word);   //  reference is not reliable)
            acc[2 * k] += wgt * (float)x[0];
            acc[2 * k + 1] += wgt * (float)x[1];
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = f32_to_bf16_rne(acc[2 * k] * inv) | ((uint32_t)f32_to_bf16_rne(acc[2 * k + 1] * inv) << 16);
    *reinterpret_cast<u32x4 *>(a.out + qh * D + e) = w;
}

}  // namespace

int attn_default_splits(int n_heads, int n_q, int n_valid) {
    const int n_qb = (n_q + kQB - 1) / kQB;
    const int tiles = (n_valid + kKT - 1) / kKT;
    const int units = n_heads * n_qb;
    int s = (256 + units / 2) / units;           // about one workgroup per CU
    if (s < 1) s = 1;
    if (s > tiles) s = tiles;
    return s;
}

size_t attn_workspace_bytes(int n_heads, int head_dim, int n_q, int n_splits) {
    if (n_splits <= 1) return 0;
    const size_t rows = (size_t)n_splits * n_q * n_heads;
    const size_t o_bytes = (rows * head_dim * sizeof(uint16_t) + 255) / 256 * 256;
    return o_bytes + rows * 2 * sizeof(float);
}

hipError_t launch_attention(const AttnArgs &a, int head_dim, hipStream_t s) {
    const int n_qb = (a.n_q + kQB - 1) / kQB;
    const int grid = n_qb * a.n_heads * a.n_splits;
    const int64_t rows = (int64_t)a.n_q * a.n_heads;
    if (head_dim == 128) {
        hipLaunchKernelGGL(attn_kernel<128>, dim3(grid), dim3(kThreads), Lds<128>::TOTAL, s, a);
        if (a.n_splits > 1)
            hipLaunchKernelGGL(combine_kernel<128>, dim3((rows + 15) / 16), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(attn_kernel<64>, dim3(grid), dim3(kThreads), Lds<64>::TOTAL, s, a);
        if (a.n_splits > 1)
            hipLaunchKernelGGL(combine_kernel<64>, dim3((rows + 31) / 32), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kvr
