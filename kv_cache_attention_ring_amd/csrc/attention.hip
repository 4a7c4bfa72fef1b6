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
// "split" of the 64-key tiles: with S splits, split s takes tiles s, s + S,
// s + 2S, ... in that order; each of its 8 waves (two per SIMD) owns 32
// queries.  Key tiles go global -> LDS with direct loads
// (global_load_lds, 16 bytes a lane, no VGPR staging) into five buffers, four
// tiles in flight.  The two waves of a SIMD alternate between a VALU
// half-step and a matrix half-step (see the main loop); two LDS-only
// barriers per tile.
//   S^T[key][query] = K . Q^T   on v_mfma_scale_f32_32x32x64_f8f6f4: A = FP8 K
//                               rows from LDS, B = Q as two E4M3 terms (hi + lo)
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
// slice.  Each query has its own power-of-two scale, applied by the matrix
// core as the E8M0 scale of its B column, and softmax_scale * log2(e) is
// folded into Q before it is split, so the accumulator holds the score in log2
// units up to the K row scale: one FMA per score applies sk_j.  The weights
// and V^T are bf16 (8 significant bits), so the second product needs no
// split.  Softmax runs in the log2 domain with a lazily updated running max
// (rescale only when a score passes it by more than 16, so weights stay below
// 2^16 and the fp32 sums cannot overflow).  Splits of one (head, query block)
// are merged by a second kernel in split order, so a call is deterministic and
// a linear window gives the same bits as the ring.
//
// Fused form (the chunk's write carried by the call that first reads it,
// [AI-cache]: every call's window holds the chunk's new rows).  The new keys
// are the last n_new in logical order, so with the tiles dealt in turn they
// sit at the end of every split.  Every workgroup writes its share of the
// chunk's rows after issuing its first tiles (the upkeep kernels' row
// arithmetic, rowquant.h, with stores that write through to memory), prepares
// its queries while they complete, then waits for them and counts itself
// done; before it streams its
// first tile holding new keys it waits (bounded) for the count to reach the
// grid, and it streams those tiles with device-scope loads, which miss any
// stale copy.  At the production shape that tile comes ~11 tiles into a
// split, long after the writes, so the wait is a single poll.  The host takes
// this form only when the whole grid can be resident at once.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "kvr_internal.h"
#include "rowquant.h"

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
constexpr int kNBuf = 5;          // FP8 tile buffers (tiles in flight + the one consumed)

template <int D>
struct Lds {
    static constexpr int CH = D / 16;            // 16-byte chunks per row
    // dequantised V^T of one tile: [d][64 keys] bf16, 128-byte rows, triple buffered
    static constexpr int VT_BYTES = D * kKT * 2;
    // one FP8 tile buffer: K rows, V rows, then the row scales, 64 floats per
    // wave of which the first 16 are used: wave w < 4 holds sk_j of keys
    // 16w .. 16w+15, wave w >= 4 sv_j of keys 16(w-4) .. +15 (keys past n_valid
    // hold the scale of a valid row; their weights are exactly zero)
    static constexpr int K_BYTES = kKT * D;
    static constexpr int V_BYTES = kKT * D;
    static constexpr int F_OFF = K_BYTES + V_BYTES;
    static constexpr int BUF = F_OFF + kNW * 64 * 4;
    static constexpr int TILE_OFF = 3 * VT_BYTES;
    static constexpr int FLAG_OFF = TILE_OFF + kNBuf * BUF;   // one word: the outcome of a wait
    static constexpr int TOTAL = FLAG_OFF + 16;
    // after the loop the tile buffers stage the output rows (2D bytes each)
    static constexpr int OUT_WAVE = kQW * 2 * D;
    static_assert(kNW * OUT_WAVE <= kNBuf * BUF, "output staging fits the tile buffers");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// LDS bank groups.  A 16-byte-per-lane read is served 16 consecutive lanes at
// a time over a 256-byte span (16 bank groups of 16 bytes), a 16-byte write 8
// lanes at a time over 128 bytes, the 8-byte transposing read 32 lanes at a
// time over 256 bytes (measured: SQ_LDS_BANK_CONFLICT of variants with one
// access pattern removed).  Chunk c of a row is stored at chunk position
// c ^ swizzle(row), with the swizzles chosen so that every access pattern below
// hits distinct bank groups within a step:
//   K rows (D bytes): one 16-lane step of the operand reads takes rows
//     {0..3, 16..19, 4..7, 20..23} (or those plus 8) of a 32-key block and one
//     chunk; with 128-byte rows the group is 8 * (row & 1) + position, so per
//     row parity the swizzle must be a permutation of the remaining row bits
//     (1, 2, 4); with 64-byte rows the group is 4 * (row & 3) + position (bits 2, 4).
//   V rows: the transposing reads of a step cover 16 consecutive rows of one
//     chunk: row >> 1 (128-byte rows), row >> 2 (64-byte rows).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
    return D == 128 ? (((row >> 1) & 3) | (((row >> 4) & 1) << 2)) : (((row >> 2) & 1) | (((row >> 4) & 1) << 1));
}
template <int D>
__device__ __forceinline__ int swz_v(int row) { return D == 128 ? row >> 1 : row >> 2; }
// V^T rows (one per d, 128 bytes = 8 chunks of 8 keys): chunk c of row d sits at
// c ^ f(d), f(d) = 4 d2 + 2 d1 + (d3 ^ d0) (bits of d), a permutation of 0..7
// both over 8 consecutive rows (the conversion writes) and, per row parity,
// over 16 consecutive rows (the MFMA operand reads).
__device__ __forceinline__ int vt_pos(int d, int c) {
    return d * (2 * kKT) + 16 * (c ^ ((((d >> 1) & 3) << 1) | (((d >> 3) ^ d) & 1)));
}

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two floats -> packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf2));
}

// E4M3 x E4M3 with E8M0 scales: 2^(sb-127) (byte 0 of sb) scales the B column
// of this lane over its 32-wide half of the contraction; the A rows are
// unscaled (127 = 2^0).
__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// Exponent k of the smallest power of two with 448 * 2^k >= a (a >= 0),
// clamped below at -127; from the fp32 fields, 448 = 1.75 * 2^8.
__device__ __forceinline__ int scale_exponent(float a) {
    const uint32_t b = __float_as_uint(a);
    const int k = (int)(b >> 23) - ((b & 0x7FFFFFu) <= 0x600000u ? 135 : 134);
    return k < -127 ? -127 : k;
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

// ds_read_b64_tr_b8 issued from inline assembly.  The compiler treats a
// transposing read of a direct-to-LDS (global_load_lds) target as aliasing
// every load still in flight and waits for all of them (vmcnt(0)) first,
// which would serialise the tile prefetch; here the read's own completion is
// waited for explicitly with lds_wait(), which also orders the uses of the
// result after the wait.  Loads the compiler does not see only make its
// own lgkmcnt waits more conservative, never insufficient, since LDS
// operations complete in issue order.
__device__ __forceinline__ v2i lds_read_tr8(const uint8_t *p) {
    v2i r;
    const uint32_t addr = (uint32_t)(uintptr_t)(LDS_AS const void *)p;
    asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
__device__ __forceinline__ void lds_wait(v2i &r) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r)); }

// Q words are loaded with inline assembly and waited for explicitly: the
// compiler's own wait before their first use would be vmcnt(0) once tile
// loads (global_load_lds) have been issued behind them, i.e. it would wait
// for the whole tile prefetch.  qwait<N> leaves the N newest loads in flight.
__device__ __forceinline__ u32x4 gload16(const void *p) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p));
    return r;
}
template <int N, int W>
__device__ __forceinline__ void qwait(u32x4 (&q)[W]) {
    asm volatile("s_waitcnt vmcnt(%1)" : "+v"(q[0]) : "n"(N));
#pragma unroll
    for (int i = 1; i < W; ++i) asm volatile("" : "+v"(q[i]));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also orders
// global memory, and because a global_load_lds counts as an outstanding
// memory write the compiler would put s_waitcnt vmcnt(0) in front of it,
// i.e. wait for every tile still streaming in.  Tiles are made visible by
// each wave's own vmcnt wait before the barrier instead.  The "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Cache slot of key idx in logical order: with PREFIX, the prefix rows first,
// then the ring's keys, oldest first (ring slot s is cache slot prefix + s);
// without, the ring alone (prefix 0, capacity = window).  A separate
// instantiation keeps the mapping of a pure ring free of the prefix test.
template <bool PREFIX>
__device__ __forceinline__ int slot_of(const AttnArgs &a, int idx) {
    idx = idx < a.n_valid ? idx : a.n_valid - 1;       // keys past the window: any valid row
    if constexpr (PREFIX) {
        if (idx < a.prefix) return idx;
        const int s = a.slot_start + idx - a.prefix;
        return a.prefix + (s >= a.cap ? s - a.cap : s);
    } else {
        const int s = a.slot_start + idx;
        return s >= a.window ? s - a.window : s;
    }
}

// Tile streaming.  Every wave loads its eighth of each tile straight into
// LDS (global_load_lds, no VGPR staging), with all 64 lanes active so the
// loads carry no control flow: 16-byte chunks of K and V rows (D = 128: each
// wave 1 KB of K and 1 KB of V; D = 64: waves 0..3 1 KB of K, 4..7 1 KB of
// V), where LDS chunk position p of row p / CH receives global chunk
// (p % CH) ^ swizzle(row); and the per-key scales, 4 bytes a lane (lanes
// 16..63 repeat lanes 0..15).  That is a fixed number of loads per wave and
// tile, so a wave's vmcnt says how many of its tiles are still in flight;
// each wave waits for its own part of a tile before the barrier that
// publishes it.
template <int D>
constexpr int ops_per_tile() { return D == 128 ? 3 : 2; }

// AUX: the loads' cache policy (kSc1: device scope, for rows written in this
// launch by workgroups that may run on other XCDs; such a load misses in any
// cache that may hold an older copy of the line).
constexpr int kSc1 = 16;
template <int D, bool PREFIX, int AUX = 0>
__device__ __forceinline__ void issue_tile(const AttnArgs &a, const uint8_t *kh, const uint8_t *vh,
                                           const float *scales_h, int tile, uint8_t *buf, int wave) {
    using L = Lds<D>;
    constexpr int CH = L::CH;
    const int lane = threadIdx.x % 64;
    if constexpr (D == 128) {
        const int p0 = 64 * wave;
        const int p = p0 + lane;
        const int row = p / CH, pos = p % CH;
        const uint32_t srow = (uint32_t)slot_of<PREFIX>(a, tile * kKT + row) * D;
        const uint32_t offk = srow + 16 * (pos ^ (swz_k<D>(row) & (CH - 1)));
        const uint32_t offv = srow + 16 * (pos ^ (swz_v<D>(row) & (CH - 1)));
        __builtin_amdgcn_global_load_lds(kh + offk, (LDS_AS void *)(buf + 16 * p0), 16, 0, AUX);
        __builtin_amdgcn_global_load_lds(vh + offv, (LDS_AS void *)(buf + L::K_BYTES + 16 * p0), 16, 0, AUX);
    } else {
        const bool is_k = wave < 4;
        const int p0 = 64 * (wave % 4);
        const int p = p0 + lane;
        const int row = p / CH, pos = p % CH;
        const uint32_t off = (uint32_t)slot_of<PREFIX>(a, tile * kKT + row) * D +
                             16 * (pos ^ ((is_k ? swz_k<D>(row) : swz_v<D>(row)) & (CH - 1)));
        __builtin_amdgcn_global_load_lds((is_k ? kh : vh) + off,
                                         (LDS_AS void *)(buf + (is_k ? 0 : L::K_BYTES) + 16 * p0), 16, 0, AUX);
    }
    const int key = 16 * (wave % 4) + lane % 16;
    __builtin_amdgcn_global_load_lds(scales_h + slot_of<PREFIX>(a, tile * kKT + key),
                                     (LDS_AS void *)(buf + L::F_OFF + 256 * wave), 4, 0, AUX);
}

// scale slot of key k (0..63): K sk_j or V sv_j
__device__ __forceinline__ int fk_index(int k) { return 64 * (k >> 4) + (k & 15); }
__device__ __forceinline__ int fv_index(int k) { return 64 * (4 + (k >> 4)) + (k & 15); }

// Wait until at most `later` of this wave's tiles issued after the awaited
// one are still in flight (the count must be an immediate).
template <int D>
__device__ __forceinline__ void wait_tiles(int later) {
    constexpr int OPT = ops_per_tile<D>();
    static_assert(OPT * (kNBuf - 2) <= 63, "vmcnt range");
    if (later <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPT) : "memory");
    else if (later == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * OPT) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * OPT) : "memory");
}

// Fused form, workgroup w's share of the chunk: its rows, each written
// exactly as the write kernel writes it (rowquant.h) but with stores that
// write through to memory, since workgroups on other XCDs read them in this
// launch.  Rows are numbered (K/V, token, head) in the inputs' order;
// workgroup w takes rows 64 (w + i n_writers) + g, one row per 8-lane group
// g, the loads of two rows in flight together.
template <int D, bool BF16>
__device__ __forceinline__ void fused_write(const AttnArgs &a, int w) {
    constexpr int EPT = D / rowq::kRowLanes;
    constexpr int kGroups = kThreads / rowq::kRowLanes;
    constexpr int kRows = 2;                               // rows per group with loads in flight together
    const int lane8 = threadIdx.x % rowq::kRowLanes;
    const int per_kv = a.w_n_new * a.n_heads, rows = 2 * per_kv;
    const int step = a.n_writers * kGroups;
    for (int r0 = w * kGroups + (int)threadIdx.x / rowq::kRowLanes; r0 < rows; r0 += kRows * step) {
        rowq::RawChunk<EPT, BF16> raw[kRows];
        float4 csv[kRows][EPT / 4];
        int rem[kRows];
        bool is_v[kRows];
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            const int r = min(r0 + u * step, rows - 1);
            is_v[u] = r >= per_kv;
            rem[u] = is_v[u] ? r - per_kv : r;             // token * n_heads + head
            raw[u].load(is_v[u] ? a.w_v : a.w_k, (int64_t)rem[u] * D + lane8 * EPT);
            const int j = rem[u] / a.n_heads;
            const float4 *t = reinterpret_cast<const float4 *>(a.w_cs + (int64_t)j * D + lane8 * EPT);
#pragma unroll
            for (int v = 0; v < EPT / 4; ++v) csv[u][v] = is_v[u] ? float4{} : t[v];
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            if (r0 + u * step >= rows) break;
            const int j = rem[u] / a.n_heads, h = rem[u] - j * a.n_heads;
            float x[EPT];
            raw[u].to_f32(x);
            if (!is_v[u]) rowq::rotate_pairs<EPT>(x, reinterpret_cast<const float *>(csv[u]));
            int slot = a.w_head + j;
            if (slot >= a.cap) slot -= a.cap;
            const int64_t row = (int64_t)h * a.window + a.prefix + slot;
            rowq::quantize_store<EPT, true>(x, (is_v[u] ? a.w_v_codes : a.w_k_codes) + row * D + lane8 * EPT,
                                            (is_v[u] ? a.w_v_scales : a.w_k_scales) + row, lane8 == 0);
        }
    }
}

// Fused form, before a workgroup streams its first tile holding new keys:
// thread 0 polls until every workgroup has counted its share of the chunk
// written (sync[0] == n_writers), at most sync[3] polls (when nonzero; else
// kFusedSpinLimit); the last of the n_waiters workgroups through clears
// sync[0] and sync[1] for the next call.  A wait that gives up adds one to
// sync[2].  Thread 0 leaves the outcome (1: gave up) in *flag, which the
// caller's barrier publishes to the workgroup.  No cache is invalidated: the
// tiles that hold new keys are streamed with device-scope loads.
__device__ __forceinline__ void poll_writers(const AttnArgs &a, uint32_t *flag) {
    if (threadIdx.x == 0) {
        uint32_t *sync = a.sync;
        const uint32_t lim = __hip_atomic_load(sync + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t limit = lim ? lim : kFusedSpinLimit;
        uint32_t polls = 0, gave_up = 0;
        while (__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)a.n_writers) {
            if (++polls >= limit) {
                gave_up = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (gave_up) __hip_atomic_fetch_add(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__hip_atomic_fetch_add(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (uint32_t)a.n_waiters - 1) {
            __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *flag = gave_up;
    }
}

// QTAB: the queries' rotation comes from (cos, sin) rows, one per query
// (a.q_cs, [n_q][D/2][2] fp32: the 3-D form, where the angle of a pair is its
// own axis coordinate times its frequency), instead of position times frequency.
// PREFIX: keys start with the cache's fixed prefix rows (see slot_of).
// FUSE: the fused form (the chunk's write; position form only).
template <int D, bool BF16, bool QTAB, bool PREFIX, bool FUSE = false>
__global__ void __launch_bounds__(kThreads, 2) attn_kernel(AttnArgs a) {
    static_assert(!(FUSE && QTAB), "the fused form takes query positions");
    using L = Lds<D>;
    constexpr int CH = L::CH;
    constexpr int NH = D / 64;          // 64-wide d slices of the QK^T contraction
    constexpr int ND = D / 32;          // 32-row d blocks of O^T
    constexpr int P = kNBuf - 1;        // tiles in flight ahead of the one consumed
    static_assert(P - 1 <= 3, "wait_tiles covers up to three later tiles");
    extern __shared__ __align__(16) uint8_t smem[];

    // ---- (head, split, query block) ------------------------------------------
    // Workgroups are dealt round-robin over the 8 XCDs (block b runs on XCD
    // b % 8).  Renumber them so that the blocks of one XCD take consecutive
    // slots of the (unit, query block) order: the query blocks of a (head,
    // split) key range then share an XCD and its L2, and the range is read
    // from HBM once rather than once per query block (at most 7 ranges
    // straddle two XCDs).
    const int n_qb = (a.n_q + kQB - 1) / kQB;
    bool bad = false;
    int unit, qb;
    {
        const int b = blockIdx.x, G = gridDim.x;
        const int xcd = b % 8, k = b / 8;
        const int per = G / 8, extra = G % 8;             // XCDs below `extra` hold per + 1
        const int slot = xcd * per + min(xcd, extra) + k;
        unit = slot / n_qb;
        qb = slot % n_qb;
    }
    const int head = unit / a.n_splits;
    const int split = unit % a.n_splits;
    // The 64-key tiles are dealt to the splits in turn: split s takes tiles
    // s, s + S, s + 2S, ... (S = n_splits), visited in that order (local
    // index u = 0 .. n-1), so every split's keys stay in logical order and
    // the newest keys of the window sit at the end of every split.
    const int n_tiles = (a.n_valid + kKT - 1) / kKT;
    const int S = a.n_splits;
    const int n = (n_tiles - split + S - 1) / S;
    auto tile_at = [&](int u) { return split + min(u, n - 1) * S; };
    // fused form: the first local tile holding a key of the chunk; n + P when
    // none does (no wait below can match it, and every tile loads plainly)
    int u_new = n + P;
    if constexpr (FUSE) {
        const int ft = a.first_new / kKT;
        const int c = ft <= split ? 0 : (ft - split + S - 1) / S;
        if (c < n) u_new = c;
    }
    uint32_t *flag = reinterpret_cast<uint32_t *>(smem + L::FLAG_OFF);

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int g = lane / 32, col = lane % 32;
    const int qi = qb * kQB + wave * kQW + col;         // this lane's query
    const bool q_ok = qi < a.n_q;
    const bool lead = wave < kNW / 2;
    const int64_t hoff = (int64_t)head * a.window;
    const uint8_t *kh = a.k_codes + hoff * D, *vh = a.v_codes + hoff * D;
    const float *scales_h = (wave < 4 ? a.k_scales : a.v_scales) + hoff;
    uint8_t *tiles = smem + L::TILE_OFF;
    uint8_t *vt_base = smem + 0;

    // ---- Q straight into MFMA B-operand order ----------------------------------
    // Lane (query, g) holds d in [64h + 32g, +32) of its query for each slice h:
    // 64 contiguous bytes (bf16) per slice.  The raw words are loaded first
    // (rows past n_q read row n_q-1; their results are never stored), the tiles are
    // issued behind them, and only then are the words unpacked, so the wait
    // for Q does not hold back the tile stream.
    constexpr int QV = NH * 32;                           // Q elements per lane
    constexpr int QW = BF16 ? QV / 8 : QV / 4;            // 16-byte words per lane
    constexpr int CW = QTAB ? QV / 4 : 1;                 // 16-byte words of (cos, sin) per lane
    u32x4 qraw[QW];
    u32x4 csraw[CW];
    {
        const int64_t qrow = min(qi, a.n_q - 1);
        const int64_t row = (qrow * a.n_heads + head) * D;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int d0 = 64 * h + 32 * g;
            const u32x4 *src = BF16 ? reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) + row + d0)
                                    : reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(a.q) + row + d0);
#pragma unroll
            for (int c = 0; c < QW / NH; ++c) qraw[(QW / NH) * h + c] = gload16(src + c);
        }
        if constexpr (QTAB) {
            // word c (of 8 per slice h = c / 8) of the lane's (cos, sin):
            //   lane layout: load c of the wave reads 64 consecutive 16-byte
            //     words, one per lane (whole lines): lane_base + 64 c;
            //   row layout: the (cos, sin) of the lane's pairs 32h + 16g ..
            //     +15 of each slice h, 128 contiguous bytes per slice:
            //     row_base + 16 (c / 8) + c % 8.
            // One sequence of loads for both (the layout is uniform), so the
            // loads carry no control flow.
            const bool lanes = a.q_cs_lanes != 0;
            const u32x4 *lane_base = reinterpret_cast<const u32x4 *>(a.q_cs) +
                                     (int64_t)(qb * kNW + wave) * (8 * NH) * 64 + lane;
            const u32x4 *row_base = reinterpret_cast<const u32x4 *>(a.q_cs + 2 * (qrow * (D / 2) + 16 * g));
            const u32x4 *base = lanes ? lane_base : row_base;
#pragma unroll
            for (int c = 0; c < 8 * NH; ++c) csraw[c] = gload16(base + (lanes ? 64 * c : 16 * (c / 8) + c % 8));
        }
    }

    // start streaming the first P tiles (and their scales); always P of them,
    // so the compiler can count them in its wait for Q (a split shorter than
    // P tiles reloads its last tile into the spare buffers).  Fused form: the
    // tiles before u_new now, then this workgroup's share of the chunk.
#pragma unroll
    for (int k = 0; k < P; ++k) {
        if constexpr (FUSE) {
            if (k < u_new) issue_tile<D, PREFIX>(a, kh, vh, scales_h, tile_at(k), tiles + k * L::BUF, wave);
        } else {
            issue_tile<D, PREFIX>(a, kh, vh, scales_h, tile_at(k), tiles + k * L::BUF, wave);
        }
    }
    if constexpr (FUSE) fused_write<D, BF16>(a, (int)blockIdx.x);

    // position form: the rotation depends on the query's position only, so its
    // (cos, sin) are formed while Q and the first tiles are in flight.  Pair i
    // of the lane's slice h has frequency index 32h + 16g + i; the angle
    // (position times theta_i / 2pi, in revolutions) is formed in fp64 and its
    // fractional part, in [0, 1), goes to the hardware sine and cosine.  theta
    // for the g = 1 half is theta_{32h+i} * base^(-32/D) (exact to an ulp of
    // fp64).
    constexpr int PC = QTAB ? 1 : QV / 2;
    float pcos[PC], psin[PC];
    if constexpr (!QTAB) {
        const double pos = (double)(a.q_pos0 + qi);
        const double gmul = g ? a.rev_step : 1.0;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const double r = pos * (a.rev.t[32 * h + i] * gmul);
                const float fr = (float)__builtin_amdgcn_fract(r);
                pcos[16 * h + i] = __builtin_amdgcn_cosf(fr);
                psin[16 * h + i] = __builtin_amdgcn_sinf(fr);
            }
        // keep them ahead of the wait below
#pragma unroll
        for (int j = 0; j < PC; ++j) asm volatile("" : "+v"(pcos[j]), "+v"(psin[j]));
    }
    if constexpr (FUSE) {
        // the chunk's rows went to memory through the caches: once every
        // lane's stores are acknowledged, the workgroup counts itself done
        // (no write-back of this XCD's L2 is needed for them).  A workgroup
        // that waits in this prologue counts itself first; the others count
        // after preparing their queries (below), behind which the stores'
        // latency is hidden -- every workgroup counts itself before it waits
        if (u_new < P) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // a tile holding new keys is among the first P: wait for every
            // share of the chunk, then stream those tiles past stale copies
            poll_writers(a, flag);
            lds_barrier();
            bad = __builtin_amdgcn_readfirstlane(*flag) != 0;
#pragma unroll
            for (int k = 0; k < P; ++k)
                if (k >= u_new)
                    issue_tile<D, PREFIX, kSc1>(a, kh, vh, scales_h, tile_at(k), tiles + k * L::BUF, wave);
        }
    }
    qwait<P * ops_per_tile<D>()>(qraw);
    if constexpr (QTAB) {
        // issued before the tiles, so the wait above covered them too; order
        // their uses after it
#pragma unroll
        for (int i = 0; i < CW; ++i) asm volatile("" : "+v"(csraw[i]));
    }

    float qv[QV];
#pragma unroll
    for (int w = 0; w < QW; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (BF16) {
                qv[8 * w + 2 * e] = __uint_as_float(qraw[w][e] << 16);
                qv[8 * w + 2 * e + 1] = __uint_as_float(qraw[w][e] & 0xFFFF0000u);
            } else {
                qv[4 * w + e] = __uint_as_float(qraw[w][e]);
            }
        }

    // rotate (rotation rows, or the (cos, sin) formed above)
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float cc, ss;
            if constexpr (QTAB) {
                const u32x4 w = csraw[8 * h + i / 2];
                cc = __uint_as_float(w[2 * (i % 2)]);
                ss = __uint_as_float(w[2 * (i % 2) + 1]);
            } else {
                cc = pcos[16 * h + i];
                ss = psin[16 * h + i];
            }
            const float x0 = qv[32 * h + 2 * i], x1 = qv[32 * h + 2 * i + 1];
            qv[32 * h + 2 * i] = x0 * cc - x1 * ss;
            qv[32 * h + 2 * i + 1] = x0 * ss + x1 * cc;
        }
    // scores in log2 units: softmax_scale * log2(e) (c2) times a per-query
    // power-of-two scale 2^-qk (lanes l and l ^ 32 hold the two halves of one
    // query) multiplies q, so the scaled query has absmax in (224, 448]; the
    // product by 2^-qk c2 equals that by c2 then by 2^-qk bit for bit (a power
    // of two commutes with rounding), and rounding is monotone, so the absmax
    // of c2 q is c2 times the absmax of q.  Lanes of queries past n_q hold row
    // n_q - 1 (their results are never stored).
    const float c2 = a.softmax_scale * kLog2e;
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < QV; ++e) am = fmaxf(am, fabsf(qv[e]));
    am *= c2;
    am = fmaxf(am, __shfl_xor(am, 32));
    const int qk = scale_exponent(am);
    const int qsc = qk + 127;                                   // E8M0 byte
    const float qscale = __uint_as_float((uint32_t)(127 - qk) << 23) * c2;   // 2^-qk c2

    // Q hi/lo E4M3 operands: byte k of qop[h][hl] is element k of the lane's slice h
    v8i qop[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int w4 = 0; w4 < 8; ++w4) {
            uint32_t hi, lo;
            const float *x = qv + 32 * h + 4 * w4;
            split4(x[0] * qscale, x[1] * qscale, x[2] * qscale, x[3] * qscale, hi, lo);
            qop[h][0][w4] = (int)hi;
            qop[h][1][w4] = (int)lo;
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
                koff[kb][h][e] = row * D + 16 * ((4 * h + 2 * g + e) ^ (swz_k<D>(row) & (CH - 1)));
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
        cv_src[i] = L::K_BYTES + row * D + 16 * (dc ^ (swz_v<D>(row) & (CH - 1))) + 8 * (j % 2);
        cv_dst[i] = vt_pos(16 * dc + j, kg);
        cv_kg[i] = kg;
    }
    static_assert(NBLK % (4 * kNW) == 0, "whole dequantisation rounds");
    auto convert_read = [&](const uint8_t *buf, v2i (&ut)[NCV], f32x4 (&sv)[NCV][2]) {
        const float *fv = reinterpret_cast<const float *>(buf + L::F_OFF);
#pragma unroll
        for (int i = 0; i < NCV; ++i) ut[i] = lds_read_tr8(buf + cv_src[i]);
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            sv[i][0] = *reinterpret_cast<const f32x4 *>(fv + fv_index(8 * cv_kg[i]));
            sv[i][1] = *reinterpret_cast<const f32x4 *>(fv + fv_index(8 * cv_kg[i] + 4));
        }
    };
    auto convert_write = [&](const v2i (&ut)[NCV], const f32x4 (&sv)[NCV][2], uint8_t *vt) {
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const v2i u = ut[i];
            const f32x4 s0 = sv[i][0], s1 = sv[i][1];
            const auto x0 = __builtin_amdgcn_cvt_pk_f32_fp8(u[0], false);
            const auto x1 = __builtin_amdgcn_cvt_pk_f32_fp8(u[0], true);
            const auto x2 = __builtin_amdgcn_cvt_pk_f32_fp8(u[1], false);
            const auto x3 = __builtin_amdgcn_cvt_pk_f32_fp8(u[1], true);
            const u32x4 w = {pack_bf16(x0[0] * s0[0], x0[1] * s0[1]), pack_bf16(x1[0] * s0[2], x1[1] * s0[3]),
                             pack_bf16(x2[0] * s1[0], x2[1] * s1[1]), pack_bf16(x3[0] * s1[2], x3[1] * s1[3])};
            *reinterpret_cast<u32x4 *>(vt + cv_dst[i]) = w;
        }
    };

    // ---- main loop: two wave groups in ping-pong --------------------------------
    // Per tile t a wave runs two half-steps:
    //   V(t): scores, running max, weights p = 2^x and their sum -> bf16 B
    //         operands; its share of the dequantisation of V(t+1) into V^T
    //   M(t): O^T += V^T(t) . P^T(t); S^T(t+1) = K(t+1) . Q^T; the K scales of
    //         tile t+1 for V(t+1) (they land during the barrier wait)
    // (t a local tile index) in the order M(-1) V(0) M(0) V(1) ... M(n-1),
    // where M(-1) only holds the tile-0 parts.  Half-steps are separated by
    // workgroup barriers,
    // and waves 4..7 run one half-step behind waves 0..3, so the two waves
    // sharing a SIMD are in different half-steps: one keeps the matrix core
    // busy while the other uses the VALU.
    // Buffers: local tile k sits in tile buffer k mod kNBuf.  Each wave issues
    // its part of local tile u+P at the end of its M(u), behind the last
    // MFMAs (so that M(u) starts with its operand reads),
    // and lands (waits for) its part of tile u+2 at the end of V(u); the
    // barrier that follows publishes it before its first use, in V(u+1) and
    // M(u+1).  Tile u+1 is read in V(u) and M(u); its last reader, the
    // trailing group's M(u), ends at least two intervals before the buffer is
    // reloaded (with tile u+6, at the end of M(u+2)).  V^T is triple buffered
    // (below).
    v16f o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = v16f{};
    float lsum0 = 0.0f, lsum1 = 0.0f;   // this lane's share of the softmax denominator
    float cofs = 0.0f;                  // kShift - running max (log2 units)
    v16f s[2];                          // S^T of the tile of the next V half-step
    v8bf pb[2][2];                      // P of the tile of the next M half-step

    f32x4 fkr[2][4];                    // K scales of the tile of the next V half-step
    auto read_fk = [&](const uint8_t *bk) {
        const float *fk = reinterpret_cast<const float *>(bk + L::F_OFF);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                fkr[kb][q] = *reinterpret_cast<const f32x4 *>(fk + fk_index(32 * kb + 16 * g + 4 * q));
    };
    auto half_v = [&](int t, const uint8_t *buf, const uint8_t *buf1, uint8_t *vt_next) {
        (void)buf;
        v2i ut[NCV];
        f32x4 sv[NCV][2];
        convert_read(buf1, ut, sv);
        // scores (log2 units, shifted by cofs): the accumulator times the K row
        // scale; register r of block kb is key 32kb + 16g + r of the tile
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 f = fkr[kb][q];
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kb][4 * q + r] = s[kb][4 * q + r] * f[r] + cofs;
            }
        // running max as a tree of three-input maxima (16 of them for 32
        // values, depth 4): ten of three scores, four of three of those, then
        // the last two with the two scores left over
        float m10[10];
#pragma unroll
        for (int i = 0; i < 10; ++i)
            m10[i] = fmaxf(fmaxf(s[(3 * i) / 16][(3 * i) % 16], s[(3 * i + 1) / 16][(3 * i + 1) % 16]),
                           s[(3 * i + 2) / 16][(3 * i + 2) % 16]);
        float m4[4];
#pragma unroll
        for (int i = 0; i < 3; ++i) m4[i] = fmaxf(fmaxf(m10[3 * i], m10[3 * i + 1]), m10[3 * i + 2]);
        m4[3] = fmaxf(fmaxf(m10[9], s[1][14]), s[1][15]);
        float mx = fmaxf(fmaxf(fmaxf(m4[0], m4[1]), m4[2]), m4[3]);
        const int lim = a.n_valid - tile_at(t) * kKT;     // valid keys of this tile
        if (lim < kKT) {                                  // last tile of the window
            mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = 32 * kb + 16 * g + r < lim ? s[kb][r] : -INFINITY;
                    s[kb][r] = v;
                    mx = fmaxf(mx, v);
                }
        }
        {
            // max with the other half of the wave (lanes l and l ^ 32 hold the
            // same query): swap the halves across two copies
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const bool first = t == 0;
        const bool over = mx > kShift + kTau;
        if (__any(first || over)) {
            float shift = 0.0f;                  // new cofs = cofs - shift
            if (first) {
                shift = mx - kShift;
            } else if (over) {
                shift = mx - kShift;
                const float alpha = __builtin_amdgcn_exp2f(-shift);
                lsum0 *= alpha;
                lsum1 *= alpha;
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
                    float &acc = (e & 1) ? lsum1 : lsum0;
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, (uint32_t)w[e]), one2, acc,
                                                          false);
                }
                // keep the weights computed in this half-step (not sunk
                // into the matrix half-step that consumes them); a use, not
                // a redefinition, so they stay in the registers they are
                // formed in
                asm volatile("" ::"v"(w));
                pb[kb][ks] = __builtin_bit_cast(v8bf, w);
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < NCV; ++i) asm volatile("" : "+v"(ut[i]));
        if (t + 1 < n) convert_write(ut, sv, vt_next);  // V^T of tile t+1
    };

    // M half-step.  PV and PREP select the parts (both in the steady state).
    auto half_m = [&](int t, const uint8_t *buf1, const uint8_t *vt, auto PV, auto PREP_) {
        constexpr bool PREP = decltype(PREP_)::value;
        const bool PREP_on = PREP && t + 1 < n;
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
        v8i ka[NH][2];                                 // K operands of tile t+1
        if constexpr (decltype(PV)::value) {
            // O^T += V^T . P^T; A-operand lane (d, g) holds keys 32kb + 16g + 8ks + 0..7.
            // The K operands of tile t+1 are read behind the V^T reads (reading
            // the next buffer is harmless when there is no tile t+1).
            u32x4 va[4][ND];
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) read_v(grp, va[grp]);
            if constexpr (PREP) {
#pragma unroll
                for (int h = 0; h < NH; ++h) read_k(h, ka[h]);
            }
#pragma unroll
            for (int grp = 0; grp < 4; ++grp)
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    o[d] = mfma_bf16(__builtin_bit_cast(v8bf, va[grp][d]), pb[grp / 2][grp % 2], o[d]);
            // reads run one MFMA group ahead; the K reads behind the last groups
            constexpr int KPER = PREP ? (4 * NH + ND - 1) / ND : 0;   // K reads per last-group MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
#pragma unroll
            for (int i = 0; i < 3 * ND; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (KPER > 0) __builtin_amdgcn_sched_group_barrier(0x100, KPER, 0);
            }
        } else if constexpr (PREP) {
#pragma unroll
            for (int h = 0; h < NH; ++h) read_k(h, ka[h]);
        }
        if (PREP_on) {
            // S^T of tile t+1 = K . Q^T (Q hi and lo terms), both 32-key blocks
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = v16f{};
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma(ka[h][kb], qop[h][hl], s[kb], qsc);
            read_fk(buf1);                             // K scales of tile t+1
        }
    };
    // (the barrier after a matrix half-step waits for every LDS read, the K
    // scales included; the loop redefines them after it so the compiler, which
    // does not see that wait, places none of its own before their use)
    using yes = std::true_type;
    using no = std::false_type;

    // Every wave lands its own part of a tile (waits for it) two tiles ahead,
    // at the end of its V(u): tile u+2, whose V rows the next V half-step
    // dequantises; the barrier that follows publishes it.  The newest tile a
    // wave has issued before V(u) ends is max(P-1, min(u+P-1, n-1)).
    auto land = [&](int u, int m) {                    // local tile m
        if (m < n) wait_tiles<D>(max(P - 1, min(u + P - 1, n - 1)) - m);
    };
    if constexpr (FUSE) {
        if (u_new >= P) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    land(-1, 0);
    land(-1, 1);
    lds_barrier();
    if (lead) half_m(-1, tiles, vt_base, no{}, yes{});  // S^T of local tile 0 (lead group)
    {                                                  // V^T of local tile 0
        v2i ut[NCV];
        f32x4 sv[NCV][2];
        convert_read(tiles, ut, sv);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < NCV; ++i) asm volatile("" : "+v"(ut[i]));
        convert_write(ut, sv, vt_base);
    }
    lds_barrier();

    // Both groups run the same loop; the trailing group enters it one
    // interval late (its S^T of local tile 0 and an extra barrier first), the lead
    // group leaves it with an extra barrier, so both pass the same 2n+1
    // barriers.
    //   V(u): scores and weights of tile u, V^T of tile u+1 (buffer (u+1)%3)
    //   M(u): O^T += V^T(u) . P^T(u), S^T of tile u+1
    // V^T(u+1) is written in intervals 2u, 2u+1 and read in 2u+3, 2u+4; its
    // buffer last held V^T(u-2), read in 2u-3, 2u-2.
    if (!lead) {
        // the trailing group's S^T of local tile 0, in the interval in which
        // the lead group runs V(0) (its matrix work then pairs with that VALU
        // half-step rather than with the lead group's own S^T in the prologue)
        __builtin_amdgcn_s_setprio(1);
        half_m(-1, tiles, vt_base, no{}, yes{});
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(fkr[kb][q]));
    }
    int bcur = 0;                                      // tile buffer of local tile u
    int vcur = 0;                                      // V^T buffer of local tile u
    for (int u = 0; u < n; ++u) {
        const int bnext = bcur + 1 == kNBuf ? 0 : bcur + 1;
        const int vnext = vcur + 1 == 3 ? 0 : vcur + 1;
        uint8_t *buf = tiles + bcur * L::BUF;
        uint8_t *buf1 = tiles + bnext * L::BUF;
        half_v(u, buf, buf1, vt_base + vnext * L::VT_BYTES);
        land(u, u + 2);
        // fused form: before the first tile holding new keys is streamed,
        // wait for every share of the chunk (thread 0 polls; the barrier
        // below publishes the outcome)
        const bool wait_here = FUSE && u + P == u_new;
        if (wait_here) poll_writers(a, flag);
        lds_barrier();
        if (wait_here) bad = __builtin_amdgcn_readfirstlane(*flag) != 0;
        __builtin_amdgcn_s_setprio(1);                 // the MFMA half-step issues first
        half_m(u, buf1, vt_base + vcur * L::VT_BYTES, yes{}, yes{});
        if (u + P < n) {                               // stream local tile u+P (the barrier
            int bl = bcur + P;                         // before M(u) ended every read of its buffer)
            bl = bl >= kNBuf ? bl - kNBuf : bl;
            if (FUSE && u + P >= u_new)
                issue_tile<D, PREFIX, kSc1>(a, kh, vh, scales_h, tile_at(u + P), tiles + bl * L::BUF, wave);
            else
                issue_tile<D, PREFIX>(a, kh, vh, scales_h, tile_at(u + P), tiles + bl * L::BUF, wave);
        }
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(fkr[kb][q]));
        bcur = bnext;
        vcur = vnext;
    }
    if (lead) lds_barrier();
    // a split shorter than P tiles may still be reloading its last tile into
    // spare buffers: let every load land before the buffers stage the output
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();

    // ---- epilogue ------------------------------------------------------------
    // Normalised rows o = O / l go through this wave's LDS area (inside the
    // tile buffers, all consumed), rows of 2*D bytes whose 8-byte units are
    // XOR-swizzled by an even function of the row, then out to HBM in whole
    // 16-byte chunks:
    // bf16 outputs when there is one split, fp16 partials plus (max, sum,
    // exponent) else.  A partial row whose largest element reaches 2^15 is
    // stored times 2^-e (e the power of two that brings it below 2^15; fp16
    // holds values below 65504), and e goes beside it for the merge; every
    // other row has e = 0 and is stored as is.
    const float lsum = lsum0 + lsum1;
    const float ltot = lsum + __shfl_xor(lsum, 32);
    float f = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    if constexpr (FUSE) {
        if (bad) f = __builtin_nanf("");                 // the wait for the writers gave up
    }
    const bool to_out = a.n_splits == 1;
    uint8_t *ob = tiles + wave * L::OUT_WAVE;
    int ex = 0;
    float post = 1.0f;
    if (!to_out) {
        float om = 0.0f;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) om = fmaxf(om, fabsf(o[d][r]));
        om *= f;
        om = fmaxf(om, __shfl_xor(om, 32));
        if (om >= 32768.0f) {                             // exponent of om, minus 14
            ex = (int)((__float_as_uint(om) >> 23) & 0xFF) - 127 - 14;
            post = __uint_as_float((uint32_t)(127 - ex) << 23);
        }
    }
    // the format is uniform: one straight-line pass per format
    auto stage = [&](auto BF) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = 8 * d + 2 * q + g;          // 8-byte unit of d = 4u .. 4u+3
                float x0 = o[d][4 * q] * f, x1 = o[d][4 * q + 1] * f;
                float x2 = o[d][4 * q + 2] * f, x3 = o[d][4 * q + 3] * f;
                if constexpr (!decltype(BF)::value) {      // exact: a power of two
                    x0 *= post;
                    x1 *= post;
                    x2 *= post;
                    x3 *= post;
                }
                uint32_t w0, w1;
                if constexpr (decltype(BF)::value) {      // round to nearest even
                    w0 = pack_bf16(x0, x1);
                    w1 = pack_bf16(x2, x3);
                } else {
                    w0 = __builtin_bit_cast(uint32_t, h2{(_Float16)x0, (_Float16)x1});
                    w1 = __builtin_bit_cast(uint32_t, h2{(_Float16)x2, (_Float16)x3});
                }
                *reinterpret_cast<v2i *>(ob + col * (2 * D) + 8 * (u ^ ((2 * col) & (D / 4 - 2)))) =
                    v2i{(int)w0, (int)w1};
            }
    };
    if (to_out) stage(std::true_type{});
    else stage(std::false_type{});
    if (!to_out && g == 0 && q_ok) {
        const int64_t row = ((int64_t)split * a.n_q + qi) * a.n_heads + head;
        // running max (log2 units), denominator, exponent of the stored row;
        // written through to memory like the partial rows (below)
        const f32x4 mlv = {kShift - cofs, ltot, (float)ex, 0.0f};
        rowq::store_wt(a.part_ml + 4 * row, __builtin_bit_cast(rowq::u32x4v, mlv));
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
        // written once, read by another kernel (or the caller).  Output rows:
        // nontemporal.  Split partials: written through to memory, so that
        // the L2s hold no dirty partial lines when the launch ends (their
        // write-back at the end of the launch delays the merge: 0.5-0.7 us a
        // call against nontemporal stores)
        if (to_out) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + 8 * k));
        else rowq::store_wt(dst + 8 * k, __builtin_bit_cast(rowq::u32x4v, v));
    }
}

// Merge the split partials of (query, head) rows in split order: each split
// s holds a normalised row o_s, stored in fp16 as o_s 2^-e_s, with its running
// max m_s (log2 units), denominator l_s and e_s;
// out = sum_s w_s o_s / sum_s w_s, w_s = l_s 2^(m_s - M).
// D/8 lanes per row, eight elements per lane.
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(AttnArgs a) {
    constexpr int LPR = D / 8;                       // lanes per row
    constexpr int RPB = 256 / LPR;                   // rows per workgroup
    const int64_t rows = (int64_t)a.n_q * a.n_heads;
    const int64_t qh = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (qh >= rows) return;
    const int e = 8 * (threadIdx.x % LPR);
    const f32x4 *ml = reinterpret_cast<const f32x4 *>(a.part_ml);
    float l = 0.0f;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    // up to kCombineBatch splits are loaded in one go (max, sum and the row part
    // together), then merged in split order; more splits go batch by batch
    // with the running max carried over
    constexpr int kCombineBatch = 8;
    float m = -INFINITY;
    for (int s0 = 0; s0 < a.n_splits; s0 += kCombineBatch) {
        const int nb = min(kCombineBatch, a.n_splits - s0);
        f32x4 mls[kCombineBatch];
        u32x4 v[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const int64_t row = (int64_t)(s0 + min(i, nb - 1)) * rows + qh;
            mls[i] = ml[row];
            v[i] = *reinterpret_cast<const u32x4 *>(a.part_o + row * D + e);
        }
        float mb = m;
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i)
            if (i < nb) mb = fmaxf(mb, mls[i][0]);
        if (mb > m) {                                  // rescale what is merged so far
            const float r = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mb);
            l *= r;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] *= r;
            m = mb;
        }
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            if (i >= nb) break;
            const float wgt = mls[i][1] > 0.0f ? mls[i][1] * __builtin_amdgcn_exp2f(mls[i][0] - m) : 0.0f;
            l += wgt;
            const float wrow = __builtin_ldexpf(wgt, (int)mls[i][2]);   // the row's 2^e_s (exact)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t word = v[i][k];           // (bit_cast of a vector element
                const h2 x = __builtin_bit_cast(h2, word);   //  reference is not reliable)
                acc[2 * k] += wrow * (float)x[0];
                acc[2 * k + 1] += wrow * (float)x[1];
            }
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = pack_bf16(acc[2 * k] * inv, acc[2 * k + 1] * inv);
    *reinterpret_cast<u32x4 *>(a.out + qh * D + e) = w;
}

// One 16-byte word per thread: word c of lane l of wave w of query block b is
// the (cos, sin) of pairs 32 (c / 8) + 16 (l / 32) + 2 (c % 8) and + 1 of query
// 256 b + 32 w + l % 32 (the last query for the padding of the last block).
__global__ void __launch_bounds__(256) query_lanes_kernel(const float *cs, int n_q, int D, float *lanes,
                                                           int64_t n_words) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_words) return;
    const int lane = (int)(idx % 64);
    const int nc = D / 8;
    const int c = (int)((idx / 64) % nc);
    const int64_t bw = idx / (64 * nc);               // b * 8 + w
    const int q = (int)min<int64_t>(bw * kQW + lane % 32, (int64_t)n_q - 1);
    const int p = 32 * (c / 8) + 16 * (lane / 32) + 2 * (c % 8);
    const f32x4 v = *reinterpret_cast<const f32x4 *>(cs + ((int64_t)q * (D / 2) + p) * 2);
    *reinterpret_cast<f32x4 *>(lanes + idx * 4) = v;
}

}  // namespace

size_t query_lanes_bytes(int n_q, int head_dim) {
    const size_t n_qb = (size_t)(n_q + kQB - 1) / kQB;
    return n_qb * kQB * (size_t)head_dim * 4;          // D/2 (cos, sin) pairs per query, padded block
}

hipError_t launch_query_lanes(const float *cs_rows, int n_q, int head_dim, float *lanes, hipStream_t s) {
    const int64_t n_words = (int64_t)query_lanes_bytes(n_q, head_dim) / 16;
    hipLaunchKernelGGL(query_lanes_kernel, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, s, cs_rows, n_q,
                       head_dim, lanes, n_words);
    return hipGetLastError();
}

int attn_query_blocks(int n_q) { return (n_q + kQB - 1) / kQB; }

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
    return o_bytes + rows * 4 * sizeof(float);
}

template <int D>
static void launch_merge_d(const AttnArgs &a, hipStream_t s) {
    constexpr int RPB = 256 / (D / 8);               // rows per combine workgroup
    const int64_t rows = (int64_t)a.n_q * a.n_heads;
    hipLaunchKernelGGL(combine_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(256), 0, s, a);
}

template <int D, bool BF16>
static void launch_fused_d(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
    if (a.prefix > 0) hipLaunchKernelGGL((attn_kernel<D, BF16, false, true, true>), grid, block, Lds<D>::TOTAL, s, a);
    else hipLaunchKernelGGL((attn_kernel<D, BF16, false, false, true>), grid, block, Lds<D>::TOTAL, s, a);
}

template <int D, bool BF16, bool QTAB>
static void launch_main_d(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
    if (a.prefix > 0) hipLaunchKernelGGL((attn_kernel<D, BF16, QTAB, true>), grid, block, Lds<D>::TOTAL, s, a);
    else hipLaunchKernelGGL((attn_kernel<D, BF16, QTAB, false>), grid, block, Lds<D>::TOTAL, s, a);
}

hipError_t launch_attention_main(const AttnArgs &a, int head_dim, hipStream_t s) {
    const int n_qb = (a.n_q + kQB - 1) / kQB;
    const dim3 grid(n_qb * a.n_heads * a.n_splits), block(kThreads);
    const bool bf16 = a.dtype == KVR_BF16;
    const bool tab = a.q_cs != nullptr;
    if (head_dim == 128) {
        if (tab) bf16 ? launch_main_d<128, true, true>(a, grid, block, s) : launch_main_d<128, false, true>(a, grid, block, s);
        else bf16 ? launch_main_d<128, true, false>(a, grid, block, s) : launch_main_d<128, false, false>(a, grid, block, s);
    } else {
        if (tab) bf16 ? launch_main_d<64, true, true>(a, grid, block, s) : launch_main_d<64, false, true>(a, grid, block, s);
        else bf16 ? launch_main_d<64, true, false>(a, grid, block, s) : launch_main_d<64, false, false>(a, grid, block, s);
    }
    return hipGetLastError();
}

template <int D, bool BF16>
static const void *fused_kernel(bool prefix) {
    return prefix ? reinterpret_cast<const void *>(&attn_kernel<D, BF16, false, true, true>)
                  : reinterpret_cast<const void *>(&attn_kernel<D, BF16, false, false, true>);
}

hipError_t attention_fused_resident(int head_dim, int dtype, bool prefix, int device, int *max_blocks) {
    const bool bf16 = dtype == KVR_BF16;
    const void *k = head_dim == 128 ? (bf16 ? fused_kernel<128, true>(prefix) : fused_kernel<128, false>(prefix))
                                    : (bf16 ? fused_kernel<64, true>(prefix) : fused_kernel<64, false>(prefix));
    const size_t lds = head_dim == 128 ? Lds<128>::TOTAL : Lds<64>::TOTAL;
    int per_cu = 0, cus = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return e;
    *max_blocks = per_cu * cus;
    return hipSuccess;
}

hipError_t launch_attention_fused(const AttnArgs &a, int head_dim, hipStream_t s) {
    const int n_qb = (a.n_q + kQB - 1) / kQB;
    const dim3 grid(n_qb * a.n_heads * a.n_splits), block(kThreads);
    const bool bf16 = a.dtype == KVR_BF16;
    if (head_dim == 128) bf16 ? launch_fused_d<128, true>(a, grid, block, s) : launch_fused_d<128, false>(a, grid, block, s);
    else bf16 ? launch_fused_d<64, true>(a, grid, block, s) : launch_fused_d<64, false>(a, grid, block, s);
    return hipGetLastError();
}

hipError_t launch_attention_merge(const AttnArgs &a, int head_dim, hipStream_t s) {
    if (a.n_splits <= 1) return hipSuccess;
    if (head_dim == 128) launch_merge_d<128>(a, s);
    else launch_merge_d<64>(a, s);
    return hipGetLastError();
}

}  // namespace kvr
