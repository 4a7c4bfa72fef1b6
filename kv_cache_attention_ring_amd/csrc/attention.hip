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
// with k^_j = e4m3(code) * sk_j and v^_j = e4m3(code) * sv_j (one fp32 scale per
// cached row).  Keys are visited in logical window order (slot_start + j) mod W.
//
// Work decomposition: a workgroup owns one head, a block of 128 queries and a
// contiguous range of 64-key tiles (a "split"); its 4 waves own 32 queries each.
// K and V tiles are staged through LDS (double buffered, one barrier per
// tile).  Both products run on v_mfma_f32_32x32x64_f8f6f4 in transposed form:
//   S^T[key][query] = K . Q^T      (A = K rows from LDS, B = Q held in VGPRs)
//   O^T[d][query]  += V^T . P^T    (A = V^T from LDS,   B = P from S^T regs)
// so the softmax weights leave the first MFMA already in the B-operand layout
// of the second: lane l holds query l%32 and the keys 8q + 4g + r (g = l/32).
// V is transposed into LDS while staging (4x4 byte transposes with v_perm).
//
// Precision: E4M3 has 3 mantissa bits, so Q and P each go in as two E4M3
// terms (hi + lo, lo = e4m3(x - hi)), giving ~8 significant bits and two
// MFMAs per product.  The per-key K scale and the Q block scale fold into one
// fp32 factor per key (a_j); the per-key V scale folds into the weights
// (w_j = sv_j / max sv) before they are split.  Softmax runs in the log2
// domain with a lazily updated running max (rescale only when a score exceeds
// it by more than 2), weights shifted by 2^6 to use the E4M3 range.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvr_internal.h"

namespace kvr {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;       // 4 waves
constexpr int kQB = 128;          // queries per workgroup
constexpr int kQW = 32;           // queries per wave
constexpr int kKT = 64;           // keys per tile
constexpr float kTau = 2.0f;      // lazy-rescale threshold (log2 units)
constexpr float kShift = 6.0f;    // weights are 2^(x - m + 6) <= 2^8
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Lds {
    static constexpr int KSTR = D + 16;          // bytes per K row (pad: conflict-free b128)
    static constexpr int VSTR = kKT + 16;        // bytes per V^T row
    static constexpr int K_BYTES = kKT * KSTR;
    static constexpr int V_BYTES = D * VSTR;
    static constexpr int BUF = K_BYTES + V_BYTES + 2 * kKT * 4;
    static constexpr int TOTAL = 2 * BUF;
};

__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, pk, true);
    return (uint32_t)pk;
}

// hi = e4m3(x), lo = e4m3(x - hi) for four values; returns the two packed words.
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

// 4x4 byte transpose: out[d] byte k = in[k] byte d.
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t &o0, uint32_t &o1, uint32_t &o2,
                                             uint32_t &o3) {
    const uint32_t t01l = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
    const uint32_t t01h = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
    const uint32_t t23l = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    const uint32_t t23h = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    o0 = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
    o1 = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
    o2 = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
    o3 = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

// Column of key k (0..63) inside a V^T row: the 32 keys a lane group g needs
// for one PV MFMA are contiguous, in the byte order of the P operand.
__device__ __forceinline__ int vt_col(int k) {
    const int b = k >> 5, q = (k >> 3) & 3, g = (k >> 2) & 1, r = k & 3;
    return 32 * g + 16 * b + 4 * q + r;
}

// Global -> register staging of one tile (K rows, a 4-key x D/16 V block and
// the per-key factors), then register -> LDS.
template <int D>
struct Stage {
    static constexpr int KB = D / 4;               // K bytes per thread (one quarter row)
    static constexpr int VB = D / 16;              // V bytes per key row per thread
    u32x4 k[KB / 16];
    uint32_t v[4][VB / 4];
    float sa, sw;

    __device__ __forceinline__ void load(const AttnArgs &a, int head, int tile, float qfac,
                                         float inv_cv) {
        const int t = threadIdx.x;
        const int base = tile * kKT;
        // K: thread t -> key t/4, bytes [(t%4) * KB, +KB)
        {
            int idx = base + t / 4;
            idx = idx < a.n_valid ? idx : a.n_valid - 1;
            int slot = a.slot_start + idx;
            slot = slot >= a.window ? slot - a.window : slot;
            const u32x4 *p = reinterpret_cast<const u32x4 *>(
                a.k_codes + ((int64_t)head * a.window + slot) * D + (t % 4) * KB);
#pragma unroll
            for (int i = 0; i < KB / 16; ++i) k[i] = p[i];
        }
        // V: thread t -> keys 4*(t%16) .. +3, d in [(t/16) * VB, +VB)
        {
            const int kg = t % 16, dc = t / 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int idx = base + 4 * kg + r;
                idx = idx < a.n_valid ? idx : a.n_valid - 1;
                int slot = a.slot_start + idx;
                slot = slot >= a.window ? slot - a.window : slot;
                const uint8_t *p = a.v_codes + ((int64_t)head * a.window + slot) * D + dc * VB;
                if constexpr (VB == 8) {
                    const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
                    v[r][0] = u.x;
                    v[r][1] = u.y;
                } else {
                    v[r][0] = *reinterpret_cast<const uint32_t *>(p);
                }
            }
        }
        // per-key factors: a_j = sk_j * qfac, w_j = sv_j / max sv
        if (t < kKT) {
            const int idx = base + t;
            if (idx < a.n_valid) {
                int slot = a.slot_start + idx;
                slot = slot >= a.window ? slot - a.window : slot;
                sa = a.k_scales[(int64_t)head * a.window + slot] * qfac;
                sw = a.v_scales[(int64_t)head * a.window + slot] * inv_cv;
            } else {
                sa = 0.0f;
                sw = 0.0f;
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t *buf) const {
        using L = Lds<D>;
        const int t = threadIdx.x;
        uint8_t *ks = buf;
        uint8_t *vt = buf + L::K_BYTES;
        float *fa = reinterpret_cast<float *>(buf + L::K_BYTES + L::V_BYTES);
        {
            u32x4 *p = reinterpret_cast<u32x4 *>(ks + (t / 4) * L::KSTR + (t % 4) * KB);
#pragma unroll
            for (int i = 0; i < KB / 16; ++i) p[i] = k[i];
        }
        {
            const int kg = t % 16, dc = t / 16;
            const int col = vt_col(4 * kg);
#pragma unroll
            for (int w = 0; w < VB / 4; ++w) {
                uint32_t o0, o1, o2, o3;
                transpose4x4(v[0][w], v[1][w], v[2][w], v[3][w], o0, o1, o2, o3);
                const int d = dc * VB + 4 * w;
                *reinterpret_cast<uint32_t *>(vt + (d + 0) * L::VSTR + col) = o0;
                *reinterpret_cast<uint32_t *>(vt + (d + 1) * L::VSTR + col) = o1;
                *reinterpret_cast<uint32_t *>(vt + (d + 2) * L::VSTR + col) = o2;
                *reinterpret_cast<uint32_t *>(vt + (d + 3) * L::VSTR + col) = o3;
            }
        }
        if (t < kKT) {
            fa[t] = sa;
            fa[kKT + t] = sw;
        }
    }
};

template <int D>
__global__ void __launch_bounds__(kBlock) attn_kernel(AttnArgs a) {
    using L = Lds<D>;
    constexpr int NH = D / 64;          // 64-wide d halves of one QK^T MFMA chain
    constexpr int ND = D / 32;          // 32-row d blocks of O^T
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[8];

    // ---- decode (head, split, query block), keeping a (head, split) key range
    //      on one XCD (workgroups are dealt round-robin over the 8 XCDs) ------
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

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int g = lane / 32, col = lane % 32;
    const int qi = qb * kQB + wave * kQW + col;         // this lane's query
    const bool q_ok = qi < a.n_q;

    // ---- Q: load, rotate (fp32), block absmax -------------------------------
    float qv[NH][32];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int d0 = 64 * h + 32 * g;
        if (q_ok) {
            const int64_t off = ((int64_t)qi * a.n_heads + head) * D + d0;
            if (a.dtype == KVR_BF16) {
                const uint4 *p = reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const uint16_t *>(a.q) + off);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 u = p[v];
                    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qv[h][8 * v + 2 * e] = __uint_as_float(w[e] << 16);
                        qv[h][8 * v + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                    }
                }
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(
                    reinterpret_cast<const float *>(a.q) + off);
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float4 f = p[v];
                    qv[h][4 * v] = f.x;
                    qv[h][4 * v + 1] = f.y;
                    qv[h][4 * v + 2] = f.z;
                    qv[h][4 * v + 3] = f.w;
                }
            }
            const float4 *cs = reinterpret_cast<const float4 *>(a.cs + (int64_t)qi * D + d0);
#pragma unroll
            for (int v = 0; v < 8; ++v) {           // two pairs per float4 (c0, s0, c1, s1)
                const float4 c = cs[v];
                const float x0 = qv[h][4 * v], x1 = qv[h][4 * v + 1];
                const float x2 = qv[h][4 * v + 2], x3 = qv[h][4 * v + 3];
                qv[h][4 * v] = x0 * c.x - x1 * c.y;
                qv[h][4 * v + 1] = x0 * c.y + x1 * c.x;
                qv[h][4 * v + 2] = x2 * c.z - x3 * c.w;
                qv[h][4 * v + 3] = x2 * c.w + x3 * c.z;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) qv[h][e] = 0.0f;
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(qv[h][e]));
    am = wave_max(am);

    // ---- max V scale over this split's keys (folds sv_j into the weights) ---
    float cvm = 0.0f;
    {
        const int k0 = t0 * kKT, k1 = min(a.n_valid, t1 * kKT);
        for (int idx = k0 + tid; idx < k1; idx += kBlock) {
            int slot = a.slot_start + idx;
            slot = slot >= a.window ? slot - a.window : slot;
            cvm = fmaxf(cvm, a.v_scales[(int64_t)head * a.window + slot]);
        }
        cvm = wave_max(cvm);
    }
    if (lane == 0) {
        red[wave] = am;
        red[4 + wave] = cvm;
    }
    __syncthreads();
    const float qmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float cv = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
    const float qscale = qmax > 0.0f ? 448.0f / qmax : 1.0f;
    const float qfac = (qmax > 0.0f ? qmax / 448.0f : 1.0f) * a.softmax_scale * kLog2e;
    const float inv_cv = cv > 0.0f ? 1.0f / cv : 0.0f;

    // ---- Q -> hi/lo E4M3 B operands ------------------------------------------
    v8i qhi[NH], qlo[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            uint32_t hi, lo;
            split4(qv[h][4 * w] * qscale, qv[h][4 * w + 1] * qscale, qv[h][4 * w + 2] * qscale,
                   qv[h][4 * w + 3] * qscale, hi, lo);
            qhi[h][w] = (int)hi;
            qlo[h][w] = (int)lo;
        }
    }

    // ---- main loop over key tiles ----------------------------------------------
    v16f o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = v16f{};
    float lsum = 0.0f;      // this lane's share of the softmax denominator
    float cofs = 0.0f;      // 6 - running max (log2 units); weights are 2^(x + cofs)
    bool started = false;

    Stage<D> st;
    if (t0 < t1) {
        st.load(a, head, t0, qfac, inv_cv);
        st.store(smem);
    }
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
        uint8_t *buf = smem + ((t - t0) & 1) * L::BUF;
        const bool more = t + 1 < t1;
        if (more) st.load(a, head, t + 1, qfac, inv_cv);

        const uint8_t *ks = buf;
        const uint8_t *vt = buf + L::K_BYTES;
        const float *fa = reinterpret_cast<const float *>(buf + L::K_BYTES + L::V_BYTES);

        // S^T = K . Q^T, two 32-key blocks
        v16f s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = v16f{};
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(
                    ks + (32 * kb + col) * L::KSTR + 64 * h + 32 * g);
                const u32x4 u0 = p[0], u1 = p[1];
                v8i ka;
                ka[0] = u0.x; ka[1] = u0.y; ka[2] = u0.z; ka[3] = u0.w;
                ka[4] = u1.x; ka[5] = u1.y; ka[6] = u1.z; ka[7] = u1.w;
                s[kb] = mfma(ka, qhi[h], s[kb]);
                s[kb] = mfma(ka, qlo[h], s[kb]);
            }
        }

        // scores in log2 units shifted by cofs; S^T register r of block kb is
        // key 32kb + 8(r/4) + 4g + r%4 of the tile
        float x[2][16];
        float mx = -INFINITY;
        const bool partial = (t + 1) * kKT > a.n_valid;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 f = *reinterpret_cast<const float4 *>(fa + 32 * kb + 8 * q + 4 * g);
                const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = s[kb][4 * q + r] * fv[r] + cofs;
                    if (partial && t * kKT + 32 * kb + 8 * q + 4 * g + r >= a.n_valid) v = -INFINITY;
                    x[kb][4 * q + r] = v;
                    mx = fmaxf(mx, v);
                }
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = !started || mx > kShift + kTau;
        if (__any(need)) {
            float shift = 0.0f;                  // new cofs = cofs - shift
            if (!started) {
                shift = mx - kShift;
            } else if (mx > kShift + kTau) {
                shift = mx - kShift;
                const float alpha = __builtin_amdgcn_exp2f(-shift);
                lsum *= alpha;
#pragma unroll
                for (int d = 0; d < ND; ++d) o[d] *= alpha;
            }
            cofs -= shift;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) x[kb][r] -= shift;
            started = true;
        }

        // weights p = 2^x, denominator, V-scale fold, hi/lo split -> B operands
        v8i phi, plo;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 f = *reinterpret_cast<const float4 *>(fa + kKT + 32 * kb + 8 * q + 4 * g);
                const float fv[4] = {f.x, f.y, f.z, f.w};
                float pw[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(x[kb][4 * q + r]);
                    lsum += p;
                    pw[r] = p * fv[r];
                }
                uint32_t hi, lo;
                split4(pw[0], pw[1], pw[2], pw[3], hi, lo);
                phi[4 * kb + q] = (int)hi;
                plo[4 * kb + q] = (int)lo;
            }
        }

        // O^T += V^T . P^T
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(vt + (32 * d + col) * L::VSTR + 32 * g);
            const u32x4 u0 = p[0], u1 = p[1];
            v8i va;
            va[0] = u0.x; va[1] = u0.y; va[2] = u0.z; va[3] = u0.w;
            va[4] = u1.x; va[5] = u1.y; va[6] = u1.z; va[7] = u1.w;
            o[d] = mfma(va, phi, o[d]);
            o[d] = mfma(va, plo, o[d]);
        }

        if (more) st.store(smem + ((t + 1 - t0) & 1) * L::BUF);
        __syncthreads();
    }

    // ---- epilogue ------------------------------------------------------------
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!q_ok) return;
    if (a.n_splits == 1) {
        const float f = ltot > 0.0f ? cv / ltot : 0.0f;
        uint16_t *dst = a.out + ((int64_t)qi * a.n_heads + head) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dd = 32 * d + 8 * q + 4 * g;
                const uint32_t w0 = f32_to_bf16_rne(o[d][4 * q] * f) |
                                    ((uint32_t)f32_to_bf16_rne(o[d][4 * q + 1] * f) << 16);
                const uint32_t w1 = f32_to_bf16_rne(o[d][4 * q + 2] * f) |
                                    ((uint32_t)f32_to_bf16_rne(o[d][4 * q + 3] * f) << 16);
                *reinterpret_cast<uint2 *>(dst + dd) = make_uint2(w0, w1);
            }
        }
    } else {
        const int64_t row = ((int64_t)split * a.n_q + qi) * a.n_heads + head;
        float *dst = a.part_o + row * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dd = 32 * d + 8 * q + 4 * g;
                *reinterpret_cast<float4 *>(dst + dd) =
                    make_float4(o[d][4 * q] * cv, o[d][4 * q + 1] * cv, o[d][4 * q + 2] * cv,
                                o[d][4 * q + 3] * cv);
            }
        }
        if (g == 0) {
            // running max in log2 units is kShift - cofs
            a.part_ml[2 * row] = started ? kShift - cofs : -INFINITY;
            a.part_ml[2 * row + 1] = ltot;
        }
    }
}

// Combine the split partials of one (query, head) in split order.
template <int D>
__global__ void __launch_bounds__(64) combine_kernel(AttnArgs a) {
    const int qh = blockIdx.x;                   // query * n_heads + head
    const int e = threadIdx.x * (D / 64);        // first element of this thread
    const int64_t stride = (int64_t)a.n_q * a.n_heads;
    float m = -INFINITY;
    for (int s = 0; s < a.n_splits; ++s) m = fmaxf(m, a.part_ml[2 * (s * stride + qh)]);
    float l = 0.0f;
    float acc[D / 64];
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] = 0.0f;
    for (int s = 0; s < a.n_splits; ++s) {
        const int64_t row = s * stride + qh;
        const float ms = a.part_ml[2 * row];
        const float wgt = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - m);
        l += wgt * a.part_ml[2 * row + 1];
        const float *src = a.part_o + row * D + e;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) acc[i] += wgt * src[i];
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t *dst = a.out + (int64_t)qh * D + e;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) dst[i] = f32_to_bf16_rne(acc[i] * inv);
}

}  // namespace

int attn_default_splits(int n_heads, int n_q, int n_valid) {
    const int n_qb = (n_q + kQB - 1) / kQB;
    const int tiles = (n_valid + kKT - 1) / kKT;
    const int units = n_heads * n_qb;
    int s = (2 * 256 + units / 2) / units;       // about two workgroups per CU
    if (s < 1) s = 1;
    if (s > tiles) s = tiles;
    return s;
}

size_t attn_workspace_bytes(int n_heads, int head_dim, int n_q, int n_splits) {
    if (n_splits <= 1) return 0;
    const size_t rows = (size_t)n_splits * n_q * n_heads;
    return rows * head_dim * sizeof(float) + rows * 2 * sizeof(float);
}

hipError_t launch_attention(const AttnArgs &a, int head_dim, hipStream_t s) {
    const int n_qb = (a.n_q + kQB - 1) / kQB;
    const int grid = n_qb * a.n_heads * a.n_splits;
    if (head_dim == 128) {
        hipLaunchKernelGGL(attn_kernel<128>, dim3(grid), dim3(kBlock), Lds<128>::TOTAL, s, a);
        if (a.n_splits > 1)
            hipLaunchKernelGGL(combine_kernel<128>, dim3(a.n_q * a.n_heads), dim3(64), 0, s, a);
    } else {
        hipLaunchKernelGGL(attn_kernel<64>, dim3(grid), dim3(kBlock), Lds<64>::TOTAL, s, a);
        if (a.n_splits > 1)
            hipLaunchKernelGGL(combine_kernel<64>, dim3(a.n_q * a.n_heads), dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kvr
