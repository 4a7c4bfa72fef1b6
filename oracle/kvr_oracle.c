/*
 * kvr_oracle.c -- CPU ORACLE for the write-time RoPE + FP8 ring KV cache,
 * the delta rebase, the naive per-call upkeep and FP8-cache window attention.
 *
 * This file is TEST INFRASTRUCTURE.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant generator with the HIP library: every step below is the
 * plain definition, written out, in the order the method states it, with no
 * blocking, fusion or reordering.  Build flags: -O2 -ffp-contract=off
 * -fno-fast-math (each fp32 operation rounds on its own, no FMA contraction).
 *
 * Page references (web pages on the method; cited by title and section):
 *   [AI-cache]   ai.info, "Characters funziona in tempo reale su quattro H100,
 *                afferma Runway", section "La gestione della cache spostata al
 *                momento della scrittura".
 *   [AI-latency] same page, section "Latenza dei turni e altre configurazioni GPU".
 *   [NC-cache]   neurocartel.com, "Runway Characters ... 4 H100" blog post,
 *                section "Кэш: 240 attention calls и работа на запись".
 *   [WC]         wechild.cn news item 1943 (commentary on the Runway real-time
 *                characters paper), paragraphs on the cache upkeep.
 * External specification:
 *   [OFP8]       OCP 8-bit Floating Point Specification (OFP8), rev. 1.0,
 *                format E4M3 (bias 7, no infinities, S.1111.111 = NaN).
 *
 * Readings where the pages are silent (all recorded in the design notes):
 *   - FP8 is OCP E4M3 with one fp32 scale per (token, head) row; the scale is
 *     the row absmax / 448 and codes are RNE(y * (448 / absmax)), saturating.
 *   - RoPE is the 1-D rotary encoding on interleaved pairs (x[2i], x[2i+1]),
 *     theta_i = base^(-2i/D), angle = p * theta_i formed in fp64, cos/sin in
 *     fp64 and rounded to fp32, rotation in fp32 without FMA.
 *   - K is rotated at write time, Q at attention time, V never.
 *   - A position reset by Delta rotates every stored K row by -Delta.
 *
 * Parity status: every function here is pinned by the CPU tests (spec values,
 * brute force, closed forms, group identities, library routines); see the
 * header of each function for its pin.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E4M3_MAX 448.0

/* ------------------------------------------------------------------------ */
/* OCP E4M3 (FN) encode / decode                                    [OFP8]  */
/* Pins: spec code values, exhaustive round trip over all finite codes,    */
/* brute-force nearest-value search with ties to the even mantissa.        */
/* ------------------------------------------------------------------------ */

/* Value of one E4M3 code (exact in double).  S.EEEE.MMM, bias 7.
 * E == 0: subnormal m * 2^-9; otherwise (1 + m/8) * 2^(E-7); S.1111.111 is NaN. */
double orc_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Round-to-nearest-even into E4M3, saturating at +-448 (no infinities in
 * this format), sign of zero kept.  NaN maps to 0x7F. */
uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return 0x7F;
    double a = fabs((double)v);
    if (a > ORC_E4M3_MAX) a = ORC_E4M3_MAX;
    if (a < 0x1p-6) {
        /* subnormal binade: spacing 2^-9; m == 8 is the smallest normal 0x08 */
        double m = nearbyint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e;
    double f = frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                      /* a = (2f) * 2^E, 2f in [1, 2) */
    double mant = nearbyint((2.0 * f - 1.0) * 8.0);   /* 3 mantissa bits, RNE */
    if (mant == 8.0) { mant = 0.0; E += 1; }
    int code = ((E + 7) << 3) | (int)mant;
    if (code > 0x7E) code = 0x7E;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* Row quantisation (per token, per head)            [AI-cache] [NC-cache]  */
/* Pins: absmax element encodes to +-448 exactly; dequantisation error is  */
/* within half an E4M3 ulp; zero rows give scale 0 and zero codes; rows    */
/* whose absmax is far below 1 (down to the smallest fp32 denormal) keep   */
/* those properties and decode to finite values.                           */
/*                                                                          */
/* The code of element d is the E4M3 rounding of y_d * (448 / a).  The     */
/* fp32 inverse 448 / a overflows once a < 448 / FLT_MAX (about 1.3e-36),  */
/* so for a < 2^-64 both a and the row are first multiplied by 2^64, which */
/* is exact; the product y_d 2^64 * fl(448 / (a 2^64)) is then the same    */
/* real number as y_d * fl(448 / a) wherever that inverse is finite, so    */
/* every such row keeps its bits, and the rows where it is not get the     */
/* codes the definition asks for instead of NaN.                            */
/* ------------------------------------------------------------------------ */
#define ORC_TINY_ROW 0x1p-64f
#define ORC_TINY_LIFT 0x1p64f

void orc_quant_row(const float *y, int D, uint8_t *codes, float *scale)
{
    float a = 0.0f;
    for (int d = 0; d < D; ++d) {
        float t = fabsf(y[d]);
        if (t > a) a = t;
    }
    if (a == 0.0f) {
        *scale = 0.0f;
        memset(codes, 0, (size_t)D);
        return;
    }
    *scale = a / 448.0f;
    float lift = a < ORC_TINY_ROW ? ORC_TINY_LIFT : 1.0f;
    float inv = 448.0f / (a * lift);
    for (int d = 0; d < D; ++d) {
        float t = (y[d] * lift) * inv;
        codes[d] = orc_e4m3_encode(t);
    }
}

void orc_dequant_row(const uint8_t *codes, float scale, int D, float *x)
{
    for (int d = 0; d < D; ++d) x[d] = (float)orc_e4m3_decode(codes[d]) * scale;
}

/* ------------------------------------------------------------------------ */
/* Rotary position encoding, interleaved pairs                  [AI-cache]  */
/* Pins: agreement with the interleaved ("rotate every two") rotary        */
/* implementation of a third-party library; R(-D) R(p) == R(p - D); p = 0  */
/* is the identity; pair norms kept; q.k depends only on position offsets. */
/* ------------------------------------------------------------------------ */
void orc_rope_cs(int64_t pos, int i, int D, double base, float *c, float *s)
{
    double theta = pow(base, -2.0 * (double)i / (double)D);
    double ang = (double)pos * theta;
    *c = (float)cos(ang);
    *s = (float)sin(ang);
}

/* y = R(pos) x on each pair (x[2i], x[2i+1]); y may alias x. */
void orc_rope_row(const float *x, float *y, int D, int64_t pos, double base)
{
    for (int i = 0; i < D / 2; ++i) {
        float c, s;
        orc_rope_cs(pos, i, D, base, &c, &s);
        float x0 = x[2 * i], x1 = x[2 * i + 1];
        float a = x0 * c;
        float b = x1 * s;
        float e = x0 * s;
        float f = x1 * c;
        y[2 * i] = a - b;
        y[2 * i + 1] = e + f;
    }
}

/* ------------------------------------------------------------------------ */
/* Circular-buffer cache: slot of the t-th token ever written is t mod W.   */
/* (no copies as the window advances)                           [AI-cache]  */
/* Pin: brute-force deque simulation of the last W tokens.                 */
/* ------------------------------------------------------------------------ */
int32_t orc_slot_of_token(int64_t t, int32_t W)
{
    int64_t r = t % W;
    return (int32_t)(r < 0 ? r + W : r);
}

/* ------------------------------------------------------------------------ */
/* Write-time upkeep for one layer                  [AI-cache] [NC-cache] [WC]
 * New chunk token j (0 <= j < N) was the (total_before + j)-th token ever
 * written; it lands in slot (total_before + j) mod W with position
 * pos_before + j.  K rows are rotated at that position and quantised, V rows
 * are quantised.  Cache layout: codes [H][W][D], scales [H][W].
 * New rows: k_new / v_new [N][H][D] (fp32 values).
 * Pin: identical codes and scales to the naive per-call path.              */
/* ------------------------------------------------------------------------ */
void orc_write(uint8_t *k_codes, uint8_t *v_codes, float *k_scales, float *v_scales,
               int H, int D, int W, int64_t total_before, int64_t pos_before,
               const float *k_new, const float *v_new, int N, double base)
{
#pragma omp parallel
    {
        float *y = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
        for (int j = 0; j < N; ++j) {
            for (int h = 0; h < H; ++h) {
                int32_t slot = orc_slot_of_token(total_before + j, W);
                int64_t pos = pos_before + j;
                const float *kr = k_new + ((size_t)j * H + h) * D;
                const float *vr = v_new + ((size_t)j * H + h) * D;
                size_t row = (size_t)h * W + slot;
                orc_rope_row(kr, y, D, pos, base);
                orc_quant_row(y, D, k_codes + row * D, &k_scales[row]);
                orc_quant_row(vr, D, v_codes + row * D, &v_scales[row]);
            }
        }
        free(y);
    }
}

/* ------------------------------------------------------------------------ */
/* Delta rebase of the stored window on a position reset         [AI-cache] */
/* Every valid K row (logical index 0..n_valid-1 at slot (start+i) mod W) is
 * dequantised, rotated by -delta (so a key stored at position p now encodes
 * p - delta) and re-quantised with a fresh absmax scale.  V is untouched.
 * Pin: R(-D)R(p) == R(p-D); rebase(+D) then rebase(-D) returns the row
 * within quantisation error; attention is unchanged when queries move too. */
/* ------------------------------------------------------------------------ */
void orc_rebase(uint8_t *k_codes, float *k_scales, int H, int D, int W,
                int32_t start, int32_t n_valid, int64_t delta, double base)
{
#pragma omp parallel
    {
        float *x = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
        for (int h = 0; h < H; ++h) {
            for (int i = 0; i < n_valid; ++i) {
                int32_t slot = orc_slot_of_token((int64_t)start + i, W);
                size_t row = (size_t)h * W + slot;
                orc_dequant_row(k_codes + row * D, k_scales[row], D, x);
                orc_rope_row(x, x, D, -delta, base);
                orc_quant_row(x, D, k_codes + row * D, &k_scales[row]);
            }
        }
        free(x);
    }
}

/* ------------------------------------------------------------------------ */
/* Naive per-call upkeep (the original implementation)      [WC] [AI-cache] */
/* On every call: shift the linear, un-rotated window (drop the oldest
 * max(0, n_valid + N - W) rows, append the N new rows), then rotate every K
 * row at its absolute position and quantise every K and V row into a linear
 * FP8 window.  Linear windows: [H][W][D]; new rows [N][H][D].
 * Row i of the new window holds position pos_before + N - n_after + i.
 * Pin: identical codes and scales to the write-time ring path.            */
/* ------------------------------------------------------------------------ */
void orc_naive(const float *lin_k_src, const float *lin_v_src,
               const float *k_new, const float *v_new, int N,
               int32_t n_valid_before, int64_t pos_before,
               int H, int D, int W, double base,
               float *lin_k_dst, float *lin_v_dst,
               uint8_t *k_codes, uint8_t *v_codes, float *k_scales, float *v_scales)
{
    int32_t n_after = n_valid_before + N < W ? n_valid_before + N : W;
    int32_t drop = n_valid_before + N - n_after;
    int32_t kept = n_valid_before - drop;
    int64_t pos_first = pos_before + N - n_after;
#pragma omp parallel
    {
    float *y = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
    for (int h = 0; h < H; ++h) {
        for (int i = 0; i < n_after; ++i) {
            const float *ks, *vs;
            if (i < kept) {
                ks = lin_k_src + ((size_t)h * W + (i + drop)) * D;
                vs = lin_v_src + ((size_t)h * W + (i + drop)) * D;
            } else {
                int j = i - kept;
                ks = k_new + ((size_t)j * H + h) * D;
                vs = v_new + ((size_t)j * H + h) * D;
            }
            size_t row = (size_t)h * W + i;
            memcpy(lin_k_dst + row * D, ks, sizeof(float) * (size_t)D);
            memcpy(lin_v_dst + row * D, vs, sizeof(float) * (size_t)D);
            orc_rope_row(ks, y, D, pos_first + i, base);
            orc_quant_row(y, D, k_codes + row * D, &k_scales[row]);
            orc_quant_row(vs, D, v_codes + row * D, &v_scales[row]);
        }
    }
    free(y);
    }
}

/* ------------------------------------------------------------------------ */
/* Window attention over the dequantised cache     [AI-cache] [AI-latency]  */
/* For head h and query i (rotated in fp32 at position q_pos + i):
 *   O = sum_j softmax_j(sm_scale * q . k^_j) v^_j
 * over the n_valid keys at slots (start + j) mod W, j < n_valid, with
 * k^ = dec(code) * scale and v^ likewise (fp32 products), everything after
 * that in fp64, softmax in two passes (max, then normalised exponentials).
 * Only the (query, head) pairs listed in qh (pairs of int32) are computed;
 * out is [n_list][D] fp64.
 * Pins: a dense fp64 softmax(QK^T)V on the same dequantised cache, a
 * library softmax, and closed-form special cases (one key, zero query,
 * equal keys, weights summing to one).                                    */
/* ------------------------------------------------------------------------ */
void orc_attention_rows(const uint8_t *k_codes, const uint8_t *v_codes,
                        const float *k_scales, const float *v_scales,
                        int H, int D, int W, int32_t start, int32_t n_valid,
                        const float *q, int n_q, int64_t q_pos, double base,
                        double sm_scale, const int32_t *qh, int n_list, double *out)
{
    (void)n_q;
#pragma omp parallel
    {
        float *qr = (float *)malloc(sizeof(float) * (size_t)D);
        float *kh = (float *)malloc(sizeof(float) * (size_t)D);
        double *sc = (double *)malloc(sizeof(double) * (size_t)(n_valid > 0 ? n_valid : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_list; ++t) {
            int i = qh[2 * t], h = qh[2 * t + 1];
            double *o = out + (size_t)t * D;
            orc_rope_row(q + ((size_t)i * H + h) * D, qr, D, q_pos + i, base);
            double m = -INFINITY;
            for (int j = 0; j < n_valid; ++j) {
                size_t row = (size_t)h * W + orc_slot_of_token((int64_t)start + j, W);
                orc_dequant_row(k_codes + row * D, k_scales[row], D, kh);
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += (double)qr[d] * (double)kh[d];
                s *= sm_scale;
                sc[j] = s;
                if (s > m) m = s;
            }
            double l = 0.0;
            for (int j = 0; j < n_valid; ++j) {
                sc[j] = exp(sc[j] - m);
                l += sc[j];
            }
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int j = 0; j < n_valid; ++j) {
                size_t row = (size_t)h * W + orc_slot_of_token((int64_t)start + j, W);
                double w = sc[j] / l;
                const uint8_t *vc = v_codes + row * D;
                float vsc = v_scales[row];
                for (int d = 0; d < D; ++d) {
                    float vh = (float)orc_e4m3_decode(vc[d]) * vsc;
                    o[d] += w * (double)vh;
                }
            }
        }
        free(qr);
        free(kh);
        free(sc);
    }
}

/* ------------------------------------------------------------------------ */
/* 3-D (t, y, x) rotary encoding for video tokens                           */
/* The pages describe the model as a video diffusion transformer and say no */
/* more about its rotary encoding.  Reading taken: the D/2 interleaved pairs */
/* are cut into three contiguous groups of n_t, n_y, n_x pairs, one per axis */
/* (frame index, row, column of the token); group a is the 1-D rotary rule  */
/* of a 2 n_a-dimensional vector at that axis's coordinate, i.e. its pair k  */
/* has theta = base^(-k / n_a).  A position reset moves the frame index     */
/* only, so the rebase rotates each group by its own axis delta (temporal   */
/* only: (delta, 0, 0)).                                                    */
/* Pins: split (D/2, 0, 0) is the 1-D encoding bit for bit; every group is  */
/* the 1-D encoding of its slice at its coordinate; groups of axes with a   */
/* zero coordinate are left bit-identical; R(-d) R(c) = R(c - d) per axis;  */
/* q.k depends only on coordinate offsets, axis by axis.                    */
/* ------------------------------------------------------------------------ */
void orc_rope3d_cs(const int64_t coord[3], int i, const int32_t npairs[3], double base,
                   float *c, float *s)
{
    int a = 0, k = i;
    while (a < 2 && k >= npairs[a]) { k -= npairs[a]; ++a; }
    double theta = pow(base, -(double)k / (double)npairs[a]);
    double ang = (double)coord[a] * theta;
    *c = (float)cos(ang);
    *s = (float)sin(ang);
}

/* y = R(coord) x on each pair (x[2i], x[2i+1]); y may alias x. */
void orc_rope3d_row(const float *x, float *y, int D, const int64_t coord[3],
                    const int32_t npairs[3], double base)
{
    for (int i = 0; i < D / 2; ++i) {
        float c, s;
        orc_rope3d_cs(coord, i, npairs, base, &c, &s);
        float x0 = x[2 * i], x1 = x[2 * i + 1];
        float a = x0 * c;
        float b = x1 * s;
        float e = x0 * s;
        float f = x1 * c;
        y[2 * i] = a - b;
        y[2 * i + 1] = e + f;
    }
}

/* Write-time upkeep with 3-D coordinates: as orc_write, with new token j
 * rotated at coords[j] (int64 triples) instead of a 1-D position. */
void orc_write3d(uint8_t *k_codes, uint8_t *v_codes, float *k_scales, float *v_scales,
                 int H, int D, int W, int64_t total_before, const int64_t *coords,
                 const int32_t npairs[3], const float *k_new, const float *v_new, int N,
                 double base)
{
#pragma omp parallel
    {
        float *y = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
        for (int j = 0; j < N; ++j) {
            for (int h = 0; h < H; ++h) {
                int32_t slot = orc_slot_of_token(total_before + j, W);
                const float *kr = k_new + ((size_t)j * H + h) * D;
                const float *vr = v_new + ((size_t)j * H + h) * D;
                size_t row = (size_t)h * W + slot;
                orc_rope3d_row(kr, y, D, coords + 3 * (size_t)j, npairs, base);
                orc_quant_row(y, D, k_codes + row * D, &k_scales[row]);
                orc_quant_row(vr, D, v_codes + row * D, &v_scales[row]);
            }
        }
        free(y);
    }
}

/* Rebase with a delta per axis: every valid K row dequantised, rotated by
 * R(-delta) (delta a triple; a reset of the frame index is (d, 0, 0)),
 * re-quantised.  V untouched. */
void orc_rebase3d(uint8_t *k_codes, float *k_scales, int H, int D, int W,
                  int32_t start, int32_t n_valid, const int64_t delta[3],
                  const int32_t npairs[3], double base)
{
    const int64_t neg[3] = {-delta[0], -delta[1], -delta[2]};
#pragma omp parallel
    {
        float *x = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
        for (int h = 0; h < H; ++h) {
            for (int i = 0; i < n_valid; ++i) {
                int32_t slot = orc_slot_of_token((int64_t)start + i, W);
                size_t row = (size_t)h * W + slot;
                orc_dequant_row(k_codes + row * D, k_scales[row], D, x);
                orc_rope3d_row(x, x, D, neg, npairs, base);
                orc_quant_row(x, D, k_codes + row * D, &k_scales[row]);
            }
        }
        free(x);
    }
}

/* Window attention with queries rotated at 3-D coordinates q_coords[i]
 * (int64 triples); otherwise exactly orc_attention_rows. */
void orc_attention_rows3d(const uint8_t *k_codes, const uint8_t *v_codes,
                          const float *k_scales, const float *v_scales,
                          int H, int D, int W, int32_t start, int32_t n_valid,
                          const float *q, const int64_t *q_coords, const int32_t npairs[3],
                          double base, double sm_scale, const int32_t *qh, int n_list,
                          double *out)
{
#pragma omp parallel
    {
        float *qr = (float *)malloc(sizeof(float) * (size_t)D);
        float *kh = (float *)malloc(sizeof(float) * (size_t)D);
        double *sc = (double *)malloc(sizeof(double) * (size_t)(n_valid > 0 ? n_valid : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_list; ++t) {
            int i = qh[2 * t], h = qh[2 * t + 1];
            double *o = out + (size_t)t * D;
            orc_rope3d_row(q + ((size_t)i * H + h) * D, qr, D, q_coords + 3 * (size_t)i, npairs, base);
            double m = -INFINITY;
            for (int j = 0; j < n_valid; ++j) {
                size_t row = (size_t)h * W + orc_slot_of_token((int64_t)start + j, W);
                orc_dequant_row(k_codes + row * D, k_scales[row], D, kh);
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += (double)qr[d] * (double)kh[d];
                s *= sm_scale;
                sc[j] = s;
                if (s > m) m = s;
            }
            double l = 0.0;
            for (int j = 0; j < n_valid; ++j) {
                sc[j] = exp(sc[j] - m);
                l += sc[j];
            }
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int j = 0; j < n_valid; ++j) {
                size_t row = (size_t)h * W + orc_slot_of_token((int64_t)start + j, W);
                double w = sc[j] / l;
                const uint8_t *vc = v_codes + row * D;
                float vsc = v_scales[row];
                for (int d = 0; d < D; ++d) {
                    float vh = (float)orc_e4m3_decode(vc[d]) * vsc;
                    o[d] += w * (double)vh;
                }
            }
        }
        free(qr);
        free(kh);
        free(sc);
    }
}

/* ------------------------------------------------------------------------ */
/* The same three steps over explicit slot lists: a cache whose first slots  */
/* hold a fixed prefix (written once, never overwritten) and whose other     */
/* slots form the ring.  Reading where the pages are silent: the prefix keeps */
/* its own coordinates, so a frame reset rotates the ring's rows only.       */
/* Pins: with the ring's slots in logical order these are orc_write3d,       */
/* orc_rebase3d and orc_attention_rows3d bit for bit; attention does not     */
/* depend on the order of the key list (keys are a set).                     */
/* ------------------------------------------------------------------------ */
/* new token j goes to slots[j] */
void orc_write3d_list(uint8_t *k_codes, uint8_t *v_codes, float *k_scales, float *v_scales,
                      int H, int D, int W, const int32_t *slots, const int64_t *coords,
                      const int32_t npairs[3], const float *k_new, const float *v_new, int N,
                      double base)
{
    (void)W;
#pragma omp parallel
    {
        float *y = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
        for (int j = 0; j < N; ++j) {
            for (int h = 0; h < H; ++h) {
                const float *kr = k_new + ((size_t)j * H + h) * D;
                const float *vr = v_new + ((size_t)j * H + h) * D;
                size_t row = (size_t)h * W + slots[j];
                orc_rope3d_row(kr, y, D, coords + 3 * (size_t)j, npairs, base);
                orc_quant_row(y, D, k_codes + row * D, &k_scales[row]);
                orc_quant_row(vr, D, v_codes + row * D, &v_scales[row]);
            }
        }
        free(y);
    }
}

/* the K rows at slots[0 .. n-1] rotated by R(-delta) and re-quantised */
void orc_rebase3d_list(uint8_t *k_codes, float *k_scales, int H, int D, int W,
                       const int32_t *slots, int32_t n, const int64_t delta[3],
                       const int32_t npairs[3], double base)
{
    const int64_t neg[3] = {-delta[0], -delta[1], -delta[2]};
#pragma omp parallel
    {
        float *x = (float *)malloc(sizeof(float) * (size_t)D);
#pragma omp for collapse(2) schedule(static)
        for (int h = 0; h < H; ++h) {
            for (int i = 0; i < n; ++i) {
                size_t row = (size_t)h * W + slots[i];
                orc_dequant_row(k_codes + row * D, k_scales[row], D, x);
                orc_rope3d_row(x, x, D, neg, npairs, base);
                orc_quant_row(x, D, k_codes + row * D, &k_scales[row]);
            }
        }
        free(x);
    }
}

/* attention of the listed (query, head) pairs over the keys at slots[0 .. n_keys-1] */
void orc_attention_list3d(const uint8_t *k_codes, const uint8_t *v_codes,
                          const float *k_scales, const float *v_scales,
                          int H, int D, int W, const int32_t *slots, int32_t n_keys,
                          const float *q, const int64_t *q_coords, const int32_t npairs[3],
                          double base, double sm_scale, const int32_t *qh, int n_list,
                          double *out)
{
#pragma omp parallel
    {
        float *qr = (float *)malloc(sizeof(float) * (size_t)D);
        float *kh = (float *)malloc(sizeof(float) * (size_t)D);
        double *sc = (double *)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_list; ++t) {
            int i = qh[2 * t], h = qh[2 * t + 1];
            double *o = out + (size_t)t * D;
            orc_rope3d_row(q + ((size_t)i * H + h) * D, qr, D, q_coords + 3 * (size_t)i, npairs, base);
            double m = -INFINITY;
            for (int j = 0; j < n_keys; ++j) {
                size_t row = (size_t)h * W + slots[j];
                orc_dequant_row(k_codes + row * D, k_scales[row], D, kh);
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += (double)qr[d] * (double)kh[d];
                s *= sm_scale;
                sc[j] = s;
                if (s > m) m = s;
            }
            double l = 0.0;
            for (int j = 0; j < n_keys; ++j) {
                sc[j] = exp(sc[j] - m);
                l += sc[j];
            }
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int j = 0; j < n_keys; ++j) {
                size_t row = (size_t)h * W + slots[j];
                double w = sc[j] / l;
                const uint8_t *vc = v_codes + row * D;
                float vsc = v_scales[row];
                for (int d = 0; d < D; ++d) {
                    float vh = (float)orc_e4m3_decode(vc[d]) * vsc;
                    o[d] += w * (double)vh;
                }
            }
        }
        free(qr);
        free(kh);
        free(sc);
    }
}

/* rows x [n][D] rotated at 3-D coordinates coords[n][3] into y [n][D] */
void orc_rope3d_rows(const float *x, float *y, int64_t n, int D, const int64_t *coords,
                     const int32_t npairs[3], double base)
{
    for (int64_t r = 0; r < n; ++r)
        orc_rope3d_row(x + r * D, y + r * D, D, coords + 3 * r, npairs, base);
}

void orc_rope3d_cs_n(const int64_t *coords, int64_t n, int D, const int32_t npairs[3],
                     double base, float *cs)
{
    for (int64_t r = 0; r < n; ++r)
        for (int i = 0; i < D / 2; ++i)
            orc_rope3d_cs(coords + 3 * r, i, npairs, base, &cs[(r * (D / 2) + i) * 2],
                          &cs[(r * (D / 2) + i) * 2 + 1]);
}

/* ------------------------------------------------------------------------ */
/* Thread count of the OpenMP loops above (the CPU-baseline timing runs the */
/* oracle on all host cores and on one).                                    */
/* ------------------------------------------------------------------------ */
void orc_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

int orc_max_threads(void)
{
    return omp_get_max_threads();
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the test harness (loops over the scalar definitions). */
/* ------------------------------------------------------------------------ */
void orc_e4m3_encode_n(const float *v, uint8_t *codes, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) codes[i] = orc_e4m3_encode(v[i]);
}

void orc_e4m3_decode_n(const uint8_t *codes, double *v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) v[i] = orc_e4m3_decode(codes[i]);
}

/* rows x [n][D] rotated at positions pos[n] into y [n][D] */
void orc_rope_rows(const float *x, float *y, int64_t n, int D, const int64_t *pos, double base)
{
    for (int64_t r = 0; r < n; ++r) orc_rope_row(x + r * D, y + r * D, D, pos[r], base);
}

void orc_rope_cs_n(const int64_t *pos, int64_t n, int D, double base, float *cs)
{
    for (int64_t r = 0; r < n; ++r)
        for (int i = 0; i < D / 2; ++i)
            orc_rope_cs(pos[r], i, D, base, &cs[(r * (D / 2) + i) * 2], &cs[(r * (D / 2) + i) * 2 + 1]);
}

void orc_quant_rows(const float *y, int64_t n, int D, uint8_t *codes, float *scales)
{
    for (int64_t r = 0; r < n; ++r) orc_quant_row(y + r * D, D, codes + r * D, &scales[r]);
}

void orc_dequant_rows(const uint8_t *codes, const float *scales, int64_t n, int D, float *x)
{
    for (int64_t r = 0; r < n; ++r) orc_dequant_row(codes + r * D, scales[r], D, x + r * D);
}
