/*
 * sanitize_driver.c -- exercises every function of the CPU oracle on small
 * shapes (a window that wraps mid-chunk, a position reset, the 3-D form, a
 * fixed prefix) so that a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer can check the oracle's memory accesses and arithmetic.  Test
 * infrastructure, like the oracle itself: built and run by the CPU tests only.
 * Exit status 0 when every call returned and a few results are finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e4m3_decode(uint8_t code);
uint8_t orc_e4m3_encode(float v);
void orc_write(uint8_t *, uint8_t *, float *, float *, int, int, int, int64_t, int64_t,
               const float *, const float *, int, double);
void orc_rebase(uint8_t *, float *, int, int, int, int32_t, int32_t, int64_t, double);
void orc_naive(const float *, const float *, const float *, const float *, int, int32_t, int64_t,
               int, int, int, double, float *, float *, uint8_t *, uint8_t *, float *, float *);
void orc_attention_rows(const uint8_t *, const uint8_t *, const float *, const float *, int, int, int,
                        int32_t, int32_t, const float *, int, int64_t, double, double,
                        const int32_t *, int, double *);
void orc_write3d(uint8_t *, uint8_t *, float *, float *, int, int, int, int64_t, const int64_t *,
                 const int32_t *, const float *, const float *, int, double);
void orc_rebase3d(uint8_t *, float *, int, int, int, int32_t, int32_t, const int64_t *, const int32_t *,
                  double);
void orc_attention_rows3d(const uint8_t *, const uint8_t *, const float *, const float *, int, int, int,
                          int32_t, int32_t, const float *, const int64_t *, const int32_t *, double,
                          double, const int32_t *, int, double *);
void orc_write3d_list(uint8_t *, uint8_t *, float *, float *, int, int, int, const int32_t *,
                      const int64_t *, const int32_t *, const float *, const float *, int, double);
void orc_rebase3d_list(uint8_t *, float *, int, int, int, const int32_t *, int32_t, const int64_t *,
                       const int32_t *, double);
void orc_attention_list3d(const uint8_t *, const uint8_t *, const float *, const float *, int, int, int,
                          const int32_t *, int32_t, const float *, const int64_t *, const int32_t *,
                          double, double, const int32_t *, int, double *);

static float frand(unsigned *s)
{
    *s = *s * 1664525u + 1013904223u;
    return ((float)(*s >> 8) / 16777216.0f) * 4.0f - 2.0f;
}

int main(void)
{
    enum { H = 2, D = 64, W = 100, N = 16, P = 12 };
    unsigned seed = 12345u;
    size_t cw = (size_t)H * W * D, sw = (size_t)H * W;
    uint8_t *kc = calloc(cw, 1), *vc = calloc(cw, 1), *lkc = calloc(cw, 1), *lvc = calloc(cw, 1);
    float *ks = calloc(sw, 4), *vs = calloc(sw, 4), *lks = calloc(sw, 4), *lvs = calloc(sw, 4);
    float *lin[4];
    for (int i = 0; i < 4; ++i) lin[i] = calloc(cw, 4);
    float *kn = malloc(sizeof(float) * N * H * D), *vn = malloc(sizeof(float) * N * H * D);
    float *q = malloc(sizeof(float) * N * H * D);
    double *out = malloc(sizeof(double) * N * H * D);
    int32_t qh[2 * N * H];
    for (int i = 0; i < N; ++i)
        for (int h = 0; h < H; ++h) { qh[2 * (i * H + h)] = i; qh[2 * (i * H + h) + 1] = h; }
    int ok = 1;
    for (int c = 0; c < 256; ++c) {                       /* every code round-trips or is NaN */
        double v = orc_e4m3_decode((uint8_t)c);
        if (!isnan(v) && orc_e4m3_decode(orc_e4m3_encode((float)v)) != v) ok = 0;
    }
    int64_t total = 0, pos = 0;
    int32_t n_valid = 0, ping = 0;
    for (int step = 0; step < 9; ++step) {              /* 144 tokens: wraps at 100 mid-chunk */
        for (int e = 0; e < N * H * D; ++e) { kn[e] = frand(&seed); vn[e] = frand(&seed); q[e] = frand(&seed); }
        orc_naive(lin[2 * ping], lin[2 * ping + 1], kn, vn, N, n_valid, pos, H, D, W, 10000.0,
                  lin[2 - 2 * ping], lin[3 - 2 * ping], lkc, lvc, lks, lvs);
        ping = 1 - ping;
        orc_write(kc, vc, ks, vs, H, D, W, total, pos, kn, vn, N, 10000.0);
        total += N;
        pos += N;
        n_valid = n_valid + N < W ? n_valid + N : W;
        int32_t start = (int32_t)((total - n_valid) % W);
        orc_attention_rows(kc, vc, ks, vs, H, D, W, start, n_valid, q, N, pos - N, 10000.0, 0.125, qh,
                           N * H, out);
        if (step == 4) { orc_rebase(kc, ks, H, D, W, start, n_valid, 64, 10000.0); pos -= 64; }
    }
    for (int e = 0; e < N * H * D; ++e) ok &= isfinite(out[e]);
    /* the 3-D form over explicit slot lists: a prefix of P slots and a ring of W - P */
    int32_t npairs[3] = {12, 10, 10};
    int64_t coords[3 * N], delta[3] = {3, 0, 0};
    int32_t slots[N], keys[W];
    memset(kc, 0, cw);
    memset(ks, 0, sw * 4);
    for (int j = 0; j < P; ++j) { slots[j] = j; coords[3 * j] = -1; coords[3 * j + 1] = j / 5; coords[3 * j + 2] = j % 5; }
    orc_write3d_list(kc, vc, ks, vs, H, D, W, slots, coords, npairs, kn, vn, P, 10000.0);
    int64_t t_tok = 0;
    for (int step = 0; step < 8; ++step) {
        for (int j = 0; j < N; ++j) {
            slots[j] = P + (int32_t)((t_tok + j) % (W - P));
            coords[3 * j] = step; coords[3 * j + 1] = j / 5; coords[3 * j + 2] = j % 5;
        }
        orc_write3d_list(kc, vc, ks, vs, H, D, W, slots, coords, npairs, kn, vn, N, 10000.0);
        t_tok += N;
    }
    int32_t n_ring = (int32_t)(t_tok < W - P ? t_tok : W - P), nk = 0;
    for (int j = 0; j < P; ++j) keys[nk++] = j;
    for (int32_t i = 0; i < n_ring; ++i) keys[nk++] = P + (int32_t)((t_tok - n_ring + i) % (W - P));
    orc_attention_list3d(kc, vc, ks, vs, H, D, W, keys, nk, q, coords, npairs, 10000.0, 0.125, qh, N * H, out);
    orc_rebase3d_list(kc, ks, H, D, W, keys + P, n_ring, delta, npairs, 10000.0);
    orc_write3d(kc, vc, ks, vs, H, D, W, 0, coords, npairs, kn, vn, N, 10000.0);
    orc_rebase3d(kc, ks, H, D, W, 0, N, delta, npairs, 10000.0);
    orc_attention_rows3d(kc, vc, ks, vs, H, D, W, 0, N, q, coords, npairs, 10000.0, 0.125, qh, N * H, out);
    for (int e = 0; e < N * H * D; ++e) ok &= isfinite(out[e]);
    for (int i = 0; i < 4; ++i) free(lin[i]);
    free(kc); free(vc); free(lkc); free(lvc); free(ks); free(vs); free(lks); free(lvs);
    free(kn); free(vn); free(q); free(out);
    printf("oracle sanitize driver: %s\n", ok ? "ok" : "FAILED");
    return ok ? 0 : 1;
}
