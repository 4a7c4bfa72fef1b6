"""Comparison helpers for the GPU parity tests (imported by tests, not collected).

Bars (per element, against the CPU oracle on the same seeded inputs):
* FP8 codes: identical in at least 99.9% of elements, the rest within one
  E4M3 step (codes compared as sign-magnitude integers, +0 == -0);
* per-row scales: within 1e-6 relative;
* attention outputs: max-abs <= 2e-2 and mean-abs <= 2e-3 against the fp64
  oracle run on the same dequantised cache.
"""
import numpy as np

CODE_MATCH_MIN = 0.999
SCALE_RTOL = 1e-6
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3


def _sm(c):
    c = np.asarray(c, np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def code_stats(gpu, ref):
    a, b = _sm(gpu), _sm(ref)
    d = np.abs(a - b)
    return float((d == 0).mean()) if d.size else 1.0, int(d.max()) if d.size else 0


def assert_codes(gpu, ref, what=""):
    frac, worst = code_stats(gpu, ref)
    assert frac >= CODE_MATCH_MIN and worst <= 1, f"{what}: {frac:.6f} identical, worst step {worst}"
    return frac


def assert_scales(gpu, ref, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r) / np.maximum(np.abs(r), 1e-30)
    err = np.where((g == 0) & (r == 0), 0.0, err)
    assert err.max(initial=0.0) <= SCALE_RTOL, f"{what}: scale rel err {err.max():.3g}"


def assert_attention(gpu_bf16, ref, what=""):
    g = np.asarray(gpu_bf16, np.float64)
    e = np.abs(g - ref)
    mx, mean = float(e.max()), float(e.mean())
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    assert mx <= ATTN_MAX_ABS and mean <= ATTN_MEAN_ABS, f"{what}: max-abs {mx:.4g} mean-abs {mean:.4g}"
    return mx, mean


def logical_rows(arr, start, n_valid, window):
    """Rows of [H][W] or [H][W][D] arrays in logical order (start + i) mod W."""
    idx = (start + np.arange(n_valid)) % window
    return arr[:, idx]
