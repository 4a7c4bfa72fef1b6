"""Precision emulation of FP8 window-attention schemes.

TEST INFRASTRUCTURE, and not the parity reference: the GPU parity tests
compare the HIP path with the exact oracle (``oracle.attention``, fp64 over
the dequantised cache).  The functions here model where a GPU kernel would
round on the way -- the query as one or two E4M3 terms, the softmax weights
in bf16, as one E4M3 term or as two, V as bf16 rows or as its E4M3 codes --
so that the error each choice adds can be measured on the CPU before a kernel
is built around it.  The FP8 attention of the pages accepts per-head scales
(ai.info, "Characters funziona in tempo reale su quattro H100, afferma
Runway", section "Latenza dei turni e altre configurazioni GPU"); the cache
it reads holds rows rotated and quantised once, at write time (same page,
section "La gestione della cache spostata al momento della scrittura").  The
pages say nothing about the precision of Q or of the weights inside the
kernel; these emulations are how that choice is made.

Scheme of a call (per head; every step below is one rounding point):
  1. q is rotated in fp32 (the oracle's rule), multiplied by
     c2 = softmax_scale * log2(e) and by a per-query power of two 2^-k (k the
     smallest with 448 * 2^k >= max|c2 q|), then
       "hilo":   q8 = e4m3(x) + e4m3(x - e4m3(x))   (two FP8 products)
       "single": q8 = e4m3(x)                        (one FP8 product)
       "exact":  q8 = x                              (no rounding)
  2. scores s = 2^k (q8 . code_j) sk_j in log2 units (products of E4M3
     values are exact; the accumulation is modelled in fp64);
  3. weights p_j = 2^(s_j - max s) (fp32);
  4. the weighted sum of V rows v_j = e4m3(code_j) sv_j:
       "bf16":   sum bf16(p_j) bf16(v_j) / sum bf16(p_j)
       "fp8":    the weights times sv_j, one power of two per (query,
                 32-key block) bringing the block's largest to 448, one
                 E4M3 term: sum e4m3(p_j sv_j) code_j / sum p_j
       "fp8x2":  as "fp8" with two E4M3 terms (hi + lo) of p_j sv_j
  5. the output row rounded to bf16.
``SCHEMES`` names the combinations the tests measure.
"""
from __future__ import annotations

import numpy as np

from . import dequant_rows, e4m3_decode, e4m3_encode, rope_rows

LOG2E = 1.4426950408889634

#: name -> (Q rounding, weights/V rounding)
SCHEMES = {
    "gpu_hilo_q_bf16_pv": ("hilo", "bf16"),   # the kernel as built
    "exact_q_bf16_pv": ("exact", "bf16"),     # only the bf16 weights and V
    "single_q_bf16_pv": ("single", "bf16"),   # half the QK^T matrix work
    "hilo_q_fp8_pv": ("hilo", "fp8"),         # P.V on FP8 codes, one weight term
    "single_q_fp8_pv": ("single", "fp8"),     # both products in plain FP8
    "hilo_q_fp8x2_pv": ("hilo", "fp8x2"),     # P.V on FP8 codes, two weight terms
}


def bf16_round(x) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), as fp32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def e4m3_round(x) -> np.ndarray:
    """fp32 values rounded to E4M3 (ties to even, saturating at 448), as fp64."""
    return e4m3_decode(e4m3_encode(np.asarray(x, np.float32)))


def pow2_exponent(a) -> np.ndarray:
    """Smallest integer k with 448 * 2^k >= a (a > 0), elementwise."""
    a = np.asarray(a, np.float64)
    k = np.ceil(np.log2(np.maximum(a, 1e-300) / 448.0))
    # guard the log2 rounding at exact powers of two
    k = np.where(448.0 * 2.0 ** (k - 1) >= a, k - 1, k)
    k = np.where(448.0 * 2.0 ** k < a, k + 1, k)
    return k


def quantize_queries(q_rot, sm_scale: float, mode: str) -> np.ndarray:
    """Step 1: the rotated queries [n][D] (fp32) as the scaled values the
    score product sees, in log2 units: 2^k * (the E4M3 terms)."""
    c2 = np.float32(sm_scale * LOG2E)
    x = np.asarray(q_rot, np.float32) * c2                      # fp32
    if mode == "exact":
        return x.astype(np.float64)
    k = pow2_exponent(np.abs(x).max(axis=1))[:, None]
    xs = (x.astype(np.float64) * 2.0 ** -k).astype(np.float32)  # exact: a power of two
    hi = e4m3_round(xs)
    if mode == "single":
        t = hi
    elif mode == "hilo":
        t = hi + e4m3_round((xs.astype(np.float64) - hi).astype(np.float32))
    else:
        raise ValueError(mode)
    return t * 2.0 ** k


def weighted_sum(p, codes_v, sv, mode: str) -> np.ndarray:
    """Step 4 for one head: p [n_q][n] fp32 weights, codes_v [n][D] E4M3 codes,
    sv [n] row scales -> normalised rows [n_q][D] (fp64)."""
    v_hat = e4m3_decode(codes_v)                                 # exact code values
    if mode == "bf16":
        pb = bf16_round(p).astype(np.float64)
        vb = bf16_round((v_hat.astype(np.float32) * sv[:, None].astype(np.float32))).astype(np.float64)
        return (pb @ vb) / pb.sum(axis=1, keepdims=True)
    if mode not in ("fp8", "fp8x2"):
        raise ValueError(mode)
    w = p.astype(np.float64) * sv[None, :].astype(np.float64)   # fold the V row scale
    n = w.shape[1]
    w8 = np.empty_like(w)
    for b0 in range(0, n, 32):                                   # one scale per (query, 32-key block)
        blk = w[:, b0:b0 + 32]
        bm = blk.max(axis=1, keepdims=True)
        k = np.where(bm > 0, pow2_exponent(np.where(bm > 0, bm, 1.0)), 0.0)
        xs = (blk * 2.0 ** -k).astype(np.float32)
        hi = e4m3_round(xs)
        t = hi if mode == "fp8" else hi + e4m3_round((xs.astype(np.float64) - hi).astype(np.float32))
        w8[:, b0:b0 + 32] = t * 2.0 ** k
    return (w8 @ v_hat) / p.astype(np.float64).sum(axis=1, keepdims=True)


def attention_emulated(cache, start: int, n_valid: int, q, q_pos: int, scheme: str,
                       sm_scale: float | None = None, base: float = 10000.0, heads=None) -> np.ndarray:
    """One call over an oracle.LayerCache with the rounding points of `scheme`
    (a key of SCHEMES): q [n_q][H][D] fp32 values (not rotated), queries at
    positions q_pos + i, keys at slots (start + j) mod W, j < n_valid.
    Returns [n_q][len(heads)][D] fp64 (bf16-rounded output rows)."""
    qmode, pmode = SCHEMES[scheme]
    q = np.asarray(q, np.float32)
    n_q, H, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    idx = (start + np.arange(n_valid)) % cache.W
    out = np.empty((n_q, len(heads), D), np.float64)
    pos = q_pos + np.arange(n_q)
    for hi_, h in enumerate(heads):
        q_rot = rope_rows(q[:, h], pos, base)                                   # fp32 [n_q][D]
        q8 = quantize_queries(q_rot, sm_scale, qmode)                           # log2 units
        kc = e4m3_decode(cache.k_codes[h, idx])                                  # exact codes [n][D]
        sk = cache.k_scales[h, idx].astype(np.float64)
        s = (q8 @ kc.T) * sk[None, :]                                            # log2 units
        p = np.exp2(s - s.max(axis=1, keepdims=True)).astype(np.float32)
        o = weighted_sum(p, cache.v_codes[h, idx], cache.v_scales[h, idx], pmode)
        out[:, hi_] = bf16_round(o.astype(np.float32)).astype(np.float64)
    return out


def attention_exact(cache, start: int, n_valid: int, q, q_pos: int, sm_scale: float | None = None,
                    base: float = 10000.0, heads=None) -> np.ndarray:
    """The oracle's definition (fp64 softmax over the dequantised cache, q
    rotated in fp32), dense per head, for the same heads: the reference the
    emulations are measured against."""
    q = np.asarray(q, np.float32)
    n_q, H, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    idx = (start + np.arange(n_valid)) % cache.W
    pos = q_pos + np.arange(n_q)
    out = np.empty((n_q, len(heads), D), np.float64)
    for hi_, h in enumerate(heads):
        q_rot = rope_rows(q[:, h], pos, base).astype(np.float64)
        k_hat = dequant_rows(cache.k_codes[h, idx], cache.k_scales[h, idx]).astype(np.float64)
        v_hat = dequant_rows(cache.v_codes[h, idx], cache.v_scales[h, idx]).astype(np.float64)
        s = (q_rot @ k_hat.T) * sm_scale
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, hi_] = (p @ v_hat) / p.sum(axis=1, keepdims=True)
    return out
