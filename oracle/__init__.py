"""CPU oracle for the write-time RoPE + FP8 ring KV cache path.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the library and its Python
binding never do.  Nothing here is shared with the HIP path: the C part
(``kvr_oracle.c``) is a plain definition of every step, built with gcc
(-O2 -ffp-contract=off, OpenMP), and this module adds

* ctypes wrappers around the C functions,
* ``dense_attention`` -- an fp64 NumPy softmax(Q K^T * scale) V, the dense
  definition the C attention is checked against on small inputs,
* ``RingDeque`` -- a brute-force model of a window of the last W tokens, the
  definition the ring bookkeeping is checked against.

Page references (cited by title and section):
  [AI-cache]  ai.info, "Characters funziona in tempo reale su quattro H100,
              afferma Runway", section "La gestione della cache spostata al
              momento della scrittura" (circular buffer, RoPE and FP8 once at
              write time, one delta rotation on every position reset).
  [WC]        wechild.cn news item 1943, paragraphs on the original per-call
              upkeep (re-rotate, re-quantise, shift the window on every call).
"""
from __future__ import annotations

import collections
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvr_oracle.so")
_lib = None

_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_c_i32p = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile the C oracle into oracle/libkvr_oracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_n.argtypes = [_c_f32p, _c_u8p, ctypes.c_int64]
        L.orc_e4m3_decode_n.argtypes = [_c_u8p, _c_f64p, ctypes.c_int64]
        L.orc_rope_rows.argtypes = [_c_f32p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_i64p,
                                    ctypes.c_double]
        L.orc_rope_cs_n.argtypes = [_c_i64p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, _c_f32p]
        L.orc_quant_rows.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p, _c_f32p]
        L.orc_dequant_rows.argtypes = [_c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_f32p]
        L.orc_slot_of_token.restype = ctypes.c_int32
        L.orc_slot_of_token.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.orc_write.argtypes = [_c_u8p, _c_u8p, _c_f32p, _c_f32p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _c_f32p, _c_f32p,
                                ctypes.c_int, ctypes.c_double]
        L.orc_rebase.argtypes = [_c_u8p, _c_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_double]
        L.orc_naive.argtypes = [_c_f32p, _c_f32p, _c_f32p, _c_f32p, ctypes.c_int, ctypes.c_int32,
                                ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_double, _c_f32p, _c_f32p, _c_u8p, _c_u8p, _c_f32p, _c_f32p]
        L.orc_attention_rows.argtypes = [_c_u8p, _c_u8p, _c_f32p, _c_f32p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                         _c_f32p, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                                         ctypes.c_double, _c_i32p, ctypes.c_int, _c_f64p]
        L.orc_rope3d_rows.argtypes = [_c_f32p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_i64p,
                                      _c_i32p, ctypes.c_double]
        L.orc_rope3d_cs_n.argtypes = [_c_i64p, ctypes.c_int64, ctypes.c_int, _c_i32p, ctypes.c_double,
                                      _c_f32p]
        L.orc_write3d.argtypes = [_c_u8p, _c_u8p, _c_f32p, _c_f32p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int64, _c_i64p, _c_i32p, _c_f32p, _c_f32p,
                                  ctypes.c_int, ctypes.c_double]
        L.orc_rebase3d.argtypes = [_c_u8p, _c_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int32, ctypes.c_int32, _c_i64p, _c_i32p, ctypes.c_double]
        L.orc_attention_rows3d.argtypes = [_c_u8p, _c_u8p, _c_f32p, _c_f32p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                           _c_f32p, _c_i64p, _c_i32p, ctypes.c_double,
                                           ctypes.c_double, _c_i32p, ctypes.c_int, _c_f64p]
        L.orc_write3d_list.argtypes = [_c_u8p, _c_u8p, _c_f32p, _c_f32p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, _c_i32p, _c_i64p, _c_i32p, _c_f32p, _c_f32p,
                                       ctypes.c_int, ctypes.c_double]
        L.orc_rebase3d_list.argtypes = [_c_u8p, _c_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        _c_i32p, ctypes.c_int32, _c_i64p, _c_i32p, ctypes.c_double]
        L.orc_attention_list3d.argtypes = [_c_u8p, _c_u8p, _c_f32p, _c_f32p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, _c_i32p, ctypes.c_int32,
                                           _c_f32p, _c_i64p, _c_i32p, ctypes.c_double,
                                           ctypes.c_double, _c_i32p, ctypes.c_int, _c_f64p]
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (for the CPU-baseline timing)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def _p(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ct)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# E4M3 and rows
# --------------------------------------------------------------------------
def e4m3_encode(v) -> np.ndarray:
    v = _f32(v)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_n(_p(v, _c_f32p), _p(out, _c_u8p), v.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_n(_p(c, _c_u8p), _p(out, _c_f64p), c.size)
    return out


def rope_rows(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate rows x[..., D] at integer positions pos (broadcast to x.shape[:-1])."""
    x = _f32(x)
    D = x.shape[-1]
    n = x.size // D
    p = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, np.int64), x.shape[:-1]).reshape(-1))
    y = np.empty_like(x)
    lib().orc_rope_rows(_p(x, _c_f32p), _p(y, _c_f32p), n, D, _p(p, _c_i64p), float(base))
    return y


def rope_cs(pos, D: int, base: float = 10000.0) -> np.ndarray:
    """fp32 (cos, sin) of pos * theta_i: array [n_pos][D/2][2]."""
    p = np.ascontiguousarray(np.asarray(pos, np.int64).reshape(-1))
    out = np.empty((p.size, D // 2, 2), np.float32)
    lib().orc_rope_cs_n(_p(p, _c_i64p), p.size, D, float(base), _p(out, _c_f32p))
    return out


def quant_rows(y):
    y = _f32(y)
    D = y.shape[-1]
    n = y.size // D
    codes = np.empty(y.shape, np.uint8)
    scales = np.empty(y.shape[:-1], np.float32)
    lib().orc_quant_rows(_p(y, _c_f32p), n, D, _p(codes, _c_u8p), _p(scales, _c_f32p))
    return codes, scales


def dequant_rows(codes, scales) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = _f32(scales)
    D = c.shape[-1]
    x = np.empty(c.shape, np.float32)
    lib().orc_dequant_rows(_p(c, _c_u8p), _p(s, _c_f32p), c.size // D, D, _p(x, _c_f32p))
    return x


def slot_of_token(t: int, W: int) -> int:
    return int(lib().orc_slot_of_token(int(t), int(W)))


# --------------------------------------------------------------------------
# One layer's cache
# --------------------------------------------------------------------------
class LayerCache:
    """Codes [H][W][D] u8 and scales [H][W] f32 for K and V of one layer."""

    def __init__(self, H: int, D: int, W: int):
        self.H, self.D, self.W = H, D, W
        self.k_codes = np.zeros((H, W, D), np.uint8)
        self.v_codes = np.zeros((H, W, D), np.uint8)
        self.k_scales = np.zeros((H, W), np.float32)
        self.v_scales = np.zeros((H, W), np.float32)

    def copy(self) -> "LayerCache":
        c = LayerCache(self.H, self.D, self.W)
        for n in ("k_codes", "v_codes", "k_scales", "v_scales"):
            setattr(c, n, getattr(self, n).copy())
        return c


def write(cache: LayerCache, total_before: int, pos_before: int, k_new, v_new,
          base: float = 10000.0) -> None:
    """Write-time upkeep of one chunk into one layer [AI-cache]."""
    k = _f32(k_new)
    v = _f32(v_new)
    N = k.shape[0]
    assert k.shape == (N, cache.H, cache.D) and v.shape == k.shape
    lib().orc_write(_p(cache.k_codes, _c_u8p), _p(cache.v_codes, _c_u8p),
                    _p(cache.k_scales, _c_f32p), _p(cache.v_scales, _c_f32p),
                    cache.H, cache.D, cache.W, int(total_before), int(pos_before),
                    _p(k, _c_f32p), _p(v, _c_f32p), N, float(base))


def rebase(cache: LayerCache, start: int, n_valid: int, delta: int, base: float = 10000.0) -> None:
    """Rotate every valid K row by -delta and re-quantise [AI-cache]."""
    lib().orc_rebase(_p(cache.k_codes, _c_u8p), _p(cache.k_scales, _c_f32p),
                     cache.H, cache.D, cache.W, int(start), int(n_valid), int(delta), float(base))


def naive(lin_k_src, lin_v_src, k_new, v_new, n_valid_before: int, pos_before: int,
          base: float = 10000.0):
    """Naive per-call upkeep [WC]: returns (lin_k_dst, lin_v_dst, LayerCache linear)."""
    ks = _f32(lin_k_src)
    vs = _f32(lin_v_src)
    kn = _f32(k_new)
    vn = _f32(v_new)
    H, W, D = ks.shape
    N = kn.shape[0]
    kd = np.zeros_like(ks)
    vd = np.zeros_like(vs)
    lin = LayerCache(H, D, W)
    lib().orc_naive(_p(ks, _c_f32p), _p(vs, _c_f32p), _p(kn, _c_f32p), _p(vn, _c_f32p), N,
                    int(n_valid_before), int(pos_before), H, D, W, float(base),
                    _p(kd, _c_f32p), _p(vd, _c_f32p), _p(lin.k_codes, _c_u8p),
                    _p(lin.v_codes, _c_u8p), _p(lin.k_scales, _c_f32p), _p(lin.v_scales, _c_f32p))
    return kd, vd, lin


def attention(cache: LayerCache, start: int, n_valid: int, q, q_pos: int,
              sm_scale: float | None = None, base: float = 10000.0, rows=None) -> np.ndarray:
    """fp64 window attention over the dequantised cache.

    q: [n_q][H][D] (fp32 values, not yet rotated).  Returns [n_q][H][D] fp64, or
    [len(rows)][D] when rows (a list of (query, head) pairs) is given.
    """
    qq = _f32(q)
    n_q, H, D = qq.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    if rows is None:
        qh = np.array([(i, h) for i in range(n_q) for h in range(H)], np.int32).reshape(-1, 2)
    else:
        qh = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    out = np.zeros((qh.shape[0], D), np.float64)
    lib().orc_attention_rows(_p(cache.k_codes, _c_u8p), _p(cache.v_codes, _c_u8p),
                             _p(cache.k_scales, _c_f32p), _p(cache.v_scales, _c_f32p),
                             H, D, cache.W, int(start), int(n_valid), _p(qq, _c_f32p), n_q,
                             int(q_pos), float(base), float(sm_scale), _p(qh, _c_i32p),
                             qh.shape[0], _p(out, _c_f64p))
    if rows is None:
        return out.reshape(n_q, H, D)
    return out


# --------------------------------------------------------------------------
# 3-D (t, y, x) rotary encoding: pairs cut into per-axis groups
# --------------------------------------------------------------------------
def _npairs(npairs) -> np.ndarray:
    n = np.ascontiguousarray(np.asarray(npairs, np.int32).reshape(3))
    assert (n >= 0).all() and n[0] >= 1, "the temporal group needs at least one pair"
    return n


def _coords(coords, n: int) -> np.ndarray:
    c = np.ascontiguousarray(np.broadcast_to(np.asarray(coords, np.int64), (n, 3)))
    return c


def rope3d_rows(x, coords, npairs, base: float = 10000.0) -> np.ndarray:
    """Rotate rows x[..., D] at (t, y, x) coordinates coords[..., 3]."""
    x = _f32(x)
    D = x.shape[-1]
    n = x.size // D
    npr = _npairs(npairs)
    assert int(npr.sum()) == D // 2
    c = _coords(np.asarray(coords, np.int64).reshape(-1, 3) if np.ndim(coords) > 1 else coords, n)
    y = np.empty_like(x)
    lib().orc_rope3d_rows(_p(x, _c_f32p), _p(y, _c_f32p), n, D, _p(c, _c_i64p), _p(npr, _c_i32p),
                          float(base))
    return y


def rope3d_cs(coords, D: int, npairs, base: float = 10000.0) -> np.ndarray:
    """fp32 (cos, sin) per token and pair: array [n_tok][D/2][2]."""
    c = np.ascontiguousarray(np.asarray(coords, np.int64).reshape(-1, 3))
    npr = _npairs(npairs)
    assert int(npr.sum()) == D // 2
    out = np.empty((c.shape[0], D // 2, 2), np.float32)
    lib().orc_rope3d_cs_n(_p(c, _c_i64p), c.shape[0], D, _p(npr, _c_i32p), float(base),
                          _p(out, _c_f32p))
    return out


def write3d(cache: LayerCache, total_before: int, coords, npairs, k_new, v_new,
            base: float = 10000.0) -> None:
    """Write-time upkeep of one chunk whose tokens carry (t, y, x) coordinates."""
    k = _f32(k_new)
    v = _f32(v_new)
    N = k.shape[0]
    assert k.shape == (N, cache.H, cache.D) and v.shape == k.shape
    c = np.ascontiguousarray(np.asarray(coords, np.int64).reshape(N, 3))
    npr = _npairs(npairs)
    lib().orc_write3d(_p(cache.k_codes, _c_u8p), _p(cache.v_codes, _c_u8p),
                      _p(cache.k_scales, _c_f32p), _p(cache.v_scales, _c_f32p),
                      cache.H, cache.D, cache.W, int(total_before), _p(c, _c_i64p),
                      _p(npr, _c_i32p), _p(k, _c_f32p), _p(v, _c_f32p), N, float(base))


def rebase3d(cache: LayerCache, start: int, n_valid: int, delta, npairs,
             base: float = 10000.0) -> None:
    """Rotate every valid K row by -delta (a (t, y, x) triple) and re-quantise."""
    d = np.ascontiguousarray(np.asarray(delta, np.int64).reshape(3))
    npr = _npairs(npairs)
    lib().orc_rebase3d(_p(cache.k_codes, _c_u8p), _p(cache.k_scales, _c_f32p),
                       cache.H, cache.D, cache.W, int(start), int(n_valid), _p(d, _c_i64p),
                       _p(npr, _c_i32p), float(base))


def attention3d(cache: LayerCache, start: int, n_valid: int, q, q_coords, npairs,
                sm_scale: float | None = None, base: float = 10000.0, rows=None) -> np.ndarray:
    """As attention(), with query i rotated at q_coords[i] = (t, y, x)."""
    qq = _f32(q)
    n_q, H, D = qq.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    if rows is None:
        qh = np.array([(i, h) for i in range(n_q) for h in range(H)], np.int32).reshape(-1, 2)
    else:
        qh = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    c = np.ascontiguousarray(np.asarray(q_coords, np.int64).reshape(n_q, 3))
    npr = _npairs(npairs)
    out = np.zeros((qh.shape[0], D), np.float64)
    lib().orc_attention_rows3d(_p(cache.k_codes, _c_u8p), _p(cache.v_codes, _c_u8p),
                               _p(cache.k_scales, _c_f32p), _p(cache.v_scales, _c_f32p),
                               H, D, cache.W, int(start), int(n_valid), _p(qq, _c_f32p),
                               _p(c, _c_i64p), _p(npr, _c_i32p), float(base), float(sm_scale),
                               _p(qh, _c_i32p), qh.shape[0], _p(out, _c_f64p))
    if rows is None:
        return out.reshape(n_q, H, D)
    return out


# --------------------------------------------------------------------------
# explicit slot lists (a fixed prefix beside the ring)
# --------------------------------------------------------------------------
def _slots(slots) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(slots, np.int32).reshape(-1))


def write3d_list(cache: LayerCache, slots, coords, npairs, k_new, v_new, base: float = 10000.0) -> None:
    """Token j of the chunk (coordinates coords[j]) into slot slots[j]."""
    k = _f32(k_new)
    v = _f32(v_new)
    N = k.shape[0]
    sl = _slots(slots)
    assert sl.size == N and k.shape == (N, cache.H, cache.D) and v.shape == k.shape
    assert sl.min() >= 0 and sl.max() < cache.W
    c = np.ascontiguousarray(np.asarray(coords, np.int64).reshape(N, 3))
    lib().orc_write3d_list(_p(cache.k_codes, _c_u8p), _p(cache.v_codes, _c_u8p),
                           _p(cache.k_scales, _c_f32p), _p(cache.v_scales, _c_f32p),
                           cache.H, cache.D, cache.W, _p(sl, _c_i32p), _p(c, _c_i64p),
                           _p(_npairs(npairs), _c_i32p), _p(k, _c_f32p), _p(v, _c_f32p), N, float(base))


def rebase3d_list(cache: LayerCache, slots, delta, npairs, base: float = 10000.0) -> None:
    """The K rows at the listed slots rotated by -delta (a (t, y, x) triple), re-quantised."""
    sl = _slots(slots)
    assert sl.size == 0 or (sl.min() >= 0 and sl.max() < cache.W)
    d = np.ascontiguousarray(np.asarray(delta, np.int64).reshape(3))
    lib().orc_rebase3d_list(_p(cache.k_codes, _c_u8p), _p(cache.k_scales, _c_f32p), cache.H, cache.D,
                            cache.W, _p(sl, _c_i32p), sl.size, _p(d, _c_i64p), _p(_npairs(npairs), _c_i32p),
                            float(base))


def attention3d_list(cache: LayerCache, slots, q, q_coords, npairs, sm_scale: float | None = None,
                     base: float = 10000.0, rows=None) -> np.ndarray:
    """fp64 attention over the keys at the listed slots, query i rotated at q_coords[i]."""
    qq = _f32(q)
    n_q, H, D = qq.shape
    sl = _slots(slots)
    assert sl.size >= 1 and sl.min() >= 0 and sl.max() < cache.W
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    if rows is None:
        qh = np.array([(i, h) for i in range(n_q) for h in range(H)], np.int32).reshape(-1, 2)
    else:
        qh = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    c = np.ascontiguousarray(np.asarray(q_coords, np.int64).reshape(n_q, 3))
    out = np.zeros((qh.shape[0], D), np.float64)
    lib().orc_attention_list3d(_p(cache.k_codes, _c_u8p), _p(cache.v_codes, _c_u8p),
                               _p(cache.k_scales, _c_f32p), _p(cache.v_scales, _c_f32p),
                               H, D, cache.W, _p(sl, _c_i32p), sl.size, _p(qq, _c_f32p), _p(c, _c_i64p),
                               _p(_npairs(npairs), _c_i32p), float(base), float(sm_scale),
                               _p(qh, _c_i32p), qh.shape[0], _p(out, _c_f64p))
    if rows is None:
        return out.reshape(n_q, H, D)
    return out


class PrefixRing:
    """Brute-force slot model of a cache whose slots [0, n_prefix) hold a fixed
    prefix and whose slots [n_prefix, W) are a ring of the last W - n_prefix
    tokens (the deque model of RingDeque, offset by the prefix)."""

    def __init__(self, W: int, n_prefix: int):
        assert 0 <= n_prefix < W
        self.P, self.ring = n_prefix, RingDeque(W - n_prefix)

    def write(self, n: int):
        return [self.P + s for s in self.ring.write(n)]

    def key_slots(self):
        """Prefix slots, then the ring's valid slots in logical order."""
        return list(range(self.P)) + [self.P + s for s in self.ring.logical_slots()]

    def ring_slots(self):
        return [self.P + s for s in self.ring.logical_slots()]


def window_dequant(cache: LayerCache, start: int, n_valid: int):
    """Dequantised K^, V^ [H][n_valid][D] (fp32) in logical window order."""
    idx = (start + np.arange(n_valid)) % cache.W
    k = dequant_rows(cache.k_codes[:, idx], cache.k_scales[:, idx])
    v = dequant_rows(cache.v_codes[:, idx], cache.v_scales[:, idx])
    return k, v


# --------------------------------------------------------------------------
# Dense fp64 definition of attention (the pin of the C attention)
# --------------------------------------------------------------------------
def dense_attention(q_rot, k_hat, v_hat, sm_scale: float) -> np.ndarray:
    """softmax(Q K^T * scale) V per head in fp64.

    q_rot [n_q][H][D], k_hat/v_hat [H][n][D] -> [n_q][H][D].
    """
    q = np.asarray(q_rot, np.float64).transpose(1, 0, 2)      # [H][n_q][D]
    k = np.asarray(k_hat, np.float64)
    v = np.asarray(v_hat, np.float64)
    s = np.matmul(q, k.transpose(0, 2, 1)) * sm_scale          # [H][n_q][n]
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.matmul(p, v).transpose(1, 0, 2)


# --------------------------------------------------------------------------
# Brute-force ring model [AI-cache]: the last W tokens in time order
# --------------------------------------------------------------------------
class RingDeque:
    """Keeps the ids of the last W tokens written, oldest first.

    A circular buffer filled in order stores token t in slot t mod W; this
    model recomputes everything from the deque, with no modular bookkeeping.
    """

    def __init__(self, W: int):
        self.W = W
        self.total = 0
        self.dq = collections.deque(maxlen=W)
        self.slot_of = {}
        self.slots = [None] * W   # slot -> token id, filled by simulation
        self.next_free = 0

    def write(self, n: int):
        new_slots = []
        for _ in range(n):
            t = self.total
            # the buffer overwrites the oldest entry once full; before that it
            # fills slots in order
            if len(self.dq) == self.W:
                old = self.dq[0]
                s = self.slot_of.pop(old)
            else:
                s = self.next_free
                self.next_free += 1
            self.dq.append(t)
            self.slot_of[t] = s
            self.slots[s] = t
            new_slots.append(s)
            self.total += 1
        return new_slots

    @property
    def n_valid(self) -> int:
        return len(self.dq)

    def logical_slots(self):
        """Slots of the valid tokens, oldest first."""
        return [self.slot_of[t] for t in self.dq]

    @property
    def next_slot(self) -> int:
        """Slot the next token will occupy."""
        if len(self.dq) < self.W:
            return self.next_free
        return self.slot_of[self.dq[0]]
