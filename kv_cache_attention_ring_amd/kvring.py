"""ctypes binding of libkvring.so (declared in include/kvring.h).

Argument marshalling only: every function here passes raw device pointers
(``tensor.data_ptr()``) and the current HIP stream to the C entry point of
the same name; all arithmetic of the cache path runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  When the library is
missing this module raises at load time; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvring.so")

KVR_OK, KVR_EINVAL, KVR_EALIGN, KVR_EUNSUPPORTED, KVR_ELAUNCH = 0, -1, -2, -3, -4
KVR_F32, KVR_BF16 = 0, 1


class KVRError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvring status {status}: {msg}")
        self.status = status


class kvr_ring(ctypes.Structure):
    """Ring state (host POD): head, n_valid, pos_next."""
    _fields_ = [("head", ctypes.c_int32), ("n_valid", ctypes.c_int32), ("pos_next", ctypes.c_int64)]

    def __repr__(self):
        return f"kvr_ring(head={self.head}, n_valid={self.n_valid}, pos_next={self.pos_next})"

    def copy(self) -> "kvr_ring":
        return kvr_ring(self.head, self.n_valid, self.pos_next)


class kvr_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_prefix", ctypes.c_int32)]


class kvr_rope_table(ctypes.Structure):
    _fields_ = [("cs", ctypes.c_void_p), ("pos0", ctypes.c_int64), ("n_pos", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _F32, _F64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t

_SIGS = {
    "kvr_ring_init": (None, [ctypes.POINTER(kvr_ring)]),
    "kvr_ring_slot": (_I32, [ctypes.POINTER(kvr_ring), _I32, _I32]),
    "kvr_ring_logical_start": (_I32, [ctypes.POINTER(kvr_ring), _I32]),
    "kvr_ring_after_write": (_I32, [ctypes.POINTER(kvr_ring), _I32, _I32]),
    "kvr_ring_after_rebase": (_I32, [ctypes.POINTER(kvr_ring), _I64]),
    "kv_rope_table_fill": (_I32, [_P, _I64, _I32, _I32, _F64, _P]),
    "kv_write_rope_quant": (_I32, [ctypes.POINTER(kvr_cache), ctypes.POINTER(kvr_ring), _I32, _I32,
                                   _P, _P, _I32, _I64, _I32, ctypes.POINTER(kvr_rope_table), _P]),
    "kv_delta_rebase": (_I32, [ctypes.POINTER(kvr_cache), ctypes.POINTER(kvr_ring), _I32, _I32,
                               _I64, _F64, _P]),
    "attn_fp8_window_workspace_bytes": (_SZ, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32]),
    "attn_fp8_window": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _I32, _I32, _I64,
                               _F32, _F64, _P, _I32, _P, _SZ, _P]),
    "attn_fp8_window_partial": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _I32, _I32, _I64,
                                       _F32, _F64, _P, _I32, _P, _SZ, _P]),
    "attn_fp8_window_merge": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "attn_fp8_window_write_workspace_bytes": (_SZ, [ctypes.POINTER(kvr_cache), ctypes.POINTER(kvr_ring),
                                                     _I32, _I32]),
    "attn_fp8_window_write": (_I32, [ctypes.POINTER(kvr_cache), ctypes.POINTER(kvr_ring), _I32, _P, _P, _P,
                                     _I32, _I32, ctypes.POINTER(kvr_rope_table), _F32, _F64, _P, _I32, _P,
                                     _SZ, _P]),
    "attn_fp8_window_noalloc": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _I32, _I32, _I64,
                                       _F32, _F64, _P, _I32, _P]),
    "naive_upkeep": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32,
                            ctypes.POINTER(kvr_rope_table), _P, _P, _P, _P, _P, _P, _P]),
    "kv_rope3d_table_fill": (_I32, [_P, _P, _I32, _I32, ctypes.POINTER(_I32), _F64, _P]),
    "kv_write_rope_quant_rows": (_I32, [ctypes.POINTER(kvr_cache), ctypes.POINTER(kvr_ring), _I32, _I32,
                                        _P, _P, _I32, _I64, _I32, _P, _P]),
    "kv_delta_rebase_axes": (_I32, [ctypes.POINTER(kvr_cache), ctypes.POINTER(kvr_ring), _I32, _I32,
                                    ctypes.POINTER(_I64), ctypes.POINTER(_I32), _F64, _P]),
    "attn_fp8_window_rows": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _I32, _I32, _P,
                                    _F32, _P, _I32, _P, _SZ, _P]),
    "kv_write_prefix_rows": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _P, _I32, _I64, _I32,
                                    _P, _P]),
    "kv_rope_query_lanes_bytes": (_SZ, [_I32, _I32]),
    "kv_rope_query_lanes": (_I32, [_P, _I32, _I32, _P, _P]),
    "attn_fp8_window_lanes": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _I32, _I32, _P,
                                     _F32, _P, _I32, _P, _SZ, _P]),
    "attn_fp8_window_lanes_partial": (_I32, [ctypes.POINTER(kvr_cache), _I32, _I32, _I32, _P, _I32, _I32, _P,
                                             _F32, _P, _I32, _P, _SZ, _P]),
    "kvr_last_error": (ctypes.c_char_p, []),
    "kvr_version": (ctypes.c_char_p, []),
}

#: every symbol include/kvring.h declares
EXPORTED = tuple(_SIGS)


def lib():
    """Load libkvring.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_attention_ring_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != KVR_OK:
        raise KVRError(status, lib().kvr_last_error().decode())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVR_BF16
    if t.dtype == torch.float32:
        return KVR_F32
    raise KVRError(KVR_EUNSUPPORTED, f"dtype {t.dtype} not supported (bf16, fp32)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise KVRError(KVR_EINVAL, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise KVRError(KVR_EINVAL, f"{name} must be contiguous")
    return t.data_ptr()


# ---------------------------------------------------------------------------
# device-memory holders (allocation is the caller's, i.e. torch's)
# ---------------------------------------------------------------------------
class KVCache:
    """FP8 K/V codes [L][H][W][D] (uint8) and fp32 scales [L][H][W], on a device.
    With n_prefix > 0, slots [0, n_prefix) hold a fixed prefix and the ring is
    the other ring_window = window - n_prefix slots."""

    def __init__(self, n_layers: int, n_heads: int, head_dim: int, window: int, device="cuda",
                 n_prefix: int = 0):
        self.shape = (n_layers, n_heads, window, head_dim)
        self.k_codes = torch.zeros(self.shape, dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros(self.shape, dtype=torch.uint8, device=device)
        self.k_scales = torch.zeros(self.shape[:3], dtype=torch.float32, device=device)
        self.v_scales = torch.zeros(self.shape[:3], dtype=torch.float32, device=device)
        self.n_layers, self.n_heads, self.head_dim, self.window = n_layers, n_heads, head_dim, window
        self.n_prefix = int(n_prefix)
        self.ring_window = window - self.n_prefix

    def desc(self) -> kvr_cache:
        return kvr_cache(self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                         self.k_scales.data_ptr(), self.v_scales.data_ptr(),
                         self.n_layers, self.n_heads, self.head_dim, self.window, self.n_prefix)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.k_codes, self.v_codes, self.k_scales, self.v_scales))


class RopeTable:
    """Device (cos, sin) table of positions pos0 .. pos0+n_pos-1 (kv_rope_table_fill)."""

    def __init__(self, pos0: int, n_pos: int, head_dim: int, base: float = 10000.0, device="cuda",
                 stream=None):
        self.cs = torch.empty((n_pos, head_dim // 2, 2), dtype=torch.float32, device=device)
        self.pos0, self.n_pos, self.head_dim, self.base = int(pos0), int(n_pos), head_dim, float(base)
        kv_rope_table_fill(self.cs, self.pos0, self.n_pos, head_dim, self.base, stream)

    def desc(self) -> kvr_rope_table:
        return kvr_rope_table(self.cs.data_ptr(), self.pos0, self.n_pos, self.head_dim)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def kvr_ring_init() -> kvr_ring:
    r = kvr_ring()
    lib().kvr_ring_init(ctypes.byref(r))
    return r


def kvr_ring_slot(r: kvr_ring, window: int, j: int) -> int:
    return int(lib().kvr_ring_slot(ctypes.byref(r), window, j))


def kvr_ring_logical_start(r: kvr_ring, window: int) -> int:
    return int(lib().kvr_ring_logical_start(ctypes.byref(r), window))


def kvr_ring_after_write(r: kvr_ring, window: int, n_new: int) -> None:
    _check(lib().kvr_ring_after_write(ctypes.byref(r), window, n_new))


def kvr_ring_after_rebase(r: kvr_ring, delta: int) -> None:
    _check(lib().kvr_ring_after_rebase(ctypes.byref(r), int(delta)))


def kv_rope_table_fill(cs: torch.Tensor, pos0: int, n_pos: int, head_dim: int, base: float,
                       stream=None) -> None:
    _check(lib().kv_rope_table_fill(_dev(cs, "cs"), int(pos0), int(n_pos), int(head_dim),
                                    float(base), _stream(stream)))


def kv_write_rope_quant(cache: KVCache, before: kvr_ring, layer0: int, k_new: torch.Tensor,
                        v_new: torch.Tensor, rope: RopeTable, stream=None) -> None:
    """k_new / v_new: [N][H][D] (one layer) or [n_layers][N][H][D] (layers layer0..)."""
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise KVRError(KVR_EINVAL, "k_new and v_new must match in shape and dtype")
    if k_new.dim() == 3:
        n_layers, (n_new, _, _) = 1, k_new.shape
        stride = k_new.numel()
    elif k_new.dim() == 4:
        n_layers, n_new = k_new.shape[0], k_new.shape[1]
        stride = k_new[0].numel()
    else:
        raise KVRError(KVR_EINVAL, "k_new must be [N][H][D] or [L][N][H][D]")
    if k_new.shape[-2:] != (cache.n_heads, cache.head_dim):
        raise KVRError(KVR_EINVAL, f"k_new trailing shape {tuple(k_new.shape[-2:])} != "
                                   f"({cache.n_heads}, {cache.head_dim})")
    c = cache.desc()
    t = rope.desc()
    _check(lib().kv_write_rope_quant(ctypes.byref(c), ctypes.byref(before), layer0, n_layers,
                                     _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new),
                                     stride, n_new, ctypes.byref(t), _stream(stream)))


def _new_rows(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor):
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise KVRError(KVR_EINVAL, "k_new and v_new must match in shape and dtype")
    if k_new.dim() == 3:
        n_layers, (n_new, _, _) = 1, k_new.shape
        stride = k_new.numel()
    elif k_new.dim() == 4:
        n_layers, n_new = k_new.shape[0], k_new.shape[1]
        stride = k_new[0].numel()
    else:
        raise KVRError(KVR_EINVAL, "k_new must be [N][H][D] or [L][N][H][D]")
    if k_new.shape[-2:] != (cache.n_heads, cache.head_dim):
        raise KVRError(KVR_EINVAL, f"k_new trailing shape {tuple(k_new.shape[-2:])} != "
                                   f"({cache.n_heads}, {cache.head_dim})")
    return n_layers, n_new, stride


def _axes(v, ct):
    a = (ct * 3)(*[int(x) for x in v])
    if len(v) != 3:
        raise KVRError(KVR_EINVAL, "three axes (t, y, x) expected")
    return a


class Rope3DRows:
    """Device (cos, sin) rows [n_tok][D/2][2] of tokens at (t, y, x) coordinates
    (kv_rope3d_table_fill); coords: int [n_tok][3] (host or device)."""

    def __init__(self, coords, head_dim: int, axis_pairs, base: float = 10000.0, device="cuda",
                 stream=None):
        c64 = torch.as_tensor(coords).reshape(-1, 3)
        if c64.dtype.is_floating_point or (c64.numel() and int(c64.abs().max()) >= 2 ** 31):
            raise KVRError(KVR_EINVAL, "coordinates must be integers below 2^31 in magnitude")
        c = c64.to(torch.int32).to(device).contiguous()
        self.coords = c
        self.n_tok, self.head_dim, self.base = c.shape[0], head_dim, float(base)
        self.axis_pairs = tuple(int(x) for x in axis_pairs)
        self.cs = torch.empty((self.n_tok, head_dim // 2, 2), dtype=torch.float32, device=device)
        _check(lib().kv_rope3d_table_fill(_dev(self.cs, "cs"), _dev(c, "coords"), self.n_tok, head_dim,
                                          _axes(self.axis_pairs, _I32), self.base, _stream(stream)))


def kv_write_rope_quant_rows(cache: KVCache, before: kvr_ring, layer0: int, k_new: torch.Tensor,
                             v_new: torch.Tensor, cs_rows: torch.Tensor, stream=None) -> None:
    """As kv_write_rope_quant, token j rotated by cs_rows[j] ([N][D/2][2] fp32)."""
    n_layers, n_new, stride = _new_rows(cache, k_new, v_new)
    if cs_rows.dtype != torch.float32 or cs_rows.shape != (n_new, cache.head_dim // 2, 2):
        raise KVRError(KVR_EINVAL, "cs_rows must be fp32 [n_new][head_dim/2][2]")
    c = cache.desc()
    _check(lib().kv_write_rope_quant_rows(ctypes.byref(c), ctypes.byref(before), layer0, n_layers,
                                          _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new),
                                          stride, n_new, _dev(cs_rows, "cs_rows"), _stream(stream)))


def kv_write_prefix_rows(cache: KVCache, slot0: int, layer0: int, k_new: torch.Tensor, v_new: torch.Tensor,
                         cs_rows: torch.Tensor, stream=None) -> None:
    """Prefix tokens j -> prefix slots slot0 + j, rotated by cs_rows[j] ([n][D/2][2] fp32)."""
    n_layers, n_tok, stride = _new_rows(cache, k_new, v_new)
    if cs_rows.dtype != torch.float32 or cs_rows.shape != (n_tok, cache.head_dim // 2, 2):
        raise KVRError(KVR_EINVAL, "cs_rows must be fp32 [n_tok][head_dim/2][2]")
    c = cache.desc()
    _check(lib().kv_write_prefix_rows(ctypes.byref(c), int(slot0), layer0, n_layers, _dev(k_new, "k_new"),
                                      _dev(v_new, "v_new"), _dtype_code(k_new), stride, n_tok,
                                      _dev(cs_rows, "cs_rows"), _stream(stream)))


def kv_delta_rebase_axes(cache: KVCache, ring: kvr_ring, layer0: int, n_layers: int, delta, axis_pairs,
                         rope_base: float = 10000.0, stream=None) -> None:
    """Rotate every valid K row by -delta[a] on the pairs of axis a (delta = (t, y, x))."""
    c = cache.desc()
    _check(lib().kv_delta_rebase_axes(ctypes.byref(c), ctypes.byref(ring), layer0, n_layers,
                                      _axes(delta, _I64), _axes(axis_pairs, _I32), float(rope_base),
                                      _stream(stream)))


def attn_fp8_window_rows(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
                         q_cs_rows: torch.Tensor, out: torch.Tensor | None = None, n_splits: int = 0,
                         ws: torch.Tensor | None = None, softmax_scale: float | None = None,
                         stream=None) -> torch.Tensor:
    """As attn_fp8_window, query i rotated by q_cs_rows[i] ([n_q][D/2][2] fp32)."""
    args, out, _, _c = _attn_args(cache, layer, slot_start, n_valid, q, 0, 10000.0, out, n_splits, ws,
                                  softmax_scale, stream)
    if q_cs_rows.dtype != torch.float32 or q_cs_rows.shape != (q.shape[0], cache.head_dim // 2, 2):
        raise KVRError(KVR_EINVAL, "q_cs_rows must be fp32 [n_q][head_dim/2][2]")
    # the position form's (q_pos_start, rope_base) pair is replaced by the rows
    rows_args = args[:7] + (_dev(q_cs_rows, "q_cs_rows"), args[8]) + args[10:]
    _check(lib().attn_fp8_window_rows(*rows_args))
    return out


def kv_rope_query_lanes(cs_rows: torch.Tensor, stream=None) -> torch.Tensor:
    """The queries' (cos, sin) rows [n_q][D/2][2] in the attention kernel's load
    layout (an opaque device buffer for attn_fp8_window_lanes)."""
    if cs_rows.dtype != torch.float32 or cs_rows.dim() != 3 or cs_rows.shape[2] != 2:
        raise KVRError(KVR_EINVAL, "cs_rows must be fp32 [n_q][head_dim/2][2]")
    n_q, D = cs_rows.shape[0], 2 * cs_rows.shape[1]
    nbytes = int(lib().kv_rope_query_lanes_bytes(n_q, D))
    if nbytes == 0:
        raise KVRError(KVR_EINVAL, f"unsupported query rows shape {tuple(cs_rows.shape)}")
    lanes = torch.empty(nbytes // 4, dtype=torch.float32, device=cs_rows.device)
    _check(lib().kv_rope_query_lanes(_dev(cs_rows, "cs_rows"), n_q, D, _dev(lanes, "lanes"), _stream(stream)))
    return lanes


def attn_fp8_window_lanes(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
                          q_lanes: torch.Tensor, out: torch.Tensor | None = None, n_splits: int = 0,
                          ws: torch.Tensor | None = None, softmax_scale: float | None = None,
                          stream=None) -> torch.Tensor:
    """attn_fp8_window_rows with the rows already in the kernel's load layout
    (kv_rope_query_lanes); same results bit for bit."""
    args, out, _, _c = _attn_args(cache, layer, slot_start, n_valid, q, 0, 10000.0, out, n_splits, ws,
                                  softmax_scale, stream)
    need = int(lib().kv_rope_query_lanes_bytes(q.shape[0], cache.head_dim))
    if q_lanes.dtype != torch.float32 or q_lanes.numel() * 4 < need:
        raise KVRError(KVR_EINVAL, f"q_lanes must be an fp32 buffer of at least {need} bytes")
    lanes_args = args[:7] + (_dev(q_lanes, "q_lanes"), args[8]) + args[10:]
    _check(lib().attn_fp8_window_lanes(*lanes_args))
    return out


def attn_fp8_window_lanes_partial(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
                                  q_lanes: torch.Tensor, out: torch.Tensor | None = None, n_splits: int = 0,
                                  ws: torch.Tensor | None = None, softmax_scale: float | None = None,
                                  stream=None):
    """The attention kernel of attn_fp8_window_lanes alone (merge with
    attn_fp8_window_merge); returns (out, ws)."""
    args, out, ws, _c = _attn_args(cache, layer, slot_start, n_valid, q, 0, 10000.0, out, n_splits, ws,
                                   softmax_scale, stream)
    need = int(lib().kv_rope_query_lanes_bytes(q.shape[0], cache.head_dim))
    if q_lanes.dtype != torch.float32 or q_lanes.numel() * 4 < need:
        raise KVRError(KVR_EINVAL, f"q_lanes must be an fp32 buffer of at least {need} bytes")
    lanes_args = args[:7] + (_dev(q_lanes, "q_lanes"), args[8]) + args[10:]
    _check(lib().attn_fp8_window_lanes_partial(*lanes_args))
    return out, ws


def rope_table_rows(rope: RopeTable, pos0: int, n: int) -> torch.Tensor:
    """The table's (cos, sin) rows of positions pos0 .. pos0+n-1 (a view)."""
    i = int(pos0) - rope.pos0
    if i < 0 or i + n > rope.n_pos:
        raise KVRError(KVR_EINVAL, f"positions [{pos0},{pos0 + n}) outside the rotary table")
    return rope.cs[i:i + n]


def kv_delta_rebase(cache: KVCache, ring: kvr_ring, layer0: int, n_layers: int, delta: int,
                    rope_base: float = 10000.0, stream=None) -> None:
    c = cache.desc()
    _check(lib().kv_delta_rebase(ctypes.byref(c), ctypes.byref(ring), layer0, n_layers, int(delta),
                                 float(rope_base), _stream(stream)))


def attn_fp8_window_workspace_bytes(cache: KVCache, n_q: int, n_valid: int, n_splits: int = 0) -> int:
    c = cache.desc()
    return int(lib().attn_fp8_window_workspace_bytes(ctypes.byref(c), n_q, n_valid, n_splits))


def _attn_args(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
               q_pos_start: int, rope_base: float, out, n_splits: int, ws, softmax_scale, stream):
    n_q = q.shape[0]
    if q.dim() != 3 or q.shape[1:] != (cache.n_heads, cache.head_dim):
        raise KVRError(KVR_EINVAL, f"q shape {tuple(q.shape)} does not match the cache")
    # tensors allocated here are used by kernels on `stream`: when that is not
    # the current stream, the caching allocator is told so (record_stream), or
    # it could hand their memory to a new tensor while those kernels still run
    side = stream is not None and stream != torch.cuda.current_stream(q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if side:
            out.record_stream(stream)
    if out.dtype != torch.bfloat16 or out.shape != q.shape:
        raise KVRError(KVR_EINVAL, "out must be bf16 with q's shape")
    need = attn_fp8_window_workspace_bytes(cache, n_q, n_valid, n_splits)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        if side:
            ws.record_stream(stream)
    ws_ptr = _dev(ws, "ws") if ws is not None else None
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    if softmax_scale is None:
        softmax_scale = 0.0                      # the library's default, 1/sqrt(head_dim)
    c = cache.desc()
    args = (ctypes.byref(c), layer, slot_start, n_valid, _dev(q, "q"), _dtype_code(q), n_q,
            int(q_pos_start), float(softmax_scale), float(rope_base), _dev(out, "out"), int(n_splits),
            ws_ptr, ws_len, _stream(stream))
    return args, out, ws, c


def attn_fp8_window(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
                    q_pos_start: int, rope_base: float = 10000.0, out: torch.Tensor | None = None,
                    n_splits: int = 0, ws: torch.Tensor | None = None,
                    softmax_scale: float | None = None, stream=None) -> torch.Tensor:
    """q: [n_q][H][D] bf16/fp32 -> out: [n_q][H][D] bf16."""
    args, out, _, _c = _attn_args(cache, layer, slot_start, n_valid, q, q_pos_start, rope_base, out,
                                  n_splits, ws, softmax_scale, stream)
    _check(lib().attn_fp8_window(*args))
    return out


def attn_fp8_window_partial(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
                            q_pos_start: int, rope_base: float = 10000.0, out: torch.Tensor | None = None,
                            n_splits: int = 0, ws: torch.Tensor | None = None,
                            softmax_scale: float | None = None, stream=None):
    """The attention kernel alone: out for one split, partials in ws otherwise.
    Returns (out, ws) for attn_fp8_window_merge."""
    args, out, ws, _c = _attn_args(cache, layer, slot_start, n_valid, q, q_pos_start, rope_base, out,
                                   n_splits, ws, softmax_scale, stream)
    _check(lib().attn_fp8_window_partial(*args))
    return out, ws


def attn_fp8_window_merge(cache: KVCache, n_q: int, n_valid: int, out: torch.Tensor,
                          n_splits: int = 0, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Merge the split partials in ws into out (nothing to do for one split)."""
    c = cache.desc()
    ws_ptr = _dev(ws, "ws") if ws is not None else None
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().attn_fp8_window_merge(ctypes.byref(c), n_q, n_valid, int(n_splits), _dev(out, "out"),
                                       ws_ptr, ws_len, _stream(stream)))
    return out


def attn_fp8_window_write_workspace_bytes(cache: KVCache, before: kvr_ring, n_new: int,
                                          n_splits: int = 0) -> int:
    c = cache.desc()
    return int(lib().attn_fp8_window_write_workspace_bytes(ctypes.byref(c), ctypes.byref(before), n_new,
                                                            n_splits))


#: size of the control block at the end of a fused-write workspace (uint32 words: writers done,
#: waiting workgroups through, waits that gave up, poll limit)
FUSED_SYNC_BYTES = 256


def attn_fp8_window_write(cache: KVCache, before: kvr_ring, layer: int, k_new: torch.Tensor,
                          v_new: torch.Tensor, q: torch.Tensor, rope: RopeTable, rope_base: float = 10000.0,
                          out: torch.Tensor | None = None, n_splits: int = 0, ws: torch.Tensor | None = None,
                          softmax_scale: float | None = None, stream=None) -> torch.Tensor:
    """Write the chunk k_new/v_new ([N][H][D]) of `layer` at ring state `before`
    and attend with q ([N][H][D], the chunk's tokens) over the window holding
    it -> out [N][H][D] bf16.  ws: zeroed before its first use (a workspace
    allocated here is)."""
    n_layers, n_new, _ = _new_rows(cache, k_new, v_new)
    if n_layers != 1 or q.shape != k_new.shape or q.dtype != k_new.dtype:
        raise KVRError(KVR_EINVAL, "k_new, v_new and q must be one layer's [N][H][D] of one dtype")
    side = stream is not None and stream != torch.cuda.current_stream(q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if side:
            out.record_stream(stream)
    if out.dtype != torch.bfloat16 or out.shape != q.shape:
        raise KVRError(KVR_EINVAL, "out must be bf16 with q's shape")
    if ws is None:
        ws = torch.zeros(attn_fp8_window_write_workspace_bytes(cache, before, n_new, n_splits),
                         dtype=torch.uint8, device=q.device)
        if side:
            ws.record_stream(stream)
    c = cache.desc()
    t = rope.desc()
    _check(lib().attn_fp8_window_write(ctypes.byref(c), ctypes.byref(before), layer, _dev(k_new, "k_new"),
                                       _dev(v_new, "v_new"), _dev(q, "q"), _dtype_code(q), n_new, ctypes.byref(t),
                                       float(softmax_scale or 0.0), float(rope_base), _dev(out, "out"),
                                       int(n_splits), _dev(ws, "ws"), ws.numel() * ws.element_size(),
                                       _stream(stream)))
    return out


#: bytes of the library's per-GPU scratch array for attn_fp8_window_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_fp8_window_noalloc(cache: KVCache, layer: int, slot_start: int, n_valid: int, q: torch.Tensor,
                            q_pos_start: int, rope_base: float = 10000.0, out: torch.Tensor | None = None,
                            n_splits: int = 0, softmax_scale: float | None = None, stream=None) -> torch.Tensor:
    """attn_fp8_window with the split partials in the library's own scratch
    array (the C entry point allocates nothing; pass `out` to allocate nothing
    here either)."""
    n_q = q.shape[0]
    if q.dim() != 3 or q.shape[1:] != (cache.n_heads, cache.head_dim):
        raise KVRError(KVR_EINVAL, f"q shape {tuple(q.shape)} does not match the cache")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if stream is not None and stream != torch.cuda.current_stream(q.device):
            out.record_stream(stream)
    if out.dtype != torch.bfloat16 or out.shape != q.shape:
        raise KVRError(KVR_EINVAL, "out must be bf16 with q's shape")
    c = cache.desc()
    _check(lib().attn_fp8_window_noalloc(ctypes.byref(c), layer, slot_start, n_valid, _dev(q, "q"), _dtype_code(q),
                                         n_q, int(q_pos_start), float(softmax_scale or 0.0), float(rope_base),
                                         _dev(out, "out"), int(n_splits), _stream(stream)))
    return out


def naive_upkeep(lin_k_src: torch.Tensor, lin_v_src: torch.Tensor, k_new: torch.Tensor,
                 v_new: torch.Tensor, n_valid_before: int, pos_next_before: int, rope: RopeTable,
                 lin_k_dst: torch.Tensor, lin_v_dst: torch.Tensor, k_codes: torch.Tensor,
                 v_codes: torch.Tensor, k_scales: torch.Tensor, v_scales: torch.Tensor,
                 stream=None) -> None:
    """Linear windows [H][W][D]; new rows [N][H][D]; codes [H][W][D]; scales [H][W]."""
    H, W, D = lin_k_src.shape
    n_new = k_new.shape[0]
    for name, t in (("lin_v_src", lin_v_src), ("lin_k_dst", lin_k_dst), ("lin_v_dst", lin_v_dst)):
        if t.shape != lin_k_src.shape or t.dtype != lin_k_src.dtype:
            raise KVRError(KVR_EINVAL, f"{name} must match lin_k_src")
    if k_new.dtype != lin_k_src.dtype or k_new.shape[1:] != (H, D) or v_new.shape != k_new.shape:
        raise KVRError(KVR_EINVAL, "new rows must be [N][H][D] in the window dtype")
    if k_codes.shape != (H, W, D) or v_codes.shape != (H, W, D) or k_scales.shape != (H, W) \
            or v_scales.shape != (H, W):
        raise KVRError(KVR_EINVAL, "codes [H][W][D] and scales [H][W] expected")
    t = rope.desc()
    _check(lib().naive_upkeep(_dev(lin_k_src, "lin_k_src"), _dev(lin_v_src, "lin_v_src"),
                              _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new), n_new,
                              int(n_valid_before), int(pos_next_before), H, D, W, ctypes.byref(t),
                              _dev(lin_k_dst, "lin_k_dst"), _dev(lin_v_dst, "lin_v_dst"),
                              _dev(k_codes, "k_codes"), _dev(v_codes, "v_codes"),
                              _dev(k_scales, "k_scales"), _dev(v_scales, "v_scales"),
                              _stream(stream)))


def kvr_last_error() -> str:
    return lib().kvr_last_error().decode()


def kvr_version() -> str:
    return lib().kvr_version().decode()
