"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random tensors
(and the integer shift of a position reset) from named sub-seeds, so that the
HIP path and the CPU oracle are fed exactly the same values.

Workloads (the pages publish no activations, so these stand in for them at
the production attention shape: 60 blocks x 4 denoise passes = 240 attention
calls per step, each over a 5788-slot cache of which 757 slots are new):

* ``TINY``  -- 1 layer, 2 heads, head_dim 64, window 96, 16 new tokens; Q, K, V
  fp32 ~ N(0, 1); 8 chunk steps with a position reset by 64 after step 4.
* ``PAGE``  -- one GPU's head share of one layer: 12 heads, head_dim 128,
  window 5788, 757 new tokens per chunk.  K and V are bf16(N(0,1) * s_h) with
  per-head scales s_h ~ U(0.5, 2) drawn separately for K and V of each layer;
  Q is bf16(N(0, 1)), drawn fresh for every denoise pass.

Seeds: base seed 20261105; every tensor has a sub-seed derived from
(workload, step, layer, pass, tensor) through numpy's SeedSequence.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BASE_SEED = 20261105

_TENSOR_IDS = {"k": 1, "v": 2, "q": 3, "scale_k": 4, "scale_v": 5, "delta": 6, "src": 7}
_WORKLOAD_IDS = {"tiny": 1, "layer": 2, "step": 3, "rebase": 4, "naive": 5, "wrap": 6, "test": 7,
                 "prefix": 8}


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    n_layers: int
    n_heads: int
    head_dim: int
    window: int
    n_new: int
    passes: int = 4
    rope_base: float = 10000.0


TINY = Shape("tiny", 1, 2, 64, 96, 16)
TINY_WRAP = Shape("wrap", 1, 2, 64, 100, 16)        # 100 is not a multiple of 16: wraps mid-chunk
PAGE_LAYER = Shape("layer", 1, 12, 128, 5788, 757)
PAGE_STEP = Shape("step", 60, 12, 128, 5788, 757)

#: position reset period (steps) and the largest shift it can apply
RESET_PERIOD = 42
DELTA_MAX = RESET_PERIOD * 757


def set_base_seed(seed: int) -> None:
    """Change the base seed every sub-seed is derived from (default 20261105)."""
    global BASE_SEED
    BASE_SEED = int(seed)


def _seed_seq(workload: str, step: int, layer: int, pss: int, tensor: str) -> np.random.SeedSequence:
    return np.random.SeedSequence([BASE_SEED, _WORKLOAD_IDS[workload], int(step) + 1000,
                                   int(layer), int(pss) + 10, _TENSOR_IDS[tensor]])


def np_rng(workload: str, step: int = 0, layer: int = 0, pss: int = 0,
           tensor: str = "k") -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seed_seq(workload, step, layer, pss, tensor)))


def torch_seed(workload: str, step: int = 0, layer: int = 0, pss: int = 0, tensor: str = "k") -> int:
    st = _seed_seq(workload, step, layer, pss, tensor).generate_state(2, dtype=np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


# ---------------------------------------------------------------------------
# fp32 NumPy inputs (small shapes)
# ---------------------------------------------------------------------------
def np_chunk(shape: Shape, step: int, layer: int = 0, workload: str | None = None, pss: int = 0):
    """New K, V rows of one chunk: fp32 [N][H][D] ~ N(0, 1).  `pss` > 0 draws
    the rows of a later denoise pass of the same step (pass 0 is the default)."""
    w = workload or shape.name
    sz = (shape.n_new, shape.n_heads, shape.head_dim)
    k = np_rng(w, step, layer, pss, "k").standard_normal(sz, dtype=np.float32)
    v = np_rng(w, step, layer, pss, "v").standard_normal(sz, dtype=np.float32)
    return k, v


def np_queries(shape: Shape, step: int, pss: int, layer: int = 0, workload: str | None = None,
               n_q: int | None = None):
    w = workload or shape.name
    sz = (n_q or shape.n_new, shape.n_heads, shape.head_dim)
    return np_rng(w, step, layer, pss, "q").standard_normal(sz, dtype=np.float32)


# ---------------------------------------------------------------------------
# torch inputs (page shapes); generated on `device` with a seeded generator
# ---------------------------------------------------------------------------
def head_scales(shape: Shape, layer: int, workload: str | None = None):
    """Per-head K and V scales s_h ~ U(0.5, 2) of one layer (fp32 numpy [H])."""
    w = workload or shape.name
    sk = np_rng(w, 0, layer, 0, "scale_k").uniform(0.5, 2.0, shape.n_heads).astype(np.float32)
    sv = np_rng(w, 0, layer, 0, "scale_v").uniform(0.5, 2.0, shape.n_heads).astype(np.float32)
    return sk, sv


def torch_chunk(shape: Shape, step: int, layer: int, device, dtype=None, workload: str | None = None,
                n_layers: int = 1, pss: int = 0):
    """New K, V rows: [n_layers][N][H][D] in dtype (bf16 default), scaled per head.
    `pss` > 0 draws the rows of a later denoise pass of the same step."""
    import torch
    dtype = dtype or torch.bfloat16
    w = workload or shape.name
    sz = (shape.n_new, shape.n_heads, shape.head_dim)
    ks, vs = [], []
    for li in range(layer, layer + n_layers):
        sk, sv = head_scales(shape, li, w)
        out = []
        for t, s in (("k", sk), ("v", sv)):
            g = torch.Generator(device=device)
            g.manual_seed(torch_seed(w, step, li, pss, t))
            x = torch.randn(sz, generator=g, device=device, dtype=torch.float32)
            x = x * torch.as_tensor(s, device=device).view(1, -1, 1)
            out.append(x.to(dtype))
        ks.append(out[0])
        vs.append(out[1])
    return torch.stack(ks), torch.stack(vs)


def torch_queries(shape: Shape, step: int, pss: int, layer: int, device, dtype=None,
                  workload: str | None = None):
    import torch
    dtype = dtype or torch.bfloat16
    w = workload or shape.name
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(w, step, layer, pss, "q"))
    sz = (shape.n_new, shape.n_heads, shape.head_dim)
    return torch.randn(sz, generator=g, device=device, dtype=torch.float32).to(dtype)


def rebase_delta(workload: str = "rebase") -> int:
    """Shift of a position reset, uniform in [1, 42 * 757]."""
    return int(np_rng(workload, 0, 0, 0, "delta").integers(1, DELTA_MAX + 1))


# ---------------------------------------------------------------------------
# 3-D (t, y, x) token coordinates (video tokens)
# ---------------------------------------------------------------------------
#: latent frame width in tokens: a chunk's tokens are numbered row-major over a
#: grid this many columns wide (757 is prime, so its last row is partial)
FRAME_COLS = 28
#: the frame-index shift of a position reset at most: one frame per chunk step
DELTA_T_MAX = RESET_PERIOD


def axis_pairs(head_dim: int):
    """Pairs per axis (t, y, x): the row and column groups get floor(D/6) pairs
    each and the frame group the rest (D = 128: 22, 21, 21; D = 64: 12, 10, 10)."""
    half = head_dim // 2
    s = half // 3
    return (half - 2 * s, s, s)


def chunk_coords(n_new: int, frame: int, cols: int = FRAME_COLS) -> np.ndarray:
    """(t, y, x) of the n_new tokens of the chunk that carries frame `frame`:
    int64 [n_new][3], t = frame, token j at row j // cols, column j % cols."""
    j = np.arange(n_new, dtype=np.int64)
    return np.stack([np.full(n_new, frame, np.int64), j // cols, j % cols], axis=1)


def rebase_delta_t(workload: str = "rebase") -> int:
    """Frame-index shift of a position reset, uniform in [1, 42]."""
    return int(np_rng(workload, 0, 0, 0, "delta").integers(1, DELTA_T_MAX + 1))
