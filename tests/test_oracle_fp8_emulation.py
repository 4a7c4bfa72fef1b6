"""The precision emulation of FP8 attention schemes (oracle/fp8_emulation.py),
and what it measures at the production shape (no GPU).

The emulation is not the parity reference; it predicts the error each choice
of rounding points inside an attention kernel adds, so that the kernel's
scheme can be chosen against the bars the GPU parity tests hold the kernel
to (max-abs 2e-2 and mean-abs 2e-3 against the fp64 oracle).

Pins of the emulation's parts: bf16 rounding against PyTorch's fp32 -> bf16
conversion (round to nearest even) including ties; the per-query power of
two against its definition at the boundaries; the "exact" query path is the
fp32 rotated query; the dense reference equals the C oracle's attention row
by row.

Measurement (one production-shape layer: 12 heads, head_dim 128, a full
5788-slot window written in 8 chunks of 757, the chunk's 757 queries; all
9084 output rows): the scheme the kernel uses -- Q as two E4M3 terms, weights
and V in bf16 -- is within the bars; each scheme that would halve the matrix
work -- a single E4M3 term for Q, or a single E4M3 term for the weights with
P.V on the FP8 codes, or both -- is not.  A two-term E4M3 weight (P.V on the
FP8 codes at the bf16 product's cost) is within the bars too.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_emulation as E
from kv_cache_attention_ring_amd import inputs

BAR_MAX, BAR_MEAN = 2e-2, 2e-3


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3e38, 1e-40], np.float32)]).astype(np.float32)
    # exact ties: bf16 values plus half their last place
    b = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    ties = (b.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = E.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_pow2_exponent_boundaries():
    for k in range(-60, 60):
        edge = 448.0 * 2.0 ** k
        assert E.pow2_exponent(edge) == k
        assert E.pow2_exponent(np.nextafter(edge, np.inf)) == k + 1
        assert E.pow2_exponent(np.nextafter(edge, 0.0)) == k


def test_query_modes():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((50, 128)).astype(np.float32)
    sc = 1.0 / np.sqrt(128.0)
    c2 = np.float32(sc * E.LOG2E)
    assert np.array_equal(E.quantize_queries(q, sc, "exact"), (q * c2).astype(np.float64))
    x = (q * c2).astype(np.float64)
    one = E.quantize_queries(q, sc, "single")
    two = E.quantize_queries(q, sc, "hilo")
    # a single E4M3 term keeps 3 mantissa bits, two terms about 8
    rel1 = np.abs(one - x).max(axis=1) / np.abs(x).max(axis=1)
    rel2 = np.abs(two - x).max(axis=1) / np.abs(x).max(axis=1)
    assert rel1.max() <= 2.0 ** -4 and rel2.max() <= 2.0 ** -8 and rel2.max() < rel1.max() / 8


def _page_layer():
    """One production-shape layer written by the oracle from the seeded chunks
    (bf16 K/V with per-head scales), and the last chunk's queries."""
    shp = inputs.PAGE_LAYER
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    cache = oracle.LayerCache(H, D, W)
    total = 0
    for step in range(8):
        k, v = inputs.torch_chunk(shp, step, 0, "cpu")
        oracle.write(cache, total, total, k[0].float().numpy(), v[0].float().numpy())
        total += N
    q = inputs.torch_queries(shp, 8, 0, 0, "cpu").float().numpy()
    start = oracle.slot_of_token(total - W, W)
    return cache, start, W, q, total - N


def test_dense_reference_is_the_oracle():
    cache, start, n, q, qpos = _page_layer()
    rows = [(0, 0), (1, 3), (100, 5), (756, 11), (300, 7)]
    want = oracle.attention(cache, start, n, q, qpos, rows=rows)
    for h in sorted({h for _, h in rows}):
        got = E.attention_exact(cache, start, n, q, qpos, heads=[h])
        for r, (i, hh) in enumerate(rows):
            if hh == h:
                assert np.abs(got[i, 0] - want[r]).max() <= 1e-12


@pytest.mark.slow
def test_scheme_errors_at_production_shape(capsys):
    cache, start, n, q, qpos = _page_layer()
    ref = E.attention_exact(cache, start, n, q, qpos)
    errs = {}
    for name in E.SCHEMES:
        got = E.attention_emulated(cache, start, n, q, qpos, name)
        e = np.abs(got - ref)
        errs[name] = (float(e.max()), float(e.mean()))
    with capsys.disabled():
        print("\nFP8 scheme emulation, production layer, all 757 x 12 rows (max-abs, mean-abs):")
        for name, (mx, mean) in errs.items():
            ok = mx <= BAR_MAX and mean <= BAR_MEAN
            print(f"  {name:20s} {mx:.4f}  {mean:.5f}  {'within' if ok else 'outside'} the bars")
    within = lambda s: errs[s][0] <= BAR_MAX and errs[s][1] <= BAR_MEAN
    # the kernel's scheme, with margin; and the other two-term schemes
    assert errs["gpu_hilo_q_bf16_pv"][0] <= BAR_MAX / 2 and within("gpu_hilo_q_bf16_pv")
    assert within("exact_q_bf16_pv") and within("hilo_q_fp8x2_pv")
    # every scheme that halves the matrix work misses the max-abs bar
    for s in ("single_q_bf16_pv", "hilo_q_fp8_pv", "single_q_fp8_pv"):
        assert not within(s), (s, errs[s])
