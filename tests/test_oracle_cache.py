"""Pins of the oracle's ring, write, naive, rebase and attention (no GPU).

* Ring: the slot of every token equals what a brute-force deque of the last W
  tokens says, over every small (W, N) and enough steps to wrap several times,
  including W = 100, N = 16 (a chunk that wraps in the middle).
* Write vs naive: the write-time ring cache and the naive per-call window are
  bit-identical before any reset (codes and scales, lin[i] == ring[(start+i) % W]).
* Rebase: R(-delta) applied to the stored window then R(+delta) returns the
  dequantised keys within two requantisation errors; two rebases compose; after a
  reset the ring stays within the requantisation bound of the naive window.
* Attention: the C oracle equals a dense fp64 NumPy softmax(QK^T)V, which equals
  SciPy's softmax and PyTorch's CPU scaled_dot_product_attention in fp64, plus
  closed forms (one key, zero query, equal keys, weights summing to one).
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from kv_cache_attention_ring_amd import inputs


# ---------------------------------------------------------------------------
# ring
# ---------------------------------------------------------------------------
def _ring_cases():
    for W in (1, 2, 3, 5, 8, 16, 31, 64, 96, 100, 128):
        for N in sorted({1, 2, 3, W // 3 or 1, W // 2 or 1, W - 1 or 1, W, 16 if W >= 16 else 1}):
            if 1 <= N <= W:
                yield W, N


@pytest.mark.parametrize("W,N", list(_ring_cases()))
def test_ring_slots_match_deque(W, N):
    dq = oracle.RingDeque(W)
    total = 0
    for _ in range(3 * W // N + 2):
        slots = dq.write(N)
        assert slots == [oracle.slot_of_token(total + j, W) for j in range(N)]
        total += N
        start = dq.logical_slots()[0]
        assert start == oracle.slot_of_token(total - dq.n_valid, W)
        assert dq.logical_slots() == [(start + i) % W for i in range(dq.n_valid)]


def test_wrap_mid_chunk_case_exists():
    # W = 100, N = 16: the 7th chunk occupies slots 96..99 then 0..11
    dq = oracle.RingDeque(100)
    for _ in range(6):
        dq.write(16)
    assert dq.write(16) == list(range(96, 100)) + list(range(0, 12))


# ---------------------------------------------------------------------------
# write vs naive
# ---------------------------------------------------------------------------
def _run_write_vs_naive(shape, steps, check_steps):
    H, D, W, N = shape.n_heads, shape.head_dim, shape.window, shape.n_new
    ring = oracle.LayerCache(H, D, W)
    lin_k = np.zeros((H, W, D), np.float32)
    lin_v = np.zeros((H, W, D), np.float32)
    total, pos, n_valid = 0, 0, 0
    for step in range(steps):
        k, v = inputs.np_chunk(shape, step)
        oracle.write(ring, total, pos, k, v)
        lin_k, lin_v, lin = oracle.naive(lin_k, lin_v, k, v, n_valid, pos)
        total += N
        pos += N
        n_valid = min(n_valid + N, W)
        if step in check_steps:
            start = oracle.slot_of_token(total - n_valid, W)
            idx = (start + np.arange(n_valid)) % W
            for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
                a = getattr(lin, name)[:, :n_valid]
                b = getattr(ring, name)[:, idx]
                assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8)), (step, name)
    return ring


def test_write_equals_naive_tiny():
    _run_write_vs_naive(inputs.TINY, 8, set(range(8)))


def test_write_equals_naive_wrap_mid_chunk():
    _run_write_vs_naive(inputs.TINY_WRAP, 16, set(range(16)))


@pytest.mark.slow
def test_write_equals_naive_page_shape_small_window():
    s = inputs.Shape("test", 1, 3, 128, 5788 // 4, 757 // 4)
    _run_write_vs_naive(s, 9, {5, 6, 8})


# ---------------------------------------------------------------------------
# rebase
# ---------------------------------------------------------------------------
def _filled_cache(shape, steps, workload="test"):
    H, D, W, N = shape.n_heads, shape.head_dim, shape.window, shape.n_new
    c = oracle.LayerCache(H, D, W)
    total = 0
    for step in range(steps):
        k, v = inputs.np_chunk(shape, step, workload=workload)
        oracle.write(c, total, total, k, v)
        total += N
    n_valid = min(total, W)
    start = oracle.slot_of_token(total - n_valid, W)
    return c, start, n_valid, total


def _row_bound(c, n_quant):
    # one requantisation moves a scaled element by at most half an ulp of the
    # top binade, 16 codes = absmax / 28; a rotation of an error pair keeps its norm
    a = np.abs(oracle.dequant_rows(c.k_codes, c.k_scales)).max(axis=-1, keepdims=True)
    return a * (n_quant * np.sqrt(2.0) / 28.0) * 1.001 + 1e-6


def test_rebase_round_trip():
    shp = inputs.TINY_WRAP
    c, start, n_valid, _ = _filled_cache(shp, 9)
    x0 = oracle.dequant_rows(c.k_codes, c.k_scales)
    c2 = c.copy()
    oracle.rebase(c2, start, n_valid, 12345)
    oracle.rebase(c2, start, n_valid, -12345)
    x2 = oracle.dequant_rows(c2.k_codes, c2.k_scales)
    assert np.all(np.abs(x2 - x0) <= _row_bound(c, 2))
    # V untouched, and the rebase really moved K in between
    c3 = c.copy()
    oracle.rebase(c3, start, n_valid, 12345)
    assert np.array_equal(c3.v_codes, c.v_codes) and np.array_equal(c3.v_scales, c.v_scales)
    assert not np.array_equal(c3.k_codes, c.k_codes)


def test_rebase_composes():
    c, start, n_valid, _ = _filled_cache(inputs.TINY, 8)
    a = c.copy()
    oracle.rebase(a, start, n_valid, 1000)
    oracle.rebase(a, start, n_valid, 31)
    b = c.copy()
    oracle.rebase(b, start, n_valid, 1031)
    xa = oracle.dequant_rows(a.k_codes, a.k_scales)
    xb = oracle.dequant_rows(b.k_codes, b.k_scales)
    assert np.all(np.abs(xa - xb) <= _row_bound(c, 3))


def test_rebase_tracks_naive_rotation():
    """Ring after a reset vs re-rotating the raw keys at p - delta."""
    shp = inputs.TINY
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    c = oracle.LayerCache(H, D, W)
    raw = []
    for step in range(4):
        k, v = inputs.np_chunk(shp, step)
        oracle.write(c, step * N, step * N, k, v)
        raw.append(k)
    delta = 64
    n_valid, start = 4 * N, 0
    oracle.rebase(c, start, n_valid, delta)
    kraw = np.concatenate(raw)                                  # [64][H][D], positions 0..63
    want = oracle.rope_rows(kraw, (np.arange(4 * N) - delta)[:, None], 10000.0)
    wc, ws = oracle.quant_rows(want)
    got = oracle.dequant_rows(c.k_codes[:, :n_valid], c.k_scales[:, :n_valid]).transpose(1, 0, 2)
    ref = oracle.dequant_rows(wc, ws)
    a = np.maximum(np.abs(got).max(-1, keepdims=True), np.abs(ref).max(-1, keepdims=True))
    assert np.all(np.abs(got - ref) <= a * (np.sqrt(2.0) + 2.0) / 28.0 * 1.001 + 1e-6)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _tiny_state(steps=6, shape=inputs.TINY_WRAP):
    c, start, n_valid, total = _filled_cache(shape, steps)
    q = inputs.np_queries(shape, steps, 0, workload="test")
    return c, start, n_valid, total, q


def test_attention_matches_dense_fp64():
    for steps in (1, 3, 7, 9):
        c, start, n_valid, total, q = _tiny_state(steps)
        qpos = total - 16
        out = oracle.attention(c, start, n_valid, q, qpos)
        k, v = oracle.window_dequant(c, start, n_valid)
        qr = oracle.rope_rows(q, (qpos + np.arange(q.shape[0]))[:, None])
        ref = oracle.dense_attention(qr, k, v, 1.0 / np.sqrt(c.D))
        assert np.abs(out - ref).max() < 1e-12


def test_dense_matches_library_routines():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 3, 16))
    k = rng.standard_normal((3, 11, 16))
    v = rng.standard_normal((3, 11, 16))
    sc = 0.3
    ref = oracle.dense_attention(q, k, v, sc)
    p = scipy.special.softmax(np.einsum("qhd,hkd->hqk", q, k) * sc, axis=-1)
    alt = np.einsum("hqk,hkd->qhd", p, v)
    assert np.abs(ref - alt).max() < 1e-13
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2)).contiguous(), torch.from_numpy(k),
        torch.from_numpy(v), scale=sc).numpy().transpose(1, 0, 2)
    assert np.abs(ref - t).max() < 1e-13


def test_attention_closed_forms():
    c, start, n_valid, total, q = _tiny_state(9)
    k, v = oracle.window_dequant(c, start, n_valid)
    # one valid key: the output is that key's value row
    out1 = oracle.attention(c, start, 1, q, total - 16)
    assert np.abs(out1 - v[:, 0][None]).max() < 1e-15
    # zero query: uniform weights -> mean of the value rows
    out0 = oracle.attention(c, start, n_valid, np.zeros_like(q), total - 16)
    assert np.abs(out0 - v.astype(np.float64).mean(axis=1)[None]).max() < 1e-12
    # all keys equal: uniform weights again
    ce = c.copy()
    idx = (start + np.arange(n_valid)) % c.W
    ce.k_codes[:, idx] = c.k_codes[:, idx[:1]]
    ce.k_scales[:, idx] = c.k_scales[:, idx[:1]]
    oute = oracle.attention(ce, start, n_valid, q, total - 16)
    assert np.abs(oute - v.astype(np.float64).mean(axis=1)[None]).max() < 1e-12
    # weights sum to one: all value rows equal to 1.0 give outputs of exactly ~1
    c1 = c.copy()
    c1.v_codes[:] = 0x7E
    c1.v_scales[:] = np.float32(1.0 / 448.0)
    out_one = oracle.attention(c1, start, n_valid, q, total - 16)
    assert np.abs(out_one - 1.0).max() < 1e-12


def test_attention_rows_subset_matches_full():
    c, start, n_valid, total, q = _tiny_state(9)
    full = oracle.attention(c, start, n_valid, q, total - 16)
    rows = [(0, 0), (5, 1), (15, 1), (3, 0)]
    sub = oracle.attention(c, start, n_valid, q, total - 16, rows=rows)
    for t, (i, h) in enumerate(rows):
        assert np.array_equal(sub[t], full[i, h])
