"""Pins of the oracle's 3-D (t, y, x) rotary encoding, its per-axis rebase and
attention with 3-D query coordinates (no GPU).

The 3-D form cuts the D/2 interleaved pairs into a frame, a row and a column
group; group a is the 1-D rotary rule of its slice at that axis's coordinate.
Pins: with all pairs in the frame group it is the 1-D encoding bit for bit
(the 1-D encoding is itself pinned to a third-party rotary implementation);
each group equals the 1-D encoding of its slice alone, at its coordinate, bit
for bit; a group whose coordinate is zero is left unchanged; R(-d) R(c) =
R(c - d) per axis in fp32 to 1e-5; q.k depends only on coordinate offsets,
axis by axis; a frame-only rebase tracks re-rotating the raw keys at t - d
within the requantisation bound, is the 1-D rebase bit for bit when all pairs
are temporal, and leaves attention unchanged when the queries move too.
"""
import numpy as np
import pytest

import oracle
from kv_cache_attention_ring_amd import inputs

BASE = 10000.0


def _coords(rng, n, tmax=40000, smax=64):
    return np.stack([rng.integers(-tmax, tmax, n), rng.integers(0, smax, n), rng.integers(0, smax, n)],
                    axis=1).astype(np.int64)


@pytest.mark.parametrize("D", [64, 128])
def test_all_temporal_split_is_the_1d_encoding(D):
    rng = np.random.default_rng(11)
    n = 500
    x = rng.standard_normal((n, D)).astype(np.float32)
    c = _coords(rng, n)
    got = oracle.rope3d_rows(x, c, (D // 2, 0, 0), BASE)
    want = oracle.rope_rows(x, c[:, 0], BASE)
    assert np.array_equal(got, want)
    cs3 = oracle.rope3d_cs(c, D, (D // 2, 0, 0), BASE)
    assert np.array_equal(cs3, oracle.rope_cs(c[:, 0], D, BASE))


@pytest.mark.parametrize("D", [64, 128])
def test_each_group_is_the_1d_encoding_of_its_slice(D):
    rng = np.random.default_rng(12)
    n = 400
    x = rng.standard_normal((n, D)).astype(np.float32)
    c = _coords(rng, n)
    npr = inputs.axis_pairs(D)
    got = oracle.rope3d_rows(x, c, npr, BASE)
    lo = 0
    for a, na in enumerate(npr):
        sl = slice(2 * lo, 2 * (lo + na))
        want = oracle.rope_rows(np.ascontiguousarray(x[:, sl]), c[:, a], BASE)
        assert np.array_equal(got[:, sl], want), a
        lo += na


def test_zero_coordinate_leaves_its_group_unchanged():
    rng = np.random.default_rng(13)
    D, n = 128, 300
    npr = inputs.axis_pairs(D)
    x = rng.standard_normal((n, D)).astype(np.float32)
    c = _coords(rng, n)
    c[:, 1:] = 0
    y = oracle.rope3d_rows(x, c, npr, BASE)
    t_dims = 2 * npr[0]
    assert np.array_equal(y[:, t_dims:], x[:, t_dims:])
    assert not np.array_equal(y[:, :t_dims], x[:, :t_dims])
    c2 = _coords(rng, n)
    c2[:, 0] = 0
    y2 = oracle.rope3d_rows(x, c2, npr, BASE)
    assert np.array_equal(y2[:, :t_dims], x[:, :t_dims])


def test_group_identity_per_axis_fp32():
    rng = np.random.default_rng(14)
    D, n = 128, 3000
    npr = inputs.axis_pairs(D)
    x = rng.standard_normal((n, D)).astype(np.float32)
    c = _coords(rng, n, tmax=37583)
    d = np.stack([rng.integers(1, 31795, n), rng.integers(-40, 40, n), rng.integers(-40, 40, n)], axis=1)
    a = oracle.rope3d_rows(oracle.rope3d_rows(x, c, npr, BASE), -d, npr, BASE)
    b = oracle.rope3d_rows(x, c - d, npr, BASE)
    assert np.abs(a - b).max() <= 1e-5


def test_relative_coordinate_invariance_per_axis():
    rng = np.random.default_rng(15)
    D, n = 128, 200
    npr = inputs.axis_pairs(D)
    q = rng.standard_normal((n, D)).astype(np.float32)
    k = rng.standard_normal((n, D)).astype(np.float32)
    cq, ck = _coords(rng, n, tmax=2000), _coords(rng, n, tmax=2000)
    s0 = (oracle.rope3d_rows(q, cq, npr, BASE).astype(np.float64) *
          oracle.rope3d_rows(k, ck, npr, BASE)).sum(-1)
    for a in range(3):
        sh = np.zeros(3, np.int64)
        sh[a] = 777
        s1 = (oracle.rope3d_rows(q, cq + sh, npr, BASE).astype(np.float64) *
              oracle.rope3d_rows(k, ck + sh, npr, BASE)).sum(-1)
        assert np.abs(s1 - s0).max() <= 1e-4, a


def _filled3d(shape, steps, npr):
    H, D, W, N = shape.n_heads, shape.head_dim, shape.window, shape.n_new
    c = oracle.LayerCache(H, D, W)
    raw, coords = [], []
    for s in range(steps):
        k, v = inputs.np_chunk(shape, s)
        cc = inputs.chunk_coords(N, s, cols=5)
        oracle.write3d(c, s * N, cc, npr, k, v, BASE)
        raw.append(k)
        coords.append(cc)
    return c, np.concatenate(raw), np.concatenate(coords)


def test_write3d_with_all_temporal_pairs_is_the_1d_write():
    shp = inputs.TINY_WRAP
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    a, b = oracle.LayerCache(H, D, W), oracle.LayerCache(H, D, W)
    for s in range(9):
        k, v = inputs.np_chunk(shp, s)
        coords = np.stack([s * N + np.arange(N), np.full(N, 3), np.full(N, 5)], axis=1)
        oracle.write3d(a, s * N, coords, (D // 2, 0, 0), k, v, BASE)
        oracle.write(b, s * N, s * N, k, v, BASE)
    for f in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    oracle.rebase3d(a, 0, W, (17, 0, 0), (D // 2, 0, 0), BASE)
    oracle.rebase(b, 0, W, 17, BASE)
    assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.k_scales, b.k_scales)


def test_frame_rebase_tracks_rerotation_at_t_minus_delta():
    shp = inputs.TINY
    D, N = shp.head_dim, shp.n_new
    npr = inputs.axis_pairs(D)
    steps = 4
    c, kraw, coords = _filled3d(shp, steps, npr)
    n_valid = steps * N
    c0 = c.copy()
    oracle.rebase3d(c, 0, n_valid, (3, 0, 0), npr, BASE)
    # V untouched, K moved
    assert np.array_equal(c.v_codes, c0.v_codes) and not np.array_equal(c.k_codes, c0.k_codes)
    want = oracle.rope3d_rows(kraw, np.repeat((coords - [3, 0, 0])[:, None, :], shp.n_heads, 1), npr, BASE)
    wc, ws = oracle.quant_rows(want)
    got = oracle.dequant_rows(c.k_codes[:, :n_valid], c.k_scales[:, :n_valid]).transpose(1, 0, 2)
    ref = oracle.dequant_rows(wc, ws)
    amax = np.maximum(np.abs(got).max(-1, keepdims=True), np.abs(ref).max(-1, keepdims=True))
    assert np.all(np.abs(got - ref) <= amax * (np.sqrt(2.0) + 2.0) / 28.0 * 1.001 + 1e-6)


def test_attention3d_all_temporal_is_1d_and_frame_rebase_keeps_outputs():
    shp = inputs.TINY
    H, D, N = shp.n_heads, shp.head_dim, shp.n_new
    # all pairs temporal at t = position: the 1-D attention bit for bit
    c = oracle.LayerCache(H, D, shp.window)
    for s in range(3):
        k, v = inputs.np_chunk(shp, s)
        oracle.write(c, s * N, s * N, k, v, BASE)
    q = inputs.np_queries(shp, 3, 0, workload="test")
    qc = np.stack([2 * N + np.arange(N), np.zeros(N), np.zeros(N)], axis=1)
    a = oracle.attention3d(c, 0, 3 * N, q, qc, (D // 2, 0, 0))
    b = oracle.attention(c, 0, 3 * N, q, 2 * N)
    assert np.array_equal(a, b)
    # 3-D split: a frame rebase by d with the queries moved by -d in t keeps outputs
    npr = inputs.axis_pairs(D)
    c3, _, coords = _filled3d(shp, 4, npr)
    qc3 = coords[-N:]
    before = oracle.attention3d(c3, 0, 4 * N, q, qc3, npr)
    oracle.rebase3d(c3, 0, 4 * N, (5, 0, 0), npr, BASE)
    after = oracle.attention3d(c3, 0, 4 * N, q, qc3 - [5, 0, 0], npr)
    err = np.abs(after - before)
    # the rebase requantises every key (each element moves by up to
    # (sqrt 2 + 2)/28 of its row's largest one): on this 64-key window the
    # outputs agree to twice the attention bound
    assert err.max() <= 4e-2 and err.mean() <= 4e-3
    # the check separates: a rebase in the wrong direction is far outside it
    c5 = c3.copy()
    oracle.rebase3d(c5, 0, 4 * N, (-10, 0, 0), npr, BASE)      # net +5 from the original
    wrong = np.abs(oracle.attention3d(c5, 0, 4 * N, q, qc3 - [5, 0, 0], npr) - before)
    assert wrong.mean() > 10 * err.mean()
    # and with no shift at all the queries see exactly the same scores
    c4 = c3.copy()
    oracle.rebase3d(c4, 0, 4 * N, (0, 0, 0), npr, BASE)
    assert np.array_equal(c4.k_codes, c3.k_codes) and np.array_equal(c4.k_scales, c3.k_scales)


# ---------------------------------------------------------------------------
# a fixed prefix beside the ring (explicit slot lists)
# ---------------------------------------------------------------------------
def test_slot_lists_reduce_to_the_ring_functions():
    """With no prefix and the ring's slots in logical order, the list forms are
    the ring forms bit for bit."""
    shp = inputs.TINY_WRAP
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    npr = inputs.axis_pairs(D)
    a, b = oracle.LayerCache(H, D, W), oracle.LayerCache(H, D, W)
    pr = oracle.PrefixRing(W, 0)
    for s in range(9):
        k, v = inputs.np_chunk(shp, s)
        cc = inputs.chunk_coords(N, s, cols=5)
        oracle.write3d_list(a, pr.write(N), cc, npr, k, v)
        oracle.write3d(b, s * N, cc, npr, k, v)
    for f in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    start, n_valid = pr.ring_slots()[0], pr.ring.n_valid
    q = inputs.np_queries(shp, 9, 0, workload="test")
    x = oracle.attention3d_list(a, pr.key_slots(), q, cc, npr)
    y = oracle.attention3d(b, start, n_valid, q, cc, npr)
    assert np.array_equal(x, y)
    oracle.rebase3d_list(a, pr.ring_slots(), (4, 0, 0), npr)
    oracle.rebase3d(b, start, n_valid, (4, 0, 0), npr)
    assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.k_scales, b.k_scales)


def test_prefix_ring_slots_and_key_order_invariance():
    W, P, N = 100, 12, 16
    pr = oracle.PrefixRing(W, P)
    seen = []
    for _ in range(12):
        new = pr.write(N)
        assert all(P <= s < W for s in new)
        seen += new
    # the ring holds the last W - P tokens in slots P + (t mod (W - P))
    assert seen == [P + t % (W - P) for t in range(12 * N)]
    ks = pr.key_slots()
    assert ks[:P] == list(range(P)) and sorted(ks) == list(range(W))
    # attention over a set of keys does not depend on their order
    rng = np.random.default_rng(21)
    H, D = 2, 64
    c = oracle.LayerCache(H, D, W)
    c.k_codes[:] = rng.integers(0, 0x7F, c.k_codes.shape).astype(np.uint8) & 0x77
    c.v_codes[:] = rng.integers(0, 0xFF, c.v_codes.shape).astype(np.uint8) & 0xF7
    c.k_scales[:] = rng.uniform(0.001, 0.005, c.k_scales.shape)
    c.v_scales[:] = rng.uniform(0.001, 0.005, c.v_scales.shape)
    q = rng.standard_normal((5, H, D)).astype(np.float32)
    qc = np.stack([np.arange(5), np.zeros(5), np.arange(5)], 1)
    npr = inputs.axis_pairs(D)
    a = oracle.attention3d_list(c, ks, q, qc, npr)
    b = oracle.attention3d_list(c, rng.permutation(ks), q, qc, npr)
    assert np.abs(a - b).max() <= 1e-12


def test_frame_rebase_leaves_the_prefix():
    shp = inputs.TINY
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    P = 10
    npr = inputs.axis_pairs(D)
    c = oracle.LayerCache(H, D, W)
    pr = oracle.PrefixRing(W, P)
    kp, vp = inputs.np_chunk(shp, 99)
    oracle.write3d_list(c, range(P), np.stack([np.full(P, -1), np.arange(P) // 5, np.arange(P) % 5], 1),
                        npr, kp[:P], vp[:P])
    for s in range(3):
        k, v = inputs.np_chunk(shp, s)
        oracle.write3d_list(c, pr.write(N), inputs.chunk_coords(N, s, cols=5), npr, k, v)
    before = c.copy()
    oracle.rebase3d_list(c, pr.ring_slots(), (3, 0, 0), npr)
    assert np.array_equal(c.k_codes[:, :P], before.k_codes[:, :P])
    assert np.array_equal(c.k_scales[:, :P], before.k_scales[:, :P])
    assert not np.array_equal(c.k_codes[:, P:], before.k_codes[:, P:])
