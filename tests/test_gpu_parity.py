"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case feeds both sides the same seeded inputs and compares element by
element with the bars in tests/_parity.py.  Cases:
  * rotary table, E4M3 conversion sweep (ties, subnormals, saturation edge);
  * the small workload end to end (1 layer, 2 heads, D 64, W 96, N 16; 8 steps,
    reset by 64 after step 4), ring and naive paths, 4 attention passes per
    step, one and two key splits; a W = 100 variant whose chunks wrap mid-chunk;
  * one attention layer at the production shape (12 heads, D 128, W 5788,
    N 757): all writes, 4 passes on sampled queries of every head, default and
    single split, determinism, the naive path, the rebase;
  * the key tiles dealt to the splits: a W = 1000 window (2 heads, D 64, 37
    queries) at 11 lengths around tile boundaries, with 1 to 16 splits;
  * the 60-layer batched write of a full step (sampled layers), and the full-
    step configuration the benchmark times: 42 steps of 60-layer writes, all
    4 passes of layers 0 and 59 at steps 1 and 42, then the 60-layer rebase;
  * 20 heads (more rows per write workgroup than it has row groups), chunks of
    33 tokens wrapping mid-chunk;
  * edge cases: ring not yet full, one valid key, one query, ragged query
    counts, fp32 inputs at D 128, all-zero rows, scores that grow along the
    window past the lazy-rescale threshold, a chunk as large as the window
    (also wrapping from a non-zero head) and 3000 queries over it.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_ring_amd import inputs
from kv_cache_attention_ring_amd import kvring as K

from _parity import assert_attention, assert_codes, assert_scales, logical_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    K.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().cpu().numpy()


def _f32(t):
    return t.detach().float().cpu().numpy()


# ---------------------------------------------------------------------------
def test_rope_table_matches_oracle():
    for D in (64, 128):
        _say(f"rope table D={D}")
        pos0, n = -200, 40000
        t = K.RopeTable(pos0, n, D)
        torch.cuda.synchronize()
        got = _np(t.cs)
        sel = np.concatenate([np.arange(0, 400), np.random.default_rng(D).integers(0, n, 3000)])
        want = oracle.rope_cs(pos0 + sel, D)
        g = got[sel]
        same = (g.view(np.uint32) == want.view(np.uint32)).mean()
        ulps = np.abs(g.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        assert same >= 0.9999 and ulps.max() <= 1, (same, ulps.max())


def test_row_magnitudes_through_write():
    """Rows whose absmax runs from 448 * 2^-100 to 448 * 2^100 (each power of
    two, and one fp32 step either side): codes and scales (IEEE divisions
    a / 448 and 448 / a) bit-exact against the oracle."""
    _say("row magnitudes")
    D = 64
    heads = []
    for j in range(-100, 101):
        b = np.float32(448.0 * 2.0 ** j)
        heads += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    heads = np.array(heads, np.float32)
    n = heads.size
    rng = np.random.default_rng(17)
    v = (rng.uniform(-1, 1, (n, D)) * heads[:, None]).astype(np.float32)
    v[:, 0] = np.where(rng.random(n) < 0.5, heads, -heads)
    v = np.where(np.abs(v) <= np.abs(v[:, :1]), v, v[:, :1]).astype(np.float32)
    H, W = 1, n
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(0, n, D)
    k = torch.zeros((n, H, D), dtype=torch.float32, device="cuda")
    vt = torch.from_numpy(v).view(n, H, D).cuda()
    K.kv_write_rope_quant(cache, K.kvr_ring_init(), 0, k, vt, rope)
    torch.cuda.synchronize()
    want_c, want_s = oracle.quant_rows(v)
    got_s = _np(cache.v_scales)[0, 0]
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), \
        np.argwhere(got_s.view(np.uint32) != want_s.view(np.uint32))[:5]
    got_c = _np(cache.v_codes)[0, 0]
    assert np.array_equal(got_c, want_c), np.argwhere(got_c != want_c)[:5]


def _tiny_head_rows(lo, hi, D, rng):
    heads = []
    for j in range(lo, hi):
        b = np.float32(2.0 ** j)
        heads += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    heads = np.array([h for h in heads if h > 0], np.float32)
    n = heads.size
    v = (rng.uniform(-1, 1, (n, D)) * heads[:, None].astype(np.float64)).astype(np.float32)
    v[:, 0] = np.where(rng.random(n) < 0.5, heads, -heads)
    return np.where(np.abs(v) <= np.abs(v[:, :1]), v, v[:, :1]).astype(np.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tiny_rows_through_write_and_rebase(dtype):
    """Rows whose absmax runs down to the smallest denormal of the input type
    (fp32 2^-149, bf16 2^-133), where the fp32 inverse 448 / absmax overflows:
    codes and scales bit-exact against the oracle, no NaN code, finite decoded
    values; the same rows as K at position 0 (identity rotation) through the
    rebase by +-1 (dequantise, rotate, re-quantise) against the oracle too."""
    lo = -149 if dtype == torch.float32 else -133
    _say(f"tiny rows {dtype}")
    D = 128
    v32 = _tiny_head_rows(lo, -59, D, np.random.default_rng(23))
    vt = torch.from_numpy(v32).to(dtype)
    v = _f32(vt)                                          # the values the kernel sees
    n = v.shape[0]
    cache = K.KVCache(1, 1, D, n)
    rope = K.RopeTable(-4, n + 8, D)
    # every row as token 0 of its own one-token chunk: K at position 0
    for i in range(n):
        ring = K.kvr_ring(i, i, 0)
        K.kv_write_rope_quant(cache, ring, 0, vt[i:i + 1].view(1, 1, D).cuda(), vt[i:i + 1].view(1, 1, D).cuda(),
                              rope)
    torch.cuda.synchronize()
    # K goes through the rotation at position 0 (cos 1, sin 0: the values stay,
    # but a -0 element can come out as +0), V does not
    want = {"k": oracle.quant_rows(oracle.rope_rows(v, 0)), "v": oracle.quant_rows(v)}
    for name in ("k", "v"):
        want_c, want_s = want[name]
        got_c = _np(getattr(cache, f"{name}_codes"))[0, 0]
        got_s = _np(getattr(cache, f"{name}_scales"))[0, 0]
        assert not np.any((got_c & 0x7F) == 0x7F), f"{name}: NaN code"
        assert np.array_equal(got_c, want_c), (name, np.argwhere(got_c != want_c)[:5])
        assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), name
        assert np.isfinite(oracle.dequant_rows(got_c, got_s)).all()
    orc = oracle.LayerCache(1, D, n)
    orc.k_codes[0], orc.k_scales[0] = want["k"]
    ring = K.kvr_ring(0, n, 1)
    for delta in (1, -1):
        K.kv_delta_rebase(cache, ring, 0, 1, delta)
        oracle.rebase(orc, 0, n, delta)
        torch.cuda.synchronize()
        got_c = _np(cache.k_codes)[0, 0]
        assert not np.any((got_c & 0x7F) == 0x7F), f"rebase {delta}: NaN code"
        assert_codes(got_c, orc.k_codes[0], f"tiny rebase {delta}")
        assert_scales(_np(cache.k_scales)[0, 0], orc.k_scales[0], f"tiny rebase {delta}")


def test_large_values_through_split_partials():
    """V rows near 1e6 (fp32 inputs): outputs of that size overflow an fp16
    partial row unless it carries its own power-of-two exponent; one split,
    several and the default all match the oracle (compared at the data's
    scale: attention is linear in V) and each other within bf16 rounding."""
    shp = inputs.Shape("test", 1, 3, 128, 1100, 600)
    run = SmallRun(shp, dtype=torch.float32)
    for step in range(2):
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v * 1e6)
    q = inputs.np_queries(shp, 1, 0)
    outs = {}
    for splits in (1, 4, 0):
        _say(f"large values, splits={splits}")
        got, ref = run.attention(q, n_splits=splits, naive_too=False)
        assert np.isfinite(got).all(), f"splits={splits}: non-finite output"
        assert np.abs(ref).max() > 65504.0                   # past the fp16 range
        assert_attention(got / 1e6, ref / 1e6, f"large values, splits {splits}")
        outs[splits] = got
    # against the single-split rows, relative to each row's largest element
    row_max = np.abs(outs[1]).max(axis=-1, keepdims=True)
    for splits in (4, 0):
        d = np.abs(outs[splits] - outs[1]) / row_max
        assert d.max() <= 2.0 ** -7, (splits, d.max())


def test_call_on_a_side_stream_without_its_context():
    """attn_fp8_window on an explicit stream that is not the current one, with
    the binding allocating the output and the workspace: same bits as the call
    on the current stream."""
    shp = inputs.Shape("test", 1, 3, 128, 1100, 600)
    run = SmallRun(shp, dtype=torch.bfloat16)
    for step in range(2):
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
    q = torch.from_numpy(inputs.np_queries(shp, 1, 2)).to(torch.bfloat16).cuda()
    W = shp.window
    start = K.kvr_ring_logical_start(run.ring, W)
    want = K.attn_fp8_window(run.cache, 0, start, run.ring.n_valid, q, run.ring.pos_next - 600, run.rope.base,
                             n_splits=4)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(3):
        _say(f"side stream call {i}")
        outs.append(K.attn_fp8_window(run.cache, 0, start, run.ring.n_valid, q, run.ring.pos_next - 600,
                                      run.rope.base, n_splits=4, stream=side))
        # work on the current stream that allocates while the side stream runs
        junk = torch.full((1 << 20,), 3.0, device="cuda")
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, want)


def test_e4m3_conversion_sweep_through_write():
    """V rows whose absmax is 448 are encoded without scaling (448/448 = 1)."""
    _say("e4m3 sweep")
    codes = np.arange(0x7F, dtype=np.uint8)
    tv = np.sort(oracle.e4m3_decode(codes)).astype(np.float32)
    mids = ((tv[1:].astype(np.float64) + tv[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([tv, mids, np.nextafter(mids, np.float32(1e9)),
                           np.nextafter(mids, np.float32(-1e9)),
                           np.random.default_rng(3).uniform(-448, 448, 4000).astype(np.float32),
                           np.array([1e-12, 2e-4, 447.99, 448.0], np.float32)])
    vals = np.concatenate([vals, -vals])
    D = 128
    per = D - 1
    n = (vals.size + per - 1) // per
    rows = np.zeros((n, per), np.float32)
    rows.ravel()[: vals.size] = vals
    v = np.concatenate([np.full((n, 1), 448.0, np.float32), rows], axis=1)      # [n][D]
    H, W = 1, n
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(0, n, D)
    k = torch.zeros((n, H, D), dtype=torch.float32, device="cuda")
    vt = torch.from_numpy(v).view(n, H, D).cuda()
    K.kv_write_rope_quant(cache, K.kvr_ring_init(), 0, k, vt, rope)
    torch.cuda.synchronize()
    got = _np(cache.v_codes)[0, 0]
    want = oracle.e4m3_encode(v)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    assert np.all(_np(cache.v_scales) == np.float32(1.0))
    # all-zero K rows: scale 0, zero codes
    assert not _np(cache.k_codes).any() and not _np(cache.k_scales).any()


# ---------------------------------------------------------------------------
class SmallRun:
    """Ring path, naive path and oracle side by side on one layer."""

    def __init__(self, shape, dtype=torch.float32, table=(-256, 4096)):
        self.s = shape
        H, D, W = shape.n_heads, shape.head_dim, shape.window
        self.dtype = dtype
        self.cache = K.KVCache(1, H, D, W)
        self.ring = K.kvr_ring_init()
        self.rope = K.RopeTable(table[0], table[1], D)
        self.lin = [torch.zeros((H, W, D), dtype=dtype, device="cuda") for _ in range(4)]
        self.ping = 0
        self.lc = torch.zeros((H, W, D), dtype=torch.uint8, device="cuda")
        self.lv = torch.zeros((H, W, D), dtype=torch.uint8, device="cuda")
        self.lks = torch.zeros((H, W), dtype=torch.float32, device="cuda")
        self.lvs = torch.zeros((H, W), dtype=torch.float32, device="cuda")
        self.orc = oracle.LayerCache(H, D, W)
        # the oracle's own bookkeeping, independent of the library's ring: the
        # number of tokens written and the sum of the position resets
        self.total = 0
        self.shift = 0

    # reference window state from the token count alone (the oracle's t mod W
    # slot rule): valid keys, oldest slot, next position
    def ref_n_valid(self):
        return min(self.total, self.s.window)

    def ref_start(self):
        return oracle.slot_of_token(self.total - self.ref_n_valid(), self.s.window)

    def ref_pos_next(self):
        return self.total - self.shift

    def check_ring(self):
        """The library's ring state equals the reference bookkeeping."""
        assert (self.ring.n_valid, K.kvr_ring_logical_start(self.ring, self.s.window), self.ring.pos_next) == \
            (self.ref_n_valid(), self.ref_start(), self.ref_pos_next()), self.ring

    def step(self, k, v):
        """k, v: fp32 numpy [N][H][D]."""
        s = self.s
        kd = torch.from_numpy(k).to(self.dtype).cuda()
        vd = torch.from_numpy(v).to(self.dtype).cuda()
        kf, vf = _f32(kd), _f32(vd)
        src_k, src_v = self.lin[2 * self.ping], self.lin[2 * self.ping + 1]
        dst_k, dst_v = self.lin[2 * (1 - self.ping)], self.lin[2 * (1 - self.ping) + 1]
        K.naive_upkeep(src_k, src_v, kd, vd, self.ring.n_valid, self.ring.pos_next, self.rope,
                       dst_k, dst_v, self.lc, self.lv, self.lks, self.lvs)
        self.ping = 1 - self.ping
        K.kv_write_rope_quant(self.cache, self.ring, 0, kd, vd, self.rope)
        oracle.write(self.orc, self.total, self.ref_pos_next(), kf, vf)
        K.kvr_ring_after_write(self.ring, s.window, k.shape[0])
        self.total += k.shape[0]
        self.check_ring()

    def write_pass(self, k, v, before, total_before):
        """Write a chunk again from the step-start ring state `before` (the
        same slots and positions as that step's first write); the ring path
        and the oracle only."""
        kd = torch.from_numpy(k).to(self.dtype).cuda()
        vd = torch.from_numpy(v).to(self.dtype).cuda()
        K.kv_write_rope_quant(self.cache, before, 0, kd, vd, self.rope)
        oracle.write(self.orc, total_before, total_before - self.shift, _f32(kd), _f32(vd))

    def rebase(self, delta):
        K.kv_delta_rebase(self.cache, self.ring, 0, 1, delta)
        oracle.rebase(self.orc, self.ref_start(), self.ref_n_valid(), delta)
        K.kvr_ring_after_rebase(self.ring, delta)
        self.shift += delta
        self.check_ring()

    def check_cache(self, what, naive_too=True):
        torch.cuda.synchronize()
        for name in ("k", "v"):
            assert_codes(_np(getattr(self.cache, f"{name}_codes"))[0],
                         getattr(self.orc, f"{name}_codes"), f"{what} ring {name} codes")
            assert_scales(_np(getattr(self.cache, f"{name}_scales"))[0],
                          getattr(self.orc, f"{name}_scales"), f"{what} ring {name} scales")
        if naive_too:
            W, n = self.s.window, self.ref_n_valid()
            start = self.ref_start()
            for ring_t, lin_t in ((self.cache.k_codes, self.lc), (self.cache.v_codes, self.lv),
                                  (self.cache.k_scales, self.lks), (self.cache.v_scales, self.lvs)):
                r = logical_rows(_np(ring_t)[0], start, n, W)
                l = _np(lin_t)[:, :n]
                assert np.array_equal(np.ascontiguousarray(r).view(np.uint8),
                                      np.ascontiguousarray(l).view(np.uint8)), f"{what}: ring != naive"

    def attention(self, q, n_splits=0, naive_too=True, ws=None):
        """q fp32 numpy [n_q][H][D]; returns (gpu bf16 as fp32, oracle fp64)."""
        W = self.s.window
        qd = torch.from_numpy(q).to(self.dtype).cuda()
        n_q = q.shape[0]
        # the library call takes its arguments from the library's ring; the
        # oracle below from the reference bookkeeping
        out = K.attn_fp8_window(self.cache, 0, K.kvr_ring_logical_start(self.ring, W), self.ring.n_valid, qd,
                                self.ring.pos_next - n_q, self.rope.base, n_splits=n_splits, ws=ws)
        if naive_too:
            lin_cache = K.KVCache(1, self.s.n_heads, self.s.head_dim, W)
            lin_cache.k_codes[0].copy_(self.lc)
            lin_cache.v_codes[0].copy_(self.lv)
            lin_cache.k_scales[0].copy_(self.lks)
            lin_cache.v_scales[0].copy_(self.lvs)
            out_lin = K.attn_fp8_window(lin_cache, 0, 0, self.ring.n_valid, qd, self.ring.pos_next - n_q,
                                        self.rope.base, n_splits=n_splits, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(out, out_lin), "ring and naive attention differ"
        torch.cuda.synchronize()
        ref = oracle.attention(self.orc, self.ref_start(), self.ref_n_valid(), _f32(qd), self.ref_pos_next() - n_q)
        return _f32(out), ref


def test_small_workload_end_to_end():
    shp = inputs.TINY
    run = SmallRun(shp)
    for step in range(8):
        _say(f"small step {step}")
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
        run.check_cache(f"step {step}", naive_too=step < 4)
        for p in range(shp.passes):
            q = inputs.np_queries(shp, step, p)
            got, ref = run.attention(q, n_splits=1 + (p % 2), naive_too=step < 4)
            assert_attention(got, ref, f"step {step} pass {p}")
        if step == 3:
            _say("small rebase by 64")
            run.rebase(64)
            run.check_cache("after rebase", naive_too=False)


def test_wrap_mid_chunk():
    shp = inputs.TINY_WRAP
    run = SmallRun(shp)
    for step in range(16):
        _say(f"wrap step {step}")
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
        run.check_cache(f"wrap step {step}")
        if step in (0, 6, 7, 15):
            got, ref = run.attention(inputs.np_queries(shp, step, 0), n_splits=0)
            assert_attention(got, ref, f"wrap step {step}")


@pytest.mark.parametrize("D,dtype", [(64, torch.bfloat16), (128, torch.float32)])
def test_many_heads_odd_chunks(D, dtype):
    """20 heads: a two-token run of the write is 40 rows, more than one pass of
    the workgroup's 32 row groups; chunks of 33 tokens (the last run holds one
    token) wrap mid-chunk in a window of 100.  Caches (ring and naive) against
    the oracle after every write, attention on some steps."""
    shp = inputs.Shape("test", 1, 20, D, 100, 33)
    run = SmallRun(shp, dtype=dtype)
    for step in range(7):
        _say(f"20 heads D={D} {dtype} step {step}")
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
        run.check_cache(f"20 heads step {step}")
        if step in (0, 3, 6):
            got, ref = run.attention(inputs.np_queries(shp, step, 0), n_splits=0)
            assert_attention(got, ref, f"20 heads step {step}")


def test_edge_cases_small():
    shp = inputs.TINY_WRAP
    run = SmallRun(shp)
    k, v = inputs.np_chunk(shp, 0)
    k[3] = 0.0                                         # an all-zero K and V row
    v[5, 1] = 0.0
    run.step(k, v)
    run.check_cache("zero rows")
    assert float(run.cache.k_scales[0, 0, 3]) == 0.0 and float(run.cache.v_scales[0, 1, 5]) == 0.0
    for n_q in (1, 3, 16):
        _say(f"edge n_q={n_q}")
        q = inputs.np_queries(shp, 0, 0)[:n_q].copy()
        out = K.attn_fp8_window(run.cache, 0, 0, run.ring.n_valid, torch.from_numpy(q).cuda(),
                                run.ring.pos_next - n_q, run.rope.base)
        torch.cuda.synchronize()
        assert_attention(_f32(out), oracle.attention(run.orc, 0, run.ref_n_valid(), q, run.ref_pos_next() - n_q),
                         f"n_q={n_q}")
    # a single valid key: the output is that key's dequantised value row
    _say("edge n_valid=1")
    q = inputs.np_queries(shp, 0, 1)
    qd = torch.from_numpy(q).cuda()
    out = K.attn_fp8_window(run.cache, 0, 0, 1, qd, 0, run.rope.base)
    torch.cuda.synchronize()
    ref = oracle.attention(run.orc, 0, 1, q, 0)
    assert_attention(_f32(out), ref, "n_valid=1")
    # zero queries: uniform weights
    out0 = K.attn_fp8_window(run.cache, 0, 0, 16, torch.zeros_like(qd), 0, run.rope.base)
    torch.cuda.synchronize()
    assert_attention(_f32(out0), oracle.attention(run.orc, 0, 16, np.zeros_like(q), 0), "q=0")


def test_key_tiles_dealt_to_splits():
    """The 64-key tiles are dealt to the splits in turn (split s of S takes
    tiles s, s + S, ...): windows ending just before, on and just after tile
    boundaries, against split counts that do and do not divide the tile count
    (and more splits than tiles, which the library reduces), every output row
    against the oracle."""
    shp = inputs.Shape("test", 1, 2, 64, 1000, 125)
    run = SmallRun(shp, table=(-256, 2048))
    for step in range(8):
        run.step(*inputs.np_chunk(shp, step))
    assert run.ref_n_valid() == 1000
    q = inputs.np_queries(shp, 8, 0, n_q=37)
    qd = torch.from_numpy(q).cuda()
    q_pos = run.ref_pos_next() - 37
    for n_valid in (1, 63, 64, 65, 127, 128, 129, 448, 449, 640, 1000):
        # the newest n_valid keys of the window
        start_ref = oracle.slot_of_token(run.total - n_valid, shp.window)
        ref = oracle.attention(run.orc, start_ref, n_valid, q, q_pos)
        for splits in (1, 2, 3, 4, 5, 6, 7, 9, 13, 16):
            _say(f"tiles dealt to splits: n_valid {n_valid}, splits {splits}")
            out = K.attn_fp8_window(run.cache, 0, start_ref, n_valid, qd, q_pos, run.rope.base, n_splits=splits)
            torch.cuda.synchronize()
            assert_attention(_f32(out), ref, f"n_valid {n_valid}, splits {splits}")


def test_lazy_rescale_when_scores_grow():
    """Scores of the first 128 keys sit ~18 log2 units below the later ones,
    so the running max of every query moves by more than the lazy-rescale
    threshold inside a split (the accumulators are rescaled mid-window)."""
    shp = inputs.Shape("test", 1, 2, 128, 512, 128)
    run = SmallRun(shp, dtype=torch.float32)
    H, D, N = shp.n_heads, shp.head_dim, shp.n_new
    rng = np.random.default_rng(2024)
    t = rng.standard_normal((H, D)).astype(np.float32)
    t *= 12.0 / np.linalg.norm(t, axis=1, keepdims=True)          # |t| = 12 per head
    for c in range(4):
        pos = run.ref_pos_next() + np.arange(N)
        k_rot = (-t[None] if c == 0 else 0.0 * t[None]) + rng.standard_normal((N, H, D)).astype(np.float32) * (
            0.3 if c == 0 else 1.0)
        k = oracle.rope_rows(k_rot, -pos[:, None])                # stored rotated: k_rot
        v = rng.standard_normal((N, H, D)).astype(np.float32)
        run.step(np.ascontiguousarray(k), v)
    q_pos = run.ref_pos_next() - N + np.arange(N)
    q = oracle.rope_rows(t[None] + 0.3 * rng.standard_normal((N, H, D)).astype(np.float32), -q_pos[:, None])
    q = np.ascontiguousarray(q)
    for n_splits in (1, 2):
        _say(f"rescale n_splits={n_splits}")
        got, ref = run.attention(q, n_splits=n_splits, naive_too=False)
        assert_attention(got, ref, f"growing scores, {n_splits} splits")


def test_fp32_inputs_head_dim_128():
    shp = inputs.Shape("test", 1, 3, 128, 300, 70)
    run = SmallRun(shp, dtype=torch.float32)
    for step in range(6):
        _say(f"fp32 D128 step {step}")
        k, v = inputs.np_chunk(shp, step)
        run.step(k * 1.7, v * 0.6)
        run.check_cache(f"fp32 D128 step {step}")
        got, ref = run.attention(inputs.np_queries(shp, step, 0), n_splits=(step % 3) + 1)
        assert_attention(got, ref, f"fp32 D128 step {step}")


def test_write_on_every_pass():
    """Each denoise pass brings new K/V for the step's chunk: they are written
    again, to the same slots at the same positions (the ring advances once per
    step), before that pass's attention.  After every pass the cache equals
    the oracle's and attention matches it; the window wraps mid-chunk."""
    shp = inputs.Shape("test", 1, 3, 128, 300, 70)
    run = SmallRun(shp, dtype=torch.bfloat16)
    W, N = shp.window, shp.n_new
    for step in range(6):
        before = K.kvr_ring(run.ring.head, run.ring.n_valid, run.ring.pos_next)
        total_before = run.total
        after = K.kvr_ring(before.head, before.n_valid, before.pos_next)
        K.kvr_ring_after_write(after, W, N)
        run.total = total_before + N                   # the oracle's count after this step's write
        for p in range(shp.passes):
            _say(f"write every pass: step {step} pass {p}")
            k, v = inputs.np_chunk(shp, step, pss=p)
            run.write_pass(k, v, before, total_before)
            run.ring = K.kvr_ring(after.head, after.n_valid, after.pos_next)
            run.check_cache(f"step {step} pass {p}", naive_too=False)
            got, ref = run.attention(inputs.np_queries(shp, step, p), naive_too=False)
            assert_attention(got, ref, f"write every pass: step {step} pass {p}")


def test_split_merge_shares_one_workspace():
    """One workspace serves a run of calls with different split and query
    counts (3, 2 and 1 query blocks; up to 17 requested splits): every output
    matches the oracle, and the linear window bit for bit."""
    shp = inputs.Shape("test", 1, 3, 128, 1100, 600)
    run = SmallRun(shp, dtype=torch.bfloat16)
    for step in range(2):
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
    calls = [(600, 2), (600, 17), (257, 5), (600, 3), (1, 9), (600, 7), (513, 4)]
    cap = max(K.attn_fp8_window_workspace_bytes(run.cache, n_q, run.ring.n_valid, sp) for n_q, sp in calls)
    ws = torch.empty(cap, dtype=torch.uint8, device="cuda")
    for i, (n_q, splits) in enumerate(calls):
        _say(f"shared workspace call {i}: n_q {n_q}, splits {splits}")
        q = inputs.np_queries(shp, 1, i)[:n_q]
        got, ref = run.attention(q, n_splits=splits, ws=ws)
        assert_attention(got, ref, f"shared workspace call {i}")


def test_partial_then_merge_equals_the_call():
    """attn_fp8_window_partial followed by attn_fp8_window_merge gives the
    same bits as attn_fp8_window, for one split, several and the default."""
    shp = inputs.Shape("test", 1, 3, 128, 1100, 600)
    run = SmallRun(shp, dtype=torch.bfloat16)
    for step in range(2):
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
    W = shp.window
    start = K.kvr_ring_logical_start(run.ring, W)
    for i, (n_q, splits) in enumerate([(600, 1), (600, 3), (513, 0), (1, 5)]):
        _say(f"partial + merge {i}: n_q {n_q}, splits {splits}")
        q = torch.from_numpy(inputs.np_queries(shp, 1, i)[:n_q]).to(torch.bfloat16).cuda()
        qpos = run.ring.pos_next - n_q
        whole = K.attn_fp8_window(run.cache, 0, start, run.ring.n_valid, q, qpos, run.rope.base, n_splits=splits)
        out, ws = K.attn_fp8_window_partial(run.cache, 0, start, run.ring.n_valid, q, qpos, run.rope.base,
                                            n_splits=splits)
        K.attn_fp8_window_merge(run.cache, n_q, run.ring.n_valid, out, n_splits=splits, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(whole, out), i


def test_bf16_ragged_queries_head_dim_64():
    shp = inputs.Shape("test", 1, 4, 64, 1000, 161)
    run = SmallRun(shp, dtype=torch.bfloat16)
    for step in range(8):
        _say(f"bf16 D64 step {step}")
        k, v = inputs.np_chunk(shp, step)
        run.step(k, v)
        if step in (0, 6, 7):
            run.check_cache(f"bf16 D64 step {step}")
            got, ref = run.attention(inputs.np_queries(shp, step, 1))
            assert_attention(got, ref, f"bf16 D64 step {step}")


# ---------------------------------------------------------------------------
# production shape: one layer, 12 heads, D 128, W 5788, N 757
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def page_layer():
    shp = inputs.PAGE_LAYER
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(-40000, 100000, D)
    ring = K.kvr_ring_init()
    orc = oracle.LayerCache(H, D, W)
    total = 0
    for step in range(8):
        _say(f"page write step {step}")
        k, v = inputs.torch_chunk(shp, step, 0, "cpu")
        K.kv_write_rope_quant(cache, ring, 0, k[0].cuda(), v[0].cuda(), rope)
        oracle.write(orc, total, total, _f32(k[0]), _f32(v[0]))
        K.kvr_ring_after_write(ring, W, N)
        total += N
    torch.cuda.synchronize()
    # the oracle's window from the token count alone: the last W tokens, the
    # oldest at slot (total - W) mod W; queries at the last chunk's positions
    ref = dict(n_valid=min(total, W), start=oracle.slot_of_token(total - min(total, W), W), q_pos=total - N)
    assert (ring.n_valid, K.kvr_ring_logical_start(ring, W), ring.pos_next - N) == \
        (ref["n_valid"], ref["start"], ref["q_pos"])
    return dict(shape=shp, cache=cache, rope=rope, ring=ring, orc=orc, ref=ref)


def test_page_write_parity(page_layer):
    _say("page write parity")
    c, o = page_layer["cache"], page_layer["orc"]
    assert page_layer["ring"].head == (8 * 757) % 5788          # the 8th chunk wrapped
    for name in ("k", "v"):
        assert_codes(_np(getattr(c, f"{name}_codes"))[0], getattr(o, f"{name}_codes"), f"page {name}")
        assert_scales(_np(getattr(c, f"{name}_scales"))[0], getattr(o, f"{name}_scales"), f"page {name}")


def _page_rows(n_q, H, seed=0, per_head=40):
    rng = np.random.default_rng(seed)
    qs = np.unique(np.concatenate([[0, 31, 32, 127, 128, n_q - 1], rng.integers(0, n_q, per_head)]))
    return [(int(i), h) for h in range(H) for i in qs]


def _all_rows(n_q, H):
    return [(i, h) for i in range(n_q) for h in range(H)]


def test_page_attention_parity(page_layer):
    """Production layer, 4 passes: every one of the 757 x 12 output rows of
    pass 0 (default and single split), sampled rows of every head on the
    other passes; the oracle's window and positions come from the token count."""
    shp, c, rope, ring, orc, r = (page_layer[k] for k in ("shape", "cache", "rope", "ring", "orc", "ref"))
    W = shp.window
    start = K.kvr_ring_logical_start(ring, W)
    for p in range(shp.passes):
        _say(f"page attention pass {p}")
        q = inputs.torch_queries(shp, 8, p, 0, "cpu")
        qd = q.cuda()
        rows = _all_rows(shp.n_new, shp.n_heads) if p == 0 else _page_rows(shp.n_new, shp.n_heads, seed=p)
        ref = oracle.attention(orc, r["start"], r["n_valid"], _f32(q), r["q_pos"], rows=rows)
        for n_splits in ((0, 1) if p == 0 else (0,)):
            out = K.attn_fp8_window(c, 0, start, ring.n_valid, qd, ring.pos_next - shp.n_new, rope.base,
                                    n_splits=n_splits)
            torch.cuda.synchronize()
            got = _f32(out)
            g = np.stack([got[i, h] for i, h in rows])
            mx, mean = assert_attention(g, ref, f"page pass {p} splits {n_splits} ({len(rows)} rows)")
            _say(f"  splits={n_splits} max-abs {mx:.4g} mean-abs {mean:.4g}")
            assert np.isfinite(got).all()
        if p == 0:
            # the same call twice (same split count) gives bit-identical outputs
            again = K.attn_fp8_window(c, 0, start, ring.n_valid, qd, ring.pos_next - shp.n_new, rope.base,
                                      n_splits=n_splits)
            torch.cuda.synchronize()
            assert torch.equal(out, again), "attention is not deterministic"


def test_page_rebase_parity(page_layer):
    shp, c, ring, orc, r = (page_layer[k] for k in ("shape", "cache", "ring", "orc", "ref"))
    delta = inputs.rebase_delta()
    _say(f"page rebase delta={delta}")
    c2 = K.KVCache(1, shp.n_heads, shp.head_dim, shp.window)
    for n in ("k_codes", "v_codes", "k_scales", "v_scales"):
        getattr(c2, n).copy_(getattr(c, n))
    o2 = orc.copy()
    K.kv_delta_rebase(c2, ring, 0, 1, delta)
    oracle.rebase(o2, r["start"], r["n_valid"], delta)
    torch.cuda.synchronize()
    assert_codes(_np(c2.k_codes)[0], o2.k_codes, "rebase k")
    assert_scales(_np(c2.k_scales)[0], o2.k_scales, "rebase k")
    assert torch.equal(c2.v_codes, c.v_codes) and torch.equal(c2.v_scales, c.v_scales)


def test_page_naive_matches_ring():
    """Naive per-call upkeep at production shape: identical caches and outputs."""
    shp = inputs.PAGE_LAYER
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(0, 16 * N, D)
    ring = K.kvr_ring_init()
    lin = [torch.zeros((H, W, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    lc = K.KVCache(1, H, D, W)
    ping = 0
    for step in range(9):
        _say(f"page naive step {step}")
        k, v = inputs.torch_chunk(shp, step, 0, "cuda")
        K.naive_upkeep(lin[2 * ping], lin[2 * ping + 1], k[0], v[0], ring.n_valid, ring.pos_next,
                       rope, lin[2 - 2 * ping], lin[3 - 2 * ping], lc.k_codes[0], lc.v_codes[0],
                       lc.k_scales[0], lc.v_scales[0])
        ping = 1 - ping
        K.kv_write_rope_quant(cache, ring, 0, k[0], v[0], rope)
        K.kvr_ring_after_write(ring, W, N)
    start = K.kvr_ring_logical_start(ring, W)
    idx = torch.from_numpy((start + np.arange(W)) % W).cuda()
    for n in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(cache, n)[0][:, idx], getattr(lc, n)[0]), n
    q = inputs.torch_queries(shp, 9, 0, 0, "cuda")
    a = K.attn_fp8_window(cache, 0, start, W, q, ring.pos_next - N, rope.base)
    b = K.attn_fp8_window(lc, 0, 0, W, q, ring.pos_next - N, rope.base)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_step_batched_write_60_layers():
    """The 60-layer write of one denoise step in one launch, every layer against
    the oracle (the launch's workgroups are renumbered into per-XCD runs, with
    the grid's last blocks left in place: every (layer, K/V, token) row must
    still be written exactly once)."""
    shp = inputs.PAGE_STEP
    H, D, W, N, L = shp.n_heads, shp.head_dim, shp.window, shp.n_new, shp.n_layers
    cache = K.KVCache(L, H, D, W)
    rope = K.RopeTable(0, 8000, D)
    ring = K.kvr_ring(5299, 5788, 5299)          # full ring, the chunk wraps at the end
    k, v = inputs.torch_chunk(shp, 0, 0, "cpu", n_layers=L)
    _say("60-layer batched write")
    K.kv_write_rope_quant(cache, ring, 0, k.cuda(), v.cuda(), rope)
    torch.cuda.synchronize()
    slots = (5299 + np.arange(N)) % W
    got = {n: _np(getattr(cache, n)) for n in ("k_codes", "v_codes", "k_scales", "v_scales")}
    for layer in range(L):
        orc = oracle.LayerCache(H, D, W)
        oracle.write(orc, 5299, 5299, _f32(k[layer]), _f32(v[layer]))
        for n in ("k", "v"):
            assert_codes(got[f"{n}_codes"][layer][:, slots], getattr(orc, f"{n}_codes")[:, slots],
                         f"layer {layer} {n}")
            assert_scales(got[f"{n}_scales"][layer][:, slots], getattr(orc, f"{n}_scales")[:, slots],
                          f"layer {layer} {n}")
    # slots outside the chunk were not touched
    untouched = np.setdiff1d(np.arange(W), (5299 + np.arange(N)) % W)
    for n, arr in got.items():
        assert not arr[:, :, untouched].any(), n


@pytest.mark.parametrize("L,H,D,N,dtype", [(5, 3, 64, 200, torch.float32), (3, 5, 128, 300, torch.bfloat16)])
def test_multi_layer_write_mid_sizes(L, H, D, N, dtype):
    """Multi-layer writes whose grids hold both workgroups renumbered into
    per-XCD runs and the grid's last blocks left in place (5 layers x 100
    token pairs: 896 + 104 blocks; 3 layers x 150: 896 + 4), against the
    oracle on every layer, the chunk wrapping at the end of the ring."""
    W = 2 * N + 37
    shp = inputs.Shape("test", L, H, D, W, N)
    cache = K.KVCache(L, H, D, W)
    rope = K.RopeTable(0, 4 * N, D)
    head = W - N // 3                                   # the chunk wraps
    ring = K.kvr_ring(head, W, 2 * N)
    k, v = inputs.torch_chunk(shp, 1, 0, "cpu", dtype=dtype, n_layers=L)
    _say(f"{L}-layer write, {H} heads, D {D}, N {N}, {dtype}")
    K.kv_write_rope_quant(cache, ring, 0, k.cuda(), v.cuda(), rope)
    torch.cuda.synchronize()
    slots = (head + np.arange(N)) % W
    got = {n: _np(getattr(cache, n)) for n in ("k_codes", "v_codes", "k_scales", "v_scales")}
    for layer in range(L):
        orc = oracle.LayerCache(H, D, W)
        oracle.write(orc, head, 2 * N, _f32(k[layer]), _f32(v[layer]))
        for n in ("k", "v"):
            assert_codes(got[f"{n}_codes"][layer][:, slots], getattr(orc, f"{n}_codes")[:, slots],
                         f"layer {layer} {n}")
            assert_scales(got[f"{n}_scales"][layer][:, slots], getattr(orc, f"{n}_scales")[:, slots],
                          f"layer {layer} {n}")
    untouched = np.setdiff1d(np.arange(W), slots)
    for n, arr in got.items():
        assert not arr[:, :, untouched].any(), n


def test_extreme_sizes():
    """A chunk as large as the window (every slot rewritten in one write, twice,
    the second time wrapping from a non-zero head), and 3000 queries (12 query
    blocks) over it; one and several splits."""
    shp = inputs.Shape("test", 1, 2, 128, 200, 200)
    run = SmallRun(shp, dtype=torch.bfloat16)
    for step in range(2):
        _say(f"extreme: chunk == window, step {step}")
        k, v = inputs.np_chunk(shp, step)
        kb = _f32(torch.from_numpy(k).to(torch.bfloat16))
        vb = _f32(torch.from_numpy(v).to(torch.bfloat16))
        run.step(kb, vb)
        run.check_cache(f"chunk == window step {step}")
        if step == 0:
            # shift the head so the second full-window chunk wraps in the middle
            run.step(kb[:70].copy(), vb[:70].copy())
    n_q = 3000
    q = np.random.default_rng(77).standard_normal((n_q, 2, 128)).astype(np.float32)
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    start = K.kvr_ring_logical_start(run.ring, 200)
    rows = [(i, h) for i in (0, 1, 255, 256, 1023, 1024, 2047, 2999) for h in range(2)]
    ref = oracle.attention(run.orc, run.ref_start(), 200, _f32(qd), 0, rows=rows)
    for splits in (1, 0, 4):
        _say(f"extreme: n_q={n_q} splits={splits}")
        out = K.attn_fp8_window(run.cache, 0, start, 200, qd, 0, run.rope.base, n_splits=splits)
        torch.cuda.synchronize()
        got = _f32(out)
        assert np.isfinite(got).all()
        assert_attention(np.stack([got[i, h] for i, h in rows]), ref, f"n_q={n_q} splits={splits}")


def test_full_step_parity_layers_0_and_59():
    """The full-step configuration the benchmark times: a 60-layer cache, one
    60-layer write per step with the ring head advancing 757 slots, then the
    pass-major attention calls with the default splits.  All 4 passes of layers
    0 and 59 are checked at steps 1 and 42 (positions up to ~37K, the ring
    wrapped many times) on sampled queries of every head, then a rebase of all
    60 layers by a drawn delta is checked on both layers."""
    shp = inputs.PAGE_STEP
    H, D, W, N, L, P = shp.n_heads, shp.head_dim, shp.window, shp.n_new, shp.n_layers, shp.passes
    cache = K.KVCache(L, H, D, W)
    rope = K.RopeTable(-inputs.DELTA_MAX - 1024, 45 * N + inputs.DELTA_MAX + 2048, D)
    ring = K.kvr_ring_init()
    orcs = {0: oracle.LayerCache(H, D, W), 59: oracle.LayerCache(H, D, W)}
    total = 0
    rng = np.random.default_rng(42)
    for step in range(1, 43):
        k, v = inputs.torch_chunk(shp, step, 0, "cuda", n_layers=L)
        K.kv_write_rope_quant(cache, ring, 0, k, v, rope)
        for layer, orc in orcs.items():
            oracle.write(orc, total, total, _f32(k[layer]), _f32(v[layer]))
        K.kvr_ring_after_write(ring, W, N)
        total += N
        # the oracle's window from the step count: the last W of the step * N tokens
        n_ref = min(total, W)
        start_ref = oracle.slot_of_token(total - n_ref, W)
        assert (ring.n_valid, K.kvr_ring_logical_start(ring, W), ring.pos_next) == (n_ref, start_ref, total)
        if step not in (1, 42):
            continue
        start = K.kvr_ring_logical_start(ring, W)
        qs = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.integers(0, N, 12)]))
        rows = [(int(i), h) for h in range(H) for i in qs]
        for p in range(P):
            for layer in (0, 59):
                _say(f"full step {step} pass {p} layer {layer}")
                q = inputs.torch_queries(shp, step, p, layer, "cuda")
                out = K.attn_fp8_window(cache, layer, start, ring.n_valid, q, ring.pos_next - N, rope.base)
                torch.cuda.synchronize()
                got = _f32(out)
                # every row of pass 0 of layer 59 at the last step; sampled rows otherwise
                rr = _all_rows(N, H) if (step == 42 and p == 0 and layer == 59) else rows
                ref = oracle.attention(orcs[layer], start_ref, n_ref, _f32(q), total - N, rows=rr)
                assert_attention(np.stack([got[i, h] for i, h in rr]), ref,
                                 f"step {step} pass {p} layer {layer} ({len(rr)} rows)")
    for layer, orc in orcs.items():
        assert_codes(_np(cache.k_codes[layer]), orc.k_codes, f"layer {layer} k after 42 steps")
        assert_scales(_np(cache.v_scales[layer]), orc.v_scales, f"layer {layer} v after 42 steps")
    delta = inputs.rebase_delta()
    _say(f"full-step rebase of 60 layers by {delta}")
    K.kv_delta_rebase(cache, ring, 0, L, delta)
    torch.cuda.synchronize()
    for layer, orc in orcs.items():
        oracle.rebase(orc, start_ref, n_ref, delta)
        assert_codes(_np(cache.k_codes[layer]), orc.k_codes, f"layer {layer} rebase")
        assert_scales(_np(cache.k_scales[layer]), orc.k_scales, f"layer {layer} rebase")


def test_graph_replay_matches_eager():
    """A step (the write of a chunk that wraps mid-chunk, four attention calls
    with one and two splits) captured as a graph: every replay, with other
    eager work and synchronisations between replays, gives the eager outputs
    and cache bit for bit, and those match the oracle."""
    shp = inputs.TINY_WRAP
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(-256, 4096, D)
    ring = K.kvr_ring_init()
    orc = oracle.LayerCache(H, D, W)
    for step in range(6):                              # 96 tokens: the 7th chunk wraps
        k, v = inputs.np_chunk(shp, step)
        K.kv_write_rope_quant(cache, ring, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), rope)
        K.kvr_ring_after_write(ring, W, N)
        oracle.write(orc, step * N, step * N, k, v)
    oracle.write(orc, 6 * N, 6 * N, *inputs.np_chunk(shp, 6))
    k, v = (torch.from_numpy(a).cuda() for a in inputs.np_chunk(shp, 6))
    qs = [torch.from_numpy(inputs.np_queries(shp, 6, p)).cuda() for p in range(4)]
    after = ring.copy()
    K.kvr_ring_after_write(after, W, N)
    start = K.kvr_ring_logical_start(after, W)
    outs = [torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    ws = torch.empty(K.attn_fp8_window_workspace_bytes(cache, N, after.n_valid, 2), dtype=torch.uint8,
                     device="cuda")

    def step():
        K.kv_write_rope_quant(cache, ring, 0, k, v, rope)
        for p in range(4):
            K.attn_fp8_window(cache, 0, start, after.n_valid, qs[p], after.pos_next - N, rope.base,
                              out=outs[p], n_splits=1 + p % 2, ws=ws)

    _say("graph: eager step")
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs] + [cache.k_codes.clone(), cache.k_scales.clone()]
    # the eager step (and so every replay) against the oracle: 7 * 16 = 112
    # tokens written, the window the last 100, the queries at 96 .. 111
    assert_codes(_np(cache.k_codes)[0], orc.k_codes, "graph step k")
    assert_scales(_np(cache.k_scales)[0], orc.k_scales, "graph step k")
    for p in range(4):
        ref = oracle.attention(orc, oracle.slot_of_token(112 - W, W), W, _np(qs[p]), 6 * N)
        assert_attention(_f32(outs[p]), ref, f"graph step pass {p}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("graph: capture")
    with torch.cuda.graph(g):
        step()
    other = K.KVCache(1, H, D, W)
    slots = torch.tensor([K.kvr_ring_slot(ring, W, j) for j in range(N)], device="cuda")
    assert int(slots[0]) == 96 and int(slots[-1]) == 11      # the chunk wraps
    for r in range(3):
        _say(f"graph: replay {r}")
        for o in outs:
            o.fill_(7.0)
        cache.k_codes[0, :, slots] = 0                 # undone by the replay's write
        # eager work of the program between replays
        K.kv_write_rope_quant(other, K.kvr_ring_init(), 0, k, v, rope)
        K.attn_fp8_window(other, 0, 0, N, qs[r], 0, rope.base)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o for o in outs] + [cache.k_codes, cache.k_scales]
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {r}: tensor {i} differs from the eager run"


def test_position_rows_in_load_order(page_layer):
    """The 1-D call with the queries' (cos, sin) taken from the rotary table at
    the chunk's positions, rearranged once into the kernel's load order
    (kv_rope_query_lanes + attn_fp8_window_lanes, what the benchmark's step
    uses), against the oracle: production layer, all 4 passes, default and
    single split; and the small W = 100 workload that wraps mid-chunk."""
    shp, c, rope, ring, orc, r = (page_layer[k] for k in ("shape", "cache", "rope", "ring", "orc", "ref"))
    W, N = shp.window, shp.n_new
    start = K.kvr_ring_logical_start(ring, W)
    lanes = K.kv_rope_query_lanes(K.rope_table_rows(rope, ring.pos_next - N, N))
    for p in range(shp.passes):
        _say(f"rows in load order, page pass {p}")
        q = inputs.torch_queries(shp, 8, p, 0, "cpu")
        rows = _all_rows(N, shp.n_heads) if p == 0 else _page_rows(N, shp.n_heads, seed=10 + p)
        ref = oracle.attention(orc, r["start"], r["n_valid"], _f32(q), r["q_pos"], rows=rows)
        for n_splits in ((0, 1) if p == 0 else (0,)):
            out = K.attn_fp8_window_lanes(c, 0, start, ring.n_valid, q.cuda(), lanes, n_splits=n_splits)
            torch.cuda.synchronize()
            got = _f32(out)
            mx, mean = assert_attention(np.stack([got[i, h] for i, h in rows]), ref, f"lanes pass {p}")
            _say(f"  splits={n_splits} max-abs {mx:.4g} mean-abs {mean:.4g}")
    run = SmallRun(inputs.TINY_WRAP)
    for step in range(9):
        k, v = inputs.np_chunk(inputs.TINY_WRAP, step)
        run.step(k, v)
        q = inputs.np_queries(inputs.TINY_WRAP, step, 0)
        lanes = K.kv_rope_query_lanes(K.rope_table_rows(run.rope, run.ring.pos_next - 16, 16))
        out = K.attn_fp8_window_lanes(run.cache, 0, K.kvr_ring_logical_start(run.ring, 100), run.ring.n_valid,
                                      torch.from_numpy(q).cuda(), lanes, n_splits=1 + step % 2)
        torch.cuda.synchronize()
        assert_attention(_f32(out), oracle.attention(run.orc, run.ref_start(), run.ref_n_valid(), q,
                                                     run.ref_pos_next() - 16), f"lanes small step {step}")
