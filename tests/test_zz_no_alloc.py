"""attn_fp8_window_noalloc (through the C ABI) against attn_fp8_window.

The allocation-free call runs the same kernels as attn_fp8_window with its
split partials in the library's own per-GPU scratch instead of a caller
workspace, so its outputs must equal the workspace call's bit for bit.
Checked on two calls in a row on one stream (the second smaller than the
first, so it reuses the scratch the first one filled), then a one-split call
(no scratch), each against the oracle as well; and a call whose partials
would not fit the scratch is refused on the host.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_ring_amd import inputs
from kv_cache_attention_ring_amd import kvring as K

from _parity import assert_attention

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _layer(shp, steps, dtype=torch.bfloat16):
    """A cache written with `steps` chunks, its oracle twin and the window."""
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(0, (steps + 2) * N, D)
    ring = K.kvr_ring_init()
    orc = oracle.LayerCache(H, D, W)
    total = 0
    for step in range(steps):
        k, v = inputs.torch_chunk(shp, step, 0, "cpu", dtype=dtype)
        K.kv_write_rope_quant(cache, ring, 0, k[0].cuda(), v[0].cuda(), rope)
        oracle.write(orc, total, total, k[0].float().numpy(), v[0].float().numpy())
        K.kvr_ring_after_write(ring, W, N)
        total += N
    torch.cuda.synchronize()
    n = min(total, W)
    return dict(cache=cache, rope=rope, ring=ring, orc=orc, start=oracle.slot_of_token(total - n, W), n=n,
                q_pos=total - N)


def test_noalloc_two_calls_in_a_row_match_the_workspace_call():
    assert torch.cuda.is_available()
    big_shape = inputs.PAGE_LAYER                                # 12 heads x 757 queries, 7 splits
    small_shape = inputs.Shape("test", 1, 3, 128, 1100, 300)     # 3 heads x 300 queries, 4 splits
    big, small = _layer(big_shape, 8), _layer(small_shape, 4)
    calls = []
    for lay, shp, splits in ((big, big_shape, 0), (small, small_shape, 4)):
        ring = lay["ring"]
        q = inputs.torch_queries(shp, 9, 0, 0, "cuda")
        need = K.attn_fp8_window_workspace_bytes(lay["cache"], shp.n_new, ring.n_valid, splits)
        assert 0 < need <= K.NOALLOC_SCRATCH_BYTES
        calls.append((lay, shp, splits, q, need))
    outs = []
    # the two allocation-free calls back to back on one stream, the second smaller
    for i, (lay, shp, splits, q, need) in enumerate(calls):
        _say(f"noalloc call {i}: {shp.n_heads} heads x {shp.n_new} queries, {need} bytes of partials")
        ring = lay["ring"]
        out = torch.full(q.shape, 7.0, dtype=torch.bfloat16, device="cuda")
        K.attn_fp8_window_noalloc(lay["cache"], 0, K.kvr_ring_logical_start(ring, shp.window), ring.n_valid, q,
                                  ring.pos_next - shp.n_new, lay["rope"].base, out=out, n_splits=splits)
        outs.append(out)
    torch.cuda.synchronize()
    for i, ((lay, shp, splits, q, need), got) in enumerate(zip(calls, outs)):
        ring = lay["ring"]
        want = K.attn_fp8_window(lay["cache"], 0, K.kvr_ring_logical_start(ring, shp.window), ring.n_valid, q,
                                 ring.pos_next - shp.n_new, lay["rope"].base, n_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {i}: noalloc differs from the workspace call"
        rows = [(j, h) for j in (0, 1, 255, 256, shp.n_new - 1) for h in range(shp.n_heads)]
        ref = oracle.attention(lay["orc"], lay["start"], lay["n"], q.float().cpu().numpy(), lay["q_pos"], rows=rows)
        g = got.float().cpu().numpy()
        assert_attention(np.stack([g[j, h] for j, h in rows]), ref, f"noalloc call {i}")
    # one split: no scratch at all
    lay, shp = small, small_shape
    ring = lay["ring"]
    q = inputs.torch_queries(shp, 9, 1, 0, "cuda")
    _say("noalloc call with one split")
    a = K.attn_fp8_window_noalloc(lay["cache"], 0, K.kvr_ring_logical_start(ring, shp.window), ring.n_valid, q,
                                  ring.pos_next - shp.n_new, lay["rope"].base, n_splits=1)
    b = K.attn_fp8_window(lay["cache"], 0, K.kvr_ring_logical_start(ring, shp.window), ring.n_valid, q,
                          ring.pos_next - shp.n_new, lay["rope"].base, n_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # partials beyond the scratch: refused on the host, nothing launched
    q_big = torch.zeros((8000, shp.n_heads, shp.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(K.KVRError) as err:
        K.attn_fp8_window_noalloc(lay["cache"], 0, 0, ring.n_valid, q_big, 0, lay["rope"].base, n_splits=17)
    assert err.value.status == K.KVR_EINVAL
