"""GPU parity of the chunk's write fused into the attention call that first
reads it (attn_fp8_window_write), through the C ABI.

The fused call must store exactly the codes and scales kv_write_rope_quant
stores and return exactly the rows attn_fp8_window returns over the window
after that write; its outputs are also checked against the oracle on every
row (window, slots and positions from the oracle's own token count).  Cases:
  * the production layer (12 heads, D 128, W 5788, N 757; 7 splits, 252
    workgroups, each writing a share and each waiting before its last tiles),
    two steps, the first chunk wrapping past the end of the ring;
  * small shapes: W 96 and W 100 (chunks wrap mid-chunk), fp32 and bf16, head_dim 64 and 128, two query blocks, a ring
    filling up over the steps, the workspace reused by every step;
  * a sweep of windows (130, 300, 640), chunks (33, 64, 65, 129 tokens) and
    split counts, stepped until the ring wraps: the first new key falls in
    every local tile of every split;
  * a fixed prefix beside the ring;
  * one split, a chunk most of the window (every tile of some splits holds new
    keys: those wait before their first tile), and a launch with more
    workgroups than the GPU holds at once (the write kernel and the plain call
    are launched instead);
  * the control block back at zero after every call, in one workspace reused
    by every step while the partials before it change size;
  * a poll limit of one (the bounded wait's give-up path): output rows are
    NaN exactly when a wait gave up, and are otherwise the plain call's.
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


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    K.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().cpu().numpy()


def _bits_equal(a, b):
    return a.shape == b.shape and a.dtype == b.dtype and \
        torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _control(ws):
    return _np(ws[-K.FUSED_SYNC_BYTES:].view(torch.int32))[:4]


class Twin:
    """Two caches with one history: `fused` is written by attn_fp8_window_write,
    `plain` by kv_write_rope_quant followed by attn_fp8_window; the oracle
    (pure rings only) follows by its own token count."""

    def __init__(self, H, D, W, N, dtype, prefix=0, steps=16):
        self.shape = inputs.Shape("test", 1, H, D, W, N)
        self.dtype = dtype
        self.fused = K.KVCache(1, H, D, W, n_prefix=prefix)
        self.plain = K.KVCache(1, H, D, W, n_prefix=prefix)
        self.ring = K.kvr_ring_init()
        self.rope = K.RopeTable(0, (steps + 1) * N, D)
        self.orc = oracle.LayerCache(H, D, W) if prefix == 0 else None
        self.total = 0
        # one workspace for every step, larger than any step needs: the calls'
        # partials change size as the window fills and the split count moves,
        # while the control block stays in the buffer's last 256 bytes
        self.ws = torch.zeros(24 << 20, dtype=torch.uint8, device="cuda")

    def chunk(self, step):
        k, v = inputs.torch_chunk(self.shape, step, 0, "cuda", dtype=self.dtype)
        q = inputs.torch_queries(self.shape, step, 0, 0, "cuda", dtype=self.dtype)
        return k[0], v[0], q

    def prefill(self, step):
        """Both caches take the chunk through the plain write."""
        k, v, _ = self.chunk(step)
        for c in (self.fused, self.plain):
            K.kv_write_rope_quant(c, self.ring, 0, k, v, self.rope)
        if self.orc is not None:
            oracle.write(self.orc, self.total, self.total, _np(k.float()), _np(v.float()))
        self.total += self.shape.n_new
        K.kvr_ring_after_write(self.ring, self.fused.ring_window, self.shape.n_new)

    def fused_step(self, step, n_splits, oracle_check=True, poll_limit=0):
        N, W = self.shape.n_new, self.fused.ring_window
        k, v, q = self.chunk(step)
        before = self.ring.copy()
        need = K.attn_fp8_window_write_workspace_bytes(self.fused, before, N, n_splits)
        assert need <= self.ws.numel()
        if poll_limit:
            self.ws[-K.FUSED_SYNC_BYTES + 12:-K.FUSED_SYNC_BYTES + 16].view(torch.int32).fill_(poll_limit)
        out_f = K.attn_fp8_window_write(self.fused, before, 0, k, v, q, self.rope, self.rope.base,
                                        n_splits=n_splits, ws=self.ws)
        K.kv_write_rope_quant(self.plain, before, 0, k, v, self.rope)
        after = before.copy()
        K.kvr_ring_after_write(after, W, N)
        out_p = K.attn_fp8_window(self.plain, 0, K.kvr_ring_logical_start(after, W), after.n_valid, q,
                                  before.pos_next, self.rope.base, n_splits=n_splits)
        torch.cuda.synchronize()
        for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
            assert _bits_equal(getattr(self.fused, name), getattr(self.plain, name)), name
        ctl = _control(self.ws)
        self.ring = after
        if self.orc is not None:
            oracle.write(self.orc, self.total, self.total, _np(k.float()), _np(v.float()))
            q_pos = self.total
            self.total += N
        if poll_limit:
            # the give-up path: rows are NaN exactly when some wait gave up
            gave_up = int(ctl[2])
            nan_rows = torch.isnan(out_f.float()).any(dim=-1)
            _say(f"  poll limit {poll_limit}: {gave_up} waits gave up, {int(nan_rows.sum())} NaN rows")
            assert (gave_up > 0) == bool(nan_rows.any())
            if gave_up == 0:
                assert _bits_equal(out_f, out_p)
            self.ws[-K.FUSED_SYNC_BYTES:].zero_()
            return
        assert ctl[0] == 0 and ctl[1] == 0 and ctl[2] == 0, ctl
        if not _bits_equal(out_f, out_p) and self.orc is not None:
            # name the culprit before failing: both outputs against the oracle
            n_valid = min(self.total, self.shape.window)
            start = oracle.slot_of_token(self.total - n_valid, self.shape.window)
            ref = oracle.attention(self.orc, start, n_valid, _np(q.float()), q_pos)
            ef = np.abs(_np(out_f.float()) - ref).max(axis=-1)
            ep = np.abs(_np(out_p.float()) - ref).max(axis=-1)
            diff = (out_f.view(torch.int16) != out_p.view(torch.int16)).any(dim=-1).cpu().numpy()
            _say(f"  fused max-abs {ef.max():.4g}, plain max-abs {ep.max():.4g}; rows that differ: "
                 f"{int(diff.sum())} of {diff.size}, heads {sorted(set(np.nonzero(diff)[1].tolist()))}, "
                 f"queries {sorted(set(np.nonzero(diff)[0].tolist()))[:12]}")
        assert _bits_equal(out_f, out_p), "fused output differs from the write + plain call"
        if self.orc is not None and oracle_check:
            n_valid = min(self.total, self.shape.window)
            start = oracle.slot_of_token(self.total - n_valid, self.shape.window)
            ref = oracle.attention(self.orc, start, n_valid, _np(q.float()), q_pos)
            mx, mean = assert_attention(_np(out_f.float()), ref, f"fused step {step}")
            _say(f"  oracle max-abs {mx:.4g} mean-abs {mean:.4g}")


def test_fused_write_production_layer():
    shp = inputs.PAGE_LAYER
    t = Twin(shp.n_heads, shp.head_dim, shp.window, shp.n_new, torch.bfloat16, steps=10)
    for s in range(7):
        _say(f"production prefill {s}")
        t.prefill(s)
    _say("production fused step 7 (the chunk wraps; 252 workgroups)")
    t.fused_step(7, 0)
    _say("production fused step 8")
    t.fused_step(8, 0, oracle_check=False)


@pytest.mark.parametrize("H,D,W,N,dtype,splits,steps,prefill", [
    (2, 64, 96, 16, torch.float32, 2, 10, 0),
    (2, 64, 100, 16, torch.bfloat16, 2, 12, 0),
    (5, 128, 578, 35, torch.float32, 0, 20, 2),
    (3, 128, 1000, 300, torch.bfloat16, 3, 6, 0),
    (3, 64, 900, 260, torch.float32, 4, 6, 1),
    (20, 64, 300, 33, torch.bfloat16, 3, 12, 0),
    # 64 heads: with 5 splits 320 workgroups, more than the GPU holds at once
    # (the write kernel and the plain call instead); with 3 splits 192, fused
    (64, 64, 300, 33, torch.bfloat16, 5, 4, 7),
    (64, 64, 300, 33, torch.bfloat16, 3, 4, 7),
])
def test_fused_write_small(H, D, W, N, dtype, splits, steps, prefill):
    t = Twin(H, D, W, N, dtype, steps=steps + prefill)
    for s in range(prefill):
        t.prefill(s)
    for s in range(prefill, prefill + steps):
        _say(f"fused H={H} D={D} W={W} N={N} {dtype} splits={splits} step {s} (n_valid {t.ring.n_valid})")
        t.fused_step(s, splits)


@pytest.mark.parametrize("W", [130, 300, 640])
def test_fused_write_sweep(W):
    """Chunks of 33, 64, 65 and 129 tokens with the default and 2, 3 and 5
    splits, stepped until the ring has filled and wrapped (at most 12 steps):
    where the new keys start moves through every local tile of every split,
    and each step must equal the write + plain call bit for bit and leave the
    control block at zero."""
    for N in (33, 64, 65, 129):
        steps = min(-(-W // N) + 2, 12)
        for splits in (0, 2, 3, 5):
            t = Twin(3, 64, W, N, torch.bfloat16, steps=steps)
            for s in range(steps):
                _say(f"fused sweep W={W} N={N} splits={splits} step {s} (n_valid {t.ring.n_valid})")
                t.fused_step(s, splits, oracle_check=False)


@pytest.mark.parametrize("D,dtype,splits", [(128, torch.bfloat16, 0), (64, torch.float32, 3)])
def test_fused_write_with_prefix(D, dtype, splits):
    t = Twin(4, D, 600, 50, dtype, prefix=40, steps=16)
    for s in range(14):
        _say(f"fused with prefix D={D} {dtype} step {s} (n_valid {t.ring.n_valid})")
        t.fused_step(s, splits)


@pytest.mark.parametrize("W,N,splits", [(96, 16, 1), (96, 80, 2), (5788, 757, 1)])
def test_fused_write_new_keys_everywhere(W, N, splits):
    """One split, or a chunk that is most of the window: workgroups wait
    before their first tile or soon after."""
    t = Twin(2 if W < 1000 else 12, 64 if W < 1000 else 128, W, N, torch.bfloat16, steps=4)
    for s in range(3):
        _say(f"new keys in every split W={W} N={N} splits={splits} step {s}")
        t.fused_step(s, splits, oracle_check=W < 1000)


def test_fused_write_wait_give_up():
    """A poll limit of one: waiting workgroups that find the writers not yet
    done give up at once; their rows come out NaN and the timeouts are counted."""
    t = Twin(5, 128, 578, 35, torch.float32, steps=24)
    for s in range(17):
        t.prefill(s)
    for s in range(17, 20):
        _say(f"poll limit 1, step {s}")
        t.fused_step(s, 0, poll_limit=1)
    # the control block zeroed again: the next call is exact
    _say("after the give-up steps")
    t.fused_step(20, 0)
