"""Benchmark: ms per denoise step of the write-time RoPE + FP8 ring cache path.

One step (the production attention shape on one GPU's 12-head share):
  * one launch writing the new chunk (757 tokens) of all 60 layer caches
    (RoPE + FP8 at write time), then
  * 240 FP8 window-attention calls (4 denoise passes x 60 layers, pass-major),
    each from the 757 new-token queries over the full 5788-slot window.
Also reported: the delta rebase of the whole 60-layer window (ms, GB/s), the
naive per-call upkeep path on the same shapes (re-rotate, re-quantise and
shift the window on all 240 calls), and the CPU oracle timed on a bounded
sample.  Inputs are seeded synthetic tensors (kv_cache_attention_ring_amd.inputs).

    python bench.py [--gpus 1] [--steps 42] [--warmup 5]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per denoise step (240 attn calls + KV upkeep); HBM GB/s and FP8 MFMA % of peak"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


# the sources the attention kernels are compiled from
KERNEL_SOURCES = ("attention.hip", "rowquant.h", "kvr_internal.h")


def kernel_code_digest(root=None):
    """sha256 of the attention kernels' sources with comments and whitespace
    removed: it changes with the code, not with its comments."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(root or ROOT, "kv_cache_attention_ring_amd", "csrc", name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update((name + "\n" + " ".join(src.split()) + "\n").encode())
    return h.hexdigest()


def counted_traffic(key="attn_kernel_traffic_bytes"):
    """HBM bytes per launch from the committed counter summary (the attention
    kernel's by default, or `attn_call_traffic_bytes` for the whole call), or
    None when the kernels' code has changed since the counters were taken."""
    import re
    prof = os.path.join(ROOT, "profiles", "attn_traffic_counters.md")
    try:
        text = open(prof).read()
        digest = kernel_code_digest()
    except OSError:
        return None
    m = re.search(r"kernel code sha256: ([0-9a-f]{64})", text)
    t = re.search(key + r": (\d+)", text)
    if not m or not t or m.group(1) != digest:
        return None
    return int(t.group(1))


def pct(sorted_vals, p):
    """p-th percentile (nearest rank) of an ascending list."""
    k = max(0, min(len(sorted_vals) - 1, math.ceil(p / 100.0 * len(sorted_vals) - 1e-9) - 1))
    return sorted_vals[k]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=42)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--naive-steps", type=int, default=3)
    ap.add_argument("--every-pass-steps", type=int, default=5,
                    help="steps timed with the chunk written again on every denoise pass (0 = skip)")
    ap.add_argument("--rebase-iters", type=int, default=20)
    ap.add_argument("--seed", type=int, default=20261105, help="base seed of the synthetic inputs")
    ap.add_argument("--pos-steps", type=int, default=10,
                    help="timed steps with the position form of the attention call (0 = skip)")
    ap.add_argument("--fused-steps", type=int, default=10,
                    help="steps with each layer's chunk written by its first attention call (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="replays of one whole step captured as a graph (0 = skip)")
    ap.add_argument("--rope3d-steps", type=int, default=10,
                    help="timed steps of the 3-D (frame, row, column) rotary form (0 = skip)")
    ap.add_argument("--splits", type=int, default=0, help="attention key splits (0 = default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB and exit "
                         "(reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--mix-mb", type=int, default=0,
                    help="only time PyTorch's bf16 -> FP8 conversion of this many MiB of bf16 (the write "
                         "kernel's 2:1 read:write mix, a reference rate) and exit")
    ap.add_argument("--attn-calls", type=int, default=0,
                    help="only time this many attention calls on one production-shape layer "
                         "(12 heads x 128, window 5788, 757 queries) and exit (for counter runs)")
    return ap.parse_args()


def attn_only(calls, splits):
    """One layer cache written with 8 chunks (full, wrapped ring), then `calls`
    timed attention calls after 3 warm-up calls: the attention kernel alone,
    for profiler counter runs."""
    import torch
    from kv_cache_attention_ring_amd import inputs
    from kv_cache_attention_ring_amd import kvring as K
    shp = inputs.PAGE_LAYER
    H, D, W, N = shp.n_heads, shp.head_dim, shp.window, shp.n_new
    cache = K.KVCache(1, H, D, W)
    rope = K.RopeTable(0, 12 * N, D)
    ring = K.kvr_ring_init()
    for s in range(8):
        k, v = inputs.torch_chunk(shp, s, 0, "cuda")
        K.kv_write_rope_quant(cache, ring, 0, k[0], v[0], rope)
        K.kvr_ring_after_write(ring, W, N)
    qs = [inputs.torch_queries(shp, 8, p, 0, "cuda") for p in range(4)]
    out = torch.empty_like(qs[0])
    need = K.attn_fp8_window_workspace_bytes(cache, N, W, splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    start = K.kvr_ring_logical_start(ring, W)
    lanes = K.kv_rope_query_lanes(K.rope_table_rows(rope, ring.pos_next - N, N))
    call = lambda i: K.attn_fp8_window_lanes(cache, 0, start, W, qs[i % 4], lanes, out=out, n_splits=splits,
                                             ws=ws)
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(calls):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / calls * 1e3
    print(json.dumps({"attention_calls": calls, "splits": splits or "default", "attention_call_us": round(us, 3),
                      "TFLOPs": round(4.0 * N * W * H * D / (us * 1e-6) / 1e12, 1)}), flush=True)


def copy_only(mib):
    """A plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE readings
    calibrate the counters used for the attention kernel's HBM traffic."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 13, "copy_ms": round(ms, 4),
                      "copy_GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def mix_only(mib):
    """PyTorch's own bf16 -> FP8 (E4M3) conversion of a mib-MiB bf16 tensor: a
    streaming kernel with the write kernel's 2:1 read:write byte mix, timed over
    four distinct sources so the reads come from HBM (a reference rate for the
    write kernel)."""
    import torch
    n = (mib << 20) // 2
    srcs = [torch.randn(n, device="cuda").to(torch.bfloat16) for _ in range(4)]
    dst = torch.empty(n, dtype=torch.float8_e4m3fn, device="cuda")
    for s in srcs:
        dst.copy_(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(12):
        dst.copy_(srcs[i % 4])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 12
    print(json.dumps({"mix_read_bytes": 2 * n, "mix_write_bytes": n, "mix_ms": round(ms, 4),
                      "mix_GBps_read_plus_write": round(3 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.copy_mb:
        copy_only(args.copy_mb)
        return
    if args.mix_mb:
        mix_only(args.mix_mb)
        return
    if args.attn_calls:
        attn_only(args.attn_calls, args.splits)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(the path shards over heads, see the design notes)"}))
        sys.exit(2)
    import torch

    from kv_cache_attention_ring_amd import inputs
    from kv_cache_attention_ring_amd import kvring as K

    dev = "cuda"
    inputs.set_base_seed(args.seed)
    shp = inputs.PAGE_STEP
    L, H, D, W, N, P = shp.n_layers, shp.n_heads, shp.head_dim, shp.window, shp.n_new, shp.passes
    pre = 8
    total_steps = (pre + args.warmup + args.steps + args.pos_steps + args.fused_steps + 4 +
                   (args.every_pass_steps + 1 if args.every_pass_steps > 0 else 0))
    pos_lo = -inputs.DELTA_MAX - 8 * N
    rope = K.RopeTable(pos_lo, total_steps * N - pos_lo, D, device=dev)
    cache = K.KVCache(L, H, D, W, device=dev)
    ring = K.kvr_ring_init()
    log(f"cache {cache.nbytes / 1e9:.3f} GB, rope table {rope.cs.numel() * 4 / 1e6:.1f} MB")

    pool = 8
    chunks = [inputs.torch_chunk(shp, s, 0, dev, n_layers=L) for s in range(pool)]
    qpool = [inputs.torch_queries(shp, 0, p, l, dev) for p in range(P) for l in range(L)]
    outs = [torch.empty((N, H, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ws_bytes = K.attn_fp8_window_workspace_bytes(cache, N, W, args.splits)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    for s in range(pre):
        k, v = chunks[s % pool]
        K.kv_write_rope_quant(cache, ring, 0, k, v, rope)
        K.kvr_ring_after_write(ring, W, N)
    torch.cuda.synchronize()
    log(f"prefilled {pre} chunks: head {ring.head}, n_valid {ring.n_valid}")

    def write(step_idx):
        k, v = chunks[step_idx % pool]
        K.kv_write_rope_quant(cache, ring, 0, k, v, rope)
        K.kvr_ring_after_write(ring, W, N)

    # The queries of every call of a step are the chunk's tokens at the chunk's
    # positions: their (cos, sin) rows (a slice of the rotary table) are put in
    # the attention kernel's load order once per step and shared by the 240 calls.
    cur = {}

    def set_lanes():
        cur["lanes"] = K.kv_rope_query_lanes(K.rope_table_rows(rope, ring.pos_next - N, N))

    def attend(layer, pss, start):
        K.attn_fp8_window_lanes(cache, layer, start, ring.n_valid, qpool[pss * L + layer], cur["lanes"],
                                out=outs[layer], n_splits=args.splits, ws=ws)

    def attend_pos(layer, pss, start):
        # the position form: the kernel forms the rotation of each query itself
        K.attn_fp8_window(cache, layer, start, ring.n_valid, qpool[pss * L + layer], ring.pos_next - N,
                          rope.base, out=outs[layer], n_splits=args.splits, ws=ws)

    def step(step_idx, call=None):
        write(step_idx)
        set_lanes()
        start = K.kvr_ring_logical_start(ring, W)
        for p in range(P):
            for layer in range(L):
                (call or attend)(layer, p, start)

    sidx = pre
    for _ in range(args.warmup):
        step(sidx)
        sidx += 1
    torch.cuda.synchronize()

    # ---- timed steps ---------------------------------------------------------
    # one event per step boundary (recording an event does not synchronise)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step(sidx)
        sidx += 1
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    log(f"{args.steps} steps: {ms_step:.4f} ms/step (wall {wall_ms / args.steps:.4f}); median "
        f"{pct(per_step, 50):.4f}, p90 {pct(per_step, 90):.4f}, max {per_step[-1]:.4f}")

    # ---- the same steps with the position form of the attention call ------------
    pos_ms = None
    if args.pos_steps > 0:
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for _ in range(args.pos_steps):
            step(sidx, attend_pos)
            sidx += 1
        p1.record()
        torch.cuda.synchronize()
        pos_ms = p0.elapsed_time(p1) / args.pos_steps
        log(f"position form: {pos_ms:.4f} ms/step")

    # ---- the chunk's write fused into each layer's first call -----------------
    # attn_fp8_window_write: the pass-0 call of layer l writes layer l's chunk
    # and attends over the window holding it (one launch pair, no separate
    # write); the other passes are the position-form calls.  Compared with the
    # position-form step above (same query form, one 60-layer write launch).
    fused = None
    if args.fused_steps > 0:
        wsf = torch.zeros(max(K.attn_fp8_window_write_workspace_bytes(cache, ring, N, args.splits), 256),
                          dtype=torch.uint8, device=dev)

        def step_fused(step_idx):
            k, v = chunks[step_idx % pool]
            before = ring.copy()
            K.kvr_ring_after_write(ring, W, N)
            start = K.kvr_ring_logical_start(ring, W)
            for p in range(P):
                for layer in range(L):
                    if p == 0:
                        K.attn_fp8_window_write(cache, before, layer, k[layer], v[layer], qpool[layer], rope,
                                                rope.base, out=outs[layer], n_splits=args.splits, ws=wsf)
                    else:
                        attend_pos(layer, p, start)

        step_fused(sidx)                         # untimed: first use of the fused kernels
        sidx += 1
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(args.fused_steps):
            step_fused(sidx)
            sidx += 1
        f1.record()
        torch.cuda.synchronize()
        ctl = wsf[-K.FUSED_SYNC_BYTES:].view(torch.int32)[:3].tolist()
        fused = {"ms_per_step": round(f0.elapsed_time(f1) / args.fused_steps, 5), "steps": args.fused_steps,
                 "control_block_after": ctl}
        log(f"write fused into each layer's first call: {fused['ms_per_step']:.4f} ms/step "
            f"(control block {ctl})")

    # ---- the chunk written on every denoise pass ------------------------------
    # each pass brings new K/V rows for the step's chunk: they are written to
    # the same slots at the same positions (ring state of the step's start)
    # before that pass's 60 calls; the ring advances once per step
    every_pass = None
    if args.every_pass_steps > 0:
        def step_every_pass(step_idx):
            before = ring.copy()
            K.kvr_ring_after_write(ring, W, N)
            set_lanes()
            start = K.kvr_ring_logical_start(ring, W)
            for p in range(P):
                k, v = chunks[(step_idx + p) % pool]
                K.kv_write_rope_quant(cache, before, 0, k, v, rope)
                for layer in range(L):
                    attend(layer, p, start)
        step_every_pass(sidx)
        sidx += 1
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        for _ in range(args.every_pass_steps):
            step_every_pass(sidx)
            sidx += 1
        q1.record()
        torch.cuda.synchronize()
        ep_ms = q0.elapsed_time(q1) / args.every_pass_steps
        every_pass = {"ms_per_step": round(ep_ms, 5), "steps": args.every_pass_steps,
                      "writes_per_step": P, "upkeep_bytes_per_step": P * L * (2 * N * H * D * 2 + 2 * N * H * D + 2 * N * H * 4)}
        log(f"write on every pass: {ep_ms:.4f} ms/step ({P} writes of 60 layers per step)")

    # ---- the whole step as one captured graph -----------------------------------
    # one step (the 60-layer write + 240 calls at the ring state of the step after
    # the last timed one) captured once and replayed; each replay redoes the same
    # work on the same slots, so its outputs must equal those of the same step
    # launched eagerly, bit for bit
    graph = None
    if args.graph_steps > 0:
        ring_g = ring.copy()
        kg, vg = chunks[sidx % pool]
        after = ring_g.copy()
        K.kvr_ring_after_write(after, W, N)
        start_g = K.kvr_ring_logical_start(after, W)
        lanes_g = K.kv_rope_query_lanes(K.rope_table_rows(rope, after.pos_next - N, N))

        def step_fixed():
            K.kv_write_rope_quant(cache, ring_g, 0, kg, vg, rope)
            for p in range(P):
                for layer in range(L):
                    K.attn_fp8_window_lanes(cache, layer, start_g, after.n_valid, qpool[p * L + layer], lanes_g,
                                            out=outs[layer], n_splits=args.splits, ws=ws)
        step_fixed()
        torch.cuda.synchronize()
        eager = [o.clone() for o in outs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_fixed()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_fixed()
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(outs, eager))
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.graph_steps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.graph_steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.graph_steps):
            step_fixed()
        e1.record()
        torch.cuda.synchronize()
        ems = e0.elapsed_time(e1) / args.graph_steps
        graph = {"ms_per_step_replayed": round(gms, 5), "ms_per_step_launched": round(ems, 5),
                 "steps": args.graph_steps, "replay_equals_eager": bool(same)}
        log(f"whole step as a graph: {gms:.4f} ms/step replayed, {ems:.4f} launched; outputs equal: {same}")
        del g

    # ---- per-kernel times, measured with events on the launch stream -----------
    # (1) every launch of one kind back to back between two events: the average
    #     launch duration of the attention kernel alone (the call's first launch,
    #     attn_fp8_window_partial), of the split merge alone, and of whole calls;
    # (2) one event pair around each whole call, for the per-call percentiles.
    def batch_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start = K.kvr_ring_logical_start(ring, W)
        e0.record()
        for p in range(P):
            for layer in range(L):
                fn(layer, p, start)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (P * L)

    def partial(layer, p, start):
        K.attn_fp8_window_lanes_partial(cache, layer, start, ring.n_valid, qpool[p * L + layer], cur["lanes"],
                                        out=outs[layer], n_splits=args.splits, ws=ws)

    def partial_pos(layer, p, start):
        K.attn_fp8_window_partial(cache, layer, start, ring.n_valid, qpool[p * L + layer], ring.pos_next - N,
                                  rope.base, out=outs[layer], n_splits=args.splits, ws=ws)

    def merge(layer, p, start):
        K.attn_fp8_window_merge(cache, N, ring.n_valid, outs[layer], n_splits=args.splits, ws=ws)

    kern_ms = sum(batch_ms(partial) for _ in range(2)) / 2
    kern_pos_ms = sum(batch_ms(partial_pos) for _ in range(2)) / 2
    # the merge alone takes less GPU time than the host needs to submit one call
    # through the binding, so merges launched back to back measure the host; the
    # merge's own duration comes from a graph of the 60 layers' merges replayed
    # P times (the same kernel launches, no host work between them)
    merge_host_ms = sum(batch_ms(merge) for _ in range(2)) / 2
    start_m = K.kvr_ring_logical_start(ring, W)
    side_m = torch.cuda.Stream()
    side_m.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side_m):
        for layer in range(L):
            merge(layer, 0, start_m)
    torch.cuda.current_stream().wait_stream(side_m)
    torch.cuda.synchronize()
    g_m = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_m):
        for layer in range(L):
            merge(layer, 0, start_m)
    g_m.replay()
    torch.cuda.synchronize()
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record()
    for _ in range(P):
        g_m.replay()
    m1.record()
    torch.cuda.synchronize()
    merge_ms = m0.elapsed_time(m1) / (P * L)
    del g_m
    call_batch_ms = sum(batch_ms(attend) for _ in range(2)) / 2
    n_meas = 2
    w_ms, a_ms = [], []
    # ring state before the writes below (their positions lie inside the rotary table)
    ring_w = K.kvr_ring(ring.head, ring.n_valid, ring.pos_next)
    chunk_w = chunks[sidx % pool]
    for _ in range(n_meas):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 + 2 * P * L)]
        e[0].record()
        write(sidx)
        e[1].record()
        set_lanes()
        start = K.kvr_ring_logical_start(ring, W)
        i = 2
        for p in range(P):
            for layer in range(L):
                e[i].record()
                attend(layer, p, start)
                e[i + 1].record()
                i += 2
        torch.cuda.synchronize()
        sidx += 1
        w_ms.append(e[0].elapsed_time(e[1]))
        a_ms += [e[j].elapsed_time(e[j + 1]) for j in range(2, len(e), 2)]
    write_in_step_ms = sum(w_ms) / len(w_ms)
    # the write kernel's own rate: launches back to back between two events (a write
    # without the ring bookkeeping stores rows in the same slots each time); each
    # launch takes the next chunk of the pool (8 x 280 MB of bf16 rows), so its
    # source rows come from HBM rather than from the 256 MB last-level cache; the
    # single launch inside a step above also counts the host's submission gap
    # after the preceding synchronisation
    K.kv_write_rope_quant(cache, ring_w, 0, chunk_w[0], chunk_w[1], rope)
    torch.cuda.synchronize()
    we0, we1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_w = 2 * pool
    we0.record()
    for i in range(n_w):
        k_w, v_w = chunks[(sidx + 1 + i) % pool]
        K.kv_write_rope_quant(cache, ring_w, 0, k_w, v_w, rope)
    we1.record()
    torch.cuda.synchronize()
    write_ms = we0.elapsed_time(we1) / n_w
    attn_ms = call_batch_ms
    a_sorted = sorted(a_ms)
    attn_flops = 4.0 * N * W * H * D
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    kern_tflops = attn_flops / (kern_ms * 1e-3) / 1e12
    write_bytes = L * (2 * N * H * D * 2 + 2 * N * H * D + 2 * N * H * 4)
    write_gbs = write_bytes / (write_ms * 1e-3) / 1e9
    log(f"write (60 layers) {write_ms * 1e3:.1f} us = {write_gbs:.0f} GB/s (one launch inside a step "
        f"{write_in_step_ms * 1e3:.1f} us); attention call "
        f"{attn_ms * 1e3:.2f} us = {attn_tflops:.1f} TFLOP/s (kernel {kern_ms * 1e3:.2f} us = "
        f"{kern_tflops:.1f} TFLOP/s, merge {merge_ms * 1e3:.2f} us; launched one by one through the binding "
        f"the merges take {merge_host_ms * 1e3:.2f} us each, the host's submission time)")

    # ---- rebase (position reset) -------------------------------------------------
    delta = inputs.rebase_delta()
    reb_bytes = 2 * (L * H * W * D + L * H * W * 4)
    for i in range(5):
        K.kv_delta_rebase(cache, ring, 0, L, delta if i % 2 == 0 else -delta)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for i in range(args.rebase_iters):
        K.kv_delta_rebase(cache, ring, 0, L, delta if i % 2 == 0 else -delta)
    r1.record()
    torch.cuda.synchronize()
    reb_ms = r0.elapsed_time(r1) / args.rebase_iters
    reb_gbs = reb_bytes / (reb_ms * 1e-3) / 1e9
    # a reset comes once every 42 steps, right after a step's attention calls:
    # one rebase timed on its own after a full step (and one back, untimed)
    step(sidx)
    sidx += 1
    r0.record()
    K.kv_delta_rebase(cache, ring, 0, L, delta)
    r1.record()
    K.kv_delta_rebase(cache, ring, 0, L, -delta)
    torch.cuda.synchronize()
    reb_single_ms = r0.elapsed_time(r1)
    log(f"rebase delta={delta}: {reb_ms:.4f} ms = {reb_gbs:.0f} GB/s (one after a step: {reb_single_ms:.4f} ms)")

    # ---- naive per-call upkeep -------------------------------------------------------
    naive = None
    if not args.no_naive and args.naive_steps > 0:
        naive = run_naive(args, K, inputs, shp, rope, chunks, qpool, outs, ws, torch, dev, pre)

    # ---- CPU oracle on a bounded sample -----------------------------------------------
    # ---- the 3-D (frame, row, column) rotary form ----------------------------------
    # the same step with every token at (t, y, x): one latent frame per chunk on a
    # 28-column grid; per step one (cos, sin) row fill for the chunk's tokens, the
    # row-driven write of 60 layers and 240 row-driven attention calls; then the
    # frame-only rebase of all 60 layers
    rope3d = None
    if args.rope3d_steps > 0:
        npr = inputs.axis_pairs(D)
        ring3 = ring.copy()

        def step3d(frame, lanes=True):
            # one row fill per step; the queries' rows are rearranged once into
            # the attention kernel's load layout and shared by all 240 calls
            rows = K.Rope3DRows(inputs.chunk_coords(N, frame), D, npr)
            qr = K.kv_rope_query_lanes(rows.cs) if lanes else None
            k, v = chunks[frame % pool]
            K.kv_write_rope_quant_rows(cache, ring3, 0, k, v, rows.cs)
            K.kvr_ring_after_write(ring3, W, N)
            start = K.kvr_ring_logical_start(ring3, W)
            for p in range(P):
                for layer in range(L):
                    if lanes:
                        K.attn_fp8_window_lanes(cache, layer, start, ring3.n_valid, qpool[p * L + layer], qr,
                                                out=outs[layer], n_splits=args.splits, ws=ws)
                    else:
                        K.attn_fp8_window_rows(cache, layer, start, ring3.n_valid, qpool[p * L + layer], rows.cs,
                                               out=outs[layer], n_splits=args.splits, ws=ws)
        for f in range(2):
            step3d(f)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for f in range(args.rope3d_steps):
            step3d(2 + f)
        t1.record()
        torch.cuda.synchronize()
        ms3 = t0.elapsed_time(t1) / args.rope3d_steps
        t0.record()
        for f in range(args.rope3d_steps):
            step3d(2 + args.rope3d_steps + f, lanes=False)
        t1.record()
        torch.cuda.synchronize()
        ms3_rows = t0.elapsed_time(t1) / args.rope3d_steps
        d_t = inputs.rebase_delta_t()
        for i in range(3):
            K.kv_delta_rebase_axes(cache, ring3, 0, L, (d_t if i % 2 == 0 else -d_t, 0, 0), npr)
        torch.cuda.synchronize()
        r0.record()
        for i in range(args.rebase_iters):
            K.kv_delta_rebase_axes(cache, ring3, 0, L, (d_t if i % 2 == 0 else -d_t, 0, 0), npr)
        r1.record()
        torch.cuda.synchronize()
        reb3 = r0.elapsed_time(r1) / args.rebase_iters
        rope3d = {"ms_per_step": round(ms3, 5), "ms_per_step_rows_layout": round(ms3_rows, 5),
                  "steps": args.rope3d_steps, "axis_pairs": list(npr),
                  "frame_cols": inputs.FRAME_COLS, "frame_rebase_ms": round(reb3, 4),
                  "frame_rebase_GBps": round(reb_bytes / (reb3 * 1e-3) / 1e9, 1), "frame_delta": d_t}
        log(f"3-D rotary form: {ms3:.4f} ms/step ({ms3_rows:.4f} with the rows read in their own layout); "
            f"frame rebase by {d_t}: {reb3:.4f} ms")

        # the window as a fixed 489-token prefix (one frame at t = -1, written
        # once) and a ring of 7 x 757 slots; attention sees prefix + ring
        n_pre = W - 7 * N
        cap = W - n_pre
        pcache = K.KVCache(L, H, D, W, device=dev, n_prefix=n_pre)
        jj = torch.arange(n_pre)
        prow = K.Rope3DRows(torch.stack([torch.full((n_pre,), -1), jj // inputs.FRAME_COLS,
                                         jj % inputs.FRAME_COLS], 1), D, npr)
        pk, pv = inputs.torch_chunk(inputs.Shape("prefix", L, H, D, W, n_pre), 0, 0, dev, n_layers=L)
        K.kv_write_prefix_rows(pcache, 0, 0, pk, pv, prow.cs)
        pring = K.kvr_ring_init()

        def step_prefix(frame):
            rows = K.Rope3DRows(inputs.chunk_coords(N, frame), D, npr)
            qr = K.kv_rope_query_lanes(rows.cs)
            k, v = chunks[frame % pool]
            K.kv_write_rope_quant_rows(pcache, pring, 0, k, v, rows.cs)
            K.kvr_ring_after_write(pring, cap, N)
            start = K.kvr_ring_logical_start(pring, cap)
            for p in range(P):
                for layer in range(L):
                    K.attn_fp8_window_lanes(pcache, layer, start, pring.n_valid, qpool[p * L + layer], qr,
                                            out=outs[layer], n_splits=args.splits, ws=ws)
        for f in range(8):                                   # fill the ring
            step_prefix(f)
        torch.cuda.synchronize()
        t0.record()
        for f in range(args.rope3d_steps):
            step_prefix(8 + f)
        t1.record()
        torch.cuda.synchronize()
        msp = t0.elapsed_time(t1) / args.rope3d_steps
        r0.record()
        for i in range(args.rebase_iters):
            K.kv_delta_rebase_axes(pcache, pring, 0, L, (d_t if i % 2 == 0 else -d_t, 0, 0), npr)
        r1.record()
        torch.cuda.synchronize()
        rebp = r0.elapsed_time(r1) / args.rebase_iters
        rebp_bytes = 2 * (L * H * cap * D + L * H * cap * 4)
        rope3d["prefix"] = {"prefix_slots": n_pre, "ring_slots": cap, "ms_per_step": round(msp, 5),
                            "frame_rebase_ms": round(rebp, 4),
                            "frame_rebase_GBps": round(rebp_bytes / (rebp * 1e-3) / 1e9, 1)}
        log(f"3-D form with a {n_pre}-slot prefix: {msp:.4f} ms/step; frame rebase of the ring {rebp:.4f} ms")
        del pcache, pk, pv

    if naive is not None:
        # the before/after comparison of the two upkeep designs on the same shapes
        naive["upkeep_ratio_naive_over_write"] = round(naive["upkeep_ms_per_step"] / write_ms, 1)
        naive["step_ratio_naive_over_ring"] = round(naive["ms_per_step"] / ms_step, 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(K, inputs, shp, cache, qpool, ring, chunks, torch)

    line = {
        "metric": METRIC,
        "value": round(ms_step, 5),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": "full denoise step: 60 layer caches x 12 heads x head_dim 128, ring window "
                        "5788 slots, 757 new tokens per step; one 60-layer write + 240 attention calls",
            "layers": L, "heads": H, "head_dim": D, "window": W, "new_tokens": N, "passes": P,
            "attention_splits": args.splits or "default", "seed": args.seed,
        },
        "roofline": {
            "kernel": "attn_kernel<128, bf16 Q, rotation rows> (attn_fp8_window_lanes_partial), per launch",
            "bound": "mfma",
            "achieved": round(kern_tflops, 2),
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / FP8_PEAK_TFLOPS, 4),
            "traffic": counted_traffic(),
        },
        "step_ms": {"mean": round(ms_step, 5), "median": round(pct(per_step, 50), 5),
                    "p90": round(pct(per_step, 90), 5), "max": round(per_step[-1], 5)},
        "breakdown": {
            "write_60_layers_us": round(write_ms * 1e3, 2),
            "write_60_layers_us_in_step": round(write_in_step_ms * 1e3, 2),
            "write_GBps": round(write_gbs, 1),
            "write_frac_hbm": round(write_gbs / HBM_PEAK_GBS, 4),
            "attention_call_us": round(attn_ms * 1e3, 3),
            "attention_call_TFLOPs": round(attn_tflops, 2),
            "attention_kernel_us": round(kern_ms * 1e3, 3),
            "attention_kernel_us_position_form": round(kern_pos_ms * 1e3, 3),
            "attention_merge_us": round(merge_ms * 1e3, 3),
            "attention_merge_us_host_bound": round(merge_host_ms * 1e3, 3),
            "attention_call_traffic_bytes": counted_traffic("attn_call_traffic_bytes"),
            "attention_call_us_median_single": round(pct(a_sorted, 50) * 1e3, 3),
            "attention_call_us_p90_single": round(pct(a_sorted, 90) * 1e3, 3),
            "upkeep_share_of_step": round(write_ms / ms_step, 4),
            # each figure above comes from its own loop of launches back to back,
            # so they are rates, not parts of one step (240 back-to-back calls
            # alone, below, need not add up with the write to ms_per_step); the
            # step's own split is step_split
            "attention_ms_per_step_back_to_back": round(attn_ms * P * L, 4),
            "step_split": {"write_ms": round(write_in_step_ms, 4),
                           "attention_ms": round(ms_step - write_in_step_ms, 4),
                           "note": "write_ms: one event pair around the write inside a step; attention_ms: "
                                   "the step time minus it (the 240 calls and the query rows' rearrangement)"},
            "rebase_ms": round(reb_ms, 4),
            "rebase_GBps": round(reb_gbs, 1),
            "rebase_frac_hbm": round(reb_gbs / HBM_PEAK_GBS, 4),
            "rebase_ms_single_after_step": round(reb_single_ms, 4),
            "rebase_delta": delta,
        },
        "position_form": None if pos_ms is None else {"ms_per_step": round(pos_ms, 5), "steps": args.pos_steps},
        "fused_write": fused,
        "naive": naive,
        "write_every_pass": every_pass,
        "graph": graph,
        "rope3d": rope3d,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_naive(args, K, inputs, shp, rope, chunks, qpool, outs, ws, torch, dev, pre):
    """Naive path: on every one of the 240 calls, rebuild the shifted bf16 window
    and re-rotate / re-quantise all of it, then attend over the linear window."""
    L, H, D, W, N, P = shp.n_layers, shp.n_heads, shp.head_dim, shp.window, shp.n_new, shp.passes
    wins = [[torch.zeros((H, W, D), dtype=torch.bfloat16, device=dev) for _ in range(4)]
            for _ in range(L)]
    lin = K.KVCache(L, H, D, W, device=dev)
    ring = K.kvr_ring_init()
    ping = [0]

    def upkeep(layer, k, v):
        a = wins[layer]
        s = ping[0]
        K.naive_upkeep(a[2 * s], a[2 * s + 1], k[layer], v[layer], ring.n_valid, ring.pos_next, rope,
                       a[2 - 2 * s], a[3 - 2 * s], lin.k_codes[layer], lin.v_codes[layer],
                       lin.k_scales[layer], lin.v_scales[layer])

    for s in range(pre):
        k, v = chunks[s % len(chunks)]
        for layer in range(L):
            upkeep(layer, k, v)
        ping[0] = 1 - ping[0]
        K.kvr_ring_after_write(ring, W, N)
    torch.cuda.synchronize()

    def nstep(sidx, with_attn=True):
        k, v = chunks[sidx % len(chunks)]
        n_valid = min(ring.n_valid + N, W)
        # the same attention call as the ring path (query rows in load order)
        lanes = K.kv_rope_query_lanes(K.rope_table_rows(rope, ring.pos_next, N)) if with_attn else None
        for p in range(P):
            for layer in range(L):
                upkeep(layer, k, v)
                if with_attn:
                    K.attn_fp8_window_lanes(lin, layer, 0, n_valid, qpool[p * L + layer], lanes,
                                            out=outs[layer], n_splits=args.splits, ws=ws)
        ping[0] = 1 - ping[0]
        K.kvr_ring_after_write(ring, W, N)

    sidx = pre
    nstep(sidx)
    sidx += 1
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.naive_steps):
        nstep(sidx)
        sidx += 1
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.naive_steps
    e0.record()
    for _ in range(args.naive_steps):
        nstep(sidx, with_attn=False)
        sidx += 1
    e1.record()
    torch.cuda.synchronize()
    up_ms = e0.elapsed_time(e1) / args.naive_steps
    call_bytes = 2 * H * W * D * 2 * 2 + 2 * H * W * D + 2 * H * W * 4
    gbs = P * L * call_bytes / (up_ms * 1e-3) / 1e9
    log(f"naive: {ms_step:.3f} ms/step, upkeep {up_ms:.3f} ms/step = {gbs:.0f} GB/s")
    del wins, lin
    return {"ms_per_step": round(ms_step, 4), "upkeep_ms_per_step": round(up_ms, 4),
            "upkeep_GBps": round(gbs, 1), "upkeep_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_call": call_bytes}


def cpu_baseline(K, inputs, shp, cache, qpool, ring, chunks, torch):
    """The oracle, as it stands: one full attention call (x240, extrapolated),
    and the step's 60-layer write, 60-layer rebase and 240 naive rebuilds
    timed in full at their own shapes."""
    import numpy as np

    import oracle
    L, H, D, W, N, P = shp.n_layers, shp.n_heads, shp.head_dim, shp.window, shp.n_new, shp.passes
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    oracle.set_threads(int(os.environ["OMP_NUM_THREADS"]))
    # every layer's cache on the host (1.1 GB), and one chunk of all layers
    lcs = []
    for layer in range(L):
        lc = oracle.LayerCache(H, D, W)
        lc.k_codes[:] = cache.k_codes[layer].cpu().numpy()
        lc.v_codes[:] = cache.v_codes[layer].cpu().numpy()
        lc.k_scales[:] = cache.k_scales[layer].cpu().numpy()
        lc.v_scales[:] = cache.v_scales[layer].cpu().numpy()
        lcs.append(lc)
    lc = lcs[0]
    q = qpool[0].float().cpu().numpy()
    k, v = chunks[0]
    kall, vall = k.float().cpu().numpy(), v.float().cpu().numpy()          # [L][N][H][D]
    kn, vn = kall[0], vall[0]
    start = K.kvr_ring_logical_start(ring, W)
    t = time.perf_counter()
    oracle.attention(lc, start, ring.n_valid, q, ring.pos_next - N)
    t_attn = time.perf_counter() - t
    # the step's write: the chunk into all 60 layers (the slots after the window)
    total = ring.pos_next                      # token count consistent with the positions (no reset yet)
    t = time.perf_counter()
    for layer in range(L):
        oracle.write(lcs[layer], total, ring.pos_next, kall[layer], vall[layer])
    t_write_step = time.perf_counter() - t
    # a rebase of all 60 layers' windows
    delta = inputs.rebase_delta()
    t = time.perf_counter()
    for layer in range(L):
        oracle.rebase(lcs[layer], start, ring.n_valid, delta)
    t_rebase_step = time.perf_counter() - t
    # the naive path's 240 per-call rebuilds of a step (the same window shape each call)
    lin_k = np.ascontiguousarray(np.repeat(kn[:1].transpose(1, 0, 2), W, axis=1))   # [H][W][D] fp32
    lin_v = np.ascontiguousarray(np.repeat(vn[:1].transpose(1, 0, 2), W, axis=1))
    t = time.perf_counter()
    for _ in range(P * L):
        oracle.naive(lin_k, lin_v, kn, vn, W, ring.pos_next)
    t_naive_step = time.perf_counter() - t
    ms = P * L * t_attn * 1e3 + t_write_step * 1e3
    threads = oracle.max_threads()
    log(f"oracle ({threads} threads): attention call {t_attn:.2f} s (x{P * L} extrapolated); write of {L} layers "
        f"{t_write_step * 1e3:.0f} ms -> {ms:.0f} ms/step; rebase of {L} layers {t_rebase_step * 1e3:.0f} ms, "
        f"naive upkeep of a step ({P * L} rebuilds) {t_naive_step:.2f} s")
    # the same oracle on one thread: a sixteenth of the call's (query, head)
    # rows (every 16th row) and one layer's write, scaled to a step
    one = {}
    oracle.set_threads(1)
    try:
        rows = [(i, h) for i in range(N) for h in range(H)][::16]
        t = time.perf_counter()
        oracle.attention(lc, start, ring.n_valid, q, ring.pos_next - N, rows=rows)
        t_rows = time.perf_counter() - t
        t = time.perf_counter()
        oracle.write(lc.copy(), total, ring.pos_next, kn, vn)
        t_write1 = time.perf_counter() - t
        t_attn1 = t_rows * (N * H) / len(rows)
        ms1 = (P * L * t_attn1 + L * t_write1) * 1e3
        one = {"value": round(ms1, 1), "unit": "ms/step", "cores": 1,
               "sample": f"{len(rows)} of the call's {N * H} (query, head) rows (every 16th) and one layer's "
                         "write on one thread, scaled to the whole call, x240 calls and x60 layers (extrapolated)",
               "attention_call_s": round(t_attn1, 2), "layer_write_ms": round(t_write1 * 1e3, 2)}
        log(f"oracle (1 thread): {len(rows)} rows in {t_rows:.2f} s -> attention call {t_attn1:.1f} s, "
            f"layer write {t_write1 * 1e3:.1f} ms -> {ms1:.0f} ms/step")
    finally:
        oracle.set_threads(threads)
    return {"value": round(ms, 1), "unit": "ms/step", "cores": threads, "kind": "oracle",
            "sample": "one full attention call (757 queries x 12 heads x 5788 keys, fp64) timed and scaled "
                      "x240 calls (extrapolated), plus the step's write of all 60 layers timed in full; also "
                      "the 60-layer rebase and the naive path's 240 rebuilds of a step, timed in full",
            "attention_call_s": round(t_attn, 3), "write_60_layers_ms": round(t_write_step * 1e3, 1),
            "rebase_60_layers_ms": round(t_rebase_step * 1e3, 1),
            "naive_upkeep_ms_per_step": round(t_naive_step * 1e3, 1),
            "single_thread": one}


if __name__ == "__main__":
    main()
