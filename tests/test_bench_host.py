"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the traffic
figure tied to the kernel code it was counted on, the percentile rule."""
import importlib.util
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_counts_belong_to_the_code_they_were_taken_on(tmp_path):
    b = _bench()
    # the committed counters match the committed kernel code
    kern = b.counted_traffic()
    call = b.counted_traffic("attn_call_traffic_bytes")
    assert kern is not None and call is not None and call > kern > 23_000_000
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "attn_traffic_counters.md"), tmp_path / "profiles")
    src_dir = tmp_path / "kv_cache_attention_ring_amd" / "csrc"
    src_dir.mkdir(parents=True)
    for name in b.KERNEL_SOURCES[1:]:
        shutil.copy(os.path.join(ROOT, "kv_cache_attention_ring_amd", "csrc", name), src_dir)
    with open(os.path.join(ROOT, "kv_cache_attention_ring_amd", "csrc", "attention.hip")) as f:
        src = f.read()
    b.ROOT = str(tmp_path)
    # a comment or a blank line more keeps them
    (src_dir / "attention.hip").write_text(src + "\n// a note\n/* and\n another */\n\n")
    assert b.counted_traffic() == kern
    # a code change voids them
    (src_dir / "attention.hip").write_text(src + "\nstatic int one_more;\n")
    assert b.counted_traffic() is None


def test_percentile_is_nearest_rank():
    b = _bench()
    v = list(range(1, 11))
    assert b.pct(v, 50) == 5 and b.pct(v, 90) == 9 and b.pct(v, 100) == 10 and b.pct(v, 0) == 1
    assert b.pct([7.0], 90) == 7.0
