"""bench.py on the CPU: the one-GPU contract and the algorithmic byte counts
that its roofline divides by (the figures the measurement plan states for the
five configurations)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes():
    b = _bench_module()
    # long prefill: 1 KiB per token-head plus 128 KiB of state per request-head
    assert b.prefill_bytes(131072, 64, 1) == 8_598_323_200
    # decode B=256 and chain verify B=128 x 5 at H=64
    assert b.step_bytes(256, 64, 256) == 2_164_260_864
    assert b.step_bytes(128, 64, 640) == 1_115_684_864
    # tree verify: one state read per request-head, one state write per draft-head
    assert b.tree_bytes(128, 5, 64) == 3_263_168_512


def test_useful_flops_per_token_head():
    b = _bench_module()
    # 4 d^2 (state update and inter term) + 2 C d (causal-half intra term), C = 64
    assert b.prefill_useful_flops(1, 1) == 4 * 128 * 128 + 2 * 64 * 128
    assert b.prefill_useful_flops(131072, 64) == 131072 * 64 * 81920


def test_code_text_drops_comments_and_spacing_only():
    b = _bench_module()
    src = 'int a = 1; // note\n/* block\n   comment */  const char *s = "x // y \\" z";\n\tint  b;\n'
    assert b.code_text(src) == 'int a = 1; const char *s = "x // y \\" z"; int b;'
    # a comment or layout edit keeps the digest, a code edit changes it
    assert b.code_text("x = y + 1; // one") == b.code_text("x = y + 1;   /* other */")
    assert b.code_text("x = y + 1;") != b.code_text("x = y + 2;")


def test_committed_traffic_entries_are_well_formed():
    import json
    b = _bench_module()
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert 0.99 < t["copy_read_scale"] < 1.01 and 0.99 < t["copy_write_scale"] < 1.01
    for kernel in b.KERNEL_SOURCES:
        for workload, e in t[kernel].items():
            assert len(e["source_sha256"]) == 64, (kernel, workload)
            assert e["traffic_bytes"] == e["read_bytes"] + e["write_bytes"]
            assert e["read_bytes"] > 0 and e["write_bytes"] > 0
            assert e["traffic_bytes"] >= 0.99 * e["algorithmic_bytes"], (kernel, workload)
