#!/usr/bin/env python3
"""Benchmark of the seg_la hot path on one MI355X.

One step is one pass over every entry point, each on its own synthetic batch
already resident in HBM, launched back to back on one stream:
  * la_prefill  long prefill: 1 request x 131072 tokens, H=64, d=128, bf16
  * la_decode   256 requests x 1 token, H=64, bf16, pool of 512 fp32 states
  * la_verify   128 requests x 5 chained draft tokens, H=64, bf16, pool of 256
HIP events on that stream bracket every call inside the timed region, so each
entry point's own rate is reported beside the step time.  `value` is the
prefill rate in tokens/s; the decode rate (requests/s) and the verify rate
are reported in their own objects, each with its roofline.

After the timed steps, outside the step time:
  * la_verify_tree  the verify batch (128 x 5 drafts, H=64) as a seeded random
           draft tree per request, writing every per-position state
  * graph  32 small decode calls (1 request, H=64, one pool per call, as one
           per layer) launched eagerly and as one captured HIP graph: host
           launch overhead per call, eager vs graph
  * prefill variants on slices of the long-prefill tensors (made on the
    device): a state-tracking snapshot at token 65536; grouped heads with
    8 kv heads for the 64 query heads; head_dim 64 over 16384 tokens

Algorithmic traffic (bytes the method must move; bf16 I/O, fp32 state):
  prefill: 1024 B per (token, head) for q, k, v in and o out, plus 128 KiB of
           state read + write per (request, head)
  decode / verify: 128 KiB of state read + write per (request, head) plus
           1 KiB of q, k, v, o per (token, head)
  tree verify: 64 KiB state read per (request, head), 64 KiB state written
           per (draft, head), 1 KiB of q, k, v, o per (draft, head)
Peaks: HBM 8 TB/s, bf16 dense MFMA 2.5 PFLOP/s.

The CPU baseline runs the fp64 oracle on the host cores over a bounded sample
of the prefill workload (four heads per core, at most all 64, every token),
scaled to tokens/s of the whole workload, and over the whole decode and
verify batches (requests/s).

The pages this path comes from publish correctness tolerances for it but no
throughput figure on any hardware, so `vs_baseline` is null.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "prefill tokens/s (MFMA %) + decode req/s (HBM GB/s %), H=64 d=128"
D = 128
STATE_BYTES = D * D * 4


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "prefill_chunked_kernel": ["prefill_chunked.hip", "common.h", "host_logic.h"],
    "recurrent_kernel<bf16>": ["recurrent.hip", "common.h"],
    "tree_kernel<bf16>": ["recurrent.hip", "common.h"],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_text(src):
    """C/C++ source without its comments and with every run of white space
    made one blank: the part of a file that can change the compiled kernel,
    so that editing a comment does not detach the committed counters."""
    out, i, n, in_str = [], 0, len(src), False
    while i < n:
        c = src[i]
        if in_str:
            out.append(c)
            if c == "\\" and i + 1 < n:
                out.append(src[i + 1])
                i += 2
                continue
            in_str = c != '"'
            i += 1
        elif c == '"':
            in_str = True
            out.append(c)
            i += 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_sha256(kernel):
    """sha256 of the code (code_text) of the kernel's source files, in order."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "linear_attention_amd", "csrc", name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode("utf-8"))
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counts of L2-to-memory
    requests (profiles/traffic.json: read requests by size class, write
    requests and their 64-byte share, scaled by a plain copy's counts), or None
    when they were taken on a different version of the kernel's source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f).get(kernel, {}).get(workload)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("source_sha256") != source_sha256(kernel):
        return None
    return entry.get("traffic_bytes")


def prefill_bytes(T, H, B):
    return T * H * 4 * D * 2 + B * H * 2 * STATE_BYTES


def prefill_useful_flops(T, H, chunk=64):
    # per (token, head): state update 2d^2, inter-chunk term 2d^2, causal-half
    # intra-chunk terms 2*chunk*d (scores and values), with a 64-token chunk
    return T * H * (4 * D * D + 2 * chunk * D)


def step_bytes(B, H, tokens):
    return B * H * 2 * STATE_BYTES + tokens * H * 4 * D * 2


def tree_bytes(B, n, H):
    return B * H * STATE_BYTES + B * n * H * STATE_BYTES + B * n * H * 4 * D * 2


def prefill_variants(ms, ms_min, T, H):
    """Rates of the prefill variants timed after the steps."""
    if "prefill_track" not in ms:
        return None
    T64 = 16384
    gqa_bytes = T * H * (2 * D * 2) + T * 8 * (2 * D * 2) + H * 2 * STATE_BYTES
    d64_bytes = T64 * H * 4 * 64 * 2 + H * 2 * 64 * 64 * 4
    tp8_bytes = prefill_bytes(T, 8, 1)
    return {
        "track_snapshot": {"workload": f"long prefill T={T} H={H} d={D}, snapshot after {T // 2} tokens",
                           "avg_ms": ms["prefill_track"], "min_ms": ms_min["prefill_track"],
                           "tokens_per_s": T / (ms["prefill_track"] * 1e-3),
                           "vs_untracked": ms["prefill"] / ms["prefill_track"]},
        "grouped_heads": {"workload": f"prefill T={T} H={H} Hkv=8 d={D}", "avg_ms": ms["prefill_gqa"],
                          "min_ms": ms_min["prefill_gqa"], "tokens_per_s": T / (ms["prefill_gqa"] * 1e-3),
                          "hbm_gbs": gqa_bytes / (ms["prefill_gqa"] * 1e-3) / 1e9},
        "head_dim_64": {"workload": f"prefill T={T64} H={H} d=64 (chunked kernel, 2 column blocks per head, "
                                    "2 sequence segments)",
                        "avg_ms": ms["prefill_d64"], "min_ms": ms_min["prefill_d64"],
                        "tokens_per_s": T64 / (ms["prefill_d64"] * 1e-3),
                        "hbm_gbs": d64_bytes / (ms["prefill_d64"] * 1e-3) / 1e9,
                        "hbm_frac": d64_bytes / (ms["prefill_d64"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "unsegmented_avg_ms": ms["prefill_d64_unseg"],
                        "segment_speedup": ms["prefill_d64_unseg"] / ms["prefill_d64"]},
        "tp8_share": {"workload": f"prefill T={T} H=8 d={D}: heads 0..7 of the long request, one GPU's "
                                  "share at 8-way head parallelism (8 sequence segments)",
                      "avg_ms": ms["prefill_tp8"], "min_ms": ms_min["prefill_tp8"],
                      "tokens_per_s": T / (ms["prefill_tp8"] * 1e-3),
                      "hbm_gbs": tp8_bytes / (ms["prefill_tp8"] * 1e-3) / 1e9,
                      "hbm_frac": tp8_bytes / (ms["prefill_tp8"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "unsegmented_avg_ms": ms["prefill_tp8_unseg"],
                      "segment_speedup": ms["prefill_tp8_unseg"] / ms["prefill_tp8"]},
        "fp32": {"workload": f"prefill T={T64} H={H} d={D} fp32 (token-recurrent kernel, one workgroup per head)",
                 "avg_ms": ms["prefill_fp32"], "min_ms": ms_min["prefill_fp32"],
                 "tokens_per_s": T64 / (ms["prefill_fp32"] * 1e-3)},
    }


def varlen_prefill(ms, ms_min, wl):
    """Rate of the packed varlen prefill (8 requests of U[1, 4096] tokens, H=16)."""
    T, H, B = wl.total_tokens, wl.num_heads, wl.batch
    nbytes = prefill_bytes(T, H, B)
    gbs = nbytes / (ms["prefill_varlen"] * 1e-3) / 1e9
    return {"workload": f"varlen prefill H={H} d={D} bf16, {B} requests, lengths "
                        f"{[int(wl.cu_seqlens[i + 1] - wl.cu_seqlens[i]) for i in range(B)]}, T={T}",
            "avg_ms": ms["prefill_varlen"], "min_ms": ms_min["prefill_varlen"],
            "tokens_per_s": T / (ms["prefill_varlen"] * 1e-3),
            "algorithmic_bytes": nbytes, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "mfma_useful_frac": prefill_useful_flops(T, H) / (ms["prefill_varlen"] * 1e-3) / 1e12
                                / BF16_PEAK_TFLOPS}


def d2d_copy(torch, dev, nbytes=2 << 30, reps=5):
    """A plain 2 GiB device-to-device copy (torch copy_), the achievable-bandwidth
    reference beside the datasheet peak: GB/s of bytes read plus written."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del src, dst
    best = min(times)
    gbs = 2 * nbytes / (best * 1e-3) / 1e9
    return {"bytes_copied": nbytes, "best_ms": best, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


def graph_latency(la, W, np, torch, dev, upload, warmup, reps, layers=32, batch=1):
    """Per-call time of `layers` small decode calls (one pool per call), launched
    eagerly from Python and replayed as one captured HIP graph."""
    wl = W.make("graph-decode", "decode", "bf16", 64, np.ones(batch, dtype=np.int64), batch,
                seed=9, fill_all_slots=True)
    g = upload(wl)
    pools = [g["pool"].clone() for _ in range(layers)]
    outs = [torch.empty_like(g["q"]) for _ in range(layers)]

    def all_layers():
        for l in range(layers):
            la.la_decode(g["q"], g["k"], g["v"], pools[l], g["slot"], g["slopes"], outs[l])

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / (reps * layers)

    eager_us = timed(all_layers)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        all_layers()
    graph_us = timed(graph.replay)
    return {"batch": batch, "num_heads": 64, "calls_per_graph": layers,
            "eager_us_per_call": eager_us, "graph_us_per_call": graph_us,
            "speedup": eager_us / graph_us}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, np, wp, wd, wv):
    """The fp64 oracle on the host cores, timed on bounded samples of the
    workloads: the long prefill over `cpu_heads` heads (four per core, at most
    all 64) in groups of one head per core, every token; the whole decode and
    verify batches.  Inputs are upcast to fp64 and gathered before each timed
    call, so only the oracle's recurrence is timed."""
    import oracle

    cores = oracle.default_threads()
    H = wp.num_heads
    nh = args.cpu_heads or min(H, 4 * cores)
    slopes = oracle.alibi_slopes(H, wp.layer_id, wp.num_layers)
    init = oracle.gather(wp.pool, wp.slot_idx)
    prefill_s = 0.0
    for g0 in range(0, nh, cores):
        heads = list(range(g0, min(nh, g0 + cores)))
        q, k, v = (oracle.to_f64(np.ascontiguousarray(x[:, heads])) for x in (wp.q, wp.k, wp.v))
        s0 = np.ascontiguousarray(init[:, heads])
        log(f"cpu baseline: prefill heads {heads[0]}..{heads[-1]} x {wp.total_tokens} tokens")
        c0 = time.perf_counter()
        oracle.run(q, k, v, wp.cu_seqlens, s0, slopes[heads], threads=cores)
        prefill_s += time.perf_counter() - c0
        del q, k, v, s0

    def batch_rate(wl):
        sl = oracle.alibi_slopes(wl.num_heads, wl.layer_id, wl.num_layers)
        q, k, v = (oracle.to_f64(x) for x in (wl.q, wl.k, wl.v))
        s0 = oracle.gather(wl.pool, wl.slot_idx)
        c0 = time.perf_counter()
        oracle.run(q, k, v, wl.cu_seqlens, s0, sl, threads=cores)
        dt = time.perf_counter() - c0
        return {"value": wl.batch / dt, "unit": "req/s", "seconds": dt,
                "sample": f"the whole batch: {wl.batch} requests x {wl.total_tokens // wl.batch} token(s), "
                          f"H={wl.num_heads}, d={D}"}

    log("cpu baseline: decode and verify batches")
    return {
        "value": wp.total_tokens * (nh / H) / prefill_s, "unit": "tokens/s", "cores": min(cores, nh),
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": f"long-prefill workload, heads 0..{nh - 1} of {H} in groups of {cores}, all "
                  f"{wp.total_tokens} tokens ({prefill_s:.1f} s of oracle time); scaled by {nh}/{H} to "
                  f"whole-workload tokens/s",
        "decode": batch_rate(wd),
        "verify": batch_rate(wv),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle CPU baseline (for quick local runs)")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads in the CPU-baseline sample (default: four per host core, <= 64)")
    ap.add_argument("--only", choices=["prefill", "decode", "verify", "tree"], default=None,
                    help="run one entry point only (profiling aid; the JSON line then "
                         "reports that call alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy 5 times and exit (reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import linear_attention_amd as la
    from linear_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5}), flush=True)
        return 0
    la.load()

    def io(x):
        return torch.from_numpy(x).view(torch.int16).view(torch.bfloat16).to(dev)

    t_gen = time.time()
    want = {args.only} if args.only else {"prefill", "decode", "verify", "tree"}
    wp = W.config(4) if "prefill" in want else None
    wd = W.config(3) if "decode" in want else None
    wv = W.config(5) if want & {"verify", "tree"} else None
    log(f"inputs generated in {time.time() - t_gen:.1f} s")

    def upload(wl):
        return dict(q=io(wl.q), k=io(wl.k), v=io(wl.v), pool=torch.from_numpy(wl.pool).to(dev),
                    cu=torch.from_numpy(wl.cu_seqlens.astype(np.int32)).to(dev),
                    slot=torch.from_numpy(wl.slot_idx.astype(np.int32)).to(dev),
                    slopes=torch.from_numpy(la.la_alibi_slopes(wl.num_heads, wl.layer_id,
                                                               wl.num_layers)).to(dev))

    P = upload(wp) if wp else None
    Dd = upload(wd) if wd else None
    V = upload(wv) if wv else None
    for X in (P, Dd, V):
        if X is not None:
            X["out"] = torch.empty_like(X["q"])
    if V is not None:
        V["state_out"] = torch.empty((wv.batch, wv.num_heads, D, D), device=dev)
    if "tree" in want:
        # a seeded random draft tree per request: parent of draft j in [-1, j)
        rng = np.random.default_rng(2024)
        par = np.full((wv.batch, wv.num_draft), -1, dtype=np.int32)
        for b in range(wv.batch):
            for j in range(1, wv.num_draft):
                par[b, j] = rng.integers(-1, j)
        V["parents"] = torch.from_numpy(par).to(dev)
        V["tree_out"] = torch.empty_like(V["q"])
        V["draft_states"] = torch.empty((wv.batch, wv.num_draft, wv.num_heads, D, D), device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    # the long request's 256 (head, column block) units fill the GPU: no split,
    # no workspace (la_prefill_workspace_bytes gives 0 for it)
    def run_prefill():
        la.la_prefill(P["q"], P["k"], P["v"], P["cu"], P["pool"], P["slot"], P["slopes"],
                      P["out"], wp.max_seqlen, workspace=None, stream=stream)

    def run_decode():
        la.la_decode(Dd["q"], Dd["k"], Dd["v"], Dd["pool"], Dd["slot"], Dd["slopes"], Dd["out"],
                     stream=stream)

    def run_verify():
        la.la_verify(V["q"], V["k"], V["v"], wv.num_draft, V["pool"], V["slot"], V["slopes"],
                     V["out"], V["state_out"], stream=stream)

    def run_tree():
        la.la_verify_tree(V["q"], V["k"], V["v"], wv.num_draft, V["pool"], V["slot"], V["parents"],
                          V["slopes"], V["tree_out"], V["draft_states"], stream=stream)

    calls = [(n, f) for n, f in (("prefill", run_prefill), ("decode", run_decode),
                                 ("verify", run_verify)) if n in want]
    extra = [("tree", run_tree)] if "tree" in want else []
    if "prefill" in want and not args.only:
        # variants of the long prefill, made from its device tensors
        T4 = wp.total_tokens
        V4 = {"track_lens": torch.tensor([T4 // 2], dtype=torch.int32, device=dev),
              "track_slot": torch.tensor([1], dtype=torch.int32, device=dev),
              "k8": P["k"][:, :8].contiguous(), "v8": P["v"][:, :8].contiguous(),
              "out_g": torch.empty_like(P["q"]),
              "pool_g": torch.zeros((2, 64, D, D), device=dev)}
        T64 = 16384
        V4.update({"q64": P["q"][:T64, :, :64].contiguous(), "k64": P["k"][:T64, :, :64].contiguous(),
                   "v64": P["v"][:T64, :, :64].contiguous(),
                   "cu64": torch.tensor([0, T64], dtype=torch.int32, device=dev),
                   "pool64": torch.zeros((2, 64, 64, 64), device=dev)})
        V4["out64"] = torch.empty_like(V4["q64"])

        def run_track():
            la.la_prefill(P["q"], P["k"], P["v"], P["cu"], P["pool"], P["slot"], P["slopes"], P["out"],
                          wp.max_seqlen, track_lens=V4["track_lens"], track_slot_idx=V4["track_slot"],
                          workspace=None, stream=stream)

        def run_gqa():
            la.la_prefill(P["q"], V4["k8"], V4["v8"], P["cu"], V4["pool_g"], P["slot"], P["slopes"],
                          V4["out_g"], wp.max_seqlen, workspace=None, stream=stream)

        def workspace(B, T, L, H, d):
            n = la.la_prefill_workspace_bytes(B, T, L, H, d)
            return torch.empty(n, dtype=torch.uint8, device=dev) if n else None

        V4["ws64"] = workspace(1, T64, T64, 64, 64)

        def run_d64(ws="prealloc"):
            la.la_prefill(V4["q64"], V4["k64"], V4["v64"], V4["cu64"], V4["pool64"], P["slot"], P["slopes"],
                          V4["out64"], T64, workspace=V4["ws64"] if ws == "prealloc" else ws, stream=stream)

        # the packed varlen workload: H=16, 8 requests of U[1, 4096] tokens, half with prefix states
        w2 = W.config(2)
        P2 = upload(w2)
        P2["out"] = torch.empty_like(P2["q"])

        P2["ws"] = workspace(w2.batch, w2.total_tokens, w2.max_seqlen, w2.num_heads, D)

        def run_varlen():
            la.la_prefill(P2["q"], P2["k"], P2["v"], P2["cu"], P2["pool"], P2["slot"], P2["slopes"],
                          P2["out"], w2.max_seqlen, workspace=P2["ws"], stream=stream)

        # the tensor-parallel share of the long request: heads 0..7 (8 of 64), which
        # fills 32 CUs unless the request is split into sequence segments
        V4.update({"q8h": P["q"][:, :8].contiguous(), "k8h": P["k"][:, :8].contiguous(),
                   "v8h": P["v"][:, :8].contiguous(), "pool8h": torch.zeros((2, 8, D, D), device=dev),
                   "slopes8h": P["slopes"][:8].contiguous()})
        V4["out8h"] = torch.empty_like(V4["q8h"])
        V4["ws8h"] = workspace(1, T4, wp.max_seqlen, 8, D)

        def run_tp8(ws="prealloc"):
            la.la_prefill(V4["q8h"], V4["k8h"], V4["v8h"], P["cu"], V4["pool8h"], P["slot"], V4["slopes8h"],
                          V4["out8h"], wp.max_seqlen, workspace=V4["ws8h"] if ws == "prealloc" else ws,
                          stream=stream)

        def unsegmented(fn):
            # no workspace: the call runs unsplit
            return lambda: fn(ws=None)

        # fp32 inputs (the same values, upcast exactly): the token-recurrent kernel
        V4.update({"q32": P["q"][:T64].float(), "k32": P["k"][:T64].float(), "v32": P["v"][:T64].float(),
                   "pool32": torch.zeros((2, 64, D, D), device=dev)})
        V4["out32"] = torch.empty_like(V4["q32"])

        def run_fp32():
            la.la_prefill(V4["q32"], V4["k32"], V4["v32"], V4["cu64"], V4["pool32"], P["slot"], P["slopes"],
                          V4["out32"], T64, workspace=None, stream=stream)

        extra += [("prefill_track", run_track), ("prefill_gqa", run_gqa), ("prefill_d64", run_d64),
                  ("prefill_varlen", run_varlen), ("prefill_tp8", run_tp8),
                  ("prefill_tp8_unseg", unsegmented(run_tp8)), ("prefill_d64_unseg", unsegmented(run_d64)),
                  ("prefill_fp32", run_fp32)]
        V4["varlen"] = w2
    for _ in range(args.warmup):
        for _, fn in calls + extra:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(K)] for name, _ in calls}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        for name, fn in calls:
            a, b = ev[name][s]
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1000.0 / K
    # entry points outside the step: timed the same way, after it
    for name, fn in extra:
        ev[name] = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(K)]
        for s in range(K):
            a, b = ev[name][s]
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    ms = {name: float(np.mean([a.elapsed_time(b) for a, b in ev[name]])) for name in ev}
    ms_min = {name: float(np.min([a.elapsed_time(b) for a, b in ev[name]])) for name in ev}

    if args.only:
        name = args.only
        print(json.dumps({"only": name, "avg_ms": ms[name], "min_ms": ms_min[name],
                          "ms_per_step": ms_per_step, "steps": K}), flush=True)
        return 0

    H = 64
    Tp = wp.total_tokens
    pb = prefill_bytes(Tp, H, wp.batch)
    p_gbs = pb / (ms["prefill"] * 1e-3) / 1e9
    p_tflops = prefill_useful_flops(Tp, H) / (ms["prefill"] * 1e-3) / 1e12
    db = step_bytes(wd.batch, H, wd.total_tokens)
    vb = step_bytes(wv.batch, H, wv.total_tokens)
    d_gbs = db / (ms["decode"] * 1e-3) / 1e9
    v_gbs = vb / (ms["verify"] * 1e-3) / 1e9
    tb = tree_bytes(wv.batch, wv.num_draft, H)
    t_gbs = tb / (ms["tree"] * 1e-3) / 1e9
    graph = graph_latency(la, W, np, torch, dev, upload, args.warmup, K)
    copy = d2d_copy(torch, dev)

    result = {
        "metric": METRIC,
        "value": Tp / (ms["prefill"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "published_throughput": "none: the pages give correctness tolerances for this kernel but no "
                                "throughput figure on any hardware",
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v, 0.05*N(0,1) fp32 prefix states)",
        "config": {
            "workload": "long prefill T=131072 H=64 d=128 bf16 (value) + decode B=256 H=64 "
                        "pool 512 + chain verify B=128 k=5 H=64 pool 256, one call each per step",
            "prefill": {"batch": wp.batch, "seq_len": Tp, "num_heads": H, "head_dim": D},
            "decode": {"batch": wd.batch, "num_heads": H, "pool_slots": wd.pool_slots},
            "verify": {"batch": wv.batch, "num_draft": wv.num_draft, "num_heads": H,
                       "pool_slots": wv.pool_slots},
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "achieved": p_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": p_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic("prefill_chunked_kernel", "long-prefill"),
            "kernel": "prefill_chunked_kernel", "algorithmic_bytes": pb,
            "avg_ms": ms["prefill"],
            "mfma_useful_tflops": p_tflops, "mfma_useful_frac": p_tflops / BF16_PEAK_TFLOPS,
        },
        "decode": {
            "value": wd.batch / (ms["decode"] * 1e-3), "unit": "req/s", "avg_ms": ms["decode"],
            "min_ms": ms_min["decode"],
            "roofline": {"bound": "hbm", "achieved": d_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("recurrent_kernel<bf16>", "decode"),
                         "kernel": "recurrent_kernel<bf16>", "algorithmic_bytes": db},
        },
        "verify": {
            "value": wv.batch / (ms["verify"] * 1e-3), "unit": "req/s",
            "tokens_per_s": wv.total_tokens / (ms["verify"] * 1e-3), "avg_ms": ms["verify"],
            "min_ms": ms_min["verify"],
            "roofline": {"bound": "hbm", "achieved": v_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": v_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("recurrent_kernel<bf16>", "verify"),
                         "kernel": "recurrent_kernel<bf16>", "algorithmic_bytes": vb},
        },
        "tree_verify": {
            "value": wv.batch / (ms["tree"] * 1e-3), "unit": "req/s",
            "tokens_per_s": wv.total_tokens / (ms["tree"] * 1e-3), "avg_ms": ms["tree"],
            "min_ms": ms_min["tree"],
            "config": {"batch": wv.batch, "num_draft": wv.num_draft, "num_heads": H,
                       "tree": "seeded random parents in [-1, j)", "draft_states": True},
            "roofline": {"bound": "hbm", "achieved": t_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": t_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("tree_kernel<bf16>", "tree-verify"),
                         "kernel": "tree_kernel<bf16>", "algorithmic_bytes": tb},
        },
        "decode_graph": graph,
        "d2d_copy": copy,
        "prefill_variants": prefill_variants(ms, ms_min, wp.total_tokens, H),
        "varlen_prefill": varlen_prefill(ms, ms_min, V4["varlen"]) if "prefill_varlen" in ms else None,
        "prefill_min_ms": ms_min["prefill"],
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, np, wp, wd, wv)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
