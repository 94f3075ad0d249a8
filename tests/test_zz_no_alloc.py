"""la_prefill_noalloc (the prefill for callers that cannot allocate) against
la_prefill with a caller workspace, on two calls in a row, the second with
a smaller input: both split into sequence segments, so the second call reuses
the static scratch the first one filled.  Outputs and pools must be bit-equal
to la_prefill's (same kernels, same segment plan) and within the bf16 bound
of the fp64 oracle; an unsplit call and an empty one as well."""
import numpy as np
import pytest
import torch

import linear_attention_amd as la
from linear_attention_amd import workloads as W

from gpu_util import check_against_oracle, check_untouched, device_inputs, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def _both(wl):
    """(out, pool) of la_prefill with its own workspace and of la_prefill_noalloc."""
    res = []
    for fn in (la.la_prefill, la.la_prefill_noalloc):
        d = device_inputs(wl)
        out = torch.full_like(d["q"], 5.0)
        fn(d["q"], d["k"], d["v"], d["cu"], d["pool"], d["slot"], d["slopes"], out, wl.max_seqlen)
        torch.cuda.synchronize()
        res.append((out, d["pool"]))
    return res


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), what


@pytest.mark.parametrize("order", ["large-then-small"])
def test_noalloc_matches_workspace_prefill_twice(order):
    big = W.make("noalloc-big", "prefill", "bf16", 8, [20000, 700], 5, seed=2301, prefix=[True, False])
    small = W.make("noalloc-small", "prefill", "bf16", 4, [9000, 3000, 0], 6, seed=2302,
                   prefix=[False, True, True])
    for wl in (big, small):
        need = la.la_prefill_workspace_bytes(wl.batch, wl.total_tokens, wl.max_seqlen, wl.num_heads, 128)
        log(f"case {wl.name} lens={wl.lengths.tolist()} H={wl.num_heads} split workspace {need} B")
        assert 0 < need <= (32 << 20)
        (o1, p1), (o2, p2) = _both(wl)
        _same(o2, o1, f"{wl.name} out")
        _same(p2, p1, f"{wl.name} pool")
        check_against_oracle(wl, o2, p2)
        check_untouched(wl, p2)


def test_noalloc_unsplit_and_empty():
    wl = W.make("noalloc-short", "prefill", "bf16", 16, [70, 1, 200], 4, seed=2303, prefix=[True, False, True])
    assert la.la_prefill_workspace_bytes(wl.batch, wl.total_tokens, wl.max_seqlen, wl.num_heads, 128) == 0
    (o1, p1), (o2, p2) = _both(wl)
    _same(o2, o1, "short out")
    _same(p2, p1, "short pool")
    check_against_oracle(wl, o2, p2)
    wl0 = W.make("noalloc-empty", "prefill", "bf16", 2, [0, 0], 3, seed=2304)
    d = device_inputs(wl0)
    la.la_prefill_noalloc(d["q"], d["k"], d["v"], d["cu"], d["pool"], d["slot"], d["slopes"],
                          torch.empty_like(d["q"]), 0)
    torch.cuda.synchronize()
    assert np.array_equal(d["pool"].cpu().numpy().view(np.uint32), wl0.pool.view(np.uint32))


def test_noalloc_and_workspace_prefill_in_a_hip_graph():
    """Both split prefills captured in one HIP graph (the allocation-free one
    needs no allocation at capture or replay; the other gets its workspace
    before capture) and replayed three times with eager pool resets and output
    scribbles between replays; every replay matches the oracle and the eager
    results bit for bit."""
    wl = W.make("noalloc-graph", "prefill", "bf16", 8, [17000, 300], 4, seed=2305, prefix=[True, True])
    d1, d2 = device_inputs(wl), device_inputs(wl)
    pool0 = d1["pool"].clone()
    need = la.la_prefill_workspace_bytes(wl.batch, wl.total_tokens, wl.max_seqlen, wl.num_heads, 128)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1, o2 = torch.empty_like(d1["q"]), torch.empty_like(d2["q"])

    def step():
        la.la_prefill_noalloc(d1["q"], d1["k"], d1["v"], d1["cu"], d1["pool"], d1["slot"], d1["slopes"], o1,
                              wl.max_seqlen)
        la.la_prefill(d2["q"], d2["k"], d2["v"], d2["cu"], d2["pool"], d2["slot"], d2["slopes"], o2,
                      wl.max_seqlen, workspace=ws)

    step()
    torch.cuda.synchronize()
    check_against_oracle(wl, o1, d1["pool"])
    ref = [t.clone() for t in (o1, d1["pool"], o2, d2["pool"])]
    _same(ref[0], ref[2], "eager out")
    for p in (d1["pool"], d2["pool"]):
        p.copy_(pool0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for p in (d1["pool"], d2["pool"]):
            p.copy_(pool0)
        o1.fill_(-1.0)
        o2.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("noalloc out", "noalloc pool", "workspace out", "workspace pool"),
                              (o1, d1["pool"], o2, d2["pool"]), ref):
            _same(a, b, f"replay {rep}: {name}")
        check_against_oracle(wl, o1, d1["pool"])
        log(f"graph replay {rep} ok")
