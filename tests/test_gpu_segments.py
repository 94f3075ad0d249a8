"""GPU parity of the sequence-segmented prefill.

A bf16 prefill whose (request, head, column block) units fill only part of
the GPU splits each request into segments of whole chunks: one pass stores
every segment's state contribution, a second chains them into each segment's
initial state, and the chunked kernel then runs all segments side by side.
These cases are sized so that the launch takes that path (few heads, long
requests) and are checked against the fp64 oracle on every output and final
state.  LA_PREFILL_MAX_SEGMENTS=1 turns the split off, for comparison.
"""

import numpy as np
import pytest
import torch

import linear_attention_amd as la
import oracle
from linear_attention_amd import workloads as W

from gpu_util import (TOL, assert_close, check_against_oracle, check_untouched, device_inputs, host_io, log,
                      run_gpu, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


@pytest.fixture
def max_segments(monkeypatch):
    def set_cap(n):
        monkeypatch.setenv("LA_PREFILL_MAX_SEGMENTS", str(n))
    return set_cap


def _check(wl):
    log(f"case {wl.name} B={wl.batch} T={wl.total_tokens} H={wl.num_heads} d={wl.head_dim} "
        f"lens={wl.lengths.tolist()}")
    out, pool, _ = run_gpu(wl)
    check_against_oracle(wl, out, pool)
    check_untouched(wl, pool)
    return out, pool


def test_one_long_request_eight_heads():
    """A tensor-parallel share of a long request: 8 heads, 8 segments of 79
    chunks each (the last shorter), from a nonzero prefix state."""
    wl = W.make("seg-tp8", "prefill", "bf16", 8, [40000], 3, seed=1201, prefix=[True], slot_idx=[2])
    _check(wl)


def test_mixed_lengths_short_and_empty_requests():
    """Requests of very different lengths in one segmented launch: the short
    ones have fewer non-empty segments than the launch (one of them a single
    chunk), and one request is empty."""
    lens = [20000, 100, 1, 0, 9000]
    wl = W.make("seg-mixed", "prefill", "bf16", 4, lens, 8, seed=1202, prefix=[True, False, True, True, False])
    _check(wl)


def test_head_dim_64_and_grouped_heads():
    wl = W.make("seg-d64", "prefill", "bf16", 4, [20000, 7000], 4, head_dim=64, seed=1203, prefix=[True, True])
    _check(wl)
    wl = W.make("seg-gqa", "prefill", "bf16", 8, [17000], 2, seed=1204, prefix=[True], slot_idx=[0],
                num_kv_heads=2)
    _check(wl)


def test_segmented_equals_unsegmented(max_segments):
    """The same inputs with the split on and off agree to the bf16 bound,
    and the oracle holds for both."""
    wl = W.make("seg-onoff", "prefill", "bf16", 4, [33000, 4100], 4, seed=1205, prefix=[True, False])
    max_segments(1)
    out1, pool1 = _check(wl)
    max_segments(8)
    out8, pool8 = _check(wl)
    assert_close(host_io(out8), to_f64(host_io(out1)), TOL["bf16"], "segmented vs unsegmented out")
    idx = torch.from_numpy(wl.slot_idx.astype(np.int64)).cuda()
    assert_close(pool8.index_select(0, idx).cpu().numpy(), pool1.index_select(0, idx).cpu().numpy(),
                 TOL["bf16"], "segmented vs unsegmented state")


def test_out_of_range_slot_in_a_segmented_launch():
    """Every segment of a request with an out-of-range slot writes zeros and
    no state; the other request is computed normally."""
    lens = [12000, 9000]
    wl = W.make("seg-badslot", "prefill", "bf16", 4, lens, 4, seed=1206, prefix=[True, True])
    log(f"case {wl.name} lens={lens}")
    dv = device_inputs(wl)
    bad = wl.slot_idx.astype(np.int32).copy()
    bad[1] = wl.pool_slots + 3
    out = torch.full_like(dv["q"], 7.0)
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], torch.from_numpy(bad).cuda(), dv["slopes"],
                  out, wl.max_seqlen)
    torch.cuda.synchronize()
    cu = wl.cu_seqlens
    got = host_io(out)
    assert not to_f64(got[cu[1]:cu[2]]).any(), "request 1 output not zero"
    slopes = oracle.alibi_slopes(4, wl.layer_id, wl.num_layers)
    ref_out, ref_fin = oracle.prefill(wl.q[:cu[1]], wl.k[:cu[1]], wl.v[:cu[1]], np.array([0, lens[0]]), wl.pool,
                                      wl.slot_idx[:1], slopes)
    assert_close(got[:cu[1]], ref_out, TOL["bf16"], f"{wl.name} out")
    fin = dv["pool"].index_select(0, torch.from_numpy(wl.slot_idx[:1].astype(np.int64)).cuda()).cpu().numpy()
    assert_close(fin, ref_fin, TOL["bf16"], f"{wl.name} final state")
    untouched = [s for s in range(wl.pool_slots) if s != wl.slot_idx[0]]
    after = dv["pool"].index_select(0, torch.tensor(untouched, device="cuda")).cpu().numpy()
    assert np.array_equal(after.view(np.uint32), wl.pool[untouched].view(np.uint32)), "state touched"


def test_snapshot_request_on_a_splittable_shape():
    """A long request with few heads would be split, but a snapshot forces the
    unsplit two-pass path: the track slot gets the state after track_len
    tokens and the active slot the final state."""
    wl = W.make("seg-track", "prefill", "bf16", 4, [12345], 3, seed=1207, prefix=[True], slot_idx=[1])
    tl = 6000
    log(f"case {wl.name} T={wl.total_tokens} track_len={tl}")
    dv = device_inputs(wl)
    out = torch.empty_like(dv["q"])
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out, wl.max_seqlen,
                  track_lens=torch.tensor([tl], dtype=torch.int32, device="cuda"),
                  track_slot_idx=torch.tensor([0], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    slopes = oracle.alibi_slopes(4, wl.layer_id, wl.num_layers)
    ref_out, ref_fin, ref_snap = oracle.prefill(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.pool, wl.slot_idx, slopes,
                                                track_lens=[tl])
    assert_close(host_io(out), ref_out, TOL["bf16"], f"{wl.name} out")
    pool = dv["pool"].cpu().numpy()
    assert_close(pool[1], ref_fin[0], TOL["bf16"], f"{wl.name} final state")
    assert_close(pool[0], ref_snap[0], TOL["bf16"], f"{wl.name} snapshot")
    assert np.array_equal(pool[2].view(np.uint32), wl.pool[2].view(np.uint32)), "untouched slot changed"


def test_caller_workspace_exact_size_none_and_too_small():
    """The split runs in the caller's workspace: a buffer of exactly the queried
    size (filled with garbage first, so nothing may rely on its contents), a
    larger one, and no workspace at all (the call then runs unsplit) all match
    the oracle; a buffer one float short is rejected before anything runs,
    leaving the pool and the output untouched."""
    wl = W.make("seg-ws", "prefill", "bf16", 8, [20000], 3, seed=1208, prefix=[True], slot_idx=[2])
    need = la.la_prefill_workspace_bytes(wl.batch, wl.total_tokens, wl.max_seqlen, wl.num_heads, wl.head_dim)
    log(f"case {wl.name} T={wl.total_tokens} workspace {need} B")
    assert need > 0
    for what, ws in (("exact", torch.full((need // 4,), float("nan"), device="cuda")),
                     ("larger", torch.full((need // 4 + 1000,), 1e30, device="cuda")),
                     ("none", None)):
        dv = device_inputs(wl)
        out = torch.empty_like(dv["q"])
        la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                      wl.max_seqlen, workspace=ws)
        torch.cuda.synchronize()
        log(f"  workspace {what}")
        check_against_oracle(wl, out, dv["pool"])
        check_untouched(wl, dv["pool"])
    dv = device_inputs(wl)
    out = torch.full_like(dv["q"], 3.0)
    short = torch.empty(need // 4 - 1, device="cuda")
    with pytest.raises(la.LAError) as e:
        la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                      wl.max_seqlen, workspace=short)
    assert e.value.status == la.LA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0)
    assert np.array_equal(dv["pool"].cpu().numpy().view(np.uint32), wl.pool.view(np.uint32))
