"""GPU parity of the full-width bf16 prefill kernel (head_dim 128).

With LA_PREFILL_WIDE=1 a bf16, d = 128 prefill without snapshots runs one
workgroup per (request, head, segment) that keeps the whole 128 x 128 state,
instead of one per 32-column block.  These cases cover it unsplit and split
into sequence segments, with ragged and empty requests, grouped heads,
decay rates on both sides of the scaled-state threshold and out-of-range
slots, each checked against the fp64 oracle on every output and final state,
and against the column-block kernel on the same inputs.
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


@pytest.fixture(autouse=True)
def wide(monkeypatch):
    monkeypatch.setenv("LA_PREFILL_WIDE", "1")

    def set_wide(on):
        monkeypatch.setenv("LA_PREFILL_WIDE", "1" if on else "0")
    return set_wide


def _check(wl, heads=None):
    log(f"case {wl.name} B={wl.batch} T={wl.total_tokens} H={wl.num_heads} HK={wl.num_kv_heads} "
        f"lens={wl.lengths.tolist()}")
    out, pool, _ = run_gpu(wl)
    check_against_oracle(wl, out, pool, heads=heads)
    check_untouched(wl, pool)
    return out, pool


def test_ragged_requests_unsplit():
    """Requests of 1, 63, 64, 65 and a few thousand tokens (full and partial
    last chunks), half from prefix states; too short to be split."""
    lens = [1, 63, 64, 65, 3000, 777]
    wl = W.make("wide-ragged", "prefill", "bf16", 16, lens, 8, seed=1301,
                prefix=[True, False, True, False, True, True])
    _check(wl)


def test_empty_requests_unsplit():
    lens = [0, 130, 0, 2]
    wl = W.make("wide-empty", "prefill", "bf16", 4, lens, 6, seed=1302, prefix=[True] * 4)
    _check(wl)


def test_one_long_request_in_segments():
    """A tensor-parallel share of a long request: 8 heads split into 8
    segments, from a nonzero prefix state."""
    wl = W.make("wide-seg-tp8", "prefill", "bf16", 8, [40000], 3, seed=1303, prefix=[True], slot_idx=[2])
    _check(wl)


def test_mixed_lengths_in_segments():
    lens = [20000, 100, 1, 0, 9000]
    wl = W.make("wide-seg-mixed", "prefill", "bf16", 4, lens, 8, seed=1304,
                prefix=[True, False, True, True, False])
    _check(wl)


def test_grouped_heads():
    wl = W.make("wide-gqa", "prefill", "bf16", 8, [17000], 2, seed=1305, prefix=[True], slot_idx=[0],
                num_kv_heads=2)
    _check(wl)
    wl = W.make("wide-gqa-short", "prefill", "bf16", 8, [300, 65, 4000], 4, seed=1306,
                prefix=[True, False, True], num_kv_heads=4)
    _check(wl)


SLOPES = [0.0, 1e-3, 0.25, 2.0, 2.0001, 3.0, 8.0, 0.9]


@pytest.mark.parametrize("lens", [[1, 64, 65, 200, 130], [9000, 70]])
def test_slopes_on_both_sides_of_two(lens):
    """Slopes in [0, 2] take the scaled-state frame, larger ones explicit
    per-token weights; the second case is split into segments."""
    H = len(SLOPES)
    wl = W.make(f"wide-slopes-{len(lens)}", "prefill", "bf16", H, lens, len(lens) + 2, seed=1307 + len(lens),
                prefix=[True] * len(lens))
    log(f"case {wl.name} lens={lens} slopes={SLOPES}")
    dv = device_inputs(wl)
    slopes = np.array(SLOPES, dtype=np.float32)
    out = torch.empty_like(dv["q"])
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], torch.from_numpy(slopes).cuda(),
                  out, wl.max_seqlen)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.prefill(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.pool, wl.slot_idx, slopes)
    assert_close(host_io(out), ref_out, TOL["bf16"], f"{wl.name} out")
    fin = dv["pool"].index_select(0, torch.from_numpy(wl.slot_idx.astype(np.int64)).cuda()).cpu().numpy()
    assert_close(fin, ref_fin, TOL["bf16"], f"{wl.name} final state")
    check_untouched(wl, dv["pool"])


@pytest.mark.parametrize("lens,seed", [([70, 130, 5, 64], 1311), ([12000, 9000, 300, 64], 1312)])
def test_out_of_range_slot(lens, seed):
    """A request with slot -1 and one with slot == pool_slots get zero output
    and touch no state; the others are computed normally (the second case is
    split into segments)."""
    wl = W.make(f"wide-badslot-{lens[0]}", "prefill", "bf16", 4, lens, 6, seed=seed, prefix=[True] * 4)
    log(f"case {wl.name} lens={lens}")
    dv = device_inputs(wl)
    bad = wl.slot_idx.astype(np.int32).copy()
    bad[1], bad[3] = -1, wl.pool_slots
    out = torch.full_like(dv["q"], 7.0)
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], torch.from_numpy(bad).cuda(), dv["slopes"],
                  out, wl.max_seqlen)
    torch.cuda.synchronize()
    cu = wl.cu_seqlens
    got = host_io(out)
    for b in (1, 3):
        assert not to_f64(got[cu[b]:cu[b + 1]]).any(), f"request {b} output not zero"
    good = [0, 2]
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in good])
    sub_cu = np.concatenate([[0], np.cumsum([lens[b] for b in good])])
    slopes = oracle.alibi_slopes(4, wl.layer_id, wl.num_layers)
    ref_out, ref_fin = oracle.prefill(wl.q[rows], wl.k[rows], wl.v[rows], sub_cu, wl.pool, wl.slot_idx[good],
                                      slopes)
    assert_close(got[rows], ref_out, TOL["bf16"], f"{wl.name} out")
    fin = dv["pool"].index_select(0, torch.from_numpy(wl.slot_idx[good].astype(np.int64)).cuda()).cpu().numpy()
    assert_close(fin, ref_fin, TOL["bf16"], f"{wl.name} final state")
    untouched = [s for s in range(wl.pool_slots) if s not in wl.slot_idx[good]]
    after = dv["pool"].index_select(0, torch.tensor(untouched, device="cuda")).cpu().numpy()
    assert np.array_equal(after.view(np.uint32), wl.pool[untouched].view(np.uint32)), "state touched"


def test_wide_equals_column_blocks(wide):
    """The same inputs through both kernels agree to the bf16 bound."""
    wl = W.make("wide-vs-blocks", "prefill", "bf16", 8, [20000, 515, 64], 4, seed=1320,
                prefix=[True, False, True])
    wide(False)
    out0, pool0 = _check(wl, heads=[0, 5])
    wide(True)
    out1, pool1 = _check(wl, heads=[0, 5])
    assert_close(host_io(out1), to_f64(host_io(out0)), TOL["bf16"], "wide vs column blocks out")
    idx = torch.from_numpy(wl.slot_idx.astype(np.int64)).cuda()
    assert_close(pool1.index_select(0, idx).cpu().numpy(), pool0.index_select(0, idx).cpu().numpy(),
                 TOL["bf16"], "wide vs column blocks state")
