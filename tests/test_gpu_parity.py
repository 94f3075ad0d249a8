"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every case uses the seeded synthetic workloads; tolerances are 3e-2 for bf16
inputs and 1e-4 for fp32 inputs (|got - ref| <= tol + tol*|ref|), on outputs
and final states; pool slots no request names must be bit-identical.
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_amd as la
from linear_attention_amd import workloads as W

from gpu_util import (TOL, assert_close, check_against_oracle, check_untouched, device_inputs,
                      host_io, log, oracle_ref, run_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def _full_check(wl, state_out=False):
    log(f"case {wl.name} seed={wl.seed} B={wl.batch} T={wl.total_tokens} H={wl.num_heads}")
    out, pool, so = run_gpu(wl, state_out=state_out)
    check_against_oracle(wl, out, pool, so)
    check_untouched(wl, pool, addressed=(so is None))
    return out, pool, so


def test_config1_tiny_fp32():
    _full_check(W.config(1))


def test_config2_varlen_bf16():
    _full_check(W.config(2))


def test_config3_decode():
    _full_check(W.config(3))


def test_config5_chain_verify_state_out():
    _full_check(W.config(5), state_out=True)


def test_config4_long_prefill_all_heads():
    """The full 131072-token request at H=64: every output and the final state
    of every head against the oracle, eight heads at a time (so that only one
    group is upcast to fp64 on the host at once)."""
    wl = W.config(4)
    log(f"case {wl.name} T={wl.total_tokens} H={wl.num_heads}")
    out, pool, _ = run_gpu(wl)
    for g in range(0, wl.num_heads, 8):
        heads = list(range(g, g + 8))
        log(f"  heads {heads[0]}..{heads[-1]}")
        check_against_oracle(wl, out, pool, heads=heads)
    check_untouched(wl, pool)


EDGE_LENGTHS = [1, 63, 64, 65, 0, 131, 2, 200, 127, 128, 129]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_lengths_with_prefixes(dtype):
    n = len(EDGE_LENGTHS)
    prefix = [i % 2 == 0 for i in range(n)]
    wl = W.make(f"edge-{dtype}", "prefill", dtype, 4, EDGE_LENGTHS, 16, seed=31, prefix=prefix,
                layer_id=2, num_layers=5)
    _full_check(wl)


@pytest.mark.parametrize("H", [1, 3, 8, 9, 24])
def test_head_counts(H):
    """Head counts that do not fill the XCD groups of 8 (request, head) pairs."""
    wl = W.make(f"heads-{H}", "prefill", "bf16", H, [70, 5, 190], 5, seed=40 + H,
                prefix=[True, False, True])
    _full_check(wl)


def test_decode_small_and_fp32():
    for dtype in ("bf16", "fp32"):
        wl = W.make(f"decode-{dtype}", "decode", dtype, 6, np.ones(7, dtype=np.int64), 11, seed=50,
                    prefix=[True] * 7)
        _full_check(wl)


@pytest.mark.parametrize("num_draft", [1, 2, 5, 8])
def test_verify_in_place_and_lengths(num_draft):
    wl = W.make(f"verify-k{num_draft}", "verify", "bf16", 4,
                np.full(6, num_draft, dtype=np.int64), 9, seed=60 + num_draft,
                prefix=[True] * 6, num_draft=num_draft)
    _full_check(wl, state_out=False)
    _full_check(wl, state_out=True)


def test_split_invariance_prefill_then_decode():
    """prefill(n) == prefill(m) followed by n-m decode steps, on the GPU."""
    n, m, H = 150, 97, 8
    wl = W.make("split", "prefill", "bf16", H, [n], 3, seed=70, prefix=[True], slot_idx=[1])
    d = device_inputs(wl)
    full_out = torch.empty_like(d["q"])
    pool_full = d["pool"].clone()
    la.la_prefill(d["q"], d["k"], d["v"], d["cu"], pool_full, d["slot"], d["slopes"], full_out, n)
    pool = d["pool"].clone()
    part_out = torch.empty_like(d["q"])
    cu_m = torch.tensor([0, m], dtype=torch.int32, device="cuda")
    la.la_prefill(d["q"][:m].contiguous(), d["k"][:m].contiguous(), d["v"][:m].contiguous(), cu_m,
                  pool, d["slot"], d["slopes"], part_out[:m], m)
    for t in range(m, n):
        o = torch.empty_like(d["q"][t:t + 1])
        la.la_decode(d["q"][t:t + 1].contiguous(), d["k"][t:t + 1].contiguous(),
                     d["v"][t:t + 1].contiguous(), pool, d["slot"], d["slopes"], o)
        part_out[t:t + 1] = o
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle_ref(wl)
    assert_close(host_io(part_out), ref_out, TOL["bf16"], "split out")
    assert_close(pool[1].cpu().numpy(), ref_fin[0], TOL["bf16"], "split final")
    assert_close(host_io(full_out), ref_out, TOL["bf16"], "full out")


def test_verify_equals_chain_prefill():
    B, kd, H = 5, 5, 4
    wl = W.make("verify-vs-prefill", "verify", "bf16", H, np.full(B, kd, dtype=np.int64), 8,
                seed=80, prefix=[True] * B, num_draft=kd)
    d = device_inputs(wl)
    so = torch.empty((B, H, 128, 128), device="cuda")
    o1 = torch.empty_like(d["q"])
    la.la_verify(d["q"], d["k"], d["v"], kd, d["pool"], d["slot"], d["slopes"], o1, so)
    pool2 = d["pool"].clone()
    o2 = torch.empty_like(d["q"])
    la.la_prefill(d["q"], d["k"], d["v"], d["cu"], pool2, d["slot"], d["slopes"], o2, kd)
    torch.cuda.synchronize()
    idx = torch.from_numpy(wl.slot_idx.astype(np.int64)).cuda()
    assert_close(host_io(o1), host_io(o2), TOL["bf16"], "verify vs prefill out")
    assert_close(so.cpu().numpy(), pool2.index_select(0, idx).cpu().numpy(), TOL["bf16"],
                 "verify vs prefill state")


def test_request_order_invariance():
    lens = [40, 1, 90, 65]
    wl = W.make("order", "prefill", "bf16", 4, lens, 6, seed=90, prefix=[True, False, True, True])
    out, pool, _ = run_gpu(wl)
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(wl.cu_seqlens[b], wl.cu_seqlens[b + 1]) for b in order])
    wl2 = W.make("order2", "prefill", "bf16", 4, [lens[b] for b in order], 6, seed=90,
                 slot_idx=wl.slot_idx[order])
    wl2.q, wl2.k, wl2.v, wl2.pool = wl.q[idx], wl.k[idx], wl.v[idx], wl.pool
    out2, pool2, _ = run_gpu(wl2)
    np.testing.assert_array_equal(host_io(out2), host_io(out)[idx])
    np.testing.assert_array_equal(pool2.cpu().numpy(), pool.cpu().numpy())


@pytest.mark.parametrize("B,H,head_dim", [(200, 8, 128), (257, 2, 128), (48, 4, 64)])
def test_many_requests_with_tied_lengths(B, H, head_dim):
    """Batches that the prefill dispatches longest request first (B <= 256)
    and one just past that limit, in natural order.  The lengths repeat a few
    values, so most requests tie, and include empty requests; the grids are
    several times what the GPU holds at once."""
    rng = np.random.default_rng(1000 + B)
    lens = rng.choice([0, 1, 63, 64, 65, 130, 200], size=B)
    prefix = [b % 3 == 0 for b in range(B)]
    wl = W.make(f"ties-{B}-{H}-{head_dim}", "prefill", "bf16", H, lens, B + 5, head_dim=head_dim,
                seed=1100 + B, prefix=prefix)
    _full_check(wl)


def test_debug_mode_rejects_bad_metadata():
    wl = W.make("debug", "prefill", "bf16", 2, [3, 4], 4, seed=95)
    d = device_inputs(wl)
    out = torch.empty_like(d["q"])
    os.environ["LA_DEBUG"] = "1"
    try:
        la.la_prefill(d["q"], d["k"], d["v"], d["cu"], d["pool"], d["slot"], d["slopes"], out, 4)
        dup = torch.tensor([1, 1], dtype=torch.int32, device="cuda")
        with pytest.raises(la.LAError) as e:
            la.la_prefill(d["q"], d["k"], d["v"], d["cu"], d["pool"], dup, d["slopes"], out, 4)
        assert e.value.status == la.LA_ERR_INVALID_ARG
        oob = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
        with pytest.raises(la.LAError):
            la.la_prefill(d["q"], d["k"], d["v"], d["cu"], d["pool"], oob, d["slopes"], out, 4)
        bad_cu = torch.tensor([0, 5, 7], dtype=torch.int32, device="cuda")
        with pytest.raises(la.LAError):   # request longer than max_seqlen
            la.la_prefill(d["q"], d["k"], d["v"], bad_cu, d["pool"], d["slot"], d["slopes"], out, 4)
        bad_cu = torch.tensor([0, 5, 4], dtype=torch.int32, device="cuda")
        with pytest.raises(la.LAError):   # decreasing offsets
            la.la_prefill(d["q"], d["k"], d["v"], bad_cu, d["pool"], d["slot"], d["slopes"], out, 8)
        with pytest.raises(la.LAError):
            la.la_decode(d["q"][:2].contiguous(), d["k"][:2].contiguous(), d["v"][:2].contiguous(),
                         d["pool"], dup, d["slopes"], out[:2])
    finally:
        del os.environ["LA_DEBUG"]
    torch.cuda.synchronize()
