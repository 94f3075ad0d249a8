"""GPU parity for the widened path: state-tracking snapshots, grouped kv heads,
head_dim 64, tree verify with per-position states, and HIP-graph capture.

Everything is checked against the fp64 oracle on seeded inputs with the same
tolerances as the base parity tests (3e-2 bf16, 1e-4 fp32, as
|got - ref| <= tol + tol*|ref|); pool slots a call must not write are compared
bit for bit.  Citations name the page "SGLang Lightning Attention 能力矩阵与
seg_la 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_amd as la
import oracle
from linear_attention_amd import workloads as W

from gpu_util import (TOL, assert_close, check_against_oracle, check_untouched, device_inputs,
                      host_io, log, oracle_ref, run_gpu, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")


# ---------------------------------------------------------------- state tracking

TRACK_LENS = [130, 64, 200, 1, 0, 77, 129, 300, 5]
TRACK_AT = [64, 0, 137, 1, 0, 80, 65, 300, 3]    # request 5: beyond its end -> no snapshot
TRACK_NONE = 8                                     # request 8: negative track slot


def _track_case(dtype, d, H, HK, seed):
    n = len(TRACK_LENS)
    wl = W.make(f"track-{dtype}-d{d}-H{H}/{HK}", "prefill", dtype, H, TRACK_LENS, 3 * n, head_dim=d,
                seed=seed, prefix=[i % 2 == 1 for i in range(n)], num_kv_heads=HK, layer_id=1,
                num_layers=3)
    rest = [s for s in np.random.default_rng(seed).permutation(3 * n) if s not in set(wl.slot_idx)]
    ts = np.array(rest[:n], dtype=np.int32)
    ts[TRACK_NONE] = -1
    return wl, ts


@pytest.mark.parametrize("dtype,d,H,HK", [("bf16", 128, 4, 4), ("bf16", 128, 4, 2), ("fp32", 128, 2, 2),
                                          ("bf16", 64, 4, 4), ("fp32", 64, 4, 1)])
def test_prefill_track_snapshot(dtype, d, H, HK):
    """[LA-page] §额外覆盖: active slots advance to the final state, track slots
    hold the state after track_len tokens, every other slot is untouched."""
    wl, ts = _track_case(dtype, d, H, HK, seed=300 + d + H + HK)
    log(f"case {wl.name} T={wl.total_tokens} track_at={TRACK_AT} track_slots={ts.tolist()}")
    dv = device_inputs(wl)
    out = torch.empty_like(dv["q"])
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                  wl.max_seqlen, track_lens=i32(TRACK_AT), track_slot_idx=i32(ts))
    torch.cuda.synchronize()
    slopes = oracle.alibi_slopes(H, wl.layer_id, wl.num_layers)
    ref_out, ref_fin, ref_snap = oracle.prefill(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.pool, wl.slot_idx,
                                                slopes, track_lens=TRACK_AT)
    tol = TOL[dtype]
    assert_close(host_io(out), ref_out, tol, f"{wl.name} out")
    got_pool = dv["pool"].cpu().numpy()
    exp_pool = oracle.scatter(wl.pool, wl.slot_idx, ref_fin, track_slots=ts, track_states=ref_snap)
    written = set(int(s) for s in wl.slot_idx)
    written |= {int(s) for b, s in enumerate(ts) if s >= 0 and TRACK_AT[b] <= TRACK_LENS[b]}
    w = sorted(written)
    assert_close(got_pool[w], exp_pool[w], tol, f"{wl.name} active+track slots")
    keep = [s for s in range(wl.pool_slots) if s not in written]
    assert np.array_equal(got_pool[keep].view(np.uint32), wl.pool[keep].view(np.uint32)), \
        "a slot that no request may write changed"
    # a snapshot after 0 tokens is the prefix state itself
    for b in (1, 4):
        assert np.array_equal(got_pool[ts[b]].view(np.uint32), wl.pool[wl.slot_idx[b]].view(np.uint32))


def test_track_snapshot_long_request_at_chunk_edges():
    """One long bf16 request (the chunked kernel) with snapshots exactly on and
    next to 64-token chunk boundaries, each in its own call."""
    base = W.make("track-long", "prefill", "bf16", 8, [4099], 4, seed=333, prefix=[True], slot_idx=[2])
    slopes = oracle.alibi_slopes(8, 0, 1)
    for tl in (63, 64, 65, 2048, 4098):
        dv = device_inputs(base)
        out = torch.empty_like(dv["q"])
        la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                      base.max_seqlen, track_lens=i32([tl]), track_slot_idx=i32([0]))
        torch.cuda.synchronize()
        log(f"case track-long tl={tl}")
        ref_out, ref_fin, ref_snap = oracle.prefill(base.q, base.k, base.v, base.cu_seqlens, base.pool,
                                                    base.slot_idx, slopes, track_lens=[tl])
        assert_close(host_io(out), ref_out, TOL["bf16"], f"track-long tl={tl} out")
        pool = dv["pool"].cpu().numpy()
        assert_close(pool[2], ref_fin[0], TOL["bf16"], f"track-long tl={tl} final")
        assert_close(pool[0], ref_snap[0], TOL["bf16"], f"track-long tl={tl} snapshot")
        for s in (1, 3):
            assert np.array_equal(pool[s].view(np.uint32), base.pool[s].view(np.uint32))


def test_track_debug_mode_rejects_bad_track_arrays(monkeypatch):
    wl, ts = _track_case("bf16", 128, 2, 2, seed=5)
    dv = device_inputs(wl)
    out = torch.empty_like(dv["q"])
    monkeypatch.setenv("LA_DEBUG", "1")
    bad_len = list(TRACK_AT)   # request 5 tracks past its end: an error in debug mode
    with pytest.raises(la.LAError):
        la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                      wl.max_seqlen, track_lens=i32(bad_len), track_slot_idx=i32(ts))
    ok_len = list(TRACK_AT)
    ok_len[5] = 10
    clash = ts.copy()
    clash[0] = wl.slot_idx[3]  # a track slot that is another request's active slot
    with pytest.raises(la.LAError):
        la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                      wl.max_seqlen, track_lens=i32(ok_len), track_slot_idx=i32(clash))
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out,
                  wl.max_seqlen, track_lens=i32(ok_len), track_slot_idx=i32(ts))
    torch.cuda.synchronize()


# ---------------------------------------------------------------- grouped heads, head_dim 64

def _full(wl, state_out=False):
    log(f"case {wl.name} B={wl.batch} T={wl.total_tokens} H={wl.num_heads}/{wl.num_kv_heads} "
        f"d={wl.head_dim}")
    out, pool, so = run_gpu(wl, state_out=state_out)
    check_against_oracle(wl, out, pool, so)
    check_untouched(wl, pool, addressed=(so is None))


VARLEN = [1, 63, 64, 65, 200, 513, 0, 129]


@pytest.mark.parametrize("dtype,d,H,HK", [("bf16", 128, 8, 2), ("bf16", 128, 8, 1), ("fp32", 128, 6, 3),
                                          ("bf16", 64, 4, 4), ("bf16", 64, 8, 2), ("fp32", 64, 3, 3)])
def test_prefill_grouped_heads_and_head_dim(dtype, d, H, HK):
    wl = W.make(f"prefill-{dtype}-d{d}-H{H}/{HK}", "prefill", dtype, H, VARLEN, 12, head_dim=d,
                seed=400 + H + HK + d, prefix=[i % 3 != 0 for i in range(len(VARLEN))], num_kv_heads=HK,
                layer_id=2, num_layers=4)
    _full(wl)


@pytest.mark.parametrize("dtype,d,H,HK", [("bf16", 128, 16, 4), ("fp32", 128, 4, 1), ("bf16", 64, 8, 8),
                                          ("fp32", 64, 8, 2)])
def test_decode_grouped_heads_and_head_dim(dtype, d, H, HK):
    wl = W.make(f"decode-{dtype}-d{d}-H{H}/{HK}", "decode", dtype, H, np.ones(32, dtype=np.int64), 40,
                head_dim=d, seed=500 + H + d, fill_all_slots=True, num_kv_heads=HK)
    _full(wl)


@pytest.mark.parametrize("dtype,d,HK,state_out", [("bf16", 128, 2, True), ("fp32", 64, 1, False),
                                                  ("bf16", 64, 4, True)])
def test_chain_verify_grouped_heads_and_head_dim(dtype, d, HK, state_out):
    wl = W.make(f"verify-{dtype}-d{d}-H8/{HK}", "verify", dtype, 8, np.full(24, 3, dtype=np.int64), 30,
                head_dim=d, seed=600 + d + HK, prefix=np.ones(24, dtype=bool), num_kv_heads=HK,
                num_draft=3)
    _full(wl, state_out=state_out)


def test_head_dim_64_long_prefill_sampled_heads():
    """A 16384-token head_dim-64 request (256 chunks of the chunked kernel) on sampled heads."""
    wl = W.make("prefill-d64-long", "prefill", "bf16", 16, [16384], 2, head_dim=64, seed=611,
                prefix=[True], slot_idx=[1])
    log(f"case {wl.name} T={wl.total_tokens}")
    out, pool, _ = run_gpu(wl)
    check_against_oracle(wl, out, pool, heads=[0, 7, 15])
    check_untouched(wl, pool)


# ---------------------------------------------------------------- slope regimes, invalid slots

# slopes in [0, 2] take the chunked kernel's scaled-state decay, larger ones
# its explicit per-token weights; in the token-recurrent kernel (fp32) the
# decay groups shrink as the slope grows (8 tokens up to 32/7, 5 at 8, one
# token at 40)
SLOPES = [0.0, 1e-3, 0.25, 2.0, 2.0001, 3.0, 8.0, 0.9, 40.0]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64), ("fp32", 128)])
def test_prefill_slopes_on_both_sides_of_two(dtype, d):
    lens = [1, 64, 65, 200, 130]
    H = len(SLOPES)
    wl = W.make(f"slopes-{dtype}-d{d}", "prefill", dtype, H, lens, 8, head_dim=d, seed=950 + d,
                prefix=[True, False, True, True, False])
    log(f"case {wl.name} lens={lens} slopes={SLOPES}")
    dv = device_inputs(wl)
    slopes = np.array(SLOPES, dtype=np.float32)
    out = torch.empty_like(dv["q"])
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], torch.from_numpy(slopes).cuda(),
                  out, wl.max_seqlen)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.prefill(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.pool, wl.slot_idx, slopes)
    assert_close(host_io(out), ref_out, TOL[dtype], f"{wl.name} out")
    fin = dv["pool"].index_select(0, torch.from_numpy(wl.slot_idx.astype(np.int64)).cuda()).cpu().numpy()
    assert_close(fin, ref_fin, TOL[dtype], f"{wl.name} final state")
    check_untouched(wl, dv["pool"])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128)])
def test_prefill_out_of_range_slot_gives_zero_output(dtype, d):
    """Without the debug checks, a request whose slot index is out of range
    gets a zero output and touches no state; the other requests are unaffected."""
    lens = [70, 130, 5, 64]
    wl = W.make(f"badslot-{dtype}-d{d}", "prefill", dtype, 4, lens, 6, head_dim=d, seed=960 + d,
                prefix=[True] * 4)
    log(f"case {wl.name} lens={lens}")
    dv = device_inputs(wl)
    bad = wl.slot_idx.astype(np.int32).copy()
    bad[1], bad[3] = -1, wl.pool_slots
    out = torch.full_like(dv["q"], 7.0)
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], i32(bad), dv["slopes"], out, wl.max_seqlen)
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
    assert_close(got[rows], ref_out, TOL[dtype], f"{wl.name} out")
    fin = dv["pool"].index_select(0, torch.from_numpy(wl.slot_idx[good].astype(np.int64)).cuda()).cpu().numpy()
    assert_close(fin, ref_fin, TOL[dtype], f"{wl.name} final state")
    keep = np.setdiff1d(np.arange(wl.pool_slots), wl.slot_idx[good])
    after = dv["pool"].index_select(0, torch.from_numpy(keep).cuda()).cpu().numpy()
    assert np.array_equal(after.view(np.uint32), wl.pool[keep].view(np.uint32)), "untouched slot changed"


# ---------------------------------------------------------------- tree verify

TREES = {
    "chain": [-1, 0, 1, 2, 3, 4, 5],
    "star": [-1, -1, -1, -1, -1],
    "binary": [-1, 0, 0, 1, 1, 2, 2],
    "two_roots": [-1, 0, -1, 2, 1, 3, 0],
    "single": [-1],
}


def _tree_workload(name, dtype, d, H, HK, B, n, seed):
    return W.make(name, "verify", dtype, H, np.full(B, n, dtype=np.int64), B + 5, head_dim=d, seed=seed,
                  prefix=[b % 4 != 3 for b in range(B)], num_kv_heads=HK, num_draft=n)


def _run_tree(wl, parents, with_states=True):
    dv = device_inputs(wl)
    pool_before = dv["pool"].clone()
    out = torch.empty_like(dv["q"])
    B, n = parents.shape
    ds = (torch.empty((B, n, wl.num_heads, wl.head_dim, wl.head_dim), device="cuda")
          if with_states else None)
    la.la_verify_tree(dv["q"], dv["k"], dv["v"], n, dv["pool"], dv["slot"], i32(parents), dv["slopes"],
                      out, ds)
    torch.cuda.synchronize()
    assert torch.equal(dv["pool"].view(torch.int32), pool_before.view(torch.int32)), "tree verify wrote the pool"
    return out, ds


def _oracle_tree(wl, parents, reqs=None):
    slopes = oracle.alibi_slopes(wl.num_heads, wl.layer_id, wl.num_layers)
    n = parents.shape[1]
    if reqs is None:
        reqs = np.arange(wl.batch)
    tok = (reqs[:, None] * n + np.arange(n)[None, :]).reshape(-1)
    return oracle.tree_verify(wl.q[tok], wl.k[tok], wl.v[tok], n, parents[reqs], wl.pool,
                              wl.slot_idx[reqs], slopes)


@pytest.mark.parametrize("tree", sorted(TREES))
@pytest.mark.parametrize("dtype,d,HK", [("bf16", 128, 4), ("fp32", 128, 2), ("bf16", 64, 1)])
def test_tree_verify_shapes(tree, dtype, d, HK):
    """[LA-page] Next Work item 2: each draft forks from its parent's saved state;
    outputs and every per-position state against the oracle."""
    par = np.array(TREES[tree], dtype=np.int32)
    B, n = 12, len(par)
    wl = _tree_workload(f"tree-{tree}-{dtype}-d{d}", dtype, d, 4, HK, B, n, seed=700 + n + d + HK)
    parents = np.tile(par, (B, 1))
    log(f"case {wl.name} parents={par.tolist()}")
    out, ds = _run_tree(wl, parents)
    ref_out, ref_states = _oracle_tree(wl, parents)
    tol = TOL[dtype]
    assert_close(host_io(out), ref_out, tol, f"{wl.name} out")
    assert_close(ds.cpu().numpy(), ref_states, tol, f"{wl.name} draft states")
    out2, _ = _run_tree(wl, parents, with_states=False)
    assert torch.equal(out2, out), "outputs differ without draft_states"


def test_tree_verify_chain_matches_chain_verify():
    """Chain parents at the full chain-verify shape: outputs and the last
    per-position state agree with la_verify to fp32 rounding (the two kernels
    may contract their multiply-adds differently; bf16 outputs may then differ
    by one bf16 step)."""
    wl = W.config(5)
    n, B = wl.num_draft, wl.batch
    log(f"case tree-chain vs chain verify B={B} n={n}")
    parents = np.tile(np.arange(-1, n - 1, dtype=np.int32), (B, 1))
    out_t, ds = _run_tree(wl, parents)
    out_c, _, so = run_gpu(wl, state_out=True)
    assert_close(host_io(out_t), host_io(out_c), 8e-3, "tree chain out vs chain verify")
    assert_close(ds[:, n - 1].cpu().numpy(), so.cpu().numpy(), 1e-5, "tree chain state vs chain verify")


def test_tree_verify_full_size_random_trees():
    """B=128 requests of 5 drafts at H=64, d=128 (the chain-verify shape) with a
    seeded random tree per request; checked group by group against the oracle."""
    B, n = 128, 5
    rng = np.random.default_rng(777)
    parents = np.full((B, n), -1, dtype=np.int32)
    for b in range(B):
        for j in range(1, n):
            parents[b, j] = rng.integers(-1, j)
    wl = _tree_workload("tree-full", "bf16", 128, 64, 64, B, n, seed=778)
    log(f"case {wl.name} B={B} n={n} H=64")
    out, ds = _run_tree(wl, parents)
    got_out = host_io(out).reshape(B, n, 64, 128)
    for g0 in range(0, B, 32):
        reqs = np.arange(g0, g0 + 32)
        ref_out, ref_states = _oracle_tree(wl, parents, reqs)
        assert_close(got_out[reqs].reshape(-1, 64, 128), ref_out, TOL["bf16"], f"tree-full out {g0}")
        assert_close(ds[g0:g0 + 32].cpu().numpy(), ref_states, TOL["bf16"], f"tree-full states {g0}")


def test_tree_verify_bad_parents_zero_output_and_debug_error(monkeypatch):
    """A request whose parent list is invalid gets zero output and no state (the
    kernel's own check); with LA_DEBUG=1 the call is rejected instead."""
    B, n = 4, 4
    wl = _tree_workload("tree-bad", "bf16", 128, 2, 2, B, n, seed=790)
    parents = np.tile(np.array([-1, 0, 1, 2], dtype=np.int32), (B, 1))
    parents[2] = [-1, 2, 0, 1]  # parent of draft 1 is a later draft
    dv = device_inputs(wl)
    out = torch.full_like(dv["q"], 7.0)
    ds = torch.full((B, n, 2, 128, 128), 3.0, device="cuda")
    la.la_verify_tree(dv["q"], dv["k"], dv["v"], n, dv["pool"], dv["slot"], i32(parents), dv["slopes"],
                      out, ds)
    torch.cuda.synchronize()
    o = out.float().view(B, n, 2, 128)
    assert torch.all(o[2] == 0)
    assert torch.all(ds[2] == 3.0)
    good = [0, 1, 3]
    ref_out, ref_states = _oracle_tree(wl, parents, np.array(good))
    assert_close(host_io(out).reshape(B, n, 2, 128)[good].reshape(-1, 2, 128), ref_out, TOL["bf16"],
                 "tree-bad valid requests")
    monkeypatch.setenv("LA_DEBUG", "1")
    with pytest.raises(la.LAError):
        la.la_verify_tree(dv["q"], dv["k"], dv["v"], n, dv["pool"], dv["slot"], i32(parents),
                          dv["slopes"], out, ds)


# ---------------------------------------------------------------- HIP graphs

def test_graph_capture_replay_decode_and_verify():
    """Decode, chain verify and tree verify captured in one HIP graph
    ([LA-page] §生产环境不支持 item 2: graph capture covers the decode and
    target-verify modes) and replayed several times, with eager work between
    replays.  Every replay's outputs, pool and states match the fp64 oracle
    within the bf16 bound, and the eager run bit for bit."""
    dec = W.make("graph-decode", "decode", "bf16", 8, np.ones(6, dtype=np.int64), 16, seed=800,
                 fill_all_slots=True)
    ver = W.make("graph-verify", "verify", "bf16", 8, np.full(4, 3, dtype=np.int64), 8, seed=801,
                 prefix=np.ones(4, dtype=bool), num_draft=3, num_kv_heads=2)
    dd, dv = device_inputs(dec), device_inputs(ver)
    pool0 = dd["pool"].clone()
    par_np = np.tile(np.array([-1, 0, 0], dtype=np.int32), (4, 1))
    parents = i32(par_np)
    out_d = torch.empty_like(dd["q"])
    out_v = torch.empty_like(dv["q"])
    out_t = torch.empty_like(dv["q"])
    so = torch.empty((4, 8, 128, 128), device="cuda")
    ds = torch.empty((4, 3, 8, 128, 128), device="cuda")

    # the oracle's results for one step from the initial pools
    tol = TOL["bf16"]
    ref_d_out, ref_d_fin = oracle_ref(dec)
    ref_d_pool = oracle.scatter(dec.pool, dec.slot_idx, ref_d_fin)
    ref_v_out, ref_v_fin = oracle_ref(ver)
    ref_t_out, ref_t_states = _oracle_tree(ver, par_np)

    def step():
        la.la_decode(dd["q"], dd["k"], dd["v"], dd["pool"], dd["slot"], dd["slopes"], out_d)
        la.la_verify(dv["q"], dv["k"], dv["v"], 3, dv["pool"], dv["slot"], dv["slopes"], out_v, so)
        la.la_verify_tree(dv["q"], dv["k"], dv["v"], 3, dv["pool"], dv["slot"], parents, dv["slopes"],
                          out_t, ds)

    def check_oracle(what):
        assert_close(host_io(out_d), ref_d_out, tol, f"{what} decode out")
        assert_close(dd["pool"].cpu().numpy(), ref_d_pool, tol, f"{what} decode pool")
        assert_close(host_io(out_v), ref_v_out, tol, f"{what} verify out")
        assert_close(so.cpu().numpy(), ref_v_fin, tol, f"{what} verify state")
        assert_close(host_io(out_t), ref_t_out, tol, f"{what} tree out")
        assert_close(ds.cpu().numpy(), ref_t_states, tol, f"{what} tree states")

    step()
    torch.cuda.synchronize()
    check_oracle("eager")
    ref = [t.clone() for t in (out_d, dd["pool"], out_v, so, out_t, ds)]

    dd["pool"].copy_(pool0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: reset the pool, scribble over the outputs
        dd["pool"].copy_(pool0)
        for t in (out_d, out_v, out_t):
            t.fill_(-1.0)
        so.zero_()
        ds.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_oracle(f"replay {rep}")
        got = (out_d, dd["pool"], out_v, so, out_t, ds)
        for name, a, b in zip(("decode out", "decode pool", "verify out", "verify state", "tree out",
                               "tree states"), got, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"replay {rep}: {name} differs"
        log(f"graph replay {rep} ok")
