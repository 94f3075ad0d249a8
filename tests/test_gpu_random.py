"""GPU parity on seeded random configurations (prefill, decode and chain
verify; tree verify with random parents; prefill with random snapshots).

Each case draws its own configuration from a seeded generator, so that
combinations the hand-written cases do not name are covered:
* entry point (prefill, decode, chain verify with and without state_out);
* head count and kv grouping; head_dim 64 or 128; bf16 or fp32;
* request count and lengths: empty, single-token, chunk-edge, a few hundred
  or thousand tokens, and now and then one long enough to split a few-head
  launch into sequence segments;
* prefix or zero states, pool slots in any order with spares, layer factor.

Every output and final state is checked against the fp64 oracle, and every
pool slot a call must not write is compared bit for bit.  The case's
configuration is printed before it runs.
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_amd as la
import oracle
from linear_attention_amd import workloads as W

from gpu_util import TOL, assert_close, check_against_oracle, check_untouched, device_inputs, host_io, log, run_gpu

pytestmark = pytest.mark.gpu


def _seeds(default):
    """Seeds of the random cases: range(default), or range(a, a + n) when the
    environment sets LA_RANDOM_SEEDS=a:n (for a longer campaign)."""
    spec = os.environ.get("LA_RANDOM_SEEDS")
    if not spec:
        return range(default)
    a, n = (int(x) for x in spec.split(":"))
    return range(a, a + n)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def _lengths(rng, B, dtype, allow_long):
    """Per-request lengths from a mix of regimes (fp32 prefill runs the
    token-recurrent kernel, so it stays short)."""
    cap = 700 if dtype == "fp32" else 5000
    regimes = [lambda: 0, lambda: int(rng.integers(1, 4)), lambda: int(rng.choice([63, 64, 65, 127, 128, 129])),
               lambda: int(rng.integers(2, 700)), lambda: int(rng.integers(700, cap + 1))]
    p = np.array([0.08, 0.12, 0.2, 0.4, 0.2])
    lens = [regimes[rng.choice(len(regimes), p=p)]() for _ in range(B)]
    if allow_long:
        lens[int(rng.integers(B))] = int(rng.integers(8192, 14000))
    return lens


def _config(seed):
    rng = np.random.default_rng(10_000 + seed)
    kind = rng.choice(["prefill", "prefill", "prefill", "decode", "verify"])
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    d = int(rng.choice([64, 128]))
    # a long request only where the launch is small enough to be split
    allow_long = kind == "prefill" and dtype == "bf16" and rng.random() < 0.3
    H = int(rng.choice([1, 2, 3, 4] if allow_long else [1, 2, 3, 4, 6, 8, 12, 16]))
    groups = [g for g in range(1, H + 1) if H % g == 0]
    HK = H // int(rng.choice(groups))
    num_layers = int(rng.choice([1, 4, 24]))
    layer_id = int(rng.integers(num_layers))
    num_draft = 1
    if kind == "prefill":
        B = int(rng.integers(1, 4 if allow_long else 13))
        lengths = _lengths(rng, B, dtype, allow_long)
    else:
        B = int(rng.integers(1, 40))
        num_draft = 1 if kind == "decode" else int(rng.integers(1, 7))
        lengths = [num_draft] * B
    P = B + int(rng.integers(0, 4))
    prefix = (rng.random(B) < 0.6).tolist()
    state_out = kind == "verify" and rng.random() < 0.5
    wl = W.make(f"random-{seed}", kind, dtype, H, lengths, P, head_dim=d, seed=20_000 + seed, layer_id=layer_id,
                num_layers=num_layers, prefix=prefix, num_draft=num_draft, num_kv_heads=HK)
    return wl, state_out


@pytest.mark.parametrize("seed", _seeds(60))
def test_random_configuration(seed):
    wl, state_out = _config(seed)
    log(f"case {wl.name}: {wl.kind} {wl.dtype} B={wl.batch} H={wl.num_heads} HK={wl.num_kv_heads} "
        f"d={wl.head_dim} layer={wl.layer_id}/{wl.num_layers} P={wl.pool_slots} lens={wl.lengths.tolist()} "
        f"state_out={state_out}")
    out, pool, so = run_gpu(wl, state_out=state_out)
    check_against_oracle(wl, out, pool, so)
    check_untouched(wl, pool, addressed=(so is None))


def _small_config(rng):
    dtype = "fp32" if rng.random() < 0.25 else "bf16"
    d = int(rng.choice([64, 128]))
    H = int(rng.choice([1, 2, 3, 4, 6, 8]))
    groups = [g for g in range(1, H + 1) if H % g == 0]
    return dtype, d, H, H // int(rng.choice(groups))


@pytest.mark.parametrize("seed", _seeds(20))
def test_random_tree(seed):
    """Tree verify with a random parent array per request: outputs and every
    per-position state against the oracle; the pool is never written."""
    rng = np.random.default_rng(30_000 + seed)
    dtype, d, H, HK = _small_config(rng)
    B, n = int(rng.integers(1, 21)), int(rng.integers(1, 9))
    parents = np.full((B, n), -1, dtype=np.int32)
    for b in range(B):
        for j in range(1, n):
            parents[b, j] = rng.integers(-1, j)
    wl = W.make(f"random-tree-{seed}", "verify", dtype, H, [n] * B, B + int(rng.integers(0, 4)), head_dim=d,
                seed=40_000 + seed, prefix=(rng.random(B) < 0.7).tolist(), num_draft=n, num_kv_heads=HK)
    log(f"case {wl.name}: {dtype} B={B} n={n} H={H} HK={HK} d={d} parents={parents.tolist()}")
    dv = device_inputs(wl)
    pool_before = dv["pool"].clone()
    out = torch.empty_like(dv["q"])
    ds = torch.empty((B, n, H, d, d), device="cuda")
    la.la_verify_tree(dv["q"], dv["k"], dv["v"], n, dv["pool"], dv["slot"], torch.from_numpy(parents).cuda(),
                      dv["slopes"], out, ds)
    torch.cuda.synchronize()
    assert torch.equal(dv["pool"].view(torch.int32), pool_before.view(torch.int32)), "tree verify wrote the pool"
    slopes = oracle.alibi_slopes(H, wl.layer_id, wl.num_layers)
    ref_out, ref_states = oracle.tree_verify(wl.q, wl.k, wl.v, n, parents, wl.pool, wl.slot_idx, slopes)
    assert_close(host_io(out), ref_out, TOL[dtype], f"{wl.name} out")
    assert_close(ds.cpu().numpy(), ref_states, TOL[dtype], f"{wl.name} draft states")


@pytest.mark.parametrize("seed", _seeds(20))
def test_random_track(seed):
    """Prefill with state snapshots: random snapshot points (0, mid-chunk, a
    chunk edge, the whole request), some requests without one, track slots
    among the spare pool slots."""
    rng = np.random.default_rng(50_000 + seed)
    dtype, d, H, HK = _small_config(rng)
    B = int(rng.integers(1, 9))
    lengths = _lengths(rng, B, dtype, False)
    P = 2 * B + int(rng.integers(0, 3))
    perm = rng.permutation(P)
    slot_idx, spare = perm[:B], perm[B:]
    track_lens, track_slots = np.zeros(B, dtype=np.int32), np.full(B, -1, dtype=np.int32)
    for b in range(B):
        n = lengths[b]
        track_lens[b] = rng.choice([0, n, n // 2, (n // 64) * 64, int(rng.integers(0, n + 1))])
        if rng.random() < 0.8:
            track_slots[b] = spare[b]
    wl = W.make(f"random-track-{seed}", "prefill", dtype, H, lengths, P, head_dim=d, seed=60_000 + seed,
                prefix=(rng.random(B) < 0.6).tolist(), slot_idx=slot_idx, num_kv_heads=HK)
    log(f"case {wl.name}: {dtype} H={H} HK={HK} d={d} lens={lengths} track_lens={track_lens.tolist()} "
        f"track_slots={track_slots.tolist()} slots={slot_idx.tolist()}")
    dv = device_inputs(wl)
    out = torch.empty_like(dv["q"])
    la.la_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], dv["pool"], dv["slot"], dv["slopes"], out, wl.max_seqlen,
                  track_lens=torch.from_numpy(track_lens).cuda(), track_slot_idx=torch.from_numpy(track_slots).cuda())
    torch.cuda.synchronize()
    slopes = oracle.alibi_slopes(H, wl.layer_id, wl.num_layers)
    ref_out, ref_fin, ref_snap = oracle.prefill(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.pool, wl.slot_idx, slopes,
                                                track_lens=track_lens)
    assert_close(host_io(out), ref_out, TOL[dtype], f"{wl.name} out")
    got = dv["pool"].cpu().numpy()
    exp = oracle.scatter(wl.pool, wl.slot_idx, ref_fin, track_slots=track_slots, track_states=ref_snap)
    written = sorted(set(int(s) for s in slot_idx) | {int(s) for s in track_slots if s >= 0})
    assert_close(got[written], exp[written], TOL[dtype], f"{wl.name} active and track slots")
    keep = [s for s in range(P) if s not in written]
    assert np.array_equal(got[keep].view(np.uint32), wl.pool[keep].view(np.uint32)), "an unnamed slot changed"
