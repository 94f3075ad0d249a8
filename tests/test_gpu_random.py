"""GPU parity on seeded random configurations.

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
import numpy as np
import pytest
import torch

import linear_attention_amd as la
from linear_attention_amd import workloads as W

from gpu_util import check_against_oracle, check_untouched, log, run_gpu

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("seed", range(60))
def test_random_configuration(seed):
    wl, state_out = _config(seed)
    log(f"case {wl.name}: {wl.kind} {wl.dtype} B={wl.batch} H={wl.num_heads} HK={wl.num_kv_heads} "
        f"d={wl.head_dim} layer={wl.layer_id}/{wl.num_layers} P={wl.pool_slots} lens={wl.lengths.tolist()} "
        f"state_out={state_out}")
    out, pool, so = run_gpu(wl, state_out=state_out)
    check_against_oracle(wl, out, pool, so)
    check_untouched(wl, pool, addressed=(so is None))
