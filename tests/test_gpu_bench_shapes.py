"""GPU parity at the exact shapes of the benchmark's prefill variants, against
the fp64 oracle, so that every rate the benchmark reports comes from a call
checked at its own shape:

  * one GPU's share at 8-way head parallelism: heads 0..7 of the 131072-token
    request (split into sequence segments, with a caller workspace);
  * head_dim 64: the first 16384 tokens and 64 features of every head, 64
    heads (two sequence segments);
  * grouped heads: 64 query heads over the first 8 kv heads, all 131072 tokens;
  * a state-tracking snapshot after 65536 tokens of the long request.

The inputs are slices of the long-prefill workload (T=131072, H=64, d=128), as
in the benchmark.  Tolerance 3e-2 (|got - ref| <= tol + tol * |ref|) on outputs,
final states and snapshots; the oracle runs eight heads at a time.
"""
import numpy as np
import pytest
import torch

import linear_attention_amd as la
import oracle
from linear_attention_amd import workloads as W

from gpu_util import TOL, assert_close, dev_io, host_io, log

pytestmark = pytest.mark.gpu
TOLB = TOL["bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


@pytest.fixture(scope="module")
def long_wl():
    return W.config(4)


def _slopes(wl):
    return oracle.alibi_slopes(wl.num_heads, wl.layer_id, wl.num_layers)


def test_tp8_share(long_wl):
    wl = long_wl
    T, heads = wl.total_tokens, list(range(8))
    q, k, v = (np.ascontiguousarray(x[:, heads]) for x in (wl.q, wl.k, wl.v))
    pool = np.ascontiguousarray(wl.pool[:, heads])
    sl = _slopes(wl)[heads]
    need = la.la_prefill_workspace_bytes(1, T, T, 8, 128)
    log(f"tp8 share: T={T} H=8, workspace {need} B")
    assert need > 0
    dpool = torch.from_numpy(pool).cuda()
    out = torch.empty((T, 8, 128), dtype=torch.bfloat16, device="cuda")
    la.la_prefill(dev_io(q, "bf16"), dev_io(k, "bf16"), dev_io(v, "bf16"),
                  torch.tensor([0, T], dtype=torch.int32, device="cuda"), dpool,
                  torch.tensor([0], dtype=torch.int32, device="cuda"), torch.from_numpy(sl).cuda(), out, T,
                  workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.prefill(q, k, v, np.array([0, T]), pool, np.array([0]), sl)
    assert_close(host_io(out), ref_out, TOLB, "tp8 share out")
    assert_close(dpool[0].cpu().numpy(), ref_fin[0], TOLB, "tp8 share final state")
    assert np.array_equal(dpool[1].cpu().numpy().view(np.uint32), pool[1].view(np.uint32)), "sentinel slot changed"


def test_head_dim_64_shape(long_wl):
    wl = long_wl
    T = 16384
    q, k, v = (np.ascontiguousarray(x[:T, :, :64]) for x in (wl.q, wl.k, wl.v))
    pool = np.zeros((2, 64, 64, 64), dtype=np.float32)
    sl = _slopes(wl)
    log(f"head_dim 64: T={T} H=64, workspace {la.la_prefill_workspace_bytes(1, T, T, 64, 64)} B")
    dpool = torch.from_numpy(pool).cuda()
    out = torch.empty((T, 64, 64), dtype=torch.bfloat16, device="cuda")
    la.la_prefill(dev_io(q, "bf16"), dev_io(k, "bf16"), dev_io(v, "bf16"),
                  torch.tensor([0, T], dtype=torch.int32, device="cuda"), dpool,
                  torch.tensor([0], dtype=torch.int32, device="cuda"), torch.from_numpy(sl).cuda(), out, T)
    torch.cuda.synchronize()
    got = host_io(out)
    fin = dpool[0].cpu().numpy()
    for g in range(0, 64, 8):
        hs = list(range(g, g + 8))
        ref_out, ref_fin = oracle.prefill(q[:, hs], k[:, hs], v[:, hs], np.array([0, T]), pool[:, hs],
                                          np.array([0]), sl[hs])
        assert_close(got[:, hs], ref_out, TOLB, f"d64 heads {g}..{g + 7} out")
        assert_close(fin[hs], ref_fin[0], TOLB, f"d64 heads {g}..{g + 7} final state")


def test_grouped_heads_shape(long_wl):
    wl = long_wl
    T = wl.total_tokens
    k8, v8 = (np.ascontiguousarray(x[:, :8]) for x in (wl.k, wl.v))
    pool = np.zeros((2, 64, 128, 128), dtype=np.float32)
    sl = _slopes(wl)
    log(f"grouped heads: T={T} H=64 Hkv=8")
    dpool = torch.from_numpy(pool).cuda()
    out = torch.empty((T, 64, 128), dtype=torch.bfloat16, device="cuda")
    la.la_prefill(dev_io(wl.q, "bf16"), dev_io(k8, "bf16"), dev_io(v8, "bf16"),
                  torch.tensor([0, T], dtype=torch.int32, device="cuda"), dpool,
                  torch.tensor([0], dtype=torch.int32, device="cuda"), torch.from_numpy(sl).cuda(), out, T)
    torch.cuda.synchronize()
    fin = dpool[0].cpu().numpy()
    for g in range(0, 64, 8):
        hs = list(range(g, g + 8))  # one kv group: kv head g // 8
        ref_out, ref_fin = oracle.prefill(np.ascontiguousarray(wl.q[:, hs]), k8[:, [g // 8]], v8[:, [g // 8]],
                                          np.array([0, T]), pool[:, hs], np.array([0]), sl[hs])
        assert_close(host_io(out[:, g:g + 8]), ref_out, TOLB, f"grouped heads {g}..{g + 7} out")
        assert_close(fin[hs], ref_fin[0], TOLB, f"grouped heads {g}..{g + 7} final state")


def test_snapshot_shape_sampled_heads(long_wl):
    """The bench's snapshot variant (track length 65536 into slot 1) on the
    full request; outputs, final state and snapshot checked on two groups of
    heads (the largest and the smallest slopes)."""
    wl = long_wl
    T, tl = wl.total_tokens, wl.total_tokens // 2
    log(f"snapshot: T={T} H=64 track_len={tl}")
    dpool = torch.from_numpy(wl.pool).cuda()
    out = torch.empty((T, 64, 128), dtype=torch.bfloat16, device="cuda")
    la.la_prefill(dev_io(wl.q, "bf16"), dev_io(wl.k, "bf16"), dev_io(wl.v, "bf16"),
                  torch.tensor([0, T], dtype=torch.int32, device="cuda"), dpool,
                  torch.tensor([0], dtype=torch.int32, device="cuda"), torch.from_numpy(_slopes(wl)).cuda(), out, T,
                  track_lens=torch.tensor([tl], dtype=torch.int32, device="cuda"),
                  track_slot_idx=torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    sl = _slopes(wl)
    for hs in (list(range(8)), list(range(56, 64))):
        ref_out, ref_fin, ref_snap = oracle.prefill(
            np.ascontiguousarray(wl.q[:, hs]), np.ascontiguousarray(wl.k[:, hs]), np.ascontiguousarray(wl.v[:, hs]),
            np.array([0, T]), np.ascontiguousarray(wl.pool[:, hs]), np.array([0]), sl[hs], track_lens=[tl])
        assert_close(host_io(out[:, hs[0]:hs[-1] + 1]), ref_out, TOLB, f"snapshot heads {hs[0]}.. out")
        assert_close(dpool[0, hs[0]:hs[-1] + 1].cpu().numpy(), ref_fin[0], TOLB, f"snapshot heads {hs[0]}.. final")
        assert_close(dpool[1, hs[0]:hs[-1] + 1].cpu().numpy(), ref_snap[0], TOLB, f"snapshot heads {hs[0]}.. snapshot")
