"""Helpers for the GPU parity tests: move seeded workloads to the device, run
the C ABI through the Python binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import linear_attention_amd as la
import oracle

# Tolerances: bf16 inputs 3e-2 (the page's eager tolerance) and fp32 inputs
# 1e-4, applied as |got - ref| <= tol + tol * |ref| to outputs and final states.
TOL = {"bf16": 3e-2, "fp32": 1e-4}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_io(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def host_io(t: torch.Tensor) -> np.ndarray:
    """Device output -> numpy (bf16 as uint16 bits, fp32 as float32)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def slopes_dev(wl) -> torch.Tensor:
    return torch.from_numpy(la.la_alibi_slopes(wl.num_heads, wl.layer_id, wl.num_layers)).cuda()


def device_inputs(wl):
    return dict(
        q=dev_io(wl.q, wl.dtype), k=dev_io(wl.k, wl.dtype), v=dev_io(wl.v, wl.dtype),
        pool=torch.from_numpy(wl.pool).cuda(),
        cu=torch.from_numpy(wl.cu_seqlens.astype(np.int32)).cuda(),
        slot=torch.from_numpy(wl.slot_idx.astype(np.int32)).cuda(),
        slopes=slopes_dev(wl),
    )


def run_gpu(wl, d=None, state_out=False):
    """Run the workload's entry point on the GPU.  Returns (out, pool_after,
    state_out or None) as device tensors."""
    d = d or device_inputs(wl)
    out = torch.empty_like(d["q"])
    so = None
    if wl.kind == "prefill":
        la.la_prefill(d["q"], d["k"], d["v"], d["cu"], d["pool"], d["slot"], d["slopes"], out,
                      wl.max_seqlen)
    elif wl.kind == "decode":
        la.la_decode(d["q"], d["k"], d["v"], d["pool"], d["slot"], d["slopes"], out)
    else:
        if state_out:
            so = torch.empty((wl.batch, wl.num_heads, wl.head_dim, wl.head_dim), device="cuda")
        la.la_verify(d["q"], d["k"], d["v"], wl.num_draft, d["pool"], d["slot"], d["slopes"], out,
                     so)
    torch.cuda.synchronize()
    return out, d["pool"], so


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact upcast (bf16 bit patterns as uint16), the oracle's own pinned one."""
    return oracle.to_f64(x)


def assert_close(got, ref, tol, what):
    got = to_f64(np.asarray(got))
    ref = to_f64(np.asarray(ref))
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    bad = ~(err <= bound)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    msg = (f"{what}: max_abs={err.max() if err.size else 0:.3e} "
           f"max_rel={rel.max() if rel.size else 0:.3e} violations={int(bad.sum())}/{bad.size}")
    log(msg)
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{msg}; worst at {i}: got {got[i]} ref {ref[i]}")


def oracle_ref(wl, heads=None):
    """Oracle outputs and final states (optionally restricted to `heads`)."""
    slopes = oracle.alibi_slopes(wl.num_heads, wl.layer_id, wl.num_layers)
    if heads is None:
        q, k, v, pool = wl.q, wl.k, wl.v, wl.pool
    else:
        # each selected query head keeps its own kv head (one kv head per head)
        g = wl.num_heads // wl.num_kv_heads
        kvh = [h // g for h in heads]
        q, k, v = wl.q[:, heads], wl.k[:, kvh], wl.v[:, kvh]
        pool = wl.pool[:, heads]
        slopes = slopes[heads]
    return oracle.prefill(q, k, v, wl.cu_seqlens, pool, wl.slot_idx, slopes)


def check_against_oracle(wl, out, pool_after, state_out=None, heads=None):
    tol = TOL[wl.dtype]
    ref_out, ref_fin = oracle_ref(wl, heads)
    hsel = slice(None) if heads is None else heads
    got_out = host_io(out[:, hsel] if heads is not None else out)
    assert_close(got_out, ref_out, tol, f"{wl.name} out")
    idx = torch.from_numpy(wl.slot_idx.astype(np.int64)).cuda()
    if state_out is not None:
        fin = state_out
    else:
        fin = pool_after.index_select(0, idx)
    fin = fin[:, hsel] if heads is not None else fin
    assert_close(fin.cpu().numpy(), ref_fin, tol, f"{wl.name} final state")


def check_untouched(wl, pool_after, addressed=True):
    """Slots no request names (all slots, if not addressed) are bit-identical."""
    P = wl.pool_slots
    keep = np.ones(P, dtype=bool)
    if addressed:
        keep[wl.slot_idx] = False
    idx = np.nonzero(keep)[0]
    if idx.size == 0:
        return
    got = pool_after.index_select(0, torch.from_numpy(idx).cuda()).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), wl.pool[idx].view(np.uint32)), "untouched slot changed"
