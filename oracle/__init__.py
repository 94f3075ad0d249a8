"""fp64 CPU oracle for segmented linear attention (seg_la).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does.  It shares no code with the HIP library (``linear_attention_amd``) and
does not import it.

Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page] and its
sections by their headings.

The arithmetic lives in ``la_oracle.c`` (plain C, fp64, one token at a time).
This module only marshals arrays: it upcasts the inputs exactly to float64,
gathers the initial states from the pool by slot index and hands everything to
the C routine.  The pool semantics follow [LA-page] §独立参考实现 (the prefix
state is read from the request's slot and the final state written back) and
§额外覆盖 (slots no request names are never written).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblaoracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c with gcc into liblaoracle.so (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.la_oracle_alibi_slopes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.la_oracle_alibi_slopes.restype = ctypes.c_int
        I, P = ctypes.c_int, ctypes.c_void_p
        lib.la_oracle_run.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P, P, I]
        lib.la_oracle_run.restype = ctypes.c_int
        lib.la_oracle_tree.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I]
        lib.la_oracle_tree.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host cores this process may run on."""
    return len(os.sched_getaffinity(0))


def alibi_slopes(num_heads: int, layer_id: int = 0, num_layers: int = 1) -> np.ndarray:
    """fp32 per-head slopes: ALiBi geometric sequence times the layer factor
    ([LA-page] §独立参考实现, slope bullet)."""
    out = np.empty(num_heads, dtype=np.float32)
    rc = _load().la_oracle_alibi_slopes(int(num_heads), int(layer_id), int(num_layers),
                                        out.ctypes.data)
    if rc != 0:
        raise ValueError(f"invalid slope arguments H={num_heads} layer={layer_id}/{num_layers}")
    return out


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact upcast to float64.  uint16 arrays hold bfloat16 bit patterns: the
    16 bits are the top half of an IEEE float32."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64, copy=False)
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _qkv(q, k, v, H, d):
    """q as [N, H, d], k and v as [N, Hkv, d] float64 (Hkv divides H)."""
    qd = np.ascontiguousarray(to_f64(q)).reshape(-1, H, d)
    kd = np.ascontiguousarray(to_f64(k))
    if kd.ndim != 3:
        kd = kd.reshape(-1, H, d)
    vd = np.ascontiguousarray(to_f64(v)).reshape(kd.shape)
    hk = kd.shape[1]
    if hk <= 0 or H % hk:
        raise ValueError(f"kv heads {hk} must divide heads {H}")
    return qd, kd, vd, hk


def run(q, k, v, cu_seqlens, init_states, slopes, threads: int | None = None, track_lens=None):
    """The recurrence over a packed varlen batch with explicit initial states.

    q: [T, H, d]; k, v: [T, Hkv, d] with Hkv dividing H (query head h reads
    key/value head h // (H // Hkv)); float32, float64 or bf16 bits as uint16
    cu_seqlens: [B+1] non-decreasing, starting at 0
    init_states: [B, H, d, d] (any float dtype; upcast exactly)
    slopes: [H] (float32 values are upcast exactly)
    track_lens: optional [B]; request b's state after its first track_lens[b]
        tokens ([LA-page] §额外覆盖 state tracking), NaN where the length is
        outside [0, len]
    Returns (out [T, H, d], final_states [B, H, d, d]) as float64, plus
    track_states [B, H, d, d] when track_lens is given.
    """
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    B = cu.shape[0] - 1
    S0 = np.ascontiguousarray(to_f64(init_states))
    if S0.ndim != 4 or S0.shape[0] != B:
        raise ValueError("init_states must be [B, H, d, d]")
    H, d = S0.shape[1], S0.shape[2]
    qd, kd, vd, hk = _qkv(q, k, v, H, d)
    T = int(cu[-1]) if B > 0 else 0
    if not (qd.shape[0] == kd.shape[0] == vd.shape[0] == T):
        raise ValueError(f"q/k/v token count {qd.shape[0]} != cu_seqlens[-1] {T}")
    sl = np.ascontiguousarray(to_f64(np.asarray(slopes)))
    if sl.shape != (H,):
        raise ValueError("slopes must be [H]")
    out = np.zeros((T, H, d), dtype=np.float64)
    fin = np.zeros((B, H, d, d), dtype=np.float64)
    tl = snap = None
    if track_lens is not None:
        tl = np.ascontiguousarray(np.asarray(track_lens, dtype=np.int64))
        if tl.shape != (B,):
            raise ValueError("track_lens must be [B]")
        snap = np.full((B, H, d, d), np.nan)
    rc = _load().la_oracle_run(B, H, hk, d, _ptr(cu), _ptr(qd), _ptr(kd), _ptr(vd), _ptr(S0),
                               _ptr(sl), _ptr(tl), _ptr(out), _ptr(fin), _ptr(snap),
                               int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"la_oracle_run failed with code {rc}")
    return (out, fin) if track_lens is None else (out, fin, snap)


def tree(q, k, v, num_draft, parents, init_states, slopes, threads: int | None = None):
    """Tree verify with explicit initial states ([LA-page] §生产环境不支持 item 3
    and Next Work item 2: each draft forks from its parent's saved state).

    q: [B*n, H, d]; k, v: [B*n, Hkv, d]; parents: [B, n] int, parents[b][j] in
    [-1, j) (-1: the request's initial state); init_states: [B, H, d, d].
    Returns (out [B*n, H, d], states [B, n, H, d, d]) as float64: states[b][j]
    is the state after draft j.
    """
    S0 = np.ascontiguousarray(to_f64(init_states))
    if S0.ndim != 4:
        raise ValueError("init_states must be [B, H, d, d]")
    B, H, d = S0.shape[0], S0.shape[1], S0.shape[2]
    n = int(num_draft)
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    if par.shape != (B, n):
        raise ValueError("parents must be [B, num_draft]")
    qd, kd, vd, hk = _qkv(q, k, v, H, d)
    if not (qd.shape[0] == kd.shape[0] == vd.shape[0] == B * n):
        raise ValueError("q, k, v must hold num_draft tokens per request")
    sl = np.ascontiguousarray(to_f64(np.asarray(slopes)))
    if sl.shape != (H,):
        raise ValueError("slopes must be [H]")
    out = np.zeros((B * n, H, d))
    states = np.zeros((B, n, H, d, d))
    rc = _load().la_oracle_tree(B, n, H, hk, d, _ptr(qd), _ptr(kd), _ptr(vd), _ptr(S0), _ptr(sl),
                                _ptr(par), _ptr(out), _ptr(states), int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"la_oracle_tree failed with code {rc}")
    return out, states


def gather(pool: np.ndarray, slot_idx) -> np.ndarray:
    """Initial states of the requests: pool[slot_idx[b]] for every b, as float64."""
    idx = np.asarray(slot_idx, dtype=np.int64)
    P = pool.shape[0]
    if idx.size and (idx.min() < 0 or idx.max() >= P):
        raise ValueError("slot index out of range")
    if len(set(idx.tolist())) != idx.size:
        raise ValueError("slot indices must be distinct")
    return to_f64(pool[idx])


def scatter(pool: np.ndarray, slot_idx, final_states: np.ndarray, track_slots=None,
            track_states=None) -> np.ndarray:
    """Expected pool after a call: the input pool (float64 copy) with each
    addressed slot replaced by that request's final state and, for requests
    that took a snapshot, their track slot by the snapshot; other slots
    unchanged ([LA-page] §额外覆盖: active, track and untouched slots)."""
    exp = to_f64(pool).copy()
    exp[np.asarray(slot_idx, dtype=np.int64)] = final_states
    if track_slots is not None:
        for b, ts in enumerate(np.asarray(track_slots, dtype=np.int64)):
            if ts >= 0 and not np.isnan(track_states[b]).any():
                exp[ts] = track_states[b]
    return exp


def prefill(q, k, v, cu_seqlens, pool, slot_idx, slopes, threads=None, track_lens=None):
    """Packed varlen prefill: returns (out, final_states[, track_states]) for the
    requests; the pool itself is not modified ([LA-page] §独立参考实现)."""
    return run(q, k, v, cu_seqlens, gather(pool, slot_idx), slopes, threads, track_lens)


def decode(q, k, v, pool, slot_idx, slopes, threads=None):
    """One token per request: q is [B, H, d], k and v [B, Hkv, d]."""
    B = int(np.asarray(slot_idx).shape[0])
    return run(q, k, v, np.arange(B + 1, dtype=np.int64), gather(pool, slot_idx), slopes, threads)


def verify(q, k, v, num_draft, pool, slot_idx, slopes, threads=None):
    """Chain verify: request b owns draft tokens b*num_draft .. b*num_draft+num_draft-1
    and processes them as one chain ([LA-page] §生产环境不支持 item 3: chain only).
    Returns (out [B*k, H, d], final_states [B, H, d, d])."""
    B = int(np.asarray(slot_idx).shape[0])
    cu = np.arange(B + 1, dtype=np.int64) * int(num_draft)
    return run(q, k, v, cu, gather(pool, slot_idx), slopes, threads)


def tree_verify(q, k, v, num_draft, parents, pool, slot_idx, slopes, threads=None):
    """Tree verify from the pool: returns (out [B*n, H, d], states [B, n, H, d, d])."""
    return tree(q, k, v, num_draft, parents, gather(pool, slot_idx), slopes, threads)
