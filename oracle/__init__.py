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
        lib.la_oracle_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.la_oracle_run.restype = ctypes.c_int
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
        return x.astype(np.float64)
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def run(q, k, v, cu_seqlens, init_states, slopes, threads: int | None = None):
    """The recurrence over a packed varlen batch with explicit initial states.

    q, k, v: [T, H, d] (float32, float64 or bf16 bits as uint16)
    cu_seqlens: [B+1] non-decreasing, starting at 0
    init_states: [B, H, d, d] (any float dtype; upcast exactly)
    slopes: [H] (float32 values are upcast exactly)
    Returns (out [T, H, d] float64, final_states [B, H, d, d] float64).
    """
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    B = cu.shape[0] - 1
    S0 = np.ascontiguousarray(to_f64(init_states))
    if S0.ndim != 4 or S0.shape[0] != B:
        raise ValueError("init_states must be [B, H, d, d]")
    H, d = S0.shape[1], S0.shape[2]
    qd = np.ascontiguousarray(to_f64(q)).reshape(-1, H, d)
    kd = np.ascontiguousarray(to_f64(k)).reshape(-1, H, d)
    vd = np.ascontiguousarray(to_f64(v)).reshape(-1, H, d)
    T = int(cu[-1]) if B > 0 else 0
    if not (qd.shape[0] == kd.shape[0] == vd.shape[0] == T):
        raise ValueError(f"q/k/v token count {qd.shape[0]} != cu_seqlens[-1] {T}")
    sl = np.ascontiguousarray(to_f64(np.asarray(slopes)))
    if sl.shape != (H,):
        raise ValueError("slopes must be [H]")
    out = np.zeros((T, H, d), dtype=np.float64)
    fin = np.zeros((B, H, d, d), dtype=np.float64)
    rc = _load().la_oracle_run(B, H, d, cu.ctypes.data, qd.ctypes.data, kd.ctypes.data,
                               vd.ctypes.data, S0.ctypes.data, sl.ctypes.data,
                               out.ctypes.data, fin.ctypes.data,
                               int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"la_oracle_run failed with code {rc}")
    return out, fin


def gather(pool: np.ndarray, slot_idx) -> np.ndarray:
    """Initial states of the requests: pool[slot_idx[b]] for every b, as float64."""
    idx = np.asarray(slot_idx, dtype=np.int64)
    P = pool.shape[0]
    if idx.size and (idx.min() < 0 or idx.max() >= P):
        raise ValueError("slot index out of range")
    if len(set(idx.tolist())) != idx.size:
        raise ValueError("slot indices must be distinct")
    return to_f64(pool[idx])


def scatter(pool: np.ndarray, slot_idx, final_states: np.ndarray) -> np.ndarray:
    """Expected pool after a call: the input pool (float64 copy) with each
    addressed slot replaced by that request's final state; other slots unchanged."""
    exp = to_f64(pool).copy()
    exp[np.asarray(slot_idx, dtype=np.int64)] = final_states
    return exp


def prefill(q, k, v, cu_seqlens, pool, slot_idx, slopes, threads=None):
    """Packed varlen prefill: returns (out, final_states) for the requests; the
    pool itself is not modified ([LA-page] §独立参考实现)."""
    return run(q, k, v, cu_seqlens, gather(pool, slot_idx), slopes, threads)


def decode(q, k, v, pool, slot_idx, slopes, threads=None):
    """One token per request: q, k, v are [B, H, d]."""
    B = int(np.asarray(slot_idx).shape[0])
    return run(q, k, v, np.arange(B + 1, dtype=np.int64), gather(pool, slot_idx), slopes, threads)


def verify(q, k, v, num_draft, pool, slot_idx, slopes, threads=None):
    """Chain verify: request b owns draft tokens b*num_draft .. b*num_draft+num_draft-1
    and processes them as one chain ([LA-page] §生产环境不支持 item 3: chain only).
    Returns (out [B*k, H, d], final_states [B, H, d, d])."""
    B = int(np.asarray(slot_idx).shape[0])
    cu = np.arange(B + 1, dtype=np.int64) * int(num_draft)
    return run(q, k, v, cu, gather(pool, slot_idx), slopes, threads)
