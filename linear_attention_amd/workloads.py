"""Seeded synthetic inputs for segmented linear attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no slopes, no decay, no recurrence).  Both the HIP path
(through the tests and the benchmark) and the fp64 oracle consume what it
produces.

Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].

Recipe (shared by every workload):
  * q, k, v ~ N(0, 1) drawn in float32; for bf16 workloads rounded to bfloat16
    with round-to-nearest-even and stored as uint16 bit patterns, so both sides
    consume identical values.
  * Layout [T, H, d], token-major, heads interleaved (row stride H*d), the
    packed varlen ("extend") layout of [LA-page] §输入与配置覆盖.
  * Prefix states are 0.05 * N(0, 1) float32, the scale [LA-page]
    §独立参考实现 gives for injected prefix states; requests without a prefix
    start from a zero state.
  * Pool slots that no request names hold the sentinel 54321.0, the value the
    state-tracking test of [LA-page] §额外覆盖 checks for untouched slots.
  * Slot indices are a seeded permutation, so slot order is non-monotonic in
    request order ([LA-page] §输入与配置覆盖, layout-robustness cases).
Every tensor is drawn from counter-keyed streams (numpy PCG64 seeded with
SeedSequence([seed, tag, index]), one per block of 256 tokens or per pool
slot), so blocks are generated in parallel and any block can be regenerated
alone.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SENTINEL = np.float32(54321.0)
PREFIX_SCALE = np.float32(0.05)

_TAG_META, _TAG_Q, _TAG_K, _TAG_V, _TAG_STATE = 0, 1, 2, 3, 4


def _stream(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), tag, int(index)])))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.
    Inputs here are finite normals, so no NaN/Inf handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


TOKEN_BLOCK = 256


def normal_tokens(seed: int, tag: int, T: int, H: int, d: int, dtype: str) -> np.ndarray:
    """[T, H, d] N(0,1) values; tokens [256n, 256n+256) are drawn from stream
    (seed, tag, n) in row-major order."""
    out = np.empty((T, H, d), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(n):
        t0, t1 = n * TOKEN_BLOCK, min(T, (n + 1) * TOKEN_BLOCK)
        x = _stream(seed, tag, n).standard_normal((t1 - t0, H, d), dtype=np.float32)
        out[t0:t1] = bf16_round_bits(x) if dtype == "bf16" else x

    nblocks = (T + TOKEN_BLOCK - 1) // TOKEN_BLOCK
    if nblocks:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(nblocks)))
    return out


@dataclass
class Workload:
    """One batch of synthetic input.

    kind: "prefill" (packed varlen), "decode" (one token per request) or
    "verify" (num_draft chained tokens per request).
    q: [T, H, d]; k, v: [T, Hkv, d] (uint16 bf16 bits, or float32), T = cu_seqlens[-1].
    pool: [P, H, d, d] float32; slot_idx: [B] int32; cu_seqlens: [B+1] int32.
    """
    name: str
    kind: str
    dtype: str
    num_heads: int
    head_dim: int
    layer_id: int
    num_layers: int
    seed: int
    lengths: np.ndarray
    cu_seqlens: np.ndarray
    slot_idx: np.ndarray
    pool: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    num_draft: int = 1
    prefix_mask: np.ndarray = field(default=None)
    num_kv_heads: int = 0  # 0: same as num_heads

    def __post_init__(self):
        if not self.num_kv_heads:
            self.num_kv_heads = self.num_heads

    @property
    def batch(self) -> int:
        return int(self.slot_idx.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if self.lengths.size else 0

    @property
    def pool_slots(self) -> int:
        return int(self.pool.shape[0])


def _pool(seed, P, H, d, fill_slots, zero_slots):
    """float32 pool; `fill_slots` get 0.05*N(0,1) from stream (seed, STATE, slot),
    `zero_slots` get zeros, every other slot the sentinel."""
    pool = np.empty((P, H, d, d), dtype=np.float32)
    fill = set(int(s) for s in fill_slots)
    zero = set(int(s) for s in zero_slots)

    def one(s):
        if s in fill:
            x = _stream(seed, _TAG_STATE, s).standard_normal((H, d, d), dtype=np.float32)
            pool[s] = x * PREFIX_SCALE
        elif s in zero:
            pool[s] = 0.0
        else:
            pool[s] = SENTINEL

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(P)))
    return pool


def make(name, kind, dtype, num_heads, lengths, pool_slots, *, head_dim=128, seed=0,
         layer_id=0, num_layers=1, prefix=None, slot_idx=None, fill_all_slots=False,
         num_draft=1, num_kv_heads=None):
    """General workload builder.

    num_kv_heads: heads of k and v (grouped heads; default num_heads).

    lengths: per-request token counts (for "verify" every entry is num_draft).
    prefix: bool per request (True -> 0.05*N prefix state), default all False.
    slot_idx: explicit slots, else the first B entries of a seeded permutation.
    fill_all_slots: every pool slot gets a random prefix state (no sentinels).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    B = int(lengths.shape[0])
    meta = _stream(seed, _TAG_META, 1)
    if slot_idx is None:
        if B > pool_slots:
            raise ValueError("more requests than pool slots")
        slot_idx = meta.permutation(pool_slots)[:B]
    slot_idx = np.asarray(slot_idx, dtype=np.int32)
    prefix = np.zeros(B, dtype=bool) if prefix is None else np.asarray(prefix, dtype=bool)
    if fill_all_slots:
        fill, zero = range(pool_slots), []
    else:
        fill = [int(s) for s, p in zip(slot_idx, prefix) if p]
        zero = [int(s) for s, p in zip(slot_idx, prefix) if not p]
    cu = np.zeros(B + 1, dtype=np.int32)
    np.cumsum(lengths, out=cu[1:])
    T = int(cu[-1])
    hk = num_kv_heads or num_heads
    q = normal_tokens(seed, _TAG_Q, T, num_heads, head_dim, dtype)
    k = normal_tokens(seed, _TAG_K, T, hk, head_dim, dtype)
    v = normal_tokens(seed, _TAG_V, T, hk, head_dim, dtype)
    pool = _pool(seed, pool_slots, num_heads, head_dim, fill, zero)
    return Workload(name=name, kind=kind, dtype=dtype, num_heads=num_heads, head_dim=head_dim,
                    layer_id=layer_id, num_layers=num_layers, seed=seed, lengths=lengths,
                    cu_seqlens=cu, slot_idx=slot_idx, pool=pool, q=q, k=k, v=v,
                    num_draft=num_draft, prefix_mask=prefix, num_kv_heads=hk)


CONFIG_NAMES = {
    1: "tiny-ref fp32 H=2 d=128 lengths (17,40)",
    2: "varlen-prefill bf16 H=16 d=128 8 requests U[1,4096]",
    3: "decode bf16 B=256 H=64 d=128 pool 512",
    4: "long-prefill bf16 T=131072 H=64 d=128",
    5: "chain-verify bf16 B=128 k=5 H=64 d=128 pool 256",
}


def config(n: int, seed: int | None = None) -> Workload:
    """The five synthetic configurations (seed defaults to the config number)."""
    s = n if seed is None else seed
    name = CONFIG_NAMES[n]
    if n == 1:
        # request 1 (second) carries a prefix in slot 3; request 0 starts from a
        # zero state in slot 1; slots 0 and 2 hold the sentinel
        return make(name, "prefill", "fp32", 2, [17, 40], 4, seed=s, layer_id=0, num_layers=1,
                    prefix=[False, True], slot_idx=[1, 3])
    if n == 2:
        meta = _stream(s, _TAG_META, 0)
        lengths = meta.integers(1, 4097, size=8)
        prefix = np.zeros(8, dtype=bool)
        prefix[meta.permutation(8)[:4]] = True
        return make(name, "prefill", "bf16", 16, lengths, 64, seed=s, layer_id=1, num_layers=4,
                    prefix=prefix)
    if n == 3:
        return make(name, "decode", "bf16", 64, np.ones(256, dtype=np.int64), 512, seed=s,
                    fill_all_slots=True)
    if n == 4:
        return make(name, "prefill", "bf16", 64, [131072], 2, seed=s, prefix=[False],
                    slot_idx=[0])
    if n == 5:
        return make(name, "verify", "bf16", 64, np.full(128, 5, dtype=np.int64), 256, seed=s,
                    prefix=np.ones(128, dtype=bool), num_draft=5)
    raise ValueError(f"unknown config {n}")
