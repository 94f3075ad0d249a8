"""fp64 numpy model of the decomposition the chunked bf16 prefill computes.

Test code: it restates, in float64 and with numpy matmuls, the algebra of the
HIP prefill path (chunks of C tokens, the scaled decay frame for slopes in
[0, 2], explicit weights otherwise, the split of a request into sequence
segments and sub-segments with a state-only pass and a combine step), so
that the CPU suite can check that algebra against the per-token oracle
without a GPU.  It shares no code with either.  Operand rounding to bf16
and the hi/lo splits are not modelled; they are what the GPU parity tests
bound.

The recurrence of [LA-page] §独立参考实现 (S <- e^{-l} S + k v^T,
o = q S / sqrt(d)) over a chunk of c tokens with prior state S, local
indices i, j:
    o_i    = scale [ sum_{j<=i} e^{-l(i-j)} (q_i . k_j) v_j + e^{-l(i+1)} q_i S ]
    S_next = e^{-l c} S + sum_j k_j (e^{-l(c-1-j)} v_j)^T
([LA-page] = the page "SGLang Lightning Attention 能力矩阵与 seg_la 线性注意力测试覆盖深度解析",
www.2kiu.com/news/4599301.)
"""
from __future__ import annotations

import numpy as np


def frame_center(C: int) -> int:
    """Token index m of a chunk around which the scaled frame is taken (31 for
    C = 64): weights become e^{l(j-m)} and e^{-l(i-m)}, the state S e^{-l(m+1)}."""
    return (C - 1) // 2


def chunk_pass(q, k, v, S, lam, C, scale, factored):
    """One request (one head) through the chunk loop from state S.
    q, k, v: [n, d] float64; S: [d, d].  Returns (out [n, d], final state)."""
    n, d = q.shape
    out = np.zeros((n, d))
    m = frame_center(C)
    S = S * np.exp(-lam * (m + 1)) if factored else S.copy()
    for c0 in range(0, n, C):
        c = min(C, n - c0)
        Q, K, V = q[c0:c0 + c], k[c0:c0 + c], v[c0:c0 + c]
        i = np.arange(c)[:, None]
        j = np.arange(c)[None, :]
        A = Q @ K.T
        if factored:
            P = np.where(j <= i, A * np.exp(lam * np.minimum(j, i) - lam * m), 0.0)
            O = (P @ V + Q @ S) * np.exp(-lam * (np.arange(c) - m))[:, None]
            Vd = V * np.exp(-lam * (c - 1 - np.arange(c) + (m + 1)))[:, None]
        else:
            P = np.where(j <= i, A * np.exp(-lam * np.maximum(i - j, 0)), 0.0)
            O = P @ V + (Q @ S) * np.exp(-lam * (np.arange(c) + 1))[:, None]
            Vd = V * np.exp(-lam * (c - 1 - np.arange(c)))[:, None]
        out[c0:c0 + c] = scale * O
        S = S + np.expm1(-lam * c) * S + K.T @ Vd
    if factored:
        S = S * np.exp(lam * (m + 1))
    return out, S


def segment_geometry(n, C, segments):
    """(chunks, chunks per segment, non-empty segments) of an n-token request."""
    nchunks = -(-n // C)
    cps = -(-nchunks // segments)
    ne = -(-nchunks // cps) if cps > 0 else 0
    return nchunks, cps, ne


def subsegment_range(cps, subsegs, qi):
    """Chunks [c0, c0 + count) of sub-segment qi of a segment of cps chunks."""
    spc = -(-cps // subsegs)
    c0 = qi * spc
    return c0, (0 if c0 >= cps else min(spc, cps - c0))


def delta_pass(k, v, lam, C):
    """State contribution of whole chunks from a zero state (the state-only
    pass): acc <- e^{-l C} acc + K^T (e^{-l(C-1-j)} v_j) per chunk."""
    d = k.shape[1]
    acc = np.zeros((d, d))
    w = np.exp(-lam * (C - 1 - np.arange(C)))[:, None]
    for c0 in range(0, k.shape[0], C):
        acc = acc + np.expm1(-lam * C) * acc + k[c0:c0 + C].T @ (v[c0:c0 + C] * w)
    return acc


def prefill(q, k, v, S_init, lam, C=64, segments=1, subsegs=1, factored=None):
    """One request and head: the chunked prefill, optionally split into
    `segments` sequence segments of whole chunks with `subsegs` state-only
    sub-segments each.  factored=None picks the frame as the kernel does
    (0 <= l <= 2)."""
    n, d = q.shape
    lam = float(lam)
    if factored is None:
        factored = 0.0 <= lam <= 2.0
    scale = d ** -0.5
    if n == 0:
        return np.zeros((0, d)), S_init.copy()
    if segments <= 1:
        return chunk_pass(q, k, v, S_init, lam, C, scale, factored)
    nchunks, cps, ne = segment_geometry(n, C, segments)
    # 1. state-only pass over the sub-segments of every non-final segment
    deltas = {}
    for s in range(ne - 1):
        for qi in range(subsegs):
            c0, cnt = subsegment_range(cps, subsegs, qi)
            if cnt:
                t0 = (s * cps + c0) * C
                deltas[s, qi] = (cnt, delta_pass(k[t0:t0 + cnt * C], v[t0:t0 + cnt * C], lam, C))
    # 2. combine: initial state of every segment
    starts = [S_init.copy()]
    for s in range(ne - 1):
        S = starts[-1].copy()
        for qi in range(subsegs):
            if (s, qi) in deltas:
                cnt, dS = deltas[s, qi]
                S = S + np.expm1(-lam * cnt * C) * S + dS
        starts.append(S)
    # 3. every segment from its own initial state
    out = np.zeros((n, d))
    fin = None
    for s in range(ne):
        t0, t1 = s * cps * C, min(n, (s + 1) * cps * C)
        out[t0:t1], fin = chunk_pass(q[t0:t1], k[t0:t1], v[t0:t1], starts[s], lam, C, scale, factored)
    return out, fin
