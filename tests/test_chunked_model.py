"""The chunked prefill's decomposition, modelled in fp64 (tests/chunked_model.py),
against the per-token oracle.

The GPU path re-associates the recurrence of [LA-page] §独立参考实现 over
chunks, in a scaled decay frame for slopes in [0, 2], and splits long
requests into segments and sub-segments combined afterwards.  Each of these
steps is exact algebra, so in fp64 the model must reproduce the oracle to
rounding: this checks the algebra on the CPU, apart from the kernel's bf16
operand rounding, which the GPU parity tests bound.  Chunk lengths 1, 7, 64
and 128, slopes on both sides of the frame's limit, lengths at chunk and
segment edges, and 200 drawn decompositions (hypothesis, derandomized).
([LA-page]: the page "SGLang Lightning Attention 能力矩阵与 seg_la
线性注意力测试覆盖深度解析", www.2kiu.com/news/4599301.)
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from chunked_model import frame_center, prefill, segment_geometry

SLOPES = [0.0, 1e-7, 0.9, 2.0, 2.0001, 8.0]


def _inputs(n, d, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    S0 = 0.05 * rng.standard_normal((d, d))
    return q, k, v, S0


def _oracle(q, k, v, S0, lam):
    n, d = q.shape
    out, fin = oracle.run(q[:, None], k[:, None], v[:, None], np.array([0, n]), S0[None, None],
                          np.array([lam], dtype=np.float32), threads=1)
    return out[:, 0], fin[0, 0]


def _close(got, ref, what):
    err = np.abs(got - ref).max() if got.size else 0.0
    assert err <= 1e-10 * max(1.0, np.abs(ref).max()), f"{what}: max abs err {err:.3e}"


@pytest.mark.parametrize("lam", SLOPES)
@pytest.mark.parametrize("C,lengths", [(1, [1, 2, 5]), (7, [1, 6, 7, 8, 15, 22]),
                                       (64, [1, 63, 64, 65, 127, 128, 129, 200]),
                                       (128, [1, 127, 128, 129, 300])])
def test_chunked_equals_recurrence(C, lengths, lam):
    lam32 = float(np.float32(lam))  # the kernel sees the fp32 slope
    for n in lengths:
        q, k, v, S0 = _inputs(n, 16, seed=n * 131 + C)
        got_o, got_s = prefill(q, k, v, S0, lam32, C=C)
        ref_o, ref_s = _oracle(q, k, v, S0, lam32)
        _close(got_o, ref_o, f"C={C} n={n} lam={lam} out")
        _close(got_s, ref_s, f"C={C} n={n} lam={lam} state")


@pytest.mark.parametrize("lam", [1e-7, 0.9, 2.0])
def test_both_decay_forms_agree_inside_the_frame_limit(lam):
    """Inside [0, 2] the scaled frame and the explicit weights are the same
    algebra; the kernel takes the frame there."""
    lam32 = float(np.float32(lam))
    q, k, v, S0 = _inputs(150, 16, seed=5)
    fo, fs = prefill(q, k, v, S0, lam32, factored=True)
    eo, es = prefill(q, k, v, S0, lam32, factored=False)
    _close(fo, eo, "frame vs explicit out")
    _close(fs, es, "frame vs explicit state")


@pytest.mark.parametrize("lam", [0.0, 1e-7, 0.9, 2.0001])
@pytest.mark.parametrize("n,segments,subsegs", [
    (64 * 24, 3, 1), (64 * 24 + 1, 3, 2), (64 * 24 - 1, 3, 4), (64 * 25, 8, 4), (64 * 9 + 17, 8, 3),
    (64 * 2, 8, 4), (65, 4, 2), (64 * 16 + 63, 5, 4)])
def test_segments_and_subsegments_equal_recurrence(n, segments, subsegs, lam):
    """Segments of whole chunks (the last one shorter, some possibly empty),
    each from the state the state-only pass and the combine step give it."""
    lam32 = float(np.float32(lam))
    q, k, v, S0 = _inputs(n, 16, seed=n + 7 * segments + subsegs)
    got_o, got_s = prefill(q, k, v, S0, lam32, C=64, segments=segments, subsegs=subsegs)
    ref_o, ref_s = _oracle(q, k, v, S0, lam32)
    _close(got_o, ref_o, f"n={n} S={segments} Q={subsegs} out")
    _close(got_s, ref_s, f"n={n} S={segments} Q={subsegs} state")


def test_segment_geometry_covers_every_chunk_once():
    for n in range(1, 64 * 40, 37):
        for S in range(1, 9):
            nchunks, cps, ne = segment_geometry(n, 64, S)
            assert 1 <= ne <= S and (ne - 1) * cps < nchunks <= ne * cps


def test_full_head_dim_case():
    q, k, v, S0 = _inputs(300, 128, seed=11)
    lam32 = float(np.float32(2.0 ** -8))
    got_o, got_s = prefill(q, k, v, S0, lam32, segments=3, subsegs=2)
    ref_o, ref_s = _oracle(q, k, v, S0, lam32)
    _close(got_o, ref_o, "d=128 out")
    _close(got_s, ref_s, "d=128 state")


def test_frame_factors_stay_in_float32_range_for_64_token_chunks():
    """The kernel keeps the frame's factors in fp32 and bf16 (same exponent
    range).  For C = 64 and slopes up to 2, the score weights e^{l(j-m)}, the
    output factors e^{-l(i-m)} and the frame factor e^{-l(m+1)} and its
    inverse all lie inside the normal range; the decayed-V weights
    e^{-l(c-1-j+m+1)} of the first keys may underflow to zero, but their weight
    relative to the largest one in the chunk is below 1e-10 (under fp32 rounding).  A
    128-token chunk at slope 2 would need e^{2*64}, past fp32's largest value."""
    f32 = np.finfo(np.float32)

    for C, ok in ((64, True), (128, False)):
        m = frame_center(C)
        fits = True
        for lam in np.linspace(0.0, 2.0, 41):
            j = np.arange(C)
            factors = np.concatenate([np.exp(lam * (j - m)), np.exp(-lam * (j - m)),
                                      [np.exp(-lam * (m + 1)), np.exp(lam * (m + 1))]])
            fits &= bool(np.all((factors > f32.tiny) & (factors < f32.max)))
            vw = np.exp(-lam * (C - 1 - j + m + 1))
            small = vw[~((vw > f32.tiny) & (vw < f32.max))]
            fits &= bool(small.size == 0 or small.max() / vw.max() < 1e-10)
        assert fits == ok, C


@settings(max_examples=200, deadline=None, derandomize=True)
@given(n=st.integers(1, 260), C=st.sampled_from([1, 3, 7, 16, 64, 100, 128]),
       lam=st.one_of(st.floats(0.0, 2.0), st.floats(2.0, 12.0)),
       segments=st.integers(1, 8), subsegs=st.integers(1, 4), d=st.sampled_from([4, 16]),
       seed=st.integers(0, 2**16))
def test_random_decompositions_equal_recurrence(n, C, lam, segments, subsegs, d, seed):
    """Drawn chunk lengths, slopes on both sides of the frame's limit, request
    lengths and segment/sub-segment splits: the decomposition equals the
    per-token recurrence in fp64.  (The scaled frame is only ever used with
    C = 64 by the kernel; at larger C and slopes its factors leave the fp64
    range too, so it is drawn only where they stay inside it.)"""
    lam32 = float(np.float32(lam))
    factored = 0.0 <= lam32 <= 2.0 and lam32 * C < 600
    q, k, v, S0 = _inputs(n, d, seed)
    got_o, got_s = prefill(q, k, v, S0, lam32, C=C, segments=segments, subsegs=subsegs, factored=factored)
    ref_o, ref_s = _oracle(q, k, v, S0, lam32)
    _close(got_o, ref_o, f"n={n} C={C} lam={lam32} S={segments} Q={subsegs} out")
    _close(got_s, ref_s, f"n={n} C={C} lam={lam32} S={segments} Q={subsegs} state")
