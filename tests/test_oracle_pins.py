"""Pins that tie the fp64 oracle to the mathematics, not to itself.

Each test checks the oracle against something fixed independently of its code:
a closed form summed directly, a library routine the slope-0 case reduces to,
hand-derived values, invariants of the recurrence, and published ALiBi slopes.
Citations name the page "SGLang Lightning Attention 能力矩阵与 seg_la
线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def closed_form(q, k, v, S0, lam):
    """Unrolled recurrence, summed directly for every t ([LA-page] §独立参考实现):
    S_t = e^{-lam(t+1)} S0 + sum_{s<=t} e^{-lam(t-s)} k_s v_s^T,  o_t = d^-1/2 q_t S_t."""
    T, d = q.shape
    out = np.zeros((T, d))
    S = S0
    for t in range(T):
        w = np.exp(-lam * (t - np.arange(t + 1)))
        S = math.exp(-lam * (t + 1)) * S0 + np.einsum("s,si,sj->ij", w, k[: t + 1], v[: t + 1])
        out[t] = (q[t] @ S) / math.sqrt(d)
    return out, S


@pytest.mark.parametrize("d,T", [(4, 48), (16, 33), (128, 20)])
def test_closed_form_bruteforce(d, T):
    rng = np.random.default_rng(100 + d)
    H = 3
    lams = np.array([0.917, 0.05, 0.0039])
    lens = [T, 1, T // 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (_rand(rng, cu[-1], H, d) for _ in range(3))
    S0 = 0.05 * _rand(rng, len(lens), H, d, d)
    out, fin = oracle.run(q, k, v, cu, S0, lams, threads=3)
    for b in range(len(lens)):
        sl = slice(cu[b], cu[b + 1])
        for h in range(H):
            o_ref, s_ref = closed_form(q[sl, h], k[sl, h], v[sl, h], S0[b, h], lams[h])
            np.testing.assert_allclose(out[sl, h], o_ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(fin[b, h], s_ref, rtol=1e-12, atol=1e-12)


def test_slope_zero_is_cumulative_sum():
    """slope 0: O = d^-1/2 (tril(Q K^T) V + Q S0), S_final = S0 + K^T V (numpy matmul)."""
    rng = np.random.default_rng(7)
    T, H, d = 37, 2, 16
    q, k, v = (_rand(rng, T, H, d) for _ in range(3))
    S0 = _rand(rng, 1, H, d, d)
    out, fin = oracle.run(q, k, v, [0, T], S0, np.zeros(H), threads=2)
    for h in range(H):
        Q, K, V = q[:, h], k[:, h], v[:, h]
        o_ref = (np.tril(Q @ K.T) @ V + Q @ S0[0, h]) / math.sqrt(d)
        np.testing.assert_allclose(out[:, h], o_ref, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(fin[0, h], S0[0, h] + K.T @ V, rtol=1e-12, atol=1e-12)


def test_worked_example_hand_derived():
    with open(os.path.join(GOLDEN, "worked_example_d2.json")) as f:
        g = json.load(f)
    d = g["head_dim"]
    lam = g["slope"]
    reqs = g["requests"]
    lens = [len(r["q"]) for r in reqs]
    cu = np.concatenate([[0], np.cumsum(lens)])
    cat = lambda key: np.array([row for r in reqs for row in r[key]], dtype=np.float64)[:, None, :]
    S0 = np.array([r["init_state"] for r in reqs], dtype=np.float64)[:, None]
    out, fin = oracle.run(cat("q"), cat("k"), cat("v"), cu, S0, np.array([lam]), threads=1)
    scale = d ** -0.5
    for b, r in enumerate(reqs):
        np.testing.assert_allclose(out[cu[b]:cu[b + 1], 0], scale * np.array(r["out_over_scale"]),
                                   rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(fin[b, 0], np.array(r["final_state"]), rtol=1e-14, atol=1e-15)


def test_orientation_basis_vectors():
    """k = e_a, v = e_b: S = e_a e_b^T, so q = e_a gives o = scale e_b and q = e_b (b != a) gives 0."""
    d, a, b = 8, 2, 5
    e = np.eye(d)
    q = np.stack([e[a], e[b]])[:, None]
    # two single-token requests, both with k = e_a, v = e_b, one queried with e_a, one with e_b
    k = np.stack([e[a], e[a]])[:, None]
    v = np.stack([e[b], e[b]])[:, None]
    out, fin = oracle.run(q, k, v, [0, 1, 2], np.zeros((2, 1, d, d)), np.array([0.3]), threads=1)
    np.testing.assert_array_equal(out[0, 0], e[b] / math.sqrt(d))
    np.testing.assert_array_equal(out[1, 0], np.zeros(d))
    assert fin[0, 0, a, b] == 1.0 and np.count_nonzero(fin[0, 0]) == 1


def test_large_slope_forgets_history():
    """slope 60: e^-60 ~ 9e-27, so o_t = scale (q_t . k_t) v_t and S_final = k_last v_last^T."""
    rng = np.random.default_rng(3)
    T, d = 9, 16
    q, k, v = (_rand(rng, T, 1, d) for _ in range(3))
    out, fin = oracle.run(q, k, v, [0, T], _rand(rng, 1, 1, d, d), np.array([60.0]), threads=1)
    ref = (np.sum(q[:, 0] * k[:, 0], axis=1)[:, None] * v[:, 0]) / math.sqrt(d)
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-12, atol=1e-20)
    np.testing.assert_allclose(fin[0, 0], np.outer(k[-1, 0], v[-1, 0]), rtol=1e-12, atol=1e-20)


@pytest.mark.parametrize("m", [0, 1, 5, 12, 13])
def test_split_invariance(m):
    """prefill(n) == prefill(m) followed by n-m single-token decode steps."""
    rng = np.random.default_rng(11)
    n, H, d, P = 13, 2, 16, 3
    q, k, v = (_rand(rng, n, H, d) for _ in range(3))
    pool = (0.05 * rng.standard_normal((P, H, d, d))).astype(np.float32)
    slopes = np.array([0.7, 0.01], dtype=np.float32)
    slot = [2]
    out_full, fin_full = oracle.prefill(q, k, v, [0, n], pool, slot, slopes, threads=2)
    out_a, fin_a = oracle.prefill(q[:m], k[:m], v[:m], [0, m], pool, slot, slopes, threads=2)
    outs = [out_a]
    S = fin_a
    for t in range(m, n):
        o, S = oracle.run(q[t:t + 1], k[t:t + 1], v[t:t + 1], [0, 1], S, slopes, threads=2)
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs), out_full, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S, fin_full, rtol=1e-13, atol=1e-15)


def test_verify_equals_prefill_of_chains():
    rng = np.random.default_rng(12)
    B, kd, H, d, P = 3, 4, 2, 8, 5
    q, k, v = (_rand(rng, B * kd, H, d) for _ in range(3))
    pool = (0.05 * rng.standard_normal((P, H, d, d))).astype(np.float32)
    slopes = np.array([0.2, 0.02], dtype=np.float32)
    slot = [4, 0, 2]
    o1, f1 = oracle.verify(q, k, v, kd, pool, slot, slopes)
    o2, f2 = oracle.prefill(q, k, v, np.arange(B + 1) * kd, pool, slot, slopes)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_linearity_in_values_and_state():
    """o and S_final are jointly linear in (V, S0); scaling q scales o only."""
    rng = np.random.default_rng(5)
    T, H, d = 15, 2, 8
    q, k = _rand(rng, T, H, d), _rand(rng, T, H, d)
    v1, v2 = _rand(rng, T, H, d), _rand(rng, T, H, d)
    s1, s2 = _rand(rng, 1, H, d, d), _rand(rng, 1, H, d, d)
    lam = np.array([0.3, 0.001])
    a, b = 1.75, -0.5
    o1, f1 = oracle.run(q, k, v1, [0, T], s1, lam, threads=1)
    o2, f2 = oracle.run(q, k, v2, [0, T], s2, lam, threads=1)
    o3, f3 = oracle.run(q, k, a * v1 + b * v2, [0, T], a * s1 + b * s2, lam, threads=1)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=1e-12, atol=1e-12)
    o4, f4 = oracle.run(3.0 * q, k, v1, [0, T], s1, lam, threads=1)
    np.testing.assert_allclose(o4, 3.0 * o1, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(f4, f1)


def test_request_order_and_slot_permutation():
    """Each request's result depends only on its own tokens and slot: reordering
    the batch and permuting the slots gives the same per-request results, and each
    request alone equals its part of the batch."""
    rng = np.random.default_rng(21)
    H, d, P = 2, 8, 6
    lens = [5, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (_rand(rng, cu[-1], H, d) for _ in range(3))
    pool = (0.05 * rng.standard_normal((P, H, d, d))).astype(np.float32)
    slopes = np.array([0.5, 0.05], dtype=np.float32)
    slot = [3, 0, 5, 1]
    out, fin = oracle.prefill(q, k, v, cu, pool, slot, slopes)
    order = [2, 0, 3, 1]
    perm_pool = pool[::-1].copy()          # slot s moves to P-1-s
    perm_slot = [P - 1 - slot[b] for b in order]
    segs = [np.arange(cu[b], cu[b + 1]) for b in order]
    idx = np.concatenate(segs).astype(np.int64)
    cu2 = np.concatenate([[0], np.cumsum([lens[b] for b in order])])
    out2, fin2 = oracle.prefill(q[idx], k[idx], v[idx], cu2, perm_pool, perm_slot, slopes)
    np.testing.assert_array_equal(out2, out[idx])
    np.testing.assert_array_equal(fin2, fin[order])
    for b in range(len(lens)):
        sl = slice(cu[b], cu[b + 1])
        ob, fb = oracle.prefill(q[sl], k[sl], v[sl], [0, lens[b]], pool, [slot[b]], slopes)
        np.testing.assert_array_equal(ob, out[sl])
        np.testing.assert_array_equal(fb[0], fin[b])


def test_zero_length_request_is_noop_and_sentinels_kept():
    H, d, P = 1, 4, 3
    pool = np.full((P, H, d, d), 54321.0, dtype=np.float32)
    pool[1] = 0.25
    out, fin = oracle.prefill(np.zeros((0, H, d)), np.zeros((0, H, d)), np.zeros((0, H, d)),
                              [0, 0], pool, [1], np.array([0.1], dtype=np.float32))
    assert out.shape == (0, H, d)
    np.testing.assert_array_equal(fin[0], pool[1])
    exp = oracle.scatter(pool, [1], fin)
    np.testing.assert_array_equal(exp[[0, 2]], pool[[0, 2]].astype(np.float64))


def test_oracle_rejects_bad_slots():
    pool = np.zeros((2, 1, 4, 4), dtype=np.float32)
    z = np.zeros((2, 1, 4))
    with pytest.raises(ValueError):
        oracle.prefill(z, z, z, [0, 1, 2], pool, [0, 0], np.array([0.1], dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.prefill(z, z, z, [0, 2], pool, [2], np.array([0.1], dtype=np.float32))


def _factor(expr):
    """Layer factor from the fixture's text, written as on the page: "1 + 1e-5" or "1 - a/b + 1e-5"."""
    if expr == "1 + 1e-5":
        return 1.0 + 1e-5
    num, den = (float(x) for x in expr.split(" ")[2].split("/"))
    return 1.0 - num / den + 1e-5


def test_alibi_slopes_published_values():
    with open(os.path.join(GOLDEN, "alibi_slopes.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        H = case["num_heads"]
        base = np.array([2.0 ** e for e in case["log2_base"]])
        for lf in g["layer_factors"]:
            got = oracle.alibi_slopes(H, lf["layer_id"], lf["num_layers"])
            want = (base * _factor(lf["factor"])).astype(np.float32)
            np.testing.assert_array_equal(got, want, err_msg=f"H={H} {lf}")


@pytest.mark.parametrize("H", [1, 2, 4, 16, 32, 64, 128])
def test_alibi_power_of_two_ratio(H):
    """Power-of-two head counts: a geometric sequence starting at 2^(-8/H) with that ratio."""
    s = oracle.alibi_slopes(H, 0, 1).astype(np.float64) / (1 + 1e-5)
    r = 2.0 ** (-8.0 / H)
    np.testing.assert_allclose(s[0], r, rtol=1e-7)
    if H > 1:
        np.testing.assert_allclose(s[1:] / s[:-1], r, rtol=2e-7)
    np.testing.assert_allclose(s[-1], 2.0 ** -8, rtol=1e-7)


def test_bf16_upcast_matches_torch_on_every_bit_pattern():
    """oracle.to_f64 reads uint16 arrays as bfloat16 bit patterns.  Every one of
    the 65536 patterns (both zeros, subnormals, the largest finite values,
    infinities, NaNs, and the patterns on either side of every rounding tie)
    must upcast to exactly what torch's own bfloat16 -> float64 conversion
    gives; a shifted, sign-dropping or truncating upcast fails here."""
    import torch

    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # -0.0 stays -0.0
    # spot values fixed by the format: sign bit, exponent bias 127, 7 mantissa bits
    assert got[0x3F80] == 1.0 and got[0xBF80] == -1.0 and got[0x4000] == 2.0
    assert got[0x0001] == 2.0 ** -133                    # smallest subnormal
    assert got[0x7F7F] == (2 - 2 ** -7) * 2.0 ** 127     # largest finite
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf
    # float32 and float64 inputs pass through unchanged
    x = np.array([1.5, -0.0, 3e-39, np.float32(1e38)], dtype=np.float32)
    assert np.array_equal(oracle.to_f64(x).view(np.uint64), x.astype(np.float64).view(np.uint64))
