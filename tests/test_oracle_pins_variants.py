"""Pins for the oracle's grouped-head mapping, state-tracking snapshot and tree
verify, each against a closed form summed directly in numpy.

Citations name the page "SGLang Lightning Attention 能力矩阵与 seg_la
线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
"""
import math

import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def state_after(k, v, S0, lam, n):
    """State once n tokens are absorbed: e^{-lam n} S0 + sum_{s<n} e^{-lam(n-1-s)} k_s v_s^T."""
    w = np.exp(-lam * (n - 1 - np.arange(n)))
    return math.exp(-lam * n) * S0 + np.einsum("s,si,sj->ij", w, k[:n], v[:n])


@pytest.mark.parametrize("H,HK", [(4, 2), (6, 3), (4, 1), (3, 3)])
def test_grouped_heads_closed_form(H, HK):
    """Query head h uses key/value head h // (H // HK); every kv head holds
    different values, so a wrong mapping changes the result."""
    rng = np.random.default_rng(40 + H + HK)
    d, lens = 8, [6, 11]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _rand(rng, cu[-1], H, d)
    k, v = _rand(rng, cu[-1], HK, d), _rand(rng, cu[-1], HK, d)
    S0 = 0.1 * _rand(rng, 2, H, d, d)
    lam = np.linspace(0.6, 0.01, H)
    out, fin = oracle.run(q, k, v, cu, S0, lam, threads=2)
    G = H // HK
    for b in range(2):
        sl = slice(cu[b], cu[b + 1])
        for h in range(H):
            kh, vh = k[sl, h // G], v[sl, h // G]
            for t in range(lens[b]):
                S = state_after(kh, vh, S0[b, h], lam[h], t + 1)
                np.testing.assert_allclose(out[cu[b] + t, h], q[cu[b] + t, h] @ S / math.sqrt(d),
                                           rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(fin[b, h], S, rtol=1e-11, atol=1e-12)


def test_grouped_heads_rejects_non_divisor():
    z = np.zeros((2, 3, 4))
    with pytest.raises(ValueError):
        oracle.run(np.zeros((2, 4, 4)), z, z, [0, 2], np.zeros((1, 4, 4, 4)), np.ones(4))


def test_track_snapshot_closed_form():
    """[LA-page] §额外覆盖: the snapshot is the state once track_len tokens are
    absorbed; 0 gives the prefix state, len the final state, anything outside
    [0, len] no snapshot."""
    rng = np.random.default_rng(50)
    H, d = 2, 8
    lens = [9, 9, 9, 9, 9, 0, 4]
    tls = [0, 1, 5, 8, 9, 0, 7]   # last: beyond the request, no snapshot
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (_rand(rng, cu[-1], H, d) for _ in range(3))
    S0 = 0.1 * _rand(rng, len(lens), H, d, d)
    lam = np.array([0.45, 0.02])
    out, fin, snap = oracle.run(q, k, v, cu, S0, lam, threads=2, track_lens=tls)
    out2, fin2 = oracle.run(q, k, v, cu, S0, lam, threads=2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(fin, fin2)
    for b, (n, tl) in enumerate(zip(lens, tls)):
        sl = slice(cu[b], cu[b + 1])
        if tl > n:
            assert np.isnan(snap[b]).all()
            continue
        for h in range(H):
            ref = state_after(k[sl, h], v[sl, h], S0[b, h], lam[h], tl)
            np.testing.assert_allclose(snap[b, h], ref, rtol=1e-11, atol=1e-12)
        if tl == 0:
            np.testing.assert_array_equal(snap[b], S0[b])
        if tl == n:
            np.testing.assert_array_equal(snap[b], fin[b])


def test_track_scatter_slot_rules():
    """Active slots get the final state, track slots the snapshot, every other
    slot keeps its value ([LA-page] §额外覆盖: active / track / untouched)."""
    rng = np.random.default_rng(51)
    H, d, P = 1, 4, 6
    pool = np.full((P, H, d, d), 54321.0, dtype=np.float32)
    pool[4] = 0.25
    q, k, v = (_rand(rng, 5, H, d) for _ in range(3))
    out, fin, snap = oracle.prefill(q, k, v, [0, 5], pool, [4], np.array([0.3], np.float32),
                                    track_lens=[2])
    exp = oracle.scatter(pool, [4], fin, track_slots=[1], track_states=snap)
    np.testing.assert_array_equal(exp[4], fin[0])
    np.testing.assert_array_equal(exp[1], snap[0])
    for s in (0, 2, 3, 5):
        np.testing.assert_array_equal(exp[s], pool[s].astype(np.float64))


def _depths_and_paths(parents):
    n = len(parents)
    depth, path = [0] * n, [None] * n
    for j in range(n):
        p = parents[j]
        depth[j] = 1 if p < 0 else depth[p] + 1
        path[j] = ([] if p < 0 else path[p]) + [j]
    return depth, path


TREES = {
    "chain": [-1, 0, 1, 2, 3],
    "star": [-1, -1, -1, -1],
    "binary": [-1, 0, 0, 1, 1, 2, 2],
    "two_roots": [-1, 0, -1, 2, 1, 3, 0],
    "single": [-1],
}


@pytest.mark.parametrize("name", sorted(TREES))
def test_tree_path_closed_form(name):
    """[LA-page] Next Work item 2: draft j forks from its parent's state, so along
    its root path a_1..a_m = j: S_j = e^{-lam m} S0 + sum_i e^{-lam(m-i)} k_{a_i} v_{a_i}^T."""
    par = TREES[name]
    n = len(par)
    B, H, HK, d = 2, 4, 2, 8
    rng = np.random.default_rng(60 + n)
    q = _rand(rng, B * n, H, d)
    k, v = _rand(rng, B * n, HK, d), _rand(rng, B * n, HK, d)
    S0 = 0.1 * _rand(rng, B, H, d, d)
    lam = np.array([0.8, 0.2, 0.05, 0.001])
    parents = np.array([par, par], dtype=np.int32)
    out, states = oracle.tree(q, k, v, n, parents, S0, lam, threads=2)
    depth, path = _depths_and_paths(par)
    for b in range(B):
        for h in range(H):
            hk = h // (H // HK)
            for j in range(n):
                m = depth[j]
                S = math.exp(-lam[h] * m) * S0[b, h]
                for i, a in enumerate(path[j], start=1):
                    S = S + math.exp(-lam[h] * (m - i)) * np.outer(k[b * n + a, hk], v[b * n + a, hk])
                np.testing.assert_allclose(states[b, j, h], S, rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(out[b * n + j, h], q[b * n + j, h] @ S / math.sqrt(d),
                                           rtol=1e-11, atol=1e-12)


def test_tree_rejects_bad_parents():
    z = np.zeros((3, 1, 4))
    S0 = np.zeros((1, 1, 4, 4))
    for bad in ([-1, 1, 0], [-2, 0, 1], [0, 0, 1], [-1, 0, 3]):
        with pytest.raises(ValueError):
            oracle.tree(z, z, z, 3, [bad], S0, np.ones(1))


def test_tree_verify_from_pool_chain_and_star():
    """Chain parents reproduce chain verify at every position (each prefix's
    final state); star parents are independent single decode steps."""
    rng = np.random.default_rng(70)
    B, n, H, d, P = 3, 4, 2, 8, 5
    q, k, v = (_rand(rng, B * n, H, d) for _ in range(3))
    pool = (0.05 * rng.standard_normal((P, H, d, d))).astype(np.float32)
    slopes = np.array([0.3, 0.01], dtype=np.float32)
    slot = [2, 4, 0]
    chain = np.tile(np.arange(-1, n - 1, dtype=np.int32), (B, 1))
    o, st = oracle.tree_verify(q, k, v, n, chain, pool, slot, slopes)
    o2, _ = oracle.verify(q, k, v, n, pool, slot, slopes)
    np.testing.assert_array_equal(o, o2)
    for j in range(n):
        idx = np.concatenate([np.arange(b * n, b * n + j + 1) for b in range(B)])
        _, fj = oracle.prefill(q[idx], k[idx], v[idx], np.arange(B + 1) * (j + 1), pool, slot, slopes)
        np.testing.assert_array_equal(st[:, j], fj)
    star = np.full((B, n), -1, dtype=np.int32)
    o3, st3 = oracle.tree_verify(q, k, v, n, star, pool, slot, slopes)
    for j in range(n):
        idx = np.arange(B) * n + j
        od, fd = oracle.decode(q[idx], k[idx], v[idx], pool, slot, slopes)
        np.testing.assert_array_equal(o3[idx], od)
        np.testing.assert_array_equal(st3[:, j], fd)
