"""Planted-mistake check of the oracle's pins (CPU only).

Each mutant copies oracle/la_oracle.c to a temporary directory, plants one
plausible mistake (a dropped term, a wrong sign or index, a transposed
operand, a wrong layer factor), builds it with gcc, and runs the independent
checks below against it: closed form, slope-0 cumulative sum, the hand-derived
worked example, and the ALiBi fixture.  Every mutant must fail at least one.
The unmodified source must pass them all, so the checks are not vacuous.
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "la_oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden")

MUTANTS = {
    "add_before_decay": ("S[(size_t)i * d + j] * decay + kt[i] * vt[j]",
                         "(S[(size_t)i * d + j] + kt[i] * vt[j]) * decay"),
    "transposed_outer": ("* decay + kt[i] * vt[j]", "* decay + kt[j] * vt[i]"),
    "output_contracts_columns": ("acc += qt[i] * S[(size_t)i * d + j];",
                                 "acc += qt[i] * S[(size_t)j * d + i];"),
    "missing_scale": ("ot[j] = acc * scale;", "ot[j] = acc;"),
    "scale_not_sqrt": ("1.0 / sqrt((double)d)", "1.0 / (double)d"),
    "decay_sign": ("exp(-jb->slopes[h])", "exp(jb->slopes[h])"),
    "decay_twice": ("exp(-jb->slopes[h])", "exp(-2.0 * jb->slopes[h])"),
    "dropped_prefix": ("memcpy(S, jb->init + ((size_t)b * H + h) * sdd, sdd * sizeof(double));",
                       "memset(S, 0, sdd * sizeof(double));"),
    "dropped_last_token": ("t < t1; ++t", "t + 1 < t1; ++t"),
    "layer_factor_L": ("(double)layer_id / (double)(num_layers - 1)",
                       "(double)layer_id / (double)(num_layers)"),
    "layer_factor_no_eps": ("(double)(num_layers - 1) + 1e-5", "(double)(num_layers - 1)"),
    "alibi_odd_offset": ("(2 * j + 1)", "(2 * j + 2)"),
    "alibi_exponent": ("-8.0 * (double)(i + 1) / (double)m", "-8.0 * (double)(i) / (double)m"),
    "wrong_head_stride": ("jb->k + ((size_t)t * HK + hk) * d", "jb->k + ((size_t)t * HK + (hk ^ 1) % HK) * d"),
    "gqa_interleaved": ("const int hk = h / (H / HK); /* key/value head of query head h */",
                        "const int hk = h % HK;"),
    "track_one_late": ("if (snap && t - t0 == tl)", "if (snap && t - t0 == tl + 1)"),
    "track_end_missing": ("if (snap && tl == t1 - t0)", "if (snap && tl == t1 - t0 && 0)"),
    "tree_ignores_parent": ("const int p = jb->parents[(size_t)b * n + j];", "const int p = j - 1;"),
    "tree_always_root": ("const double *from = p < 0 ?", "const double *from = 1 ?"),
    "tree_parent_off_by_one": ("jb->draft_state + (((size_t)b * n + p) * H + h) * sdd",
                               "jb->draft_state + (((size_t)b * n + (p > 0 ? p - 1 : p)) * H + h) * sdd"),
    "tree_no_decay": ("""const int hk = h / (H / HK);
    const double decay = exp(-jb->slopes[h]);
    const double scale = 1.0 / sqrt((double)d);
    const size_t sdd = (size_t)d * d;

    for (int j = 0;""", """const int hk = h / (H / HK);
    const double decay = 1.0;
    const double scale = 1.0 / sqrt((double)d);
    const size_t sdd = (size_t)d * d;

    for (int j = 0;"""),
}


def _build(tmp_path, name, text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(text)
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-o",
                    str(so), str(c), "-lm", "-lpthread"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.la_oracle_run.restype = ctypes.c_int
    lib.la_oracle_alibi_slopes.restype = ctypes.c_int
    lib.la_oracle_tree.restype = ctypes.c_int
    return lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _run(lib, q, k, v, cu, S0, slopes, track=None):
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    B = cu.shape[0] - 1
    H, d = S0.shape[1], S0.shape[2]
    HK = k.shape[1]
    q, k, v, S0 = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, S0))
    sl = np.ascontiguousarray(slopes, dtype=np.float64)
    out = np.zeros((int(cu[-1]), H, d))
    fin = np.zeros((B, H, d, d))
    tl = None if track is None else np.ascontiguousarray(track, dtype=np.int64)
    snap = None if track is None else np.full((B, H, d, d), np.nan)
    rc = lib.la_oracle_run(B, H, HK, d, _p(cu), _p(q), _p(k), _p(v), _p(S0), _p(sl), _p(tl),
                           _p(out), _p(fin), _p(snap), 2)
    assert rc == 0
    return (out, fin) if track is None else (out, fin, snap)


def _state_after(k, v, S0, lam, n):
    w = np.exp(-lam * (n - 1 - np.arange(n)))
    return math.exp(-lam * n) * S0 + np.einsum("s,si,sj->ij", w, k[:n], v[:n])


def _gqa_ok(lib):
    """Grouped heads: query head h against the closed form with kv head h // 2."""
    rng = np.random.default_rng(4)
    H, HK, d, T = 4, 2, 4, 6
    q = rng.standard_normal((T, H, d))
    k, v = rng.standard_normal((T, HK, d)), rng.standard_normal((T, HK, d))
    S0 = 0.2 * rng.standard_normal((1, H, d, d))
    lam = np.array([0.5, 0.2, 0.1, 0.02])
    out, fin = _run(lib, q, k, v, [0, T], S0, lam)
    for h in range(H):
        S = _state_after(k[:, h // 2], v[:, h // 2], S0[0, h], lam[h], T)
        if not np.allclose(fin[0, h], S, rtol=1e-10, atol=1e-12):
            return False
        if not np.allclose(out[T - 1, h], q[T - 1, h] @ S / math.sqrt(d), rtol=1e-10, atol=1e-12):
            return False
    return True


def _track_ok(lib):
    """Snapshots at 0, inside and at the end of a request against the closed form."""
    rng = np.random.default_rng(5)
    d, lens, tls = 4, [6, 6, 6], [0, 3, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (rng.standard_normal((cu[-1], 1, d)) for _ in range(3))
    S0 = 0.2 * rng.standard_normal((3, 1, d, d))
    lam = 0.35
    _, _, snap = _run(lib, q, k, v, cu, S0, np.array([lam]), track=tls)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        if not np.allclose(snap[b, 0], _state_after(k[sl, 0], v[sl, 0], S0[b, 0], lam, tls[b]),
                           rtol=1e-10, atol=1e-12):
            return False
    return True


def _tree_ok(lib):
    """A branching tree against the root-path closed form of every draft's state."""
    rng = np.random.default_rng(6)
    par = [-1, 0, 0, 2, -1, 4]
    n, d = len(par), 4
    q, k, v = (rng.standard_normal((n, 1, d)) for _ in range(3))
    S0 = 0.2 * rng.standard_normal((1, 1, d, d))
    lam = 0.3
    out = np.zeros((n, 1, d))
    st = np.zeros((1, n, 1, d, d))
    pr = np.array(par, dtype=np.int32)
    rc = lib.la_oracle_tree(1, n, 1, 1, d, _p(q), _p(k), _p(v), _p(S0), _p(np.array([lam])),
                            _p(pr), _p(out), _p(st), 1)
    if rc != 0:
        return False
    for j in range(n):
        path, a = [], j
        while a >= 0:
            path.append(a)
            a = par[a]
        path = path[::-1]
        m = len(path)
        S = math.exp(-lam * m) * S0[0, 0]
        for i, a in enumerate(path, start=1):
            S = S + math.exp(-lam * (m - i)) * np.outer(k[a, 0], v[a, 0])
        if not np.allclose(st[0, j, 0], S, rtol=1e-10, atol=1e-12):
            return False
        if not np.allclose(out[j, 0], q[j, 0] @ S / math.sqrt(d), rtol=1e-10, atol=1e-12):
            return False
    return True


def _closed_form_ok(lib):
    rng = np.random.default_rng(1)
    H, d, lens = 2, 8, [7, 3]
    lams = np.array([0.4, 0.03])
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (rng.standard_normal((cu[-1], H, d)) for _ in range(3))
    S0 = 0.3 * rng.standard_normal((2, H, d, d))
    out, fin = _run(lib, q, k, v, cu, S0, lams)
    for b in range(2):
        for h in range(H):
            sl = slice(cu[b], cu[b + 1])
            S = S0[b, h]
            for t in range(lens[b]):
                w = np.exp(-lams[h] * (t - np.arange(t + 1)))
                S = math.exp(-lams[h] * (t + 1)) * S0[b, h] + np.einsum(
                    "s,si,sj->ij", w, k[sl, h][: t + 1], v[sl, h][: t + 1])
                if not np.allclose(out[cu[b] + t, h], q[cu[b] + t, h] @ S / math.sqrt(d),
                                   rtol=1e-10, atol=1e-12):
                    return False
            if not np.allclose(fin[b, h], S, rtol=1e-10, atol=1e-12):
                return False
    return True


def _cumsum_ok(lib):
    rng = np.random.default_rng(2)
    T, d = 9, 8
    q, k, v = (rng.standard_normal((T, 1, d)) for _ in range(3))
    S0 = rng.standard_normal((1, 1, d, d))
    out, fin = _run(lib, q, k, v, [0, T], S0, np.zeros(1))
    Q, K, V = q[:, 0], k[:, 0], v[:, 0]
    return (np.allclose(out[:, 0], (np.tril(Q @ K.T) @ V + Q @ S0[0, 0]) / math.sqrt(d))
            and np.allclose(fin[0, 0], S0[0, 0] + K.T @ V))


def _worked_example_ok(lib):
    with open(os.path.join(GOLDEN, "worked_example_d2.json")) as f:
        g = json.load(f)
    reqs = g["requests"]
    cu = np.concatenate([[0], np.cumsum([len(r["q"]) for r in reqs])])
    cat = lambda key: np.array([row for r in reqs for row in r[key]], dtype=np.float64)[:, None, :]
    S0 = np.array([r["init_state"] for r in reqs], dtype=np.float64)[:, None]
    out, fin = _run(lib, cat("q"), cat("k"), cat("v"), cu, S0, np.array([g["slope"]]))
    for b, r in enumerate(reqs):
        if not np.allclose(out[cu[b]:cu[b + 1], 0], np.array(r["out_over_scale"]) / math.sqrt(2)):
            return False
        if not np.allclose(fin[b, 0], np.array(r["final_state"])):
            return False
    return True


def _slopes_ok(lib):
    with open(os.path.join(GOLDEN, "alibi_slopes.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        H = case["num_heads"]
        base = np.array([2.0 ** e for e in case["log2_base"]])
        for lf, fac in (((0, 1), 1 + 1e-5), ((1, 4), 1 - 1 / 3 + 1e-5), ((3, 4), 1e-5)):
            got = np.empty(H, dtype=np.float32)
            if lib.la_oracle_alibi_slopes(H, lf[0], lf[1], ctypes.c_void_p(got.ctypes.data)) != 0:
                return False
            if not np.array_equal(got, (base * fac).astype(np.float32)):
                return False
    return True


CHECKS = [_closed_form_ok, _cumsum_ok, _worked_example_ok, _slopes_ok, _gqa_ok, _track_ok,
          _tree_ok]


def test_unmodified_oracle_passes_checks(tmp_path):
    lib = _build(tmp_path, "orig", open(SRC).read())
    assert all(check(lib) for check in CHECKS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    lib = _build(tmp_path, name, text.replace(old, new, 1))
    failed = [c.__name__ for c in CHECKS if not c(lib)]
    assert failed, f"mutant {name} passed every pin"
