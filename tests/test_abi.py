"""C-ABI checks that need no GPU: symbols, host-side slopes, argument validation.

Validation runs before any HIP call, so these calls are safe on a machine
without a device; the non-null pointer values below are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch  # noqa: F401  -- the library binds to torch's HIP runtime

import linear_attention_amd as la
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")
FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.LIB_PATH):
        pytest.fail("liblinattn.so is not built (run __graft_entry__.build())")
    return la.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:la_status|const char \*|size_t)\s*\*?\s*(la_\w+)\(", text, re.M)))


def test_header_declares_the_bound_functions():
    assert declared_functions() == sorted(la.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (la_\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_single_hip_runtime_mapped(lib):
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_status_strings(lib):
    for s in (la.LA_OK, la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED, la.LA_ERR_HIP):
        assert la.la_status_string(s).startswith("LA_")
    assert "unknown" in la.la_status_string(17)


@pytest.mark.parametrize("H", list(range(1, 130)))
def test_slopes_match_oracle_bitwise(lib, H):
    for layer_id, L in ((0, 1), (0, 4), (1, 4), (3, 4), (5, 48)):
        np.testing.assert_array_equal(la.la_alibi_slopes(H, layer_id, L),
                                      oracle.alibi_slopes(H, layer_id, L), err_msg=f"H={H} {layer_id}/{L}")


def test_slopes_reject_bad_arguments(lib):
    buf = np.zeros(4, dtype=np.float32)
    for args in ((0, 0, 1), (4, 1, 1), (4, -1, 2), (4, 0, 0)):
        assert lib.la_alibi_slopes(*args, buf.ctypes.data) == la.LA_ERR_INVALID_ARG
    assert lib.la_alibi_slopes(4, 0, 1, None) == la.LA_ERR_INVALID_ARG


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=la.LA_DTYPE_BF16, cu=FAKE, batch=2, T=10, max_seqlen=8,
             H=4, HK=4, d=128, pool=FAKE, P=4, slot=FAKE, tl=None, ts=None, slopes=FAKE, out=FAKE,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.la_prefill(a["q"], a["k"], a["v"], a["dtype"], a["cu"], a["batch"], a["T"],
                          a["max_seqlen"], a["H"], a["HK"], a["d"], a["pool"], a["P"], a["slot"],
                          a["tl"], a["ts"], a["slopes"], a["out"], a["ws"], a["ws_bytes"], a["stream"])


def test_prefill_validation(lib):
    E, U = la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED
    assert _prefill(lib, d=32) == U           # head_dim must be 64 or 128
    assert _prefill(lib, d=256) == U
    assert _prefill(lib, d=64, q=None) == E   # 64 passes the head_dim check
    assert _prefill(lib, dtype=5) == U
    assert _prefill(lib, q=None) == E
    assert _prefill(lib, out=None) == E
    assert _prefill(lib, pool=None) == E
    assert _prefill(lib, slot=None) == E
    assert _prefill(lib, slopes=None) == E
    assert _prefill(lib, cu=None) == E
    assert _prefill(lib, batch=-1) == E
    assert _prefill(lib, T=-1) == E
    assert _prefill(lib, H=0) == E
    assert _prefill(lib, HK=0) == E
    assert _prefill(lib, HK=3) == E           # kv heads must divide heads
    assert _prefill(lib, H=4, HK=8) == E
    assert _prefill(lib, tl=FAKE) == E        # track arrays go together
    assert _prefill(lib, ts=FAKE) == E
    assert _prefill(lib, max_seqlen=-1) == E
    assert _prefill(lib, batch=5, P=4) == E   # more requests than distinct slots
    assert _prefill(lib, P=0) == E
    assert _prefill(lib, batch=2 ** 28, P=2 ** 30) == E  # grid too large
    for name in ("q", "k", "v", "out", "pool"):   # 16-byte vector accesses need aligned pointers
        assert _prefill(lib, **{name: FAKE + 8}) == E, name
    # empty work returns before any HIP call
    assert _prefill(lib, batch=0, T=0, max_seqlen=0, q=None, k=None, v=None, out=None, cu=FAKE,
                    slot=None) == la.LA_OK
    # workspace: NULL only with 0 bytes, 16-byte aligned
    assert _prefill(lib, ws=None, ws_bytes=64) == E
    assert _prefill(lib, ws=FAKE + 4, ws_bytes=1 << 30) == E


def test_prefill_noalloc_validation(lib):
    """The allocation-free prefill validates like la_prefill, before any HIP call."""
    E, U = la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=la.LA_DTYPE_BF16, cu=FAKE, batch=2, T=10, max_seqlen=8,
                 H=4, HK=4, d=128, pool=FAKE, P=4, slot=FAKE, tl=None, ts=None, slopes=FAKE, out=FAKE)
        a.update(kw)
        return lib.la_prefill_noalloc(a["q"], a["k"], a["v"], a["dtype"], a["cu"], a["batch"], a["T"],
                                      a["max_seqlen"], a["H"], a["HK"], a["d"], a["pool"], a["P"], a["slot"],
                                      a["tl"], a["ts"], a["slopes"], a["out"], None)

    assert call(d=32) == U
    assert call(q=None) == E
    assert call(cu=None) == E
    assert call(max_seqlen=-1) == E
    assert call(HK=3) == E
    assert call(pool=FAKE + 4) == E
    assert "static scratch" in la.la_status_string(la.LA_ERR_NO_SCRATCH)


def test_workspace_query_matches_the_documented_size(lib):
    """la_prefill_workspace_bytes: batch*H*(S + (S-1)*Q) head_dim^2 floats, S
    segments (as many as fill the compute units, at most 8 and at most
    max_seqlen/1024), Q sub-segments (as many as fill the compute units, at
    most 4); 0 when the call would not split (units >= CUs, max_seqlen < 8192)."""
    q = la.la_prefill_workspace_bytes
    cus = 256  # MI355X; also the library's fallback without a device
    for B, T, L, H, d in [(1, 131072, 131072, 8, 128), (1, 16384, 16384, 64, 64), (2, 60000, 40000, 4, 128),
                          (1, 9000, 9000, 1, 64), (3, 30000, 12000, 2, 128)]:
        units = B * H * (d // 32)
        S = min(8, cus // units, L // 1024)
        if S <= 1:
            assert q(B, T, L, H, d) == 0
            continue
        per = B * H * (S - 1)
        Q = max(1, min(4, cus // per))
        assert q(B, T, L, H, d) == (per * Q + B * H * S) * d * d * 4, (B, T, L, H, d)
    assert q(1, 131072, 131072, 64, 128) == 0      # 256 units fill the GPU
    assert q(1, 8191, 8191, 8, 128) == 0           # below the split threshold
    assert q(1, 8192, 8192, 8, 128) > 0
    assert q(1, 100000, 100000, 8, 96) == 0        # unsupported head_dim
    assert q(-1, 100000, 100000, 8, 128) == 0
    assert q(1, -5, 100000, 8, 128) == 0


def test_workspace_too_small_is_rejected(lib):
    """A call that would split into sequence segments rejects a non-NULL
    workspace smaller than the query's size, before launching anything; a NULL
    workspace is accepted (the call then runs unsplit, which needs a GPU, so
    only the rejection is checked here)."""
    E = la.LA_ERR_INVALID_ARG
    need = la.la_prefill_workspace_bytes(1, 131072, 131072, 8, 128)
    assert need > 0
    kw = dict(batch=1, T=131072, max_seqlen=131072, H=8, HK=8, P=2)
    assert _prefill(lib, ws=FAKE, ws_bytes=need - 16, **kw) == E
    assert _prefill(lib, ws=FAKE, ws_bytes=16, **kw) == E
    assert _prefill(lib, ws=FAKE, ws_bytes=0, **kw) == E


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=la.LA_DTYPE_BF16, batch=2, H=4, HK=4, d=128, pool=FAKE,
             P=4, slot=FAKE, slopes=FAKE, out=FAKE, stream=None)
    a.update(kw)
    return lib.la_decode(a["q"], a["k"], a["v"], a["dtype"], a["batch"], a["H"], a["HK"], a["d"],
                         a["pool"], a["P"], a["slot"], a["slopes"], a["out"], a["stream"])


def _verify(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=la.LA_DTYPE_BF16, batch=2, nd=5, H=4, HK=2, d=128,
             pool=FAKE, P=4, slot=FAKE, slopes=FAKE, out=FAKE, so=FAKE, stream=None)
    a.update(kw)
    return lib.la_verify(a["q"], a["k"], a["v"], a["dtype"], a["batch"], a["nd"], a["H"], a["HK"],
                         a["d"], a["pool"], a["P"], a["slot"], a["slopes"], a["out"], a["so"],
                         a["stream"])


def _tree(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=la.LA_DTYPE_BF16, batch=2, nd=5, H=4, HK=1, d=64,
             pool=FAKE, P=4, slot=FAKE, par=FAKE, slopes=FAKE, out=FAKE, ds=FAKE, stream=None)
    a.update(kw)
    return lib.la_verify_tree(a["q"], a["k"], a["v"], a["dtype"], a["batch"], a["nd"], a["H"],
                              a["HK"], a["d"], a["pool"], a["P"], a["slot"], a["par"], a["slopes"],
                              a["out"], a["ds"], a["stream"])


def test_decode_and_verify_validation(lib):
    E, U = la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED
    assert _decode(lib, d=48) == U
    assert _decode(lib, dtype=3) == U
    assert _decode(lib, q=None) == E
    assert _decode(lib, batch=9, P=4) == E
    assert _decode(lib, slopes=None) == E
    assert _decode(lib, HK=3) == E
    assert _verify(lib, nd=0) == U            # chain length must be positive
    assert _verify(lib, nd=-2) == U
    assert _verify(lib, d=96) == U
    assert _verify(lib, out=None) == E
    assert _verify(lib, batch=-1) == E
    assert _verify(lib, HK=-1) == E
    assert _verify(lib, batch=0, q=None, k=None, v=None, out=None, slot=None) == la.LA_OK
    assert _decode(lib, pool=FAKE + 4) == E
    assert _verify(lib, so=FAKE + 2) == E


def test_tree_verify_validation(lib):
    E, U = la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED
    assert _tree(lib, nd=0) == U
    assert _tree(lib, d=100) == U
    assert _tree(lib, dtype=9) == U
    assert _tree(lib, par=None) == E          # parents are required
    assert _tree(lib, pool=None) == E
    assert _tree(lib, HK=3) == E
    assert _tree(lib, batch=7, P=4) == E
    assert _tree(lib, batch=-1) == E
    assert _tree(lib, ds=FAKE + 12) == E
    # draft_states may be NULL, and an empty batch launches nothing
    assert _tree(lib, batch=0, q=None, k=None, v=None, out=None, slot=None, par=None,
                 ds=None) == la.LA_OK


def test_binding_rejects_host_tensors(lib):
    q = torch.zeros(3, 2, 128, dtype=torch.bfloat16)
    pool = torch.zeros(2, 2, 128, 128)
    with pytest.raises(TypeError):
        la.la_decode(q, q, q, pool, torch.zeros(3, dtype=torch.int32), torch.zeros(2), q)
    with pytest.raises(TypeError):
        la.la_decode(q, q, q.float(), pool, torch.zeros(3, dtype=torch.int32), torch.zeros(2), q)


def test_binding_rejects_pool_and_slopes_of_the_wrong_shape(lib):
    """The kernels index the pool as [P, H, d, d] and read H slopes; the
    binding refuses other shapes before any HIP call."""
    q = torch.zeros(3, 2, 128, dtype=torch.bfloat16)
    slot = torch.zeros(3, dtype=torch.int32)
    good_pool, good_slopes = torch.zeros(4, 2, 128, 128), torch.zeros(2)
    cu = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    for pool in (torch.zeros(4, 1, 128, 128), torch.zeros(4, 2, 64, 128), torch.zeros(4, 2 * 128 * 128)):
        with pytest.raises(ValueError, match="state_pool"):
            la.la_decode(q, q, q, pool, slot, good_slopes, q)
        with pytest.raises(ValueError, match="state_pool"):
            la.la_prefill(q, q, q, cu, pool, slot, good_slopes, q, 1)
        with pytest.raises(ValueError, match="state_pool"):
            la.la_verify(q, q, q, 1, pool, slot, good_slopes, q)
    with pytest.raises(ValueError, match="slopes"):
        la.la_decode(q, q, q, good_pool, slot, torch.zeros(3), q)
    with pytest.raises(ValueError, match="slopes"):
        la.la_verify_tree(q, q, q, 1, good_pool, slot, torch.full((3, 1), -1, dtype=torch.int32), torch.zeros(1),
                          q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """The product path has no fallback: without liblinattn.so, loading the
    library and calling an entry point both raise ImportError."""
    monkeypatch.setattr(la, "_lib", None)
    monkeypatch.setattr(la, "LIB_PATH", str(tmp_path / "liblinattn.so"))
    with pytest.raises(ImportError, match="not built"):
        la.load()
    q = torch.zeros(3, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ImportError, match="not built"):
        la.la_decode(q, q, q, torch.zeros(4, 2, 128, 128), torch.zeros(3, dtype=torch.int32), torch.zeros(2), q)
