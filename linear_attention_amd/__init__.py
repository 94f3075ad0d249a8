"""MI355X-native segmented linear attention (seg_la).

Thin Python binding over the C ABI of ``liblinattn.so`` (declared in
``include/linattn.h``).  The functions carry the C names and only marshal
arguments: they check that tensors are contiguous device tensors of the right
dtype, pass raw pointers and the current HIP stream, and raise on a non-zero
status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  PyTorch supplies device memory and streams.

The library binds to the HIP runtime that PyTorch has already loaded (torch is
imported before the library is opened), so tensors, streams and kernels share
one runtime.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP, LA_ERR_NO_SCRATCH = 0, -1, -2, -3, -4
LA_DTYPE_BF16, LA_DTYPE_F32 = 0, 1

EXPORTED = ("la_status_string", "la_alibi_slopes", "la_prefill_workspace_bytes", "la_prefill",
            "la_prefill_noalloc", "la_decode", "la_verify", "la_verify_tree")

_lib = None


class LAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {la_status_string(status)} ({status})")


def load():
    """Open liblinattn.so (built in-tree by ``linear_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- load torch's HIP runtime first

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run linear_attention_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.la_status_string.argtypes = [I]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_alibi_slopes.argtypes = [I, I, I, P]
    lib.la_alibi_slopes.restype = I
    lib.la_prefill_workspace_bytes.argtypes = [I, L, I, I, I]
    lib.la_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.la_prefill.argtypes = [P, P, P, I, P, I, L, I, I, I, I, P, L, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.la_prefill.restype = I
    lib.la_prefill_noalloc.argtypes = [P, P, P, I, P, I, L, I, I, I, I, P, L, P, P, P, P, P, P]
    lib.la_prefill_noalloc.restype = I
    lib.la_decode.argtypes = [P, P, P, I, I, I, I, I, P, L, P, P, P, P]
    lib.la_decode.restype = I
    lib.la_verify.argtypes = [P, P, P, I, I, I, I, I, I, P, L, P, P, P, P, P]
    lib.la_verify.restype = I
    lib.la_verify_tree.argtypes = [P, P, P, I, I, I, I, I, I, P, L, P, P, P, P, P, P]
    lib.la_verify_tree.restype = I
    _lib = lib
    return lib


def la_status_string(status: int) -> str:
    return load().la_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != LA_OK:
        raise LAError(status, where)


def la_alibi_slopes(num_heads: int, layer_id: int = 0, num_layers: int = 1) -> np.ndarray:
    """Host fp32 slopes [num_heads] (ALiBi sequence times the layer factor)."""
    out = np.empty(max(int(num_heads), 0), dtype=np.float32)
    _check(load().la_alibi_slopes(int(num_heads), int(layer_id), int(num_layers),
                                  out.ctypes.data if out.size else None), "la_alibi_slopes")
    return out


def _ptr(t, name, dtypes, allow_none=False):
    import torch

    if t is None:
        if allow_none:
            return None
        raise TypeError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() and not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else None


def _io_dtype(q):
    import torch

    return {torch.bfloat16: LA_DTYPE_BF16, torch.float32: LA_DTYPE_F32}[q.dtype]


def _stream(t, stream):
    import torch

    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dev = t.device if t.is_cuda else torch.device("cuda", torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def _shape(t):
    return tuple(t.shape)


def _qkv_shapes(q, k, v, out, what):
    """(N, H, Hkv, d) from q/out [N, H, d] and k/v [N, Hkv, d]; one dtype for all."""
    N, H, d = _shape(q)
    if _shape(out) != (N, H, d):
        raise ValueError(f"out must have the shape of q [{what}, H, d]")
    if k.dim() != 3 or k.shape[0] != N or k.shape[2] != d or _shape(v) != _shape(k):
        raise ValueError(f"k and v must be [{what}, Hkv, d] with q's token count and head_dim")
    if not (k.dtype == v.dtype == out.dtype == q.dtype):
        raise TypeError("q, k, v, out must share one dtype")
    return N, H, k.shape[1], d


def _pool_and_slopes(state_pool, slopes, H, d, *others):
    """The kernels index the pool as [P, H, d, d] and read H slopes: a tensor
    of another shape would send them past its allocation, so check here (the C
    ABI sees only pointers).  Every tensor must sit on the pool's device."""
    if state_pool.dim() != 4 or _shape(state_pool)[1:] != (H, d, d):
        raise ValueError(f"state_pool must be [P, H, d, d] = [P, {H}, {d}, {d}], got {_shape(state_pool)}")
    if slopes.numel() != H:
        raise ValueError(f"slopes must have one entry per head ({H}), got {slopes.numel()}")
    for t in (slopes,) + others:
        if t is not None and t.numel() and t.device != state_pool.device:
            raise ValueError(f"all tensors must be on {state_pool.device}, found one on {t.device}")


def la_prefill_workspace_bytes(batch: int, total_tokens: int, max_seqlen: int, num_heads: int,
                               head_dim: int) -> int:
    """Bytes of scratch a bf16 prefill of these sizes uses on the current device
    (0 when it runs unsplit)."""
    return int(load().la_prefill_workspace_bytes(int(batch), int(total_tokens), int(max_seqlen),
                                                 int(num_heads), int(head_dim)))


def la_prefill(q, k, v, cu_seqlens, state_pool, slot_idx, slopes, out, max_seqlen,
               track_lens=None, track_slot_idx=None, workspace="auto", stream=None):
    """Packed varlen prefill.  q, out: [T, H, d]; k, v: [T, Hkv, d] (bf16 or fp32,
    d = 64 or 128, Hkv dividing H); cu_seqlens [B+1] int32; state_pool
    [P, H, d, d] fp32 (updated in place); slot_idx [B] int32; slopes [H] fp32;
    max_seqlen: host int >= every length.  track_lens / track_slot_idx ([B] int32,
    both or neither): snapshot of request b's state after track_lens[b] tokens
    written to pool slot track_slot_idx[b] (negative: none).
    workspace: a device tensor (any dtype, contiguous) lent to the call as
    scratch; "auto" takes one of la_prefill_workspace_bytes(...) bytes from
    torch's allocator on the pool's device; None runs a call that would split
    into sequence segments unsplit."""
    import torch

    io = (torch.bfloat16, torch.float32)
    T, H, HK, d = _qkv_shapes(q, k, v, out, "T")
    B = cu_seqlens.numel() - 1
    if slot_idx.numel() != B:
        raise ValueError("slot_idx must have one entry per request")
    if (track_lens is None) != (track_slot_idx is None):
        raise ValueError("track_lens and track_slot_idx go together")
    if track_lens is not None and (track_lens.numel() != B or track_slot_idx.numel() != B):
        raise ValueError("track arrays must have one entry per request")
    _pool_and_slopes(state_pool, slopes, H, d, q, k, v, out, cu_seqlens, slot_idx, track_lens, track_slot_idx)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be a tensor, None or "auto"')
        need = 0
        if q.dtype == torch.bfloat16 and track_lens is None:
            with torch.cuda.device(state_pool.device):
                need = la_prefill_workspace_bytes(B, T, max_seqlen, H, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=state_pool.device) if need else None
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous device tensor")
        if workspace.device != state_pool.device:
            raise ValueError(f"workspace must be on {state_pool.device}")
        ws_bytes = workspace.numel() * workspace.element_size()
        ws_ptr = workspace.data_ptr() if ws_bytes else None
    i32 = (torch.int32,)
    rc = load().la_prefill(_ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io), _io_dtype(q),
                           _ptr(cu_seqlens, "cu_seqlens", i32), B, T, int(max_seqlen), H, HK, d,
                           _ptr(state_pool, "state_pool", (torch.float32,)), state_pool.shape[0],
                           _ptr(slot_idx, "slot_idx", i32, True),
                           _ptr(track_lens, "track_lens", i32, True),
                           _ptr(track_slot_idx, "track_slot_idx", i32, True),
                           _ptr(slopes, "slopes", (torch.float32,)), _ptr(out, "out", io),
                           ws_ptr, ws_bytes, _stream(state_pool, stream))
    _check(rc, "la_prefill")


def la_prefill_noalloc(q, k, v, cu_seqlens, state_pool, slot_idx, slopes, out, max_seqlen,
                       track_lens=None, track_slot_idx=None, stream=None):
    """la_prefill without a workspace, for callers that cannot allocate: a split
    into sequence segments uses the library's static per-GPU scratch (calls
    that overlap on one GPU race).  Arguments as for la_prefill."""
    import torch

    io = (torch.bfloat16, torch.float32)
    T, H, HK, d = _qkv_shapes(q, k, v, out, "T")
    B = cu_seqlens.numel() - 1
    if slot_idx.numel() != B:
        raise ValueError("slot_idx must have one entry per request")
    if (track_lens is None) != (track_slot_idx is None):
        raise ValueError("track_lens and track_slot_idx go together")
    if track_lens is not None and (track_lens.numel() != B or track_slot_idx.numel() != B):
        raise ValueError("track arrays must have one entry per request")
    _pool_and_slopes(state_pool, slopes, H, d, q, k, v, out, cu_seqlens, slot_idx, track_lens, track_slot_idx)
    i32 = (torch.int32,)
    with torch.cuda.device(state_pool.device):
        rc = load().la_prefill_noalloc(_ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io), _io_dtype(q),
                                       _ptr(cu_seqlens, "cu_seqlens", i32), B, T, int(max_seqlen), H, HK, d,
                                       _ptr(state_pool, "state_pool", (torch.float32,)), state_pool.shape[0],
                                       _ptr(slot_idx, "slot_idx", i32, True),
                                       _ptr(track_lens, "track_lens", i32, True),
                                       _ptr(track_slot_idx, "track_slot_idx", i32, True),
                                       _ptr(slopes, "slopes", (torch.float32,)), _ptr(out, "out", io),
                                       _stream(state_pool, stream))
    _check(rc, "la_prefill_noalloc")


def la_decode(q, k, v, state_pool, slot_idx, slopes, out, stream=None):
    """One token per request: q, out [B, H, d]; k, v [B, Hkv, d]; the pool is
    updated in place."""
    import torch

    io = (torch.bfloat16, torch.float32)
    B, H, HK, d = _qkv_shapes(q, k, v, out, "B")
    if slot_idx.numel() != B:
        raise ValueError("slot_idx must have one entry per request")
    _pool_and_slopes(state_pool, slopes, H, d, q, k, v, out, slot_idx)
    rc = load().la_decode(_ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io), _io_dtype(q), B, H,
                          HK, d, _ptr(state_pool, "state_pool", (torch.float32,)),
                          state_pool.shape[0], _ptr(slot_idx, "slot_idx", (torch.int32,), True),
                          _ptr(slopes, "slopes", (torch.float32,)), _ptr(out, "out", io),
                          _stream(state_pool, stream))
    _check(rc, "la_decode")


def la_verify(q, k, v, num_draft, state_pool, slot_idx, slopes, out, state_out=None, stream=None):
    """Chain verify: q, out [B*num_draft, H, d]; k, v [B*num_draft, Hkv, d]; the
    final states go to state_out [B, H, d, d] (pool untouched) or, if None,
    back to the pool."""
    import torch

    io = (torch.bfloat16, torch.float32)
    N, H, HK, d = _qkv_shapes(q, k, v, out, "B*num_draft")
    B = slot_idx.numel()
    if N != B * int(num_draft):
        raise ValueError("q must hold num_draft tokens per request")
    if state_out is not None and _shape(state_out) != (B, H, d, d):
        raise ValueError("state_out must be [B, H, d, d]")
    _pool_and_slopes(state_pool, slopes, H, d, q, k, v, out, slot_idx, state_out)
    rc = load().la_verify(_ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io), _io_dtype(q), B,
                          int(num_draft), H, HK, d, _ptr(state_pool, "state_pool", (torch.float32,)),
                          state_pool.shape[0], _ptr(slot_idx, "slot_idx", (torch.int32,), True),
                          _ptr(slopes, "slopes", (torch.float32,)), _ptr(out, "out", io),
                          _ptr(state_out, "state_out", (torch.float32,), True),
                          _stream(state_pool, stream))
    _check(rc, "la_verify")


def la_verify_tree(q, k, v, num_draft, state_pool, slot_idx, parent_idx, slopes, out,
                   draft_states=None, stream=None):
    """Tree verify: q, out [B*n, H, d]; k, v [B*n, Hkv, d]; parent_idx [B, n] int32
    with parent_idx[b][j] in [-1, j) (-1: the pool state); draft_states
    [B, n, H, d, d] fp32 receives the state after every draft (None: outputs only).
    The pool is not written."""
    import torch

    io = (torch.bfloat16, torch.float32)
    N, H, HK, d = _qkv_shapes(q, k, v, out, "B*num_draft")
    B, n = slot_idx.numel(), int(num_draft)
    if N != B * n:
        raise ValueError("q must hold num_draft tokens per request")
    if parent_idx.numel() != B * n:
        raise ValueError("parent_idx must be [B, num_draft]")
    if draft_states is not None and _shape(draft_states) != (B, n, H, d, d):
        raise ValueError("draft_states must be [B, num_draft, H, d, d]")
    _pool_and_slopes(state_pool, slopes, H, d, q, k, v, out, slot_idx, parent_idx, draft_states)
    rc = load().la_verify_tree(_ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io), _io_dtype(q),
                               B, n, H, HK, d, _ptr(state_pool, "state_pool", (torch.float32,)),
                               state_pool.shape[0], _ptr(slot_idx, "slot_idx", (torch.int32,), True),
                               _ptr(parent_idx, "parent_idx", (torch.int32,), True),
                               _ptr(slopes, "slopes", (torch.float32,)), _ptr(out, "out", io),
                               _ptr(draft_states, "draft_states", (torch.float32,), True),
                               _stream(state_pool, stream))
    _check(rc, "la_verify_tree")
