"""GPU parity at sizes whose element offsets pass 2^31: a prefill whose token
tensors hold more than 2^31 elements, and a decode whose state pool does.

The oracle checks sampled heads (prefill) and the addressed slots (decode);
untouched pool slots are compared bit for bit on a sample.
"""
import numpy as np
import pytest
import torch

import linear_attention_amd as la
import oracle
from linear_attention_amd import workloads as W

from gpu_util import TOL, assert_close, check_against_oracle, device_inputs, host_io, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def test_prefill_token_offsets_beyond_2pow31():
    """T=131073 tokens at H=128, d=128: q/k/v/out hold 2^31 + 16384 elements
    each, so the last token's offsets need more than 31 bits."""
    T, H = 131073, 128
    assert T * H * 128 > 2 ** 31
    log(f"case prefill-2^31 T={T} H={H}: generating inputs")
    wl = W.make("prefill-2^31", "prefill", "bf16", H, [T], 2, seed=901, prefix=[True], slot_idx=[1])
    log("inputs ready; running the GPU path")
    out, pool, _ = run_gpu(wl)
    heads = [0, 77, 127]
    log(f"oracle on heads {heads}")
    check_against_oracle(wl, out, pool, heads=heads)
    tail = out[T - 64:].float()
    assert torch.isfinite(tail).all()


def test_decode_pool_offsets_beyond_2pow31():
    """A pool of 2100 slots x 64 heads holds 2.2e9 floats; the requests use the
    last slots, whose state offsets need more than 31 bits."""
    P, H, B = 2100, 64, 8
    assert P * H * 128 * 128 > 2 ** 31
    slots = np.arange(P - B, P, dtype=np.int32)[::-1].copy()
    log(f"case decode-2^31 P={P} H={H} slots={slots.tolist()}")
    wl = W.make("decode-2^31", "decode", "bf16", H, np.ones(B, dtype=np.int64), P, seed=902,
                prefix=np.ones(B, dtype=bool), slot_idx=slots)
    out, pool, _ = run_gpu(wl)
    check_against_oracle(wl, out, pool)
    sample = np.array([0, 1, P // 2, P - B - 1], dtype=np.int64)
    got = pool.index_select(0, torch.from_numpy(sample).cuda()).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), wl.pool[sample].view(np.uint32)), "untouched slot changed"
