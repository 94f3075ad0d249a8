"""The README's usage example, run as written and checked against the fp64
oracle: the prefill's outputs and states, then the decode step's outputs and
states (tolerance 3e-2, |got - ref| <= tol + tol * |ref|)."""
import os
import re

import numpy as np
import pytest
import torch

import oracle

from gpu_util import TOL, assert_close, host_io

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_matches_the_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    text = open(os.path.join(ROOT, "README.md"), encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "expected one python example in the README"
    torch.manual_seed(0)
    ns = {}
    # run the prefill part, keep the pool it leaves, then the decode part
    code = blocks[0]
    cut = code.index("# pool[5]")
    exec(compile(code[:cut], "README.md", "exec"), ns)
    torch.cuda.synchronize()
    pool_after_prefill = ns["pool"].clone()
    exec(compile(code[cut:], "README.md", "exec"), ns)
    torch.cuda.synchronize()

    bits = host_io  # bf16 tensors as their bit patterns, which the oracle upcasts exactly
    H, d, lens = ns["H"], ns["d"], ns["lens"]
    slot = ns["slot"].cpu().numpy()
    slopes = oracle.alibi_slopes(H, 3, 24)
    pool0 = np.zeros((8, H, d, d), dtype=np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    ref_out, ref_fin = oracle.prefill(bits(ns["q"]), bits(ns["k"]), bits(ns["v"]), cu, pool0, slot, slopes)
    assert_close(host_io(ns["out"]), ref_out, TOL["bf16"], "readme prefill out")
    got_fin = pool_after_prefill.cpu().numpy()[slot]
    assert_close(got_fin, ref_fin, TOL["bf16"], "readme prefill states")

    ref_od, ref_dfin = oracle.decode(bits(ns["qd"]), bits(ns["kd"]), bits(ns["vd"]),
                                     pool_after_prefill.cpu().numpy(), slot, slopes)
    assert_close(host_io(ns["od"]), ref_od, TOL["bf16"], "readme decode out")
    assert_close(ns["pool"].cpu().numpy()[slot], ref_dfin, TOL["bf16"], "readme decode states")
