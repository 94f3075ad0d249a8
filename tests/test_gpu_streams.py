"""Calls on several streams at once.  The library keeps no per-call state of
its own (the caller lends each split prefill its workspace), so prefills,
a decode and a chain verify launched side by side on different streams must
each give what they give alone: every output and state is compared with the
fp64 oracle (tolerance 3e-2), and pool slots no call names stay untouched."""
import numpy as np
import pytest
import torch

import linear_attention_amd as la
from linear_attention_amd import workloads as W

from gpu_util import check_against_oracle, check_untouched, device_inputs, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def test_four_entry_points_on_four_streams():
    # a prefill long enough to split into sequence segments at 2 heads, a
    # varlen prefill, a decode and a chain verify, each with its own pool
    wls = [
        W.make("streams-split", "prefill", "bf16", 2, [20000], 2, seed=2101, prefix=[True]),
        W.make("streams-varlen", "prefill", "bf16", 4, [300, 0, 1200, 65], 6, seed=2102,
               prefix=[True, False, True, False]),
        W.make("streams-decode", "decode", "bf16", 8, [1] * 24, 30, seed=2103, prefix=[True] * 24),
        W.make("streams-verify", "verify", "bf16", 8, [4] * 12, 14, seed=2104, prefix=[True] * 12, num_draft=4),
    ]
    for wl in wls:
        log(f"case {wl.name}")
    ins = [device_inputs(wl) for wl in wls]
    outs = [torch.empty_like(d["q"]) for d in ins]
    ws = []
    for wl, d in zip(wls, ins):
        n = la.la_prefill_workspace_bytes(wl.batch, wl.total_tokens, wl.max_seqlen, wl.num_heads, wl.head_dim) \
            if wl.kind == "prefill" else 0
        ws.append(torch.empty(n, dtype=torch.uint8, device="cuda") if n else None)
    assert ws[0] is not None, "the long prefill should split"
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in wls]
    for _ in range(2):  # the second round runs from the states the first left
        for wl, d, out, w, st in zip(wls, ins, outs, ws, streams):
            with torch.cuda.stream(st):
                if wl.kind == "prefill":
                    la.la_prefill(d["q"], d["k"], d["v"], d["cu"], d["pool"], d["slot"], d["slopes"], out,
                                  wl.max_seqlen, workspace=w)
                elif wl.kind == "decode":
                    la.la_decode(d["q"], d["k"], d["v"], d["pool"], d["slot"], d["slopes"], out)
                else:
                    la.la_verify(d["q"], d["k"], d["v"], wl.num_draft, d["pool"], d["slot"], d["slopes"], out)
        torch.cuda.synchronize()
        for wl, d, out in zip(wls, ins, outs):
            check_against_oracle(wl, out, d["pool"])
            check_untouched(wl, d["pool"])
            # the next round starts from the states this one wrote
            wl.pool = d["pool"].cpu().numpy()
