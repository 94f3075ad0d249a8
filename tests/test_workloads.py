"""Seeded input generators: determinism, bf16 rounding, layout and pool recipe."""
import numpy as np
import torch

from linear_attention_amd import workloads as w


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    # exact ties and values one ulp either side of a tie
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.nextafter(ties, 0), np.nextafter(ties, np.inf)])
    ours = w.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(w.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_config_determinism_and_recipe():
    a, b = w.config(2), w.config(2)
    for name in ("q", "k", "v", "pool", "slot_idx", "cu_seqlens"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.q.dtype == np.uint16 and a.q.shape == (a.total_tokens, 16, 128)
    assert a.batch == 8 and a.pool_slots == 64 and len(set(a.slot_idx.tolist())) == 8
    assert 1 <= a.lengths.min() and a.lengths.max() <= 4096
    assert a.prefix_mask.sum() == 4
    used = set(a.slot_idx.tolist())
    for s in range(64):
        if s not in used:
            assert np.all(a.pool[s] == w.SENTINEL)
    for s, p in zip(a.slot_idx, a.prefix_mask):
        if p:
            assert 0.03 < a.pool[s].std() < 0.07
        else:
            assert np.all(a.pool[s] == 0)
    c = w.config(2, seed=99)
    assert not np.array_equal(c.lengths, a.lengths)


def test_config1_layout():
    c = w.config(1)
    assert c.dtype == "fp32" and c.q.dtype == np.float32
    assert list(c.lengths) == [17, 40] and list(c.slot_idx) == [1, 3]
    assert np.all(c.pool[1] == 0) and np.all(c.pool[0] == w.SENTINEL) and np.all(c.pool[2] == w.SENTINEL)
    assert abs(c.pool[3].std() - 0.05) < 0.005


def test_token_blocks_regenerate_identically():
    c = w.make("t", "prefill", "bf16", 4, [300, 7], 3, seed=5)
    blk = w.normal_tokens(5, 1, 307, 4, 128, "bf16")
    np.testing.assert_array_equal(blk, c.q)
    part = w._stream(5, 1, 1).standard_normal((51, 4, 128), dtype=np.float32)
    np.testing.assert_array_equal(w.bf16_round_bits(part), c.q[256:])
