"""Seeded input generators: determinism and bf16 round-to-nearest-even."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch_rne():
    rs = np.random.default_rng(0)
    x = np.concatenate([rs.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 65504.0, 1e-40, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.bf16_round(x), ref)
    assert synth.bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_generators_are_deterministic():
    a = synth.attn_inputs(2, np.array([40, 7]), 4, 2, 64, block=8)
    b = synth.attn_inputs(2, np.array([40, 7]), 4, 2, 64, block=8)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.page_table, b.page_table)
    assert all(np.array_equal(x[0], y[0]) for x, y in zip(a.kv, b.kv))


def test_page_layout_round_trips():
    a = synth.attn_inputs(3, np.array([33, 0, 100]), 4, 2, 16, block=8)
    for b, (k, v) in enumerate(a.kv):
        n = k.shape[0]
        pos = np.arange(n)
        phys = a.page_table[b, pos // a.page_size]
        np.testing.assert_array_equal(a.pages_k[phys, :, pos % a.page_size].reshape(n, -1), k.reshape(n, -1))
        np.testing.assert_array_equal(a.pages_v[phys, :, pos % a.page_size].reshape(n, -1), v.reshape(n, -1))
    used = {int(p) for b, (k, _) in enumerate(a.kv) for p in a.page_table[b, : -(-k.shape[0] // a.page_size)]}
    assert len(used) == sum(-(-k.shape[0] // a.page_size) for k, _ in a.kv)


def test_prompt_ids_never_use_mask():
    ids = synth.prompt_ids(synth.TINY, 1, 4, 5000)
    assert ids.max() <= synth.TINY.vocab - 2 and ids.min() >= 0
