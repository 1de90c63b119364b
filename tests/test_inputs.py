"""CPU checks of the seeded input generators shared by the oracle's tests and the GPU path."""
import numpy as np
import torch

from online_softmax_fa2_amd.inputs import (attn_bits_large, attn_inputs, bf16_bits_to_f32, bf16_round,
                                           decode_inputs, decode_slice, softmax_rows_inputs)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        # exact ties: low 16 bits == 0x8000, both parities of bit 16
                        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, 1e-40, -3.0e38, 3.0e38], np.float32)])
    bits, vals = bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(vals, ref.to(torch.float32).numpy())
    assert np.array_equal(bf16_bits_to_f32(bits), vals)


def test_attn_inputs_deterministic_and_bf16_exact():
    a = attn_inputs(2, 3, 50, 16, dtype="bf16", seed=7, n_big_keys=5)
    b = attn_inputs(2, 3, 50, 16, dtype="bf16", seed=7, n_big_keys=5)
    for n in ("q", "k", "v"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
        assert np.array_equal(bf16_bits_to_f32(getattr(a, n + "_bits")), getattr(a, n))
    # big keys are exact multiples by 8 of the rounded draw
    c = attn_inputs(2, 3, 50, 16, dtype="bf16", seed=7)
    assert np.array_equal(a.k[:, :, a.big_keys], c.k[:, :, a.big_keys] * 8)
    other = np.setdiff1d(np.arange(50), a.big_keys)
    assert np.array_equal(a.k[:, :, other], c.k[:, :, other])


def test_decode_slice_matches_full():
    full = decode_inputs(1, 3, 70, 8, seed=9)
    for h in range(3):
        q, k, v, qb, kb, vb = decode_slice(9, 0, h, 70, 8)
        assert np.array_equal(q, full["q"][0, h]) and np.array_equal(k, full["k"][0, h])
        assert np.array_equal(vb, full["v_bits"][0, h])


def test_softmax_inputs_blocks_are_independent_of_row_count():
    a = softmax_rows_inputs(300, 40, seed=1)
    b = softmax_rows_inputs(600, 40, seed=1)
    assert np.array_equal(a, b[:300])


def test_attn_bits_large_regions():
    regions = [(0, 1, 5, 40), (1, 0, 0, 3)]
    a = attn_bits_large(2, 2, 64, 16, regions, seed=3, count=4)
    b = attn_bits_large(2, 2, 64, 16, regions, seed=3, count=4)
    assert len(a) == 4 and all(np.array_equal(x, y) for x, y in zip(a, b))
    for x in a:
        v = bf16_bits_to_f32(x)
        mask = np.zeros(v.shape, bool)
        for bb, h, r0, r1 in regions:
            mask[bb, h, r0:r1] = True
        assert np.all(v[~mask] == 0)
        m = np.abs(v[mask])
        assert m.min() >= 0.125 and m.max() < 2.0 and (v[mask] < 0).any() and (v[mask] > 0).any()
    assert not np.array_equal(a[0], a[1])
