"""The seeded input generators shared by the tests and the benchmark (CPU)."""

import pytest

from chunked_gated_linear_amd import inputs as I


def test_varlen_lengths_sum_and_bounds():
    for nseq, T, seed in [(64, 65536, 1006), (1, 5, 0), (7, 7, 3), (300, 12000, 1)]:
        L = I.varlen_lengths(nseq, T, seed=seed)
        assert len(L) == nseq and sum(L) == T and min(L) >= 1
        assert L == I.varlen_lengths(nseq, T, seed=seed)          # seeded
    assert I.varlen_lengths(64, 65536, seed=1) != I.varlen_lengths(64, 65536, seed=2)
    with pytest.raises(ValueError):
        I.varlen_lengths(10, 5)


def test_make_inputs_shapes_and_unit_keys():
    inp = I.make_inputs(2, 33, 3, 64, 16, dtype="fp32", seed=4, h0_std=0.02)
    assert tuple(inp["q"].shape) == (2, 33, 3, 64) and tuple(inp["v"].shape) == (2, 33, 3, 16)
    assert tuple(inp["h0"].shape) == (2, 3, 64, 16)
    n = inp["k"].double().norm(dim=-1)
    assert float((n - 1).abs().max()) < 1e-6
    b = inp["beta"]
    assert float(b.min()) > 0 and float(b.max()) < 1


def test_channel_gate_shape_seed_and_moments():
    x = I.make_channel_gate(1, 512, 2, 64, seed=9, mu=-8.0, std=1.0)
    assert tuple(x.shape) == (1, 512, 2, 64)
    assert bool((x == I.make_channel_gate(1, 512, 2, 64, seed=9, mu=-8.0, std=1.0)).all())
    assert abs(float(x.mean()) + 8.0) < 0.05 and abs(float(x.std()) - 1.0) < 0.05
    # its own stream: the other inputs of the same seed do not move
    a = I.make_inputs(1, 8, 2, 64, 16, dtype="fp32", seed=9)
    I.make_channel_gate(1, 8, 2, 64, seed=9)
    b = I.make_inputs(1, 8, 2, 64, 16, dtype="fp32", seed=9)
    assert bool((a["q"] == b["q"]).all()) and bool((a["x"] == b["x"]).all())
