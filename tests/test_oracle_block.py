"""Pins of the oracle's pre-FFN RMSNorm and residual add (the block around the layer; CPU only).

The norm is checked against closed forms (constant rows, the eps term, a hand-worked two-element row),
invariants (unit mean square, scale invariance, the weight acting element-wise) and the residual against a
layer whose experts are all zero (the block output is then the residual stream itself, exactly). A dropped
mean, square root, eps or weight, or a residual added with the wrong sign or taken after the norm, fails one of
them.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _ones(H):
    return np.ones(H, np.float32)


@pytest.mark.parametrize("c", [1.0, -2.5, 0.125, 3.0e4])
def test_constant_row_normalises_to_its_sign(c):
    H = 256
    x = np.full((1, H), c, np.float32)
    y = oracle.rms_norm(x, _ones(H), 0.0)
    assert np.max(np.abs(y - math.copysign(1.0, c))) < 1e-15


@pytest.mark.parametrize("c,eps", [(1.0, 1e-6), (0.01, 1e-4), (3.0, 0.5)])
def test_eps_sits_inside_the_root(c, eps):
    H = 512
    x = np.full((2, H), c, np.float32)
    y = oracle.rms_norm(x, _ones(H), eps)
    ref = float(np.float32(c)) / math.sqrt(float(np.float32(c)) ** 2 + eps)
    assert np.max(np.abs(y - ref)) < 1e-13 * abs(ref)  # rounding of the sum of H equal squares


def test_hand_worked_row():
    # x = (3, 4): mean square (9 + 16) / 2 = 12.5; g = (1, 2); eps = 0
    y = oracle.rms_norm(np.array([[3.0, 4.0]], np.float32), np.array([1.0, 2.0], np.float32), 0.0)
    assert abs(y[0, 0] - 3.0 / math.sqrt(12.5)) < 1e-15
    assert abs(y[0, 1] - 8.0 / math.sqrt(12.5)) < 1e-15


def test_unit_mean_square_and_scale_invariance():
    H = 2048
    x = synth.gen_x(4, 0, 8, H)
    y = oracle.rms_norm(x, _ones(H), 0.0)
    assert np.max(np.abs(np.mean(y * y, axis=1) - 1.0)) < 1e-13
    # a power-of-two scale of the row is exact in fp32, so the normalised row is unchanged
    y2 = oracle.rms_norm(x * np.float32(8.0), _ones(H), 0.0)
    assert np.max(np.abs(y2 - y)) < 1e-14


def test_weight_acts_element_wise():
    H = 1024
    x = synth.gen_x(5, 0, 3, H)
    g = synth.gen_norm(5, 0, H)
    y1 = oracle.rms_norm(x, _ones(H), 1e-6)
    yg = oracle.rms_norm(x, g, 1e-6)
    assert np.max(np.abs(yg - y1 * g.astype(np.float64)) / (np.abs(yg) + 1e-300)) < 1e-15


def test_zero_row_with_eps_gives_zero():
    H = 256
    y = oracle.rms_norm(np.zeros((1, H), np.float32), synth.gen_norm(0, 0, H), 1e-6)
    assert np.all(y == 0.0)


def test_block_with_zero_experts_is_the_residual_stream():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl, seed=2)
    zero = np.zeros_like(inp.gate)  # d = dmin = 0: every dequantised weight is 0
    zd = np.zeros_like(inp.down)
    g = synth.gen_norm(2, 0, wl.hidden)
    r = oracle.block(inp.x, g, synth.NORM_EPS, inp.router, inp.bias, zero, zero, zd, wl.top_k)
    assert np.array_equal(r["out"], inp.x.astype(np.float64))


def test_block_adds_the_layer_of_the_normalised_rows():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl, seed=3)
    g = synth.gen_norm(3, 0, wl.hidden)
    r = oracle.block(inp.x, g, synth.NORM_EPS, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)
    # the layer's input: normalised rows rounded to fp32, as numpy computes them here
    x64 = inp.x.astype(np.float64)
    xn = (x64 * g.astype(np.float64) / np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True) + synth.NORM_EPS))
    assert np.array_equal(r["xn"], xn.astype(np.float32))
    # and the layer's own output on those rows (the whole-layer oracle is pinned elsewhere)
    ffn = oracle.forward(xn.astype(np.float32), inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)["out"]
    assert np.max(np.abs(r["out"] - (x64 + ffn))) <= 1e-12 * np.max(np.abs(x64 + ffn))
