"""Pins of the oracle's Q8_K-style activation quantisation and its quantised-activation layer (CPU only).

Hand-worked blocks (the largest magnitude maps to +-127 with d = amax / 127, halves round to even, zero blocks),
the round-trip error bound |d q - v| <= d / 2 on random data, and the layer: with x rows that are already integers
of largest magnitude 127 the quantised x equals x, so the gate/up side matches the oracle's own expert exactly and
only h's quantisation differs; and the quantised layer stays close to the exact one (cosine), which fails if the
quantised values were dropped, mis-scaled or sign-flipped.
"""
import numpy as np

import oracle
import synth


def _block(vals):
    v = np.zeros(256, np.float32)
    v[: len(vals)] = vals
    return v


def test_hand_worked_block():
    d, q = oracle.q8k_quantize(_block([127.0, -63.5, 0.5, 1.5, -2.5, 126.6]))
    assert d[0] == np.float32(1.0)
    assert list(q[:6]) == [127, -64, 0, 2, -2, 127]
    assert np.all(q[6:] == 0)


def test_scale_and_extremes():
    v = _block([-3.0, 1.5, 0.75])
    d, q = oracle.q8k_quantize(v)
    assert d[0] == np.float32(3.0) / np.float32(127.0)
    assert q[0] == -127  # the largest magnitude maps to the end of the range
    assert q[1] == int(np.rint(np.float32(1.5) * (np.float32(127.0) / np.float32(3.0))))


def test_zero_block_and_independent_blocks():
    v = np.concatenate([np.zeros(256, np.float32), _block([5.0, -1.0])])
    d, q = oracle.q8k_quantize(v)
    assert d[0] == 0.0 and np.all(q[:256] == 0)
    assert d[1] == np.float32(5.0) / np.float32(127.0) and q[256] == 127


def test_round_trip_error_bound():
    g = np.random.default_rng(8)
    v = (g.standard_normal(256 * 40) * g.uniform(0.01, 100.0, 256 * 40)).astype(np.float32)
    d, q = oracle.q8k_quantize(v)
    back = np.repeat(d.astype(np.float64), 256) * q.astype(np.float64)
    assert np.all(np.abs(back - v) <= np.repeat(d.astype(np.float64), 256) * (0.5 + 1e-6))
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.abs(q.reshape(-1, 256)).max(axis=1) == 127)


def test_integer_rows_pass_x_through_unchanged():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl, seed=9)
    g = np.random.default_rng(9)
    x = g.integers(-127, 128, size=inp.x.shape).astype(np.float32)
    x[:, 0] = 127.0  # every 256-block of every row reaches 127 (H = 256: one block per row)
    ref = oracle.forward(x, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)
    q8 = oracle.forward(x, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k, q8=True)
    assert np.array_equal(q8["idx"], ref["idx"]) and np.array_equal(q8["logits"], ref["logits"])
    # per token and slot: the down projection of the Q8_K values of the exact h
    for t in range(x.shape[0]):
        acc = np.zeros(wl.hidden)
        for j, e in enumerate(ref["idx"][t]):
            _, _, _, h = oracle.expert_q4k(x[t], inp.gate[e], inp.up[e], inp.down[e])
            d, q = oracle.q8k_quantize(h.astype(np.float32))
            hq = np.repeat(d.astype(np.float64), 256) * q
            wd = oracle.q4k_dequant(inp.down[e])
            acc += ref["w"][t, j] * (wd @ hq)
        assert np.max(np.abs(q8["out"][t] - acc)) <= 1e-9 * np.max(np.abs(acc))


def test_quantised_layer_stays_close_to_the_exact_one():
    wl = synth.WORKLOADS["30b-batch"]
    inp = synth.make_inputs(wl, seed=10, tokens=8)
    ref = oracle.forward(inp.x, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)
    q8 = oracle.forward(inp.x, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k, q8=True)
    a, b = ref["out"].ravel(), q8["out"].ravel()
    cos = a @ b / np.sqrt((a @ a) * (b @ b))
    assert 0.999 < cos < 1.0
    l1 = np.abs(a - b).sum() / np.abs(a).sum()
    assert 1e-4 < l1 < 5e-2  # visibly lossy, but the same layer
