"""The seeded input generator: determinism and the distributions it promises."""
import numpy as np

import synth


def test_same_seed_same_bytes():
    wl = synth.WORKLOADS["tiny"]
    a = synth.digest(synth.make_inputs(wl, seed=3))
    b = synth.digest(synth.make_inputs(wl, seed=3))
    c = synth.digest(synth.make_inputs(wl, seed=3, replica=1))
    assert a == b and a != c


def test_shapes_and_fields():
    wl = synth.WORKLOADS["30b-decode"]
    inp = synth.make_inputs(wl, seed=1)
    assert inp.x.shape == (1, 2048) and inp.x.dtype == np.float32
    assert inp.router.shape == (128, 2048)
    assert inp.gate.shape == (128, 768, 8, 144) and inp.down.shape == (128, 2048, 3, 144)
    d = inp.gate[..., 0:2].copy().view(np.float16).astype(np.float64)
    assert np.all(d >= 0) and 0.006 < d.mean() < 0.01  # E|N(0, 0.01)| = 0.00798
    q = inp.gate[..., 16:]
    lo, hi = q & 15, q >> 4
    assert abs(lo.mean() - 7.5) < 0.01 and abs(hi.mean() - 7.5) < 0.01
    assert abs(inp.router.std() - 0.02) < 2e-4


def test_zipf_bias():
    b = synth.gen_bias(128, 1.1)
    assert b[0] == 0.0 and np.all(np.diff(b) < 0)
    assert synth.gen_bias(8, 0.0) is None
