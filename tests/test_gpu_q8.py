"""GPU parity of moe_ffn_forward_q8 (Q8_K-style int8 expert activations) against the oracle's quantised-activation
layer, to the layer's bar, on the decode path (T <= 4) and on the bucketed path (grouped GEMMs in one MFMA pass on
the codes) at every workload size, plus its accuracy against the exact layer (cosine, as the pages report for their
int8-activation path).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 4), ("30b-decode", 1), ("30b-decode", 3),
                                    ("235b-shape", 2), ("tiny", 5), ("tiny", 37), ("30b-batch", 64),
                                    ("30b-batch", 300), ("30b-prefill", 2048), ("235b-shape", 512)])
def test_q8_parity(name, T):
    import torch

    print(f"[q8] {name} T={T}", flush=True)
    inp = synth.make_inputs(synth.WORKLOADS[name], seed=12, tokens=T)
    layer, dev = parity.make_layer(inp)
    g = parity.run_gpu(layer, dev["x"], q8=True)
    layer.close()
    rep = {}
    parity.check_parity(inp, g, report=rep, q8=True)
    exact = oracle.forward(inp.x, inp.router, inp.bias, inp.gate, inp.up, inp.down, inp.wl.top_k)["out"]
    a, b = exact.ravel(), g.out.astype(np.float64).ravel()
    cos = a @ b / np.sqrt((a @ a) * (b @ b))
    print(f"[q8] {name} T={T}: {rep} cosine vs exact layer {cos:.8f}", flush=True)
    assert cos > 0.999
    del torch
