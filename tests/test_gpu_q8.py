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


_cache = {}


def _layer(name, **repl):
    import dataclasses

    import torch

    key = (name, tuple(sorted(repl.items())))
    if key not in _cache:
        wl = synth.WORKLOADS[name]
        if repl:
            wl = dataclasses.replace(wl, name=f"{name}-{'-'.join(f'{k}{v}' for k, v in sorted(repl.items()))}", **repl)
        inp = synth.make_inputs(wl, seed=17)
        layer, dev = parity.make_layer(inp)
        for v in _cache.values():
            v[1].close()
        _cache.clear()  # one layer resident at a time
        torch.cuda.synchronize()
        _cache[key] = (inp, layer)
    return _cache[key]


def _run_q8(inp, layer, x):
    import torch

    inp2 = synth.LayerInputs(inp.wl.with_tokens(x.shape[0]), x, inp.router, inp.bias, inp.gate, inp.up, inp.down)
    g = parity.run_gpu(layer, torch.from_numpy(np.ascontiguousarray(x)).cuda(), q8=True)
    return inp2, g


@pytest.mark.parametrize("T", [5, 17, 33, 100])
def test_q8_ragged_token_counts(T):
    """Bucketed path with 16-row tiles only (T = 5), both tile kinds and the last-round split (T >= 17)."""
    print(f"[q8] 30b-batch ragged T={T}", flush=True)
    inp, layer = _layer("30b-batch")
    x = synth.gen_x(40 + T, 3, T, inp.wl.hidden)
    inp2, g = _run_q8(inp, layer, x)
    parity.check_parity(inp2, g, q8=True)


def test_q8_zero_rows_and_blocks():
    """All-zero rows and all-zero super-blocks of x: their Q8 blocks have d = 0 and codes 0 (the GEMM's row scale
    then counts as 1); an all-zero input gives an all-zero output."""
    print("[q8] zero rows and blocks", flush=True)
    inp, layer = _layer("30b-batch")
    x = synth.gen_x(55, 3, 24, inp.wl.hidden)
    x[1::4, :] = 0.0
    x[::2, 256:512] = 0.0
    x[3, 1792:] = 0.0
    inp2, g = _run_q8(inp, layer, x)
    parity.check_parity(inp2, g, q8=True)
    z = np.zeros((6, inp.wl.hidden), np.float32)
    inp3, gz = _run_q8(inp, layer, z)
    assert np.all(gz.out == 0.0)
    parity.check_parity(inp3, gz, q8=True)


@pytest.mark.parametrize("scale", [1e-4, 1e4])
def test_q8_dynamic_range(scale):
    """Rows and columns of very different magnitudes: each 256-value block takes its own Q8 scale."""
    print(f"[q8] 30b-batch x scaled by {scale}", flush=True)
    inp, layer = _layer("30b-batch")
    x = synth.gen_x(9, 7, 24, inp.wl.hidden) * np.float32(scale)
    x[::3] *= np.float32(1e3)
    x[:, ::7] *= np.float32(1e-3)
    inp2, g = _run_q8(inp, layer, x.astype(np.float32))
    parity.check_parity(inp2, g, q8=True)


@pytest.mark.parametrize("T", [3, 20])
def test_q8_many_experts(T):
    """E = 300 > 256: the iterated-argmax top-k, and x staged by stage_kernel (Q8 codes) instead of the top-k
    launch; k = 6."""
    print(f"[q8] E=300 k=6 T={T}", flush=True)
    inp, layer = _layer("tiny", experts=300, top_k=6)
    x = synth.gen_x(31 + T, 7, T, inp.wl.hidden)
    inp2, g = _run_q8(inp, layer, x)
    parity.check_parity(inp2, g, q8=True)
