"""GPU parity of moe_ffn_forward_block (pre-FFN RMSNorm, the layer, residual add) against the oracle's block.

The oracle normalises the residual stream in float64 and rounds the rows to fp32 (the layer's input); the GPU's
routing (logits, choice, weights, bucket layout) is compared with the oracle's routing of those rows and the block
output with hidden + layer(rows), to the layer's bar. Both launch paths (at most four tokens, and the bucketed
path with a ragged tail), the zero-expert case (output = residual stream, exactly), and the error when no norm
weight was set.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _block_case(name, T, seed=0, zero_experts=False):
    import torch

    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, seed=seed)
    if zero_experts:
        inp.gate[:] = 0
        inp.up[:] = 0
        inp.down[:] = 0
    hidden = (synth.gen_x(seed, 11, T, wl.hidden) * np.float32(3.0)).astype(np.float32)
    g = synth.gen_norm(seed, 0, wl.hidden)
    layer, _ = parity.make_layer(inp)
    layer.set_norm(torch.from_numpy(g), synth.NORM_EPS)
    run = parity.run_gpu(layer, torch.from_numpy(hidden).cuda(), block=True)
    layer.close()
    return inp, hidden, g, run


# 235b-shape at T = 2: hidden 4096 (16 super-blocks), where the decode router's logit waves read each token's
# 1/rms ahead of their chunk loop instead of taking it from the chunk registers
@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 4), ("tiny", 37), ("30b-decode", 1), ("30b-decode", 3),
                                    ("30b-batch", 64), ("235b-shape", 2)])
def test_block_parity(name, T):
    print(f"[block] {name} T={T}", flush=True)
    inp, hidden, g, run = _block_case(name, T)
    xn = oracle.rms_norm(hidden, g, synth.NORM_EPS).astype(np.float32)
    inp_n = synth.LayerInputs(inp.wl.with_tokens(T), xn, inp.router, inp.bias, inp.gate, inp.up, inp.down)
    rep = {}
    parity.check_parity(inp_n, run, report=rep, resid=hidden)
    print(f"[block] {name} T={T}: {rep}", flush=True)


def test_block_with_zero_experts_returns_the_residual_stream():
    print("[block] zero experts", flush=True)
    _, hidden, _, run = _block_case("tiny", 21, zero_experts=True)
    assert np.array_equal(run.out, hidden)


def test_block_needs_a_norm_weight():
    import torch

    import quantized_moe_wave_amd as q

    inp = synth.make_inputs(synth.WORKLOADS["tiny"], seed=0)
    layer, dev = parity.make_layer(inp)
    with pytest.raises(q.MoeError):
        layer.forward_block(dev["x"])
    with pytest.raises(q.MoeError):
        layer.set_norm(torch.ones(inp.wl.hidden), float("nan"))
    layer.close()


@pytest.mark.parametrize("name,T,mode", [("30b-batch", 64, "block"), ("30b-decode", 2, "block"),
                                         ("30b-decode", 2, "q8"), ("30b-batch", 64, "q8")])
def test_graph_replay_matches_eager(name, T, mode):
    """The block (norm launch or fused norm) and the int8-activation variant captured in a HIP graph, replayed
    several times with eager work and synchronisations between replays: every replay equals the eager call,
    bit for bit."""
    import torch

    print(f"[block] graph replay {name} T={T} {mode}", flush=True)
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, seed=13, tokens=T)
    layer, dev = parity.make_layer(inp)
    layer.set_norm(torch.from_numpy(synth.gen_norm(13, 0, wl.hidden)), synth.NORM_EPS)
    layer.reserve(T)
    x = dev["x"]
    run = layer.forward_block if mode == "block" else layer.forward_q8
    eager = run(x).cpu().numpy()
    out = torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        run(x, out)
    for rep in range(3):
        out.fill_(float("nan"))
        layer.forward(x[:1], torch.empty_like(x[:1]))  # eager work on the same handle between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager.view(np.uint32)), rep
    del g
    layer.close()
