"""GPU per-stage statistics (moe_ffn_debug_stats) against the oracle's statistics of the oracle's own stages.

For the last token of a forward on both launch paths, and of a block forward: counts exactly, min / max / mean /
rms of the router logits, router weights, SwiGLU h (the k slots, from the oracle's expert evaluation) and the output
row within the layer's error bars. A NaN planted in one token's input must show first in that token's router-logit
stage, as in the oracle, while the other tokens stay clean.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _oracle_stages(inp, ref, t, out_row):
    k = inp.wl.top_k
    hs = [oracle.expert_q4k(inp.x[t], inp.gate[e], inp.up[e], inp.down[e])[3] for e in ref["idx"][t][:k]]
    return np.stack([oracle.stage_stats(ref["logits"][t]), oracle.stage_stats(ref["w"][t]),
                     oracle.stage_stats(np.concatenate(hs)), oracle.stage_stats(out_row)])


def _compare(gpu, want, ref_vals):
    assert np.array_equal(gpu[:, :3], want[:, :3]), (gpu[:, :3], want[:, :3])
    # min, max, mean against the stage's largest magnitude; rms relative
    tol = [1e-9, 1e-6, 1e-3, 1e-3]  # logits fp64; weights; h and output at the layer's precision
    for s in range(4):
        scale = max(np.max(np.abs(ref_vals[s])), 1e-30)
        assert np.all(np.abs(gpu[s, 3:6] - want[s, 3:6]) <= tol[s] * scale), (s, gpu[s], want[s])
        assert abs(gpu[s, 6] - want[s, 6]) <= max(tol[s], 1e-4) * want[s, 6], (s, gpu[s], want[s])


def _stage_values(inp, ref, t, out_row):
    k = inp.wl.top_k
    hs = [oracle.expert_q4k(inp.x[t], inp.gate[e], inp.up[e], inp.down[e])[3] for e in ref["idx"][t][:k]]
    return [ref["logits"][t], ref["w"][t], np.concatenate(hs), out_row]


@pytest.mark.parametrize("name,T", [("tiny", 4), ("30b-decode", 1), ("30b-batch", 64)])
def test_stats_match_the_oracle(name, T):
    import torch

    import quantized_moe_wave_amd as q

    print(f"[stats] {name} T={T}", flush=True)
    inp = synth.make_inputs(synth.WORKLOADS[name], seed=4, tokens=T)
    layer, dev = parity.make_layer(inp)
    out = torch.empty_like(dev["x"])
    w = torch.empty((T, inp.wl.top_k), dtype=torch.float32, device=out.device)
    layer.forward(dev["x"], out, w)
    st = q.moe_ffn_debug_stats(layer.handle, T - 1, out, w).cpu().numpy()
    torch.cuda.synchronize()
    gidx = torch.empty((T, inp.wl.top_k), dtype=torch.int32, device=out.device)
    layer.forward(dev["x"], out, w, gidx)  # same call again, for the chosen experts
    layer.close()
    ref = oracle.forward(inp.x, inp.router, inp.bias, inp.gate, inp.up, inp.down, inp.wl.top_k)
    t = T - 1
    assert np.array_equal(gidx.cpu().numpy()[t], ref["idx"][t])  # seed chosen with no near-tie there
    _compare(st, _oracle_stages(inp, ref, t, ref["out"][t]), _stage_values(inp, ref, t, ref["out"][t]))


def test_block_stats_output_row_is_the_block_output():
    import torch

    import quantized_moe_wave_amd as q

    print("[stats] block", flush=True)
    wl = synth.WORKLOADS["tiny"]
    T = 3
    inp = synth.make_inputs(wl, seed=5)
    hidden = synth.gen_x(5, 11, T, wl.hidden)
    g = synth.gen_norm(5, 0, wl.hidden)
    layer, _ = parity.make_layer(inp)
    layer.set_norm(torch.from_numpy(g), synth.NORM_EPS)
    hd = torch.from_numpy(hidden).cuda()
    out = layer.forward_block(hd)
    st = q.moe_ffn_debug_stats(layer.handle, T - 1, out).cpu().numpy()
    layer.close()
    ref = oracle.block(hidden, g, synth.NORM_EPS, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)
    want = oracle.stage_stats(ref["out"][T - 1])
    assert np.array_equal(st[3, :3], want[:3])
    scale = np.max(np.abs(ref["out"][T - 1]))
    assert np.all(np.abs(st[3, 3:6] - want[3:6]) <= 1e-3 * scale)
    assert abs(st[3, 6] - want[6]) <= 1e-4 * want[6]


def test_nan_enters_at_the_router_logits():
    import torch

    import quantized_moe_wave_amd as q

    print("[stats] planted NaN", flush=True)
    wl = synth.WORKLOADS["tiny"]
    T = 3
    inp = synth.make_inputs(wl, seed=6, tokens=T)
    x = inp.x.copy()
    x[2, 5] = np.nan
    layer, _ = parity.make_layer(inp)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    layer.forward(xd, out)
    clean = q.moe_ffn_debug_stats(layer.handle, 0, out).cpu().numpy()
    bad = q.moe_ffn_debug_stats(layer.handle, 2, out).cpu().numpy()
    layer.close()
    ref = oracle.forward(x, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)
    assert np.all(clean[:, 1:3] == 0)
    # every logit of the poisoned token is NaN, in both; the first non-finite stage is the logits
    assert bad[0, 1] == wl.experts == oracle.stage_stats(ref["logits"][2])[1]
    assert bad[0, 2] == 0
