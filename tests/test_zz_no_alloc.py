"""moe_ffn_forward_noalloc (the variant for callers that cannot allocate) against moe_ffn_forward.

Both run the same kernels in the same order, the no-alloc one on the library's fixed per-device scratch, so every
output (out, router weights, expert indices, bucket layout) must be bit-identical to moe_ffn_forward's, and within
the oracle's bar. Each case makes two calls in a row, the second with fewer tokens, so the second runs over what
the first left in the shared scratch. Cases: the general path (64 and 9 tokens of the 30b shape), the decode path
(3 then 1 token), the small-batch router with its completion counters (300 experts, 3 then 2 tokens), a token
count beyond the scratch (rejected before anything is enqueued), and the call captured in a HIP graph and
replayed with other work in between.
"""
import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _run(layer, fn, x):
    import torch

    T = x.shape[0]
    out = torch.full_like(x, float("nan"))
    w = torch.full((T, layer.top_k), float("nan"), dtype=torch.float32, device=x.device)
    idx = torch.full((T, layer.top_k), -1, dtype=torch.int32, device=x.device)
    fn(x, out, w, idx)
    import quantized_moe_wave_amd as q

    E = layer.num_experts
    counts = torch.empty(E, dtype=torch.int32, device=x.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=x.device)
    entries = torch.empty(T * layer.top_k, dtype=torch.int32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float64, device=x.device)
    q.moe_ffn_debug_routing(layer.handle, logits, counts, offsets, entries)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (out, w, idx, counts, offsets, entries, logits)]


def _same(a, b):
    for u, v in zip(a, b):
        assert u.dtype == v.dtype and u.shape == v.shape
        bits = {np.dtype(np.float32): np.uint32, np.dtype(np.float64): np.uint64}.get(u.dtype)
        assert np.array_equal(u.view(bits) if bits else u, v.view(bits) if bits else v)


def _case(wl, seed, token_counts):
    import torch

    inp = synth.make_inputs(wl, seed=seed)
    layer, dev = parity.make_layer(inp)
    try:
        for T in token_counts:
            print(f"[no-alloc] {wl.name} E={wl.experts} T={T}", flush=True)
            x = synth.gen_x(seed + 100, T, T, wl.hidden)
            xd = torch.from_numpy(x).cuda()
            got = _run(layer, layer.forward_noalloc, xd)
            want = _run(layer, layer.forward, xd)
            _same(got, want)
            # and the oracle's bar, on the no-alloc call's own outputs
            inp2 = synth.LayerInputs(wl.with_tokens(T), x, inp.router, inp.bias, inp.gate, inp.up, inp.down)
            g = parity.GpuRun(got[0], got[1], got[2], got[6], got[3], got[4], got[5])
            parity.check_parity(inp2, g)
    finally:
        layer.close()


def test_general_path_then_smaller():
    _case(synth.WORKLOADS["30b-batch"], 11, [64, 9])


def test_decode_path_then_smaller():
    _case(synth.WORKLOADS["30b-decode"], 12, [3, 1])


def test_small_batch_router_counters():
    import dataclasses

    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="e300", experts=300, top_k=6)
    _case(wl, 13, [3, 2])


def test_too_many_tokens_rejected():
    import torch

    import quantized_moe_wave_amd as q

    print("[no-alloc] 30b T=4096 rejected", flush=True)
    inp = synth.make_inputs(synth.WORKLOADS["30b-batch"], seed=14, tokens=8)
    layer, dev = parity.make_layer(inp)
    try:
        x = torch.zeros((4096, inp.wl.hidden), dtype=torch.float32, device="cuda")
        out = torch.full_like(x, 7.0)
        with pytest.raises(q.MoeError, match="INVALID_SHAPE.*at most"):
            layer.forward_noalloc(x, out)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())  # nothing was enqueued
        # the handle still works, through both entry points
        g = _run(layer, layer.forward_noalloc, dev["x"])
        _same(g, _run(layer, layer.forward, dev["x"]))
    finally:
        layer.close()


def test_graph_replay():
    """Captured in a HIP graph (where allocation is impossible) and replayed with eager work between replays."""
    import torch

    print("[no-alloc] graph replay", flush=True)
    inp = synth.make_inputs(synth.WORKLOADS["30b-batch"], seed=15, tokens=24)
    layer, dev = parity.make_layer(inp)
    try:
        x = dev["x"]
        want = _run(layer, layer.forward, x)
        out = torch.empty_like(x)
        w = torch.empty((x.shape[0], layer.top_k), dtype=torch.float32, device="cuda")
        idx = torch.empty((x.shape[0], layer.top_k), dtype=torch.int32, device="cuda")
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, capture_error_mode="relaxed"):
            layer.forward_noalloc(x, out, w, idx)
        for rep in range(4):
            out.fill_(float("nan"))
            w.zero_()
            idx.fill_(-1)
            other = torch.from_numpy(synth.gen_x(rep, 3, 5 + rep, inp.wl.hidden)).cuda()
            layer.forward_noalloc(other, torch.empty_like(other))  # other work on the same scratch in between
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint32), want[0].view(np.uint32)), rep
            assert np.array_equal(w.cpu().numpy(), want[1]) and np.array_equal(idx.cpu().numpy(), want[2]), rep
        del g
    finally:
        layer.close()
