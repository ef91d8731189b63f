"""GPU parity of the HIP layer (through the C ABI) against the fp64 oracle.

Every workload at its full size, every output element of every token compared
with the oracle (the two large ones also have a fast sampled variant). Edge
cases: ragged token counts across tile boundaries, one
expert taking every token, k = E, zero input, wide dynamic range, Q4_K
super-blocks with d = 0 (on 16-row and 64-row tiles), workspace growth,
bitwise run-to-run determinism, and the ABI's error returns.
"""
import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

_cache = {}


def _layer(name, seed=0, bias=None, k=None):
    key = (name, seed, None if bias is None else bias.tobytes(), k)
    if key not in _cache:
        import quantized_moe_wave_amd as q
        import torch

        wl = synth.WORKLOADS[name]
        if k is not None:
            import dataclasses

            wl = dataclasses.replace(wl, top_k=k)
        inp = synth.make_inputs(wl, seed=seed)
        if bias is not None:
            inp.bias = bias
        layer, dev = parity.make_layer(inp)
        _cache.clear()  # keep one layer resident at a time
        torch.cuda.synchronize()
        _cache[key] = (inp, layer, dev)
    return _cache[key]


def _x(inp, T, seed=1, scale=1.0):
    x = synth.gen_x(seed, 7, T, inp.wl.hidden) * np.float32(scale)
    return x.astype(np.float32)


def _run(inp, layer, x):
    import torch

    inp2 = synth.LayerInputs(inp.wl.with_tokens(x.shape[0]), x, inp.router, inp.bias, inp.gate, inp.up, inp.down)
    g = parity.run_gpu(layer, torch.from_numpy(x).cuda())
    return inp2, g


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_full(name):
    print(f"[parity] workload {name} full", flush=True)
    inp, layer, dev = _layer(name)
    g = parity.run_gpu(layer, dev["x"])
    rep = {}
    parity.check_parity(inp, g, report=rep)
    print(f"[parity] {name}: {rep}", flush=True)


@pytest.mark.parametrize("name,nsample", [("30b-prefill", 48), ("235b-shape", 40)])
def test_workload_sampled(name, nsample):
    """Fast variant of the full check on a seeded sample of tokens."""
    print(f"[parity] workload {name} sampled", flush=True)
    inp, layer, dev = _layer(name)
    g = parity.run_gpu(layer, dev["x"])
    T = inp.x.shape[0]
    rng = np.random.default_rng(123)
    sel = np.unique(np.concatenate([[0, T - 1], rng.choice(T, nsample, replace=False)])).astype(np.int32)
    rep = {}
    parity.check_parity(inp, g, sel=sel, report=rep)
    print(f"[parity] {name}: {rep} U={int((g.counts > 0).sum())} max_bucket={int(g.counts.max())}", flush=True)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 15, 16, 17, 33, 100])
def test_ragged_token_counts(T):
    print(f"[parity] 30b ragged T={T}", flush=True)
    inp, layer, _ = _layer("30b-batch")
    inp2, g = _run(inp, layer, _x(inp, T, seed=T))
    parity.check_parity(inp2, g)


@pytest.mark.parametrize("T", [2047, 2048, 2049])
def test_bucketing_paths(T):
    """Around the switch between the one-workgroup bucketing (up to 4096 pairs) and the two-launch one: the tiny
    layer (k = 2) at 4094, 4096 and 4098 pairs, buckets of several hundred pairs (64-row tiles)."""
    print(f"[parity] tiny T={T} ({2 * T} pairs)", flush=True)
    inp, layer, _ = _layer("tiny", seed=9)
    inp2, g = _run(inp, layer, _x(inp, T, seed=60 + T))
    parity.check_parity(inp2, g)


def test_one_expert_takes_every_token():
    print("[parity] tiny, expert 0 forced for all tokens", flush=True)
    bias = np.zeros(8, np.float32)
    bias[0] = 50.0
    inp, layer, _ = _layer("tiny", seed=3, bias=bias)
    inp2, g = _run(inp, layer, _x(inp, 45, seed=2))
    assert np.all(g.idx[:, 0] == 0) and g.counts[0] == 45
    parity.check_parity(inp2, g)


def test_k_equals_num_experts():
    print("[parity] tiny, k = E = 8", flush=True)
    inp, layer, _ = _layer("tiny", seed=4, k=8)
    inp2, g = _run(inp, layer, _x(inp, 21, seed=5))
    assert np.all(np.sort(g.idx, axis=1) == np.arange(8))
    parity.check_parity(inp2, g)


def test_zero_input():
    print("[parity] zero input", flush=True)
    inp, layer, _ = _layer("tiny", seed=5)
    x = np.zeros((6, inp.wl.hidden), np.float32)
    inp2, g = _run(inp, layer, x)
    assert np.all(g.out == 0.0)
    assert np.all(g.idx == np.array([0, 1])) and np.all(g.w == 0.5)
    parity.check_parity(inp2, g)


@pytest.mark.parametrize("scale", [1e-4, 1e4])
def test_dynamic_range(scale):
    print(f"[parity] 30b batch, x scaled by {scale}", flush=True)
    inp, layer, _ = _layer("30b-batch")
    x = _x(inp, 24, seed=9, scale=scale)
    x[::3] *= np.float32(1e3)  # rows of very different magnitude
    x[:, ::7] *= np.float32(1e-3)  # and columns within a row
    inp2, g = _run(inp, layer, x)
    parity.check_parity(inp2, g)


def test_bitwise_determinism():
    print("[parity] determinism", flush=True)
    import torch

    inp, layer, dev = _layer("30b-batch")
    a = parity.run_gpu(layer, dev["x"])
    b = parity.run_gpu(layer, dev["x"])
    torch.cuda.synchronize()
    assert np.array_equal(a.out.view(np.uint32), b.out.view(np.uint32))
    assert np.array_equal(a.w.view(np.uint32), b.w.view(np.uint32))
    assert np.array_equal(a.idx, b.idx)


def test_workspace_growth_and_reserve():
    print("[parity] workspace growth", flush=True)
    inp, layer, _ = _layer("tiny", seed=6)
    layer.reserve(2)
    for T in (1, 9, 70, 3):
        inp2, g = _run(inp, layer, _x(inp, T, seed=T + 40))
        parity.check_parity(inp2, g)


def test_error_returns():
    print("[parity] error returns", flush=True)
    import torch

    import quantized_moe_wave_amd as q

    inp, layer, dev = _layer("tiny", seed=7)
    x = dev["x"]
    with pytest.raises(q.MoeError, match="INVALID_SHAPE"):
        q.moe_ffn_forward(layer.handle, x[:0], torch.empty_like(x[:0]))
    with pytest.raises(q.MoeError, match="INVALID_ARG"):
        q.moe_ffn_forward(layer.handle, x, x)  # out aliases x
    with pytest.raises(q.MoeError, match="BLOB_SIZE"):
        q.moe_ffn_create(256, 8, 2, 256, dev["gate"][:-1], dev["up"], dev["down"], dev["router"])
    # host pointer where device memory is required
    from quantized_moe_wave_amd.binding import _lib, _vp
    import ctypes

    xh = np.zeros((4, 256), np.float32)
    st = _lib.moe_ffn_forward(_vp(layer.handle), 4, xh.ctypes.data_as(ctypes.c_void_p),
                              ctypes.c_void_p(torch.empty_like(x).data_ptr()), None, None, None)
    assert st == 2
    # token counts whose staged activations pass 4 GiB (T*4*hidden_dim >= 2^32 at hidden 256, k = 2, I = 256):
    # rejected before any pointer is read or any workspace is sized
    for T in (1 << 22, (1 << 21) + 1):
        ok = T * 4 * 256 < (1 << 32) and T * 2 * 4 * 256 < (1 << 32)
        st = _lib.moe_ffn_forward(_vp(layer.handle), T, ctypes.c_void_p(x.data_ptr()),
                                  ctypes.c_void_p(torch.empty_like(x).data_ptr()), None, None, None)
        assert not ok and st == 1, (T, st)
    # the layer still works after the rejected calls
    g = parity.run_gpu(layer, x)
    parity.check_parity(inp, g)


def test_graph_replay_matches_eager():
    """The forward captured in a HIP graph, replayed several times with eager
    work and synchronisations between replays: every replay equals eager."""
    print("[parity] graph replay", flush=True)
    import torch

    inp, layer, dev = _layer("30b-batch")
    x = dev["x"]
    eager = parity.run_gpu(layer, x)
    layer.reserve(x.shape[0])
    out = torch.empty_like(x)
    w = torch.empty((x.shape[0], layer.top_k), dtype=torch.float32, device=x.device)
    idx = torch.empty((x.shape[0], layer.top_k), dtype=torch.int32, device=x.device)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        layer.forward(x, out, w, idx)
    for rep in range(4):
        out.fill_(float("nan"))
        w.zero_()
        idx.fill_(-1)
        other = parity.run_gpu(layer, x[: 5 + rep])  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager.out.view(np.uint32)), rep
        assert np.array_equal(w.cpu().numpy(), eager.w) and np.array_equal(idx.cpu().numpy(), eager.idx), rep
        assert other.out.shape[0] == 5 + rep


def test_exact_ties_many_experts():
    """x = 0 makes all 128 logits equal: the lower-index rule picks 0..k-1."""
    print("[parity] 30b ties", flush=True)
    inp, layer, _ = _layer("30b-batch")
    for T in (1, 3, 9):
        x = np.zeros((T, inp.wl.hidden), np.float32)
        inp2, g = _run(inp, layer, x)
        assert np.array_equal(g.idx, np.tile(np.arange(8), (T, 1)))
        assert np.all(g.w == np.float32(0.125)) and np.all(g.out == 0.0)
        parity.check_parity(inp2, g)


@pytest.mark.parametrize("T", [3, 20])
def test_many_experts(T):
    """E = 300 > 256 takes the iterated-argmax selection; k = 6."""
    print(f"[parity] E=300 k=6 T={T}", flush=True)
    import dataclasses

    import synth as _s

    wl = dataclasses.replace(_s.WORKLOADS["tiny"], name="e300", experts=300, top_k=6)
    key = ("e300", T)
    inp = _s.make_inputs(wl, seed=21)
    layer, dev = parity.make_layer(inp)
    inp2, g = _run(inp, layer, _x(inp, T, seed=31 + T))
    parity.check_parity(inp2, g)
    layer.close()


@pytest.mark.parametrize("E,T", [(256, 3), (256, 40), (160, 40)])
def test_experts_up_to_256(E, T):
    """128 < E <= 256: the widest rank selection (every candidate counts 256
    keys; E = 256 uses the whole 8-bit index field of the key), on the decode
    path (T = 3) and the general path (T = 40), for the layer and the block."""
    print(f"[parity] E={E} k=8 T={T}", flush=True)
    import dataclasses

    import synth as _s

    wl = dataclasses.replace(_s.WORKLOADS["tiny"], name=f"e{E}", experts=E, top_k=8)
    inp = _s.make_inputs(wl, seed=40 + E)
    layer, dev = parity.make_layer(inp)
    inp2, g = _run(inp, layer, _x(inp, T, seed=50 + T))
    parity.check_parity(inp2, g)
    # the block too: on the general path its norm folds into the top-k launch's widest ranking
    import torch

    import oracle

    hidden = (_s.gen_x(4, 11, T, wl.hidden) * np.float32(3.0)).astype(np.float32)
    gn = _s.gen_norm(4, 0, wl.hidden)
    layer.set_norm(torch.from_numpy(gn), _s.NORM_EPS)
    run = parity.run_gpu(layer, torch.from_numpy(hidden).cuda(), block=True)
    xn = oracle.rms_norm(hidden, gn, _s.NORM_EPS).astype(np.float32)
    parity.check_parity(_s.LayerInputs(wl.with_tokens(T), xn, inp.router, inp.bias, inp.gate, inp.up, inp.down), run,
                        resid=hidden)
    layer.close()


@pytest.mark.parametrize("T", [64, 200, 256, 257])
def test_large_bucket_in_small_call(T):
    """Calls whose buckets average at most 16 pairs (T*k <= 16*E: T <= 256 here) cut every bucket into 16-row
    tiles and launch no 64-row GEMM; a bias that sends every token to expert 0 makes one bucket of T pairs there
    (4, 13 and 16 tiles of 16 rows), and at T = 257 the call takes 64-row tiles again."""
    print(f"[parity] 30b shape, expert 0 forced, T={T}", flush=True)
    bias = np.zeros(128, np.float32)
    bias[0] = 40.0
    inp, layer, _ = _layer("30b-batch", seed=8, bias=bias)
    inp2, g = _run(inp, layer, _x(inp, T, seed=88 + T))
    assert g.counts[0] == T
    parity.check_parity(inp2, g)


@pytest.mark.parametrize("name,T", [("tiny", 300), ("30b-batch", 300)])
def test_big_tiles_full_parity(name, T):
    """A bias that sends every token to expert 0 makes 128-row grouped-GEMM
    tiles (plus a remainder) that the oracle can check element by element;
    the 30b shape also has an odd super-block count on the down projection."""
    print(f"[parity] big tiles {name} T={T}", flush=True)
    E = synth.WORKLOADS[name].experts
    bias = np.zeros(E, np.float32)
    bias[0] = 40.0
    inp, layer, _ = _layer(name, seed=8, bias=bias)
    inp2, g = _run(inp, layer, _x(inp, T, seed=77))
    assert g.counts[0] == T
    parity.check_parity(inp2, g)


@pytest.mark.parametrize("H,T", [(1280, 37), (1536, 40), (4352, 21)])
def test_row_lengths(H, T):
    """Hidden sizes around the top-k launch's split of a row over four waves: 5 super-blocks (an odd tail, and the
    fourth wave holds no pair), 6 (the router split over H, partials added by the top-k launch) and 17 (longer than
    the four waves' registers hold: one wave per token, the row read twice); the layer, and the block with its
    norm (folded into the top-k launch, or a launch of its own for the 17-block row)."""
    import dataclasses

    import torch

    import oracle

    print(f"[parity] H={H} T={T}", flush=True)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"h{H}", hidden=H)
    inp = synth.make_inputs(wl, seed=60 + H // 256)
    layer, dev = parity.make_layer(inp)
    inp2, g = _run(inp, layer, _x(inp, T, seed=70 + T))
    parity.check_parity(inp2, g)
    hidden = (synth.gen_x(3, 11, T, H) * np.float32(3.0)).astype(np.float32)
    gn = synth.gen_norm(3, 0, H)
    layer.set_norm(torch.from_numpy(gn), synth.NORM_EPS)
    run = parity.run_gpu(layer, torch.from_numpy(hidden).cuda(), block=True)
    layer.close()
    xn = oracle.rms_norm(hidden, gn, synth.NORM_EPS).astype(np.float32)
    inp_n = synth.LayerInputs(wl.with_tokens(T), xn, inp.router, inp.bias, inp.gate, inp.up, inp.down)
    parity.check_parity(inp_n, run, resid=hidden)


@pytest.mark.parametrize("k,inter", [(3, 256), (1, 768), (3, 768)])
def test_decode_odd_unit_counts(k, inter):
    """Decode path (T <= 4) with an odd number of (slot, super-block) units, k * inter / 256 = 3, 3 and 9: the
    down/combine launch pairs the units two per MFMA tile, so the last pair has one unit; the layer and the block."""
    import dataclasses

    import torch

    import oracle

    print(f"[parity] decode k={k} I={inter}", flush=True)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"odd{k}_{inter}", top_k=k, inter=inter)
    inp = synth.make_inputs(wl, seed=80 + k + inter // 256)
    layer, dev = parity.make_layer(inp)
    for T in (1, 4):
        inp2, g = _run(inp, layer, _x(inp, T, seed=90 + T))
        parity.check_parity(inp2, g)
    T = 3
    hidden = (synth.gen_x(5, 11, T, wl.hidden) * np.float32(3.0)).astype(np.float32)
    gn = synth.gen_norm(5, 0, wl.hidden)
    layer.set_norm(torch.from_numpy(gn), synth.NORM_EPS)
    run = parity.run_gpu(layer, torch.from_numpy(hidden).cuda(), block=True)
    layer.close()
    xn = oracle.rms_norm(hidden, gn, synth.NORM_EPS).astype(np.float32)
    parity.check_parity(synth.LayerInputs(wl.with_tokens(T), xn, inp.router, inp.bias, inp.gate, inp.up, inp.down), run,
                        resid=hidden)


@pytest.mark.parametrize("name,T", [("30b-batch", 64), ("tiny", 200)])
def test_super_blocks_with_zero_d(name, T):
    # Q4_K super-blocks whose d is 0 (scales, quants, dmin and mins left as
    # generated): such a block's weights are -dmin * m, only its min term
    # counts. 30b-batch at 64 tokens runs every bucket on 16-row tiles (each
    # super-block's sum in its own accumulator), tiny at 200 tokens on 64-row
    # tiles (the rescaled accumulator, whose d ratios treat d = 0 as 1)
    print(f"[parity] {name} T={T}: every third super-block with d = 0", flush=True)
    import torch

    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl, seed=4)
    for m in (inp.gate, inp.up, inp.down):
        blocks = m.reshape(-1, synth.Q4K_BLOCK_BYTES)
        blocks[::3, 0:2] = 0
    _cache.clear()
    layer, _ = parity.make_layer(inp)
    try:
        x = synth.gen_x(4, 7, T, wl.hidden).astype(np.float32)
        inp2 = synth.LayerInputs(wl.with_tokens(T), x, inp.router, inp.bias, inp.gate, inp.up, inp.down)
        g = parity.run_gpu(layer, torch.from_numpy(x).cuda())
        parity.check_parity(inp2, g)
    finally:
        layer.close()
