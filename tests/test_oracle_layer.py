"""Pins of the oracle's router, bucketing, expert FFN and whole layer (CPU only).

Each check compares the oracle with something other than itself: numpy's
float64 matmul, numpy's stable full sort, scipy's softmax, closed forms, and
invariants of the method (routing weights sum to one, dense-sum equivalence
when every expert is chosen, permutation equivariance, token independence,
zero input).
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

TINY = synth.WORKLOADS["tiny"]


def _inputs(wl=TINY, seed=0, T=None):
    return synth.make_inputs(wl, seed=seed, tokens=T)


# ---------------------------------------------------------------- router


def test_logits_match_numpy_matmul():
    inp = _inputs(synth.WORKLOADS["30b-prefill"].with_tokens(64), seed=3)
    logits, _, _ = oracle.router(inp.x, inp.router, inp.bias, 8)
    ref = inp.x.astype(np.float64) @ inp.router.astype(np.float64).T + inp.bias.astype(np.float64)
    assert np.max(np.abs(logits - ref)) < 1e-12


def test_topk_matches_stable_full_sort():
    inp = _inputs(synth.WORKLOADS["30b-batch"], seed=5)
    logits, idx, _ = oracle.router(inp.x, inp.router, None, 8)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :8]
    assert np.array_equal(idx, ref)


def test_topk_ties_go_to_lower_index():
    rng = np.random.default_rng(0)
    logits = rng.integers(-3, 4, size=(200, 16)).astype(np.float64)  # many exact ties
    for k in (1, 3, 8, 16):
        idx = oracle.topk(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(idx, ref), k


def test_weights_sum_to_one_and_closed_form():
    inp = _inputs(synth.WORKLOADS["30b-batch"], seed=9)
    logits, idx, w = oracle.router(inp.x, inp.router, None, 8)
    assert np.max(np.abs(w.sum(1) - 1.0)) < 1e-12
    sel = np.take_along_axis(logits, idx, 1)
    closed = np.exp(sel - sel[:, :1]) / np.exp(sel - sel[:, :1]).sum(1, keepdims=True)
    assert np.max(np.abs(w - closed)) < 1e-14
    # listed largest first
    assert np.all(np.diff(sel, axis=1) <= 0)


def test_k_equals_e_gives_full_softmax():
    inp = _inputs(seed=2)
    logits, idx, w = oracle.router(inp.x, inp.router, None, TINY.experts)
    p = softmax(logits, axis=1)
    assert np.max(np.abs(w - np.take_along_axis(p, idx, 1))) < 1e-14


def test_zero_input_routes_to_first_k_equally():
    inp = _inputs()
    x = np.zeros_like(inp.x)
    _, idx, w = oracle.router(x, inp.router, None, 2)
    assert np.array_equal(idx, np.tile([0, 1], (x.shape[0], 1)))
    assert np.all(w == 0.5)


# ---------------------------------------------------------------- bucketing


def test_bucket_matches_stable_argsort():
    inp = _inputs(synth.WORKLOADS["30b-prefill"].with_tokens(300), seed=1)
    _, idx, _ = oracle.router(inp.x, inp.router, inp.bias, 8)
    counts, offsets, entries, pos = oracle.bucket(idx, 128)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=128))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(entries, np.argsort(flat, kind="stable"))
    assert np.array_equal(entries[pos], np.arange(flat.size))


# ---------------------------------------------------------------- expert FFN


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    for z in (0.3, 1.7, 12.5, 40.0):
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) < 1e-14 * max(1, z)
    v = oracle.silu(-800.0)  # exp overflows to inf: result is -0, not NaN
    assert v == 0.0 and not np.isnan(v)
    assert oracle.silu(800.0) == 800.0


def test_expert_matches_numpy_dense():
    wl = synth.WORKLOADS["30b-decode"]
    inp = _inputs(wl, seed=4)
    e = 17
    y, g, u, h = oracle.expert_q4k(inp.x[0], inp.gate[e], inp.up[e], inp.down[e])
    Wg = oracle.q4k_dequant(inp.gate[e])  # [I][H]
    Wu = oracle.q4k_dequant(inp.up[e])
    Wd = oracle.q4k_dequant(inp.down[e])  # [H][I]
    assert Wg.shape == (wl.inter, wl.hidden) and Wd.shape == (wl.hidden, wl.inter)
    x = inp.x[0].astype(np.float64)
    g_ref = Wg @ x
    u_ref = Wu @ x
    h_ref = g_ref / (1.0 + np.exp(-g_ref)) * u_ref
    y_ref = Wd @ h_ref
    rel = lambda a, b: np.max(np.abs(a - b)) / np.max(np.abs(b))
    assert rel(g, g_ref) < 1e-13 and rel(u, u_ref) < 1e-13
    assert rel(h, h_ref) < 1e-12 and rel(y, y_ref) < 1e-12


def _dense_expert_outputs(inp, x):
    """[E][T][H] per-expert outputs by numpy dense algebra on dequantised weights."""
    ys = []
    for e in range(inp.gate.shape[0]):
        Wg = oracle.q4k_dequant(inp.gate[e])
        Wu = oracle.q4k_dequant(inp.up[e])
        Wd = oracle.q4k_dequant(inp.down[e])
        g = x @ Wg.T
        u = x @ Wu.T
        ys.append((g / (1 + np.exp(-g)) * u) @ Wd.T)
    return np.stack(ys)


def test_dense_sum_equivalence_when_k_equals_e():
    inp = _inputs(seed=11, T=6)
    E = TINY.experts
    r = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, E)
    x = inp.x.astype(np.float64)
    p = softmax(x @ inp.router.astype(np.float64).T, axis=1)  # [T][E]
    ys = _dense_expert_outputs(inp, x)
    ref = np.einsum("te,eth->th", p, ys)
    assert np.max(np.abs(r["out"] - ref)) <= 1e-11 * np.max(np.abs(ref))


def test_topk_layer_matches_dense_selection():
    inp = _inputs(seed=12, T=5)
    r = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, 2)
    x = inp.x.astype(np.float64)
    ys = _dense_expert_outputs(inp, x)
    ref = np.stack([sum(r["w"][t, j] * ys[r["idx"][t, j], t] for j in range(2)) for t in range(5)])
    assert np.max(np.abs(r["out"] - ref)) <= 1e-11 * np.max(np.abs(ref))


def test_permutation_equivariance():
    inp = _inputs(seed=13)
    perm = np.random.default_rng(0).permutation(TINY.experts)
    r0 = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, 2)
    r1 = oracle.forward(inp.x, inp.router[perm], None, inp.gate[perm], inp.up[perm], inp.down[perm], 2)
    # the softmax denominator is summed in expert order, so only rounding differs
    assert np.max(np.abs(r0["out"] - r1["out"])) <= 1e-14 * np.max(np.abs(r0["out"]))
    assert np.array_equal(perm[r1["idx"]], r0["idx"])
    assert np.max(np.abs(r0["w"] - r1["w"])) < 1e-15


def test_token_independence():
    inp = _inputs(synth.WORKLOADS["30b-batch"].with_tokens(5), seed=14)
    k = 8
    full = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, k)
    for t in range(5):
        one = oracle.forward(inp.x[t : t + 1], inp.router, None, inp.gate, inp.up, inp.down, k)
        assert np.array_equal(one["out"][0], full["out"][t])
    sub = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, k, sel=[3, 1])
    assert np.array_equal(sub["out"], full["out"][[3, 1]])


def test_forced_indices_reproduce_own_choice():
    inp = _inputs(seed=15)
    r = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, 2)
    f = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, 2, idx_in=r["idx"])
    assert np.array_equal(r["out"], f["out"]) and np.array_equal(r["w"], f["w"])
    # swapping the slot order only permutes slots: same output up to rounding
    g = oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, 2, idx_in=r["idx"][:, ::-1].copy())
    assert np.max(np.abs(g["out"] - r["out"])) <= 1e-13 * np.max(np.abs(r["out"]))


def test_zero_input_gives_zero_output():
    inp = _inputs()
    r = oracle.forward(np.zeros_like(inp.x), inp.router, None, inp.gate, inp.up, inp.down, 2)
    assert np.all(r["out"] == 0.0)


def test_bad_arguments_rejected():
    inp = _inputs()
    with pytest.raises(ValueError):
        oracle.forward(inp.x, inp.router, None, inp.gate, inp.up, inp.down, 9)  # k > E
