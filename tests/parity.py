"""Shared parity logic: run the HIP layer and the oracle on the same seeded
inputs and compare them to the stated bar.

Bar (all five workloads):
  * expert indices and bucket layout bit-exact, except tokens whose fp64
    oracle logits have a near-tie (gap < 1e-6 between consecutive sorted
    logits among the first k+1); those are counted and checked against the
    oracle evaluated at the GPU's own choice;
  * router weights within 1e-5 absolute;
  * output max|gpu - ref| <= 2e-3 * max|ref| and sum|gpu - ref| / sum|ref| <= 1e-4
    (the mean relative error read as an L1 ratio, since element-wise ratios
    blow up near zero);
  * GPU fp64 router logits within 5e-7 of the oracle's (keeps the near-tie
    exclusion sound).
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth

TIE_GAP = 1e-6
W_ATOL = 1e-5
OUT_MAX_REL = 2e-3
OUT_L1_REL = 1e-4
LOGIT_ATOL = 5e-7


@dataclasses.dataclass
class GpuRun:
    out: np.ndarray
    w: np.ndarray
    idx: np.ndarray
    logits: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    entries: np.ndarray


def upload(inp: synth.LayerInputs):
    import torch

    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return {
        "gate": t(inp.gate.reshape(-1)),
        "up": t(inp.up.reshape(-1)),
        "down": t(inp.down.reshape(-1)),
        "router": t(inp.router),
        "bias": None if inp.bias is None else t(inp.bias),
        "x": t(inp.x),
    }


def make_layer(inp: synth.LayerInputs, dev_inputs=None):
    import quantized_moe_wave_amd as q

    d = dev_inputs or upload(inp)
    wl = inp.wl
    layer = q.MoeFfn(wl.hidden, wl.experts, wl.top_k, wl.inter, d["gate"], d["up"], d["down"], d["router"], d["bias"])
    return layer, d


def run_gpu(layer, x_dev, block: bool = False, q8: bool = False) -> GpuRun:
    """One forward (block: forward_block, x_dev then being the residual stream; q8: forward_q8) and its routing
    state."""
    import torch

    import quantized_moe_wave_amd as q

    T, H = x_dev.shape
    k, E = layer.top_k, layer.num_experts
    out = torch.empty_like(x_dev)
    w = torch.empty((T, k), dtype=torch.float32, device=x_dev.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x_dev.device)
    if block:
        layer.forward_block(x_dev, out, w, idx)
    elif q8:
        layer.forward_q8(x_dev, out, w, idx)
    else:
        layer.forward(x_dev, out, w, idx)
    logits = torch.empty((T, E), dtype=torch.float64, device=x_dev.device)
    counts = torch.empty(E, dtype=torch.int32, device=x_dev.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=x_dev.device)
    entries = torch.empty(T * k, dtype=torch.int32, device=x_dev.device)
    q.moe_ffn_debug_routing(layer.handle, logits, counts, offsets, entries)
    torch.cuda.synchronize()
    c = lambda a: a.cpu().numpy()
    return GpuRun(c(out), c(w), c(idx), c(logits), c(counts), c(offsets), c(entries))


def near_tie_tokens(logits: np.ndarray, k: int) -> np.ndarray:
    """Boolean [T]: some gap among the k+1 largest fp64 logits is below TIE_GAP."""
    s = -np.sort(-logits, axis=1)
    m = min(k + 1, logits.shape[1])
    if m < 2:
        return np.zeros(logits.shape[0], bool)
    gaps = s[:, : m - 1] - s[:, 1:m]
    return (gaps < TIE_GAP).any(axis=1)


def out_errors(gpu: np.ndarray, ref: np.ndarray):
    diff = np.abs(gpu.astype(np.float64) - ref)
    max_rel = diff.max() / max(np.abs(ref).max(), 1e-300)
    l1_rel = diff.sum() / max(np.abs(ref).sum(), 1e-300)
    return float(max_rel), float(l1_rel)


def check_parity(inp: synth.LayerInputs, g: GpuRun, sel=None, report=None, resid=None, q8: bool = False):
    """Assert the bar. sel: token subset for the expert part (None = all). resid: the block's residual stream
    [T][H] (inp.x then holds the normalised rows the layer ran on); the reference output is resid + layer."""
    k, E = inp.wl.top_k, inp.wl.experts
    ref = oracle.forward(inp.x, inp.router, inp.bias, inp.gate, inp.up, inp.down, k, sel=sel, q8=q8)
    T = inp.x.shape[0]
    tokens = np.arange(T) if sel is None else np.asarray(sel)

    # router logits
    logit_err = float(np.max(np.abs(g.logits - ref["logits"])))
    assert logit_err < LOGIT_ATOL, f"logit error {logit_err}"

    # expert choice: exact except near-ties
    ties = near_tie_tokens(ref["logits"], k)
    same = np.all(g.idx == ref["idx"], axis=1)
    bad = ~same & ~ties
    assert not bad.any(), f"expert choice differs at non-tie tokens {np.nonzero(bad)[0][:10]}"
    tie_diff = ~same & ties

    # router weights
    ok_w = np.abs(g.w - ref["w"]) <= W_ATOL
    if tie_diff.any():
        w_at = oracle.router_weights_at(ref["logits"], g.idx)
        ok_w[tie_diff] = np.abs(g.w[tie_diff] - w_at[tie_diff]) <= W_ATOL
    assert ok_w.all(), f"router weight error {np.max(np.abs(g.w - ref['w']))}"

    # bucket layout: the oracle's stable sort of the GPU's own choice
    counts, offsets, entries, _ = oracle.bucket(g.idx, E)
    assert np.array_equal(g.counts, counts)
    assert np.array_equal(g.offsets, offsets)
    assert np.array_equal(g.entries, entries)
    if not tie_diff.any():
        rc, ro, re_, _ = oracle.bucket(ref["idx"], E)
        assert np.array_equal(g.entries, re_)

    # outputs (tie tokens that chose differently: against the oracle at the GPU's choice)
    ref_out = ref["out"].copy()
    td = tie_diff[tokens]
    if td.any():
        forced = oracle.forward(inp.x, inp.router, inp.bias, inp.gate, inp.up, inp.down, k, sel=tokens[td],
                                idx_in=g.idx, q8=q8)
        ref_out[td] = forced["out"]
    if resid is not None:
        ref_out = oracle.add_residual(np.ascontiguousarray(resid[tokens]), ref_out)
    max_rel, l1_rel = out_errors(g.out[tokens], ref_out)
    if report is not None:
        report.update(dict(logit_err=logit_err, max_rel=max_rel, l1_rel=l1_rel, ties=int(ties.sum()),
                           tie_diff=int(tie_diff.sum()), w_err=float(np.max(np.abs(g.w - ref["w"])))))
    assert max_rel <= OUT_MAX_REL, f"output max error {max_rel} > {OUT_MAX_REL} * max|ref|"
    assert l1_rel <= OUT_L1_REL, f"output L1 ratio {l1_rel} > {OUT_L1_REL}"
    return ref
