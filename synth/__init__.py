"""Seeded synthetic inputs for the routed-expert MoE FFN layer.

This module only draws numbers. It holds none of the layer's arithmetic, so the
GPU path and the CPU oracle can both take their inputs from it without sharing
any computation.

Workloads (shapes of one Qwen3-MoE decoder layer's routed-expert FFN; the pages
name the Qwen3-Coder-30B-A3B Q4_K_M file as their model):

    tiny          H=256  E=8   k=2 I=256  T=4
    30b-decode    H=2048 E=128 k=8 I=768  T=1
    30b-batch     H=2048 E=128 k=8 I=768  T=64
    30b-prefill   H=2048 E=128 k=8 I=768  T=2048  Zipf(1.1) expert bias
    235b-shape    H=4096 E=128 k=8 I=1536 T=512   Zipf(1.1) expert bias

Recipe (the same for every workload):

* x ~ N(0, 1), fp32, [T, H].
* router weight ~ N(0, 0.02), fp32, [E, H] (row e scores expert e).
* Zipf-skewed workloads add a fixed per-expert bias b[e] = -s*ln(e+1) with
  s = 1.1 (expert 0 is the hottest); the others pass no bias.
* Expert weights are Q4_K super-blocks of 144 bytes per 256 weights, stored
  expert-major, row-major, blocks along the reduction dimension:
  gate and up [E][I][H/256][144], down [E][H][I/256][144].
  In each block, bytes 0-1 and 2-3 are the fp16 super-block scale d and min
  scale dmin, each |N(0, 0.01)| rounded to fp16 (round to nearest even);
  bytes 4-143 are uniform random bytes. Because every bit of the 12 packed
  scale bytes and of the 128 quant bytes belongs to exactly one field, uniform
  bytes make every 6-bit sub-block scale and min uniform on 0..63 and every
  4-bit quant uniform on 0..15, independently.

Seeds: tensor tau of replica r under seed s comes from
PCG64(SeedSequence([s, r, tau])) with tau = 0 for x, 1 for the router weight,
2 for the expert blobs (drawn expert by expert: gate, up, down).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

Q4K_BLOCK_BYTES = 144
Q4K_BLOCK_WEIGHTS = 256

TENSOR_X = 0
TENSOR_ROUTER = 1
TENSOR_EXPERTS = 2
TENSOR_NORM = 3
NORM_EPS = 1e-6  # the RMSNorm eps of the Qwen3-MoE models


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    experts: int
    top_k: int
    inter: int
    tokens: int
    zipf: float = 0.0  # 0 = no expert bias

    @property
    def nsb_h(self) -> int:
        return self.hidden // Q4K_BLOCK_WEIGHTS

    @property
    def nsb_i(self) -> int:
        return self.inter // Q4K_BLOCK_WEIGHTS

    @property
    def expert_bytes(self) -> int:
        """Q4_K bytes of one expert's gate, up and down matrices together."""
        return 3 * self.hidden * self.inter * Q4K_BLOCK_BYTES // Q4K_BLOCK_WEIGHTS

    def with_tokens(self, tokens: int) -> "Workload":
        return dataclasses.replace(self, tokens=tokens)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 8, 2, 256, 4),
    "30b-decode": Workload("30b-decode", 2048, 128, 8, 768, 1),
    "30b-batch": Workload("30b-batch", 2048, 128, 8, 768, 64),
    "30b-prefill": Workload("30b-prefill", 2048, 128, 8, 768, 2048, zipf=1.1),
    "235b-shape": Workload("235b-shape", 4096, 128, 8, 1536, 512, zipf=1.1),
}
WORKLOAD_ORDER = ["tiny", "30b-decode", "30b-batch", "30b-prefill", "235b-shape"]


def rng(seed: int, replica: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, replica, tensor])))


def gen_x(seed: int, replica: int, tokens: int, hidden: int) -> np.ndarray:
    g = rng(seed, replica, TENSOR_X)
    return g.standard_normal((tokens, hidden), dtype=np.float64).astype(np.float32)


def gen_router(seed: int, replica: int, experts: int, hidden: int) -> np.ndarray:
    g = rng(seed, replica, TENSOR_ROUTER)
    return (g.standard_normal((experts, hidden), dtype=np.float64) * 0.02).astype(np.float32)


def gen_bias(experts: int, zipf: float) -> np.ndarray | None:
    if zipf == 0.0:
        return None
    e = np.arange(experts, dtype=np.float64)
    return (-zipf * np.log(e + 1.0)).astype(np.float32)


def gen_norm(seed: int, replica: int, hidden: int) -> np.ndarray:
    """Pre-FFN norm weight [H] fp32, uniform in [0.5, 1.5)."""
    g = rng(seed, replica, TENSOR_NORM)
    return (0.5 + g.random(hidden, dtype=np.float64)).astype(np.float32)


def _random_bytes(g: np.random.Generator, n: int) -> np.ndarray:
    words = (n + 7) // 8
    return g.bit_generator.random_raw(words).view(np.uint8)[:n]


def _fill_q4k(g: np.random.Generator, out: np.ndarray) -> None:
    """Fill a [..., 144] uint8 view with random Q4_K blocks (layout in the module doc)."""
    nblk = int(np.prod(out.shape[:-1]))
    flat = out.reshape(nblk, Q4K_BLOCK_BYTES)
    d = np.abs(g.standard_normal(nblk, dtype=np.float64) * 0.01).astype(np.float16)
    dmin = np.abs(g.standard_normal(nblk, dtype=np.float64) * 0.01).astype(np.float16)
    flat[:, 0:2] = d.view(np.uint8).reshape(nblk, 2)
    flat[:, 2:4] = dmin.view(np.uint8).reshape(nblk, 2)
    flat[:, 4:] = _random_bytes(g, nblk * (Q4K_BLOCK_BYTES - 4)).reshape(nblk, Q4K_BLOCK_BYTES - 4)


def gen_experts(seed: int, replica: int, wl: Workload):
    """Return (gate, up, down) uint8 arrays [E][rows][K/256][144]."""
    E, H, I = wl.experts, wl.hidden, wl.inter
    gate = np.empty((E, I, H // 256, Q4K_BLOCK_BYTES), np.uint8)
    up = np.empty_like(gate)
    down = np.empty((E, H, I // 256, Q4K_BLOCK_BYTES), np.uint8)
    g = rng(seed, replica, TENSOR_EXPERTS)
    for e in range(E):
        _fill_q4k(g, gate[e])
        _fill_q4k(g, up[e])
        _fill_q4k(g, down[e])
    return gate, up, down


@dataclasses.dataclass
class LayerInputs:
    wl: Workload
    x: np.ndarray
    router: np.ndarray
    bias: np.ndarray | None
    gate: np.ndarray
    up: np.ndarray
    down: np.ndarray


def make_inputs(wl: Workload, seed: int = 0, replica: int = 0, tokens: int | None = None) -> LayerInputs:
    T = wl.tokens if tokens is None else tokens
    gate, up, down = gen_experts(seed, replica, wl)
    return LayerInputs(
        wl=wl.with_tokens(T),
        x=gen_x(seed, replica, T, wl.hidden),
        router=gen_router(seed, replica, wl.experts, wl.hidden),
        bias=gen_bias(wl.experts, wl.zipf),
        gate=gate,
        up=up,
        down=down,
    )


def digest(inp: LayerInputs) -> str:
    h = hashlib.sha256()
    for a in (inp.x, inp.router, inp.gate, inp.up, inp.down):
        h.update(np.ascontiguousarray(a).tobytes())
    if inp.bias is not None:
        h.update(inp.bias.tobytes())
    return h.hexdigest()
