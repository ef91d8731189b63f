"""Python face of the plain fp64 CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product package never does, and
this module imports nothing from it. Argument marshalling only: every step of
the arithmetic is in the C file, which cites the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _P(t):
    return ctypes.POINTER(t)


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    lib.mo_set_threads.argtypes = [ctypes.c_int]
    lib.mo_set_threads.restype = ctypes.c_int
    lib.mo_half_to_double.argtypes = [ctypes.c_uint16]
    lib.mo_half_to_double.restype = f64
    lib.mo_q4k_fields.argtypes = [vp, _P(f64), _P(f64), vp, vp, vp]
    lib.mo_q4k_dequant_block.argtypes = [vp, vp]
    lib.mo_q4k_dequant_matrix.argtypes = [vp, i64, i64, vp]
    lib.mo_router_logits.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.mo_topk.argtypes = [i32, i32, i32, vp, vp]
    lib.mo_router_weights.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.mo_bucket.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.mo_silu.argtypes = [f64]
    lib.mo_silu.restype = f64
    lib.mo_expert_dense.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mo_expert_q4k.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mo_expert_q4k.restype = ctypes.c_int
    lib.mo_forward.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.mo_forward.restype = ctypes.c_int
    lib.mo_rms_norm.argtypes = [i32, i32, vp, vp, f64, vp]
    lib.mo_add_residual.argtypes = [i64, vp, vp, vp]
    lib.mo_stage_stats.argtypes = [i64, vp, vp]
    lib.mo_q8k_quantize.argtypes = [i64, vp, vp, vp]
    lib.mo_forward_q8.argtypes = lib.mo_forward.argtypes
    lib.mo_forward_q8.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> int:
    return load().mo_set_threads(int(n))


def half_to_double(bits: np.ndarray) -> np.ndarray:
    lib = load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.mo_half_to_double(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def q4k_fields(block: np.ndarray):
    """(d, dmin, sc[8], m[8], q[256]) of one 144-byte block."""
    blk = np.ascontiguousarray(block, dtype=np.uint8).reshape(144)
    d, dmin = ctypes.c_double(), ctypes.c_double()
    sc = np.zeros(8, np.int32)
    mn = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    load().mo_q4k_fields(_ptr(blk), ctypes.byref(d), ctypes.byref(dmin), _ptr(sc), _ptr(mn), _ptr(q))
    return d.value, dmin.value, sc, mn, q


def q4k_dequant(blocks: np.ndarray) -> np.ndarray:
    """[..., nb, 144] uint8 -> [..., nb*256] float64 (rows of blocks)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    nb = b.shape[-2]
    rows = int(np.prod(b.shape[:-2])) if b.ndim > 2 else 1
    out = np.empty((rows, nb * 256), np.float64)
    load().mo_q4k_dequant_matrix(_ptr(b), rows, nb * 256, _ptr(out))
    return out.reshape(b.shape[:-2] + (nb * 256,))


def router(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None, k: int):
    """(logits [T][E] f64, idx [T][k] i32, weights [T][k] f64)."""
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
    T, H = x.shape
    E = w.shape[0]
    lib = load()
    logits = np.empty((T, E), np.float64)
    idx = np.empty((T, k), np.int32)
    wts = np.empty((T, k), np.float64)
    lib.mo_router_logits(T, H, E, _ptr(x), _ptr(w), _ptr(bias), _ptr(logits))
    lib.mo_topk(T, E, k, _ptr(logits), _ptr(idx))
    lib.mo_router_weights(T, E, k, _ptr(logits), _ptr(idx), _ptr(wts))
    return logits, idx, wts


def router_weights_at(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float64)
    idx = np.ascontiguousarray(idx, np.int32)
    T, E = logits.shape
    k = idx.shape[1]
    wts = np.empty((T, k), np.float64)
    load().mo_router_weights(T, E, k, _ptr(logits), _ptr(idx), _ptr(wts))
    return wts


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    load().mo_topk(T, E, k, _ptr(logits), _ptr(idx))
    return idx


def bucket(idx: np.ndarray, E: int):
    """(counts [E], offsets [E+1], entries [T*k], pos [T*k]) as int32."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    entries = np.empty(T * k, np.int32)
    pos = np.empty(T * k, np.int32)
    load().mo_bucket(T, k, E, _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(entries), _ptr(pos))
    return counts, offsets, entries, pos


def silu(z: float) -> float:
    return load().mo_silu(float(z))


def expert_q4k(x_row: np.ndarray, gate_e: np.ndarray, up_e: np.ndarray, down_e: np.ndarray):
    """One expert on one fp32 row: (y [H], g [I], u [I], h [I]) in float64."""
    x_row = np.ascontiguousarray(x_row, np.float32)
    H = x_row.shape[0]
    I = gate_e.shape[0]
    y = np.empty(H, np.float64)
    g = np.empty(I, np.float64)
    u = np.empty(I, np.float64)
    h = np.empty(I, np.float64)
    rc = load().mo_expert_q4k(H, I, _ptr(np.ascontiguousarray(gate_e)), _ptr(np.ascontiguousarray(up_e)),
                              _ptr(np.ascontiguousarray(down_e)), _ptr(x_row), _ptr(y), _ptr(g), _ptr(u), _ptr(h))
    if rc != 0:
        raise MemoryError("oracle expert allocation failed")
    return y, g, u, h


def q8k_quantize(v):
    """Q8_K-style quantisation of fp32 values (length a multiple of 256): (d [n/256] fp32, q [n] int8)."""
    v = np.ascontiguousarray(np.asarray(v, np.float32).ravel())
    d = np.empty(v.size // 256, np.float32)
    q = np.empty(v.size, np.int8)
    load().mo_q8k_quantize(v.size, _ptr(v), _ptr(d), _ptr(q))
    return d, q


def forward(x, router_w, bias, gate, up, down, k: int, sel=None, idx_in=None, q8: bool = False):
    """Whole layer. Returns dict(out [n_sel][H] f64, idx, w, logits).

    sel: optional token list for the expert part (the router runs for all tokens).
    idx_in: optional [T][k] expert choice that replaces the top-k selection.
    q8: feed the experts' matvecs Q8_K-quantised activations (x rows and h; the router stays fp32).
    """
    x = np.ascontiguousarray(x, np.float32)
    router_w = np.ascontiguousarray(router_w, np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
    gate = np.ascontiguousarray(gate, np.uint8)
    up = np.ascontiguousarray(up, np.uint8)
    down = np.ascontiguousarray(down, np.uint8)
    T, H = x.shape
    E = router_w.shape[0]
    I = gate.shape[1]
    sel_a = None if sel is None else np.ascontiguousarray(sel, np.int32)
    n_sel = T if sel_a is None else int(sel_a.shape[0])
    idx_a = None if idx_in is None else np.ascontiguousarray(idx_in, np.int32)
    out = np.empty((n_sel, H), np.float64)
    idx = np.empty((T, k), np.int32)
    wts = np.empty((T, k), np.float64)
    logits = np.empty((T, E), np.float64)
    fn = load().mo_forward_q8 if q8 else load().mo_forward
    rc = fn(H, E, k, I, T, _ptr(x), _ptr(router_w), _ptr(bias), _ptr(gate), _ptr(up), _ptr(down),
                           _ptr(sel_a), n_sel, _ptr(idx_a), _ptr(out), _ptr(idx), _ptr(wts), _ptr(logits))
    if rc != 0:
        raise ValueError("oracle forward rejected its arguments or ran out of memory")
    return {"out": out, "idx": idx, "w": wts, "logits": logits}


def rms_norm(x, g, eps: float) -> np.ndarray:
    """Pre-FFN RMSNorm of fp32 rows x [T][H] with weight g [H]: float64 [T][H]."""
    x = np.ascontiguousarray(x, np.float32)
    g = np.ascontiguousarray(g, np.float32)
    T, H = x.shape
    y = np.empty((T, H), np.float64)
    load().mo_rms_norm(T, H, _ptr(x), _ptr(g), float(eps), _ptr(y))
    return y


def add_residual(hidden, ffn) -> np.ndarray:
    """hidden (fp32) + ffn (float64), in float64."""
    hidden = np.ascontiguousarray(hidden, np.float32)
    ffn = np.ascontiguousarray(ffn, np.float64)
    assert hidden.shape == ffn.shape
    out = np.empty(hidden.shape, np.float64)
    load().mo_add_residual(hidden.size, _ptr(hidden), _ptr(ffn), _ptr(out))
    return out


def block(hidden, norm_w, eps: float, router_w, bias, gate, up, down, k: int, sel=None):
    """The layer inside its block: out = hidden + layer(rms_norm(hidden)). The normalised rows enter the layer as
    fp32 (rounded to nearest), the type of the activation vectors the block passes between its steps.
    Returns forward()'s dict with out replaced by the block output (rows `sel` if given) and "xn" added."""
    hidden = np.ascontiguousarray(hidden, np.float32)
    xn = rms_norm(hidden, norm_w, eps).astype(np.float32)
    r = forward(xn, router_w, bias, gate, up, down, k, sel=sel)
    rows = hidden if sel is None else hidden[np.asarray(sel)]
    r["out"] = add_residual(rows, r["out"])
    r["xn"] = xn
    return r


STAT_FIELDS = ("n", "nan", "inf", "min", "max", "mean", "rms")


def stage_stats(v) -> np.ndarray:
    """Statistics of one stage's values (any shape, widened to float64): the 7 fields of STAT_FIELDS."""
    v = np.ascontiguousarray(np.asarray(v, np.float64).ravel())
    s = np.empty(7, np.float64)
    load().mo_stage_stats(v.size, _ptr(v), _ptr(s))
    return s
