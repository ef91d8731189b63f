"""ctypes binding of the C ABI in include/moe_ffn.h.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their device pointers and the current HIP stream are passed
through. Every step of the layer runs in the HIP kernels of libmoe_ffn.so;
there is no other implementation behind these names, and importing this
module fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .build import LIB

if not os.path.exists(LIB):
    raise ImportError(f"{LIB} is missing: build it first (python -m quantized_moe_wave_amd.build)")

_lib = ctypes.CDLL(LIB)

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_SHAPE", 2: "MOE_ERR_INVALID_ARG", 3: "MOE_ERR_BLOB_SIZE",
                4: "MOE_ERR_DEVICE", 5: "MOE_ERR_OOM"}


class MoeFfnShape(ctypes.Structure):
    _fields_ = [("hidden_dim", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_experts_per_tok", ctypes.c_int32), ("moe_intermediate", ctypes.c_int32)]


_vp = ctypes.c_void_p
_lib.moe_ffn_create.argtypes = [ctypes.POINTER(MoeFfnShape), _vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp,
                                ctypes.c_size_t, _vp, _vp, _vp, ctypes.POINTER(_vp)]
_lib.moe_ffn_create.restype = ctypes.c_int
_lib.moe_ffn_reserve.argtypes = [_vp, ctypes.c_int32, _vp]
_lib.moe_ffn_reserve.restype = ctypes.c_int
_lib.moe_ffn_forward.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
_lib.moe_ffn_forward.restype = ctypes.c_int
_lib.moe_ffn_forward_noalloc.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
_lib.moe_ffn_forward_noalloc.restype = ctypes.c_int
_lib.moe_ffn_forward_q8.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
_lib.moe_ffn_forward_q8.restype = ctypes.c_int
_lib.moe_ffn_set_norm.argtypes = [_vp, _vp, ctypes.c_float, _vp]
_lib.moe_ffn_set_norm.restype = ctypes.c_int
_lib.moe_ffn_forward_block.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
_lib.moe_ffn_forward_block.restype = ctypes.c_int
_lib.moe_ffn_debug_stats.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp]
_lib.moe_ffn_debug_stats.restype = ctypes.c_int
_lib.moe_ffn_debug_routing.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
_lib.moe_ffn_debug_routing.restype = ctypes.c_int
_lib.moe_ffn_destroy.argtypes = [_vp]
_lib.moe_ffn_destroy.restype = ctypes.c_int
_lib.moe_ffn_last_error.argtypes = []
_lib.moe_ffn_last_error.restype = ctypes.c_char_p
_lib.moe_ffn_abi_version.argtypes = []
_lib.moe_ffn_abi_version.restype = ctypes.c_int32
_lib.moe_ffn_profile.argtypes = [_vp, ctypes.c_uint32]
_lib.moe_ffn_profile.restype = ctypes.c_int
_lib.moe_ffn_profile_read.argtypes = [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
_lib.moe_ffn_profile_read.restype = ctypes.c_int
_lib.moe_ffn_stage_count.argtypes = []
_lib.moe_ffn_stage_count.restype = ctypes.c_int32
_lib.moe_ffn_stage_name.argtypes = [ctypes.c_int32]
_lib.moe_ffn_stage_name.restype = ctypes.c_char_p


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.moe_ffn_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def lib() -> ctypes.CDLL:
    return _lib


def abi_version() -> int:
    return int(_lib.moe_ffn_abi_version())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def moe_ffn_create(hidden_dim: int, num_experts: int, num_experts_per_tok: int, moe_intermediate: int,
                   gate_q4k: torch.Tensor, up_q4k: torch.Tensor, down_q4k: torch.Tensor,
                   router_w: torch.Tensor, router_bias: torch.Tensor | None = None, stream=None) -> int:
    """Return an opaque handle (int). Weights: uint8 blobs and fp32 router tensors on the GPU."""
    for n, t in (("gate_q4k", gate_q4k), ("up_q4k", up_q4k), ("down_q4k", down_q4k)):
        _dev(t, n, torch.uint8)
    _dev(router_w, "router_w", torch.float32)
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32)
    shape = MoeFfnShape(hidden_dim, num_experts, num_experts_per_tok, moe_intermediate)
    out = _vp()
    st = _lib.moe_ffn_create(ctypes.byref(shape), _ptr(gate_q4k), gate_q4k.numel(), _ptr(up_q4k), up_q4k.numel(),
                             _ptr(down_q4k), down_q4k.numel(), _ptr(router_w), _ptr(router_bias), _stream(stream),
                             ctypes.byref(out))
    _check(st, "moe_ffn_create")
    return out.value


def moe_ffn_reserve(handle: int, max_tokens: int, stream=None) -> None:
    _check(_lib.moe_ffn_reserve(_vp(handle), int(max_tokens), _stream(stream)), "moe_ffn_reserve")


def moe_ffn_forward(handle: int, x: torch.Tensor, out: torch.Tensor, router_out: torch.Tensor | None = None,
                    router_idx: torch.Tensor | None = None, stream=None) -> None:
    """out[T][H] <- MoE FFN of x[T][H]; router_out/router_idx [T][k] optional."""
    _dev(x, "x", torch.float32)
    _dev(out, "out", torch.float32)
    if x.dim() != 2 or out.shape != x.shape:
        raise ValueError("x and out must both be [T, hidden_dim]")
    if router_out is not None:
        _dev(router_out, "router_out", torch.float32)
    if router_idx is not None:
        _dev(router_idx, "router_idx", torch.int32)
    st = _lib.moe_ffn_forward(_vp(handle), int(x.shape[0]), _ptr(x), _ptr(out), _ptr(router_out), _ptr(router_idx),
                              _stream(stream))
    _check(st, "moe_ffn_forward")


def moe_ffn_forward_noalloc(handle: int, x: torch.Tensor, out: torch.Tensor, router_out: torch.Tensor | None = None,
                            router_idx: torch.Tensor | None = None, stream=None) -> None:
    """moe_ffn_forward on the library's fixed per-device scratch: allocates nothing (T limited by the scratch)."""
    _dev(x, "x", torch.float32)
    _dev(out, "out", torch.float32)
    if x.dim() != 2 or out.shape != x.shape:
        raise ValueError("x and out must both be [T, hidden_dim]")
    if router_out is not None:
        _dev(router_out, "router_out", torch.float32)
    if router_idx is not None:
        _dev(router_idx, "router_idx", torch.int32)
    st = _lib.moe_ffn_forward_noalloc(_vp(handle), int(x.shape[0]), _ptr(x), _ptr(out), _ptr(router_out),
                                      _ptr(router_idx), _stream(stream))
    _check(st, "moe_ffn_forward_noalloc")


def moe_ffn_forward_q8(handle: int, x: torch.Tensor, out: torch.Tensor, router_out: torch.Tensor | None = None,
                       router_idx: torch.Tensor | None = None, stream=None) -> None:
    """out[T][H] <- MoE FFN of x with Q8_K-style int8 expert activations (codes and a scale per 256 values)."""
    _dev(x, "x", torch.float32)
    _dev(out, "out", torch.float32)
    if x.dim() != 2 or out.shape != x.shape:
        raise ValueError("x and out must both be [T, hidden_dim]")
    if router_out is not None:
        _dev(router_out, "router_out", torch.float32)
    if router_idx is not None:
        _dev(router_idx, "router_idx", torch.int32)
    st = _lib.moe_ffn_forward_q8(_vp(handle), int(x.shape[0]), _ptr(x), _ptr(out), _ptr(router_out),
                                 _ptr(router_idx), _stream(stream))
    _check(st, "moe_ffn_forward_q8")


def moe_ffn_set_norm(handle: int, norm_w: torch.Tensor, eps: float, stream=None) -> None:
    """Pre-FFN RMSNorm weight [hidden_dim] fp32 (CPU or GPU tensor; copied) and eps of moe_ffn_forward_block."""
    if norm_w.dtype != torch.float32 or not norm_w.is_contiguous() or norm_w.dim() != 1:
        raise TypeError("norm_w must be a contiguous 1-D float32 tensor")
    st = _lib.moe_ffn_set_norm(_vp(handle), _vp(norm_w.data_ptr()), float(eps), _stream(stream))
    _check(st, "moe_ffn_set_norm")


def moe_ffn_forward_block(handle: int, hidden: torch.Tensor, out: torch.Tensor,
                          router_out: torch.Tensor | None = None, router_idx: torch.Tensor | None = None,
                          stream=None) -> None:
    """out[T][H] <- hidden + MoE FFN of rms_norm(hidden); router_out/router_idx [T][k] optional."""
    _dev(hidden, "hidden", torch.float32)
    _dev(out, "out", torch.float32)
    if hidden.dim() != 2 or out.shape != hidden.shape:
        raise ValueError("hidden and out must both be [T, hidden_dim]")
    if router_out is not None:
        _dev(router_out, "router_out", torch.float32)
    if router_idx is not None:
        _dev(router_idx, "router_idx", torch.int32)
    st = _lib.moe_ffn_forward_block(_vp(handle), int(hidden.shape[0]), _ptr(hidden), _ptr(out), _ptr(router_out),
                                    _ptr(router_idx), _stream(stream))
    _check(st, "moe_ffn_forward_block")


def moe_ffn_debug_routing(handle: int, logits: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                          offsets: torch.Tensor | None = None, entries: torch.Tensor | None = None,
                          stream=None) -> None:
    for n, t, dt in (("logits", logits, torch.float64), ("counts", counts, torch.int32),
                     ("offsets", offsets, torch.int32), ("entries", entries, torch.int32)):
        if t is not None:
            _dev(t, n, dt)
    st = _lib.moe_ffn_debug_routing(_vp(handle), _ptr(logits), _ptr(counts), _ptr(offsets), _ptr(entries),
                                    _stream(stream))
    _check(st, "moe_ffn_debug_routing")


STAT_STAGES = ("router_logits", "router_weights", "swiglu_h", "output")
STAT_FIELDS = ("n", "nan", "inf", "min", "max", "mean", "rms")


def moe_ffn_debug_stats(handle: int, token: int, out: torch.Tensor, router_out: torch.Tensor | None = None,
                        stats: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Per-stage statistics [4][7] float64 (STAT_STAGES x STAT_FIELDS) of one token of the last forward. out and
    router_out: the buffers that forward wrote (router_out None if it was given none)."""
    _dev(out, "out", torch.float32)
    if router_out is not None:
        _dev(router_out, "router_out", torch.float32)
    if stats is None:
        stats = torch.empty((len(STAT_STAGES), len(STAT_FIELDS)), dtype=torch.float64, device=out.device)
    _dev(stats, "stats", torch.float64)
    if stats.numel() < len(STAT_STAGES) * len(STAT_FIELDS):
        raise ValueError("stats must hold 4 x 7 values")
    st = _lib.moe_ffn_debug_stats(_vp(handle), int(token), _ptr(out), _ptr(router_out), _ptr(stats),
                                  _stream(stream))
    _check(st, "moe_ffn_debug_stats")
    return stats


def moe_ffn_stage_names() -> list[str]:
    return [_lib.moe_ffn_stage_name(i).decode() for i in range(_lib.moe_ffn_stage_count())]


def moe_ffn_profile(handle: int, stages) -> None:
    """Bracket the named stages (or stage indices) of every forward with HIP events."""
    names = moe_ffn_stage_names()
    mask = 0
    for s in stages:
        mask |= 1 << (names.index(s) if isinstance(s, str) else int(s))
    _check(_lib.moe_ffn_profile(_vp(handle), mask), "moe_ffn_profile")


def moe_ffn_profile_read(handle: int) -> dict:
    """{stage name: (total ms, launches)} since the last read."""
    n = _lib.moe_ffn_stage_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(_lib.moe_ffn_profile_read(_vp(handle), ms, cnt), "moe_ffn_profile_read")
    return {name: (ms[i], cnt[i]) for i, name in enumerate(moe_ffn_stage_names())}


def moe_ffn_destroy(handle: int) -> None:
    _check(_lib.moe_ffn_destroy(_vp(handle)), "moe_ffn_destroy")


class MoeFfn:
    """Owning wrapper: one layer's weights on the GPU plus its workspace."""

    def __init__(self, hidden_dim, num_experts, num_experts_per_tok, moe_intermediate, gate_q4k, up_q4k, down_q4k,
                 router_w, router_bias=None, stream=None):
        self.hidden_dim = hidden_dim
        self.num_experts = num_experts
        self.top_k = num_experts_per_tok
        self.moe_intermediate = moe_intermediate
        self.handle = moe_ffn_create(hidden_dim, num_experts, num_experts_per_tok, moe_intermediate, gate_q4k,
                                     up_q4k, down_q4k, router_w, router_bias, stream)

    @classmethod
    def from_host(cls, hidden_dim, num_experts, num_experts_per_tok, moe_intermediate, gate_q4k, up_q4k, down_q4k,
                  router_w, router_bias=None, device="cuda", stream=None):
        """Create the layer from host arrays (numpy or CPU tensors): the Q4_K blobs as uint8 bytes, the router
        weight and bias as float32. They are copied to the device for moe_ffn_create, which copies them again into
        the layer's own layout; the uploads are released when this returns."""
        def up(a, dt):
            t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
            if t.dtype != dt:
                raise TypeError(f"expected {dt}, got {t.dtype}")
            return t.reshape(-1).to(device) if dt == torch.uint8 else t.contiguous().to(device)

        g, u, d = up(gate_q4k, torch.uint8), up(up_q4k, torch.uint8), up(down_q4k, torch.uint8)
        rw = up(router_w, torch.float32)
        rb = None if router_bias is None else up(router_bias, torch.float32)
        layer = cls(hidden_dim, num_experts, num_experts_per_tok, moe_intermediate, g, u, d, rw, rb, stream)
        (torch.cuda.current_stream() if stream is None else stream).synchronize()
        return layer

    def reserve(self, max_tokens: int, stream=None) -> None:
        moe_ffn_reserve(self.handle, max_tokens, stream)

    def forward(self, x, out=None, router_out=None, router_idx=None, stream=None):
        if out is None:
            out = torch.empty_like(x)
        moe_ffn_forward(self.handle, x, out, router_out, router_idx, stream)
        return out

    def forward_noalloc(self, x, out, router_out=None, router_idx=None, stream=None):
        moe_ffn_forward_noalloc(self.handle, x, out, router_out, router_idx, stream)
        return out

    def forward_q8(self, x, out=None, router_out=None, router_idx=None, stream=None):
        if out is None:
            out = torch.empty_like(x)
        moe_ffn_forward_q8(self.handle, x, out, router_out, router_idx, stream)
        return out

    def set_norm(self, norm_w, eps: float, stream=None) -> None:
        moe_ffn_set_norm(self.handle, norm_w, eps, stream)

    def forward_block(self, hidden, out=None, router_out=None, router_idx=None, stream=None):
        if out is None:
            out = torch.empty_like(hidden)
        moe_ffn_forward_block(self.handle, hidden, out, router_out, router_idx, stream)
        return out

    def close(self) -> None:
        if self.handle:
            moe_ffn_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
