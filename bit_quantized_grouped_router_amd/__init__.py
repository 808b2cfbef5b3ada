"""Python binding of libmoe_w4.so, the gfx950 int4-g64 grouped MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch provides device memory and the current stream. Functions have
the names of the C entry points (include/moe_w4.h). There is no CPU
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Dict, Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_w4.so")

GROUP = 64

EXPORTS = [
    "moe_route", "moe_block_m", "moe_tile_capacity", "moe_permute_workspace_bytes",
    "moe_permute", "moe_expert_gate_up_w4", "moe_expert_down_w4", "moe_expert_ffn_w4",
    "moe_unpermute_combine", "moe_layer_workspace_bytes", "moe_layer_forward",
    "moe_dequant_w4", "moe_status_string", "moe_last_hip_error", "moe_router_logits",
    "moe_layer_forward_hidden", "moe_route_permute", "moe_layer_forward_noalloc",
]


class MoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("f_shared", ctypes.c_int32)]


class MoeW4Matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p)]


class MoeW4Weights(ctypes.Structure):
    _fields_ = [("w13", MoeW4Matrix), ("w2", MoeW4Matrix), ("s13", MoeW4Matrix),
                ("s2", MoeW4Matrix)]


class MoeError(RuntimeError):
    pass


_lib: Optional[ctypes.CDLL] = None


def load(path: str) -> ctypes.CDLL:
    """Load a build of the library at ``path`` with the C signatures declared."""
    if not os.path.exists(path):
        raise MoeError(f"{path} is missing: build it with bit_quantized_grouped_router_amd.build")
    L = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(MoeDims)
    W = ctypes.POINTER(MoeW4Weights)
    sig = {
        "moe_route": ([P, I32, I32, I32, P, P, P], I32),
        "moe_block_m": ([], I32),
        "moe_tile_capacity": ([D], I32),
        "moe_permute_workspace_bytes": ([D], SZ),
        "moe_permute": ([D, P, P, P, P, P, P, P, P, SZ, P], I32),
        "moe_expert_gate_up_w4": ([D, P, W, P, P, P, P, P], I32),
        "moe_expert_down_w4": ([D, P, W, P, P, P, P, P], I32),
        "moe_expert_ffn_w4": ([D, P, W, P, P, P, P, P, P, P], I32),
        "moe_unpermute_combine": ([D, P, P, P, P, P, P], I32),
        "moe_layer_workspace_bytes": ([D], SZ),
        "moe_layer_forward": ([D, P, P, W, P, P, SZ, P], I32),
        "moe_layer_forward_noalloc": ([D, P, P, W, P, P], I32),
        "moe_router_logits": ([P, P, I32, I32, I32, P, P], I32),
        "moe_layer_forward_hidden": ([D, P, P, W, P, P, SZ, P], I32),
        "moe_route_permute": ([D, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "moe_dequant_w4": ([ctypes.POINTER(MoeW4Matrix), I32, I32, P, P], I32),
        "moe_status_string": ([I32], ctypes.c_char_p),
        "moe_last_hip_error": ([], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Route every entry point of this module through another build of the library
    (same ABI) inside the ``with`` block, then back to the one before."""
    global _lib
    prev = lib()
    _lib = load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        extra = f", hipError {lib().moe_last_hip_error()}" if status == -5 else ""
        raise MoeError(f"{what} failed: {msg} ({status}{extra})")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise MoeError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# element types the C ABI reads each kind of tensor as
BF16 = (torch.bfloat16, torch.int16)     # bf16 bit patterns (int16 storage allowed)
I32 = (torch.int32,)
F32 = (torch.float32,)
U8 = (torch.uint8, torch.int8)           # packed 4-bit codes, raw workspace bytes


def _need(t: Optional[torch.Tensor], nbytes: int, name: str, dtypes=None) -> None:
    """Raise unless tensor t holds at least nbytes bytes (and, if dtypes is given, has
    one of those element types). The kernels index their buffers from the dims alone
    and read each tensor as one fixed type, so a smaller tensor would be read or
    written past its end, and a tensor of another type would be reinterpreted."""
    if t is None:
        raise MoeError(f"{name} is missing")
    if dtypes is not None and t.dtype not in dtypes:
        raise MoeError(f"{name} has dtype {t.dtype}; expected one of "
                       f"{', '.join(str(d) for d in dtypes)}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise MoeError(f"{name} holds {have} bytes; these dims need {nbytes}")


def _need_weights(w: "W4Weights", dm: MoeDims) -> None:
    """Byte sizes of the four int4-g64 tensor sets for dims dm (see include/moe_w4.h)."""
    d, f, E = dm.d, dm.f, dm.E
    for name, n, rows, cols in (("w13", E, 2 * f, d), ("w2", E, d, f), ("s13", 1, 2 * f, d),
                                ("s2", 1, d, f)):
        m = getattr(w, name)
        _need(m.codes, n * rows * cols // 2, f"{name}.codes", U8)
        _need(m.scales, n * rows * (cols // GROUP) * 2, f"{name}.scales", BF16)
        _need(m.biases, n * rows * (cols // GROUP) * 2, f"{name}.biases", BF16)


def _need_map(dm: MoeDims, tile_map, num_tiles) -> None:
    _need(tile_map, moe_tile_capacity(dm) * 4 * 4, "tile_map", I32)
    _need(num_tiles, 4, "num_tiles", I32)


def _need_routing(dm: MoeDims, out: Dict) -> None:
    tk = dm.T * dm.k
    _need(out.get("counts"), dm.E * 4, "counts", I32)
    _need(out.get("offsets"), (dm.E + 1) * 4, "offsets", I32)
    _need(out.get("sorted_token"), tk * 4, "sorted_token", I32)
    _need(out.get("row_of"), tk * 4, "row_of", I32)
    _need_map(dm, out.get("tile_map"), out.get("num_tiles"))


def dims(T: int, d: int, f: int, E: int, k: int, f_shared: Optional[int] = None) -> MoeDims:
    """Layer shape; the shared expert's width defaults to f (the only width the kernels run)."""
    return MoeDims(T, d, f, E, k, f if f_shared is None else f_shared)


class W4Matrix:
    """One int4-g64 tensor set: codes uint8 [n, rows, cols/2], scales/biases bf16 [n, rows, cols/64]."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor):
        self.codes, self.scales, self.biases = codes, scales, biases

    def c(self, index: int = 0) -> MoeW4Matrix:
        """C view; index selects one matrix of the n stacked (for moe_dequant_w4)."""
        if index == 0:
            return MoeW4Matrix(_ptr(self.codes), _ptr(self.scales), _ptr(self.biases))
        return MoeW4Matrix(_ptr(self.codes) + index * self.codes[0].numel(),
                           _ptr(self.scales) + index * self.scales[0].numel() * 2,
                           _ptr(self.biases) + index * self.biases[0].numel() * 2)


class W4Weights:
    """The layer's four int4-g64 tensor sets (routed gate|up and down, shared gate|up and down)."""

    def __init__(self, w13: W4Matrix, w2: W4Matrix, s13: W4Matrix, s2: W4Matrix):
        self.w13, self.w2, self.s13, self.s2 = w13, w2, s13, s2

    def c(self) -> MoeW4Weights:
        return MoeW4Weights(self.w13.c(), self.w2.c(), self.s13.c(), self.s2.c())

    @staticmethod
    def from_numpy(weights: Dict[str, Dict], device="cuda") -> "W4Weights":
        def dev(a):
            t = torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a)
            return t.to(device)
        mats = {}
        for name in ("w13", "w2", "s13", "s2"):
            m = weights[name]
            mats[name] = W4Matrix(dev(m["codes"]), dev(m["scales"]), dev(m["biases"]))
        return W4Weights(**mats)


# ------------------------------------------------------------------ entry points

def moe_block_m() -> int:
    return lib().moe_block_m()


def moe_tile_capacity(dm: MoeDims) -> int:
    return lib().moe_tile_capacity(ctypes.byref(dm))


def moe_permute_workspace_bytes(dm: MoeDims) -> int:
    return lib().moe_permute_workspace_bytes(ctypes.byref(dm))


def moe_layer_workspace_bytes(dm: MoeDims) -> int:
    return lib().moe_layer_workspace_bytes(ctypes.byref(dm))


def moe_route(logits: torch.Tensor, k: int, topk_ids=None, topk_w=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _need(logits, T * E * 4, "logits", F32)
    _need(topk_ids, T * k * 4, "topk_ids", I32)
    _need(topk_w, T * k * 4, "topk_w", F32)
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _stream(stream)),
           "moe_route")
    return topk_ids, topk_w


def moe_permute(dm: MoeDims, topk_ids: torch.Tensor, out: Optional[Dict] = None, ws=None,
                stream=None) -> Dict[str, torch.Tensor]:
    dev = topk_ids.device
    tk = dm.T * dm.k
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"counts": torch.empty(dm.E, **i32), "offsets": torch.empty(dm.E + 1, **i32),
               "sorted_token": torch.empty(max(tk, 1), **i32),
               "row_of": torch.empty(max(tk, 1), **i32),
               "tile_map": torch.empty((max(moe_tile_capacity(dm), 1), 4), **i32),
               "num_tiles": torch.zeros(4, **i32)}
    nbytes = moe_permute_workspace_bytes(dm)
    if ws is None:
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _need(topk_ids, tk * 4, "topk_ids", I32)
    _need_routing(dm, out)
    _check(lib().moe_permute(ctypes.byref(dm), _ptr(topk_ids), _ptr(out["counts"]),
                             _ptr(out["offsets"]), _ptr(out["sorted_token"]),
                             _ptr(out["row_of"]), _ptr(out["tile_map"]), _ptr(out["num_tiles"]),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_permute")
    return out


def moe_route_permute(dm: MoeDims, logits: torch.Tensor, out: Optional[Dict] = None, ws=None,
                      stream=None) -> Dict[str, torch.Tensor]:
    """moe_route then moe_permute in one call; returns ids, wts and the permutation."""
    dev = logits.device
    tk = dm.T * dm.k
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"ids": torch.empty((dm.T, dm.k), **i32),
               "wts": torch.empty((dm.T, dm.k), dtype=torch.float32, device=dev),
               "counts": torch.empty(dm.E, **i32), "offsets": torch.empty(dm.E + 1, **i32),
               "sorted_token": torch.empty(max(tk, 1), **i32),
               "row_of": torch.empty(max(tk, 1), **i32),
               "tile_map": torch.empty((max(moe_tile_capacity(dm), 1), 4), **i32),
               "num_tiles": torch.zeros(4, **i32)}
    if ws is None:
        ws = torch.empty(max(moe_permute_workspace_bytes(dm), 16), dtype=torch.uint8, device=dev)
    _need(logits, dm.T * dm.E * 4, "logits", F32)
    _need(out.get("ids"), tk * 4, "ids", I32)
    _need(out.get("wts"), tk * 4, "wts", F32)
    _need_routing(dm, out)
    _check(lib().moe_route_permute(ctypes.byref(dm), _ptr(logits), _ptr(out["ids"]),
                                   _ptr(out["wts"]), _ptr(out["counts"]), _ptr(out["offsets"]),
                                   _ptr(out["sorted_token"]), _ptr(out["row_of"]),
                                   _ptr(out["tile_map"]), _ptr(out["num_tiles"]), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "moe_route_permute")
    return out


def moe_expert_gate_up_w4(dm: MoeDims, x: torch.Tensor, w: W4Weights, sorted_token, tile_map,
                          num_tiles, h=None, stream=None):
    if h is None:
        h = torch.empty((dm.T * dm.k + dm.T, dm.f), dtype=torch.bfloat16, device=x.device)
    rows = dm.T * dm.k + dm.T
    _need(x, dm.T * dm.d * 2, "x", BF16)
    _need(sorted_token, dm.T * dm.k * 4, "sorted_token", I32)
    _need_map(dm, tile_map, num_tiles)
    _need(h, rows * dm.f * 2, "h", BF16)
    _need_weights(w, dm)
    _check(lib().moe_expert_gate_up_w4(ctypes.byref(dm), _ptr(x), ctypes.byref(w.c()),
                                       _ptr(sorted_token), _ptr(tile_map), _ptr(num_tiles),
                                       _ptr(h), _stream(stream)), "moe_expert_gate_up_w4")
    return h


def moe_expert_down_w4(dm: MoeDims, h: torch.Tensor, w: W4Weights, tile_map, num_tiles,
                       o_routed=None, o_shared=None, stream=None):
    dev = h.device
    if o_routed is None:
        o_routed = torch.empty((max(dm.T * dm.k, 1), dm.d), dtype=torch.bfloat16, device=dev)
    if o_shared is None:
        o_shared = torch.empty((max(dm.T, 1), dm.d), dtype=torch.float32, device=dev)
    _need(h, (dm.T * dm.k + dm.T) * dm.f * 2, "h", BF16)
    _need_map(dm, tile_map, num_tiles)
    _need(o_routed, dm.T * dm.k * dm.d * 2, "o_routed", BF16)
    _need(o_shared, dm.T * dm.d * 4, "o_shared", F32)
    _need_weights(w, dm)
    _check(lib().moe_expert_down_w4(ctypes.byref(dm), _ptr(h), ctypes.byref(w.c()),
                                    _ptr(tile_map), _ptr(num_tiles), _ptr(o_routed),
                                    _ptr(o_shared), _stream(stream)), "moe_expert_down_w4")
    return o_routed, o_shared


def moe_expert_ffn_w4(dm: MoeDims, x: torch.Tensor, w: W4Weights, sorted_token, tile_map,
                      num_tiles, h=None, o_routed=None, o_shared=None, stream=None):
    dev = x.device
    if h is None:
        h = torch.empty((dm.T * dm.k + dm.T, dm.f), dtype=torch.bfloat16, device=dev)
    if o_routed is None:
        o_routed = torch.empty((max(dm.T * dm.k, 1), dm.d), dtype=torch.bfloat16, device=dev)
    if o_shared is None:
        o_shared = torch.empty((max(dm.T, 1), dm.d), dtype=torch.float32, device=dev)
    _need(x, dm.T * dm.d * 2, "x", BF16)
    _need(sorted_token, dm.T * dm.k * 4, "sorted_token", I32)
    _need_map(dm, tile_map, num_tiles)
    _need(h, (dm.T * dm.k + dm.T) * dm.f * 2, "h", BF16)
    _need(o_routed, dm.T * dm.k * dm.d * 2, "o_routed", BF16)
    _need(o_shared, dm.T * dm.d * 4, "o_shared", F32)
    _need_weights(w, dm)
    _check(lib().moe_expert_ffn_w4(ctypes.byref(dm), _ptr(x), ctypes.byref(w.c()),
                                   _ptr(sorted_token), _ptr(tile_map), _ptr(num_tiles), _ptr(h),
                                   _ptr(o_routed), _ptr(o_shared), _stream(stream)),
           "moe_expert_ffn_w4")
    return h, o_routed, o_shared


def moe_unpermute_combine(dm: MoeDims, o_routed, o_shared, topk_w, row_of, y=None, stream=None):
    if y is None:
        y = torch.empty((dm.T, dm.d), dtype=torch.float32, device=o_shared.device)
    _need(o_routed, dm.T * dm.k * dm.d * 2, "o_routed", BF16)
    _need(o_shared, dm.T * dm.d * 4, "o_shared", F32)
    _need(topk_w, dm.T * dm.k * 4, "topk_w", F32)
    _need(row_of, dm.T * dm.k * 4, "row_of", I32)
    _need(y, dm.T * dm.d * 4, "y", F32)
    _check(lib().moe_unpermute_combine(ctypes.byref(dm), _ptr(o_routed), _ptr(o_shared),
                                       _ptr(topk_w), _ptr(row_of), _ptr(y), _stream(stream)),
           "moe_unpermute_combine")
    return y


def moe_layer_forward(dm: MoeDims, x: torch.Tensor, logits: torch.Tensor, w: W4Weights,
                      y=None, ws=None, stream=None, wc: Optional[MoeW4Weights] = None):
    """One layer call. ``wc`` may hold a prebuilt C weight struct (saves marshalling in loops)."""
    if y is None:
        y = torch.empty((dm.T, dm.d), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_layer_workspace_bytes(dm), 16), dtype=torch.uint8, device=x.device)
    _need(x, dm.T * dm.d * 2, "x", BF16)
    _need(logits, dm.T * dm.E * 4, "logits", F32)
    _need(y, dm.T * dm.d * 4, "y", F32)
    if wc is None:  # a prebuilt struct (wc) is the caller's to size
        _need_weights(w, dm)
    wc = w.c() if wc is None else wc
    _check(lib().moe_layer_forward(ctypes.byref(dm), _ptr(x), _ptr(logits), ctypes.byref(wc),
                                   _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_layer_forward")
    return y


def moe_layer_forward_noalloc(dm: MoeDims, x: torch.Tensor, logits: torch.Tensor, w: W4Weights,
                              y: torch.Tensor, stream=None, wc: Optional[MoeW4Weights] = None):
    """One layer call with the library's own device scratch (no workspace, nothing
    allocated by the call: y must be given)."""
    _need(x, dm.T * dm.d * 2, "x", BF16)
    _need(logits, dm.T * dm.E * 4, "logits", F32)
    _need(y, dm.T * dm.d * 4, "y", F32)
    if wc is None:  # a prebuilt struct (wc) is the caller's to size
        _need_weights(w, dm)
    wc = w.c() if wc is None else wc
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(dm), _ptr(x), _ptr(logits),
                                           ctypes.byref(wc), _ptr(y), _stream(stream)),
           "moe_layer_forward_noalloc")
    return y


def moe_router_logits(x: torch.Tensor, w_router: torch.Tensor, logits=None, stream=None):
    """logits [T, E] fp32 = x [T, d] (bf16) times w_router [E, d] (bf16) transposed."""
    if x.dim() != 2 or w_router.dim() != 2:
        raise MoeError("x and w_router must be 2-D: [T, d] and [E, d]")
    T, d = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != d:
        raise MoeError(f"w_router has {w_router.shape[1]} columns; x has d = {d}")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _need(x, T * d * 2, "x", BF16)
    _need(w_router, E * d * 2, "w_router", BF16)
    _need(logits, T * E * 4, "logits", F32)
    _check(lib().moe_router_logits(_ptr(x), _ptr(w_router), T, d, E, _ptr(logits),
                                   _stream(stream)), "moe_router_logits")
    return logits


def moe_layer_forward_hidden(dm: MoeDims, x: torch.Tensor, w_router: torch.Tensor, w: W4Weights,
                             y=None, ws=None, stream=None, wc: Optional[MoeW4Weights] = None):
    """One layer call from hidden states (router projection included)."""
    if y is None:
        y = torch.empty((dm.T, dm.d), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_layer_workspace_bytes(dm), 16), dtype=torch.uint8, device=x.device)
    _need(x, dm.T * dm.d * 2, "x", BF16)
    _need(w_router, dm.E * dm.d * 2, "w_router", BF16)
    _need(y, dm.T * dm.d * 4, "y", F32)
    if wc is None:  # a prebuilt struct (wc) is the caller's to size
        _need_weights(w, dm)
    wc = w.c() if wc is None else wc
    _check(lib().moe_layer_forward_hidden(ctypes.byref(dm), _ptr(x), _ptr(w_router),
                                          ctypes.byref(wc), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)), "moe_layer_forward_hidden")
    return y


def moe_dequant_w4(m: W4Matrix, index: int = 0, out=None, stream=None):
    rows = m.codes.shape[-2]
    cols = m.codes.shape[-1] * 2
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=m.codes.device)
    n = m.codes.shape[0] if m.codes.dim() == 3 else 1
    if not 0 <= index < n:
        raise MoeError(f"matrix index {index} outside 0..{n - 1}")
    _need(m.codes, n * rows * cols // 2, "codes", U8)
    _need(m.scales, n * rows * (cols // GROUP) * 2, "scales", BF16)
    _need(m.biases, n * rows * (cols // GROUP) * 2, "biases", BF16)
    _need(out, rows * cols * 2, "out", BF16)
    cm = m.c(index)
    _check(lib().moe_dequant_w4(ctypes.byref(cm), rows, cols, _ptr(out), _stream(stream)),
           "moe_dequant_w4")
    return out
