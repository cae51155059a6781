"""Python binding of the fmoe C-ABI library (libfmoe.so, gfx950).

Argument marshalling only: every computation runs in the library's HIP kernels. The
functions keep the C names without the ``fmoe_`` prefix. Device buffers may be given as
torch tensors (their ``data_ptr()`` is passed) or as raw integer device addresses;
``stream=None`` means torch's current stream on the current device. A non-zero status
raises :class:`FmoeError`. If ``libfmoe.so`` is missing the import of the library fails
loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_HERE, "libfmoe.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_BITS, ERR_GROUP, ERR_K, ERR_ALIGN = -1, -2, -3, -4, -5, -6
ERR_WORKSPACE, ERR_HIP, ERR_INTERNAL, ERR_DEVICE, ERR_OVERLAP, ERR_SCRATCH = -7, -8, -9, -10, -11, -12
PRENORM = 1
RESET_SCRATCH = 2
OP_EXPERT_FFN, OP_MOE_LAYER = 1, 2

EXPORTS = ("fmoe_status_string", "fmoe_version", "fmoe_codes_bytes", "fmoe_sb_bytes", "fmoe_expert_bytes",
           "fmoe_expert_view", "fmoe_pack", "fmoe_workspace_bytes", "fmoe_dequant_matvec",
           "fmoe_dequant_matvec_multi", "fmoe_route_topk", "fmoe_expert_ffn", "fmoe_moe_layer", "fmoe_batched_a16",
           "fmoe_workspace_error", "fmoe_moe_layer_noalloc")


class FmoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("sb", ctypes.c_void_p), ("rows", ctypes.c_int),
                ("cols", ctypes.c_int), ("bits", ctypes.c_int), ("group", ctypes.c_int)]


class Expert(ctypes.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class Layer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("experts", ctypes.c_void_p), ("expert_stride", ctypes.c_size_t),
                ("n_experts", ctypes.c_int), ("hidden", ctypes.c_int), ("inter", ctypes.c_int),
                ("bits", ctypes.c_int), ("group", ctypes.c_int), ("shared_gate", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libfmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        _lib = load(SO_PATH)
    return _lib


def use(library) -> None:
    """Route this module's calls to another build of the library (the same C-ABI), e.g. the
    phase-traced build that the measurement package makes; ``load`` gives such a handle."""
    global _lib
    _lib = library


def load(path: str):
    """ctypes handle of a build of the library at `path`, with every export's signature."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no non-HIP fallback")
    L = ctypes.CDLL(path)
    vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint
    L.fmoe_status_string.restype = ctypes.c_char_p
    L.fmoe_status_string.argtypes = [i32]
    L.fmoe_version.restype = ctypes.c_char_p
    L.fmoe_version.argtypes = []
    L.fmoe_codes_bytes.restype = sz
    L.fmoe_codes_bytes.argtypes = [i32, i32, i32]
    L.fmoe_sb_bytes.restype = sz
    L.fmoe_sb_bytes.argtypes = [i32, i32, i32]
    L.fmoe_expert_bytes.restype = sz
    L.fmoe_expert_bytes.argtypes = [i32, i32, i32, i32]
    L.fmoe_expert_view.restype = i32
    L.fmoe_expert_view.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(Expert)]
    L.fmoe_pack.restype = i32
    L.fmoe_pack.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.fmoe_workspace_bytes.restype = sz
    L.fmoe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.fmoe_dequant_matvec.restype = i32
    L.fmoe_dequant_matvec.argtypes = [ctypes.POINTER(QMat), vp, vp, i32, vp]
    L.fmoe_dequant_matvec_multi.restype = i32
    L.fmoe_dequant_matvec_multi.argtypes = [ctypes.POINTER(QMat), i32, vp, ctypes.POINTER(vp), i32, vp]
    L.fmoe_route_topk.restype = i32
    L.fmoe_route_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.fmoe_expert_ffn.restype = i32
    L.fmoe_expert_ffn.argtypes = [ctypes.POINTER(Expert), vp, vp, vp, sz, vp]
    L.fmoe_moe_layer.restype = i32
    L.fmoe_moe_layer.argtypes = [ctypes.POINTER(Layer), i32, vp, vp, i32, i32, ctypes.c_float, u32, vp, vp, vp,
                                 sz, vp]
    L.fmoe_moe_layer_noalloc.restype = i32
    L.fmoe_moe_layer_noalloc.argtypes = [ctypes.POINTER(Layer), i32, vp, vp, i32, i32, ctypes.c_float, u32, vp,
                                         vp, vp]
    L.fmoe_workspace_error.restype = i32
    L.fmoe_workspace_error.argtypes = [vp, sz, vp, vp]
    L.fmoe_batched_a16.restype = i32
    L.fmoe_batched_a16.argtypes = [vp, sz, i32, i32, i32, i32, i32, i32, vp, vp]
    return L


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise FmoeError(rc, what)


def status_string(status: int) -> str:
    return lib().fmoe_status_string(status).decode()


def version() -> str:
    return lib().fmoe_version().decode()


def codes_bytes(rows: int, cols: int, bits: int) -> int:
    return int(lib().fmoe_codes_bytes(rows, cols, bits))


def sb_bytes(rows: int, cols: int, group: int = 64) -> int:
    return int(lib().fmoe_sb_bytes(rows, cols, group))


def expert_bytes(hidden: int, inter: int, bits: int, group: int = 64) -> int:
    return int(lib().fmoe_expert_bytes(hidden, inter, bits, group))


def qmat(codes, sb, rows: int, cols: int, bits: int, group: int = 64) -> QMat:
    return QMat(_ptr(codes), _ptr(sb), rows, cols, bits, group)


def expert_view(blob, hidden: int, inter: int, bits: int, group: int = 64) -> Expert:
    e = Expert()
    _check(lib().fmoe_expert_view(_ptr(blob), hidden, inter, bits, group, ctypes.byref(e)), "fmoe_expert_view")
    return e


def pack(codes_canon, scale, bias, rows, cols, bits, group, codes_out, sb_out, stream=None) -> None:
    _check(lib().fmoe_pack(_ptr(codes_canon), _ptr(scale), _ptr(bias), rows, cols, bits, group, _ptr(codes_out),
                           _ptr(sb_out), _stream(stream)), "fmoe_pack")


def workspace_bytes(op: int, n_tokens: int, hidden: int, inter: int, n_experts: int, k: int) -> int:
    return int(lib().fmoe_workspace_bytes(op, n_tokens, hidden, inter, n_experts, k))


def dequant_matvec(W: QMat, x, y, n_vec: int = 1, stream=None) -> None:
    _check(lib().fmoe_dequant_matvec(ctypes.byref(W), _ptr(x), _ptr(y), n_vec, _stream(stream)),
           "fmoe_dequant_matvec")


def dequant_matvec_multi(Ws, x, ys, n_vec: int = 1, stream=None) -> None:
    """Ws: list of QMat (equal cols and bits); ys: list of output tensors, one per matrix."""
    if len(Ws) != len(ys):
        raise ValueError("one output per matrix")
    mats = (QMat * max(1, len(Ws)))(*Ws)
    outs = (ctypes.c_void_p * max(1, len(ys)))(*[_ptr(y) for y in ys])
    _check(lib().fmoe_dequant_matvec_multi(mats, len(Ws), _ptr(x), outs, n_vec, _stream(stream)),
           "fmoe_dequant_matvec_multi")


def route_topk(router, x, n_tokens, n_experts, hidden, k, idx, w, logits, stream=None) -> None:
    _check(lib().fmoe_route_topk(_ptr(router), _ptr(x), n_tokens, n_experts, hidden, k, _ptr(idx), _ptr(w),
                                 _ptr(logits), _stream(stream)), "fmoe_route_topk")


def expert_ffn(e: Expert, x, y, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().fmoe_expert_ffn(ctypes.byref(e), _ptr(x), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "fmoe_expert_ffn")


def layers_array(layers) -> ctypes.Array:
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L
    return arr


def moe_layer(layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, ws, ws_bytes, stream=None) -> None:
    """layers: a ctypes Layer array (see layers_array) or a list of Layer."""
    if not isinstance(layers, ctypes.Array):
        layers = layers_array(layers)
    _check(lib().fmoe_moe_layer(layers, len(layers), _ptr(x_in), _ptr(h_out), n_tokens, k, eps, flags, _ptr(idx_out),
                                _ptr(w_out), _ptr(ws), ws_bytes, _stream(stream)), "fmoe_moe_layer")


def moe_layer_noalloc(layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, stream=None) -> None:
    """fmoe_moe_layer on the library's static scratch (no workspace argument)."""
    if not isinstance(layers, ctypes.Array):
        layers = layers_array(layers)
    _check(lib().fmoe_moe_layer_noalloc(layers, len(layers), _ptr(x_in), _ptr(h_out), n_tokens, k, eps, flags,
                                        _ptr(idx_out), _ptr(w_out), _stream(stream)), "fmoe_moe_layer_noalloc")


def batched_a16(ws, ws_bytes, n_tokens, hidden, inter, n_experts, k, bits, a16_out, stream=None) -> None:
    """bf16 SwiGLU outputs [n_tokens][k][inter] of the last batched fmoe_moe_layer call on ws."""
    _check(lib().fmoe_batched_a16(_ptr(ws), ws_bytes, n_tokens, hidden, inter, n_experts, k, bits, _ptr(a16_out),
                                  _stream(stream)), "fmoe_batched_a16")


def workspace_error(ws, ws_bytes, err_out, stream=None) -> None:
    """Copy the workspace's error word (non-zero once a device-side wait gave up) into the
    device uint32 err_out."""
    _check(lib().fmoe_workspace_error(_ptr(ws), ws_bytes, _ptr(err_out), _stream(stream)), "fmoe_workspace_error")
