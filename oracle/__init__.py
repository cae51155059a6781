"""CPU oracle of the per-token MoE expert block -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The fmoe library never calls it and shares no
code with it. The arithmetic lives in ``oracle.c`` (plain loops, fp64); this file only
marshals numpy arrays through ctypes.

Parity status of every function is pinned by ``tests/test_oracle_pins.py`` (brute force,
closed forms, invariants); see the docstrings there for which pin covers what.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

PROVIDER_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                               ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                               ctypes.POINTER(ctypes.c_void_p))


def build() -> str:
    """Compile liboracle.so with gcc (always recompiles). No fused multiply-add contraction."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-shared", "-fPIC",
           os.path.join(_HERE, "oracle.c"), "-o", _SO, "-lm"]
    subprocess.run(cmd, check=True)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        i32, vp, dbl = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.oracle_code.restype = i32
        L.oracle_code.argtypes = [vp, i32, i32, i32, i32]
        L.oracle_weight.restype = dbl
        L.oracle_weight.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_matvec.restype = None
        L.oracle_matvec.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
        L.oracle_route.restype = None
        L.oracle_route.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [vp, i32, dbl, vp]
        L.oracle_swiglu.restype = dbl
        L.oracle_swiglu.argtypes = [dbl, dbl]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.oracle_moe_layer.restype = i32
        L.oracle_moe_layer.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl,
                                       vp, vp, vp, vp, vp, vp]
        L.oracle_stack.restype = i32
        L.oracle_stack.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, dbl, dbl,
                                   vp, vp, vp, vp, vp, vp, vp]
        L.oracle_round_bf16.restype = dbl
        L.oracle_round_bf16.argtypes = [dbl]
        L.oracle_layer_bf16.restype = i32
        L.oracle_layer_bf16.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_double, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def code(codes, cols, bits, r, c) -> int:
    codes = _c(codes, np.uint8)
    return int(lib().oracle_code(_p(codes), cols, bits, r, c))


def weight(codes, scale, bias, cols, bits, group, r, c) -> float:
    codes, scale, bias = _c(codes, np.uint8), _c(scale, np.uint16), _c(bias, np.uint16)
    return float(lib().oracle_weight(_p(codes), _p(scale), _p(bias), cols, bits, group, r, c))


def matvec(codes, scale, bias, rows, cols, bits, group, x) -> np.ndarray:
    """O2: y = dequant(W) x in fp64."""
    codes, scale, bias = _c(codes, np.uint8), _c(scale, np.uint16), _c(bias, np.uint16)
    x = _c(x, np.float64)
    assert x.size == cols
    y = np.empty(rows, dtype=np.float64)
    lib().oracle_matvec(_p(codes), _p(scale), _p(bias), rows, cols, bits, group, _p(x), _p(y))
    return y


def route(router, v, k):
    """O3: (idx int32 [k], w fp64 [k], logits fp64 [E], margin)."""
    router = _c(router, np.float32)
    E, H = router.shape
    v = _c(v, np.float64)
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    logits = np.empty(E, dtype=np.float64)
    m = ctypes.c_double()
    lib().oracle_route(_p(router), _p(v), E, H, k, _p(idx), _p(w), _p(logits), ctypes.addressof(m))
    return idx, w, logits, m.value


def rmsnorm(h, eps) -> np.ndarray:
    h = _c(h, np.float64)
    v = np.empty_like(h)
    lib().oracle_rmsnorm(_p(h), h.size, eps, _p(v))
    return v


def swiglu(g: float, u: float) -> float:
    return float(lib().oracle_swiglu(g, u))


def round_bf16(v: float) -> float:
    return float(lib().oracle_round_bf16(v))


def _triple(mats):
    """mats: 3 (codes, scale, bias) tuples -> ctypes pointer arrays (+ keepalive list)."""
    keep = []
    arrs = []
    for which in range(3):
        vals = []
        for f, dt in zip(mats[which], (np.uint8, np.uint16, np.uint16)):
            a = _c(f, dt)
            keep.append(a)
            vals.append(a)
        arrs.append(vals)
    P = ctypes.c_void_p * 3
    codes = P(*[_p(arrs[m][0]) for m in range(3)])
    scale = P(*[_p(arrs[m][1]) for m in range(3)])
    bias = P(*[_p(arrs[m][2]) for m in range(3)])
    return codes, scale, bias, keep


def expert_ffn(mats, hidden, inter, bits, group, x):
    """O4: (y fp64 [hidden], a fp64 [inter]); mats = [(codes, scale, bias)] * 3 (gate, up, down)."""
    codes, scale, bias, keep = _triple(mats)
    x = _c(x, np.float64)
    y = np.empty(hidden, dtype=np.float64)
    a = np.empty(inter, dtype=np.float64)
    lib().oracle_expert_ffn(ctypes.addressof(codes), ctypes.addressof(scale), ctypes.addressof(bias), hidden,
                            inter, bits, group, _p(x), _p(y), _p(a))
    del keep
    return y, a


class ArrayProvider:
    """Oracle provider over in-memory experts: experts[layer][e] = [(codes, scale, bias)] * 3."""

    def __init__(self, experts):
        self._experts = experts
        self._keep = None

        def _cb(ctx, layer, e, codes, scale, bias):
            try:
                mats = self._experts[layer][e]
            except (IndexError, KeyError):
                return -1
            keep = []
            for m in range(3):
                c, s, b = (_c(mats[m][0], np.uint8), _c(mats[m][1], np.uint16), _c(mats[m][2], np.uint16))
                keep += [c, s, b]
                codes[m] = _p(c)
                scale[m] = _p(s)
                bias[m] = _p(b)
            self._keep = keep
            return 0

        self._cb = PROVIDER_FN(_cb)

    @property
    def fn(self) -> int:
        return ctypes.cast(self._cb, ctypes.c_void_p).value

    @property
    def ctx(self) -> int:
        return 0


def moe_layer(provider, layer, router, h, inter, k, bits, group, prenorm, eps, shared_gate=None,
              return_shared_w=False):
    """O5: (out fp64 [H], idx [k], w [k], margin[, shared weight]). shared_gate (fp32 [H]):
    the layer also runs its shared expert (provider index E) with weight sigmoid(gate . v)."""
    router = _c(router, np.float32)
    E, H = router.shape
    h = _c(h, np.float64)
    out = np.empty(H, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    m = ctypes.c_double()
    sw = ctypes.c_double(np.nan)
    gate = None if shared_gate is None else _c(shared_gate, np.float32)
    rc = lib().oracle_moe_layer(provider.fn, provider.ctx, layer, _p(router), _p(h), H, inter, E, k, bits, group,
                                int(bool(prenorm)), eps, _p(out), _p(idx), _p(w), ctypes.addressof(m), _p(gate),
                                ctypes.addressof(sw))
    if rc != 0:
        raise RuntimeError("expert provider failed")
    if return_shared_w:
        return out, idx, w, m.value, sw.value
    return out, idx, w, m.value


def stack(provider, routers, x, inter, k, bits, group, eps, stop_margin=0.0, keep_all=True, shared_gates=None):
    """O6: dict(out, idx [L][k], w [L][k], margins [L], h_all [L][H] or None, layers_done,
    shared_w [L] when shared_gates (one fp32 [H] gate per layer) is given)."""
    routers = [_c(r, np.float32) for r in routers]
    L = len(routers)
    E, H = routers[0].shape
    ptrs = (ctypes.c_void_p * L)(*[_p(r) for r in routers])
    x = _c(x, np.float32)
    out = np.empty(H, dtype=np.float64)
    idx = np.full((L, k), -1, dtype=np.int32)
    w = np.zeros((L, k), dtype=np.float64)
    margins = np.full(L, np.nan, dtype=np.float64)
    h_all = np.zeros((L, H), dtype=np.float64) if keep_all else None
    gates = None if shared_gates is None else [_c(gv, np.float32) for gv in shared_gates]
    gptrs = None if gates is None else (ctypes.c_void_p * L)(*[_p(gv) for gv in gates])
    sws = None if gates is None else np.full(L, np.nan, dtype=np.float64)
    done = lib().oracle_stack(provider.fn, provider.ctx, ctypes.addressof(ptrs), L, _p(x), H, inter, E, k, bits,
                              group, eps, stop_margin, _p(out), _p(idx), _p(w), _p(margins), _p(h_all),
                              None if gptrs is None else ctypes.addressof(gptrs), _p(sws))
    if done < 0:
        raise RuntimeError("expert provider failed")
    return dict(out=out, idx=idx, w=w, margins=margins, h_all=h_all, layers_done=done, shared_w=sws)


def layer_bf16(provider, layer, router, X, inter, k, bits, group, a16_force=None, want_stages=False,
               prenorm=False, eps=1e-6, shared_gate=None, shared_a16_force=None):
    """O7 (batched bf16 contract). Returns dict(out [T][H], idx [T][k], w [T][k], margins [T],
    a16 [T][k][inter] fp32, g/u [T][k][inter] if want_stages; with shared_gate also
    shared_w [T] and shared_a16 [T][inter])."""
    router = _c(router, np.float32)
    E, H = router.shape
    X = _c(X, np.float32)
    T = X.shape[0]
    out = np.empty((T, H), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    margins = np.empty(T, dtype=np.float64)
    a16 = np.empty((T, k, inter), dtype=np.float32)
    force = None if a16_force is None else _c(a16_force, np.float32)
    g = np.empty((T, k, inter), dtype=np.float64) if want_stages else None
    u = np.empty((T, k, inter), dtype=np.float64) if want_stages else None
    gate = None if shared_gate is None else _c(shared_gate, np.float32)
    sw = None if gate is None else np.empty(T, dtype=np.float64)
    sa16 = None if gate is None else np.empty((T, inter), dtype=np.float32)
    sforce = None if shared_a16_force is None else _c(shared_a16_force, np.float32)
    rc = lib().oracle_layer_bf16(provider.fn, provider.ctx, layer, _p(router), _p(X), T, H, inter, E, k, bits, group,
                                 int(bool(prenorm)), float(eps), _p(out), _p(idx), _p(w), _p(margins), _p(force),
                                 _p(a16), _p(g), _p(u), _p(gate), _p(sw), _p(sforce), _p(sa16))
    if rc != 0:
        raise RuntimeError("expert provider failed")
    res = dict(out=out, idx=idx, w=w, margins=margins, a16=a16)
    if gate is not None:
        res.update(shared_w=sw, shared_a16=sa16)
    if want_stages:
        res.update(g=g, u=u)
    return res
