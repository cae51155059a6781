"""Seeded, counter-based synthetic inputs (CPU side) for the quantized MoE expert block.

Thin ctypes wrapper over ``libsynth.so`` (synth.c). The module holds none of the
method's arithmetic: it produces canonical-layout codes, bf16 scales/biases, fp32
router weights and fp32 token vectors from a seed and a coordinate. The same
generator is implemented for the GPU in ``synth_gpu.hip`` (codes, scales and biases
only), so that the 217 GB 4-bit expert set can be filled on the device and checked
against the CPU byte for byte.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_GPU_SO = os.path.join(_HERE, "libsynth_gpu.so")

GATE, UP, DOWN = 0, 1, 2
TAG_CODES, TAG_SCALE, TAG_BIAS, TAG_ROUTER, TAG_TOKEN, TAG_PLANT, TAG_NOISE = 1, 2, 3, 4, 5, 6, 7
SCALE_LO, SCALE_WIDTH = 0.001, 0.019
BIAS_LO, BIAS_WIDTH = -0.1, 0.2


def build_cpu() -> str:
    """Compile libsynth.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-shared", "-fPIC",
           os.path.join(_HERE, "synth.c"), "-o", _SO, "-lm"]
    subprocess.run(cmd, check=True)
    return _SO


def build_gpu() -> str:
    """Compile libsynth_gpu.so (the GPU fixture) with hipcc for gfx950."""
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "synth_gpu.hip"), "-o", _GPU_SO]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return _GPU_SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build_cpu()
        L = ctypes.CDLL(_SO)
        u64, u32, i32, vp, dbl, sz = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_double, ctypes.c_size_t)
        L.synth_mix64.restype = u64
        L.synth_mix64.argtypes = [u64]
        L.synth_stream.restype = u64
        L.synth_stream.argtypes = [u64, u32, u32, u32, u32]
        L.synth_hash.restype = u64
        L.synth_hash.argtypes = [u64, u64]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_matrix.restype = None
        L.synth_matrix.argtypes = [u64, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
        L.synth_router.restype = None
        L.synth_router.argtypes = [u64, i32, i32, i32, vp]
        L.synth_token.restype = None
        L.synth_token.argtypes = [u64, u64, i32, vp]
        L.synth_uniform_at.restype = dbl
        L.synth_uniform_at.argtypes = [u64, u32, u32, u32, u32, u64]
        L.synth_normal_f32.restype = None
        L.synth_normal_f32.argtypes = [u64, dbl, vp, sz]
        L.synth_provider_init.restype = i32
        L.synth_provider_init.argtypes = [vp, u64, i32, i32, i32, i32]
        L.synth_provider_free.restype = None
        L.synth_provider_free.argtypes = [vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def mix64(z: int) -> int:
    return int(lib().synth_mix64(z))


def stream(seed: int, tag: int, layer: int, expert: int, matrix: int) -> int:
    return int(lib().synth_stream(seed, tag, layer, expert, matrix))


def hash_at(stream_key: int, idx: int) -> int:
    return int(lib().synth_hash(stream_key, idx))


def matrix(seed: int, layer: int, expert: int, which: int, rows: int, cols: int, bits: int, group: int = 64):
    """Canonical (codes uint8 [rows][cols*bits/8], scale bf16-bits uint16 [rows][cols/group], bias)."""
    codes = np.empty((rows, cols * bits // 8), dtype=np.uint8)
    scale = np.empty((rows, cols // group), dtype=np.uint16)
    bias = np.empty((rows, cols // group), dtype=np.uint16)
    lib().synth_matrix(seed, layer, expert, which, rows, cols, bits, group, _ptr(codes), _ptr(scale), _ptr(bias))
    return codes, scale, bias


def expert(seed: int, layer: int, e: int, hidden: int, inter: int, bits: int, group: int = 64):
    """Canonical gate, up, down matrices of one expert: list of 3 (codes, scale, bias)."""
    return [matrix(seed, layer, e, m, inter if m != DOWN else hidden, hidden if m != DOWN else inter, bits, group)
            for m in (GATE, UP, DOWN)]


def router(seed: int, layer: int, n_experts: int, hidden: int) -> np.ndarray:
    out = np.empty((n_experts, hidden), dtype=np.float32)
    lib().synth_router(seed, layer, n_experts, hidden, _ptr(out))
    return out


def token(seed: int, draw: int, hidden: int) -> np.ndarray:
    out = np.empty(hidden, dtype=np.float32)
    lib().synth_token(seed, draw, hidden, _ptr(out))
    return out


def normal(seed: int, tag: int, a: int, b: int, c: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(stream(seed, tag, a, b, c), sigma, _ptr(out), n)
    return out


def uniform_at(seed: int, tag: int, a: int, b: int, c: int, i: int) -> float:
    return float(lib().synth_uniform_at(seed, tag, a, b, c, i))


def zipf_experts(seed: int, draw: int, n_experts: int, k: int, s: float = 1.1) -> np.ndarray:
    """k distinct experts for token `draw`, drawn one after another without replacement from
    p(e) proportional to (e + 1)^-s (expert 0 the most popular). Uniforms come from stream
    (TAG_PLANT, draw); the j-th pick uses index j."""
    p = (np.arange(n_experts, dtype=np.float64) + 1.0) ** (-s)
    out = np.empty(k, dtype=np.int32)
    for j in range(k):
        u = uniform_at(seed, TAG_PLANT, draw >> 32, draw & 0xFFFFFFFF, 0, j) * p.sum()
        e = int(np.searchsorted(np.cumsum(p), u, side="right"))
        e = min(e, n_experts - 1)
        while p[e] == 0.0:  # u landed on the edge of a removed expert
            e -= 1
        out[j] = e
        p[e] = 0.0
    return out


def planted_token(seed: int, draw: int, router: np.ndarray, k: int, gammas=(8.0, 7.0, 6.0, 5.0),
                  s: float = 1.1):
    """Token whose router winners are planted: x = z + sum_j gamma_j * r_e_j / |r_e_j| with
    z ~ N(0, I) (stream TAG_NOISE, draw) and e_j = zipf_experts(...). Returns (x fp32, experts)."""
    E, H = router.shape
    experts = zipf_experts(seed, draw, E, k, s)
    z = normal(seed, TAG_NOISE, draw >> 32, draw & 0xFFFFFFFF, 0, H).astype(np.float64)
    for j, e in enumerate(experts):
        r = router[e].astype(np.float64)
        z += gammas[j % len(gammas)] * r / np.linalg.norm(r)
    return z.astype(np.float32), experts


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        rounded[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class _ProviderStruct(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("hidden", ctypes.c_int), ("inter", ctypes.c_int),
                ("bits", ctypes.c_int), ("group", ctypes.c_int),
                ("codes", ctypes.c_void_p * 3), ("scale", ctypes.c_void_p * 3), ("bias", ctypes.c_void_p * 3)]


class Provider:
    """Expert provider for the oracle: regenerates expert (layer, e) on demand (C callback)."""

    def __init__(self, seed: int, hidden: int, inter: int, bits: int, group: int = 64):
        self._s = _ProviderStruct()
        rc = lib().synth_provider_init(ctypes.byref(self._s), seed, hidden, inter, bits, group)
        if rc != 0:
            raise MemoryError("synth provider allocation failed")
        self.seed, self.hidden, self.inter, self.bits, self.group = seed, hidden, inter, bits, group

    @property
    def fn(self) -> int:
        return ctypes.cast(lib().synth_provide, ctypes.c_void_p).value

    @property
    def ctx(self) -> int:
        return ctypes.addressof(self._s)

    def close(self):
        if self._s is not None:
            lib().synth_provider_free(ctypes.byref(self._s))
            self._s = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- GPU fixture
_glib = None


def gpu_lib():
    """ctypes handle of libsynth_gpu.so (device-side generator of codes/scales/biases)."""
    global _glib
    if _glib is None:
        if not os.path.exists(_GPU_SO):
            raise RuntimeError("libsynth_gpu.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_GPU_SO)
        u64, i32, vp, sz = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.synth_gpu_matrix.restype = i32
        L.synth_gpu_matrix.argtypes = [u64, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp, vp, sz, vp]
        _glib = L
    return _glib


def gpu_matrix(seed, layer, expert0, n_experts, which, rows, cols, bits, group,
               codes_ptr, codes_stride, scale_ptr, bias_ptr, sb_stride, stream_handle=0) -> None:
    """Fill canonical codes (+ scale/bias) of `which` for experts expert0.. on the device.

    codes of expert e go to codes_ptr + (e - expert0) * codes_stride (bytes); scale/bias
    (bf16 [rows][cols/group]) to scale_ptr/bias_ptr + (e - expert0) * sb_stride (bytes);
    a null scale/bias pointer skips that field."""
    rc = gpu_lib().synth_gpu_matrix(seed, layer, expert0, n_experts, which, rows, cols, bits, group,
                                    codes_ptr, codes_stride, scale_ptr, bias_ptr, sb_stride, stream_handle)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_matrix failed with HIP error {rc}")
