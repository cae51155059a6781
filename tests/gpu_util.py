"""Helpers for the GPU tests and the benchmark: put synthetic experts/routers on the device
in the library's packed layout (through fmoe_pack), and compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import quantized_expert_ffn_fmoe_amd as fm
import synth


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


class DevMatrix:
    """One packed quantized matrix on the device (keeps its buffers alive)."""

    def __init__(self, codes, scale, bias, rows, cols, bits, dev="cuda"):
        self.codes = torch.empty(fm.codes_bytes(rows, cols, bits), dtype=torch.uint8, device=dev)
        self.sb = torch.empty(fm.sb_bytes(rows, cols) // 4, dtype=torch.int32, device=dev)
        fm.pack(to_dev(codes, dev), to_dev(scale, dev), to_dev(bias, dev), rows, cols, bits, 64, self.codes, self.sb)
        self.q = fm.qmat(self.codes, self.sb, rows, cols, bits)


def fill_experts_cpu(blob: torch.Tensor, stride: int, layer: int, n_experts: int, H: int, I: int, bits: int,
                     seed: int = 0) -> None:
    """Experts 0..n_experts-1 of `layer` from the CPU generator, packed into blob."""
    dev = blob.device
    for e in range(n_experts):
        view = fm.expert_view(blob.data_ptr() + e * stride, H, I, bits)
        for m, q in enumerate((view.gate, view.up, view.down)):
            rows, cols = (I, H) if m < 2 else (H, I)
            codes, scale, bias = synth.matrix(seed, layer, e, m, rows, cols, bits)
            fm.pack(to_dev(codes, dev), to_dev(scale, dev), to_dev(bias, dev), rows, cols, bits, 64, q.codes, q.sb)


def fill_experts_gpu(blob: torch.Tensor, stride: int, layer: int, n_experts: int, H: int, I: int, bits: int,
                     seed: int = 0, chunk: int = 128) -> None:
    """Same as fill_experts_cpu but generated on the device (GPU fixture), in chunks of experts.
    Canonical codes and the scales/biases go to scratch buffers; fmoe_pack writes them into
    the blob in the library's packed layout."""
    dev = blob.device
    cb = fm.codes_bytes(I, H, bits)
    ngrp = I * H // 64
    codes = torch.empty((chunk, cb), dtype=torch.uint8, device=dev)
    scale = torch.empty((chunk, ngrp), dtype=torch.int16, device=dev)
    bias = torch.empty((chunk, ngrp), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for e0 in range(0, n_experts, chunk):
        ne = min(chunk, n_experts - e0)
        base = blob.data_ptr() + e0 * stride
        for m in range(3):
            rows, cols = (I, H) if m < 2 else (H, I)
            synth.gpu_matrix(seed, layer, e0, ne, m, rows, cols, bits, 64, codes.data_ptr(), cb,
                             scale.data_ptr(), bias.data_ptr(), ngrp * 2, stream)
            for j in range(ne):
                view = fm.expert_view(base + j * stride, H, I, bits)
                q = (view.gate, view.up, view.down)[m]
                fm.pack(codes[j], scale[j], bias[j], rows, cols, bits, 64, q.codes, q.sb)


class DevStack:
    """A stack of MoE layers on the device: routers (fp32) and packed expert blobs."""

    def __init__(self, n_layers, E, H, I, bits, seed=0, dev="cuda", gpu_fill=False, shared=False):
        """shared: every layer also has a shared expert (blob index E, generated like expert E)
        and a gate vector N(0, 0.02) from its own generator stream (layer 1000 + l)."""
        self.L, self.E, self.H, self.I, self.bits, self.seed = n_layers, E, H, I, bits, seed
        self.gates_np, self.gates = (None, None) if not shared else ([], [])
        nb = E + (1 if shared else 0)
        eb = fm.expert_bytes(H, I, bits)
        self.stride = (eb + 255) // 256 * 256
        self.routers_np = []
        self.routers = []
        self.blobs = []
        layers = []
        for l in range(n_layers):
            blob = torch.empty(nb * self.stride, dtype=torch.uint8, device=dev)
            if gpu_fill:
                fill_experts_gpu(blob, self.stride, l, nb, H, I, bits, seed)
            else:
                fill_experts_cpu(blob, self.stride, l, nb, H, I, bits, seed)
            R = synth.router(seed, l, E, H)
            self.routers_np.append(R)
            Rd = to_dev(R, dev)
            self.routers.append(Rd)
            self.blobs.append(blob)
            gate = 0
            if shared:
                gn = synth.router(seed, 1000 + l, 1, H)[0]
                self.gates_np.append(gn)
                self.gates.append(to_dev(gn, dev))
                gate = self.gates[-1].data_ptr()
            layers.append(fm.Layer(Rd.data_ptr(), blob.data_ptr(), self.stride, E, H, I, bits, 64, gate))
        self.layers = fm.layers_array(layers)

    def provider(self):
        return synth.Provider(self.seed, self.H, self.I, self.bits)


def check_stack_layers(stack, x, k, h_stack, tol=1e-5):
    """Every layer of a pre-normed stack against the oracle layer applied to the kernel's own
    input to it (fmoe_moe_layer runs of the first l + 1 layers): experts bit-exact, routing
    weights and output within tol. A stack's fp32 error can be amplified by later layers
    (the synthetic layers change h by orders of magnitude), so the bar is applied layer by
    layer; the last run is the whole stack, compared bit for bit with h_stack."""
    import oracle

    prov = stack.provider()
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, stack.H, stack.I, stack.E, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h_in = x.astype(np.float32)
    for l in range(stack.L):
        sub = fm.layers_array([stack.layers[j] for j in range(l + 1)])
        hd = torch.empty(stack.H, dtype=torch.float32, device="cuda")
        idx = torch.empty((l + 1, k), dtype=torch.int32, device="cuda")
        w = torch.empty((l + 1, k), dtype=torch.float32, device="cuda")
        fm.moe_layer(sub, to_dev(x.astype(np.float32)), hd, 1, k, 1e-6, fm.PRENORM, idx, w, ws, wsb)
        torch.cuda.synchronize()
        h_l = hd.cpu().numpy()
        want, i_l, w_l, _ = oracle.moe_layer(prov, l, stack.routers_np[l], h_in.astype(np.float64), stack.I, k,
                                             stack.bits, 64, 1, 1e-6,
                                             shared_gate=None if stack.gates_np is None else stack.gates_np[l])
        assert idx.cpu().numpy()[l].tolist() == i_l.tolist(), l
        assert rel_l2(w.cpu().numpy()[l], w_l) <= tol, l
        assert rel_l2(h_l, want) <= tol, l
        h_in = h_l
    assert np.array_equal(h_in, h_stack)
