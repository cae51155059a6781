"""Parity of every compiled decode shape of the 512-expert stack (hidden 4096, inter 1024)
with the oracle, the full 60-layer stacks against the stored oracle results, the rank rule
for equal router logits on the decode kernel, the error word, and one workspace reused by
calls of different shapes.

Shapes: 60 layers of 512 experts with 4 active per token, hidden 4096
(tr.news.hada.io topic 27758, 'Model mimarisi'); 2-bit experts (aibit.im, the table of
the first section, and 'Performans sonuclari' of the same hada page); 10 experts per
token and a shared expert (hada's HN comments and 'Model mimarisi').

Bar: expert indices bit-exact (inputs with an oracle top-k margin >= 1e-3), weights and
outputs within relative L2 1e-5 of the fp64 oracle.
"""
import gc
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_fmoe_amd as fm
import synth
from gpu_util import DevStack, check_stack_layers, rel_l2, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5
H, I, E = 4096, 1024, 512
ERR_OFFSET = 8 * 1024 * 4  # byte offset of the error word in a moe-layer workspace (include/fmoe.h layout)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _decode(stack, x, k, ws=None, wsb=None, prenorm=True):
    xd = to_dev(x.astype(np.float32))
    hd = torch.empty(stack.H, dtype=torch.float32, device="cuda")
    idx = torch.empty((stack.L, k), dtype=torch.int32, device="cuda")
    w = torch.empty((stack.L, k), dtype=torch.float32, device="cuda")
    if ws is None:
        wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, stack.H, stack.I, stack.E, k)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    fm.moe_layer(stack.layers, xd, hd, 1, k, 1e-6, fm.PRENORM if prenorm else 0, idx, w, ws, wsb)
    torch.cuda.synchronize()
    return hd.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _margin_tokens(stack, k, n, start=0):
    prov = stack.provider()
    out, d = [], start
    while len(out) < n:
        x = synth.token(stack.seed, d, stack.H)
        ref = oracle.stack(prov, stack.routers_np, x, stack.I, k, stack.bits, 64, 1e-6, stop_margin=1e-3,
                           shared_gates=stack.gates_np)
        if ref["layers_done"] == stack.L and np.min(ref["margins"]) >= 1e-3:
            out.append((x, ref))
        d += 1
    return out


# ------------------------------------------------------------------ compiled shapes, pre-normed stacks
@pytest.mark.parametrize("bits,k", [(4, 4), (2, 4), (2, 10), (3, 4), (3, 10)])
def test_compiled_shape_prenorm_stack(bits, k):
    """Three pre-normed layers at the compiled shapes: 4-bit top-4 (the headline), 2-bit
    top-4 (the 2-bit stack's shape), 2-bit top-10 and the 3-bit shapes (openclawradar.com
    'Optimisations efficaces': 3-bit experts)."""
    stack = DevStack(3, E, H, I, bits, gpu_fill=True)
    for x, ref in _margin_tokens(stack, k, 3):
        h, idx, w = _decode(stack, x, k)
        assert np.array_equal(idx, ref["idx"])
        check_stack_layers(stack, x, k, h)
    del stack
    _free()




@pytest.mark.parametrize("bits", [2, 3])
def test_compiled_shape_shared_expert(bits):
    """The compiled shape with a gated shared expert at 2 and 3 bits: two pre-normed layers
    of 512 + 1 experts, top-4; routing bit-exact over the stack, each layer within the bar
    against the oracle layer applied to the kernel's own input to it."""
    stack = DevStack(2, E, H, I, bits, gpu_fill=True, shared=True)
    for x, ref in _margin_tokens(stack, 4, 2):
        h, idx, w = _decode(stack, x, 4)
        assert np.array_equal(idx, ref["idx"])
        check_stack_layers(stack, x, 4, h)
    del stack
    _free()


# ------------------------------------------------------------------ the full 60-layer stacks
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_full_stack_against_stored_oracle(bits, golden_dir):
    """60 layers x 512 experts (120.8 GB at 2 bits, 169.1 at 3, 217.4 GB at 4 bits, resident), each of
    the stored tokens decoded through the whole stack: experts of every layer bit-exact,
    output within 1e-5 of the oracle's fp64 result (tests/golden/make_stack_golden.py)."""
    g = np.load(os.path.join(golden_dir, f"stack_full_{bits}bit.npz"), allow_pickle=False)
    stack = DevStack(60, E, H, I, bits, gpu_fill=True)
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H, I, E, 4)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for i, d in enumerate(g["draw"]):
        x = synth.token(0, int(d), H)
        h, idx, w = _decode(stack, x, 4, ws, wsb)
        assert np.array_equal(idx, g["idx"][i]), int(d)
        assert rel_l2(w, g["w"][i]) <= TOL
        assert rel_l2(h, g["out"][i]) <= TOL, int(d)
    del stack, ws
    _free()


# ------------------------------------------------------------------ equal router logits
def _plant(R, z, experts, gammas):
    x = z.astype(np.float64).copy()
    for e, gm in zip(experts, gammas):
        r = R[e].astype(np.float64)
        x += gm * r / np.linalg.norm(r)
    return x.astype(np.float32)


@pytest.mark.parametrize("E_,H_,I_,k,bits,pair,others", [
    (512, 4096, 1024, 4, 4, (37, 300), []),               # compiled shape: the tied pair ranks first
    (512, 4096, 1024, 4, 4, (37, 300), [5, 411, 128]),    # ... and at the cut: only 37 is selected
    (512, 4096, 1024, 4, 2, (300, 301), [7]),              # 2-bit compiled shape, neighbours in one lane row
    (512, 4096, 1024, 4, 3, (37, 300), [5, 411, 128]),     # 3-bit compiled shape, the pair at the cut
    (64, 1024, 256, 4, 4, (3, 50), [60]),                  # generic kernel, keys in registers
    (1000, 128, 64, 2, 4, (900, 901), [2]),                # more than 512 experts: keys in LDS
])
def test_decode_tie_lower_index_first(E_, H_, I_, k, bits, pair, others):
    """Two experts with identical router rows get bit-identical logits on every path, and
    the rank rule puts the lower index first (the oracle's order): planted at the top, both
    are selected in index order; planted just below k - 1 stronger experts, only the lower
    index is selected."""
    stack = DevStack(1, E_, H_, I_, bits, gpu_fill=(E_ == 512))
    R = stack.routers_np[0].copy()
    R[pair[1]] = R[pair[0]]
    stack.routers_np[0] = R
    stack.routers[0].copy_(to_dev(R))
    gam = [12.0, 11.0, 10.0]
    z = synth.token(0, 0, H_)
    if others:
        x = _plant(R, z, list(others) + [pair[0]], gam[:len(others)] + [8.0])
    else:
        x = _plant(R, z, [pair[0]], [12.0])
    prov = stack.provider()
    want, i_ref, w_ref, _ = oracle.moe_layer(prov, 0, R, x.astype(np.float64), I_, k, bits, 64, 0, 1e-6)
    _, _, lg, _ = oracle.route(R, x, k)
    assert lg[pair[0]] == lg[pair[1]]
    order = np.lexsort((np.arange(E_), -lg))
    if others:
        assert list(order[:len(others)]) == list(others)
        assert order[len(others)] == pair[0] and order[len(others) + 1] == pair[1]
        assert pair[0] in i_ref and (pair[1] in i_ref) == (len(others) + 1 < k)
    else:
        assert list(i_ref[:2]) == list(pair)
    # every other adjacent gap among the first k + 1 is decided far from rounding
    top = lg[order[:k + 1]]
    gaps = [top[j] - top[j + 1] for j in range(k) if {order[j], order[j + 1]} != set(pair)]
    assert min(gaps) >= 1e-3
    h, idx, w = _decode(stack, x, k, prenorm=False)
    assert idx[0].tolist() == i_ref.tolist()
    assert rel_l2(w[0], w_ref) <= TOL
    assert rel_l2(h, want) <= TOL
    # the standalone router and the multi-token path apply the same rule
    lgd = torch.empty((2, E_), dtype=torch.float32, device="cuda")
    idd = torch.empty((2, k), dtype=torch.int32, device="cuda")
    wd = torch.empty((2, k), dtype=torch.float32, device="cuda")
    X2 = np.stack([x, x])
    fm.route_topk(stack.routers[0], to_dev(X2), 2, E_, H_, k, idd, wd, lgd)
    torch.cuda.synchronize()
    assert idd.cpu().numpy().tolist() == [i_ref.tolist()] * 2
    if H_ % 256 == 0 and I_ % 128 == 0:
        wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 2, H_, I_, E_, k)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        hb = torch.empty((2, H_), dtype=torch.float32, device="cuda")
        ib = torch.empty((2, 1, k), dtype=torch.int32, device="cuda")
        fm.moe_layer(stack.layers, to_dev(X2), hb, 2, k, 1e-6, 0, ib, None, ws, wsb)
        torch.cuda.synchronize()
        assert ib.cpu().numpy()[:, 0].tolist() == [i_ref.tolist()] * 2
    del stack
    _free()


# ------------------------------------------------------------------ the error word
@pytest.mark.parametrize("E_,H_,I_,k,L", [(64, 1024, 256, 4, 2), (512, 4096, 1024, 4, 2)])
def test_error_word_set_by_host(E_, H_, I_, k, L):
    """A workspace whose error word is set (as after a call whose device-side wait gave
    up) makes the decode kernel end at once: every workgroup exits normally, h_out is NaN,
    the error word stays set; after zero-filling the workspace the same call is correct."""
    stack = DevStack(L, E_, H_, I_, 4, gpu_fill=(E_ == 512))
    (x, ref), = _margin_tokens(stack, k, 1)
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H_, I_, E_, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws[ERR_OFFSET] = 1
    h, _, _ = _decode(stack, x, k, ws, wsb)
    fm.workspace_error(ws, wsb, err)
    torch.cuda.synchronize()
    assert np.all(np.isnan(h))
    assert int(err.item()) != 0
    ws.zero_()
    h, idx, _ = _decode(stack, x, k, ws, wsb)
    fm.workspace_error(ws, wsb, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(idx, ref["idx"])
    assert rel_l2(h, ref["out"]) <= TOL
    del stack
    _free()


# ------------------------------------------------------------------ one workspace, calls of several shapes
def test_workspace_reused_across_shapes():
    """One workspace (sized for the largest call) serves, in this order: a 2-layer 64-token
    call, a 12-token call, a 12-token call with another k, a single-token decode, another
    64-token call and another decode. Every result equals the same call on a fresh
    zero-filled workspace (bit for bit: the paths are deterministic)."""
    H_, I_, E_ = 1024, 256, 64
    stack = DevStack(2, E_, H_, I_, 4)
    big = fm.workspace_bytes(fm.OP_MOE_LAYER, 64, H_, I_, E_, 8)
    shared_ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    X = np.stack([synth.token(0, d, H_) for d in range(64)])
    calls = [(64, 4), (12, 4), (12, 8), (1, 4), (64, 2), (1, 8)]
    for T, k in calls:
        def run(ws, wsb):
            h = torch.empty((T, H_), dtype=torch.float32, device="cuda")
            idx = torch.empty((T, 2, k), dtype=torch.int32, device="cuda")
            fm.moe_layer(stack.layers, to_dev(X[:T]), h, T, k, 1e-6, fm.PRENORM, idx, None, ws, wsb)
            torch.cuda.synchronize()
            return h.cpu().numpy(), idx.cpu().numpy()
        got = run(shared_ws, big)
        fresh_b = fm.workspace_bytes(fm.OP_MOE_LAYER, T, H_, I_, E_, k)
        want = run(torch.zeros(fresh_b, dtype=torch.uint8, device="cuda"), fresh_b)
        assert np.array_equal(got[1], want[1]), (T, k)
        assert np.array_equal(got[0], want[0]), (T, k)
        assert np.all(np.isfinite(got[0]))
    del stack
    _free()
