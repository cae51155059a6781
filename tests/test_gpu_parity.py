"""Parity of the HIP library (through the C-ABI) with the CPU oracle, on the GPU.

Tolerances: expert indices bit-exact on inputs whose oracle top-k margin is >= 1e-3;
routing weights and outputs within relative L2 error 1e-5 (fp32 accumulation against
the fp64 oracle); integer/byte work (generator fixture, packing) bit-exact.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_fmoe_amd as fm
import synth
from gpu_util import DevMatrix, DevStack, check_stack_layers, rel_l2, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _run_matvec(codes, scale, bias, rows, cols, bits, X):
    m = DevMatrix(codes, scale, bias, rows, cols, bits)
    n_vec = X.shape[0]
    xd = to_dev(X.astype(np.float32))
    yd = torch.empty((n_vec, rows), dtype=torch.float32, device="cuda")
    fm.dequant_matvec(m.q, xd, yd, n_vec)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


# ------------------------------------------------------------------ generator fixture and packing
def _layout_offset(bits, rows, row_bytes, r, b):
    """The packed code layout written out independently of the library: blocks of 32 rows,
    each row cut into pieces of 4 groups (128 bytes at 4 bits, 64 at 2 bits), piece p of the
    block's rows stored together in row order, a row's 16-byte chunks rotated inside its
    piece by r mod 8 (4-bit) or (r mod 16) // 4 (2-bit); short last pieces and short last
    blocks use their own sizes."""
    rb = 32
    pb = 32 * bits
    r0 = r // rb * rb
    nr = min(rb, rows - r0)
    p = b // pb
    piece = min(pb, row_bytes - p * pb)
    rot = r % 8 if bits == 4 else (r % 16) // 4
    pos = ((b % pb) // 16 + rot) % (piece // 16)
    return r0 * row_bytes + p * nr * pb + (r - r0) * piece + pos * 16 + b % 16


def _sb_layout_offset(rows, groups, r, g):
    """The blocked scale/bias order written out independently of the library: blocks of 32
    rows, each row's words cut into pieces of 4 groups, piece p of the block's rows stored
    together in row order; short last pieces and blocks keep their own sizes."""
    r0 = r // 32 * 32
    nr = min(32, rows - r0)
    p = g // 4
    pg = min(4, groups - p * 4)
    return r0 * groups + p * nr * 4 + (r - r0) * pg + g % 4


def _hi_layout_offset(rows, groups, r, g, h):
    """Word offset of high-plane word h (0, 1) of group g of row r of a 3-bit matrix, written
    out independently of the library: blocks of 32 rows, each row's words cut into pieces of
    4 groups (8 words), piece p of the block's rows stored together in row order; short last
    pieces and blocks keep their own sizes."""
    r0 = r // 32 * 32
    nr = min(32, rows - r0)
    p = g // 4
    pg = min(4, groups - p * 4)
    return r0 * groups * 2 + p * nr * 8 + (r - r0) * pg * 2 + (g % 4) * 2 + h


def _hi_bit(c):
    """Bit of column c (0..31 of a 32-column half group) in its high-plane word: column c of
    16-column dword t = c // 16 is operand 2t + c % 2, nibble (c % 16) // 2."""
    return 4 * ((c % 16) // 2) + 2 * (c // 16) + (c % 2)


@pytest.mark.parametrize("rows,cols", [(64, 4096), (13, 192), (40, 320), (45, 448), (300, 512), (33, 64)])
def test_pack_layout_3bit(rows, cols):
    """3-bit codes: the low 2 bits of every code land where a 2-bit matrix of the same shape
    puts its codes, the third bits in the high-plane words after it; the two planes take
    exactly rows * cols * 3 / 8 bytes."""
    rng = np.random.default_rng(rows * 1000 + cols + 3)
    row_bytes = cols * 3 // 8
    canon = rng.integers(0, 256, size=(rows, row_bytes), dtype=np.uint8)
    ng = rows * cols // 64
    groups = cols // 64
    scale = rng.integers(0, 1 << 16, size=ng, dtype=np.uint16)
    bias = rng.integers(0, 1 << 16, size=ng, dtype=np.uint16)
    cb = fm.codes_bytes(rows, cols, 3)
    assert cb == rows * row_bytes
    out = torch.full((cb + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.empty(ng, dtype=torch.int32, device="cuda")
    fm.pack(to_dev(canon), to_dev(scale), to_dev(bias), rows, cols, 3, 64, out, sb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[cb:] == 0xA5)
    lo_bytes = rows * cols // 4
    stream = np.unpackbits(canon, axis=1, bitorder="little").reshape(rows, cols, 3)
    lo2 = np.packbits(stream[:, :, :2].reshape(rows, cols * 2), axis=1, bitorder="little")  # 2-bit canonical
    want_lo = np.empty(lo_bytes, dtype=np.uint8)
    for r in range(rows):
        for b in range(0, cols // 4, 16):
            o = _layout_offset(2, rows, cols // 4, r, b)
            want_lo[o:o + 16] = lo2[r, b:b + 16]
    assert np.array_equal(got[:lo_bytes], want_lo)
    hi = got[lo_bytes:cb].view(np.uint32)
    want_hi = np.zeros(rows * groups * 2, dtype=np.uint32)
    for r in range(rows):
        for c in range(cols):
            g, h, cc = c // 64, (c % 64) // 32, c % 32
            want_hi[_hi_layout_offset(rows, groups, r, g, h)] |= np.uint32(int(stream[r, c, 2]) << _hi_bit(cc))
    assert np.array_equal(hi, want_hi)
    sbw = sb.cpu().numpy().view(np.uint32)
    words = scale.astype(np.uint32) | (bias.astype(np.uint32) << 16)
    want_sb = np.empty(ng, dtype=np.uint32)
    for r in range(rows):
        for g in range(groups):
            want_sb[_sb_layout_offset(rows, groups, r, g)] = words[r * groups + g]
    assert np.array_equal(sbw, want_sb)


@pytest.mark.parametrize("bits,rows,cols", [(4, 64, 4096), (4, 13, 192), (4, 40, 320), (2, 96, 1024),
                                            (2, 19, 128), (2, 45, 448), (4, 300, 512), (2, 520, 256)])
def test_pack_layout(bits, rows, cols):
    """fmoe_pack puts every 16-byte chunk of the canonical rows and every scale/bias word
    where the layout says, and the matrix occupies exactly rows * cols * bits / 8 bytes."""
    rng = np.random.default_rng(rows * 1000 + cols + bits)
    row_bytes = cols * bits // 8
    canon = rng.integers(0, 256, size=(rows, row_bytes), dtype=np.uint8)
    ng = rows * cols // 64
    scale = rng.integers(0, 1 << 16, size=ng, dtype=np.uint16)
    bias = rng.integers(0, 1 << 16, size=ng, dtype=np.uint16)
    cb = fm.codes_bytes(rows, cols, bits)
    assert cb == rows * row_bytes
    out = torch.full((cb + 64,), 0xA5, dtype=torch.uint8, device="cuda")  # guard bytes after the matrix
    sb = torch.empty(ng, dtype=torch.int32, device="cuda")
    fm.pack(to_dev(canon), to_dev(scale), to_dev(bias), rows, cols, bits, 64, out, sb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = np.empty(cb, dtype=np.uint8)
    for r in range(rows):
        for b in range(0, row_bytes, 16):
            o = _layout_offset(bits, rows, row_bytes, r, b)
            want[o:o + 16] = canon[r, b:b + 16]
    assert np.array_equal(got[:cb], want)
    assert np.all(got[cb:] == 0xA5)
    sbw = sb.cpu().numpy().view(np.uint32)
    words = scale.astype(np.uint32) | (bias.astype(np.uint32) << 16)
    groups = cols // 64
    want_sb = np.empty(ng, dtype=np.uint32)
    for r in range(rows):
        for g in range(groups):
            want_sb[_sb_layout_offset(rows, groups, r, g)] = words[r * groups + g]
    assert np.array_equal(sbw, want_sb)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_gpu_fixture_matches_cpu_generator(bits):
    H, I = 4096, 1024
    for (layer, e0, ne, which) in [(0, 0, 2, 0), (7, 509, 3, 2), (59, 100, 1, 1)]:
        rows, cols = (I, H) if which < 2 else (H, I)
        cb = fm.codes_bytes(rows, cols, bits)
        ng = rows * cols // 64
        codes = torch.empty(ne * cb, dtype=torch.uint8, device="cuda")
        sc = torch.empty(ne * ng, dtype=torch.int16, device="cuda")
        bi = torch.empty(ne * ng, dtype=torch.int16, device="cuda")
        synth.gpu_matrix(0, layer, e0, ne, which, rows, cols, bits, 64, codes.data_ptr(), cb, sc.data_ptr(),
                         bi.data_ptr(), ng * 2, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        c_h, s_h, b_h = codes.cpu().numpy(), sc.cpu().numpy().view(np.uint16), bi.cpu().numpy().view(np.uint16)
        for j in range(ne):
            c, s, b = synth.matrix(0, layer, e0 + j, which, rows, cols, bits)
            assert np.array_equal(c_h[j * cb:(j + 1) * cb], c.ravel())
            assert np.array_equal(s_h[j * ng:(j + 1) * ng], s.ravel())
            assert np.array_equal(b_h[j * ng:(j + 1) * ng], b.ravel())


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_pack_onehot_returns_dequantized_column(bits):
    """Packed layout end to end: one-hot x gives the dequantized column, exactly q*s+b
    rounded once to fp32 (the oracle's exact value rounded to fp32)."""
    rows, cols = 96, 256
    codes, scale, bias = synth.matrix(3, 1, 2, 0, rows, cols, bits)
    cols_probe = [0, 1, 2, 3, 31, 32, 63, 64, 65, 127, 200, 255]
    X = np.zeros((len(cols_probe), cols), dtype=np.float32)
    for i, c in enumerate(cols_probe):
        X[i, c] = 1.0
    Y = _run_matvec(codes, scale, bias, rows, cols, bits, X)
    for i, c in enumerate(cols_probe):
        want = np.array([oracle.weight(codes, scale, bias, cols, bits, 64, r, c) for r in range(rows)])
        assert np.array_equal(Y[i], want.astype(np.float32)), c


# ------------------------------------------------------------------ dequant matvec
def test_matvec_config1():
    """W 1024x4096 uint4, group 64, bf16 s ~U(0.001,0.02), b ~U(-0.1,0.1), x ~N(0,1), seed 0."""
    rows, cols, bits = 1024, 4096, 4
    codes, scale, bias = synth.matrix(0, 0, 0, 0, rows, cols, bits)
    x = synth.token(0, 0, cols)
    y = _run_matvec(codes, scale, bias, rows, cols, bits, x[None, :])[0]
    want = oracle.matvec(codes, scale, bias, rows, cols, bits, 64, x)
    assert rel_l2(y, want) <= TOL
    y2 = _run_matvec(codes, scale, bias, rows, cols, bits, x[None, :])[0]
    assert np.array_equal(y, y2)  # deterministic


@pytest.mark.parametrize("rows,cols,bits,n_vec", [
    (1, 64, 4, 1), (3, 192, 4, 2), (37, 320, 2, 1), (100, 2048, 4, 3), (64, 8192, 4, 1),
    (65, 16384, 2, 1), (513, 1024, 2, 2), (250, 4096, 2, 1), (7, 6144, 4, 1), (1000, 960, 4, 64),
    (1024, 4096, 3, 1), (3, 192, 3, 2), (37, 320, 3, 1), (100, 2048, 3, 3), (65, 16384, 3, 1), (513, 1024, 3, 2),
    (1000, 960, 3, 64), (31, 8192, 3, 1)])
def test_matvec_shapes(rows, cols, bits, n_vec):
    rng = np.random.default_rng(rows * 7 + cols + bits)
    codes, scale, bias = synth.matrix(11, rows, cols, bits, rows, cols, bits)
    X = rng.standard_normal((n_vec, cols)).astype(np.float32)
    Y = _run_matvec(codes, scale, bias, rows, cols, bits, X)
    for v in range(n_vec):
        want = oracle.matvec(codes, scale, bias, rows, cols, bits, 64, X[v])
        assert rel_l2(Y[v], want) <= TOL, v


@pytest.mark.parametrize("rows_list,cols,bits,n_vec", [
    ([4096, 512, 512], 4096, 4, 1),     # Q/K/V-like projections of one hidden vector
    ([4096, 512, 512], 4096, 2, 2),
    ([100, 37, 1], 2048, 2, 3),         # ragged row counts (partial row blocks)
    ([64] * 8, 960, 4, 2),              # the maximum of 8 matrices
    ([5, 300], 16384, 2, 1),
    ([33], 320, 4, 64),
    ([4096, 512, 512], 4096, 3, 1),
    ([100, 37, 1], 2048, 3, 3)])
def test_matvec_multi(rows_list, cols, bits, n_vec):
    """fmoe_dequant_matvec_multi against the oracle's matvec of each matrix, and bit for bit
    against fmoe_dequant_matvec of each matrix alone (same per-row arithmetic)."""
    rng = np.random.default_rng(sum(rows_list) + cols + bits + n_vec)
    X = rng.standard_normal((n_vec, cols)).astype(np.float32)
    xd = to_dev(X)
    mats, outs, host = [], [], []
    for m, rows in enumerate(rows_list):
        codes, scale, bias = synth.matrix(13, m, rows, cols, rows, cols, bits)
        mats.append(DevMatrix(codes, scale, bias, rows, cols, bits))
        outs.append(torch.full((n_vec, rows), float("nan"), dtype=torch.float32, device="cuda"))
        host.append((codes, scale, bias, rows))
    fm.dequant_matvec_multi([d.q for d in mats], xd, outs, n_vec)
    torch.cuda.synchronize()
    for m, (codes, scale, bias, rows) in enumerate(host):
        Y = outs[m].cpu().numpy()
        single = torch.empty((n_vec, rows), dtype=torch.float32, device="cuda")
        fm.dequant_matvec(mats[m].q, xd, single, n_vec)
        torch.cuda.synchronize()
        assert np.array_equal(Y, single.cpu().numpy()), m
        for v in range(n_vec):
            want = oracle.matvec(codes, scale, bias, rows, cols, bits, 64, X[v])
            assert rel_l2(Y[v], want) <= TOL, (m, v)


# ------------------------------------------------------------------ routing
def _route_dev(R, X, k):
    n, H = X.shape
    E = R.shape[0]
    idx = torch.empty((n, k), dtype=torch.int32, device="cuda")
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
    fm.route_topk(to_dev(R), to_dev(X.astype(np.float32)), n, E, H, k, idx, w, lg)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


def test_route_golden_tiny(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "route_tiny.json")))
    R = np.zeros((6, 64), dtype=np.float32)
    R[:, :2] = np.array(d["router"], dtype=np.float32)
    for case in d["cases"]:
        X = np.zeros((1, 64), dtype=np.float32)
        X[0, :2] = case["v"]
        idx, w, lg = _route_dev(R, X, case["k"])
        assert idx[0].tolist() == case["idx"]
        assert lg[0].tolist() == case["logits"]
        _, w_ref, _, _ = oracle.route(R, X[0], case["k"])
        assert np.allclose(w[0], w_ref, rtol=1e-6, atol=0)


def _margin_tokens(R, H, k, n, seed=0, start=0):
    X, draws = [], []
    d = start
    while len(X) < n:
        x = synth.token(seed, d, H)
        _, _, _, m = oracle.route(R, x, k)
        if m >= 1e-3:
            X.append(x)
            draws.append(d)
        d += 1
    return np.stack(X), draws


@pytest.mark.parametrize("E,H,k,n", [(512, 4096, 4, 24), (64, 1024, 1, 5), (300, 2048, 16, 3), (4096, 256, 8, 2)])
def test_route_topk(E, H, k, n):
    R = synth.router(0, 0, E, H)
    X, _ = _margin_tokens(R, H, k, n)
    idx, w, lg = _route_dev(R, X, k)
    for t in range(n):
        i_ref, w_ref, l_ref, m = oracle.route(R, X[t], k)
        assert idx[t].tolist() == i_ref.tolist()
        assert rel_l2(w[t], w_ref) <= TOL
        assert rel_l2(lg[t], l_ref) <= TOL
        assert abs(float(w[t].sum()) - 1.0) <= 1e-6


# ------------------------------------------------------------------ expert FFN
@pytest.mark.parametrize("H,I,bits", [(4096, 1024, 4), (4096, 1024, 2), (512, 192, 4), (256, 64, 2),
                                      (4096, 1024, 3), (512, 192, 3)])
def test_expert_ffn(H, I, bits):
    mats = synth.expert(0, 2, 5, H, I, bits)
    dm = [DevMatrix(*mats[m], *((I, H) if m < 2 else (H, I)), bits) for m in range(3)]
    e = fm.Expert(dm[0].q, dm[1].q, dm[2].q)
    x = synth.token(0, 7, H)
    xd = to_dev(x)
    yd = torch.empty(H, dtype=torch.float32, device="cuda")
    wsb = fm.workspace_bytes(fm.OP_EXPERT_FFN, 1, H, I, 1, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    fm.expert_ffn(e, xd, yd, ws, wsb)
    torch.cuda.synchronize()
    y_ref, _ = oracle.expert_ffn(mats, H, I, bits, 64, x)
    assert rel_l2(yd.cpu().numpy(), y_ref) <= TOL


# ------------------------------------------------------------------ decode path (fmoe_moe_layer, n_tokens = 1)
def _decode(stack, x, k, prenorm=True, eps=1e-6):
    H = stack.H
    xd = to_dev(x.astype(np.float32))
    hd = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty((stack.L, k), dtype=torch.int32, device="cuda")
    w = torch.empty((stack.L, k), dtype=torch.float32, device="cuda")
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H, stack.I, stack.E, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    fm.moe_layer(stack.layers, xd, hd, 1, k, eps, fm.PRENORM if prenorm else 0, idx, w, ws, wsb)
    torch.cuda.synchronize()
    return hd.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _stack_tokens(stack, k, n, prenorm=True, start=0):
    """Tokens whose oracle margins are >= 1e-3 at every layer, with their oracle results."""
    prov = stack.provider()
    out = []
    d = start
    while len(out) < n:
        x = synth.token(stack.seed, d, stack.H)
        if prenorm:
            ref = oracle.stack(prov, stack.routers_np, x, stack.I, k, stack.bits, 64, 1e-6, stop_margin=1e-3,
                               shared_gates=stack.gates_np)
            ok = ref["layers_done"] == stack.L and np.min(ref["margins"]) >= 1e-3
        else:
            assert stack.L == 1
            o, i_, w_, m = oracle.moe_layer(prov, 0, stack.routers_np[0], x.astype(np.float64), stack.I, k,
                                            stack.bits, 64, 0, 1e-6)
            ref = dict(out=o, idx=i_[None, :], w=w_[None, :], margins=np.array([m]))
            ok = m >= 1e-3
        if ok:
            out.append((x, ref))
        d += 1
    return out


@pytest.mark.parametrize("L,E,H,I,k,bits", [
    (5, 64, 1024, 256, 4, 4), (4, 64, 1024, 256, 4, 2), (3, 16, 256, 64, 1, 4), (2, 16, 512, 128, 16, 4),
    (3, 8, 4096, 1024, 4, 4), (2, 300, 2048, 512, 8, 2), (3, 1000, 128, 64, 2, 4),
    (4, 64, 1024, 256, 4, 3), (2, 300, 2048, 512, 8, 3), (3, 16, 256, 64, 1, 3), (2, 40, 8192, 128, 2, 3),
    (2, 24, 512, 8192, 1, 3)])
def test_decode_stack(L, E, H, I, k, bits):
    """Experts of the whole stack bit-exact against the oracle's fp64 trajectory, and every
    layer within the bar against the oracle layer applied to the kernel's own input to it
    (gpu_util.check_stack_layers)."""
    stack = DevStack(L, E, H, I, bits)
    for x, ref in _stack_tokens(stack, k, 3):
        h, idx, w = _decode(stack, x, k)
        assert np.array_equal(idx, ref["idx"])
        assert rel_l2(w[0], ref["w"][0]) <= TOL  # the first layer sees the exact input
        check_stack_layers(stack, x, k, h)


@pytest.mark.parametrize("L,E,H,I,k,bits", [
    (3, 64, 1024, 256, 4, 4), (3, 40, 512, 128, 2, 2), (2, 16, 256, 64, 1, 4), (2, 16, 512, 128, 15, 4),
    (2, 600, 1024, 128, 4, 2), (3, 40, 512, 128, 2, 3)])
def test_decode_shared_expert(L, E, H, I, k, bits):
    """Layers with a shared expert (blob index E) added with weight sigmoid(gate . v): routing
    of the whole stack bit-exact against the oracle stack with the same gates, and every
    layer within the bar against the oracle layer applied to the kernel's own input to it
    (runs of the first l layers). Across layers a token's fp32 error can be amplified by the
    later layers' sensitivity (measured: 1e-6 after two 2-bit layers became 1.3e-5 after the
    third, whose own error from an exact input is 2.3e-7), so the stack output is compared
    layer by layer rather than against the fp64 trajectory. k = 15 is the most with a
    shared slot."""
    _check_shared_stack(DevStack(L, E, H, I, bits, shared=True), k, 3)


def test_decode_shared_expert_full_size():
    """The compiled decode shape with a shared expert: two pre-normed layers of 512 experts
    plus the shared one, hidden 4096, inter 1024, top-4, 4-bit."""
    _check_shared_stack(DevStack(2, 512, 4096, 1024, 4, gpu_fill=True, shared=True), 4, 2)


def _check_shared_stack(stack, k, n_tokens):
    L, E, H, I, bits = stack.L, stack.E, stack.H, stack.I, stack.bits
    prov = stack.provider()
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H, I, E, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for x, ref in _stack_tokens(stack, k, n_tokens):
        h, idx, w = _decode(stack, x, k)
        assert np.array_equal(idx, ref["idx"])
        assert rel_l2(w, ref["w"]) <= TOL
        # the shared expert contributes: its weight is strictly between 0 and 1
        assert np.all((ref["shared_w"] > 0) & (ref["shared_w"] < 1))
        h_in = x.astype(np.float32)
        for l in range(L):
            sub = fm.layers_array([stack.layers[j] for j in range(l + 1)])
            hd = torch.empty(H, dtype=torch.float32, device="cuda")
            fm.moe_layer(sub, to_dev(x.astype(np.float32)), hd, 1, k, 1e-6, fm.PRENORM, None, None, ws, wsb)
            torch.cuda.synchronize()
            h_l = hd.cpu().numpy()
            want, i_l, _, _ = oracle.moe_layer(prov, l, stack.routers_np[l], h_in.astype(np.float64), I, k, bits,
                                               64, 1, 1e-6, shared_gate=stack.gates_np[l])
            assert i_l.tolist() == ref["idx"][l].tolist()
            assert rel_l2(h_l, want) <= TOL, l
            h_in = h_l
        assert np.array_equal(h_in, h)  # the last run is the whole stack


def test_decode_shared_expert_rejections():
    """k + 1 > 16 with a shared expert and mixed layers (one with, one without a gate) are
    refused before any launch."""
    stack = DevStack(2, 16, 256, 64, 4, shared=True)
    xd = to_dev(synth.token(0, 0, 256)[None, :].astype(np.float32))
    hd = torch.empty((1, 256), dtype=torch.float32, device="cuda")
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 2, 256, 64, 16, 16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    with pytest.raises(fm.FmoeError) as ei:
        fm.moe_layer(stack.layers, xd, hd, 1, 16, 1e-6, fm.PRENORM, None, None, ws, wsb)
    assert ei.value.status == fm.ERR_K
    mixed = fm.layers_array([stack.layers[0], fm.Layer(stack.layers[1].router, stack.layers[1].experts,
                                                       stack.stride, 16, 256, 64, 4, 64)])
    with pytest.raises(fm.FmoeError) as ei:
        fm.moe_layer(mixed, xd, hd, 1, 4, 1e-6, fm.PRENORM, None, None, ws, wsb)
    assert ei.value.status == fm.ERR_SHAPE


def test_decode_stack_full_size_top10():
    """Top-10 routing (k as a free parameter) at the full layer shape: two pre-normed layers
    of 512 experts, hidden 4096, inter 1024, 4-bit."""
    stack = DevStack(2, 512, 4096, 1024, 4, gpu_fill=True)
    for x, ref in _stack_tokens(stack, 10, 2):
        h, idx, w = _decode(stack, x, 10)
        assert np.array_equal(idx, ref["idx"])
        assert rel_l2(w, ref["w"]) <= TOL
        assert rel_l2(h, ref["out"]) <= TOL


def test_decode_many_layers_chunked():
    """More layers than one persistent launch holds (64): chunked launches share the state."""
    stack = DevStack(70, 8, 128, 64, 4)
    (x, ref), = _stack_tokens(stack, 2, 1)
    h, idx, w = _decode(stack, x, 2)
    assert np.array_equal(idx, ref["idx"])
    assert rel_l2(h, ref["out"]) <= TOL


def test_decode_config2_one_layer_full():
    """One MoE layer, one token: hidden 4096, 512 experts 4-bit g64 (3.6 GB), fp32 router
    N(0, 0.02), top-4 softmax-weighted, SwiGLU, residual add, no norm."""
    stack = DevStack(1, 512, 4096, 1024, 4, gpu_fill=True)
    for x, ref in _stack_tokens(stack, 4, 3, prenorm=False):
        h, idx, w = _decode(stack, x, 4, prenorm=False)
        assert idx[0].tolist() == ref["idx"][0].tolist()
        assert rel_l2(w[0], ref["w"][0]) <= TOL
        assert rel_l2(h, ref["out"]) <= TOL
        h2, _, _ = _decode(stack, x, 4, prenorm=False)
        assert np.array_equal(h, h2)  # deterministic (no atomics)
