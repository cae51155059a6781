"""fmoe_moe_layer_noalloc (the library's static scratch instead of a caller workspace)
against fmoe_moe_layer on a fresh workspace, through the C-ABI: equal results (bit for
bit: the same kernels, deterministic) on calls in a row whose inputs shrink, across the
multi-token and single-token paths; a call too large for the scratch is refused before
anything is enqueued."""
import numpy as np
import pytest
import torch

import quantized_expert_ffn_fmoe_amd as fm
import synth
from gpu_util import DevStack, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _both(stack, X, T, k, flags=fm.PRENORM, extra=0):
    H, L = stack.H, stack.L
    xd = to_dev(X[:T].astype(np.float32))
    outs = []
    for which in ("noalloc", "workspace"):
        h = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, L, k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, L, k), float("nan"), dtype=torch.float32, device="cuda")
        if which == "noalloc":
            fm.moe_layer_noalloc(stack.layers, xd, h, T, k, 1e-6, flags | extra, idx, w)
        else:
            wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, T, H, stack.I, stack.E, k)
            ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
            fm.moe_layer(stack.layers, xd, h, T, k, 1e-6, flags, idx, w, ws, wsb)
        torch.cuda.synchronize()
        outs.append((h.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    return outs


def test_noalloc_equals_workspace_calls_in_a_row():
    stack = DevStack(2, 64, 1024, 256, 4)
    X = np.stack([synth.token(0, d, 1024) for d in range(48)])
    # larger then smaller inputs: multi-token 48, 12, 2 tokens, then single tokens
    for T, k, extra in [(48, 4, 0), (12, 4, 0), (2, 8, 0), (1, 4, 0), (1, 8, fm.RESET_SCRATCH), (1, 2, 0)]:
        (h0, i0, w0), (h1, i1, w1) = _both(stack, X, T, k, extra=extra)
        assert np.all(np.isfinite(h0)), (T, k)
        assert np.array_equal(i0, i1), (T, k)
        assert np.array_equal(w0, w1), (T, k)
        assert np.array_equal(h0, h1), (T, k)


def test_noalloc_full_size_decode_then_smaller_batch():
    """The compiled 512-expert decode shape (two pre-normed layers, hidden 4096, top-4),
    then a 16-token multi-token call and a 4-token one on the same scratch."""
    stack = DevStack(2, 512, 4096, 1024, 4, gpu_fill=True)
    X = np.stack([synth.token(0, d, 4096) for d in range(16)])
    for T in (1, 16, 4, 1):
        (h0, i0, _), (h1, i1, _) = _both(stack, X, T, 4)
        assert np.all(np.isfinite(h0)), T
        assert np.array_equal(i0, i1), T
        assert np.array_equal(h0, h1), T


def test_noalloc_refuses_calls_beyond_the_scratch():
    stack = DevStack(1, 64, 1024, 256, 4)
    T = 2048
    assert fm.workspace_bytes(fm.OP_MOE_LAYER, T, 1024, 256, 64, 4) > 32 << 20
    xd = torch.zeros((T, 1024), dtype=torch.float32, device="cuda")
    h = torch.full((T, 1024), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(fm.FmoeError) as ei:
        fm.moe_layer_noalloc(stack.layers, xd, h, T, 4, 1e-6, 0, None, None)
    assert ei.value.status == fm.ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((h == 7.0).all())  # nothing was enqueued
