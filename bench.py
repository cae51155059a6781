#!/usr/bin/env python3
"""Benchmark of the MoE expert-block decode on one MI355X.

Workload (default, --config stack4): 60 layers x 512 experts, hidden 4096, expert
intermediate 1024, 4-bit codes with bf16 scale/bias per group of 64 (about 217 GB resident
in HBM), fp32 routers N(0, 0.02), top-4 softmax routing, SwiGLU, combine + residual, RMS
norm (eps 1e-6) before every layer; 256 consecutive single-token decodes (each token one
fmoe_moe_layer call through all 60 layers). Inputs are synthetic (seeded generator, token
draws 0..255 ~ N(0,1)); the expert set is generated on the device.

A step is one pass of the 256 tokens. Prints one JSON line: tokens/s, the decode kernel's
achieved HBM bandwidth against the 8 TB/s peak (HIP events around each step's launches), a parity
spot check of the full-size stack against stored oracle results, the measured inter-token
expert reuse, and the CPU oracle's throughput on a small sample (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps 5] [--warmup 1]
       [--config stack4|stack3|stack2|layer|matvec|batch64|batch64_3bit|batch64_2bit|qkv4|qkv2]
       [--top-k K] [--shared]
(layer: one MoE layer per call over the 60 distinct layers, us per layer-token; matvec: one
1024 x 4096 4-bit dequant matvec over a pool of 512 matrices, us per call; batch64: 64 tokens
through one layer on the grouped path; qkv4 / qkv2: the fused multi-output projection,
4096 + 512 + 512 rows x 4096 columns of one input, over 16 rotated weight sets.)
A run whose parity check fails, or whose outputs are not finite, prints a JSON line with an
"error" key and exits with status 1.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

L_, E_, H_, I_, K_, EPS = 60, 512, 4096, 1024, 4, 1e-6
PEAK_GBS = 8000.0
METRIC = "MoE-block decode tokens/s (60 layers, 4-bit) + achieved HBM GB/s vs peak"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


SHARED = False  # --shared: every layer also has a shared expert and its gate


def algorithmic_bytes_per_layer(bits: int) -> int:
    import quantized_expert_ffn_fmoe_amd as fm
    shared = (fm.expert_bytes(H_, I_, bits) + H_ * 4) if SHARED else 0  # the shared expert + its gate row
    return E_ * H_ * 4 + K_ * fm.expert_bytes(H_, I_, bits) + shared


def stream_read_probe(torch) -> dict:
    """The attainable read rate of plain streaming code here: the better of measure/measure.hip's
    read-only streaming kernel (best variant) and its row-stage LDS-DMA read (128-byte pieces of
    64 rows per 8-KB stage, rows of 2048 and 512 bytes, and 512-byte pieces of 2-KB rows with 4
    stages in flight), each over 4 GiB, HIP events on the launch stream."""
    import measure

    s = measure.stream_read(torch)
    r = measure.row_stages(torch, configs=((2048, 2, 128), (2048, 4, 512), (512, 2, 128)), verbose=False)
    return {"kind": "best of the read-only streaming kernel and the row-stage LDS-DMA read (measure.hip), "
                    "4 GiB each, best of 5 passes per variant",
            "gbs": max(s["gbs"], r["gbs"]), "stream_gbs": s["gbs"], "row_stage_gbs": r["gbs"],
            "variants": s["variants"], "row_stage_variants": r["rows"]}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def omp_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def fail(msg: str, **extra) -> int:
    """A run whose results are not valid: one JSON line saying why, and a non-zero status."""
    print(json.dumps(dict({"error": msg}, **extra)), flush=True)
    return 1


def workspace_error_word(torch, ws, wsb) -> int:
    import quantized_expert_ffn_fmoe_amd as fm

    err = torch.zeros(1, dtype=torch.int32, device=ws.device)
    fm.workspace_error(ws, wsb, err)
    torch.cuda.synchronize()
    return int(err.item())


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines (string literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':  # string literal
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(ln.rstrip() for ln in "".join(out).splitlines() if ln.strip())


def decode_source_hash() -> str:
    """Hash of the decode kernel's sources with comments removed: the committed HBM-traffic
    counters (profiles/) stay attached to the kernel as long as its code is unchanged."""
    h = hashlib.sha256()
    for f in ("fmoe_decode.hip", "fmoe_device.h", "fmoe_decode.h", "fmoe_intdot.h", "fmoe_layout.h"):
        h.update(_code_only(open(os.path.join(ROOT, "quantized_expert_ffn_fmoe_amd", "csrc", f)).read()).encode())
    return h.hexdigest()[:16]


def build_stack(bits: int, dev):
    import torch

    import quantized_expert_ffn_fmoe_amd as fm
    import synth
    from gpu_util import fill_experts_gpu, to_dev

    eb = fm.expert_bytes(H_, I_, bits)
    stride = (eb + 255) // 256 * 256
    blobs, routers, layers = [], [], []
    nb = E_ + (1 if SHARED else 0)  # a shared expert is blob index E_
    t0 = time.time()
    for l in range(L_):
        blob = torch.empty(nb * stride, dtype=torch.uint8, device=dev)
        fill_experts_gpu(blob, stride, l, nb, H_, I_, bits, seed=0)
        R = to_dev(synth.router(0, l, E_, H_), dev)
        blobs.append(blob)
        routers.append(R)
        gate = 0
        if SHARED:  # gate N(0, 0.02) from its own generator stream
            g = to_dev(synth.router(0, 1000 + l, 1, H_)[0], dev)
            routers.append(g)
            gate = g.data_ptr()
        layers.append(fm.Layer(R.data_ptr(), blob.data_ptr(), stride, E_, H_, I_, bits, 64, gate))
        if l % 10 == 9:
            torch.cuda.synchronize()
            log(f"filled layer {l + 1}/{L_} ({time.time() - t0:.0f}s, {(l + 1) * E_ * stride / 1e9:.1f} GB)")
    torch.cuda.synchronize()
    return blobs, routers, fm.layers_array(layers), nb * stride * L_


def cpu_baseline(bits: int, n_tokens: int = 4, runs: int = 3):
    """The oracle, as it stands, on the host: n_tokens draws through all 60 layers, `runs`
    times; the median run is reported. Expert generation (done on demand inside the
    oracle's provider) is timed separately and subtracted."""
    import oracle
    import synth

    routers = [synth.router(0, l, E_, H_) for l in range(L_)]
    gates = shared_gates_np()
    prov = synth.Provider(0, H_, I_, bits)
    times, gens = [], []
    for _ in range(runs):
        t_total = t_gen = 0.0
        for d in range(n_tokens):
            x = synth.token(0, d, H_)
            t0 = time.perf_counter()
            r = oracle.stack(prov, routers, x, I_, K_, bits, 64, EPS, keep_all=False, shared_gates=gates)
            t_total += time.perf_counter() - t0
            t0 = time.perf_counter()
            for l in range(L_):
                for e in list(r["idx"][l]) + ([E_] if SHARED else []):
                    synth.expert(0, l, int(e), H_, I_, bits)
            t_gen += time.perf_counter() - t0
        times.append(max(t_total - t_gen, 1e-9))
        gens.append(t_gen)
    t_med = float(np.median(times))
    return {"value": round(n_tokens / t_med, 6), "unit": "tokens/s", "cores": omp_threads(), "kind": "oracle",
            "sample": f"{n_tokens} tokens (draws 0-{n_tokens - 1}) through all {L_} layers ({bits}-bit, top-{K_}"
                      f"{', shared expert' if SHARED else ''}), "
                      f"fp64 plain loops, OpenMP over rows; median of {runs} runs; on-demand expert generation "
                      f"(median {np.median(gens):.1f}s per run) subtracted",
            "seconds": round(t_med, 3), "runs_s": [round(t, 3) for t in times], "cpu": cpu_model()}


def parity_check(layers, bits, dev, ws, wsb):
    import torch

    import quantized_expert_ffn_fmoe_amd as fm
    import synth

    path = os.path.join(ROOT, "tests", "golden", f"stack_full_{bits}bit.npz")
    if not os.path.exists(path):
        return None
    g = np.load(path, allow_pickle=False)
    worst, exact = 0.0, True
    for i, d in enumerate(g["draw"]):
        x = torch.from_numpy(synth.token(0, int(d), H_)).to(dev)
        h = torch.empty(H_, dtype=torch.float32, device=dev)
        idx = torch.empty((L_, K_), dtype=torch.int32, device=dev)
        fm.moe_layer(layers, x, h, 1, K_, EPS, fm.PRENORM, idx, None, ws, wsb)
        torch.cuda.synchronize()
        exact &= bool(np.array_equal(idx.cpu().numpy(), g["idx"][i]))
        ref = g["out"][i]
        rel = float(np.linalg.norm(h.cpu().numpy().astype(np.float64) - ref) / np.linalg.norm(ref))
        worst = max(worst, rel)
    return {"tokens": int(len(g["draw"])), "draws": [int(d) for d in g["draw"]], "experts_bit_exact": exact,
            "max_rel_l2": worst, "tolerance": 1e-5, "pass": bool(exact and worst <= 1e-5)}


def shared_gates_np():
    import synth

    return [synth.router(0, 1000 + l, 1, H_)[0] for l in range(L_)] if SHARED else None


def live_parity(layers, bits, dev, ws, wsb, n_tokens: int = 2):
    """Parity against the live oracle for workloads without stored results (top-k != 4, a
    shared expert), layer by layer on the kernel's own input: tokens are draws 0..n_tokens-1;
    for each layer l the kernel's h after layers 0..l is compared with the oracle layer
    applied to the kernel's h after layers 0..l-1 (experts bit-exact, output within 1e-5)
    wherever the oracle's top-k margin there is >= 1e-3 (elsewhere the selection is decided
    by rounding and either choice is right). With top-10 routing few tokens keep that margin
    through all 60 layers, so the layer is the unit; at least 90% of the layers must be
    checked."""
    import torch

    import oracle
    import quantized_expert_ffn_fmoe_amd as fm
    import synth

    routers = [synth.router(0, l, E_, H_) for l in range(L_)]
    gates = shared_gates_np()
    prov = synth.Provider(0, H_, I_, bits)
    exact, worst, checked = True, 0.0, 0
    for d in range(n_tokens):
        x = synth.token(0, d, H_)
        xd = torch.from_numpy(x).to(dev)
        hs, ids = [], []
        for l in range(L_):  # the kernel's h and experts after layers 0..l
            h = torch.empty(H_, dtype=torch.float32, device=dev)
            idx = torch.empty((l + 1, K_), dtype=torch.int32, device=dev)
            sub = fm.layers_array([layers[j] for j in range(l + 1)])
            fm.moe_layer(sub, xd, h, 1, K_, EPS, fm.PRENORM, idx, None, ws, wsb)
            torch.cuda.synchronize()
            hs.append(h.cpu().numpy().astype(np.float64))
            ids.append(idx.cpu().numpy()[l])
        h_in = x.astype(np.float64)
        for l in range(L_):
            want, i_ref, _, m = oracle.moe_layer(prov, l, routers[l], h_in, I_, K_, bits, 64, 1, EPS,
                                                 shared_gate=None if gates is None else gates[l])
            if m >= 1e-3:
                checked += 1
                exact &= bool(np.array_equal(ids[l], i_ref))
                worst = max(worst, float(np.linalg.norm(hs[l] - want) / np.linalg.norm(want)))
            h_in = hs[l]
    ok = exact and worst <= 1e-5 and checked >= 0.9 * L_ * n_tokens
    return {"tokens": n_tokens, "draws": list(range(n_tokens)), "layers_checked": checked,
            "layers_total": L_ * n_tokens, "experts_bit_exact": exact, "max_rel_l2_per_layer": worst,
            "tolerance": 1e-5, "reference": "live oracle, layer by layer on the kernel's own input",
            "pass": bool(ok)}


def traffic_from_profiles(kernel_tag: str):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, if they were taken on the
    current decode kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != decode_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def calibrate_copy(torch) -> int:
    """Three copies of 1 GiB between two device buffers: each moves exactly 2^30 bytes in and
    2^30 bytes out of HBM, which is what the FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "copies": 3}), flush=True)
    return 0


def run_batch64(args, torch, bits: int = 4) -> int:
    """64 tokens x 1 layer through the grouped (bf16 matrix-core) path, rotating over 8
    independent 512-expert layers so that no call finds its experts in cache. Expert
    popularity is Zipf(1.1), planted through each layer's router."""
    import quantized_expert_ffn_fmoe_amd as fm
    import synth
    from gpu_util import fill_experts_gpu, to_dev

    NL, T = 8, 64
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    eb = fm.expert_bytes(H_, I_, bits)
    stride = (eb + 255) // 256 * 256
    gpath = os.path.join(ROOT, "tests", "golden", f"batch64_{bits}bit.npz")
    golden = np.load(gpath, allow_pickle=False) if os.path.exists(gpath) else None
    log(f"building {NL} independent {E_}-expert {bits}-bit layers")
    blobs, routers, layers, Xs = [], [], [], []
    for l in range(NL):
        blob = torch.empty(E_ * stride, dtype=torch.uint8, device=dev)
        fill_experts_gpu(blob, stride, l, E_, H_, I_, bits, seed=0)
        Rn = synth.router(0, l, E_, H_)
        R = to_dev(Rn, dev)
        blobs.append(blob)
        routers.append(R)
        layers.append(fm.layers_array([fm.Layer(R.data_ptr(), blob.data_ptr(), stride, E_, H_, I_, bits, 64)]))
        draws = [int(d) for d in golden["draw"]] if (l == 0 and golden is not None) else list(range(T))
        Xs.append(to_dev(np.stack([synth.planted_token(0, d, Rn, K_)[0] for d in draws]), dev))
    torch.cuda.synchronize()
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, T, H_, I_, E_, K_)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    outs = torch.empty((NL, T, H_), dtype=torch.float32, device=dev)
    idxs = torch.empty((NL, T, 1, K_), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # HIP events around each step's NL back-to-back calls (an event pair around every call
    # would put its own records between the calls' kernels); a call's average duration is a
    # step's time over NL
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def call(l):
        fm.moe_layer(layers[l], Xs[l], outs[l], T, K_, EPS, 0, idxs[l], None, ws, wsb, stream.cuda_stream)

    for _ in range(args.warmup):
        for l in range(NL):
            call(l)
    torch.cuda.synchronize()
    log(f"timing {args.steps} step(s) of {NL} calls")
    t0 = time.perf_counter()
    for s_i in range(args.steps):
        ev0[s_i].record(stream)
        for l in range(NL):
            call(l)
        ev1[s_i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = np.array([ev0[i].elapsed_time(ev1[i]) for i in range(args.steps)])
    ids = idxs.cpu().numpy()
    distinct = [len(np.unique(ids[l])) for l in range(NL)]
    bytes_call = [E_ * H_ * 4 + d * eb + 2 * T * H_ * 4 for d in distinct]
    achieved = float(args.steps * sum(bytes_call) / (step_ms.sum() * 1e-3) / 1e9)
    call_us = float(step_ms.sum() * 1e3 / (args.steps * NL))
    tok_s = args.steps * NL * T / elapsed
    log(f"{tok_s:.0f} tok/s, call avg {call_us:.1f} us, {achieved:.0f} GB/s, distinct experts {distinct}")
    parity = None
    if golden is not None and not args.no_parity:
        out0 = outs[0].cpu().numpy().astype(np.float64)
        rel = [float(np.linalg.norm(out0[t] - golden["out"][t]) / np.linalg.norm(golden["out"][t])) for t in range(T)]
        exact = bool(np.array_equal(ids[0, :, 0, :], golden["idx"]))
        parity = {"tokens": T, "experts_bit_exact": exact, "max_rel_l2_vs_bf16_contract": max(rel),
                  "tokens_within_1e-5": float(np.mean(np.array(rel) <= 1e-5)), "tolerance": 2.0 ** -8,
                  "pass": bool(exact and max(rel) <= 2.0 ** -8)}
        log(f"parity: {parity}")
    elif not args.no_parity:
        # no stored expected values at this width: the oracle (O7 contract) on 8 tokens of layer 0
        import oracle

        n = 8
        ref = oracle.layer_bf16(synth.Provider(0, H_, I_, bits), 0, synth.router(0, 0, E_, H_),
                                Xs[0][:n].cpu().numpy(), I_, K_, bits, 64)
        out0 = outs[0][:n].cpu().numpy().astype(np.float64)
        rel = [float(np.linalg.norm(out0[t] - ref["out"][t]) / np.linalg.norm(ref["out"][t])) for t in range(n)]
        exact = bool(np.array_equal(ids[0, :n, 0, :], ref["idx"]))
        parity = {"tokens": n, "experts_bit_exact": exact, "max_rel_l2_vs_bf16_contract": max(rel),
                  "tolerance": 2.0 ** -8, "pass": bool(exact and max(rel) <= 2.0 ** -8), "reference": "live oracle"}
        log(f"parity: {parity}")
    if parity is not None and not parity["pass"]:
        return fail("parity check failed", parity=parity)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        Rn = synth.router(0, 0, E_, H_)
        X0 = Xs[0][:16].cpu().numpy()
        prov = synth.Provider(0, H_, I_, bits)
        t1 = time.perf_counter()
        oracle.layer_bf16(prov, 0, Rn, X0, I_, K_, bits, 64)
        t_or = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = {"value": round(16 / t_or, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "16 of the 64 tokens of layer 0, O7 bf16 contract in fp64 plain loops (OpenMP over rows), "
                         "expert generation included", "seconds": round(t_or, 3)}
    out = {
        "metric": f"MoE-block batched prefill tokens/s (64 tokens x 1 layer, {bits}-bit) + achieved HBM GB/s vs peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{T} tokens x 1 layer, {E_} experts {bits}-bit group 64, top-{K_}, Zipf(1.1) "
                               f"popularity planted through the router; {NL} independent layers rotated per call",
                   "experts": E_, "hidden": H_, "inter": I_, "top_k": K_, "bits": bits, "tokens_per_call": T,
                   "calls_per_step": NL, "distinct_experts_per_call": distinct},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": None,
                     "kernel": "fmoe batched layer call (router, route/stage/sort, gate/up, down, combine kernels)",
                     "algorithmic_bytes_per_launch": int(np.mean(bytes_call)),
                     "avg_launch_us": round(call_us, 2),
                     "timing": "HIP events around each step's back-to-back calls (a launch = one call)"},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    del blobs, routers, layers, Xs, outs, idxs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


def run_qkv(args, torch, bits: int) -> int:
    """Fused Q/K/V-like projection (fmoe_dequant_matvec_multi): 4096 + 512 + 512 rows x 4096
    columns applied to one input vector, rotating over 16 independent weight sets (189 MB at
    4 bits) so that no call finds its weights in cache. The 16 calls of a step are captured
    once in a HIP graph and replayed (a call takes about as long as its Python submission,
    so eagerly submitted calls would time the host)."""
    import quantized_expert_ffn_fmoe_amd as fm
    import oracle
    import synth
    from gpu_util import DevMatrix, rel_l2, to_dev

    NS, cols, rows_list = 16, H_, [4096, 512, 512]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host0, sets = [], []
    for i in range(NS):
        ms = []
        for m, rows in enumerate(rows_list):
            c, sc, b = synth.matrix(21, i, m, 0, rows, cols, bits)
            ms.append(DevMatrix(c, sc, b, rows, cols, bits))
            if i == 0:
                host0.append((c, sc, b, rows))
        sets.append(ms)
    xn = synth.token(0, 0, cols)
    x = to_dev(xn[None, :], dev)
    outs = [torch.empty((1, r), dtype=torch.float32, device=dev) for r in rows_list]
    nbytes = sum(fm.codes_bytes(r, cols, bits) + fm.sb_bytes(r, cols) + 4 * r for r in rows_list) + 4 * cols
    qs = [[d.q for d in ms] for ms in sets]
    # eager reference for the last set, then the graph of one step
    ref = [torch.empty_like(o) for o in outs]
    fm.dequant_matvec_multi(qs[NS - 1], x, ref, 1, torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(NS):
                fm.dequant_matvec_multi(qs[i], x, outs, 1, cap.cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    for _ in range(max(1, args.warmup)):
        g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(outs, ref))
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        ev0[st].record(stream)
        g.replay()
        ev1[st].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    same = same and all(torch.equal(a, b) for a, b in zip(outs, ref))
    call_us = np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)]) * 1e3 / NS
    avg_us = float(call_us.mean())
    if not same:
        log("graph replay differs from the eager call")
    achieved = nbytes / avg_us / 1e3
    log(f"fused projection: {avg_us:.2f} us per call (HIP events), {achieved:.0f} GB/s")
    parity = None
    if not args.no_parity:
        fm.dequant_matvec_multi(qs[0], x, outs, 1, stream.cuda_stream)
        torch.cuda.synchronize()
        rel = [rel_l2(outs[m].cpu().numpy()[0], oracle.matvec(c, sc, b, rows, cols, bits, 64, xn))
               for m, (c, sc, b, rows) in enumerate(host0)]
        parity = {"matrices": len(rel), "max_rel_l2": max(rel), "tolerance": 1e-5,
                  "graph_replay_equals_eager": bool(same), "pass": bool(max(rel) <= 1e-5 and same)}
        log(f"parity: {parity}")
        if not parity["pass"]:
            return fail("parity check failed", parity=parity)
    cpu = None
    if not args.no_cpu_baseline:
        t1 = time.perf_counter()
        for (c, sc, b, rows) in host0:
            oracle.matvec(c, sc, b, rows, cols, bits, 64, xn)
        t_or = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = {"value": round(t_or * 1e6, 1), "unit": "us per call", "cores": threads, "kind": "oracle",
               "sample": "one weight set (3 matrices), O2 in fp64", "seconds": round(t_or, 3)}
    out = {
        "metric": f"fused Q/K/V dequant projection us per call ({bits}-bit) + achieved HBM GB/s vs peak",
        "value": round(avg_us, 2), "unit": "us per call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"4096 + 512 + 512 rows x {cols} columns, {bits}-bit group 64, one input vector; "
                               f"{NS} independent weight sets rotated per call", "bits": bits,
                   "calls_per_step": NS},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": None,
                     "kernel": "fmoe::matvec_multi_kernel", "algorithmic_bytes_per_launch": int(nbytes),
                     "avg_launch_us": round(avg_us, 2),
                     "timing": "HIP events around replays of a graph of 16 calls, divided by 16"},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


def graph_of(torch, dev, fn):
    """Capture fn() (calls on the given stream handle) once in a HIP graph; returns it."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            fn(cap.cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    return g


def time_replays(torch, dev, g, steps: int) -> list:
    """HIP events on the current stream around each of `steps` replays of graph g (ms)."""
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def run_matvec(args, torch) -> int:
    """One dequantized matvec, W 1024 x 4096 4-bit group 64 (bf16 s, b), x f32[4096], seed
    0. A pool of 512 distinct matrices (1.21 GB, more than 4x the 256 MB Infinity Cache) is
    swept in one HIP graph of 512 calls, so every call streams its matrix from HBM; the
    graph holds the calls back to back, so launch gaps count. Single-call latency: one call
    captured alone, replayed (its matrix then stays in cache)."""
    import oracle
    import quantized_expert_ffn_fmoe_amd as fm
    import synth
    from gpu_util import rel_l2

    NP, rows, cols, bits = 512, 1024, 4096, 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb, nsb = fm.codes_bytes(rows, cols, bits), fm.sb_bytes(rows, cols)
    codes = torch.empty((NP, cb), dtype=torch.uint8, device=dev)
    sbs = torch.empty((NP, nsb // 4), dtype=torch.int32, device=dev)
    ng = rows * cols // 64
    chunk = 64
    c_tmp = torch.empty((chunk, cb), dtype=torch.uint8, device=dev)
    s_tmp = torch.empty((chunk, ng), dtype=torch.int16, device=dev)
    b_tmp = torch.empty((chunk, ng), dtype=torch.int16, device=dev)
    hs = torch.cuda.current_stream(dev).cuda_stream
    for m0 in range(0, NP, chunk):  # matrix m = the gate matrix of expert m of layer 0
        synth.gpu_matrix(0, 0, m0, chunk, 0, rows, cols, bits, 64, c_tmp.data_ptr(), cb, s_tmp.data_ptr(),
                         b_tmp.data_ptr(), ng * 2, hs)
        for j in range(chunk):
            fm.pack(c_tmp[j], s_tmp[j], b_tmp[j], rows, cols, bits, 64, codes[m0 + j], sbs[m0 + j])
    torch.cuda.synchronize()
    del c_tmp, s_tmp, b_tmp
    xn = synth.token(0, 0, cols)
    x = torch.from_numpy(xn).to(dev)
    Y = torch.empty((NP, rows), dtype=torch.float32, device=dev)
    qs = [fm.qmat(codes[m], sbs[m], rows, cols, bits) for m in range(NP)]

    def sweep(h):
        for m in range(NP):
            fm.dequant_matvec(qs[m], x, Y[m], 1, h)

    g_pool = graph_of(torch, dev, sweep)
    g_one = graph_of(torch, dev, lambda h: fm.dequant_matvec(qs[0], x, Y[0], 1, h))
    for _ in range(max(1, args.warmup)):
        g_pool.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} sweep(s) of {NP} calls")
    t0 = time.perf_counter()
    ms = time_replays(torch, dev, g_pool, args.steps)
    elapsed = time.perf_counter() - t0
    per_call_us = float(np.median(ms)) * 1e3 / NP
    lat = time_replays(torch, dev, g_one, 50)
    lat_us = float(np.median(lat)) * 1e3
    nbytes = cb + nsb + 4 * cols + 4 * rows
    achieved = nbytes / per_call_us / 1e3
    log(f"matvec: {per_call_us:.2f} us per call in the pool sweep ({achieved:.0f} GB/s), single call {lat_us:.2f} us")
    parity = None
    if not args.no_parity:
        worst = 0.0
        for m in (0, 1, 255, 511):
            c, sc, b = synth.matrix(0, 0, m, 0, rows, cols, bits)
            worst = max(worst, rel_l2(Y[m].cpu().numpy(), oracle.matvec(c, sc, b, rows, cols, bits, 64, xn)))
        parity = {"matrices_checked": [0, 1, 255, 511], "max_rel_l2": worst, "tolerance": 1e-5,
                  "pass": bool(worst <= 1e-5)}
        log(f"parity: {parity}")
        if not parity["pass"]:
            return fail("parity check failed", parity=parity)
    cpu = None
    if not args.no_cpu_baseline:
        c, sc, b = synth.matrix(0, 0, 0, 0, rows, cols, bits)
        ts = []
        for _ in range(3):
            t1 = time.perf_counter()
            for _ in range(20):
                oracle.matvec(c, sc, b, rows, cols, bits, 64, xn)
            ts.append((time.perf_counter() - t1) / 20)
        cpu = {"value": round(float(np.median(ts)) * 1e6, 1), "unit": "us per call", "cores": omp_threads(),
               "kind": "oracle", "sample": "matrix 0, 20 calls of O2 (fp64, OpenMP over rows) per run, median of "
                                           "3 runs", "cpu": cpu_model()}
    out = {
        "metric": "dequant matvec us per call (1024x4096 4-bit group 64) + achieved HBM GB/s vs peak",
        "value": round(per_call_us, 3), "unit": "us per call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"fmoe_dequant_matvec, W {rows}x{cols} {bits}-bit group 64, x f32[{cols}], seed 0; "
                               f"a pool of {NP} distinct matrices ({NP * (cb + nsb) / 1e9:.2f} GB) swept per step",
                   "rows": rows, "cols": cols, "bits": bits, "pool": NP},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": None, "kernel": "fmoe::matvec_kernel",
                     "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_us": round(per_call_us, 3),
                     "timing": f"HIP events around replays of a graph of the {NP}-call sweep, divided by {NP}"},
        "single_call_latency_us": round(lat_us, 3),
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    del codes, sbs, Y, g_pool, g_one
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


def run_layer(args, torch) -> int:
    """One MoE layer for one token without a norm (route, 4 experts, SwiGLU, combine, residual
    add), hidden 4096, 512 experts 4-bit. Measured per layer over the 60 distinct layers of
    the 60-layer stack (one call per layer, so each call finds its router and experts cold);
    layer l's token is the first N(0, 1) draw whose oracle top-4 margin there is >= 1e-3.
    The 60 calls of a step are captured in one HIP graph; a step's time / 60 is the time per
    layer-token (launch gaps included)."""
    import oracle
    import quantized_expert_ffn_fmoe_amd as fm
    import synth

    bits = 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"building the {L_}-layer {bits}-bit stack")
    blobs, routers, layers, resident = build_stack(bits, dev)
    routers_np = [synth.router(0, l, E_, H_) for l in range(L_)]
    X, draws = [], []
    for l in range(L_):
        d = 0
        while oracle.route(routers_np[l], synth.token(0, d, H_), K_)[3] < 1e-3:
            d += 1
        draws.append(d)
        X.append(synth.token(0, d, H_))
    Xd = torch.from_numpy(np.stack(X)).to(dev)
    Hd = torch.empty((L_, H_), dtype=torch.float32, device=dev)
    idx = torch.empty((L_, K_), dtype=torch.int32, device=dev)
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H_, I_, E_, K_)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    single = [fm.layers_array([layers[l]]) for l in range(L_)]

    def step(h):
        for l in range(L_):
            fm.moe_layer(single[l], Xd[l], Hd[l], 1, K_, EPS, 0, idx[l], None, ws, wsb, h)

    g = graph_of(torch, dev, step)
    for _ in range(max(1, args.warmup)):
        g.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} step(s) of {L_} single-layer calls")
    t0 = time.perf_counter()
    ms = time_replays(torch, dev, g, args.steps)
    elapsed = time.perf_counter() - t0
    us_layer = float(np.median(ms)) * 1e3 / L_
    nbytes = algorithmic_bytes_per_layer(bits)
    achieved = nbytes / us_layer / 1e3
    finite = bool(torch.isfinite(Hd).all().item())
    err_word = workspace_error_word(torch, ws, wsb)
    if not finite or err_word != 0:
        return fail("non-finite outputs or a device-side wait gave up", finite=finite, error_word=err_word)
    log(f"layer: {us_layer:.2f} us per layer-token, {achieved:.0f} GB/s")
    parity = None
    if not args.no_parity:
        prov = synth.Provider(0, H_, I_, bits)
        ids, hs = idx.cpu().numpy(), Hd.cpu().numpy()
        exact, worst = True, 0.0
        for l in range(L_):
            want, i_ref, _, _ = oracle.moe_layer(prov, l, routers_np[l], X[l].astype(np.float64), I_, K_, bits, 64,
                                                 0, EPS)
            exact &= bool(np.array_equal(ids[l], i_ref))
            worst = max(worst, float(np.linalg.norm(hs[l] - want) / np.linalg.norm(want)))
        parity = {"layers": L_, "experts_bit_exact": exact, "max_rel_l2": worst, "tolerance": 1e-5,
                  "pass": bool(exact and worst <= 1e-5)}
        log(f"parity: {parity}")
        if not parity["pass"]:
            return fail("parity check failed", parity=parity)
    cpu = None
    if not args.no_cpu_baseline:
        prov = synth.Provider(0, H_, I_, bits)
        ts = []
        for _ in range(3):
            t_all = t_gen = 0.0
            for l in range(0, L_, 3):
                t1 = time.perf_counter()
                _, i_ref, _, _ = oracle.moe_layer(prov, l, routers_np[l], X[l].astype(np.float64), I_, K_, bits, 64,
                                                  0, EPS)
                t_all += time.perf_counter() - t1
                t1 = time.perf_counter()
                for e in i_ref:
                    synth.expert(0, l, int(e), H_, I_, bits)
                t_gen += time.perf_counter() - t1
            ts.append((t_all - t_gen) / len(range(0, L_, 3)))
        cpu = {"value": round(float(np.median(ts)) * 1e6, 1), "unit": "us per layer-token", "cores": omp_threads(),
               "kind": "oracle", "sample": f"every third of the {L_} layers with its token, O5 in fp64 (OpenMP over "
                                           "rows), expert generation subtracted; median of 3 runs",
               "cpu": cpu_model()}
    out = {
        "metric": "MoE layer us per layer-token (1 layer, 512 experts 4-bit, no norm) + achieved HBM GB/s vs peak",
        "value": round(us_layer, 3), "unit": "us per layer-token", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"one MoE layer per call (router, top-{K_}, SwiGLU experts, combine, residual add; "
                               f"no norm), {E_} experts {bits}-bit, hidden {H_}; the {L_} distinct layers of the "
                               f"stack, one call each per step", "layers_rotated": L_, "experts": E_, "hidden": H_,
                   "inter": I_, "top_k": K_, "bits": bits, "token_draws": draws},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": None,
                     "kernel": "fmoe::decode_kernel (one launch = one layer)", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(us_layer, 3),
                     "timing": f"HIP events around replays of a graph of the {L_} calls, divided by {L_}"},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    del blobs, routers, layers, single, Xd, Hd, idx, ws, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", choices=["stack4", "stack3", "stack2", "layer", "matvec", "batch64", "batch64_3bit",
                                         "batch64_2bit", "qkv4", "qkv2"], default="stack4")
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--top-k", type=int, default=4,
                    help="experts per token for the stack configs (the headline workload is top-4)")
    ap.add_argument("--shared", action="store_true",
                    help="stack configs: every layer also runs a shared expert with a logistic gate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 1 GiB device-to-device copies (the reference kernel for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the whole expert stack fits in one "
                                   "MI355X's HBM and the path has no multi-GPU mode",
                          "n_gpus": args.gpus}))
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "launched with WORLD_SIZE > 1; one GPU only"}))
        return 2

    import torch

    if args.calibrate_copy:
        return calibrate_copy(torch)

    if args.config in ("batch64", "batch64_3bit", "batch64_2bit"):
        return run_batch64(args, torch, {"batch64": 4, "batch64_3bit": 3, "batch64_2bit": 2}[args.config])
    if args.config in ("qkv4", "qkv2"):
        return run_qkv(args, torch, 4 if args.config == "qkv4" else 2)
    if args.config == "matvec":
        return run_matvec(args, torch)
    if args.config == "layer":
        return run_layer(args, torch)
    global K_
    if not 1 <= args.top_k <= 14:
        print(json.dumps({"error": "--top-k must be 1..14 at this layer shape"}))
        return 2
    K_ = args.top_k

    import quantized_expert_ffn_fmoe_amd as fm
    import synth

    bits = {"stack4": 4, "stack3": 3, "stack2": 2}[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"building {L_}-layer {bits}-bit stack on {torch.cuda.get_device_name(dev)}")
    global SHARED
    SHARED = bool(args.shared)
    blobs, routers, layers, resident = build_stack(bits, dev)
    T = args.tokens
    X = torch.from_numpy(np.stack([synth.token(0, d, H_) for d in range(T)])).to(dev)
    Hout = torch.empty((T, H_), dtype=torch.float32, device=dev)
    idx = torch.empty((T, L_, K_), dtype=torch.int32, device=dev)
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H_, I_, E_, K_)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    s_handle = stream.cuda_stream
    # One HIP event pair per step on the launch stream, around its T back-to-back launches: an
    # event pair around every launch would put its own records between the launches (about
    # 10 us per token here); a launch's average duration is the step's time over T.
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(timed_step: int):
        if timed_step >= 0:
            ev0[timed_step].record(stream)
        for t in range(T):
            fm.moe_layer(layers, X[t], Hout[t], 1, K_, EPS, fm.PRENORM, idx[t], None, ws, wsb, s_handle)
        if timed_step >= 0:
            ev1[timed_step].record(stream)

    log(f"warmup {args.warmup} step(s) of {T} tokens")
    for _ in range(args.warmup):
        step(-1)
    torch.cuda.synchronize()
    log(f"timing {args.steps} step(s)")
    t0 = time.perf_counter()
    for s_i in range(args.steps):
        step(s_i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [ev0[i].elapsed_time(ev1[i]) for i in range(args.steps)]
    tok_s = args.steps * T / elapsed
    ms_step = elapsed * 1e3 / args.steps
    per_launch = L_ * algorithmic_bytes_per_layer(bits)
    avg_kernel_s = float(np.sum(step_ms)) * 1e-3 / (args.steps * T)
    achieved = per_launch / avg_kernel_s / 1e9
    ids = idx.cpu().numpy()
    reuse = float(np.mean([len(set(ids[t, l]) & set(ids[t - 1, l])) / K_ for t in range(1, T) for l in range(L_)]))
    reuse_l0 = float(np.mean([len(set(ids[t, 0]) & set(ids[t - 1, 0])) / K_ for t in range(1, T)]))
    log(f"{tok_s:.1f} tok/s, kernel avg {avg_kernel_s * 1e6:.1f} us, {achieved:.0f} GB/s")
    # health of the timed run: every output finite, no device-side wait gave up
    finite = bool(torch.isfinite(Hout).all().item())
    err_word = workspace_error_word(torch, ws, wsb)
    if not finite or err_word != 0:
        return fail("the timed decode produced non-finite outputs or a device-side wait gave up",
                    finite=finite, error_word=err_word)
    parity = None
    if not args.no_parity:
        # the stored oracle results are top-4 without a shared expert; others: the live oracle
        if K_ == 4 and not SHARED:
            parity = parity_check(layers, bits, dev, ws, wsb)
        else:
            log("parity against the live oracle")
            parity = live_parity(layers, bits, dev, ws, wsb)
        log(f"parity: {parity}")
        if parity is None or not parity["pass"]:
            return fail("parity check failed", parity=parity)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(bits)
    kernel_tag = f"decode_stack{bits}" + ("" if K_ == 4 else f"_top{K_}") + ("_shared" if SHARED else "")
    traffic = traffic_from_profiles(kernel_tag)
    del blobs, routers  # the stream probe needs 4 GiB of free device memory
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    probe = stream_read_probe(torch)
    log(f"stream-read probe: {probe['gbs']:.0f} GB/s")
    out = {
        "metric": METRIC.replace("4-bit)", f"{bits}-bit" + (f", top-{K_})" if K_ != 4 else ")")),
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{L_}-layer x {E_}-expert {bits}-bit MoE expert-block decode stack"
                               + ("" if K_ == 4 else f" (top-{K_})")
                               + (" with a gated shared expert per layer" if SHARED else "")
                               + f", {T} consecutive single tokens per step",
                   "layers": L_, "experts": E_, "hidden": H_, "inter": I_, "top_k": K_, "bits": bits, "group": 64,
                   "tokens_per_step": T, "resident_expert_bytes": int(resident)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "fmoe::decode_kernel (one launch = one token, 60 layers)",
                     "algorithmic_bytes_per_launch": per_launch, "avg_launch_us": round(avg_kernel_s * 1e6, 2),
                     "stream_read_probe": probe, "frac_of_stream_read_probe": round(achieved / probe["gbs"], 4),
                     "timing": "HIP events on the launch stream around each step's back-to-back launches; "
                               "avg_launch_us = step time / launches (the gaps between launches included)"},
        "cpu_baseline": cpu,
        "parity": parity,
        "wall_gbps": round(per_launch * tok_s / 1e9, 1),
        "inter_token_expert_reuse": {"all_layers": round(reuse, 4), "layer0": round(reuse_l0, 4)},
    }
    print(json.dumps(out), flush=True)
    # Release the stack explicitly so that process exit has no device memory left to tear down.
    del layers, X, Hout, idx, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
