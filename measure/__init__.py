"""Measurement kernels of the benchmark (libmeasure.so, gfx950): a read-only HBM streaming
probe and an exchange-latency probe of persistent workgroups (see measure.hip). They are
not part of the fmoe library; bench.py and the profile summaries use them.

    python -m measure stream      # JSON line: best read rate over 4 GiB
    python -m measure exchange    # JSON lines: exchange latency per mode and word count
    python -m measure replicas    # JSON lines: device-wide exchange per replica count / ack wait
    python -m measure trace       # phase trace of the decode kernel on the 60-layer 4-bit stack

The phase trace runs a copy of the fmoe library compiled with its trace hooks
(-DFMOE_TRACE, libfmoe_trace.so here, built by build_trace()); the library itself is built
without them.
"""
from __future__ import annotations

import ctypes
import json
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmeasure.so")
MODES = {0: "all 256 workgroups, 8 replicas, device scope",
         1: "32 workgroups of one XCD, device scope",
         2: "32 workgroups of one XCD, workgroup-scope atomics",
         3: "32 workgroups of one XCD, plain stores, L1 invalidated before plain loads (meet in the XCD's L2)",
         4: "32 workgroups of one XCD, plain stores, non-temporal loads"}


def build() -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "measure.hip"), "-o", _SO]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return _SO


TRACE_SO = os.path.join(_HERE, "libfmoe_trace.so")
TRACE_PHASES = 18  # phase stamps per layer and workgroup (fmoe_decode.hip, FMOE_TRACE)
MAX_GRID = 1024


def build_trace(jobs: int = 4) -> str:
    """The fmoe library compiled with its phase-trace hooks, as libfmoe_trace.so next to this file."""
    from quantized_expert_ffn_fmoe_amd import _build

    return _build.build(jobs=jobs, so=TRACE_SO, extra=["-DFMOE_TRACE"])


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is missing: build it with measure.build()")
        L = ctypes.CDLL(_SO)
        vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint32
        L.measure_cus.restype = i32
        L.measure_cus.argtypes = []
        L.measure_stream_read.restype = i32
        L.measure_stream_read.argtypes = [vp, sz, i32, i32, i32, vp, vp]
        L.measure_row_stages.restype = i32
        L.measure_row_stages.argtypes = [vp, sz, i32, i32, i32, vp, vp]
        L.measure_exchange.restype = i32
        L.measure_exchange.argtypes = [i32, i32, i32, u32, vp, vp, vp, vp, i32, i32, vp]
        _lib = L
    return _lib


def stream_read(torch, gib: int = 4, reps: int = 5, variants=(0, 1)) -> dict:
    """Best read rate (GB/s, 1e9 B/s) of the streaming kernel over a gib-GiB buffer, HIP
    events on the launch stream around each pass; plain and non-temporal loads, 4 or 8
    loads in flight per thread, 2 grid sizes; best of `reps` passes per variant after one
    untimed pass. A pass reads the whole buffer once, front to back, so no byte is served
    from the 256 MB Infinity Cache."""
    dev = torch.device("cuda:0")
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    cus = lib().measure_cus()
    best, table = 0.0, []
    for variant in variants:
        for unroll in (4, 8):
            for blocks in (cus * 8, cus * 32):
                rc = lib().measure_stream_read(buf.data_ptr(), nbytes, variant, unroll, blocks, sink.data_ptr(),
                                               stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"measure_stream_read: {rc}")
                gbs = 0.0
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    lib().measure_stream_read(buf.data_ptr(), nbytes, variant, unroll, blocks, sink.data_ptr(),
                                              stream.cuda_stream)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    gbs = max(gbs, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
                table.append({"loads": ("plain", "non-temporal", "LDS-DMA", "non-temporal LDS-DMA")[variant],
                              "in_flight": unroll,
                              "blocks": blocks, "gbs": round(gbs, 1)})
                best = max(best, gbs)
    del buf
    torch.cuda.empty_cache()
    return {"kind": f"read-only streaming kernel (measure.hip) over {gib} GiB, best of {reps} passes per variant",
            "gbs": round(best, 1), "variants": table}


ROW_STAGE_SWEEP = tuple((rb, d, p) for rb in (2048, 512) for d in (2, 4) for p in (128, 256, 512, 1024, 2048)
                        if rb % p == 0)


def row_stages(torch, gib: int = 4, reps: int = 5, configs=ROW_STAGE_SWEEP, verbose: bool = True) -> dict:
    """Read rate (GB/s) of the row-stage kernel (measure.hip item 3) over a gib-GiB buffer for
    each (row bytes, stages in flight, piece P) of `configs`; the default sweep covers rows of
    2048 bytes (a 4-bit gate/up row at hidden 4096) and 512 bytes (a 4-bit down row at
    intermediate 1024), every piece and 2 or 4 stages in flight. Best of `reps` passes after
    one untimed pass, HIP events on the launch stream."""
    dev = torch.device("cuda:0")
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    table = []
    for row_bytes, depth, piece in configs:

        def once():
            rc = lib().measure_row_stages(buf.data_ptr(), nbytes, row_bytes, piece, depth, sink.data_ptr(),
                                          stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"measure_row_stages: {rc}")

        once()
        gbs = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            once()
            e1.record(stream)
            torch.cuda.synchronize()
            gbs = max(gbs, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        table.append({"row_bytes": row_bytes, "piece": piece, "rows_per_stage": 8192 // piece,
                      "stages_in_flight": depth, "gbs": round(gbs, 1)})
        if verbose:
            print(json.dumps(table[-1]), flush=True)
    del buf
    torch.cuda.empty_cache()
    return {"kind": f"row-stage LDS-DMA read (measure.hip) over {gib} GiB, best of {reps} passes",
            "gbs": max(r["gbs"] for r in table), "rows": table}


def exchange(torch, mode: int, n_words: int, rounds: int = 200, epoch0: int = 0, buf=None, reps: int = 8,
             no_ack: bool = False) -> dict:
    """Latency of one exchange round (µs): median and 90th percentile over rounds 10.. of the
    spacing between the last workgroup's completion stamps of consecutive rounds, plus the
    spread of completion stamps inside a round and the XCC_ID check of the placement."""
    dev = torch.device("cuda:0")
    G = lib().measure_cus()
    own = buf is None
    if own:
        buf = torch.zeros(max(reps, 8) * n_words, dtype=torch.int64, device=dev)
    t_end = torch.zeros(rounds * G, dtype=torch.int64, device=dev)
    xcc = torch.zeros(G, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    rc = lib().measure_exchange(mode, n_words, rounds, epoch0, buf.data_ptr(), t_end.data_ptr(), xcc.data_ptr(),
                                err.data_ptr(), reps, int(no_ack), torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"measure_exchange: {rc}")
    torch.cuda.synchronize()
    t = t_end.cpu().numpy().reshape(rounds, G).astype(np.float64) * 0.01  # 100 MHz clock -> µs
    xc = xcc.cpu().numpy()
    last = t.max(axis=1)
    per = np.diff(last)[10:]
    spread = (t.max(axis=1) - t.min(axis=1))[10:]
    what = MODES[mode].replace("8 replicas", f"{reps} replicas") + (", polls before its stores are acknowledged"
                                                                     if no_ack else "")
    return {"mode": mode, "what": what, "words": n_words, "rounds": rounds, "replicas": reps if mode == 0 else None,
            "round_us_median": round(float(np.median(per)), 3), "round_us_p90": round(float(np.percentile(per, 90)), 3),
            "spread_us_median": round(float(np.median(spread)), 3),
            "xcc_is_g_mod_8": bool(np.all(xc == np.arange(G) % 8)), "gave_up": bool(err.item() != 0)}


def _q(x, axis=None):
    """Median and 90th percentile (µs, rounded)."""
    return [round(float(np.median(x, axis=axis)), 3), round(float(np.percentile(x, 90, axis=axis)), 3)]


def phase_trace(torch, n_tokens: int = 16, warmup: int = 4, bits: int = 4) -> dict:
    """Phase stamps of the decode kernel (traced build) on the 60-layer x 512-expert top-4
    stack (4-, 3- or 2-bit experts) with the pre-norm, one launch per token (tokens =
    synthetic draws). Per layer
    1..59 and workgroup: phase durations; per exchange, the time from the last workgroup's
    publish to each reader's completion, and the spread of the publishes. Medians and 90th
    percentiles over layers, tokens and workgroups. The tokens run back to back as in the
    benchmark (the stamp buffer is switched by a kernel on the stream); per-token launch times
    with the trace on and off (HIP events) give the hooks' own cost."""
    import bench
    import quantized_expert_ffn_fmoe_amd as fm
    import synth

    dev = torch.device("cuda:0")
    L = fm.load(TRACE_SO)
    L.fmoe_trace_set.restype = ctypes.c_int
    L.fmoe_trace_set.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    fm.use(L)
    H, I, E, K, NL = bench.H_, bench.I_, bench.E_, bench.K_, bench.L_
    blobs, routers, layers, _ = bench.build_stack(bits, dev)
    G = lib().measure_cus()
    per = NL * TRACE_PHASES * MAX_GRID
    stamps = torch.zeros(n_tokens * per, dtype=torch.int64, device=dev)
    wsb = fm.workspace_bytes(fm.OP_MOE_LAYER, 1, H, I, E, K)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    n_all = warmup + 2 * n_tokens
    xs = torch.from_numpy(np.stack([synth.token(0, t, H) for t in range(n_all)])).to(dev)
    h = torch.empty(H, dtype=torch.float32, device=dev)
    idx = torch.empty((NL, K), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_all)]

    def run(t, buf):
        if L.fmoe_trace_set(buf, sp) != 0:
            raise RuntimeError("fmoe_trace_set failed")
        ev[t][0].record(stream)
        fm.moe_layer(layers, xs[t], h, 1, K, bench.EPS, fm.PRENORM, idx, None, ws, wsb, stream)
        ev[t][1].record(stream)

    # warm-up, then n_tokens back to back with the trace off, then n_tokens traced, each into
    # its own slice of the stamp buffer; no host synchronisation in between
    for t in range(warmup):
        run(t, None)
    for t in range(warmup, warmup + n_tokens):
        run(t, None)
    for i, t in enumerate(range(warmup + n_tokens, n_all)):
        run(t, stamps.data_ptr() + i * per * 8)
    L.fmoe_trace_set(None, sp)
    torch.cuda.synchronize()
    launch_us = {"off": [ev[t][0].elapsed_time(ev[t][1]) * 1e3 for t in range(warmup, warmup + n_tokens)],
                 "on": [ev[t][0].elapsed_time(ev[t][1]) * 1e3 for t in range(warmup + n_tokens, n_all)]}
    allst = stamps.cpu().numpy().reshape(n_tokens, NL, TRACE_PHASES, MAX_GRID)[:, :, :, :G]
    per_token = [allst[i].astype(np.float64) * 0.01 for i in range(n_tokens)]
    S = np.stack(per_token)  # [token][layer][phase][workgroup], µs
    ls = slice(1, NL)  # layers with an h exchange
    layer_us = np.diff(S[:, :, 0, :], axis=1)  # start-to-start per workgroup
    out = {"workload": f"60-layer x 512-expert {bits}-bit top-4 decode stack with pre-norm, one token per launch",
           "tokens_traced": len(per_token), "workgroups": G, "clock": "s_memrealtime, 100 MHz",
           "launch_us_trace_on": _q(launch_us["on"]), "launch_us_trace_off": _q(launch_us["off"]),
           "layer_us": _q(layer_us)}
    d = lambda a, b: S[:, ls, a, :] - S[:, ls, b, :]
    ph = {"h gathered (from layer start)": d(1, 0),
          "router + logits published": d(2, 1),
          "logits gathered (after own publish)": d(3, 2),
          "top-k (all rounds, softmax)": d(4, 3)}
    for w in range(4):
        ph[f"gate/up done, wave {w} (from h gathered)"] = d(5 + w, 1)
    for w in range(4):
        ph[f"a gathered, wave {w} (from its gate/up done)"] = d(9 + w, 5 + w)
        ph[f"down done, wave {w} (from its a gathered)"] = d(13 + w, 9 + w)
    ph["h published (from layer start)"] = d(17, 0)
    out["phases_us"] = {k: _q(v) for k, v in ph.items()}
    # exchanges: time from the last publish (over workgroups) to each reader's completion
    last_h = S[:, 0:NL - 1, 17, :].max(axis=2)[:, :, None]  # layer l-1's h
    last_lg = S[:, ls, 2, :].max(axis=2)[:, :, None]
    ex = {"h": S[:, ls, 1, :] - last_h, "logits": S[:, ls, 3, :] - last_lg}
    for j in range(4):
        if bits == 4:  # slot j: produced by wave (j + 1) % 4 everywhere, read by wave j
            last_a = S[:, ls, 5 + (j + 1) % 4, :].max(axis=2)[:, :, None]
            ex[f"a slot {j}"] = S[:, ls, 9 + j, :] - last_a
        else:  # spread schedule: a slot's rows come from several waves; the last gate/up of any wave
            last_a = S[:, ls, 5:9, :].max(axis=(2, 3))[:, :, None]
            ex[f"a slot {j} (after the last gate/up of any wave)"] = S[:, ls, 9 + j, :] - last_a
    out["exchange_after_last_publish_us"] = {k: _q(v) for k, v in ex.items()}
    spread = {"layer start": S[:, ls, 0, :], "logits published": S[:, ls, 2, :], "h published": S[:, ls, 17, :]}
    for w in range(4):
        spread[f"gate/up done, wave {w}"] = S[:, ls, 5 + w, :]
    out["spread_over_workgroups_us"] = {k: _q(v.max(axis=2) - v.min(axis=2)) for k, v in spread.items()}
    del blobs, routers, layers, ws, stamps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def trace_markdown(r: dict) -> str:
    lines = [f"Workload: {r['workload']}; {r['tokens_traced']} traced tokens, {r['workgroups']} workgroups; "
             f"clock {r['clock']}. Launch (µs, median / p90): trace on {r['launch_us_trace_on']}, "
             f"off {r['launch_us_trace_off']}; layer start-to-start {r['layer_us']}.", "",
             "| phase (per workgroup, layers 1-59) | median µs | p90 µs |", "|---|---:|---:|"]
    lines += [f"| {k} | {v[0]} | {v[1]} |" for k, v in r["phases_us"].items()]
    lines += ["", "| exchange: reader's completion after the last publish | median µs | p90 µs |", "|---|---:|---:|"]
    lines += [f"| {k} | {v[0]} | {v[1]} |" for k, v in r["exchange_after_last_publish_us"].items()]
    lines += ["", "| spread over workgroups (max - min) of | median µs | p90 µs |", "|---|---:|---:|"]
    lines += [f"| {k} | {v[0]} | {v[1]} |" for k, v in r["spread_over_workgroups_us"].items()]
    return "\n".join(lines)


def main(argv) -> int:
    import torch

    torch.cuda.set_device(0)
    what = argv[1] if len(argv) > 1 else "exchange"
    if what == "stream":
        print(json.dumps(stream_read(torch)), flush=True)
        return 0
    if what == "stream_lds":  # plain, non-temporal and LDS-DMA reads
        print(json.dumps(stream_read(torch, variants=(0, 1, 2, 3))), flush=True)
        return 0
    if what == "rows":  # the batched expert kernels' stage pattern against whole rows
        print(json.dumps(row_stages(torch)), flush=True)
        return 0
    if what == "exchange":
        G = lib().measure_cus()
        for n in (G, 512, 4096):
            for mode in (0, 1, 2, 3, 4):
                if n % (G if mode == 0 else G // 8):
                    continue
                print(json.dumps(exchange(torch, mode, n)), flush=True)
        return 0
    if what == "replicas":  # the device-wide exchange's replica count and ack wait
        for n in (512, 4096):
            for reps in (1, 2, 4, 8, 16):
                for no_ack in (False, True):
                    print(json.dumps(exchange(torch, 0, n, reps=reps, no_ack=no_ack)), flush=True)
        return 0
    if what == "trace":  # phase trace of the decode kernel (traced build); optional code width
        r = phase_trace(torch, bits=int(argv[2]) if len(argv) > 2 else 4)
        print(json.dumps(r), flush=True)
        print(trace_markdown(r), flush=True)
        return 0
    print(f"unknown probe {what}", file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv))
