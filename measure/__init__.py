"""Measurement kernels of the benchmark (libmeasure.so, gfx950): a read-only HBM streaming
probe and an exchange-latency probe of persistent workgroups (see measure.hip). They are
not part of the fmoe library; bench.py and the profile summaries use them.

    python -m measure stream      # JSON line: best read rate over 4 GiB
    python -m measure exchange    # JSON lines: exchange latency per mode and word count
    python -m measure replicas    # JSON lines: device-wide exchange per replica count / ack wait
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
    print(f"unknown probe {what}", file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv))
