"""Benchmark of the fused rANS-decode GEMM on one MI355X.

One step = one pass of the hot path over one batch: dgt_fused_decode_gemm on a
resident compressed layer (LUT prologue, tile fetch, on-chip rANS decode,
matrix-core product, split-K reduction and epilogue), here on the Llama-3-8B
MLP projection shape W 14336x4096 stored as bf16 with its high byte coded
(workload "bf16_mlp"), X of M = 1 row.  Several copies of the blob rotate so
the 256 MB last-level cache cannot hold the working set.

Prints ONE JSON line: metric, value (decoded-weight GB/s at M = 1), roofline of
the fused kernel (HBM bytes it must read / kernel time), the CPU oracle timed on
the host cores, and secondary figures (bits/weight, TFLOP/s at M = 256, the
uncompressed baseline).
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
ROTATE_BYTES = 512 << 20     # working set above the 256 MB last-level cache
METRIC = "fused rANS-decode GEMM decoded-weight GB/s at M=1; TFLOP/s at M=256; bits/wt"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="bf16_mlp")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true",
                   help="time only the M=1 fused kernel (for profiler runs)")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run one plain device copy of 512 MiB (counter calibration)")
    return p.parse_args()


def source_hash() -> str:
    """Hash of the HIP sources: profile figures are valid only for this code."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "decode_gemm_tile_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_prefix: str, workload: str, per_launch_ref: float):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source hash:\s*`?([0-9a-f]{16})", text)
    m_val = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != source_hash():
        return None
    return float(m_val.group(1))


def timed(fn, steps, warmup, stream):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def launch_distribution(fn, n, stream):
    """Per-launch durations (us) of n launches, each between its own events."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"median_us": round(float(np.median(us)), 3),
            "p10_us": round(float(np.percentile(us, 10)), 3),
            "p90_us": round(float(np.percentile(us, 90)), 3), "launches": n}


def cpu_baseline(d, wl, blob):
    """The CPU oracle (decode of the compressed layer + fp64 GEMV), timed on the
    host on a bounded sample of the layer: every tile of the first strips."""
    from threadpoolctl import threadpool_limits

    from oracle import blob as oblob
    from oracle import gemm as ogemm
    from oracle import numerics
    h = oblob.parse(blob)
    kt = wl.k // wl.tile_k
    strips = wl.n // wl.tile_n
    tiles = list(range(strips * kt))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        syms = oblob.decode_symbols(blob, tiles)
        raw = np.frombuffer(blob, np.uint8, len(tiles) * wl.tile_n * wl.tile_k,
                            h["raw_off"]).reshape(len(tiles), -1)
        from oracle import order
        rows = strips * wl.tile_n
        if wl.fmt == 7:  # high-byte pairs: symbol = hi[2c] | hi[2c+1] << 8
            pairs = order.scatter_tiles(syms.astype(np.uint16), rows, wl.k // 2, wl.tile_n,
                                        wl.tile_k // 2, wl.lanes, epl=4)
            hi = np.empty((rows, wl.k), np.uint16)
            hi[:, 0::2] = pairs & 0xFF
            hi[:, 1::2] = pairs >> 8
        else:
            hi = order.scatter_tiles(syms.astype(np.uint8), rows, wl.k, wl.tile_n, wl.tile_k,
                                     wl.lanes)
        lo = order.scatter_tiles(raw, rows, wl.k, wl.tile_n, wl.tile_k, wl.lanes, raw=True)
        w = (hi.astype(np.uint16) << 8) | lo
        y = ogemm.gemm_fp64(numerics.bf16_bits_to_f64(d["x"][:1]), numerics.bf16_bits_to_f64(w))
        dt = time.perf_counter() - t0
    assert np.array_equal(w, d["codes"][:rows])
    weights = rows * wl.k
    return {"value": round(weights * 2 / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d of %d tiles (rows 0..%d, all K), decode + fp64 GEMV, %.1f s, "
                      "1 thread (numpy, BLAS limited to 1)" % (len(tiles), wl.n // wl.tile_n * kt,
                                                               rows - 1, dt),
            "seconds": round(dt, 3), "checksum": float(np.abs(y).sum())}


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_gemm_tile_amd as dgt
    import workloads
    from oracle import entropy as oentropy

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    wl = workloads.WORKLOADS[args.workload]
    d = workloads.make(args.workload)
    t0 = time.perf_counter()
    blob = dgt.dgt_compress_layer(wl.fmt, d["codes"], wl.tile_n, wl.tile_k, wl.lanes)
    encode_s = time.perf_counter() - t0
    info = dgt.dgt_layer_info(blob)
    wide = wl.fmt in (4, 6, 7)  # bf16 layers: one uint16 code per weight
    sym = (np.asarray(d["codes"]) >> 8).astype(np.uint8) if wl.fmt in (4, 7) else None
    h_hi = oentropy.empirical_entropy(sym, 256) if sym is not None else None

    copies = max(2, math.ceil(ROTATE_BYTES / len(blob)))
    layers = [dgt.DeviceLayer(blob, dev) for _ in range(copies)]
    xall = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    scales = (torch.from_numpy(d["scales"].view(np.int16)).to(dev)
              if d["scales"] is not None else None)

    # ---- headline: fused kernel at M = 1
    m = 1
    x1 = xall[:m].contiguous()
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layers[0], m), dev)
    y = torch.empty((m, wl.n), dtype=torch.float32, device=dev)

    def fused(i, x=x1, y=y, ws=ws):
        dgt.dgt_fused_decode_gemm(layers[i % copies], x, scales=scales, w_scale=d["w_scale"],
                                  y=y, ws=ws, stream=stream)

    ms = timed(fused, args.steps, args.warmup, stream)
    dist = launch_distribution(fused, 50, stream)
    nk = wl.n * wl.k
    # decoded-weight bytes at the format's storage width (int4 half a byte)
    decoded_bytes = nk * {1: 1.0, 2: 0.5, 3: 1.0, 4: 2.0, 5: 0.5, 6: 2.0, 7: 2.0}[wl.fmt]
    value = decoded_bytes / (ms * 1e-3) / 1e9
    alg_bytes = len(blob) + m * wl.k * 2 + m * wl.n * 4
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles("k_fused", args.workload, alg_bytes)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: W %dx%d %s, tiles %dx%d, R=%d, M=%d"
                               % (args.workload, wl.n, wl.k, wl.note, wl.tile_n, wl.tile_k,
                                  wl.lanes, m),
                   "m": m, "n": wl.n, "k": wl.k, "blob_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel_us": round(ms * 1e3, 3), "algorithmic_bytes": alg_bytes,
                     "per_launch": dist, "source_hash": source_hash()},
    }

    secondary = {"bits_per_weight": round(info.bits_per_weight, 4),
                 "compressed_bytes": len(blob), "encode_seconds": round(encode_s, 3)}
    if h_hi is not None:
        secondary["entropy_hi_byte_bits"] = round(h_hi, 4)
        secondary["bits_over_entropy"] = round(info.bits_per_weight - (h_hi + 8.0), 4)
    if not args.no_secondary:
        # fused at M = 256 (TFLOP/s; the workload's largest M if smaller) and
        # the uncompressed baseline at M = 1 and that M
        m2 = min(256, xall.shape[0])
        x2 = xall[:m2].contiguous()
        ws2 = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layers[0], m2), dev)
        y2 = torch.empty((m2, wl.n), dtype=torch.float32, device=dev)
        ms2 = timed(lambda i: dgt.dgt_fused_decode_gemm(layers[i % copies], x2, scales=scales,
                                                        w_scale=d["w_scale"], y=y2, ws=ws2,
                                                        stream=stream),
                    max(5, args.steps // 10), 3, stream)
        flops = 2.0 * m2 * nk
        secondary["fused_m%d_ms" % m2] = round(ms2, 4)
        secondary["fused_m%d_tflops" % m2] = round(flops / (ms2 * 1e-3) / 1e12, 3)
        secondary["fused_m%d_mfma_frac" % m2] = round(
            flops / (ms2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        codes = np.asarray(d["codes"])
        wraw = torch.from_numpy(codes.view(np.int16) if wide else codes.view(np.uint8)).to(dev)
        dcopies = max(2, math.ceil(ROTATE_BYTES / (nk * 2)))
        wd = [wraw.clone() for _ in range(dcopies)]
        del wraw
        dec = torch.empty((wl.n, wl.k), dtype=torch.int16 if wide else torch.uint8,
                          device=dev)
        reps = max(5, args.steps // 10)
        ablation = {}
        for mm in sorted({1, m2}):
            xm = xall[:mm].contiguous()
            wsd = dgt.alloc_workspace(dgt.dgt_dense_workspace(wl.fmt, wl.n, wl.k, wl.tile_n, mm), dev)
            yd = torch.empty((mm, wl.n), dtype=torch.float32, device=dev)
            msd = timed(lambda i: dgt.dgt_dense_gemm(wl.fmt, wd[i % dcopies], xm,
                                                     tile_n=wl.tile_n, scales=scales,
                                                     w_scale=d["w_scale"], y=yd, ws=wsd,
                                                     stream=stream),
                        reps, 3, stream)
            secondary["dense_m%d_ms" % mm] = round(msd, 4)
            if mm == 1:
                secondary["dense_m1_weight_gbs"] = round(nk * 2 / (msd * 1e-3) / 1e9, 3)
                secondary["fused_speedup_vs_dense_m1"] = round(msd / ms, 3)
            else:
                secondary["dense_m%d_tflops" % mm] = round(2.0 * mm * nk / (msd * 1e-3) / 1e12, 3)
            # ablation: layer-level decode to HBM, then the dense GEMM on the
            # decoded copy (two launches per step) against the fused kernel
            ms_dec = timed(lambda i: dgt.dgt_decode_tiles(layers[i % copies], out=dec,
                                                          stream=stream), reps, 3, stream)

            def two_stage(i, xm=xm, yd=yd, wsd=wsd):
                dgt.dgt_decode_tiles(layers[i % copies], out=dec, stream=stream)
                dgt.dgt_dense_gemm(wl.fmt, dec, xm, tile_n=wl.tile_n, scales=scales,
                                   w_scale=d["w_scale"], y=yd, ws=wsd, stream=stream)
            ms_two = timed(two_stage, reps, 3, stream)
            ms_fused = ms if mm == 1 else secondary["fused_m%d_ms" % mm]
            ablation["m%d" % mm] = {"decode_to_hbm_ms": round(ms_dec, 4),
                                    "two_stage_ms": round(ms_two, 4),
                                    "fused_ms": round(ms_fused, 4),
                                    "fused_speedup_vs_two_stage": round(ms_two / ms_fused, 3)}
            if mm > 16 and wl.lanes == 64:
                # the fused rung without ping-pong: one fragment buffer in the
                # large-M kernel (the library reads the switch at every call)
                os.environ["DGT_XM_SINGLE_BUFFER"] = "1"
                try:
                    ms_one = timed(lambda i: dgt.dgt_fused_decode_gemm(
                        layers[i % copies], xm, scales=scales, w_scale=d["w_scale"], y=y2,
                        ws=ws2, stream=stream), reps, 3, stream)
                finally:
                    del os.environ["DGT_XM_SINGLE_BUFFER"]
                ablation["m%d" % mm]["fused_single_buffer_ms"] = round(ms_one, 4)
                ablation["m%d" % mm]["ping_pong_speedup"] = round(ms_one / ms_fused, 3)
            # vendor GEMM on the uncompressed bf16 weight (reference point only),
            # alone and after the layer-level decode (the two-stage path with
            # the vendor library's GEMM on the decoded copy)
            if wide:
                wts = [w.view(torch.bfloat16).t().contiguous() for w in wd]
                ms_lib = timed(lambda i: torch.matmul(xm, wts[i % len(wts)]), reps, 3, stream)
                secondary["torch_matmul_bf16_m%d_ms" % mm] = round(ms_lib, 4)
                del wts
                decb = dec.view(torch.bfloat16)

                def two_stage_vendor(i, xm=xm):
                    dgt.dgt_decode_tiles(layers[i % copies], out=dec, stream=stream)
                    torch.nn.functional.linear(xm, decb)  # x @ W^T, W [N, K] as decoded
                ms_tv = timed(two_stage_vendor, reps, 3, stream)
                ablation["m%d" % mm]["two_stage_vendor_gemm_ms"] = round(ms_tv, 4)
                ablation["m%d" % mm]["fused_speedup_vs_two_stage_vendor"] = round(ms_tv / ms_fused, 3)
        secondary["ablation"] = ablation
        del wd, dec
        # the same layer in the other codings of its family: bits and time
        variants = []
        if wl.fmt in (4, 7) and wl.lanes == 64:
            other = 4 if wl.fmt == 7 else 7
            variants.append(("one_high_byte_per_symbol" if other == 4 else "high_byte_pairs",
                             other, 64))
        if wl.lanes == 64 and wl.tile_n % 32 == 0:
            variants.append(("two_states_per_lane", wl.fmt, 128))
        for vname, vfmt, vlanes in variants:
            blob2 = dgt.dgt_compress_layer(vfmt, d["codes"], wl.tile_n, wl.tile_k, vlanes)
            c2 = max(2, math.ceil(ROTATE_BYTES / len(blob2)))
            l2 = [dgt.DeviceLayer(blob2, dev) for _ in range(c2)]
            var = {"fmt": vfmt, "lanes": vlanes,
                   "bits_per_weight": round(dgt.dgt_layer_info(blob2).bits_per_weight, 4)}
            for mm, xm_ in ((1, x1), (m2, x2)):
                wsr = dgt.alloc_workspace(dgt.dgt_gemm_workspace(l2[0], mm), dev)
                yr = torch.empty((mm, wl.n), dtype=torch.float32, device=dev)
                var["fused_m%d_ms" % mm] = round(timed(
                    lambda i: dgt.dgt_fused_decode_gemm(l2[i % c2], xm_, scales=scales,
                                                        w_scale=d["w_scale"], y=yr, ws=wsr,
                                                        stream=stream),
                    reps, 3, stream), 4)
            var["decoded_gbs_m1"] = round(decoded_bytes / (var["fused_m1_ms"] * 1e-3) / 1e9, 3)
            secondary[vname] = var
            del l2
    result["secondary"] = secondary

    if args.copy_calib:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = a.numel()

    if not args.no_cpu_baseline and wl.fmt in (4, 7):
        result["cpu_baseline"] = cpu_baseline(d, wl, blob)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
