"""Benchmark of the fused rANS-decode GEMM on one MI355X.

One step = one pass of the hot path over one batch: dgt_fused_decode_gemm on a
resident compressed layer (decode-table prologue, tile fetch, on-chip rANS
decode, matrix-core product, split-K reduction and epilogue).  The default
workload is the largest single-GPU configuration, the 405B-scale FFN weight
W 53248x16384 stored as bf16 with its high byte rANS-coded and its low byte
raw ("bf16_ffn405"), X of M = 1 row.  Copies of the blob rotate so the 256 MB
last-level cache never holds the working set.

Prints ONE JSON line: metric, value (decoded-weight GB/s at M = 1), the
roofline of the fused kernel (algorithmic bytes per launch / launch time), the
CPU oracle timed on the host's cores, and secondary figures (bits/weight,
TFLOP/s at M = 256, the library's own uncompressed GEMM, the vendor GEMM, the
ablation ladder, the int4 405B-scale FFN and the Llama-3-8B MLP layer).
"""

import argparse
import hashlib
import json
import math
import multiprocessing as mp
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
# decoded-weight bytes per weight at the format's storage width (int4: half a byte)
STORAGE_BYTES = {1: 1.0, 2: 0.5, 3: 1.0, 4: 2.0, 5: 0.5, 6: 2.0, 7: 2.0, 8: 2.0}
CPU_SAMPLE_WEIGHTS = 96 << 20  # weights of W the CPU oracle decodes (whole strips)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="bf16_ffn405")
    p.add_argument("--m", type=int, default=1,
                   help="rows of X of the headline launches (the metric is quoted at M = 1)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true",
                   help="time only the headline launches (for profiler runs)")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run one plain device copy of 512 MiB (counter calibration)")
    return p.parse_args()


def source_hash() -> str:
    """Hash of the sources compiled into device code and its launch planning
    (every file under csrc/ but the host-only encoder): profile figures are
    valid only for this code."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "decode_gemm_tile_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name == "dgt_host.cpp":
            continue
        with open(os.path.join(d, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


VALU_SIMDS = 1024            # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9
VALU_CYCLES = 4              # a wave64 VALU instruction occupies a SIMD16 for 4 cycles
XCDS = 8
SEC_WARMUP = 10             # untimed launches before each secondary figure (clocks settle)


def valu_from_profiles(workload: str, m: int, kernel_us: float):
    """Fraction of the kernel time the SIMDs spend issuing VALU instructions,
    from the committed SQ counter summary (SQ_INSTS_VALU per dispatch), if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "sq_counters_%s_m%d.md" % (workload, m))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source hash:\s*`?([0-9a-f]{16})", text)
    m_val = re.search(r"\| SQ_INSTS_VALU \| ([0-9.eE+]+) \|", text)
    m_clk = re.search(r"\| GRBM_GUI_ACTIVE \| ([0-9.eE+]+) \|", text)
    if not m_hash or not m_val or m_hash.group(1) != source_hash():
        return None
    busy_cycles = float(m_val.group(1)) * VALU_CYCLES / VALU_SIMDS
    out = {"valu_instructions": float(m_val.group(1)),
           "valu_issue_frac_at_2p4ghz": round(busy_cycles / CLOCK_HZ / (kernel_us * 1e-6), 4)}
    if m_clk:
        # busy cycles of the GPU during the dispatch, summed over the 8 XCDs
        out["valu_issue_frac"] = round(busy_cycles / (float(m_clk.group(1)) / XCDS), 4)
    return out


def traffic_from_profiles(workload: str, m: int):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_m%d.md" % (workload, m))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source hash:\s*`?([0-9a-f]{16})", text)
    m_val = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != source_hash():
        return None
    return float(m_val.group(1))


# ------------------------------------------------------------- CPU oracle
_CPU = {}  # inherited by forked workers: blob, workload, codes, x row


def _cpu_strips(bounds):
    """Oracle decode of strips [s0, s1) of W plus the fp64 GEMV of X's first
    row with those rows; returns (s0, y part, decoded rows equal the input)."""
    from threadpoolctl import threadpool_limits

    from oracle import blob as oblob
    from oracle import gemm as ogemm
    from oracle import numerics, order
    s0, s1 = bounds
    blob, wl, codes, x1 = _CPU["blob"], _CPU["wl"], _CPU["codes"], _CPU["x1"]
    kt = wl.k // wl.tile_k
    tiles = list(range(s0 * kt, s1 * kt))
    rows = (s1 - s0) * wl.tile_n
    T = wl.tile_n * wl.tile_k
    with threadpool_limits(limits=1):
        h = oblob.parse(blob)
        syms = oblob.decode_symbols(blob, tiles)
        raw = np.frombuffer(blob, np.uint8, len(tiles) * T, h["raw_off"] + tiles[0] * T)
        raw = raw.reshape(len(tiles), T)
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
        y = ogemm.gemm_fp64(numerics.bf16_bits_to_f64(x1), numerics.bf16_bits_to_f64(w))
    r0 = s0 * wl.tile_n
    return s0, y, bool(np.array_equal(w, codes[r0:r0 + rows]))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, wl, blob):
    """The CPU oracle (rANS decode of the compressed layer + fp64 GEMV at
    M = 1) on a bounded sample: the first whole strips of the layer, about
    CPU_SAMPLE_WEIGHTS weights.  Timed on one core, then split over every core
    this process may run on (forked workers, one range of strips each)."""
    strips = wl.n // wl.tile_n
    s_count = max(1, min(strips, CPU_SAMPLE_WEIGHTS // (wl.tile_n * wl.k)))
    _CPU.update(blob=blob, wl=wl, codes=np.asarray(d["codes"]), x1=d["x"][:1])
    weights = s_count * wl.tile_n * wl.k
    decoded = weights * STORAGE_BYTES[wl.fmt]
    t0 = time.perf_counter()
    _, y1, ok1 = _cpu_strips((0, s_count))
    t1 = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    workers = min(cores, s_count)
    cuts = np.linspace(0, s_count, workers + 1).astype(int)
    parts = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(parts)) as pool:
        res = pool.map(_cpu_strips, parts)
    tn = time.perf_counter() - t0
    yn = np.concatenate([r[1] for r in sorted(res, key=lambda r: r[0])], axis=1)
    assert ok1 and all(r[2] for r in res), "oracle decode differs from the input weights"
    assert np.array_equal(yn, y1)
    _CPU.clear()
    return {"value": round(decoded / tn / 1e9, 6), "unit": "GB/s", "cores": len(parts),
            "kind": "oracle",
            "sample": "strips 0..%d of %d (rows 0..%d, all K: %d tiles, %.1f M weights), "
                      "rANS decode + fp64 GEMV at M=1; %d worker processes, numpy and BLAS "
                      "at 1 thread each" % (s_count - 1, strips, s_count * wl.tile_n - 1,
                                            s_count * (wl.k // wl.tile_k), weights / 1e6,
                                            len(parts)),
            "seconds": round(tn, 3), "single_core_value": round(decoded / t1 / 1e9, 6),
            "single_core_seconds": round(t1, 3), "affinity_cores": cores,
            "cpu_model": cpu_model(), "checksum": float(np.abs(y1).sum())}


# ------------------------------------------------------------------- GPU
def timed(fn, steps, warmup, stream):
    """Average ms per call over `steps` calls, bracketed by events on `stream`
    (the stream every library call is launched on)."""
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
    return start.elapsed_time(end) / steps


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


class Resident:
    """A workload's blob in HBM (rotating copies), its X, scales and workspaces."""

    def __init__(self, dgt, name, d, blob, dev):
        import torch
        self.dgt, self.d, self.dev = dgt, d, dev
        self.wl = d["workload"]
        self.blob = blob
        self.info = dgt.dgt_layer_info(blob)
        self.copies = max(2, math.ceil(ROTATE_BYTES / len(blob)))
        self.layers = [dgt.DeviceLayer(blob, dev) for _ in range(self.copies)]
        self.x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        self.scales = (torch.from_numpy(d["scales"].view(np.int16)).to(dev)
                       if d["scales"] is not None else None)
        self._ws = {}

    def call(self, m, stream):
        """A closure running one fused launch at M = m on copy i % copies."""
        import torch
        dgt = self.dgt
        xm = self.x[:m].contiguous()
        if m not in self._ws:
            self._ws[m] = (dgt.alloc_workspace(dgt.dgt_gemm_workspace(self.layers[0], m),
                                               self.dev),
                           torch.empty((m, self.wl.n), dtype=torch.float32, device=self.dev))
        ws, y = self._ws[m]

        def run(i):
            dgt.dgt_fused_decode_gemm(self.layers[i % self.copies], xm, scales=self.scales,
                                      w_scale=self.d["w_scale"], y=y, ws=ws, stream=stream)
        return run


def compress(dgt, name):
    import workloads
    d = workloads.make(name)
    wl = d["workload"]
    t0 = time.perf_counter()
    blob = dgt.dgt_compress_layer(wl.fmt, d["codes"], wl.tile_n, wl.tile_k, wl.lanes, wl.prob_bits)
    return d, blob, time.perf_counter() - t0


def entropy_over(wl, d, info):
    """Empirical entropy of the coded symbols per weight (+ raw bits) and the
    blob's excess over it."""
    from oracle import blob as oblob
    from oracle import entropy as oentropy
    sym, raw = oblob.symbolise(wl.fmt, d["codes"])
    h = oentropy.empirical_entropy(sym, oblob.alphabet_of(wl.fmt)) / oblob.weights_per_symbol(wl.fmt)
    raw_bits = 8.0 if raw is not None else 0.0
    return round(h, 4), round(info.bits_per_weight - h - raw_bits, 4)


def summary_line(dgt, name, dev, stream, reps, ms_list=(1, 256)):
    """M = 1 and M = 256 figures of another workload (compressed on the spot)."""
    d, blob, _ = compress(dgt, name)
    r = Resident(dgt, name, d, blob, dev)
    wl = r.wl
    out = {"workload": "%s: W %dx%d %s, tiles %dx%d, R=%d" % (name, wl.n, wl.k, wl.note,
                                                             wl.tile_n, wl.tile_k, wl.lanes),
           "bits_per_weight": round(r.info.bits_per_weight, 4)}
    h, over = entropy_over(wl, d, r.info)
    out["entropy_bits"], out["bits_over_entropy"] = h, over
    nk = wl.n * wl.k
    for m in ms_list:
        if m > d["x"].shape[0]:
            continue
        ms = timed(r.call(m, stream), reps, SEC_WARMUP, stream)
        out["fused_m%d_ms" % m] = round(ms, 4)
        if m == 1:
            out["decoded_gbs_m1"] = round(nk * STORAGE_BYTES[wl.fmt] / (ms * 1e-3) / 1e9, 3)
            out["hbm_frac_m1"] = round((len(blob) + wl.k * 2 + wl.n * 4) / (ms * 1e-3) / 1e9
                                       / HBM_PEAK_GBS, 4)
        else:
            out["fused_m%d_tflops" % m] = round(2.0 * m * nk / (ms * 1e-3) / 1e12, 3)
    del r
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each GPU would "
              "hold its own shard of the layer); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import decode_gemm_tile_amd as dgt
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    d, blob, encode_s = compress(dgt, args.workload)
    info = dgt.dgt_layer_info(blob)
    cpu = None
    if not args.no_cpu_baseline and wl.fmt in (4, 7):
        cpu = cpu_baseline(d, wl, blob)  # before the GPU is touched (forked workers)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    res = Resident(dgt, args.workload, d, blob, dev)
    copies = res.copies

    # ---- headline: the fused kernel at M = args.m (1 for the metric)
    m = args.m
    fused = res.call(m, stream)
    ms = timed(fused, args.steps, args.warmup, stream)
    dist = launch_distribution(fused, 50, stream)
    nk = wl.n * wl.k
    decoded_bytes = nk * STORAGE_BYTES[wl.fmt]
    value = decoded_bytes / (ms * 1e-3) / 1e9
    alg_bytes = len(blob) + m * wl.k * 2 + m * wl.n * 4
    if d["scales"] is not None:
        alg_bytes += d["scales"].nbytes
    achieved = alg_bytes / (ms * 1e-3) / 1e9

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
                     "traffic": traffic_from_profiles(args.workload, m),
                     "kernel_us": round(ms * 1e3, 3), "algorithmic_bytes": alg_bytes,
                     "per_launch": dist, "source_hash": source_hash(),
                     "valu": valu_from_profiles(args.workload, m, ms * 1e3)},
    }
    h, over = entropy_over(wl, d, info)
    secondary = {"bits_per_weight": round(info.bits_per_weight, 4), "entropy_bits": h,
                 "bits_over_entropy": over, "compressed_bytes": len(blob),
                 "encode_seconds": round(encode_s, 3)}

    if not args.no_secondary:
        reps = max(5, args.steps // 10)
        m2 = min(256, d["x"].shape[0])
        ms2 = timed(res.call(m2, stream), reps, SEC_WARMUP, stream)
        flops = 2.0 * m2 * nk
        secondary["fused_m%d_ms" % m2] = round(ms2, 4)
        secondary["fused_m%d_tflops" % m2] = round(flops / (ms2 * 1e-3) / 1e12, 3)
        secondary["fused_m%d_mfma_frac" % m2] = round(
            flops / (ms2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        # small batches (packed accumulators up to 8 rows, 16-row blocks to 16)
        # and medium ones (the large-M kernel's 16-wave subset form to 128 rows)
        for mm in (2, 4, 8, 16, 64, 128):
            if mm <= d["x"].shape[0] and mm != m2:
                secondary["fused_m%d_ms" % mm] = round(
                    timed(res.call(mm, stream), reps, SEC_WARMUP, stream), 4)
        wide = wl.fmt in (4, 6, 7, 8)
        codes = np.asarray(d["codes"])
        wraw = torch.from_numpy(codes.view(np.int16) if wide else codes.view(np.uint8)).to(dev)
        dcopies = max(2, math.ceil(ROTATE_BYTES / (nk * 2)))
        wd = [wraw.clone() for _ in range(dcopies)]
        del wraw
        dec = torch.empty((wl.n, wl.k), dtype=torch.int16 if wide else torch.uint8, device=dev)
        ablation = {}
        for mm in sorted({1, m2}):
            xm = res.x[:mm].contiguous()
            wsd = dgt.alloc_workspace(dgt.dgt_dense_workspace(wl.fmt, wl.n, wl.k, wl.tile_n, mm),
                                      dev)
            yd = torch.empty((mm, wl.n), dtype=torch.float32, device=dev)
            msd = timed(lambda i: dgt.dgt_dense_gemm(wl.fmt, wd[i % dcopies], xm,
                                                     tile_n=wl.tile_n, scales=res.scales,
                                                     w_scale=d["w_scale"], y=yd, ws=wsd,
                                                     stream=stream), reps, SEC_WARMUP, stream)
            ms_fused = ms if mm == m else secondary["fused_m%d_ms" % mm] if mm == m2 else \
                timed(res.call(mm, stream), reps, SEC_WARMUP, stream)
            secondary["dense_m%d_ms" % mm] = round(msd, 4)
            if mm == 1:
                secondary["dense_m1_weight_gbs"] = round(nk * 2 / (msd * 1e-3) / 1e9, 3)
                secondary["fused_speedup_vs_dense_m1"] = round(msd / ms_fused, 3)
            else:
                secondary["dense_m%d_tflops" % mm] = round(2.0 * mm * nk / (msd * 1e-3) / 1e12, 3)
            # ablation: layer-level decode to HBM, then the dense GEMM on the
            # decoded copy (two launches per step) against the fused kernel
            ms_dec = timed(lambda i: dgt.dgt_decode_tiles(res.layers[i % copies], out=dec,
                                                          stream=stream), reps, SEC_WARMUP, stream)

            def two_stage(i, xm=xm, yd=yd, wsd=wsd):
                dgt.dgt_decode_tiles(res.layers[i % copies], out=dec, stream=stream)
                dgt.dgt_dense_gemm(wl.fmt, dec, xm, tile_n=wl.tile_n, scales=res.scales,
                                   w_scale=d["w_scale"], y=yd, ws=wsd, stream=stream)
            ms_two = timed(two_stage, reps, SEC_WARMUP, stream)
            ablation["m%d" % mm] = {"decode_to_hbm_ms": round(ms_dec, 4),
                                    "two_stage_ms": round(ms_two, 4),
                                    "fused_ms": round(ms_fused, 4),
                                    "fused_speedup_vs_two_stage": round(ms_two / ms_fused, 3)}
            if mm > 16 and wl.lanes == 64:
                # the fused rung without ping-pong: one fragment buffer in the
                # large-M kernel (the library reads the switch at every call)
                os.environ["DGT_XM_SINGLE_BUFFER"] = "1"
                try:
                    ms_one = timed(res.call(mm, stream), reps, SEC_WARMUP, stream)
                finally:
                    del os.environ["DGT_XM_SINGLE_BUFFER"]
                ablation["m%d" % mm]["fused_single_buffer_ms"] = round(ms_one, 4)
                ablation["m%d" % mm]["ping_pong_speedup"] = round(ms_one / ms_fused, 3)
            if wide:
                # vendor GEMM on the uncompressed bf16 weight (reference point
                # only), alone and after the layer-level decode
                wts = [w.view(torch.bfloat16).t().contiguous() for w in wd]
                ms_lib = timed(lambda i: torch.matmul(xm, wts[i % len(wts)]), reps, SEC_WARMUP, stream)
                secondary["torch_matmul_bf16_m%d_ms" % mm] = round(ms_lib, 4)
                del wts
                decb = dec.view(torch.bfloat16)

                def two_stage_vendor(i, xm=xm):
                    dgt.dgt_decode_tiles(res.layers[i % copies], out=dec, stream=stream)
                    torch.nn.functional.linear(xm, decb)  # x @ W^T, W [N, K] as decoded
                ms_tv = timed(two_stage_vendor, reps, SEC_WARMUP, stream)
                ablation["m%d" % mm]["two_stage_vendor_gemm_ms"] = round(ms_tv, 4)
                ablation["m%d" % mm]["fused_speedup_vs_two_stage_vendor"] = round(
                    ms_tv / ms_fused, 3)
        secondary["ablation"] = ablation
        del wd, dec
        # the same layer in the other codings of its family: bits and time
        variants = []
        family = {4: "one_high_byte_per_symbol", 7: "high_byte_pairs", 8: "whole_words"}
        if wl.fmt in family and wl.lanes == 64:
            variants += [(nm, f, 64) for f, nm in family.items() if f != wl.fmt]
        if wl.lanes == 64 and wl.tile_n % 32 == 0 and wl.fmt != 8:
            variants.append(("two_states_per_lane", wl.fmt, 128))
        for vname, vfmt, vlanes in variants:
            blob2 = dgt.dgt_compress_layer(vfmt, d["codes"], wl.tile_n, wl.tile_k, vlanes)
            dv = dict(d)
            dv["workload"] = workloads.Workload(wl.name, vfmt, wl.n, wl.k, wl.tile_n, wl.tile_k,
                                                vlanes, wl.seed, wl.m_values, note=wl.note)
            r2 = Resident(dgt, args.workload, dv, blob2, dev)
            var = {"fmt": vfmt, "lanes": vlanes, "bits_per_weight": round(r2.info.bits_per_weight, 4)}
            for mm in (1, m2):
                var["fused_m%d_ms" % mm] = round(timed(r2.call(mm, stream), reps, SEC_WARMUP, stream), 4)
            var["decoded_gbs_m1"] = round(decoded_bytes / (var["fused_m1_ms"] * 1e-3) / 1e9, 3)
            secondary[vname] = var
            del r2
        # the other configurations the metric is quoted on
        others = {}
        for other in ("int4_ffn405", "int4_ffn405_pair", "bf16_mlp", "bf16_mlp_t128"):
            if other != args.workload:
                others[other] = summary_line(dgt, other, dev, stream, reps)
        secondary["other_workloads"] = others
    result["secondary"] = secondary

    if args.copy_calib:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = a.numel()

    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()
