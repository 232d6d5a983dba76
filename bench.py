#!/usr/bin/env python
"""Throughput of the lossless bf16/fp32 codec on one MI355X.

One step = compress + decompress of the whole workload (every stage of the
path: split, histogram, table, rANS encode, size scan, compaction, validation,
rANS decode and re-interleave), inputs already resident in HBM.  Prints one
JSON line:

  value          uncompressed GB/s of the round trip (input bytes / step time),
                 after untimed settle round trips (--settle-seconds) and W warm-ups
  compress_gbps / decompress_gbps   per direction (HIP events on the stream)
  ratio          compressed / original, and its entropy bound
  latency_ms     per call (whole call, HIP events on the stream), median and
                 minimum, per direction
  roofline       dominant kernel: algorithmic bytes per launch / its average
                 duration (two caller events the library records on the
                 launch stream around that kernel, uzip_*_batched_timed)
                 against the 8 TB/s HBM peak
  cpu_baseline   the CPU oracle (single thread, pinned to one core) on a
                 bounded sample of the same bytes, per direction; its output
                 also serves as a byte-for-byte check
  sampled_tables (full-table runs) the same workload measured again with
                 tables from each chunk's sample (uzip_compress_sampled)

Workloads (--workload): llama8b (default: the Llama-3-8B-shaped bf16 weight
set, 290 buffers, 16.06 GB, one batched call per direction), grad_bucket
(268,435,456 bf16 values, 512 MiB), pr1, fp32_grad, small_batch (4,096
buffers, batched), fp16_act (268,435,456 fp16 values), fp8_e4m3 and fp8_e5m2
(268,435,456 block-scaled fp8 weights each).  Every workload goes through the
batched entry points (a one-buffer call writes what the single-buffer call
writes).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
VALUE_DTYPE = {1: "bf16", 2: "fp32", 3: "fp16", 4: "fp8_e4m3fn", 5: "fp8_e5m2"}
# HBM bytes per launch from two rocprofv3 passes (FETCH_SIZE, then WRITE_SIZE)
# per workload and table kind (full tables, or ":sampled"), reads scaled by
# 2.000 and writes by 1.000 (what the same counters read for the benchmark's
# plain device copy of the workload's size); the kernel source they were taken
# on is identified by its digest, and a figure is reported only while the
# source is unchanged.
MEASURED_TRAFFIC_SOURCE = "8df00a0d92e6"
MEASURED_TRAFFIC = {
    ("llama8b", "k_encode"): 42806168477, ("llama8b", "k_decode"): 26857374381,
    ("llama8b:sampled", "k_encode"): 28817580774, ("llama8b:sampled", "k_decode"): 26886357178,
    ("grad_bucket", "k_encode"): 1435869249, ("grad_bucket", "k_decode"): 896979262,
    ("grad_bucket:sampled", "k_encode"): 963615543, ("grad_bucket:sampled", "k_decode"): 897817819,
}


def kernel_source_digest() -> str:
    import hashlib
    path = os.path.join(ROOT, "lossless_compression_float_amd", "csrc", "uzip_kernels.hip")
    try:
        return hashlib.sha256(open(path, "rb").read()).hexdigest()[:12]
    except OSError:
        return ""


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b",
                    choices=["grad_bucket", "pr1", "fp32_grad", "llama8b", "small_batch", "fp16_act", "fp8_e4m3",
                             "fp8_e5m2"])
    ap.add_argument("--chunk-bytes", type=int, default=0, help="uncompressed chunk size (0: the dtype's default)")
    ap.add_argument("--link-gbps", type=float, default=0.0,
                    help="compress with the per-call arbitration for a link of this many GB/s (0: plain compress)")
    ap.add_argument("--sampled", action="store_true",
                    help="tables from each chunk's sample (uzip_compress_sampled): one read of the input")
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="untimed round trips before the warm-up steps, until this much time has passed: the GPU "
                         "reaches its steady clocks only after a fraction of a second of sustained work")
    ap.add_argument("--no-sampled-line", action="store_true",
                    help="skip the second, shorter measurement with sampled tables that a full-table run appends")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU-oracle time to accumulate per direction")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


class Hip:
    """hipEvent helpers through the HIP runtime torch has already loaded."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b) -> float:
        assert self.rt.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


def make_workload(name, dev):
    import torch

    import workloads as W
    if name == "grad_bucket":
        ts = [W.gradient_bucket(W.GRAD_BUCKET_N, device=dev, seed=1)]
        desc = ("gradient bucket: 268,435,456 bf16 values (512 MiB) N(0, s^2), s log-uniform in [1e-5, 1e-2] per "
                "1M-value block, 0.01% Inf/NaN/denormal/zero, 64 KiB chunks")
        batched = False
    elif name == "pr1":
        ts = [W.pr1(dev)]
        desc = "PR1: 1,048,576 bf16 values N(0, 0.02^2) from seed 0 (2 MiB), 64 KiB chunks"
        batched = False
    elif name == "fp32_grad":
        ts = [W.fp32_gradients(W.FP32_GRAD_N, device=dev, seed=3)]
        desc = "fp32 gradients: 100,000,000 values N(0, 1e-6) + 10% Laplace(0, 1e-4) (400 MB), 256 KiB chunks"
        batched = False
    elif name == "llama8b":
        ts = [t.reshape(-1) for t in W.llama3_8b_weights(device=dev, seed=2)]
        desc = ("RL weight sync: Llama-3-8B-shaped bf16 weight set, 290 buffers, 8,030,257,152 values (16.06 GB), "
                "N(0, 0.02^2), RMSNorm vectors 1.0, one batched call, 64 KiB chunks")
        batched = True
    elif name == "fp16_act":
        ts = [W.fp16_activations(W.FP16_ACT_N, device=dev, seed=5)]
        desc = ("fp16 activations: 268,435,456 values (512 MiB), rows of 8192 N(0,1) x log-normal(0, 0.5) per-row "
                "scale")
        batched = False
    elif name in ("fp8_e4m3", "fp8_e5m2"):
        fmt = torch.float8_e4m3fn if name == "fp8_e4m3" else torch.float8_e5m2
        ts = [W.fp8_weights(W.FP8_WEIGHT_N, device=dev, seed=6, fmt=fmt)]
        desc = ("fp8 %s weights: 268,435,456 values (256 MiB), N(0,1) scaled per 8192-value block so the block "
                "absmax is the format's largest finite value" % ("e4m3fn" if name == "fp8_e4m3" else "e5m2"))
        batched = False
    else:
        ts = W.small_message_batch(device=dev, seed=4)
        desc = ("small-message batch: 4,096 bf16 activation buffers, 1-64 tokens x 8192 hidden, N(0,1) x "
                "log-normal(0, 0.5) per-token RMS, one batched launch, 64 KiB chunks")
        batched = True
    torch.cuda.synchronize()
    return ts, desc, batched


def entropy_bound(ts, code, chunk_bytes):
    """The oracle's entropy bound (sum over chunks of the raw bytes plus
    n_i H_i / 8), buffer by buffer on host copies, 16 buffers at a time (the
    oracle is plain C called through ctypes, which releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import workloads as W

    def one(t):
        return oracle.entropy_bound(code, W.bits_numpy(t), chunk_bytes) if t.numel() else 0.0

    with ThreadPoolExecutor(max_workers=16) as pool:
        return sum(pool.map(one, ts))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one MI355X: this codec runs on a single GPU (no collectives, no sharding); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import lossless_compression_float_amd as uz

    dev = "cuda:0"
    torch.cuda.set_device(0)
    hip = Hip()
    print("# workload %s: generating inputs" % args.workload, file=sys.stderr, flush=True)
    ts, desc, batched = make_workload(args.workload, dev)
    dtype = ts[0].dtype
    code = uz.dtype_code(dtype)
    eb = dtype.itemsize
    # raw (sign+mantissa) bits per value, packed back to back in the raw region
    rbits = {uz.UZIP_BF16: 8, uz.UZIP_FP32: 24, uz.UZIP_FP16: 11, uz.UZIP_FP8_E4M3: 4, uz.UZIP_FP8_E5M2: 3}[code]
    cb = args.chunk_bytes or (262144 if code == uz.UZIP_FP32 else 65536)
    chunk_elems = cb // eb
    ns = [t.numel() for t in ts]
    n_total = sum(ns)
    raw_region = sum((n * rbits + 7) // 8 for n in ns)
    in_bytes = n_total * eb

    # preallocated outputs and workspaces
    caps = [uz.uzip_max_compressed_size(code, n, cb) for n in ns]
    if 0 in caps:
        sys.exit("invalid --chunk-bytes %d" % args.chunk_bytes)
    outs = [torch.empty(c, dtype=torch.uint8, device=dev) for c in caps]
    backs = [torch.empty(n, dtype=dtype, device=dev) for n in ns]
    ws = uz.workspace(uz.uzip_workspace_size_batched(code, ns, cb), dev)
    sizes = torch.empty(len(ts), dtype=torch.int64, device=dev)
    status = torch.empty(len(ts), dtype=torch.int32, device=dev)

    L = uz.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # the calls' host arrays, built once (what a caller moving the same set of
    # buffers every step keeps); the library builds and uploads its device
    # descriptors on every call
    a_in = uz._ptrs([t.data_ptr() if t.numel() else 0 for t in ts])
    a_n = uz._sizes(ns)
    a_out = uz._ptrs([o.data_ptr() for o in outs])
    a_cap = uz._sizes([o.numel() for o in outs])
    a_inb = uz._sizes(caps)  # decompress: capacity readable; the header's total is validated against it
    a_back = uz._ptrs([b.data_ptr() if b.numel() else 0 for b in backs])

    pol = None
    if args.link_gbps > 0:
        # codec rates near this codec's own measured bf16 throughput; nothing
        # of the codec time hidden by overlap; a 10 us fixed cost per coded call
        pol = uz.policy(link_bytes_per_us=int(args.link_gbps * 1000), encode_bytes_per_us=1_250_000,
                        decode_bytes_per_us=1_600_000, fixed_ns=10_000, small_bytes=0,
                        exposed_encode_permil=1000, exposed_decode_permil=1000, min_gain_permil=20)
        plans = torch.empty(4 * len(ts), dtype=torch.int64, device=dev)

    pol_ref = ctypes.byref(pol) if pol is not None else None
    plans_ptr = plans.data_ptr() if pol is not None else None

    def compress(sampled=args.sampled, ev=(None, None)):
        st = L.uzip_compress_batched_timed(code, len(ts), a_in.ptr, a_n.ptr, cb, 1 if sampled else 0, pol_ref,
                                           a_out.ptr, a_cap.ptr, sizes.data_ptr(), plans_ptr, ws.data_ptr(),
                                           ws.numel(), stream, ev[0], ev[1])
        if st != 0:
            raise uz.UzipError(st, "uzip_compress_batched_timed")

    def decompress(ev=(None, None)):
        st = L.uzip_decompress_batched_timed(code, len(ts), a_out.ptr, a_inb.ptr, a_n.ptr, a_back.ptr,
                                             status.data_ptr(), ws.data_ptr(), ws.numel(), stream, ev[0], ev[1])
        if st != 0:
            raise uz.UzipError(st, "uzip_decompress_batched_timed")

    print("# %d buffers, %d values, %.1f MB; warmup %d, steps %d" % (len(ts), n_total, in_bytes / 1e6, args.warmup,
                                                                      args.steps), file=sys.stderr, flush=True)
    K = args.steps

    # settle: untimed round trips until the GPU has run for --settle-seconds
    # (measured: with 3 warm-up steps alone the gradient bucket's kernels run
    # 5-10% slower than in steady state)
    def settle(sampled=args.sampled):
        steps, t = 0, time.perf_counter()
        while time.perf_counter() - t < args.settle_seconds:
            for _ in range(4):
                compress(sampled)
                decompress()
            steps += 4
            torch.cuda.synchronize()
        return steps, time.perf_counter() - t

    settle_steps, settle_s = settle()

    def timed(sampled):
        """W warm-ups, then K timed steps: step time, whole-call times per
        direction (torch events) and the main coding kernels' durations (HIP
        events the library records on the launch stream)."""
        for _ in range(args.warmup):
            compress(sampled)
            decompress()
        torch.cuda.synchronize()
        enc_ev = [(hip.event(), hip.event()) for _ in range(K)]
        dec_ev = [(hip.event(), hip.event()) for _ in range(K)]
        c_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        d_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            c_ev[k][0].record()
            compress(sampled, enc_ev[k])
            c_ev[k][1].record()
            d_ev[k][0].record()
            decompress(dec_ev[k])
            d_ev[k][1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        res = ((t1 - t0) * 1e3 / K, sorted(a.elapsed_time(b) for a, b in c_ev), sorted(a.elapsed_time(b) for a, b in d_ev),
               sum(hip.elapsed_ms(a, b) for a, b in enc_ev) / K, sum(hip.elapsed_ms(a, b) for a, b in dec_ev) / K)
        for a, b in enc_ev + dec_ev:
            hip.destroy(a)
            hip.destroy(b)
        return res

    iv = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[eb]

    def roundtrip_exact():
        """correctness of what was timed: bit-exact round trip, valid status"""
        return all(s == 0 for s in status.cpu().tolist()) and all(
            torch.equal(a.view(iv), b.view(iv)) for a, b in zip(ts, backs))

    def record_bytes(comp_sizes):
        exp_offs = [((((64 + 8 * ((n + chunk_elems - 1) // chunk_elems + 1)) + 15) // 16 * 16 + (n * rbits + 7) // 8)
                     + 15) // 16 * 16
                    for n in ns]
        return exp_offs, sum(s - e for s, e in zip(comp_sizes, exp_offs))

    ms_step, comp_ms, dec_ms, enc_kernel_ms, dec_kernel_ms = timed(args.sampled)
    roundtrip_ok = roundtrip_exact()
    comp_sizes = sizes.cpu().tolist()
    comp_bytes = sum(comp_sizes)
    bound = entropy_bound(ts, code, cb)

    # algorithmic bytes per launch of the two coding kernels
    exp_offs, rec_bytes = record_bytes(comp_sizes)
    decisions = [p["decision"] for p in uz.plans_as_dicts(plans)] if pol is not None else []
    # a RAW plan's k_encode only splits (k_compact writes the RAW records)
    raw_planned = sum(n for n, dcs in zip(ns, decisions) if dcs != uz.UZIP_PLAN_CODED)
    enc_bytes = n_total * eb + raw_region + rec_bytes - sum(
        s - e for s, e, dcs in zip(comp_sizes, exp_offs, decisions) if dcs != uz.UZIP_PLAN_CODED)
    dec_bytes = raw_region + rec_bytes + sum(64 + 8 * ((n + chunk_elems - 1) // chunk_elems + 1) for n in ns) + \
        n_total * eb
    all_raw = pol is not None and raw_planned == n_total
    if enc_kernel_ms >= dec_kernel_ms and not all_raw:
        kname, kbytes, kms = "k_encode", enc_bytes, enc_kernel_ms
    else:
        kname, kbytes, kms = "k_decode", dec_bytes, dec_kernel_ms
    achieved = kbytes / (kms * 1e-3) / 1e9
    tkey = (args.workload + (":sampled" if args.sampled else ""), kname)
    traffic = MEASURED_TRAFFIC.get(tkey) if kernel_source_digest() == MEASURED_TRAFFIC_SOURCE else None
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "traffic_over_algorithmic": round(traffic / kbytes, 4) if traffic else None,
                "algorithmic_bytes": kbytes, "avg_ms": round(kms, 4),
                "k_encode_ms": round(enc_kernel_ms, 4), "k_decode_ms": round(dec_kernel_ms, 4),
                # (under a RAW plan k_encode returns at once and k_raw_frame, which
                # the events do not bracket, writes the frame: no encode figure)
                "k_encode_frac": None if all_raw else round(enc_bytes / (enc_kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "k_decode_frac": round(dec_bytes / (dec_kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    copy_gbps = copy_reference(ts, K)
    roofline["hbm_copy_gbps"] = round(copy_gbps, 1)
    roofline["frac_of_copy"] = round(achieved / copy_gbps, 4)

    med_rt_ms = ms_step
    cpu = None
    oracle_match = None
    if not args.no_cpu_baseline:
        cpu, oracle_match = cpu_baseline(ts, outs, comp_sizes, code, args.cpu_seconds, cb, pol, args.sampled,
                                         in_bytes / (med_rt_ms * 1e-3) / 1e9)

    med_c = comp_ms[len(comp_ms) // 2]
    med_d = dec_ms[len(dec_ms) // 2]
    line = {
        "metric": "compress/decompress GB/s (uncompressed) + ratio + % HBM roofline, 1 MI355X",
        "value": round(in_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "seconds": round(settle_s, 3)},
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": desc, "values": n_total, "buffers": len(ts), "input_bytes": in_bytes,
                   "value_dtype": VALUE_DTYPE[code], "chunk_bytes": chunk_elems * eb,
                   "tables": "sampled" if args.sampled else "full", "step": "compress + decompress"},
        "compress_gbps": round(in_bytes / (med_c * 1e-3) / 1e9, 2),
        "decompress_gbps": round(in_bytes / (med_d * 1e-3) / 1e9, 2),
        "latency_ms": {"compress": {"median": round(med_c, 4), "min": round(comp_ms[0], 4)},
                       "decompress": {"median": round(med_d, 4), "min": round(dec_ms[0], 4)},
                       "per": "whole call over all %d buffers" % len(ts)},
        "ratio": round(comp_bytes / in_bytes, 5),
        "entropy_bound_ratio": round(bound / in_bytes, 5),
        "ratio_over_bound": round(comp_bytes / bound, 5),
        "compressed_bytes": comp_bytes,
        "roundtrip_bit_exact": roundtrip_ok,
        "oracle_bytes_match": oracle_match,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if pol is None and not args.sampled and not args.no_sampled_line:
        # the same workload with sampled tables (uzip_compress_sampled), a
        # second and separate measurement: the headline figures above are the
        # full-table ones; settled again, since the GPU has idled through the
        # CPU baseline
        settle(True)
        s_step, s_comp, s_dec, s_enc, s_decm = timed(True)
        s_ok = roundtrip_exact()
        s_sizes = sizes.cpu().tolist()
        s_bytes = sum(s_sizes)
        _, s_rec = record_bytes(s_sizes)
        s_enc_b = n_total * eb + raw_region + s_rec
        s_dec_b = raw_region + s_rec + sum(64 + 8 * ((n + chunk_elems - 1) // chunk_elems + 1) for n in ns) + n_total * eb
        s_match = None
        if not args.no_cpu_baseline:
            import oracle
            import workloads as W
            s_match = bool(np.array_equal(oracle.compress_sampled(code, W.bits_numpy(ts[0]), cb),
                                          outs[0][:s_sizes[0]].cpu().numpy()))
        line["sampled_tables"] = {
            "value": round(in_bytes / (s_step * 1e-3) / 1e9, 2),
            "compress_gbps": round(in_bytes / (s_comp[len(s_comp) // 2] * 1e-3) / 1e9, 2),
            "decompress_gbps": round(in_bytes / (s_dec[len(s_dec) // 2] * 1e-3) / 1e9, 2),
            "ratio": round(s_bytes / in_bytes, 5), "ratio_over_bound": round(s_bytes / bound, 5),
            "k_encode_ms": round(s_enc, 4), "k_decode_ms": round(s_decm, 4),
            "k_encode_frac": round(s_enc_b / (s_enc * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "k_decode_frac": round(s_dec_b / (s_decm * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "roundtrip_bit_exact": s_ok, "oracle_bytes_match_first_buffer": s_match}
        roundtrip_ok = roundtrip_ok and s_ok
        oracle_match = oracle_match if s_match is not False else False
    if pol is not None:
        line["config"]["arbitration"] = {f: getattr(pol, f) for f, _ in pol._fields_}
        line["plans"] = {"coded": decisions.count(0), "raw": decisions.count(1), "raw_small": decisions.count(2),
                         "raw_realized": decisions.count(3), "raw_planned_values": raw_planned}
        if len(ts) == 1:
            line["plans"]["plan"] = uz.plans_as_dicts(plans)[0]
    print(json.dumps(line), flush=True)
    if not roundtrip_ok or oracle_match is False:
        sys.exit(1)


def copy_reference(ts, steps):
    """Measured HBM bandwidth of a plain device-to-device copy of the
    workload's input size (read + write bytes / time), a second reference
    beside the 8 TB/s peak.  The same copy kernel calibrates the rocprofv3
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    nbytes = sum(t.numel() * t.element_size() for t in ts)
    src = torch.empty(nbytes, dtype=torch.uint8, device=ts[0].device)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(ts, outs, comp_sizes, code, min_seconds, chunk_bytes, pol=None, sampled=False, gpu_gbps=None):
    """The oracle (plain single-threaded C, gcc -O2) on a bounded sample of the
    same workload: whole buffers, in order, up to 512 MiB of input (at least
    one buffer).  Compress and decompress are timed separately, each repeated
    until min_seconds have been spent, with the calling thread pinned to one
    core (os.sched_setaffinity on this thread; restored afterwards).  Also
    compares the oracle's compressed bytes with the GPU's for every sampled
    buffer."""
    import numpy as np

    import oracle
    import workloads as W
    budget = 512 << 20
    picked, acc = [], 0
    for i, t in enumerate(ts):
        nb = t.numel() * t.element_size()
        if picked and acc + nb > budget:
            break
        picked.append(i)
        acc += nb
    host = [W.bits_numpy(ts[i]) for i in picked]
    comp = (oracle.compress_sampled if sampled else oracle.compress)
    match = True
    frames = []
    for i, h in zip(picked, host):
        if pol is None:
            want = comp(code, h, chunk_bytes)
        else:  # the arbitrated frame (the plan may have chosen RAW)
            opol = oracle.Policy(**{f: getattr(pol, f) for f, _ in pol._fields_})
            want = oracle.compress_arbitrated(code, h, opol, chunk_bytes)[0]
        got = outs[i][:comp_sizes[i]].cpu().numpy()
        match = match and np.array_equal(want, got)
        frames.append(want)
    sample_bytes = sum(h.size * h.itemsize for h in host)
    old_aff = os.sched_getaffinity(0)
    core = min(old_aff)
    os.sched_setaffinity(0, {core})
    try:
        def timed(fn):
            spent, passes = 0.0, 0
            while passes == 0 or spent < min_seconds:
                t0 = time.perf_counter()
                fn()
                spent += time.perf_counter() - t0
                passes += 1
                if spent > 60:
                    break
            return spent, passes

        def do_compress():
            for h in host:
                comp(code, h, chunk_bytes)

        def do_decompress():
            for h, f in zip(host, frames):
                st, _ = oracle.decompress(f, code, h.size)
                assert st == 0

        c_s, c_p = timed(do_compress)
        d_s, d_p = timed(do_decompress)
    finally:
        os.sched_setaffinity(0, old_aff)
    c_gbps = sample_bytes * c_p / c_s / 1e9
    d_gbps = sample_bytes * d_p / d_s / 1e9
    rt_gbps = 1.0 / (1.0 / c_gbps + 1.0 / d_gbps)
    out = {"value": round(rt_gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "compress_gbps": round(c_gbps, 4), "decompress_gbps": round(d_gbps, 4),
           "sample": "%d of %d buffers, %d values (%.1f MB); compress %d passes in %.1f s, decompress %d passes in "
                     "%.1f s; value = round trip (input bytes over compress + decompress time), one thread pinned "
                     "to core %d" % (len(picked), len(ts), sum(h.size for h in host), sample_bytes / 1e6, c_p, c_s,
                                      d_p, d_s, core),
           "cpu_model": _cpu_model(), "nproc": os.cpu_count()}
    if gpu_gbps:
        out["gpu_over_cpu"] = round(gpu_gbps / rt_gbps, 1)
    return out, bool(match)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
