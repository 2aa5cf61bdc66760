#!/usr/bin/env python3
"""Benchmark of the KDA forward on one MI355X.

Headline: the chunked forward on the long-context workload (B=1, T=8192, H=16 q/k heads,
HV=32 value heads, K=V=128, bf16 q/k/v/beta, fp32 log2 gates clamped at -5, no initial
state, no final state). A step is one call of kda_chunk_fwd (dense mode: the Stage 1+2
kernel, then the Stage 3+4 scan) with its inputs resident in HBM. Each of the --steps
timed steps is preceded, outside its events, by a 512 MB write, so its 336 MB of inputs
come from HBM and not the 256 MB MALL; `value` is tokens per second at the median step
time, `ms_per_step` that median. Before them the same pattern (write, step) runs for
--preheat-s seconds, so the clocks have settled at the level that pattern holds (a short
timed window right after other work read up to 10% slow), then --warmup untimed steps.
Every other timed window (back-to-back reps of one call) first runs its own call for a
quarter second (at most --preheat-s).

Also reported on the same JSON line:
  * roofline     -- the forward (both kernels) against HBM peak on the method's own bytes
                    (inputs read once + o written once: 336,068,608 B per call), with the
                    average launch duration of each kernel timed live on the library's
                    stream (events recorded by kda_chunk_fwd_timed), each kernel's share of
                    the method's bytes, the bytes its records add by design, and the HBM
                    bytes the counters measured (committed rocprofv3 summary, when taken on
                    the current kernel source);
  * steps_ms     -- median, p10, p90, mean of the timed steps; back_to_back -- the same
                    forward with no flush between steps (mean);
  * path         -- matrix-core fractions (exact and dense-tile flop counts) against the
                    published peak and against the measured ceiling (`ceilings`);
  * ceilings     -- a bf16 matrix-core loop built here, the peak from the device's CU count
                    and clock, and a plain HBM stream (the decode's);
  * c2           -- the forward on B=2 T=4096 H=HV=16 with initial and final states
                    (timed like the headline) against its 205.8 MB floor;
  * gated, fused_inputs -- the headline with the gate activation (and the q/k norm and
                    beta sigmoid) fused into the loads;
  * backward     -- the chunked backward of the headline forward (every input gradient),
                    and a training step split into kda_chunk_fwd_train (the forward keeping
                    the backward's checkpoints) and kda_chunk_bwd_saved (no recompute);
  * varlen       -- the packed-sequence forward (64 slots, ~31k tokens, 4 empty slots,
                    initial and final states);
  * decode       -- the per-token recurrent forward on 4096 sequences x 32 heads (one token
                    each, fp32 states in and out): state GB/s and fraction of HBM peak, and
                    a plain-stream ceiling (torch.neg over the same state bytes);
  * cpu_baseline -- the fp64 CPU oracle on the full headline workload, host threads.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--preheat-s 1.0]
       [--only headline]   (the headline leg alone: for profiling its kernels)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LEGS = ["headline", "c2", "gated", "backward", "decode", "varlen"]
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak


def hip_runtime():
    """The HIP runtime already loaded in this process (torch's), for event timing."""
    for line in open("/proc/self/maps"):
        path = line.split()[-1]
        if "libamdhip64" in path and os.path.exists(path):
            lib = ctypes.CDLL(path)
            break
    else:
        lib = ctypes.CDLL("libamdhip64.so.7")
    vp = ctypes.c_void_p
    lib.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
    lib.hipEventRecord.argtypes = [vp, vp]
    lib.hipEventSynchronize.argtypes = [vp]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
    lib.hipEventDestroy.argtypes = [vp]
    return lib


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev[i] = e

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def record_bytes(K, V, elem, compact=False):
    """Bytes of one Stage 2 record (see the workspace layout in the library): w, qg, kg^T,
    Aqk in the operand type, u and 2^G in fp32; on the bf16 path the residuals of qg,
    kg^T and Aqk as a second bf16 tile each, or, in compact records (the layout of
    launches with many chains), as fp8 tiles (a byte per value) with one 32-bit scale
    word per 16-row band and lane."""
    b = 64 * K * elem + 2 * 64 * K * elem + 64 * 64 * elem + 64 * V * 4 + K * 4
    if elem == 2 and compact:
        b += 2 * 64 * K + 64 * 64 + (64 // 16 + K // 16 + 64 // 16) * 64 * 4
    elif elem == 2:
        b += 2 * 64 * K * elem + 64 * 64 * elem
    return b


def source_hash():
    h = hashlib.sha256()
    for f in ("kda_chunk.hip", "kda_chunk_common.h", "kda_device.h"):
        h.update(open(os.path.join(ROOT, "gated_delta_rule_64_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per launch of each forward kernel from the committed rocprofv3 counter
    summary, when it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_c3.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("bytes_per_launch")


def pctl(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(q * len(xs)))]


def stats(xs):
    return {"median": pctl(xs, 0.5), "p10": pctl(xs, 0.1), "p90": pctl(xs, 0.9),
            "mean": sum(xs) / len(xs), "n": len(xs)}


class Flusher:
    """A 512 MB buffer written between timed reps (outside their events), so a rep's
    inputs are read from HBM and not from the 256 MB MALL."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.r = 0

    def __call__(self):
        self.r += 1
        self.buf.fill_(self.r & 0xFF)


def timed_flushed(call, steps, hip, sptr, flush, nev=0):
    """``steps`` reps of ``call(events)``, each after a flush; per rep the events are
    [start, (nev inner events), end]. Returns the per-rep lists of event spans: the whole
    rep, and one list per inner segment."""
    import torch
    per = nev + 2
    ev = Events(hip, per * steps)
    for r in range(steps):
        flush()
        base = per * r
        hip.hipEventRecord(ev.ev[base], sptr)
        call(ev.ev[base: base + per])
        hip.hipEventRecord(ev.ev[base + per - 1], sptr)
    torch.cuda.synchronize()
    whole = [ev.ms(per * r, per * r + per - 1) for r in range(steps)]
    segs = [[ev.ms(per * r + i, per * r + i + 1) for r in range(steps)] for i in range(per - 1)]
    ev.close()
    return whole, segs


def back_to_back(call, steps, hip, sptr):
    import torch
    ev = Events(hip, 2)
    torch.cuda.synchronize()
    hip.hipEventRecord(ev.ev[0], sptr)
    for _ in range(steps):
        call()
    hip.hipEventRecord(ev.ev[1], sptr)
    torch.cuda.synchronize()
    ms = ev.ms(0, 1) / steps
    ev.close()
    return ms


def device_peak_tflops(hip, dev_index):
    """bf16 dense matrix-core peak from the device's own CU count and peak shader clock:
    CUs x clock x 4,096 flop per clock per CU (four SIMDs, one 16x16x32 bf16 product of
    16,384 flops every 16 clocks each)."""
    cus, khz = ctypes.c_int(), ctypes.c_int()
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    # hipDeviceAttributeMultiprocessorCount = 63, hipDeviceAttributeClockRate = 5 (kHz)
    if hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, dev_index) != 0:
        return None
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, dev_index) != 0:
        return None
    return {"cus": cus.value, "clock_mhz": khz.value / 1e3,
            "bf16_tflops": cus.value * khz.value * 1e3 * 4096 / 1e12}


def mfma_ceiling(hip, sptr, dev):
    """Time the bf16 matrix-core loop of libkda_ceiling.so (every wave eight independent
    16x16x32 products per trip, 16 waves per CU)."""
    import torch
    path = os.path.join(ROOT, "gated_delta_rule_64_amd", "libkda_ceiling.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.kda_ceiling_mfma_bf16.restype = ctypes.c_int
    lib.kda_ceiling_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, iters = 256 * 4, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    for _ in range(2):
        assert lib.kda_ceiling_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), sptr) == 0
    torch.cuda.synchronize()
    ev = Events(hip, 2)
    hip.hipEventRecord(ev.ev[0], sptr)
    assert lib.kda_ceiling_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), sptr) == 0
    hip.hipEventRecord(ev.ev[1], sptr)
    torch.cuda.synchronize()
    ms = ev.ms(0, 1)
    ev.close()
    flops = blocks * 4 * iters * 8 * 16384.0
    return {"kernel": "bf16 16x16x32 matrix-core loop (1,024 blocks x 4 waves, 8 independent chains)",
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--preheat-s", type=float, default=1.0,
                    help="seconds of back-to-back headline forwards before the warm-up steps")
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--only", choices=LEGS, default=None,
                    help="run one leg alone (for profiling its kernels); the headline leg "
                         "always runs first unless another leg is named")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch one plain elementwise kernel that reads and writes 1 GiB "
                         "(torch.neg on fp32), outside the timed region: the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(sequences and heads shard across GPUs with no communication; run one "
              "process per GPU on its own share)", file=sys.stderr)
        sys.exit(2)
    steps = max(1, args.steps)

    import torch
    from gated_delta_rule_64_amd import _lib
    if not os.path.exists(_lib.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    import gated_delta_rule_64_amd as kda
    from gated_delta_rule_64_amd import inputs

    lib = kda.load_library()
    hip = hip_runtime()
    vp = ctypes.c_void_p
    lib.kda_chunk_fwd_timed.restype = ctypes.c_int
    lib.kda_chunk_fwd_timed.argtypes = list(lib.kda_chunk_fwd.argtypes) + [vp]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = vp(stream.cuda_stream)
    flush = Flusher(dev)

    def timed_call(d, out, ws, ws_bytes, B, T, H, HV, K, V, N, final=None):
        """kda_chunk_fwd_timed on dense inputs; returns call(events) where events is a
        4-slot list [start, mid, end] mapped to the library's slots 0, 2, 3."""
        h0 = d["initial_state"]

        def call(evs):
            slots = None if evs is None else ctypes.cast((vp * 4)(evs[0], None, evs[1], evs[2]), vp)
            rc = lib.kda_chunk_fwd_timed(
                vp(d["q"].data_ptr()), vp(d["k"].data_ptr()), vp(d["v"].data_ptr()),
                vp(d["g"].data_ptr()), vp(d["beta"].data_ptr()),
                None if h0 is None else vp(h0.data_ptr()), None, N, vp(out.data_ptr()),
                None if final is None else vp(final.data_ptr()), B, T, H, HV, K, V, kda.KDA_BF16,
                kda.KDA_BF16, 0.0, 64, vp(ws.data_ptr()), ws_bytes, None, sptr, slots)
            if rc != 0:
                raise RuntimeError(lib.kda_last_error().decode())
        return call

    def want(leg):
        return args.only is None or args.only == leg

    # ---------------- headline: c3 ----------------
    w = inputs.WORKLOADS["c3"]
    d = inputs.make(w, device=dev)
    B, T, H, HV, K, V = w.B, w.T, w.H, w.HV, w.K, w.V
    N = B
    ws_bytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, 0, kda.KDA_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(d["v"])
    call = timed_call(d, out, ws, ws_bytes, B, T, H, HV, K, V, N)

    # the method's bytes: inputs read once, o written once (SURVEY's 1,282 B per
    # token-head at GVA 2); which kernel moves which share of them; and what the records
    # between the two kernels add by design
    q_b = 2 * B * T * H * K * 2                 # q, k
    v_b = B * T * HV * V * 2
    g_b = B * T * HV * K * 4
    beta_b = B * T * HV * 2
    o_b = B * T * HV * V * 2
    method_bytes = q_b + v_b + g_b + beta_b + o_b
    in_bytes = method_bytes - o_b
    tokens = B * T

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)          # 1 GiB read + 1 GiB written by one plain kernel
        torch.cuda.synchronize()
        del src, dst
    # pre-heat: a timed window's own pattern for a fixed wall time before it, so its reps
    # run at the clocks the GPU settles at under that pattern (a cold start ran both
    # kernels ~17% slower, and 20 flushed steps right after back-to-back calls 5-10%)
    if not want("headline"):
        args.preheat_s = min(args.preheat_s, 0.2)
    leg_pre_s = min(0.25, max(0.0, args.preheat_s))

    def preheat(fn, seconds, flushed=False):
        t_end = time.time() + max(0.0, seconds)
        n = 0
        while True:
            for _ in range(10):
                if flushed:
                    flush()
                fn()
            n += 10
            torch.cuda.synchronize()
            if time.time() >= t_end:
                return n

    n_pre = preheat(lambda: call(None), args.preheat_s, flushed=True)
    for _ in range(args.warmup):
        flush()
        call(None)
    torch.cuda.synchronize()
    result = {"leg": args.only, "note": "a single leg for profiling its kernels; no headline figures in this run"}
    if want("headline"):
        whole, (seg_intra, seg_scan) = timed_flushed(call, steps, hip, sptr, flush, nev=1)
        st = stats(whole)
        ms_per_step = st["median"]
        tok_s = tokens / (ms_per_step * 1e-3)
        intra_ms = sum(seg_intra) / steps
        scan_ms = sum(seg_scan) / steps
        fwd_ms = intra_ms + scan_ms
        preheat(lambda: call(None), leg_pre_s)
        b2b_ms = back_to_back(lambda: call(None), steps, hip, sptr)

        flops_exact = 141013.0 * B * T * HV
        flops_dense = 180224.0 * B * T * HV
        nchunks = B * ((T + 63) // 64)
        rec = record_bytes(K, V, 2) * nchunks * HV
        counters = traffic_from_profiles()
        traffic = None
        if counters and "intra" in counters and "scan" in counters:
            traffic = counters["intra"] + counters["scan"]
        achieved = method_bytes / (fwd_ms * 1e-3) / 1e9
        roofline = {
            "bound": "hbm", "kernel": "chunk forward: Stage 1+2 kernel + scan kernel (one call)",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic, "algorithmic_bytes": method_bytes, "avg_launch_ms": fwd_ms,
            "dominant": "scan" if scan_ms >= intra_ms else "intra",
            "kernels": {
                "intra": {"avg_ms": intra_ms, "method_bytes": in_bytes,
                          "method_GBs": in_bytes / (intra_ms * 1e-3) / 1e9,
                          "design_bytes": in_bytes + rec,
                          "counter_bytes": counters.get("intra") if counters else None},
                "scan": {"avg_ms": scan_ms, "method_bytes": o_b,
                         "method_GBs": o_b / (scan_ms * 1e-3) / 1e9,
                         "design_bytes": rec + o_b,
                         "counter_bytes": counters.get("scan") if counters else None},
            },
            "record_bytes_per_call": rec,
        }
        peak_dev = device_peak_tflops(hip, 0)
        ceil = mfma_ceiling(hip, sptr, dev)
        tflops_exact = flops_exact / (ms_per_step * 1e-3) / 1e12
        path = {
            "hbm_floor_bytes": method_bytes, "hbm_floor_us": method_bytes / HBM_PEAK_GBS / 1e3,
            "achieved_GBs": method_bytes / (ms_per_step * 1e-3) / 1e9,
            "hbm_frac": method_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tflops_exact": tflops_exact,
            "mfma_frac_exact_flops": tflops_exact / BF16_PEAK_TFLOPS,
            "mfma_frac_dense_tile_flops": flops_dense / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "mfma_frac_exact_of_measured_ceiling": tflops_exact / ceil["tflops"] if ceil else None,
        }
        result = {
            "metric": "KDA fwd tokens/s + % bf16 MFMA peak at T=8192; decode state GB/s % HBM",
            "value": tok_s,
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": args.warmup,
            "ms_per_step": ms_per_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), g=log2(sigmoid(N(2,1))) >= -5, beta=sigmoid(N(0,1)))",
            "config": {"workload": "chunk_kda fwd B=1 T=8192 H=16 HV=32 K=V=128 bf16, h0=None, no final state",
                       "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
            "timing": {"per_step": "512 MB write before each step (outside its events); value at the median step",
                       "preheat": "the same write + step pattern for preheat_s seconds, then the warm-up steps",
                       "preheat_s": args.preheat_s, "preheat_steps": n_pre},
            "steps_ms": st,
            "back_to_back": {"ms_per_step": b2b_ms, "tokens_per_s": tokens / (b2b_ms * 1e-3)},
            "roofline": roofline,
            "path": path,
            "ceilings": {"mfma_bf16_measured": ceil,
                         "mfma_bf16_device": peak_dev,
                         "mfma_bf16_published_tflops": BF16_PEAK_TFLOPS,
                         "hbm_published_GBs": HBM_PEAK_GBS},
        }
    if args.only == "headline":
        print(json.dumps(result), flush=True)
        return

    # ---------------- c2: B=2 T=4096 H=HV=16, states in and out ----------------
    if want("c2"):
        w2 = inputs.WORKLOADS["c2"]
        d2 = inputs.make(w2, device=dev)
        ws2_bytes = kda.kda_chunk_fwd_workspace_bytes(w2.B, w2.T, w2.H, w2.HV, w2.K, w2.V, w2.B, 0, kda.KDA_BF16)
        ws2 = torch.empty(ws2_bytes, dtype=torch.uint8, device=dev)
        out2 = torch.empty_like(d2["v"])
        fs2 = torch.empty_like(d2["initial_state"])
        call2 = timed_call(d2, out2, ws2, ws2_bytes, w2.B, w2.T, w2.H, w2.HV, w2.K, w2.V, w2.B, final=fs2)
        preheat(lambda: call2(None), leg_pre_s, flushed=True)
        for _ in range(args.warmup):
            flush()
            call2(None)
        whole2, (i2, s2) = timed_flushed(call2, steps, hip, sptr, flush, nev=1)
        st2 = stats(whole2)
        c2_bytes = (2 * w2.B * w2.T * w2.H * w2.K * 2 + 2 * w2.B * w2.T * w2.HV * w2.V * 2
                    + w2.B * w2.T * w2.HV * w2.K * 4 + w2.B * w2.T * w2.HV * 2
                    + 2 * d2["initial_state"].numel() * 4)
        c2_fwd = (sum(i2) + sum(s2)) / steps
        result["c2"] = {"workload": "chunk_kda fwd B=2 T=4096 H=HV=16 K=V=128 bf16, h0 N(0,0.05), final state",
                        "ms_per_step": st2["median"], "steps_ms": st2,
                        "tokens_per_s": w2.B * w2.T / (st2["median"] * 1e-3),
                        "kernels_ms": {"intra": sum(i2) / steps, "scan": sum(s2) / steps},
                        "algorithmic_bytes": c2_bytes, "hbm_floor_us": c2_bytes / HBM_PEAK_GBS / 1e3,
                        "hbm_frac": c2_bytes / (c2_fwd * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del d2, ws2, out2, fs2

    # ---------------- the headline with the fused input options ----------------
    if want("gated"):
        # the gate activation fused into Stage 1: raw bf16 gate input, A_log = log(U[1, 2])
        # per head, dt_bias N(0, 0.5^2)
        gen = torch.Generator().manual_seed(w.seed + 100)
        g_raw = torch.randn(B, T, HV, K, generator=gen).mul(2.0).to(torch.bfloat16).to(dev)
        A_log = torch.rand(HV, generator=gen).add(1.0).log().to(dev)
        dt_bias = torch.randn(HV * K, generator=gen).mul(0.5).to(dev)

        def gcall():
            kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], g_raw, d["beta"], A_log, dt_bias, None,
                                    None, None, out=out, workspace=ws)
        preheat(gcall, leg_pre_s)
        for _ in range(args.warmup):
            gcall()
        gated_ms = back_to_back(gcall, steps, hip, sptr)

        # every input fusion at once: the fused gate as above, q / k L2-normalised in the
        # loads and beta = 2 sigmoid(beta) (the recipe's q, k and beta serve as the raw inputs)
        def fcall():
            kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], g_raw, d["beta"], use_gate_in_kernel=True,
                                 A_log=A_log, dt_bias=dt_bias, use_qk_l2norm_in_kernel=True,
                                 use_beta_sigmoid_in_kernel=True, allow_neg_eigval=True, out=out,
                                 workspace=ws)
        preheat(fcall, leg_pre_s)
        for _ in range(args.warmup):
            fcall()
        fused_ms = back_to_back(fcall, steps, hip, sptr)
        del g_raw, A_log, dt_bias
        result["gated"] = {"workload": "the headline forward with the gate activation fused into Stage 1 (raw bf16 gate input, A_log, dt_bias)",
                           "ms_per_step": gated_ms, "tokens_per_s": tokens / (gated_ms * 1e-3)}
        result["fused_inputs"] = {"workload": "the headline forward with every input fusion: raw bf16 gate + A_log + dt_bias, q/k L2 norm in the loads, beta = 2 sigmoid(beta)",
                                  "ms_per_step": fused_ms, "tokens_per_s": tokens / (fused_ms * 1e-3)}

    # ---------------- backward of the headline forward ----------------
    if want("backward"):
        # do ~ N(0, 1) bf16, no final-state gradient, no initial state (so no dh0); outputs
        # and workspace allocated up front
        bws_bytes = kda.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, 0, kda.KDA_BF16)
        bws = torch.empty(bws_bytes, dtype=torch.uint8, device=dev)
        gen = torch.Generator().manual_seed(w.seed + 200)
        dout = torch.randn(tuple(d["v"].shape), generator=gen).to(torch.bfloat16).to(dev)
        gq, gk, gv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        gg = torch.empty(B, T, HV, K, dtype=torch.float32, device=dev)
        gb = torch.empty_like(d["beta"])

        def bcall():
            rc = lib.kda_chunk_bwd(
                vp(d["q"].data_ptr()), vp(d["k"].data_ptr()), vp(d["v"].data_ptr()),
                vp(d["g"].data_ptr()), vp(d["beta"].data_ptr()), None, None, N,
                vp(dout.data_ptr()), None, vp(gq.data_ptr()), vp(gk.data_ptr()), vp(gv.data_ptr()),
                vp(gg.data_ptr()), vp(gb.data_ptr()), None, B, T, H, HV, K, V, kda.KDA_BF16,
                kda.KDA_BF16, 0.0, 64, vp(bws.data_ptr()), bws_bytes, None, sptr)
            if rc != 0:
                raise RuntimeError(lib.kda_last_error().decode())
        bsteps = max(1, steps // 4)
        preheat(bcall, leg_pre_s)
        for _ in range(2):
            bcall()
        bwd_ms = back_to_back(bcall, bsteps, hip, sptr)
        # a training step's split: the forward keeping the backward's checkpoints
        # (kda_chunk_fwd_train, o written as well), then the backward from them
        # (kda_chunk_bwd_saved, no recompute)
        tws = torch.empty(bws_bytes, dtype=torch.uint8, device=dev)
        o_t = torch.empty_like(d["v"])

        def tcall():
            rc = lib.kda_chunk_fwd_train(
                vp(d["q"].data_ptr()), vp(d["k"].data_ptr()), vp(d["v"].data_ptr()),
                vp(d["g"].data_ptr()), vp(d["beta"].data_ptr()), None, None, N,
                vp(o_t.data_ptr()), None, B, T, H, HV, K, V, kda.KDA_BF16, kda.KDA_BF16, 0.0, 64,
                vp(tws.data_ptr()), bws_bytes, None, sptr)
            if rc != 0:
                raise RuntimeError(lib.kda_last_error().decode())

        def scall():
            rc = lib.kda_chunk_bwd_saved(
                vp(d["q"].data_ptr()), vp(d["k"].data_ptr()), vp(d["v"].data_ptr()),
                vp(d["g"].data_ptr()), vp(d["beta"].data_ptr()), None, None, N,
                vp(dout.data_ptr()), None, vp(gq.data_ptr()), vp(gk.data_ptr()), vp(gv.data_ptr()),
                vp(gg.data_ptr()), vp(gb.data_ptr()), None, B, T, H, HV, K, V, kda.KDA_BF16,
                kda.KDA_BF16, 0.0, 64, vp(tws.data_ptr()), bws_bytes, None, sptr)
            if rc != 0:
                raise RuntimeError(lib.kda_last_error().decode())
        preheat(tcall, leg_pre_s)
        for _ in range(2):
            tcall()
        train_fwd_ms = back_to_back(tcall, bsteps, hip, sptr)
        preheat(scall, leg_pre_s)
        for _ in range(2):
            scall()
        saved_bwd_ms = back_to_back(scall, bsteps, hip, sptr)
        # inputs, do and every gradient once (SURVEY's floor for the backward)
        bwd_bytes = 2 * (q_b + v_b + g_b + beta_b) + o_b
        result["backward"] = {"workload": "kda_chunk_bwd of the headline forward (dq, dk, dv, dg, dbeta; do ~ N(0,1) bf16, no dht)",
                              "ms_per_step": bwd_ms, "tokens_per_s": tokens / (bwd_ms * 1e-3), "steps": bsteps,
                              "algorithmic_bytes": bwd_bytes,
                              "hbm_frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "train_split": {"forward_keeping_checkpoints_ms": train_fwd_ms,
                                              "backward_from_checkpoints_ms": saved_bwd_ms,
                                              "step_ms": train_fwd_ms + saved_bwd_ms}}
        del bws, tws, o_t, dout, gq, gk, gv, gg, gb

    # ---------------- decode: 4096 sequences x 32 heads ----------------
    del ws, out
    if want("decode"):
        dd = inputs.make("dec", device=dev)
        dout = torch.empty_like(dd["v"])
        dstate = torch.empty_like(dd["initial_state"])

        def dcall():
            kda.kda_recurrent_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["initial_state"],
                                  dd["cu_seqlens"], output_final_state=True, out=dout, final_state=dstate)
        for _ in range(2):
            dcall()
        dec_ms = back_to_back(dcall, args.decode_steps, hip, sptr)

        # the same decode with q / k normalisation and beta = sigmoid(beta) fused into the loads
        def dfcall():
            kda.kda_recurrent_fwd_ex(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["initial_state"],
                                     dd["cu_seqlens"], output_final_state=True, out=dout,
                                     final_state=dstate, use_qk_l2norm_in_kernel=True,
                                     use_beta_sigmoid_in_kernel=True)
        for _ in range(2):
            dfcall()
        dec_fused_ms = back_to_back(dfcall, args.decode_steps, hip, sptr)
        # the same decode with the states stored transposed ([V][K] per head)
        h0_vk = dd["initial_state"].transpose(-1, -2).contiguous()
        dstate_vk = torch.empty_like(h0_vk)

        def dvcall():
            kda.kda_recurrent_fwd_ex(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], h0_vk,
                                     dd["cu_seqlens"], output_final_state=True, out=dout,
                                     final_state=dstate_vk, state_layout="vk")
        for _ in range(2):
            dvcall()
        dec_vk_ms = back_to_back(dvcall, args.decode_steps, hip, sptr)
        del h0_vk, dstate_vk
        # what a plain elementwise stream achieves over the same bytes: torch.neg reading the
        # 8.6 GB state tensor and writing 8.6 GB (the practical HBM ceiling the decode is read against)
        for _ in range(2):
            torch.neg(dd["initial_state"], out=dstate)
        stream_ms = back_to_back(lambda: torch.neg(dd["initial_state"], out=dstate), args.decode_steps, hip, sptr)
        stream_gbs = 2 * dd["initial_state"].numel() * 4 / (stream_ms * 1e-3) / 1e9
        dec_bytes = (2 * dd["initial_state"].numel() * 4 + 3 * dd["q"].numel() * 2 + dd["g"].numel() * 4
                     + dd["beta"].numel() * 2 + dout.numel() * 2)
        dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
        del dd, dout, dstate
        result["decode"] = {"workload": "recurrent decode N=4096 HV=32 K=V=128, 1 bf16 token each, fp32 states in+out",
                            "ms": dec_ms, "GB_s": dec_gbs, "hbm_frac": dec_gbs / HBM_PEAK_GBS,
                            "bytes": dec_bytes, "fused_inputs_ms": dec_fused_ms, "state_vk_ms": dec_vk_ms,
                            "stream_ceiling": {"kernel": "torch.neg over the fp32 state tensor (8.59 GB read + 8.59 GB written)",
                                               "ms": stream_ms, "GB_s": stream_gbs,
                                               "decode_frac": dec_gbs / stream_gbs}}
        result.setdefault("ceilings", {})["hbm_stream_GBs"] = stream_gbs

    # ---------------- packed varlen forward ----------------
    if want("varlen"):
        # 64 slots, lengths U[1, 1024] with 4 empty slots (~31k tokens), H=HV=16, K=V=128
        # bf16, fp32 initial and final states
        wv = inputs.WORKLOADS["vl"]
        dv_ = inputs.make(wv, device=dev)
        Bv, Tv = dv_["q"].shape[0], dv_["q"].shape[1]
        Nv = dv_["cu_seqlens"].numel() - 1
        vtokens = int(dv_["cu_seqlens"][-1].item())
        vws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(Bv, Tv, wv.H, wv.HV, wv.K, wv.V, Nv, 1, kda.KDA_BF16),
                          dtype=torch.uint8, device=dev)
        vout = torch.empty_like(dv_["v"])
        vstate = torch.empty_like(dv_["initial_state"])

        def vcall():
            kda.kda_chunk_fwd(dv_["q"], dv_["k"], dv_["v"], dv_["g"], dv_["beta"], dv_["initial_state"],
                              dv_["cu_seqlens"], output_final_state=True, out=vout, final_state=vstate,
                              workspace=vws)
        preheat(vcall, leg_pre_s)
        for _ in range(args.warmup):
            vcall()
        var_ms = back_to_back(vcall, steps, hip, sptr)
        del dv_, vws, vout, vstate
        result["varlen"] = {"workload": f"chunk_kda fwd packed: 64 slots (4 empty), {vtokens} tokens, H=HV=16 K=V=128 bf16, fp32 initial and final states",
                            "ms_per_step": var_ms, "tokens_per_s": vtokens / (var_ms * 1e-3)}

    if not args.no_cpu_baseline and want("headline"):
        import oracle
        host = inputs.make(w)   # same recipe on the host (the oracle's cost does not depend on values)
        threads = oracle.default_threads()
        t0 = time.time()
        oracle.recurrent(host["q"], host["k"], host["v"], host["g"], host["beta"], None, None,
                         None, nthreads=threads)
        cpu_s = time.time() - t0
        result["cpu_baseline"] = {"value": tokens / cpu_s, "unit": "tokens/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": "the full headline workload (8192 tokens x 32 value heads), fp64 token recurrence, one thread per (sequence, head) chain",
                                  "seconds": cpu_s}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
