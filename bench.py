#!/usr/bin/env python3
"""Benchmark of the GGUF block-quantized matmul on one MI355X.

Metric: decode GEMV weight GB/s (share of HBM peak) + prefill GEMM TFLOP/s at
N = 512.

One step = the decode GEMVs of one LLaMA-8B layer in Q4_0 (q_proj 4096x4096,
gate 14336x4096, up 14336x4096, down 4096x14336; x f32 ~ N(0,1)) in three
launches: q_proj and down through qmm_gemv, gate and up together through
qmm_gemv_concat (one launch, one read of x; each output has the bits of a
separate qmm_gemv call).  `value` is the step's weight bytes over its measured
GPU time.  The same layer as four separate launches (each through qmm_gemm
with N = 1, i.e. path selection -> the f32 GEMV) is reported as
"decode_unfused", with gate/up through qmm_gemv_swiglu as "decode_swiglu",
and with int8 activations (the same three launches through qmm_gemv_q8act /
qmm_gemv_concat_q8act, which quantize x to Q8_0 inside the launch) as
"decode_q8act".  The Q6_K LM head (128256 x 4096) is timed alone under
"lm_head": its GEMV and its greedy argmax, each with f32 and with int8
activations.  Weight copies are rotated so
that more than 1 GiB of distinct weights is cycled (more than the 256 MB
last-level cache): every step streams its weights from HBM.  Inputs are
resident in HBM before timing starts.

After the decode loop the same number of steps of the Q4_K prefill GEMM
(14336x4096, N = 512 tokens, f16 matrix cores) is timed and reported under
"prefill_gemm".  The CPU oracle is timed on the host cores on a bounded
sample of the same workloads ("cpu_baseline").

Kernel durations come from HIP events recorded on the stream the kernels run
on (torch's current stream) before and after each timed region, with nothing
in between; a region's launches run back to back, and the per-launch figure
is the region time over its launch count.

Extra: ``--sweep`` prints one JSON line per (workload, N) for every
configuration of the workload table (C1-C5) instead of the main line.
``--spec-verify`` prints one JSON line per N = 1..9 for the Q6_K LM head
(128256 x 4096): N separate GEMVs ("per-row") against one qmm_gemm call
("batched"), the shape of a speculative-decoding verification round, plus
the greedy argmax GEMV at N = 1.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16 matrix cores, TFLOP/s
I8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix cores, TOP/s
ROTATE_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gguf_block_quant_qmm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def load_traffic(name: str, launches_per_unit: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget per leg")
    ap.add_argument("--sweep", action="store_true", help="per-config table instead of the main line")
    ap.add_argument("--spec-verify", action="store_true",
                    help="LM-head verification table (per-row vs batched, N = 1..9) instead of the main line")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline decode step and the prefill GEMM (profiler runs: every GEMV "
                         "launch then belongs to the headline step)")
    ap.add_argument("--oracle-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.oracle_child:
        return oracle_child()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a caller shards rows across GPUs); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gguf_block_quant_qmm_amd as q
    from qmm_inputs import WORKLOADS, make_blob, make_x, rng_for

    q.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)

    if args.sweep:
        return sweep(args, q, np, torch, dev, WORKLOADS, make_blob, make_x, rng_for)
    if args.spec_verify:
        return spec_verify(args, q, torch, dev, WORKLOADS, make_blob, make_x, rng_for)

    # ---------------------------------------------------------------- decode
    layer = [("q_proj", 2, 0), ("gate", 3, 0), ("up", 3, 1), ("down", 4, 0)]
    mats = []
    for name, wid, tid in layer:
        _, dt, M, K, _ = WORKLOADS[wid]
        blob = make_blob(dt, M, K, rng_for(wid, tid))
        mats.append((name, dt, M, K, torch.from_numpy(blob).to(dev)))
    step_bytes = sum(m[4].numel() for m in mats)
    R = -(-ROTATE_BYTES // step_bytes)
    copies = [[m[4]] + [m[4].clone() for _ in range(R - 1)] for m in mats]
    xs = [torch.from_numpy(make_x(1, m[3], rng_for(2, 1001 + i))).to(dev) for i, m in enumerate(mats)]
    ys = [torch.empty((1, m[2]), device=dev) for m in mats]
    stream = torch.cuda.current_stream()

    gate_up_ys = [torch.empty(mats[1][2], device=dev), torch.empty(mats[2][2], device=dev)]
    swiglu_y = torch.empty(mats[1][2], device=dev)

    def step_unfused(c):
        for i, (name, dt, M, K, _) in enumerate(mats):
            q.qmm_gemm(copies[i][c], dt, M, K, 1, xs[i], ys[i], stream=stream)

    def step_fused(c):
        (_, dq, Mq, Kq, _), (_, dg, Mg, Kg, _), _, (_, dd, Md, Kd, _) = mats
        q.qmm_gemv(copies[0][c], dq, Mq, Kq, xs[0], ys[0], stream=stream)
        q.qmm_gemv_concat([copies[1][c], copies[2][c]], dg, [Mg, Mg], Kg, xs[1], gate_up_ys, stream=stream)
        q.qmm_gemv(copies[3][c], dd, Md, Kd, xs[3], ys[3], stream=stream)

    def step_swiglu(c):
        (_, dq, Mq, Kq, _), (_, dg, Mg, Kg, _), _, (_, dd, Md, Kd, _) = mats
        q.qmm_gemv(copies[0][c], dq, Mq, Kq, xs[0], ys[0], stream=stream)
        q.qmm_gemv_swiglu(copies[1][c % R], copies[2][c % R], dg, Mg, Kg, xs[1], swiglu_y, stream=stream)
        q.qmm_gemv(copies[3][c], dd, Md, Kd, xs[3], ys[3], stream=stream)

    # int8 activations (the CPU page's Q8_0 decode path): the same three
    # launches, each quantizing its x to Q8_0 inside the launch
    def step_q8act(c):
        (_, dq, Mq, Kq, _), (_, dg, Mg, Kg, _), _, (_, dd, Md, Kd, _) = mats
        q.qmm_gemv_q8act(copies[0][c], dq, Mq, Kq, xs[0], ys[0], stream=stream)
        q.qmm_gemv_concat_q8act([copies[1][c % R], copies[2][c % R]], dg, [Mg, Mg], Kg, xs[1], gate_up_ys, stream=stream)
        q.qmm_gemv_q8act(copies[3][c], dd, Md, Kd, xs[3], ys[3], stream=stream)

    def time_layer(step):
        """(span ms over args.steps steps, host seconds): one event before the
        first step and one after the last (an event between kernels puts a
        timestamp packet between them, which the decode loop does not have)."""
        for s in range(args.warmup):
            step(s % R)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for s in range(args.steps):
            step((args.warmup + s) % R)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b), time.perf_counter() - t0

    span_ms, wall_dec = time_layer(step_fused)
    span_unf = span_swi = span_q8 = None
    if not args.headline_only:
        span_unf, _ = time_layer(step_unfused)
        span_swi, _ = time_layer(step_swiglu)
        span_q8, _ = time_layer(step_q8act)
    dec_bytes_total = step_bytes * args.steps
    value = dec_bytes_total / (span_ms * 1e-3) / 1e9
    launches = 3
    avg_launch_us = span_ms * 1e3 / (args.steps * launches)
    achieved = value
    traffic = load_traffic("gemv_q4_0_decode_layer")
    # per-matrix time: each shape alone, back to back, between two events
    per_matrix = {}

    def time_calls(fn, nbytes):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for s in range(args.steps):
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.steps
        return {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}

    spans = span_timer(args, np, torch, stream)

    def read_probe_us(copies_list):
        """A plain streaming read of the same bytes over the same rotated
        copies (qmm_read_probe): the launch-size ceiling of a read."""
        pout = torch.empty(q.QMM_READ_PROBE_OUT_FLOATS, device=dev)
        return spans(lambda c: q.qmm_read_probe(copies_list[c % len(copies_list)],
                                                copies_list[c % len(copies_list)].numel(), pout, stream=stream))[0]

    def leg(fn, nbytes, probe_copies=None, flops=None):
        r = time_calls(fn, nbytes)
        med, mn = spans(fn)
        r.update({"us_median": round(med, 3), "us_min": round(mn, 3),
                  "GB/s_median": round(nbytes / (med * 1e-6) / 1e9, 1)})
        if flops:
            r["TFLOP/s_median"] = round(flops / (med * 1e-6) / 1e12, 2)
        if probe_copies is not None:
            p = read_probe_us(probe_copies)
            r["read_probe_us"] = round(p, 3)
            r["frac_of_read_probe"] = round(p / med, 3)
        return r

    for i, (name, dt, M, K, _) in enumerate(mats if not args.headline_only else []):
        per_matrix[name] = leg(lambda c, i=i, dt=dt, M=M, K=K: q.qmm_gemm(copies[i][c % R], dt, M, K, 1, xs[i], ys[i],
                                                                          stream=stream),
                               copies[i][0].numel(), probe_copies=copies[i])
    gu_bytes = copies[1][0].numel() + copies[2][0].numel()
    (_, dg, Mg, Kg, _) = mats[1]
    if not args.headline_only:
        gu_probe = [torch.cat([copies[1][c], copies[2][c]]) for c in range(min(R, 4))]
        per_matrix["gate+up concat"] = leg(
            lambda c: q.qmm_gemv_concat([copies[1][c % R], copies[2][c % R]], dg, [Mg, Mg], Kg, xs[1], gate_up_ys,
                                        stream=stream), gu_bytes, probe_copies=gu_probe)
        del gu_probe
        per_matrix["gate+up swiglu"] = leg(
            lambda c: q.qmm_gemv_swiglu(copies[1][c % R], copies[2][c % R], dg, Mg, Kg, xs[1], swiglu_y, stream=stream),
            gu_bytes)
        for i, (name, dt, M, K, _) in enumerate(mats):
            per_matrix[name + " q8act"] = leg(
                lambda c, i=i, dt=dt, M=M, K=K: q.qmm_gemv_q8act(copies[i][c % R], dt, M, K, xs[i], ys[i], stream=stream),
                copies[i][0].numel())
        per_matrix["gate+up concat q8act"] = leg(
            lambda c: q.qmm_gemv_concat_q8act([copies[1][c % R], copies[2][c % R]], dg, [Mg, Mg], Kg, xs[1], gate_up_ys,
                                              stream=stream), gu_bytes)
        per_matrix["gate+up swiglu q8act"] = leg(
            lambda c: q.qmm_gemv_swiglu_q8act(copies[1][c % R], copies[2][c % R], dg, Mg, Kg, xs[1], swiglu_y,
                                              stream=stream), gu_bytes)

    # the 128256 x 4096 Q6_K LM head (the largest decode GEMV): f32 and
    # int8 activations (quantized inside the launch)
    lm_head = None
    if not args.headline_only:
        _, hdt, HM, HK, _ = WORKLOADS[5]
        hblob = torch.from_numpy(make_blob(hdt, HM, HK, rng_for(5, 0))).to(dev)
        HR = max(2, -(-ROTATE_BYTES // hblob.numel()))
        hcopies = [hblob] + [hblob.clone() for _ in range(HR - 1)]
        hx = torch.from_numpy(make_x(1, HK, rng_for(5, 1001))).to(dev).reshape(-1)
        hy = torch.empty(HM, device=dev)
        for s in range(args.warmup):
            q.qmm_gemv(hcopies[s % HR], hdt, HM, HK, hx, hy, stream=stream)
        lm_head = {"workload": "Q6_K 128256x4096, N=1, x f32 ~ N(0,1)", "weight_bytes": hblob.numel(),
                   "rotation_copies": HR}
        hwork = torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8, device=dev)
        hidx = torch.empty(1, dtype=torch.int64, device=dev)
        for key, fn in (("f32", lambda c: q.qmm_gemv(hcopies[c % HR], hdt, HM, HK, hx, hy, stream=stream)),
                        ("q8act", lambda c: q.qmm_gemv_q8act(hcopies[c % HR], hdt, HM, HK, hx, hy, stream=stream)),
                        ("argmax_f32", lambda c: q.qmm_gemv_argmax(hcopies[c % HR], hdt, HM, HK, hx, hwork, hidx,
                                                                   stream=stream)),
                        ("argmax_f32_noalloc", lambda c: q.qmm_gemv_argmax_noalloc(hcopies[c % HR], hdt, HM, HK, hx,
                                                                                   hidx, stream=stream)),
                        ("argmax_q8act", lambda c: q.qmm_gemv_argmax_q8act(hcopies[c % HR], hdt, HM, HK, hx, hwork,
                                                                           hidx, stream=stream))):
            r = leg(fn, hblob.numel(), probe_copies=hcopies if key == "f32" else None)
            r["hbm_frac"] = round(r["GB/s"] / HBM_PEAK_GBS, 4)
            r["hbm_frac_median"] = round(r["GB/s_median"] / HBM_PEAK_GBS, 4)
            lm_head[key] = r
        lm_head["argmax_minus_gemv_us_median"] = round(lm_head["argmax_f32"]["us_median"] - lm_head["f32"]["us_median"],
                                                       3)
        del hcopies, hblob
        torch.cuda.empty_cache()

    # C1 (Q8_0 1024x1024 GEMV) and C4a (Q4_K 14336x4096 GEMM at N = 32): the
    # other single-launch configurations, each rotated over >= 1 GiB of weight
    # copies and also warm (one copy, its bytes served from the caches)
    small = {}
    if not args.headline_only:
        for key, wid, N in (("C1 q8_0 gemv 1024x1024", 1, 1), ("C4a q4_k gemm 14336x4096 N=32", 6, 32)):
            _, sdt, SM, SK, _ = WORKLOADS[wid]
            sblob = torch.from_numpy(make_blob(sdt, SM, SK, rng_for(wid, 0))).to(dev)
            SR = max(2, -(-ROTATE_BYTES // sblob.numel()))
            scop = [sblob] + [sblob.clone() for _ in range(SR - 1)]
            SX = torch.from_numpy(make_x(N, SK, rng_for(wid, 1000 + N))).to(dev)
            SY = torch.empty((N, SM), device=dev)
            fl = 2.0 * SM * N * SK
            for s_ in range(args.warmup):
                q.qmm_gemm(scop[s_ % SR], sdt, SM, SK, N, SX, SY, stream=stream)
            r = leg(lambda c: q.qmm_gemm(scop[c % SR], sdt, SM, SK, N, SX, SY, stream=stream), sblob.numel(),
                    probe_copies=scop, flops=fl)
            wm, wn = spans(lambda c: q.qmm_gemm(sblob, sdt, SM, SK, N, SX, SY, stream=stream))
            r.update({"kernel_id": q.gemm_kernel(sdt, SM, SK, N), "weight_bytes": sblob.numel(),
                      "hbm_frac_median": round(r["GB/s_median"] / HBM_PEAK_GBS, 4),
                      "warm_us_median": round(wm, 3), "warm_us_min": round(wn, 3),
                      "warm_note": "one weight copy, re-read from the caches: not an HBM figure"})
            small[key] = r
            del scop, sblob
        torch.cuda.empty_cache()

    # the decode step again, as 5 spans (per-step median and min), and the
    # other forms of the layer the same way
    dec_med, dec_min = spans(lambda c: step_fused(c % R))
    var_med = {}
    if not args.headline_only:
        for key, fn in (("decode_unfused", step_unfused), ("decode_swiglu", step_swiglu), ("decode_q8act", step_q8act)):
            med, mn = spans(lambda c, fn=fn: fn(c % R))
            var_med[key] = {"us_per_step_median_of_5_spans": round(med, 3), "us_per_step_min_of_5_spans": round(mn, 3),
                            "GB/s_median": round(step_bytes / (med * 1e-6) / 1e9, 1)}

    def layer_rate(span):
        if span is None:
            return None
        return {"GB/s": round(dec_bytes_total / (span * 1e-3) / 1e9, 2), "ms_per_step": round(span / args.steps, 5)}

    # --------------------------------------------------------------- prefill
    _, pdt, PM, PK, _ = WORKLOADS[6]
    PN = 512
    pblob = torch.from_numpy(make_blob(pdt, PM, PK, rng_for(6, 0))).to(dev)
    PR = -(-ROTATE_BYTES // pblob.numel())
    pcopies = [pblob] + [pblob.clone() for _ in range(PR - 1)]
    PX = torch.from_numpy(make_x(PN, PK, rng_for(6, 1000 + PN))).to(dev)
    PY = torch.empty((PN, PM), device=dev)
    for s in range(args.warmup):
        q.qmm_gemm(pcopies[s % PR], pdt, PM, PK, PN, PX, PY, stream=stream)
    torch.cuda.synchronize()
    pa, pb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    pa.record(stream)
    for s in range(args.steps):
        q.qmm_gemm(pcopies[(args.warmup + s) % PR], pdt, PM, PK, PN, PX, PY, stream=stream)
    pb.record(stream)
    torch.cuda.synchronize()
    wall_pre = time.perf_counter() - t0
    pre_ms = pa.elapsed_time(pb)
    flops = 2.0 * PM * PN * PK
    tflops = flops * args.steps / (pre_ms * 1e-3) / 1e12
    pre_med, pre_min = spans(lambda c: q.qmm_gemm(pcopies[c % PR], pdt, PM, PK, PN, PX, PY, stream=stream))
    ptraffic = load_traffic("gemm_q4_k_n512")
    # The same GEMM with int8 activations: X quantized to Q8_0 once (its codes
    # resident like X), then qmm_gemm_q8act, which takes the int8 matrix cores
    # at this size; and the quantizer plus the matmul as one step.
    pre_q8 = None
    if not args.headline_only:
        psc = torch.empty((PN, PK // 32), device=dev)
        pqq = torch.empty((PN, PK), dtype=torch.int8, device=dev)
        q.qmm_quantize_q8_0(PX, PN, PK, psc, pqq, stream=stream)
        q8_med, q8_min = spans(lambda c: q.qmm_gemm_q8act(pcopies[c % PR], pdt, PM, PK, PN, psc, pqq, PY,
                                                          stream=stream))

        def q8_step(c):
            q.qmm_quantize_q8_0(PX, PN, PK, psc, pqq, stream=stream)
            q.qmm_gemm_q8act(pcopies[c % PR], pdt, PM, PK, PN, psc, pqq, PY, stream=stream)
        q8s_med, _ = spans(q8_step)
        pre_q8 = {"path": "int8 matrix cores" if q.q8act_kernel(pdt, PM, PK, PN) == 1 else "token groups",
                  "us_median_of_5_spans": round(q8_med, 3), "us_min_of_5_spans": round(q8_min, 3),
                  "tops_median": round(flops / (q8_med * 1e-6) / 1e12, 2),
                  "frac_of_int8_mfma_peak": round(flops / (q8_med * 1e-6) / 1e12 / I8_MFMA_PEAK_TOPS, 4),
                  "quantize_plus_gemm_us_median": round(q8s_med, 3),
                  "note": "qmm_gemm_q8act on the activations quantized to Q8_0 (integer block sums, each scaled "
                          "once in f32: bounded by that scaling, not by the matrix rate)"}

    # Q6_K and Q8_0 at the prefill shape: the GEMM on the GGUF bytes and on
    # the repacked copy (qmm_repack, built once, timed alone too)
    pre_rp = None
    if not args.headline_only:
        pre_rp = {}
        for rdt, rname in ((q.QMM_Q6_K, "q6_k"), (q.QMM_Q8_0, "q8_0")):
            rblob = torch.from_numpy(make_blob(rdt, PM, PK, rng_for(6, rdt))).to(dev)
            RR = -(-ROTATE_BYTES // rblob.numel())
            rcopies = [rblob] + [rblob.clone() for _ in range(RR - 1)]
            nbr = q.repack_bytes(rdt, PM, PK)
            rpacks = [torch.empty(nbr, dtype=torch.uint8, device=dev) for _ in range(-(-ROTATE_BYTES // nbr))]
            for c, pk in enumerate(rpacks):
                q.qmm_repack(rcopies[c % RR], rdt, PM, PK, pk, stream=stream)
            g_med, g_min = spans(lambda c: q.qmm_gemm(rcopies[c % RR], rdt, PM, PK, PN, PX, PY, stream=stream))
            r_med, r_min = spans(lambda c: q.qmm_gemm_repacked(rpacks[c % len(rpacks)], rdt, PM, PK, PN, PX, PY,
                                                               stream=stream))
            rp_med, _ = spans(lambda c: q.qmm_repack(rcopies[c % RR], rdt, PM, PK, rpacks[c % len(rpacks)],
                                                     stream=stream))
            pre_rp[rname] = {"workload": f"{rname.upper()} {PM}x{PK}, N={PN}, X f32 ~ N(0,1)",
                             "gguf_us_median": round(g_med, 3), "gguf_us_min": round(g_min, 3),
                             "gguf_tflops_median": round(flops / (g_med * 1e-6) / 1e12, 2),
                             "repacked_us_median": round(r_med, 3), "repacked_us_min": round(r_min, 3),
                             "repacked_tflops_median": round(flops / (r_med * 1e-6) / 1e12, 2),
                             "repack_once_us_median": round(rp_med, 3),
                             "bytes": {"gguf": rblob.numel(), "repacked": nbr}}
            del rcopies, rpacks, rblob
        pre_rp["note"] = ("qmm_gemm_repacked gives qmm_gemm's bits at these shapes (same f16 weights and "
                          "matrix-core steps)")

    out = {
        "metric": "decode GEMV weight GB/s (% HBM peak) + prefill GEMM TFLOP/s at N=512",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((wall_dec + wall_pre) * 1e3 / args.steps, 4),
        "ms_per_step_note": "host wall clock of the two timed loops (K decode-layer steps, then K N=512 GEMM "
                            "calls) per step; the decode step alone is config.decode_ms_per_step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama8b decode layer, Q4_0 GEMVs q_proj 4096x4096 + gate/up 14336x4096 + down "
                        "4096x14336, N=1, x f32 ~ N(0,1), seed 0; gate and up in one qmm_gemv_concat launch",
            "weight_bytes_per_step": step_bytes,
            "rotation_copies": R,
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
            "decode_ms_per_step": round(span_ms / args.steps, 5),
            "decode_step_us_median_of_5_spans": round(dec_med, 3),
            "decode_step_us_min_of_5_spans": round(dec_min, 3),
            "decode_GBps_median_of_5_spans": round(step_bytes / (dec_med * 1e-6) / 1e9, 1),
            "decode_unfused": {"launches": 4, **(layer_rate(span_unf) or {}), **var_med.get("decode_unfused", {})},
            "decode_swiglu": {"launches": 3, **(layer_rate(span_swi) or {}), **var_med.get("decode_swiglu", {}),
                              "note": "gate/up through qmm_gemv_swiglu (outputs silu(g)*u instead of g and u)"},
            "decode_q8act": {"launches": 3, **(layer_rate(span_q8) or {}), **var_med.get("decode_q8act", {}),
                             "note": "int8 activations: qmm_gemv_q8act (q_proj, down) and qmm_gemv_concat_q8act "
                                     "(gate+up), each quantizing x to Q8_0 inside the launch; integer block dots, "
                                     "different numbers from the f32 path"},
            "timing": "HIP events on the launch stream before the first and after the last timed step; per-launch = "
                      "span / launches; the *_median/*_min fields: 5 further spans, each after a GPU-side spin "
                      "that keeps the queue ahead of the host (so small launches are not timed by the host's "
                      "enqueue rate)",
            "per_matrix": per_matrix,
            "lm_head": lm_head,
            "other_configs": small,
            "gpu": props.name,
            "cus": props.multi_processor_count,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "qmm::gemv_kernel<2,...> (Q4_0): q_proj, gate+up concatenated, down -- the three "
                      "decode-layer launches together",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_us, 3),
            "algorithmic_bytes_per_launch": step_bytes / launches,
        },
        "prefill_gemm": {
            "workload": "Q4_K 14336x4096, N=512 tokens, X f32 ~ N(0,1), f16 matrix cores, f32 accumulate",
            "tflops": round(tflops, 2),
            "ms_per_call": round(pre_ms / args.steps, 5),
            "us_median_of_5_spans": round(pre_med, 3),
            "us_min_of_5_spans": round(pre_min, 3),
            "tflops_median_of_5_spans": round(flops / (pre_med * 1e-6) / 1e12, 2),
            "rotation_copies": PR,
            "q8act": pre_q8,
            "repacked": pre_rp,
            "roofline": {
                "bound": "mfma",
                "kernel": "qmm::gemm_wb_kernel<12,32,128,2,8,4,2> (Q4_K)",
                "achieved": round(tflops, 2),
                "peak": F16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
                "traffic": ptraffic,
                "avg_launch_us": round(pre_ms * 1e3 / args.steps, 3),
                "algorithmic_flops_per_launch": flops,
            },
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, np, mats, WORKLOADS, make_blob, make_x, rng_for, step_bytes)
    print(json.dumps(out), flush=True)


def cpu_model() -> dict:
    """Host CPU description from /proc/cpuinfo (model, sockets, cores, threads)."""
    info = {"threads": os.cpu_count()}
    try:
        txt = open("/proc/cpuinfo").read()
        blocks = [b for b in txt.split("\n\n") if b.strip()]
        kv = [dict((l.split(":", 1)[0].strip(), l.split(":", 1)[1].strip()) for l in b.splitlines() if ":" in l)
              for b in blocks]
        info["model"] = kv[0].get("model name", "?")
        info["sockets"] = len({d.get("physical id") for d in kv})
        info["cores"] = len({(d.get("physical id"), d.get("core id")) for d in kv})
    except OSError:
        pass
    return info


# single-thread oracle samples of C1-C3: (label, workload id, row stride)
ORACLE_1T = (("C1 q8_0 1024x1024", 1, 1), ("C2a q4_0 4096x4096", 2, 1), ("C2b q4_0 14336x4096", 3, 1),
             ("C2c q4_0 4096x14336", 4, 1), ("C3 q6_k 128256x4096", 5, 4))


def oracle_child():
    """Runs in a child process with OMP_NUM_THREADS=1 (no GPU use): the oracle
    on C1-C3, whole matrices or every n-th row, weight GB/s per config."""
    import numpy as np
    import oracle
    from qmm_inputs import WORKLOADS, make_blob, make_x, rng_for
    out = {"threads": oracle.num_threads()}
    for label, wid, stride in ORACLE_1T:
        _, dt, M, K, _ = WORKLOADS[wid]
        blob = make_blob(dt, M, K, rng_for(wid, 0))
        x = make_x(1, K, rng_for(wid, 1001))
        rows = np.arange(0, M, stride)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.matmul(dt, blob, M, K, x, rows=rows if stride > 1 else None)
            ts.append(time.perf_counter() - t0)
        dt_s = float(np.median(ts))
        nbytes = blob.size * len(rows) / M
        out[label] = {"GB/s": round(nbytes / dt_s / 1e9, 4), "s_median_of_3": round(dt_s, 4),
                      "sample": "all rows" if stride == 1 else f"every {stride}th row ({len(rows)} rows)"}
    print(json.dumps(out), flush=True)


def cpu_baseline(args, np, mats, WORKLOADS, make_blob, make_x, rng_for, step_bytes):
    """The oracle, as it stands, on the host cores: whole decode layers
    (same shapes and seeds) repeated for about --cpu-seconds, plus a row
    sample of the N=512 prefill GEMM."""
    import oracle
    host = []
    for i, (name, dt, M, K, blob_d) in enumerate(mats):
        host.append((dt, M, K, blob_d.cpu().numpy(), make_x(1, K, rng_for(2, 1001 + i))))
    passes, t0 = 0, time.perf_counter()
    while True:
        for dt, M, K, blob, x in host:
            oracle.matmul(dt, blob, M, K, x)
        passes += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt_dec = time.perf_counter() - t0
    _, pdt, PM, PK, _ = WORKLOADS[6]
    pblob = make_blob(pdt, PM, PK, rng_for(6, 0))
    PX = make_x(512, PK, rng_for(6, 1512))
    rows, t0 = 0, time.perf_counter()
    while True:
        oracle.matmul(pdt, pblob, PM, PK, PX, rows=np.arange(rows, rows + 64) % PM)
        rows += 64
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt_pre = time.perf_counter() - t0
    # every config on all cores (C1, C3 head sampled), and C1-C3 on one thread
    all_cores = {}
    for label, wid, stride in ORACLE_1T:
        _, dt, M, K, _ = WORKLOADS[wid]
        blob = make_blob(dt, M, K, rng_for(wid, 0))
        x = make_x(1, K, rng_for(wid, 1001))
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.matmul(dt, blob, M, K, x)
            ts.append(time.perf_counter() - t0)
        dts = float(np.median(ts))
        all_cores[label] = {"GB/s": round(blob.size / dts / 1e9, 4), "s_median_of_3": round(dts, 4)}
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    child = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-child"], env=env,
                           capture_output=True, text=True, timeout=600)
    one_thread = json.loads(child.stdout.strip().splitlines()[-1]) if child.returncode == 0 else \
        {"error": child.stderr[-500:]}
    return {
        "value": round(step_bytes * passes / dt_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{passes} whole decode layers (4 Q4_0 GEMVs, same shapes and seeds) in {dt_dec:.1f} s",
        "prefill_gemm_tflops": round(2.0 * rows * 512 * PK / dt_pre / 1e12, 6),
        "prefill_sample": f"{rows} output rows (64 at a time, cycling over the {PM}) x 512 tokens of the "
                          f"Q4_K GEMM in {dt_pre:.1f} s",
        "all_cores_per_config": all_cores,
        "one_thread_per_config": one_thread,
        "cpu": cpu_model(),
    }


def span_timer(args, np, torch, stream):
    """spans(fn) -> per-call time (median, min) in us over 5 separate spans of
    max(10, steps / 5) calls each, every span between its own two events.

    A GPU-side spin before each span keeps the queue ahead of the host: the
    binding enqueues a call in ~6 us, about the duration of the smallest
    launches, so without it a span of small kernels would time the host.  The
    spin is calibrated to last about 1.5 ms and is outside the span."""
    t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1 << 20)
    t_a.record(stream)
    torch.cuda._sleep(1 << 20)
    t_b.record(stream)
    torch.cuda.synchronize()
    sleep_cycles = int((1 << 20) * 1.5 / max(t_a.elapsed_time(t_b), 1e-3))

    def spans(fn, n_spans=5, per_span=None):
        per_span = per_span or max(10, args.steps // n_spans)
        out, c = [], 0
        for _ in range(n_spans):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(sleep_cycles)
            a.record(stream)
            for _ in range(per_span):
                fn(c)
                c += 1
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1e3 / per_span)
        return float(np.median(out)), float(np.min(out))
    return spans


def sweep(args, q, np, torch, dev, WORKLOADS, make_blob, make_x, rng_for):
    """One JSON line per (workload, N): qmm_gemm's per-call time, median and
    min of 5 spans over rotated weight copies, with the path and kernel the
    library chose."""
    stream = torch.cuda.current_stream()
    spans = span_timer(args, np, torch, stream)
    names = {2: "Q4_0", 3: "Q4_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K"}
    for wid in sorted(WORKLOADS):
        label, dt, M, K, ns = WORKLOADS[wid]
        blob = torch.from_numpy(make_blob(dt, M, K, rng_for(wid, 0))).to(dev)
        R = max(1, -(-ROTATE_BYTES // blob.numel()))
        copies = [blob] + [blob.clone() for _ in range(R - 1)]
        # Q6_K: the repacked copy (qmm_repack) timed beside the GGUF bytes
        packs = []
        if q.repack_bytes(dt, M, K):
            nbr = q.repack_bytes(dt, M, K)
            for c in range(max(1, -(-ROTATE_BYTES // nbr))):
                packs.append(torch.empty(nbr, dtype=torch.uint8, device=dev))
                q.qmm_repack(copies[c % R], dt, M, K, packs[-1], stream=stream)
        for N in ns:
            X = torch.from_numpy(make_x(N, K, rng_for(wid, 1000 + N))).to(dev)
            Y = torch.empty((N, M), device=dev)
            for s in range(args.warmup):
                q.qmm_gemm(copies[s % R], dt, M, K, N, X, Y, stream=stream)
            med, mn = spans(lambda c: q.qmm_gemm(copies[c % R], dt, M, K, N, X, Y, stream=stream))
            wb = blob.numel()
            rec = {"workload": label, "N": N, "dtype": names[dt], "M": M, "K": K,
                   "path": "f16-mfma" if q.gemm_path(dt, M, K, N) else "f32-gemv",
                   "kernel_id": q.gemm_kernel(dt, M, K, N),
                   "us_median": round(med, 3), "us_min": round(mn, 3),
                   "weight_GBps": round(wb / (med * 1e-6) / 1e9, 1),
                   "hbm_frac": round(wb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "TFLOPs": round(2.0 * M * N * K / (med * 1e-6) / 1e12, 2)}
            if packs:
                rmed, rmn = spans(lambda c: q.qmm_gemm_repacked(packs[c % len(packs)], dt, M, K, N, X, Y,
                                                                stream=stream))
                rec["repacked"] = {"us_median": round(rmed, 3), "us_min": round(rmn, 3),
                                   "kernel_id": q.gemm_repacked_kernel(dt, M, K, N),
                                   "TFLOPs": round(2.0 * M * N * K / (rmed * 1e-6) / 1e12, 2)}
            print(json.dumps(rec), flush=True)
        del copies, blob, packs
        torch.cuda.empty_cache()


def spec_verify(args, q, torch, dev, WORKLOADS, make_blob, make_x, rng_for):
    """Verification of N drafted positions on the LM head: per-row GEMVs vs one batched call."""
    stream = torch.cuda.current_stream()
    label, dt, M, K, _ = WORKLOADS[5]
    blob = torch.from_numpy(make_blob(dt, M, K, rng_for(5, 0))).to(dev)
    R = max(2, -(-ROTATE_BYTES // blob.numel()))
    copies = [blob] + [blob.clone() for _ in range(R - 1)]

    def timed(fn):
        for s in range(args.warmup):
            fn(s % R)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for s in range(args.steps):
            fn(s % R)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / args.steps

    work = torch.empty(q.QMM_ARGMAX_WORK_BYTES, dtype=torch.uint8, device=dev)
    idx = torch.empty(1, dtype=torch.int64, device=dev)
    for N in range(1, 10):
        X = torch.from_numpy(make_x(N, K, rng_for(5, 2000 + N))).to(dev)
        Y = torch.empty((N, M), device=dev)
        per_row = timed(lambda c: [q.qmm_gemv(copies[c], dt, M, K, X[n], Y[n], stream=stream) for n in range(N)])
        batched = timed(lambda c: q.qmm_gemm(copies[c], dt, M, K, N, X, Y, stream=stream))
        # int8 activations: the N positions quantized (one launch) and one
        # qmm_gemm_q8act call reading the head once per 4 positions
        sc = torch.empty((N, K // 32), device=dev)
        qq = torch.empty((N, K), dtype=torch.int8, device=dev)

        def q8(c):
            q.qmm_quantize_q8_0(X, N, K, sc, qq, stream=stream)
            q.qmm_gemm_q8act(copies[c], dt, M, K, N, sc, qq, Y, stream=stream)
        int8 = timed(q8)
        rec = {"workload": f"{label}, verify {N} positions", "N": N, "M": M, "K": K, "dtype": "Q6_K",
               "per_row_us": round(per_row, 2), "batched_us": round(batched, 2),
               "batched_path": "f16-mfma" if q.gemm_path(dt, M, K, N) else "f32 (bits of the GEMV)",
               "batched_weight_GBps": round(blob.numel() / (batched * 1e-6) / 1e9, 1),
               "int8_quantize_plus_q8act_us": round(int8, 2)}
        if N == 1:
            rec["argmax_us"] = round(timed(lambda c: q.qmm_gemv_argmax(copies[c], dt, M, K, X[0], work, idx,
                                                                        stream=stream)), 2)
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
