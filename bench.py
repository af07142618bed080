#!/usr/bin/env python3
"""Benchmark: Gated DeltaNet chunked forward + backward on one MI355X.

One step = the whole hot path over one batch: the forward over the N
sequence chunks in order (boundary state handed S_out -> S_in) and the
backward over the chunks in reverse (dS_in -> dS_out), every kernel in the
HIP library through its C ABI.  Inputs are seeded synthetic tensors, resident
in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line (see README of the JSON fields in the design doc).
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

METRIC = "tokens/sec, gated-delta-rule fwd+bwd (H=16,dk=dv=128); MFMA util %"
DEFAULT_WORKLOAD = "gdn_bf16_H16_T8192_d128"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop/byte


def kernel_work(name: str, dk: int, dv: int, es: int, C: int = 64):
    """Algorithmic (bytes, flops) of one kernel per 64-token block and head
    (element size es; fp32 for gates and states kept in fp32).  Bytes count
    every tensor the kernel reads or writes once; flops count its dense
    products as executed (2 m n k each).  The definitions are listed per
    kernel in the design doc."""
    Ck, Cv, kv, CC, f4 = C * dk, C * dv, dk * dv, C * C, 4
    W = {
        # Gated DeltaNet (dk == dv)
        "gdn_prep": (2 * Ck * es + 2 * C * es + C * f4 + 3 * Ck * es,
                     2 * CC * dk + 2 * (2 * CC * dk) + C ** 3 // 3),
        "gdn_scan_fwd": (C * f4 + 3 * Ck * es + kv * es + Cv * es, 2 * (2 * C * kv)),
        "gdn_out": (2 * Ck * es + C * f4 + kv * es + Cv * es + Cv * es,
                    2 * CC * dk + 2 * C * kv + 2 * CC * dv),
        "gdn_scan_bwd": (C * f4 + 2 * Ck * es + kv * f4 + Cv * es + kv * es + Cv * es, 2 * (2 * C * kv)),
        # reads T^T and the decayed Gram tiles that the backward's prep wrote
        "gdn_bwd_intra": (4 * Ck * es + 2 * C * es + C * f4 + 2 * kv * es + 2 * Cv * es + 3 * Ck * es + 2 * C * es
                          + CC * es + CC * f4,
                          3 * (2 * C * kv) + 11 * (2 * CC * dk) + 2 * (2 * C ** 3)),
    }
    # GLA (per-channel gate, gk = dk gate values per token) and its scalar-gate
    # Mamba-2 member on the same kernels (gk = 1)
    for pre, gk in (("gla", dk), ("m2", 1)):
        Cg = C * gk
        W[pre + "_prep"] = (Ck * es + Cg * es + dk * f4 + Ck * es, 0)
        W[pre + "_prep_bwd"] = (2 * Ck * es + Cg * es + dk * f4 + 3 * Ck * es, 0)
        W[pre + "_scan_fwd"] = (Ck * es + Cv * es + dk * f4 + kv * es, 2 * C * kv)
        W[pre + "_out"] = (2 * Ck * es + Cv * es + Cg * es + kv * es + Cv * es,
                           2 * CC * dk + 2 * C * kv + 2 * CC * dv)
        W[pre + "_scan_bwd"] = (2 * Ck * es + Cv * es + dk * f4 + kv * es + Cv * es, 2 * (2 * C * kv))
        W[pre + "_bwd_intra"] = (2 * Ck * es + 2 * Cv * es + Cg * es + 2 * kv * es + Cv * es + 2 * Ck * es
                                 + Cv * es + Cg * es,
                                 2 * (2 * CC * dv) + 2 * CC * dk + 2 * (2 * C * kv) + 2 * (2 * CC * dk) + 2 * CC * dv)
        W[pre + "_scan_fwd_rec"] = W[pre + "_scan_fwd"]
    W["gdn_scan_fwd_rec"] = W["gdn_scan_fwd"]
    # the backward's prep also reads Q and dO and writes the reverse scan's
    # operands W^T, Kh, dvloc^T, R (fp32) and T^T, K K^T * G for the block
    # adjoints; products P = Q K^T, P^T dO, Z = Gam Q - P W, R = Z^T dO
    W["gdn_prep_bwd"] = (W["gdn_prep"][0] + 2 * Ck * es + 3 * Ck * es + kv * f4 + CC * es + CC * f4,
                         W["gdn_prep"][1] + 2 * CC * dk + 2 * CC * dv + 2 * CC * dk + 2 * C * kv)
    # KDA (per-channel gate, dk == dv): the Gated DeltaNet data flow with
    # per-channel decays (exp(b_C) per channel in place of the per-token
    # gate), U token-major, and the WY adjoints dM, dX handed to the GLA intra
    # kernel in fp32
    W["kda_prep"] = (2 * Ck * es + Cv * es + C * es + dk * f4 + 2 * Ck * es + Cv * es,
                     2 * CC * dk + 2 * CC * dk + 2 * CC * dv + C ** 3 // 3)
    W["kda_prep2"] = (5 * Ck * es + 3 * Ck * es + kv * f4, 2 * CC * dk + 2 * CC * dv + 2 * (2 * C * kv))
    W["kda_scan_fwd"] = (dk * f4 + 3 * Ck * es + kv * es + Cv * es, 2 * (2 * C * kv))
    W["kda_out"] = W["gla_out"]
    kda_scan_bwd = (dk * f4 + 2 * Ck * es + kv * f4 + Cv * es + kv * es + Cv * es, 2 * (2 * C * kv))
    W["kda_scan_pair"] = tuple(x + y for x, y in zip(W["kda_scan_fwd"], kda_scan_bwd))
    # the backward's prep also writes T^T, M and K e^b for the WY adjoint kernel
    W["kda_prep_bwd"] = (W["kda_prep"][0] + CC * es + CC * f4 + Ck * es, W["kda_prep"][1])
    W["kda_bwd_wy"] = (Ck * es + CC * es + CC * f4 + Cv * es + C * es + kv * es + Cv * es
                       + Cv * es + C * es + CC * f4 + Ck * f4,
                       2 * C * kv + 2 * CC * dv + 2 * CC * dk + 2 * (2 * C ** 3) + 2 * CC * dv + 2 * CC * dk)
    W["kda_bwd_intra"] = (5 * Ck * es + 2 * kv * es + CC * f4 + Ck * f4 + C * es + 3 * Ck * es,
                          2 * (2 * CC * dv) + 2 * (2 * C * kv) + 4 * (2 * CC * dk))
    # one launch running the forward recompute and the reverse scan side by side
    W["gdn_scan_pair"] = tuple(x + y for x, y in zip(W["gdn_scan_fwd"], W["gdn_scan_bwd"]))
    return W.get(name)


def shortconv_work(name: str, B: int, Tc: int, C: int, W: int, es: int, P: int):
    """Algorithmic (bytes, flops) of one short-convolution launch over a
    sequence chunk of Tc tokens: every token row read or written once, the
    carried rows, the fp32 weights, and (backward) the partial weight-gradient
    table of P rows.  Flops are the taps' multiply-adds (vector ALU work)."""
    rows, st, par = B * Tc * C * es, B * (W - 1) * C * es, C * (W + 1) * 4
    if name == "shortconv_fwd":
        return 2 * rows + 2 * st + par, 2 * W * B * Tc * C
    if name == "shortconv_bwd":
        return 3 * rows + 2 * st + par + P * par, 4 * W * B * Tc * C
    if name == "shortconv_reduce":
        return P * par + par, P * par // 4
    return None


def _conv_tile_groups(B: int, T: int, C: int, tt: int = 4, nv: int = 4, tg: int = 4) -> int:
    """Work-groups per batch along the tokens of the short-convolution
    backward grid: the partial rows it writes (the rule of the library's
    launcher: about 8 waves per CU, each thread a contiguous run of tiles,
    tg token groups per work-group summed in LDS)."""
    ntiles = (T + tt - 1) // tt
    want = max(1, min(ntiles, (256 * 8 * 64) // max(1, B * (C // nv))))
    per = -(-ntiles // want)
    groups = -(-ntiles // per)
    return -(-groups // tg)


def source_hash() -> str:
    """Hash of the HIP sources (ties stored counter data to a kernel build)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_linear_recurrence_chunk_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".h")):
            with open(os.path.join(csrc, fn), "rb") as f:
                h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    e = d.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(cfg: dict, x: dict, budget_chunks: int):
    """The fp64 oracle (as it stands) on the host cores over a bounded sample:
    the first `budget_chunks` sequence chunks of the workload, forward then
    backward with boundary-state hand-off."""
    import numpy as np
    from oracle import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    T, N = cfg["T"], cfg["N"]
    L = T // N
    n = max(1, min(budget_chunks, N))
    Ts = L * n
    per_token = ("x", "dy") if cfg["kind"] == "shortconv" else ("q", "k", "v", "g", "beta", "dO")
    sl = {k: (np.ascontiguousarray(v[:, :Ts]).astype(np.float64) if k in per_token else v.astype(np.float64))
          for k, v in x.items()}

    def once():
        if cfg["kind"] == "shortconv":
            st = sl["state_in"]
            states = []
            for i in range(n):
                states.append(st)
                _, st = oracle.conv_fwd(sl["x"][:, i * L:(i + 1) * L], sl["w"], sl["bias"], st, cfg["act"])
            ds = None
            for i in reversed(range(n)):
                ds = oracle.conv_bwd(sl["x"][:, i * L:(i + 1) * L], sl["w"], sl["bias"], states[i],
                                     sl["dy"][:, i * L:(i + 1) * L], ds, cfg["act"])["dstate_in"]
        elif cfg["kind"] == "gdn":
            oracle.gdn_chunked(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["S_in"], sl["dO"], None, n)
        elif cfg["kind"] == "kda":
            oracle.kda_chunked(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["S_in"], sl["dO"], None, n)
        elif cfg["kind"] == "gla":
            oracle.gla_chunked(sl["q"], sl["k"], sl["v"], sl["g"], sl["S_in"], sl["dO"], None, n)
        else:
            oracle.mamba2_chunked(sl["q"], sl["k"], sl["v"], sl["g"], sl["S_in"], sl["dO"], None, n)
    t0 = time.perf_counter()
    once()
    reps, dt = 1, time.perf_counter() - t0
    # repeat a cheap sample until about 10 s of oracle work has been timed
    while dt < 10.0 and reps < 40:
        once()
        reps += 1
        dt = time.perf_counter() - t0
    return {"value": cfg["B"] * Ts * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{'all' if n == N else f'first {n} of'} {N} sequence chunks ({cfg['B']}x{Ts} tokens, "
                      + (f"all {cfg['C']} channels" if cfg["kind"] == "shortconv" else f"all {cfg['H']} heads")
                      + f"), fp64 fwd+bwd, {reps} run(s), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-chunks", type=int, default=64, help="sequence chunks in the CPU-baseline sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by heads with no communication; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops, stateflow
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.load()  # fail loudly if the HIP library is missing

    cfg = inputs.CONFIGS[args.workload]
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    dtype = cfg["dtype"]
    x = inputs.make(cfg, seed=2)

    def dev(a, dt):
        if dt == "bf16":
            bits = inputs.bf16_bits(a)
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    if cfg["kind"] == "shortconv":
        d = {k: dev(x[k], dtype) for k in ("x", "state_in", "dy")}
        w, bias = dev(x["w"], "fp32"), dev(x["bias"], "fp32")
        drv = stateflow.ShortConvChunked(d["x"], w, bias, N, act=cfg["act"])
        y = torch.empty_like(d["x"])

        def step():
            drv.forward(d["state_in"], y=y)
            drv.backward(d["dy"], None)
    else:
        H, dv = cfg["H"], cfg["dv"]
        delta = cfg["kind"] in ("gdn", "kda")
        keys = ("q", "k", "v", "g", "beta", "dO") if delta else ("q", "k", "v", "g", "dO")
        d = {k: dev(x[k], dtype) for k in keys}
        S_in = dev(x["S_in"], "fp32")
        if delta:
            cls = stateflow.GdnChunked if cfg["kind"] == "gdn" else stateflow.KdaChunked
            drv = cls(d["q"], d["k"], d["v"], d["g"], d["beta"], N)
        elif cfg["kind"] == "gla":
            drv = stateflow.GlaChunked(d["q"], d["k"], d["v"], d["g"], N)
        else:
            drv = stateflow.Mamba2Chunked(d["q"], d["k"], d["v"], d["g"], N)
        o = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device="cuda")
        grads = {k: torch.empty_like(d[k.replace("d", "", 1)] if k != "dbeta" else d["beta"])
                 for k in (("dq", "dk", "dv", "dg", "dbeta") if delta else ("dq", "dk", "dv", "dg"))}

        def step():
            drv.forward(S_in, o=o)
            drv.backward(d["dO"], None, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    value = B * T / (ms / 1e3)
    print(f"[bench] {args.workload}: {ms:.3f} ms/step, {value / 1e6:.2f} M tokens/s", file=sys.stderr, flush=True)

    # per-kernel durations, measured with start/stop events on the launch stream
    ops.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rep = ops.timing_report()
    ops.timing_enable(False)
    es = 2 if dtype == "bf16" else 4

    def launch_work(name):
        if cfg["kind"] == "shortconv":
            P = B * _conv_tile_groups(B, T // N, cfg["C"])
            return shortconv_work(name, B, T // N, cfg["C"], cfg["W"], es, P)
        wk = kernel_work(name, cfg["dk"], cfg["dv"], es)
        nb = B * cfg["H"] * ((T // N) // 64)
        return None if wk is None else (wk[0] * nb, wk[1] * nb)

    kernels = {}
    tot_ms = sum(v[1] for v in rep.values())
    tot_flops = 0.0
    for name, (launches, total_ms) in rep.items():
        avg_us = total_ms / launches * 1e3
        work = launch_work(name)
        ent = {"launches_per_step": launches // args.steps, "avg_us": round(avg_us, 2),
               "share": round(total_ms / tot_ms, 3)}
        if work:
            byts, flops = work
            if cfg["kind"] != "shortconv":  # short-convolution flops are vector ALU work, not MFMA
                tot_flops += flops * launches / args.steps
            ent.update(alg_bytes=byts, alg_flops=flops,
                       gbs=round(byts / (avg_us * 1e-6) / 1e9, 1),
                       tflops=round(flops / (avg_us * 1e-6) / 1e12, 2))
        kernels[name] = ent
        print(f"[bench]   {name:18s} {ent}", file=sys.stderr, flush=True)
    dom = max(rep, key=lambda k: rep[k][1])
    dk_ent = kernels[dom]
    bound = "hbm" if dk_ent["alg_flops"] / dk_ent["alg_bytes"] < RIDGE else "mfma"
    peak_flops = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    if bound == "hbm":
        achieved, peak, unit = dk_ent["gbs"], PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = dk_ent["tflops"], peak_flops, "TFLOP/s"
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": load_traffic(args.workload, dom),
                "kernel": dom, "avg_us": dk_ent["avg_us"], "alg_bytes_per_launch": dk_ent["alg_bytes"],
                "alg_flops_per_launch": dk_ent["alg_flops"]}
    mfma_util = tot_flops / (ms * 1e-3) / (peak_flops * 1e12)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic",
           "config": ({"workload": args.workload, "kind": cfg["kind"], "B": B, "T": T, "C": cfg["C"], "W": cfg["W"],
                       "act": "silu" if cfg["act"] else "identity", "seq_chunks": N}
                      if cfg["kind"] == "shortconv" else
                      {"workload": args.workload, "kind": cfg["kind"], "B": B, "T": T, "H": cfg["H"], "dk": cfg["dk"],
                       "dv": cfg["dv"], "seq_chunks": N, "block": 64}),
           "mfma_util": round(mfma_util, 4),
           "roofline": roofline, "kernels": kernels}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_chunks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
