#!/usr/bin/env python3
"""Benchmark: Gated DeltaNet chunked forward + backward on one MI355X.

One step = the whole hot path over one batch: the forward over the N
sequence chunks in order (boundary state handed S_out -> S_in) and the
backward over the chunks in reverse (dS_in -> dS_out), every kernel in the
HIP library through its C ABI.  Inputs are seeded synthetic tensors, resident
in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line (the fields are described in DESIGN.md, "Measured").

    python bench.py --workload NAME --profile-summary DIR

writes profiles/NAME.md and the NAME entries of profiles/traffic.json from
the rocprofv3 output under DIR (kt/: --kernel-trace --stats; fetch/, write/:
--pmc FETCH_SIZE / WRITE_SIZE; mfma/: --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE; copy/fetch/ and
copy/write/: the same FETCH/WRITE counters on --calibrate-copy 1 GiB).
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
CLOCK_GHZ, SIMDS = 2.4, 1024  # matrix-core busy cycles are summed over the 1024 SIMDs

# The layer's own tensors each kernel reads or writes (the algorithmic I/O of
# the pages' Fwd / Bwd, one touch each); the scans touch none of them, only
# the boundary states.  Sizes per token-head in bytes, see layer_io().
KERNEL_IO = {
    "gdn_prep": "k v g beta", "gdn_out": "q k o", "gdn_prep_bwd": "q k v g beta dO",
    "gdn_bwd_intra": "q k v g beta dO dq dk dv dg dbeta",
    "kda_prep": "k v g beta", "kda_out": "q k g o", "kda_prep_bwd": "k v g beta", "kda_prep2": "q k g dO",
    "kda_bwd_wy": "v beta dv dbeta", "kda_bwd_intra": "q k g beta dO dq dk dg",
}
for _p in ("gla", "m2"):
    KERNEL_IO.update({_p + "_prep": "k g", _p + "_out": "q k g o", _p + "_out_save": "q k g o", _p + "_prep_bwd": "q k g",
                      _p + "_scan_fwd": "v", _p + "_scan_fwd_rec": "v", _p + "_scan_fwd_save": "v",
                      _p + "_scan_bwd": "dO",
                      _p + "_bwd_intra": "q k v g dO dq dk dv dg"})
# boundary states each scan reads or writes (fp32 [B, H, dk, dv])
SCAN_STATES = {"gdn_scan_fwd": 2, "gdn_scan_pair": 3, "gdn_scan_rev": 2, "kda_scan_fwd": 2, "kda_scan_pair": 3, "kda_scan_rev": 2,
               "gla_scan_fwd": 2, "gla_scan_fwd_rec": 1, "gla_scan_fwd_save": 2, "gla_scan_bwd": 2,
               "m2_scan_fwd": 2, "m2_scan_fwd_rec": 1, "m2_scan_fwd_save": 2, "m2_scan_bwd": 2}


def layer_io(name: str, kind: str, dk: int, dv: int, es: int) -> int:
    """Algorithmic bytes per token-head of one kernel: the layer tensors it
    touches (q, k, dq, dk: dk elements; v, o, dO, dv: dv; g, dg: dk for the
    per-channel gates, 1 otherwise; beta, dbeta: 1), each once."""
    gk = dk if kind in ("gla", "kda") else 1
    size = {"q": dk, "k": dk, "dq": dk, "dk": dk, "v": dv, "o": dv, "dO": dv, "dv": dv,
            "g": gk, "dg": gk, "beta": 1, "dbeta": 1}
    return sum(size[t] for t in KERNEL_IO.get(name, "").split()) * es


def scan_phase_bytes(name: str, dk: int, dv: int, es: int) -> int:
    """The state-scan phase's per-unit traffic of the survey's section 8(d):
    per token-head, one direction of the scan reads its operands (W, K, U~:
    2 dk + dv elements) and writes the new values (dv elements) and the state
    entering each 64-token block in fp32 (dk dv / 64 floats): about 2 KB at
    dk = dv = 128.  The backward's pair launch runs two directions."""
    one = (2 * dk + 2 * dv) * es + dk * dv * 4 // 64
    return 2 * one if name.endswith("_pair") else one


def kernel_work(name: str, dk: int, dv: int, es: int, C: int = 64):
    """The design's model of one kernel per 64-token block and head: (bytes,
    flops), bytes counting every tensor it reads or writes once, workspace
    included (element size es; fp32 where the design keeps fp32), flops its
    dense products as executed (2 m n k each; a split operand executes a
    product twice, two split operands three times).  This is the traffic the
    design has to move, not the algorithmic I/O (layer_io)."""
    Ck, Cv, kv, CC, f4 = C * dk, C * dv, dk * dv, C * C, 4
    W = {
        # Gated DeltaNet (dk == dv): Ut and dU fp32; dh a bf16 pair
        "gdn_prep": (2 * Ck * es + 2 * C * es + 2 * C * f4 + 2 * Ck * es + Cv * f4,
                     2 * CC * dk + 2 * (2 * (2 * CC * dk)) + C ** 3 // 3),
        # U (read by the output kernel and the block adjoints) in the element type
        "gdn_scan_fwd": (C * f4 + 2 * Ck * es + Cv * f4 + kv * es + Cv * es, 3 * (2 * C * kv)),
        "gdn_out": (2 * Ck * es + C * f4 + kv * es + Cv * es + Cv * es,
                    2 * CC * dk + 2 * C * kv + 2 * (2 * CC * dv)),
        # R and dvloc in the element type
        "gdn_scan_bwd": (C * f4 + 2 * Ck * es + kv * es + Cv * es + 2 * kv * es + Cv * f4,
                         3 * (2 * C * kv) + 2 * C * kv // 2),
        # reads T^T that the backward's prep wrote and forms the decayed Gram tiles
        # again; U in the element type, dU fp32 (split when used)
        "gdn_bwd_intra": (4 * Ck * es + 2 * C * es + C * f4 + 3 * kv * es + Cv * es + Cv * f4 + 3 * Ck * es
                          + 2 * C * es + CC * es,
                          5 * (2 * C * kv) + 14 * (2 * CC * dk) + 2 * (2 * C ** 3) + CC * dk),
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
        # saved activations: each block's state a second time, in the backward's layout
        # (stored by the output kernel, or by the scan when no output is asked for)
        W[pre + "_scan_fwd_save"] = (W[pre + "_scan_fwd"][0] + kv * es, W[pre + "_scan_fwd"][1])
        W[pre + "_out_save"] = (W[pre + "_out"][0] + kv * es, W[pre + "_out"][1])
    W["gdn_scan_fwd_rec"] = W["gdn_scan_fwd"]
    # the backward's prep also reads Q and dO and writes the reverse scan's
    # operands W^T, Kh, dvloc^T, R (element type) and T^T for the block adjoints;
    # products P = Q K^T, P^T dO, Z = Gam Q - P W, R = Z^T dO
    W["gdn_prep_bwd"] = (W["gdn_prep"][0] + 2 * Ck * es + 2 * Ck * es + Cv * es + kv * es + CC * es,
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
    # reverse scan: Kh as a hi/lo pair and W^T in, R and dvloc fp32, dh and dU out
    kda_scan_bwd = (dk * f4 + 3 * Ck * es + kv * f4 + Cv * f4 + kv * es + Cv * es, 2 * (2 * C * kv))
    W["kda_scan_pair"] = tuple(x + y for x, y in zip(W["kda_scan_fwd"], kda_scan_bwd))
    W["kda_scan_rev"] = kda_scan_bwd  # saved activations: the reverse scan alone
    # the backward's prep also writes T^T, M and K e^b for the WY adjoint kernel
    W["kda_prep_bwd"] = (W["kda_prep"][0] + CC * es + CC * f4 + Ck * es, W["kda_prep"][1])
    W["kda_bwd_wy"] = (Ck * es + CC * es + CC * f4 + Cv * es + C * es + kv * es + Cv * es
                       + Cv * es + C * es + CC * f4 + Ck * f4,
                       2 * C * kv + 2 * CC * dv + 2 * CC * dk + 2 * (2 * C ** 3) + 2 * CC * dv + 2 * CC * dk)
    W["kda_bwd_intra"] = (5 * Ck * es + 2 * kv * es + CC * f4 + Ck * f4 + C * es + 3 * Ck * es,
                          2 * (2 * CC * dv) + 2 * (2 * C * kv) + 4 * (2 * CC * dk))
    # one launch running the forward recompute and the reverse scan side by side
    W["gdn_scan_pair"] = tuple(x + y for x, y in zip(W["gdn_scan_fwd_rec"], W["gdn_scan_bwd"]))
    # with saved activations the backward runs the reverse scan alone (and the
    # forward scan also stores each block's state in the backward's layout)
    W["gdn_scan_rev"] = W["gdn_scan_bwd"]
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
    """Hash of the HIP sources' code (ties stored counter data to a kernel
    build): comments and whitespace are left out, so that editing a comment
    does not detach the counters of an unchanged kernel."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_linear_recurrence_chunk_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".h")):
            with open(os.path.join(csrc, fn), encoding="utf-8") as f:
                code = f.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            code = " ".join(code.split())
            h.update(fn.encode() + code.encode())
    return h.hexdigest()[:16]


def load_counters(workload: str, kernel: str):
    """The committed rocprofv3 counter summary of one kernel (HBM bytes per
    launch, matrix-core busy cycles and flops per launch), or None if absent
    or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    e = d.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e


def load_traffic(workload: str, kernel: str):
    e = load_counters(workload, kernel)
    return None if e is None else e.get("bytes_per_launch")


def launch_name(mangled: str, kind: str) -> str:
    """The library's launch name of a kernel symbol in a rocprofv3 trace
    (the symbol is a template instantiation; the flags that tell launches of
    one kernel apart are its bool template arguments, in order)."""
    import re
    m = re.match(r"_ZN3clr(?:12_GLOBAL__N_1)?(\d+)", mangled)  # (kernels of a file-local namespace)
    if not m:  # an unmangled symbol
        return mangled[:-len("_kernel")] if mangled.endswith("_kernel") else mangled
    n = int(m.group(1))
    base = mangled[m.end():m.end() + n]
    base = base[:-len("_kernel")] if base.endswith("_kernel") else base
    flags = re.findall(r"Lb([01])E", mangled[m.end() + n:])
    if base == "gdn_prep":
        return "gdn_prep_bwd" if flags[0] == "1" else "gdn_prep"
    if base == "gdn_scan_fwd":  # <E, DK, DV, HNAT, PCD, NP, NVS>
        return "kda_scan_fwd" if flags[1] == "1" else "gdn_scan_fwd"
    if base == "gdn_scan_pair":  # <E, DK, DV, PCD, NP, NCW>
        return "kda_scan_pair" if flags[0] == "1" else "gdn_scan_pair"
    if base == "gdn_scan_rev":  # <E, DK, DV, PCD, NP, NCW>
        return "kda_scan_rev" if flags[0] == "1" else "gdn_scan_rev"
    if base.startswith("gla_"):
        pre = {"gla": "gla_", "mamba2": "m2_", "kda": "kda_"}.get(kind, "gla_")
        rest = base[4:]
        if rest == "prep":  # <E, DK, BWD, SG>
            rest = "prep_bwd" if flags[0] == "1" else "prep"
        elif rest == "scan_fwd":  # <E, DK, DV, HNAT, HN>
            rest = "scan_fwd_rec" if flags[0] == "1" else "scan_fwd_save" if flags[1:2] == ["1"] else "scan_fwd"
        elif rest == "out" and kind != "kda":  # <E, DK, DV, SG, HN>
            rest = "out_save" if flags[1:2] == ["1"] else "out"
        return pre + rest
    return base  # kda_prep serves both the forward and the backward's prep


def profile_summary(workload: str, d: str) -> None:
    """Summarise the rocprofv3 passes under d (see the module docstring) into
    profiles/<workload>.md and the workload's entries of profiles/traffic.json."""
    import csv
    import glob
    from collections import defaultdict
    from chunked_linear_recurrence_chunk_amd import inputs
    cfg = inputs.CONFIGS[workload]
    kind = cfg["kind"]

    def one(pattern):
        f = glob.glob(os.path.join(d, pattern))
        if not f:
            raise SystemExit(f"no {pattern} under {d}")
        return list(csv.DictReader(open(f[0])))

    def counters(sub):
        per = defaultdict(lambda: defaultdict(list))
        for r in one(sub + "/*counter_collection.csv"):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in per.items()}

    copy_dir = os.path.join(d, "..", "copy")
    cf = counters_copy = {}
    for sub in ("fetch", "write"):
        rows = [r for r in csv.DictReader(open(glob.glob(os.path.join(copy_dir, sub, "*counter_collection.csv"))[0]))
                if "copyBuffer" in r["Kernel_Name"]]
        cf[sub] = sum(float(r["Counter_Value"]) for r in rows) / len(rows)
    gib_kib = (1 << 30) / 1024
    f_scale, w_scale = gib_kib / cf["fetch"], gib_kib / cf["write"]
    stats = {}
    for r in one("kt/*kernel_stats.csv"):
        name = launch_name(r["Name"], kind)
        st = stats.setdefault(name, {"calls": 0, "ns": 0.0, "pct": 0.0})
        st["calls"] += int(r["Calls"])
        st["ns"] += float(r["TotalDurationNs"])
        st["pct"] += float(r["Percentage"])
    fetch, write, mfma = counters("fetch"), counters("write"), counters("mfma")

    def by_name(c):
        out = defaultdict(list)
        for k, v in c.items():
            out[launch_name(k, kind)].append(v)
        return {k: {c2: sum(x[c2] for x in vs) / len(vs) for c2 in vs[0]} for k, vs in out.items()}
    fetch, write, mfma = by_name(fetch), by_name(write), by_name(mfma)
    h = source_hash()
    tp = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        allt = json.load(open(tp))
    except (OSError, ValueError):
        allt = {}
    ent = {}
    rows = []
    for name, st in sorted(stats.items(), key=lambda kv: -kv[1]["ns"]):
        if name not in fetch or name not in write:
            continue
        fk, wk = fetch[name]["FETCH_SIZE"], write[name]["WRITE_SIZE"]
        byts = int(round(fk * 1024 * f_scale + wk * 1024 * w_scale))
        e = {"bytes_per_launch": byts, "source_hash": h, "fetch_kib": fk, "write_kib": wk}
        mf = mfma.get(name)
        if mf:
            e.update(mfma_flops=mf["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512, mfma_busy_cycles=mf["SQ_VALU_MFMA_BUSY_CYCLES"],
                     sq_busy_cycles=mf["SQ_BUSY_CYCLES"], grbm_gui_active=mf["GRBM_GUI_ACTIVE"])
        ent[name] = e
        avg_us = st["ns"] / st["calls"] / 1e3
        busy = e.get("mfma_busy_cycles")
        rows.append(f"| {name} | {st['calls']} | {avg_us:.2f} | {st['pct']:.1f} | {fk:.1f} | {wk:.1f} | "
                    f"{byts / 1e6:.1f} | {byts / (avg_us * 1e-6) / 1e9:.0f} | "
                    + (f"{e['mfma_flops'] / 1e9:.2f} | {busy:.3g} | {busy / (SIMDS * CLOCK_GHZ * 1e3 * avg_us):.3f} | "
                       f"{e['mfma_flops'] / (avg_us * 1e-6) / 1e12:.0f} |" if busy is not None else "- | - | - | - |"))
    allt[workload] = ent
    with open(tp, "w") as f:
        json.dump(allt, f, indent=1, sort_keys=True)
    args = f"--workload {workload}"
    md = [f"# rocprofv3 summary: {workload}", "",
          f"Workload: {cfg}; one launch processes one sequence chunk.", "",
          "Commands (run from /tmp with TMPDIR=/tmp; R = repository root; O = an output directory, "
          "D = $O/" + workload + "; the copy calibration goes to $O/copy, where the summary step looks "
          "for it):", "", "```",
          f"rocprofv3 --kernel-trace --stats -T -f csv -d $D/kt -o run -- python3 $R/bench.py {args} --steps 5 --warmup 2 --no-cpu",
          f"rocprofv3 --pmc FETCH_SIZE -T -f csv -d $D/fetch -o run -- python3 $R/bench.py {args} --steps 1 --warmup 1 --no-cpu",
          f"rocprofv3 --pmc WRITE_SIZE -T -f csv -d $D/write -o run -- python3 $R/bench.py {args} --steps 1 --warmup 1 --no-cpu",
          "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -T -f csv "
          f"-d $D/mfma -o run -- python3 $R/bench.py {args} --steps 1 --warmup 1 --no-cpu",
          "rocprofv3 --pmc FETCH_SIZE -T -f csv -d $O/copy/fetch -o run -- python3 $R/bench.py --calibrate-copy 1073741824",
          "rocprofv3 --pmc WRITE_SIZE -T -f csv -d $O/copy/write -o run -- python3 $R/bench.py --calibrate-copy 1073741824",
          f"cd $R && python3 bench.py {args} --profile-summary $D", "```", "",
          f"Counter calibration (1 GiB device copy): FETCH_SIZE reads {cf['fetch']:.0f} KiB, WRITE_SIZE "
          f"{cf['write']:.0f} KiB per dispatch -> scale factors fetch x{f_scale:.3f}, write x{w_scale:.3f}.", "",
          "Matrix cores: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 is the bf16 matrix flops a launch executed; "
          "SQ_VALU_MFMA_BUSY_CYCLES counts matrix-core busy cycles summed over the 1024 SIMDs (16 per "
          "16x16x32 bf16 instruction), so busy / (1024 x 2.4 GHz x duration) is the fraction of the "
          "chip's matrix-core time in use, equal to (flops / duration) / 2.5 PFLOP/s.", "",
          f"Kernel sources hash: {h}", ""]
    if kind == "kda":
        md += ["`kda_prep` runs in the forward and, writing a few more outputs, in the backward: the trace "
               "merges both (one kernel symbol).", ""]
    md += ["| kernel | calls | avg us | share % | FETCH KiB/disp | WRITE KiB/disp | HBM MB/launch (scaled) | HBM GB/s | "
           "MFMA GFLOP/launch | MFMA busy cycles | MFMA busy frac | MFMA TFLOP/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"] + rows
    open(os.path.join(ROOT, "profiles", workload + ".md"), "w").write("\n".join(md) + "\n")
    print("wrote", os.path.join("profiles", workload + ".md"))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _compiler() -> str:
    import subprocess
    try:
        return subprocess.run(["gcc", "--version"], capture_output=True, text=True).stdout.splitlines()[0]
    except (OSError, IndexError):
        return "unknown"


def cpu_baseline(cfg: dict, x: dict, budget_chunks: int, reps: int = 20, reps1: int = 5):
    """The fp64 oracle (as it stands) on the host cores over a bounded sample:
    the first `budget_chunks` sequence chunks of the workload (at most 4096
    tokens), forward then backward with boundary-state hand-off.  The median
    of `reps` runs on all cores, and of `reps1` runs on one core."""
    import statistics

    import numpy as np
    from oracle import oracle
    threads = len(os.sched_getaffinity(0))
    T, N = cfg["T"], cfg["N"]
    L = T // N
    n = max(1, min(budget_chunks, N, max(1, 4096 // L)))
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

    def median_time(k, nthreads):
        oracle.set_threads(nthreads)
        ts = []
        for _ in range(k):
            t0 = time.perf_counter()
            once()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts), sum(ts)

    once()  # page the sample in
    med, tot = median_time(reps, threads)
    med1, tot1 = median_time(reps1, 1)
    oracle.set_threads(threads)
    tok = cfg["B"] * Ts
    return {"value": tok / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread": tok / med1, "cpu_model": _cpu_model(), "compiler": _compiler(),
            "build": "gcc -O3 -march=x86-64-v3 -fopenmp, fp64; OpenMP over (batch, head)",
            "sample": f"{'all' if n == N else f'first {n} of'} {N} sequence chunks ({cfg['B']}x{Ts} tokens, "
                      + (f"all {cfg['C']} channels" if cfg["kind"] == "shortconv" else f"all {cfg['H']} heads")
                      + f"), fp64 fwd+bwd; median of {reps} runs on {threads} threads ({tot:.1f} s) "
                      + f"and of {reps1} on one ({tot1:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-chunks", type=int, default=64, help="sequence chunks in the CPU-baseline sample")
    ap.add_argument("--profile-summary", metavar="DIR", help="summarise rocprofv3 output under DIR into profiles/")
    ap.add_argument("--scan-bv", type=int, choices=(16, 32), default=None,
                    help="value columns per work-group of the Gated DeltaNet forward scan (default: the library's, 16)")
    ap.add_argument("--fwd-split", type=int, default=None, metavar="PERMILLE",
                    help="split-and-overlap forward at PERMILLE/1000 of the blocks (0 = off, the default)")
    ap.add_argument("--saved", action="store_true",
                    help="keep each chunk's forward activations for its "
                         "backward (*_fwd_save / *_bwd_saved) instead of recomputing them")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.profile_summary:
        profile_summary(args.workload, args.profile_summary)
        return
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
    if args.scan_bv is not None:
        ops.set_scan_bv(args.scan_bv)
    if args.fwd_split is not None:
        ops.set_fwd_split(args.fwd_split)

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
            if cfg["kind"] == "gdn":
                drv = stateflow.GdnChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N, save=args.saved)
            else:
                drv = stateflow.KdaChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N, save=args.saved)
        elif cfg["kind"] == "gla":
            drv = stateflow.GlaChunked(d["q"], d["k"], d["v"], d["g"], N, save=args.saved)
        else:
            drv = stateflow.Mamba2Chunked(d["q"], d["k"], d["v"], d["g"], N, save=args.saved)
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
    conv = cfg["kind"] == "shortconv"
    th = 0 if conv else B * cfg["H"] * (T // N)  # token-heads per launch (one sequence chunk)
    nst = 0 if conv else B * cfg["H"] * cfg["dk"] * cfg["dv"] * 4  # bytes of one fp32 boundary state
    for name, (launches, total_ms) in rep.items():
        avg_us = total_ms / launches * 1e3
        ent = {"launches_per_step": launches // args.steps, "avg_us": round(avg_us, 2),
               "share": round(total_ms / tot_ms, 3)}
        work = launch_work(name)
        if conv:
            alg = work[0] if work else None
        elif "scan" in name:
            alg = scan_phase_bytes(name, cfg["dk"], cfg["dv"], es) * th + SCAN_STATES.get(name, 0) * nst
        else:
            alg = layer_io(name, cfg["kind"], cfg["dk"], cfg["dv"], es) * th
        if alg:
            ent.update(alg_bytes=alg, alg_gbs=round(alg / (avg_us * 1e-6) / 1e9, 1))
        if work:
            ent.update(model_bytes=work[0], model_flops=work[1],
                       model_tflops=round(work[1] / (avg_us * 1e-6) / 1e12, 2))
        ctr = load_counters(args.workload, name)
        if ctr:
            ent.update(hbm_bytes=ctr["bytes_per_launch"],
                       hbm_gbs=round(ctr["bytes_per_launch"] / (avg_us * 1e-6) / 1e9, 1))
            if alg:
                ent["hbm_over_alg"] = round(ctr["bytes_per_launch"] / alg, 2)
            if ctr.get("mfma_busy_cycles") is not None:
                ent["mfma_busy"] = round(ctr["mfma_busy_cycles"] / (SIMDS * CLOCK_GHZ * 1e3 * avg_us), 4)
                ent["mfma_tflops"] = round(ctr["mfma_flops"] / (avg_us * 1e-6) / 1e12, 2)
        kernels[name] = ent
        print(f"[bench]   {name:18s} {ent}", file=sys.stderr, flush=True)
    dom = max(rep, key=lambda k: rep[k][1])
    de = kernels[dom]
    flops = de.get("model_flops", 0)
    bound = "hbm" if (conv or flops / de["alg_bytes"] < RIDGE) else "mfma"
    peak_flops = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    if bound == "hbm":
        achieved, peak, unit = de["alg_gbs"], PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = round(flops / (de["avg_us"] * 1e-6) / 1e12, 2), peak_flops, "TFLOP/s"
    traffic = load_traffic(args.workload, dom)
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_over_alg": round(traffic / de["alg_bytes"], 2) if traffic else None,
                "kernel": dom, "avg_us": de["avg_us"], "alg_bytes_per_launch": de["alg_bytes"]}

    # the two phases the targets name: intra-chunk (every block-parallel
    # kernel) against the bf16 matrix-core peak, state scan against HBM
    phases = None
    if not conv:
        per_step = {k: rep[k][1] / args.steps for k in rep}  # ms
        intra = [k for k in rep if "scan" not in k]
        scan = [k for k in rep if "scan" in k]
        t_in = sum(per_step[k] for k in intra) * 1e-3
        t_sc = sum(per_step[k] for k in scan) * 1e-3
        dk, dv, C = cfg["dk"], cfg["dv"], 64
        if cfg["kind"] == "gdn":
            # section 8(d): fwd 2C(3dk+2dv) + 6 dk dv + C^2/3, bwd C(18dk+10dv) + 16 dk dv + 4.3 C^2
            # per token-head, less the scans' 12 dk dv
            f_th = (2 * C * (3 * dk + 2 * dv) + 6 * dk * dv + C * C / 3 + C * (18 * dk + 10 * dv)
                    + 16 * dk * dv + 4.3 * C * C - 12 * dk * dv)
            f_in, f_src = f_th * B * cfg["H"] * T, "algorithmic, section 8(d)"
        else:
            f_in = sum(kernels[k].get("model_flops", 0) * rep[k][0] / args.steps for k in intra)
            f_src = "products as executed"
        ph_in = {"kernels": intra, "us_per_step": round(t_in * 1e6, 1), "flops_per_step": f_in, "flops": f_src,
                 "tflops": round(f_in / t_in / 1e12, 1), "frac_of_mfma_peak": round(f_in / t_in / 1e12 / peak_flops, 4),
                 "target": 0.5}
        busy = [(load_counters(args.workload, k), k) for k in intra]
        if all(c and c.get("mfma_busy_cycles") is not None for c, _ in busy):
            cyc = sum(c["mfma_busy_cycles"] * rep[k][0] / args.steps for c, k in busy)
            ph_in["mfma_busy_counter"] = round(cyc / (SIMDS * CLOCK_GHZ * 1e9 * t_in), 4)
        tr = [load_traffic(args.workload, k) for k in scan]
        ph_sc = {"kernels": scan, "us_per_step": round(t_sc * 1e6, 1), "target": 0.6}
        if scan and all(tr):
            byts = sum(t * rep[k][0] / args.steps for t, k in zip(tr, scan))
            ph_sc.update(bytes_per_step=byts, bytes="rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated",
                         gbs=round(byts / t_sc / 1e9, 1), frac_of_hbm_peak=round(byts / t_sc / 1e9 / PEAK_HBM_GBS, 4))
        elif scan:
            byts = sum(kernels[k]["alg_bytes"] * rep[k][0] / args.steps for k in scan)
            ph_sc.update(bytes_per_step=byts, bytes="section 8(d) per-unit figure (no counters at these sources)",
                         gbs=round(byts / t_sc / 1e9, 1), frac_of_hbm_peak=round(byts / t_sc / 1e9 / PEAK_HBM_GBS, 4))
        phases = {"intra": ph_in, "scan": ph_sc}
    mfma_util = None
    cs = [(load_counters(args.workload, k), k) for k in rep]
    if not conv and all(c and c.get("mfma_flops") is not None for c, _ in cs):
        mfma_util = round(sum(c["mfma_flops"] * rep[k][0] / args.steps for c, k in cs) / (ms * 1e-3)
                          / (peak_flops * 1e12), 4)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic",
           "config": ({"workload": args.workload, "kind": cfg["kind"], "B": B, "T": T, "C": cfg["C"], "W": cfg["W"],
                       "act": "silu" if cfg["act"] else "identity", "seq_chunks": N}
                      if conv else
                      {"workload": args.workload, "kind": cfg["kind"], "B": B, "T": T, "H": cfg["H"], "dk": cfg["dk"],
                       "dv": cfg["dv"], "seq_chunks": N, "block": 64,
                       "scan_bv": ops.get_scan_bv(), "fwd_split_permille": ops.get_fwd_split(),
                       "backward": "saved activations" if args.saved
                       else "recompute from S_in"}),
           "mfma_util": mfma_util,
           "peak_mem_gb": round(torch.cuda.max_memory_allocated() / 1e9, 3),
           "roofline": roofline, "phases": phases, "kernels": kernels}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_chunks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
