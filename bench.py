"""Benchmark: MoE layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config moe7b_bf16]

A step is one moe_forward + moe_backward over one batch of synthetic tokens
(router GEMM, route, permute, gate/up grouped GEMM with SwiGLU, down grouped
GEMM, shared experts, combine; then combine backward with the router
gradient, the four routed and four shared data/weight-gradient grouped GEMMs,
the router weight gradient and the unpermute-sum).  Inputs are resident in
HBM before timing starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"
METRIC_FWD = "MoE layer fwd tokens/s; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP32_TFLOPS = 157.3
FLUSH_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="moe7b_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--all-configs-summarize", metavar="LOG",
                   help="rebuild the all-configs table under profiles/ from the JSON lines of an --all-configs run")
    p.add_argument("--all-configs", action="store_true",
                   help="run every layer configuration (forward workloads forward only) with its oracle baseline "
                        "on a token sample, and write the table under profiles/")
    p.add_argument("--no-fp8", action="store_true", help="skip the fp8 gate/up measurement")
    p.add_argument("--permuted-copy", action="store_true",
                   help="materialise the permuted token rows (x_perm) instead of gathering them")
    p.add_argument("--cpu-tokens", type=int, default=16384, help="token sample for the oracle timing")
    p.add_argument("--router-terms", action="store_true",
                   help="add the router training terms to every step: balance loss 1e-3, per-sequence balance "
                        "loss 1e-3 over 4096-token sequences, z-loss 1e-3, and the proportional bias update "
                        "at rate 1e-3")
    p.add_argument("--pmc-probe", action="store_true",
                   help="run one forward, one 1 GiB device copy and one gate/up GEMM launch, then exit "
                        "(the program that rocprofv3 --pmc passes count)")
    p.add_argument("--trace-summarize", metavar="TRACE_DIR",
                   help="write the kernel-trace summary of a profiled run (rocprofv3 --kernel-trace --stats "
                        "--output-format csv -o bench) to profiles/moe7b_bf16_fwd_bwd_kernel_stats.txt")
    p.add_argument("--pmc-report", nargs="+", metavar="PASS_DIR",
                   help="turn the counter CSVs of the pmc_mfma, pmc_ea_read and pmc_ea_write passes over "
                        "--pmc-probe into the per-product counter table under profiles/")
    p.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn the counter CSVs of a FETCH_SIZE pass and a WRITE_SIZE pass over "
                        "--pmc-probe into the traffic record under profiles/")
    return p.parse_args()


# ---- HBM traffic of the dominant kernel, from two rocprofv3 --pmc passes
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_moe7b_bf16_traffic.txt")
# the routed gate/up product: forward layout, SwiGLU, bf16, rows gathered
GATE_UP_KERNEL = "pk::gemm_kernel<0, 1, false, true, 8, 0, false, false>"
KERNEL_SOURCES = ["mixture_experts_layer_18_amd/csrc/gemm_big.hip",
                  "mixture_experts_layer_18_amd/csrc/gemm_common.h",
                  "mixture_experts_layer_18_amd/csrc/common.h",
                  "mixture_experts_layer_18_amd/csrc/kernels.h"]


def progress(msg):
    """A progress line on stderr (stdout carries the JSON result only)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _probe_values(rows, counter):
    """(copy, gemm) values of `counter`: the probe's last gate/up GEMM dispatch
    and the last device copy dispatched before it."""
    rows = [r for r in rows if r["Counter_Name"] == counter]
    gemm = [r for r in rows if GATE_UP_KERNEL in r["Kernel_Name"]]
    if not gemm:
        raise SystemExit(f"no gate/up GEMM dispatch with {counter}")
    g = max(gemm, key=lambda r: int(r["Dispatch_Id"]))
    copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]
              and int(r["Dispatch_Id"]) < int(g["Dispatch_Id"])]
    if not copies:
        raise SystemExit(f"no device copy dispatch before the GEMM with {counter}")
    c = max(copies, key=lambda r: int(r["Dispatch_Id"]))
    return float(c["Counter_Value"]) * 1024.0, float(g["Counter_Value"]) * 1024.0


TRACE_COMMAND = ("rocprofv3 --kernel-trace --stats --output-format csv -d <root>/gpurun_out/prof -o bench -- "
                 "python3 <root>/bench.py --steps 5 --warmup 2 --no-cpu-baseline")


def trace_summarize(d):
    """Per-kernel statistics of a profiled bench run, and the same trace cut
    into layer steps (each step starts at a router-logits launch), one line
    per launch position within a step."""
    import collections
    import csv
    stats = list(csv.DictReader(open(os.path.join(d, "bench_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(d, "bench_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # noqa: E731
    short = lambda r: r["Kernel_Name"].split("(")[0].replace("void ", "")  # noqa: E731
    L = ["Kernel durations of the MoE layer forward+backward, moe7b_bf16 (T=16384, d_model=2048, E=64, "
         "sigmoid top-6, d_ff=1408, 2 shared x 1408), bf16, one MI355X; 2 warm-up, 5 timed and 5 "
         "per-stage-timing steps", "",
         "Commands (from the repository root):", "  cd /tmp && export TMPDIR=/tmp", "  " + TRACE_COMMAND,
         "  python bench.py --trace-summarize gpurun_out/prof", "", "rocprofv3 --stats (per kernel symbol):", ""]
    L.append(f"{'kernel':<92s} {'calls':>5s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'%':>6s}")
    for r in stats:
        L.append(f"{r['Name'][:92]:<92s} {int(r['Calls']):5d} {float(r['AverageNs'])/1e3:9.1f} "
                 f"{float(r['MinNs'])/1e3:9.1f} {float(r['MaxNs'])/1e3:9.1f} {float(r['Percentage']):6.2f}")
    steps, cur = [], None
    for r in trace:
        if "router_logits" in r["Kernel_Name"]:
            cur = []
            steps.append(cur)
        if cur is not None:
            cur.append(r)
    # the last step also holds the launches after the timed steps (the
    # separate measurements); cut it to the length of the first step
    after = []
    if len(steps) > 1 and len(steps[-1]) > len(steps[0]):
        after = steps[-1][len(steps[0]):]
        steps[-1] = steps[-1][:len(steps[0])]
    agg = collections.OrderedDict()
    for st in steps:
        seen = collections.Counter()
        for r in st:
            seen[short(r)] += 1
            agg.setdefault(f"{short(r)} #{seen[short(r)]}", []).append(dur(r))
    L += ["", f"Same trace, one line per launch of a step ({len(steps)} steps; #n = n-th launch of that",
          "kernel within the step, in launch order):", ""]
    L.append(f"{'kernel #occurrence':<70s} {'calls':>5s} {'avg us':>9s} {'min us':>9s}")
    for k, v in agg.items():
        L.append(f"{k[:70]:<70s} {len(v):5d} {sum(v)/len(v):9.1f} {min(v):9.1f}")
    if after:
        aft = collections.OrderedDict()
        for r in after:
            aft.setdefault(short(r), []).append(dur(r))
        L += ["", "Launches after the layer steps (the separate measurements: the copy-ceiling",
              "copies and the fp8 gate/up product with its activation quantisation):", ""]
        L.append(f"{'kernel':<70s} {'calls':>5s} {'avg us':>9s} {'min us':>9s}")
        for k, v in aft.items():
            L.append(f"{k[:70]:<70s} {len(v):5d} {sum(v)/len(v):9.1f} {min(v):9.1f}")
    out = os.path.join(ROOT, "profiles", "moe7b_bf16_fwd_bwd_kernel_stats.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("wrote", out)


def pmc_summarize(fetch_dir, write_dir):
    cf, gf = _probe_values(_counter_rows(fetch_dir), "FETCH_SIZE")
    cw, gw = _probe_values(_counter_rows(write_dir), "WRITE_SIZE")
    # the counters read the copy's known bytes (COPY_BYTES read, COPY_BYTES
    # written) scaled by some factor; the GEMM's reading is divided by it
    ff, fw = cf / COPY_BYTES, cw / COPY_BYTES
    fetch, write = gf / ff, gw / fw
    rec = {"kernel_source_sha": kernel_source_hash(), "fetch_bytes": fetch, "write_bytes": write,
           "traffic_bytes": fetch + write, "copy_fetch_factor": ff, "copy_write_factor": fw,
           "raw_fetch_kib": gf / 1024.0, "raw_write_kib": gw / 1024.0}
    lines = [
        "HBM traffic of the routed gate/up grouped GEMM + SwiGLU (forward, NT), moe7b_bf16",
        "(T=16384, d_model=2048, E=64, top-6, d_ff=1408), one launch.",
        "",
        "Commands (from the repository root; each pass runs alone):",
        "  cd /tmp && export TMPDIR=/tmp",
        "  rocprofv3 --pmc FETCH_SIZE -d <root>/gpurun_out/pmc_FETCH_SIZE -o run --output-format csv "
        "-- python3 <root>/bench.py --pmc-probe",
        "  rocprofv3 --pmc WRITE_SIZE -d <root>/gpurun_out/pmc_WRITE_SIZE -o run --output-format csv "
        "-- python3 <root>/bench.py --pmc-probe",
        "  python bench.py --pmc-summarize gpurun_out/pmc_FETCH_SIZE gpurun_out/pmc_WRITE_SIZE",
        "",
        f"calibration: a {COPY_BYTES} B device copy read FETCH_SIZE {cf / 1024:.0f} KiB "
        f"(factor {ff:.4f}) and WRITE_SIZE {cw / 1024:.0f} KiB (factor {fw:.4f})",
        f"gate/up GEMM raw: FETCH_SIZE {gf / 1024:.0f} KiB, WRITE_SIZE {gw / 1024:.0f} KiB",
        f"gate/up GEMM scaled: fetch {fetch / 1e9:.3f} GB, write {write / 1e9:.3f} GB, "
        f"total {(fetch + write) / 1e9:.3f} GB per launch",
        "",
        "record: " + json.dumps(rec),
    ]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---- matrix-core utilisation, clock and LDS behaviour of every product
COUNTER_FILE = os.path.join(ROOT, "profiles", "gemm_counters_moe7b_bf16.txt")
PMC_PASSES = {
    "mfma": "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_BUSY_CU_CYCLES "
            "GRBM_GUI_ACTIVE GRBM_COUNT",
    "lds": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAVE_CYCLES",
    "ea_read": "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum",
    "ea_write": "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum",
}
SIMDS, XCDS, CUS = 1024, 8, 256
# the probe's launches, in order, named by stage (kernel symbol prefix,
# occurrence among the probe's dispatches of that symbol)
PROBE_STAGES = [
    ("pk::gemm_kernel<0, 1, false, true, 8, 0, false, false>", 1, "gate_up (in the forward)"),
    ("pk::gemm_kernel<0, 0, false, false, 8, 0, false, false>", 1, "down"),
    ("pk::gemm_kernel<0, 1, false, false, 8, 0, false, false>", 1, "shared_gate_up"),
    ("pk::gemm_kernel<0, 0, false, false, 8, 0, false, false>", 2, "shared_down"),
    ("pk::gemm_kernel<0, 1, false, true, 8, 0, false, false>", 2, "gate_up (alone, after the copy)"),
    ("pk::gemm_kernel<1, 2, false, false, 8, 0, false, false>", 1, "down_dgrad (dSwiGLU)"),
    ("pk::gemm_kernel<1, 2, false, false, 8, 0, false, false>", 2, "shared_down_dgrad"),
    ("pk::gemm_kernel<2, 0, false, false, 8, 0, false, true>", 1, "down_wgrad + shared (one launch)"),
    ("pk::gemm_kernel<2, 0, false, true, 8, 0, false, true>", 1, "gate_up_wgrad + shared (one launch)"),
    ("pk::gemm_kernel<1, 0, false, false, 8, 0, false, false>", 1, "gate_up_dgrad"),
    ("pk::gemm_kernel<1, 0, false, false, 8, 0, false, false>", 2, "shared_gate_up_dgrad"),
    ("pk::gemm_kernel<0, 1, true, false, 8, 0, false, false>", 1, "fp8 gate_up"),
]
PMC_COMMAND = ("timeout -s KILL 120 rocprofv3 --pmc {counters} -d <root>/gpurun_out/pmc_{name} -o run "
               "--output-format csv -- python3 <root>/bench.py --pmc-probe")


def _dispatches(d):
    """{dispatch id: (kernel name, duration ns, {counter: value})} of one pass."""
    out = {}
    for r in _counter_rows(d):
        i = int(r["Dispatch_Id"])
        if i not in out:
            out[i] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {})
        out[i][2][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def pmc_report(dirs):
    """Per-product counter table of the probe from the passes in dirs
    (directories named pmc_<pass>): matrix-core busy share, shader clock,
    LDS bank conflicts, and the memory-side read/write bytes by request size,
    scaled by what the same counters read for the 1 GiB device copy."""
    passes = {}
    for d in dirs:
        name = os.path.basename(os.path.normpath(d))[len("pmc_"):]
        passes[name] = _dispatches(d)
    # dispatch ids are per process (one process per pass); the probe's launch
    # sequence is the same in each, so ids line up across passes
    base = passes["mfma"]
    seen = {}
    rows = []
    copy_id = max(i for i, (k, _, _) in base.items() if "copyBuffer" in k)
    prefixes = {pre for pre, _, _ in PROBE_STAGES}
    for i in sorted(base):
        k, dur, cv = base[i]
        pre = next((p for p in prefixes if k.replace("void ", "").startswith("moe::" + p)), None)
        if pre is None:
            continue
        seen[pre] = seen.get(pre, 0) + 1
        for p, occ, label in PROBE_STAGES:
            if p == pre and occ == seen[pre]:
                rows.append((label, i, k, dur))
    def cal(pname, keys):
        ids = passes.get(pname)
        if ids is None:
            return None
        c = ids[copy_id][2]
        return {kk: c.get(kk, 0.0) for kk in keys}
    rd_keys = ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"]
    wr_keys = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"]

    def rd_bytes(c):
        n, n32, n64, n128 = (c.get(kk, 0.0) for kk in rd_keys)
        return 32 * n32 + 64 * n64 + 128 * n128, n - n32 - n64 - n128

    def wr_bytes(c):
        n, n64 = (c.get(kk, 0.0) for kk in wr_keys)
        return 64 * n64 + 32 * (n - n64)
    crd = cal("ea_read", rd_keys)
    cwr = cal("ea_write", wr_keys)
    rd_fac = rd_bytes(crd)[0] / COPY_BYTES if crd else None
    wr_fac = wr_bytes(cwr) / COPY_BYTES if cwr else None
    L = ["Hardware counters of every grouped-GEMM product of one moe7b_bf16 layer step (T=16384, d_model=2048,",
         "E=64, sigmoid top-6, d_ff=1408, 2 shared x 1408, bf16; rows gathered), one MI355X, one dispatch each.",
         "", "Commands (from the repository root; one counter set per pass, each pass its own run):",
         "  cd /tmp && export TMPDIR=/tmp"]
    for pname, ctrs in PMC_PASSES.items():
        L.append("  " + PMC_COMMAND.format(counters=ctrs, name=pname))
    L += ["  python bench.py --pmc-report " + " ".join(f"gpurun_out/pmc_{n}" for n in PMC_PASSES), "",
          "mfma busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): the share of the",
          "kernel's cycles in which a SIMD's matrix core was busy.  clock = GRBM_GUI_ACTIVE / 8 / duration.",
          "flop check = SQ_INSTS_VALU_MFMA_MOPS_* x 512 (the matrix-core work actually issued, padding rows",
          "included).  lds conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.  read / write = memory-side",
          "bytes from the request counts by size (32/64/128 B), divided by the factor the same counters read",
          "for the 1 GiB copy (read {}, write {}).".format(
              "n/a" if rd_fac is None else f"{rd_fac:.4f}", "n/a" if wr_fac is None else f"{wr_fac:.4f}"), ""]
    L.append(f"{'product':<44s} {'us':>8s} {'mfma busy':>9s} {'clock':>6s} {'issued TFLOP':>12s} "
             f"{'lds conf':>8s} {'read GB':>8s} {'write GB':>8s}")
    recs = {}
    for label, i, k, dur in rows:
        cv = dict(base[i][2])
        if "lds" in passes:
            cv.update({kk: v for kk, v in passes["lds"][i][2].items() if kk.startswith("SQ_LDS")})
        gui = cv.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        busy = cv.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * SIMDS) if gui else 0.0
        clk = gui / dur if dur else 0.0  # cycles per ns = GHz
        mops = cv.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + cv.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        lc = cv.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(cv.get("SQ_LDS_IDX_ACTIVE", 0.0), 1.0)
        rb = wb = None
        if "ea_read" in passes and rd_fac:
            rb = rd_bytes(passes["ea_read"][i][2])[0] / rd_fac
        if "ea_write" in passes and wr_fac:
            wb = wr_bytes(passes["ea_write"][i][2]) / wr_fac
        recs[label] = {"us": dur / 1e3, "mfma_busy": busy, "clock_ghz": clk, "issued_flop": mops * 512,
                       "lds_conflict": lc, "read_bytes": rb, "write_bytes": wb}
        L.append(f"{label[:44]:<44s} {dur/1e3:8.1f} {100*busy:8.1f}% {clk:6.2f} {mops*512/1e12:12.1f} "
                 f"{100*lc:7.2f}% {'' if rb is None else f'{rb/1e9:8.3f}':>8s} "
                 f"{'' if wb is None else f'{wb/1e9:8.3f}':>8s}")
    if crd:
        b, other = rd_bytes(crd)
        L += ["", f"copy calibration (1 GiB read + 1 GiB written): read requests 32B {crd[rd_keys[1]]:.0f}, 64B "
              f"{crd[rd_keys[2]]:.0f}, 128B {crd[rd_keys[3]]:.0f}, unclassified {other:.0f}; write requests "
              f"{cwr[wr_keys[0]] if cwr else 0:.0f} ({cwr[wr_keys[1]] if cwr else 0:.0f} of 64B)"]
    rec = {"kernel_source_sha": kernel_source_hash(), "products": recs, "read_factor": rd_fac,
           "write_factor": wr_fac}
    L += ["", "record: " + json.dumps(rec)]
    os.makedirs(os.path.dirname(COUNTER_FILE), exist_ok=True)
    with open(COUNTER_FILE, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L))


def measured_counters():
    """The counter record of the products, or None when it is missing or the
    kernel sources changed since it was taken."""
    try:
        with open(COUNTER_FILE) as fh:
            rec = [ln for ln in fh if ln.startswith("record: ")]
        rec = json.loads(rec[-1][len("record: "):])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec


def measured_traffic():
    """Traffic bytes per launch from the committed record, or None when the
    record is missing or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = [ln for ln in fh if ln.startswith("record: ")]
        rec = json.loads(rec[-1][len("record: "):])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec


def cpu_baseline(cfg, inp, ntok, training=True):
    """The oracle (fp64 numpy) on the first ntok tokens: forward + backward,
    or the forward alone for a forward workload."""
    import numpy as np

    import synth
    from oracle import moe_oracle as O
    ntok = min(ntok, cfg.T)
    f = lambda a: synth.as_f64(a, cfg.dtype)  # noqa: E731
    w32 = lambda a: synth.bf16_bits_to_f32(a) if (a is not None and a.dtype == np.uint16) else a  # noqa: E731
    x = f(inp["x"][:ntok])
    wgu, wd = w32(inp["w_gateup"]), w32(inp["w_down"])
    sgu, sd = f(inp.get("s_gateup")), f(inp.get("s_down"))
    dy = f(inp["dy"][:ntok]) if training else None
    t0 = time.perf_counter()
    fw = O.forward(x, inp["w_router"], inp["bias"], wgu, wd, sgu, sd, top_k=cfg.k, score=cfg.score,
                   renorm=cfg.renorm)
    if training:
        O.backward(x, inp["w_router"], wgu, wd, sgu, sd, fw, dy, score=cfg.score, renorm=cfg.renorm)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    what = "forward+backward" if training else "forward"
    return {"value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "tokens": ntok,
            "sample": f"first {ntok} of {cfg.T} tokens of {cfg.name}, fp64 numpy {what}, "
                      f"{dt:.1f} s wall, BLAS threads = all {cores} host cores"}


def fp8_gate_up(M, cfg, x, saved, w, stream, timed_ms, flop, bf16_s, gather=True):
    """The forward gate/up product in fp8 (e4m3, row-wise scales) on the same
    permuted tokens and routing: the activation quantisation and the scaled
    fp8 grouped GEMM with the SwiGLU epilogue, each timed on its own with
    events (outside the layer step, which stays bf16)."""
    import torch
    A, d, E, f = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
    xq = torch.empty(A, d, dtype=torch.uint8, device="cuda")
    xs = torch.empty(A, dtype=torch.float32, device="cuda")
    wq = torch.empty(E * 2 * f, d, dtype=torch.uint8, device="cuda")
    ws = torch.empty(E * 2 * f, dtype=torch.float32, device="cuda")
    h = torch.empty(A, f, dtype=torch.bfloat16, device="cuda")
    aux = torch.empty(A, 2 * f, dtype=torch.bfloat16, device="cuda")
    M.moe_quantize_fp8(w["w_gateup"].reshape(E * 2 * f, d), wq, ws, stream)
    # the routed token rows (the fp8 product reads a permuted copy)
    x_perm = saved["x_perm"] if saved["x_perm"] is not None else x[saved["tok"].long()].contiguous()
    t_q = timed_ms(lambda: M.moe_quantize_fp8(x_perm, xq, xs, stream), 20) * 1e-3
    t_g = timed_ms(lambda: M.moe_grouped_gemm_fp8("swiglu", E, A, 2 * f, d, saved["offsets"], xq, xs, wq, ws,
                                                  h, aux, stream), 20) * 1e-3
    # the bf16 product on the same rows, timed the same way (20 back-to-back launches)
    if gather:
        t_b = timed_ms(lambda: M.moe_grouped_gemm_gather("NT", "swiglu", E, A, 2 * f, d, saved["offsets"], x,
                                                         w["w_gateup"], h, saved["tok"], cfg.T, aux, stream),
                       20) * 1e-3
    else:
        t_b = timed_ms(lambda: M.moe_grouped_gemm("NT", "swiglu", "bf16", E, A, 2 * f, d, saved["offsets"], x_perm,
                                                  w["w_gateup"], h, aux, None, stream), 20) * 1e-3
    tf = flop / t_g / 1e12
    q_bytes = A * (2 * d + d + 4)   # bf16 rows in; codes and scales out
    return {"gemm_us": t_g * 1e6, "tflops": tf, "frac": tf / PEAK_FP8_TFLOPS, "peak": PEAK_FP8_TFLOPS,
            "quantize_us": t_q * 1e6, "quantize_gbs": q_bytes / t_q / 1e9,
            "bf16_same_loop_us": t_b * 1e6, "speedup_same_loop_incl_quantize": t_b / (t_g + t_q),
            "speedup_vs_bf16_incl_quantize": bf16_s / (t_g + t_q),
            "what": "e4m3 row-wise scaled grouped GEMM + SwiGLU on the forward gate/up shape; "
                    "activation quantisation timed separately, weights quantised once"}


def fp8_gate_up_dgrad(M, cfg, saved, w, stream, timed_ms, flop, bf16_s):
    """The gate/up data gradient dX = dGU . W_gu in fp8 on the same routing:
    dGU (synthetic, N(0, 0.01^2), the layer's shape) quantised row-wise, W_gu
    quantised along its reduction dimension and stored transposed (once,
    outside the timing), the product on the forward-layout fp8 grouped GEMM;
    quantisation and product each timed on its own with events."""
    import torch
    A, d, E, f = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
    g = torch.Generator(device="cuda").manual_seed(11)
    dgu = (torch.randn(A, 2 * f, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    aq = torch.empty(A, 2 * f, dtype=torch.uint8, device="cuda")
    asc = torch.empty(A, dtype=torch.float32, device="cuda")
    wq = torch.empty(E, d, 2 * f, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, d, dtype=torch.float32, device="cuda")
    dx = torch.empty(A, d, dtype=torch.bfloat16, device="cuda")
    M.moe_quantize_fp8_transposed(w["w_gateup"].reshape(E, 2 * f, d), wq, wsc, stream)
    t_q = timed_ms(lambda: M.moe_quantize_fp8(dgu, aq, asc, stream), 20) * 1e-3
    t_g = timed_ms(lambda: M.moe_grouped_gemm_fp8("none", E, A, d, 2 * f, saved["offsets"], aq, asc, wq, wsc,
                                                  dx, None, stream), 20) * 1e-3
    # the bf16 product dX = dGU . W_gu on the same operands, timed the same way
    t_b = timed_ms(lambda: M.moe_grouped_gemm("NN", "none", "bf16", E, A, 2 * f, d, saved["offsets"], dgu,
                                              w["w_gateup"], dx, None, None, stream), 20) * 1e-3
    tf = flop / t_g / 1e12
    return {"gemm_us": t_g * 1e6, "tflops": tf, "frac": tf / PEAK_FP8_TFLOPS, "peak": PEAK_FP8_TFLOPS,
            "quantize_us": t_q * 1e6, "bf16_same_loop_us": t_b * 1e6,
            "speedup_same_loop_incl_quantize": t_b / (t_g + t_q),
            "speedup_vs_bf16_incl_quantize": bf16_s / (t_g + t_q),
            "what": "e4m3 gate/up data gradient (dGU row-wise, W_gu quantised along 2f and stored transposed "
                    "once) on the forward-layout fp8 grouped GEMM; dGU quantisation timed separately"}


def fp8_down_dgrad(M, cfg, saved, w, stream, timed_ms, flop, bf16_s):
    """The down projection's data gradient in fp8 with the dSwiGLU epilogue
    on the same routing: dY~ (synthetic, N(0, 0.2^2), the layer's shape)
    quantised row-wise, W_d quantised along d and stored transposed (once,
    outside the timing), the layer's own pre-activations G | U; quantisation
    and product each timed on its own with events."""
    import torch
    A, d, E, f = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
    g = torch.Generator(device="cuda").manual_seed(13)
    dyp = (torch.randn(A, d, device="cuda", generator=g) * 0.2).to(torch.bfloat16)
    aq = torch.empty(A, d, dtype=torch.uint8, device="cuda")
    asc = torch.empty(A, dtype=torch.float32, device="cuda")
    wq = torch.empty(E, f, d, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, f, dtype=torch.float32, device="cuda")
    dgu = torch.empty(A, 2 * f, dtype=torch.bfloat16, device="cuda")
    M.moe_quantize_fp8_transposed(w["w_down"].reshape(E, d, f), wq, wsc, stream)
    t_q = timed_ms(lambda: M.moe_quantize_fp8(dyp, aq, asc, stream), 20) * 1e-3
    t_g = timed_ms(lambda: M.moe_grouped_gemm_fp8("dswiglu", E, A, f, d, saved["offsets"], aq, asc, wq, wsc,
                                                  dgu, saved["preact"], stream), 20) * 1e-3
    # the bf16 product with the same epilogue on the same operands, timed the same way
    t_b = timed_ms(lambda: M.moe_grouped_gemm("NN", "dswiglu", "bf16", E, A, d, f, saved["offsets"], dyp,
                                              w["w_down"], dgu, saved["preact"], None, stream), 20) * 1e-3
    tf = flop / t_g / 1e12
    return {"gemm_us": t_g * 1e6, "tflops": tf, "frac": tf / PEAK_FP8_TFLOPS, "peak": PEAK_FP8_TFLOPS,
            "quantize_us": t_q * 1e6, "bf16_same_loop_us": t_b * 1e6,
            "speedup_same_loop_incl_quantize": t_b / (t_g + t_q),
            "speedup_vs_bf16_incl_quantize": bf16_s / (t_g + t_q),
            "what": "e4m3 down data gradient with the dSwiGLU epilogue (dY~ row-wise, W_d quantised along d and "
                    "stored transposed once) on the forward-layout fp8 grouped GEMM; dY~ quantisation timed "
                    "separately"}


def paired_flops(flops):
    """Stage flops when each routed weight gradient runs in one launch with
    its shared-expert counterpart (stages down_wgrad and gate_up_wgrad)."""
    fl = dict(flops)
    fl["down_wgrad"] += fl["shared_down_wgrad"]
    fl["gate_up_wgrad"] += fl["shared_gate_up_wgrad"]
    return fl


def fp8_layer(M, cfg, desc, w, x, dy, training, stream, steps, bf16_ms, flops, wgrad_fp8=False):
    """The whole layer through the fp8 calls (moe_forward_fp8 and, for a
    training workload, moe_backward_fp8) on the same inputs, timed like the
    bf16 step: a cache flush before each step, one event pair per step.  The
    e4m3 weight copies are written once per weight update and timed on their
    own; the step time excludes them, the second speedup includes them."""
    import torch

    w8 = M.alloc_fp8_weights(desc, backward=training)
    quant = lambda: M.moe_fp8_weights_quantize(desc, w, w8, True, training, stream)  # noqa: E731
    quant()
    saved = M.alloc_saved(desc, gather=True, training=training)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    grads = M.alloc_grads(desc) if training else None
    wsf = M.alloc_workspace(desc, "forward_fp8")
    wsb = M.alloc_workspace(desc, "backward_fp8_wgrad" if wgrad_fp8 else "backward_fp8") if training else None

    def step():
        M.moe_forward_fp8(desc, w, w8, x, y, saved, wsf, stream)
        if training:
            M.moe_backward_fp8(desc, w, w8, x, saved, dy, dx, grads, wsb, stream, wgrad_fp8=wgrad_fp8)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        flush_buf.fill_(1.0)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms = sum(step_ms) / len(step_ms)
    qa = torch.cuda.Event(enable_timing=True)
    qb = torch.cuda.Event(enable_timing=True)
    flush_buf.fill_(1.0)
    qa.record(stream)
    quant()
    qb.record(stream)
    torch.cuda.synchronize()
    q_ms = qa.elapsed_time(qb)
    del flush_buf
    M.stage_timing(True)
    for _ in range(min(steps, 5)):
        step()
    torch.cuda.synchronize()
    st = M.stage_times()
    M.stage_timing(False)
    stages = {}
    paired = (cfg.n_shared > 0 and training and st.get("shared_down_wgrad", (0.0, 0))[1] == 0)
    if paired:
        flops = paired_flops(flops)
    for name, (sms, n) in st.items():
        if n == 0:
            continue
        e = {"us": sms * 1e3 / n, "launches": n}
        if paired and name in ("down_wgrad", "gate_up_wgrad"):
            e["includes"] = "shared_" + name
        if name in flops and not name.startswith("router"):
            per = n // min(steps, 5)
            tf = flops[name] / (sms * 1e-3 / n) / 1e12 if per == 1 else None
            fp8_names = FP8_PRODUCTS + (FP8_WGRADS if wgrad_fp8 else ())
            if tf is not None and name in fp8_names:
                e.update(tflops=tf, frac_fp8=tf / PEAK_FP8_TFLOPS)
            elif tf is not None:
                e.update(tflops=tf, frac=tf / PEAK_BF16_TFLOPS)
        stages[name] = e
    progress(f"{cfg.name}: fp8 layer{' (fp8 weight gradients)' if wgrad_fp8 else ''} {ms:.3f} ms per step, "
             f"weight copies {q_ms:.3f} ms")
    return {
        "ms_per_step": ms, "tokens_per_s": cfg.T / (ms * 1e-3),
        "step_ms_min": min(step_ms), "step_ms_max": max(step_ms),
        "speedup_vs_bf16_step": bf16_ms / ms,
        "weight_copies_ms": q_ms,
        "speedup_incl_weight_copies": bf16_ms / (ms + q_ms),
        "stages": stages,
        "what": "moe_forward_fp8" + (" + moe_backward_fp8" if training else "") +
                ": e4m3 row-wise expert products (forward" + (" and both data gradients" if training else "") +
                (", and the weight gradients with operands quantised along each expert's rows" if wgrad_fp8
                 else "") + "), activations quantised in the step (stage fp8_quantize)" +
                ("" if wgrad_fp8 else ", bf16 weight gradients") + "; the e4m3 weight copies "
                "(moe_fp8_weights_quantize) are written once per weight update and timed separately "
                "(weight_copies_ms)",
    }


FP8_WGRADS = ("down_wgrad", "gate_up_wgrad", "shared_down_wgrad", "shared_gate_up_wgrad")
FP8_PRODUCTS = ("gate_up", "down", "shared_gate_up", "shared_down", "down_dgrad", "gate_up_dgrad",
                "shared_down_dgrad", "shared_gate_up_dgrad")


def run_config(args, cfg_name, cpu_tokens, pmc_probe=False):
    """One configuration: inputs resident in HBM, W warm-up steps, K timed
    steps (each after a cache flush, each timed with its own event pair),
    per-stage timing over separate steps, the dominant kernel's roofline and
    the oracle timed on a token sample.  Returns the result dict."""
    import numpy as np
    import torch

    import mixture_experts_layer_18_amd as M
    import synth

    cfg = synth.CONFIG_BY_NAME[cfg_name]
    training = cfg.backward
    progress(f"{cfg.name}: generating inputs")
    inp = synth.make_inputs(cfg, with_dy=training or pmc_probe)
    progress(f"{cfg.name}: inputs ready")

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    desc = M.desc_from_config(cfg)
    w = {k: dev(inp.get(k)) for k in ("w_router", "bias", "w_gateup", "w_down", "s_gateup", "s_down")}
    x = dev(inp["x"])
    dy = dev(inp.get("dy"))
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    # bf16 layers gather the token rows through the token map; the fp32 layer
    # (vector-ALU products) reads a permuted copy
    gather = not args.permuted_copy and cfg.dtype == "bf16"
    # a forward-only workload is an inference forward: no pre-activations kept
    saved = M.alloc_saved(desc, gather=gather, training=training or pmc_probe)
    grads = M.alloc_grads(desc) if (training or pmc_probe) else None
    wsf = M.alloc_workspace(desc, "forward")
    wsb = M.alloc_workspace(desc, "backward") if (training or pmc_probe) else None
    stream = torch.cuda.current_stream()

    terms = dict(aux_coeff=1e-3, seq_aux_coeff=1e-3, z_coeff=1e-3, seq_len=4096) if args.router_terms else None
    losses = torch.zeros(4, dtype=torch.float32, device="cuda") if args.router_terms else None

    def step():
        M.moe_forward(desc, w, x, y, saved, wsf, stream)
        if training:
            M.moe_backward(desc, w, x, saved, dy, dx, grads, wsb, stream, terms=terms, losses=losses)
            if args.router_terms and cfg.score == "sigmoid":
                M.moe_bias_update(desc, saved["counts"], 1e-3, w["bias"], stream)

    if pmc_probe:
        # one forward, a 1 GiB device copy (the counters' calibration), the
        # gate/up product alone, then one backward and the fp8 gate/up product
        # with its activation quantisation: every product of the layer is one
        # counted dispatch
        M.moe_forward(desc, w, x, y, saved, wsf, stream)
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        if gather:
            M.moe_grouped_gemm_gather("NT", "swiglu", cfg.E, cfg.T * cfg.k, 2 * cfg.f, cfg.d, saved["offsets"],
                                      x, w["w_gateup"], saved["h"], saved["tok"], cfg.T, saved["preact"],
                                      stream)
        else:
            M.moe_grouped_gemm("NT", "swiglu", cfg.dtype, cfg.E, cfg.T * cfg.k, 2 * cfg.f, cfg.d,
                               saved["offsets"], saved["x_perm"], w["w_gateup"], saved["h"],
                               saved["preact"], None, stream)
        torch.cuda.synchronize()
        M.moe_backward(desc, w, x, saved, dy, dx, grads, wsb, stream)
        torch.cuda.synchronize()
        if not args.no_fp8 and cfg.dtype == "bf16":
            A, d_, E_, f_ = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
            xq = torch.empty(A, d_, dtype=torch.uint8, device="cuda")
            xs = torch.empty(A, dtype=torch.float32, device="cuda")
            wq = torch.empty(E_ * 2 * f_, d_, dtype=torch.uint8, device="cuda")
            wsc = torch.empty(E_ * 2 * f_, dtype=torch.float32, device="cuda")
            M.moe_quantize_fp8(w["w_gateup"].reshape(E_ * 2 * f_, d_), wq, wsc, stream)
            xp = saved["x_perm"] if saved["x_perm"] is not None else x[saved["tok"].long()].contiguous()
            M.moe_quantize_fp8(xp, xq, xs, stream)
            M.moe_grouped_gemm_fp8("swiglu", E_, A, 2 * f_, d_, saved["offsets"], xq, xs, wq, wsc, saved["h"],
                                   saved["preact"], stream)
            torch.cuda.synchronize()
        print("pmc probe done", flush=True)
        return None

    # a 512 MiB buffer rewritten before each timed step (outside its events)
    # evicts the L2s (8 x 4 MB) and the 256 MB Infinity Cache, so no step
    # starts on operands the previous one left in cache
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: the library records a HIP event pair around the
    # roofline kernel's stage (gate/up) on the stream its kernels run on;
    # the other stages are timed in a separate pass below, so that their
    # event pairs do not sit in the headline steps (they cost ~1 %)
    M.stage_timing(True, stages=["gate_up"])
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        flush_buf.fill_(1.0)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed_stages = M.stage_times()
    M.stage_timing(False)
    step_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    progress(f"{cfg.name}: timed {args.steps} steps, {sum(step_ms) / len(step_ms):.3f} ms per step")
    ms_step = sum(step_ms) / len(step_ms)
    # the same step captured once in a HIP graph and replayed (each replay
    # after the same flush, its own event pair): the step without the host's
    # launch cost and the gaps between launches
    graph_ms = None
    if not args.router_terms:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            if training:
                M.moe_forward(desc, w, x, y, saved, wsf, cap)
                M.moe_backward(desc, w, x, saved, dy, dx, grads, wsb, cap)
            else:
                M.moe_forward(desc, w, x, y, saved, wsf, cap)
        torch.cuda.synchronize()
        gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for e0, e1 in gevs:
            flush_buf.fill_(1.0)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = sum(e0.elapsed_time(e1) for e0, e1 in gevs) / len(gevs)
        del graph
    del flush_buf
    # every stage, over separate steps after the timed region
    M.stage_timing(True)
    for _ in range(min(args.steps, 10)):
        step()
    torch.cuda.synchronize()
    stages = M.stage_times()
    M.stage_timing(False)
    stages["gate_up"] = timed_stages["gate_up"]
    tokens_per_s = cfg.T / (ms_step * 1e-3)
    T, d, E, k, f, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.n_shared * cfg.f_shared
    A = T * k
    es = 2 if cfg.dtype == "bf16" else 4     # bytes per activation / weight element
    counts = saved["counts"].cpu().numpy()
    # algorithmic work of one launch of each stage: flops of the products
    # (2 per multiply-add, no padding), bytes of the memory-bound stages with
    # each byte moved once
    flops = {
        "router": 2.0 * T * d * E, "router_wgrad": 2.0 * T * d * E,
        "gate_up": 2.0 * A * 2 * f * d, "down": 2.0 * A * d * f,
        "down_dgrad": 2.0 * A * d * f, "down_wgrad": 2.0 * A * d * f,
        "gate_up_wgrad": 2.0 * A * 2 * f * d, "gate_up_dgrad": 2.0 * A * 2 * f * d,
        "shared_gate_up": 2.0 * T * 2 * F * d, "shared_down": 2.0 * T * d * F,
        "shared_down_dgrad": 2.0 * T * d * F, "shared_down_wgrad": 2.0 * T * d * F,
        "shared_gate_up_wgrad": 2.0 * T * 2 * F * d, "shared_gate_up_dgrad": 2.0 * T * 2 * F * d,
    }
    sh = es * d if F else 0
    hbm_bytes = {
        "router": T * (es * d + 4 * E),                                # x in, logits out
        "router_wgrad": T * (es * d + 4 * E),                          # x, dlogits in
        "route": T * (4 * E + 8 * k),                                  # logits in; idx, gate out
        # idx in; pos, src, tok out (and with a permuted copy: x in, x_perm out)
        "permute": T * (16 * k + (0 if gather else es * d * (1 + k))),
        "combine": T * (es * d * (k + 1) + 8 * k + sh),                # y_perm, gate, pos, shared in; y out
        "combine_bwd": T * (es * d * (2 * k + 1) + 12 * k + 8 * E),    # dy, y_perm, gate, pos, idx, logits
                                                                       # in; dy_perm, dlogits out
        "unpermute_sum": T * (es * d * (k + 1) + 8 * k + 4 * E + sh),  # dx_perm, pos, idx, dlogits,
                                                                       # dx_shared in; dx out
    }
    def timed_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # the shared experts' weight gradients run inside the routed launches
    # when the two are paired (no shared weight-gradient stage of their own)
    paired = F > 0 and training and stages.get("shared_down_wgrad", (0.0, 0))[1] == 0
    fl_st = paired_flops(flops) if paired else flops
    stage_out = {}
    for name, (ms, n) in stages.items():
        if n == 0:
            continue
        us = ms * 1e3 / n
        e = {"us": us, "launches": n}
        if name in ("router", "router_wgrad") and cfg.dtype == "bf16":
            # the fp32 products on the bf16 matrix cores (three exact partial
            # products per term): bound by streaming x, rated against HBM
            e.update(tflops=flops[name] / (us * 1e-6) / 1e12)
        elif name in fl_st:
            tf = fl_st[name] / (us * 1e-6) / 1e12
            peak = PEAK_FP32_TFLOPS if (name.startswith("router") or cfg.dtype == "f32") else PEAK_BF16_TFLOPS
            e.update(tflops=tf, frac=tf / peak)
        if name in hbm_bytes:
            gbs = hbm_bytes[name] / (us * 1e-6) / 1e9
            e.update(gbs=gbs, frac=gbs / PEAK_HBM_GBS)
        if paired and name in ("down_wgrad", "gate_up_wgrad"):
            e["includes"] = "shared_" + name
        stage_out[name] = e
    t_gu = stage_out["gate_up"]["us"] * 1e-6
    t_dn = stage_out["down"]["us"] * 1e-6
    fl_gu, fl_dn = flops["gate_up"], flops["down"]
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    # each operand byte once: the token rows (x once when gathered, through
    # the int32 token map; else x_perm) and W_gateup read, preact (training
    # only) and h written
    algo_bytes = (es * ((T * d + 2 * A) if gather else A * d)
                  + es * (E * 2 * f * d + (A * 2 * f if training else 0) + A * f))
    ach = fl_gu / t_gu / 1e12
    main_cfg = cfg.name == "moe7b_bf16" and gather and not args.router_terms
    tr = measured_traffic() if main_cfg else None
    ctr = measured_counters() if main_cfg else None
    gu_ctr = (ctr or {}).get("products", {}).get("gate_up (alone, after the copy)")
    fwd_tflops = (fl_gu + fl_dn) / (t_gu + t_dn) / 1e12
    # practical HBM ceiling on this device: a 1 GiB streaming copy with the
    # streaming kernels' access pattern (moe_hbm_ceiling: 16-byte vectors,
    # nontemporal), and for reference a device-to-device hipMemcpy; read +
    # write bytes, timed with events on the same stream
    cbuf = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    cdst = torch.empty_like(cbuf)
    t_copy = timed_ms(lambda: M.hbm_ceiling(cbuf, cdst, stream), 10) * 1e-3
    copy_gbs = 2.0 * COPY_BYTES / t_copy / 1e9
    t_memcpy = timed_ms(lambda: cdst.copy_(cbuf), 10) * 1e-3
    memcpy_gbs = 2.0 * COPY_BYTES / t_memcpy / 1e9
    del cbuf, cdst
    # practical matrix-core ceiling on this device: each instruction kind
    # issued back to back on register operands (no memory traffic)
    ck_out = torch.zeros(4, dtype=torch.float32, device="cuda")
    mfma_ceiling = {}
    for kind in ("bf16_32x32x16", "bf16_16x16x32", "e4m3_32x32x64", "e4m3_16x16x128"):
        flop = [0.0]

        def run_ceiling():
            flop[0] = M.mfma_ceiling(kind, 3000, ck_out, stream)
        t_ck = timed_ms(run_ceiling, 3) * 1e-3
        mfma_ceiling[kind] = flop[0] / t_ck / 1e12
    del ck_out
    with_fp8 = not args.no_fp8 and cfg.dtype == "bf16" and training
    fp8 = fp8_gate_up(M, cfg, x, saved, w, stream, timed_ms, fl_gu, t_gu, gather) if with_fp8 else None
    fp8_dg = (fp8_gate_up_dgrad(M, cfg, saved, w, stream, timed_ms, flops["gate_up_dgrad"],
                                stage_out["gate_up_dgrad"]["us"] * 1e-6)
              if with_fp8 and "gate_up_dgrad" in stage_out else None)
    fp8_dd = (fp8_down_dgrad(M, cfg, saved, w, stream, timed_ms, flops["down_dgrad"],
                             stage_out["down_dgrad"]["us"] * 1e-6)
              if with_fp8 and "down_dgrad" in stage_out and saved.get("preact") is not None else None)
    fp8_ok = cfg.dtype == "bf16" and cfg.f % 128 == 0 and (cfg.n_shared * cfg.f_shared) % 128 == 0
    fp8_whole = (fp8_layer(M, cfg, desc, w, x, dy, training, stream, args.steps, ms_step, flops)
                 if not args.no_fp8 and fp8_ok else None)
    fp8_whole_w = (fp8_layer(M, cfg, desc, w, x, dy, training, stream, args.steps, ms_step, flops, wgrad_fp8=True)
                   if not args.no_fp8 and fp8_ok and training else None)
    # the streaming memory-bound stages (route and the index-only permute are
    # latency-bound at these sizes)
    hbm3 = [n for n in ("combine", "combine_bwd", "unpermute_sum") if n in stage_out]
    hbm3_us = sum(stage_out[n]["us"] for n in hbm3)
    hbm3_gbs = sum(hbm_bytes[n] for n in hbm3) / (hbm3_us * 1e-6) / 1e9
    # the routing front end: router logits, top-k and gates, permutation
    front = [n for n in ("router", "route", "permute") if n in stage_out]
    front_us = sum(stage_out[n]["us"] for n in front)
    front_bytes = sum(hbm_bytes[n] for n in front)
    pass_name = "fwd+bwd" if training else "fwd (inference: no pre-activations kept)"

    res = {
        "metric": METRIC if training else METRIC_FWD,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights, random init)",
        "config": {
            "workload": f"{cfg.name}: MoE layer {pass_name}, T={T} tokens, d_model={d}, E={E} experts, "
                        f"{cfg.score} top-{k}, expert d_ff={f}, {cfg.n_shared} shared experts d_ff="
                        f"{cfg.f_shared}",
            "tokens_per_step": T, "d_model": d, "experts": E, "top_k": k, "d_ff": f,
            "shared": f"{cfg.n_shared}x{cfg.f_shared}", "parallelism": "single GPU",
            "token_rows": "gathered through the token map" if gather else "permuted copy (x_perm)",
            "router_terms": terms,
        },
        "timing": {
            "method": "each timed step after a 512 MiB buffer write (L2 and Infinity Cache flush) outside its "
                      "own HIP event pair; value = tokens / mean step time; per-stage times from up to 10 "
                      "further steps with event pairs around every stage (the gate/up stage's from the timed "
                      "steps themselves)",
            "step_ms_min": min(step_ms), "step_ms_max": max(step_ms), "region_wall_s": wall,
            "graph_replay_ms_per_step": graph_ms,
            "graph_replay": "the same step captured once in a HIP graph (torch.cuda.CUDAGraph on a side stream) "
                            "and replayed, each replay after the same flush inside its own event pair",
        },
        "roofline": {
            "kernel": "gate/up grouped GEMM + SwiGLU (forward, NT)",
            "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
            "frac": ach / peak, "traffic": None if tr is None else tr["traffic_bytes"],
            "flop_per_launch": fl_gu, "avg_launch_us": t_gu * 1e6,
            "algorithmic_bytes_per_launch": algo_bytes,
            # from the committed counter record (rocprofv3 --pmc over --pmc-probe), null once the
            # kernel sources change: share of cycles the matrix cores were busy, and the shader clock
            "mfma_busy": None if gu_ctr is None else gu_ctr["mfma_busy"],
            "clock_ghz": None if gu_ctr is None else gu_ctr["clock_ghz"],
        },
        "grouped_gemm_fwd": {
            "tflops": fwd_tflops, "frac_of_peak": fwd_tflops / peak,
            "gate_up_us": t_gu * 1e6, "down_us": t_dn * 1e6,
        },
        "front_end": {"stages": front, "us": front_us, "gbs": front_bytes / (front_us * 1e-6) / 1e9},
        "combine_stages_hbm": {"stages": hbm3, "gbs": hbm3_gbs, "frac": hbm3_gbs / PEAK_HBM_GBS, "us": hbm3_us,
                               "frac_of_copy": hbm3_gbs / copy_gbs},
        "hbm_copy_ceiling": {"gbs": copy_gbs, "frac": copy_gbs / PEAK_HBM_GBS, "hipmemcpy_gbs": memcpy_gbs,
                             "what": "1 GiB streaming copy (moe_hbm_ceiling: 16-byte vectors, nontemporal loads and "
                                     "stores; read + write bytes), events on the same stream; hipmemcpy_gbs: the "
                                     "same bytes through a device-to-device hipMemcpy"},
        "mfma_ceiling": {"tflops": mfma_ceiling,
                         "gate_up_frac_of_ceiling": ach / mfma_ceiling["bf16_32x32x16"],
                         "what": "moe_mfma_ceiling: 2 workgroups per CU of 8 waves issuing independent MFMAs of "
                                 "one kind on register operands, no memory traffic; events over 3 launches"},
        "stages": stage_out,
        "fp8_layer": fp8_whole,
        "fp8_layer_fp8_weight_gradients": fp8_whole_w,
        "fp8_gate_up": fp8,
        "fp8_gate_up_dgrad": fp8_dg,
        "fp8_down_dgrad": fp8_dd,
        "loads": {"max_over_mean": float(counts.max() / counts.mean()), "empty": int((counts == 0).sum())},
    }
    if not args.no_cpu_baseline:
        progress(f"{cfg.name}: oracle on {min(cpu_tokens, cfg.T)} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, cpu_tokens, training)
    return res


ALL_CONFIGS_FILE = os.path.join(ROOT, "profiles", "all_configs_moe_layer.txt")
# oracle token samples of the all-configs run (about 10-30 s of host work each)
ALL_CONFIGS_CPU_TOKENS = {"tiny_fp32": 256, "finegrained_bf16": 4096, "moe7b_bf16": 2048, "skew_bf16": 2048,
                          "large_bf16": 256}


def all_configs(args):
    """Every layer of the scope's table, each with its own pass (forward for
    the forward workloads, forward + backward for the others): one JSON line
    per layer on stdout, then the table under profiles/."""
    import synth
    rows = []
    for c in synth.CONFIGS:
        print(f"[all-configs] {c.name}", file=sys.stderr, flush=True)
        r = run_config(args, c.name, ALL_CONFIGS_CPU_TOKENS.get(c.name, 256))
        rows.append(r)
        print(json.dumps(r), flush=True)
    write_all_configs(rows, args.steps, args.warmup)


def write_all_configs(rows, steps, warmup, log=None):
    L = ["The MoE layer on every configuration of the scope's table, one MI355X (bf16 products on the matrix",
         "cores; the fp32 layer on the vector ALUs), inputs resident in HBM, caches flushed before each timed step.",
         "", "Commands (from the repository root):",
         f"  python bench.py --all-configs --steps {steps} --warmup {warmup} > gpurun_out/bench_all.log",
         "  python bench.py --all-configs-summarize gpurun_out/bench_all.log", "",
         "gate/up = the routed gate/up grouped GEMM + SwiGLU, the dominant kernel (fraction of the 2.5 PFLOP/s bf16",
         "peak; fp32: of 157.3 TFLOP/s).  front end = router logits + top-k/gates + permutation.  combine stages =",
         "combine (+ combine backward and unpermute-sum with the backward), algorithmic bytes over their time.",
         "The forward workloads run an inference forward (no pre-activations kept).  oracle = the fp64 numpy",
         "oracle on a token sample of the same layer and pass, all host cores.", ""]
    L.append(f"{'layer':<18s} {'pass':<8s} {'ms/step':>9s} {'tokens/s':>11s} {'gate/up TF':>10s} {'frac':>6s} "
             f"{'front us':>9s} {'comb GB/s':>9s} {'oracle tok/s':>12s} {'sample':>7s} {'cores':>5s}")
    for r in rows:
        cb = r.get("cpu_baseline") or {}
        L.append(f"{r['config']['workload'].split(':')[0]:<18s} "
                 f"{'fwd+bwd' if 'fwd+bwd' in r['config']['workload'] else 'fwd':<8s} {r['ms_per_step']:9.3f} "
                 f"{r['value']:11.0f} {r['roofline']['achieved']:10.1f} {r['roofline']['frac']:6.3f} "
                 f"{r['front_end']['us']:9.1f} {r['combine_stages_hbm']['gbs']:9.0f} "
                 f"{cb.get('value', float('nan')):12.1f} {cb.get('tokens', 0):7d} {cb.get('cores', 0):5d}")
    L += ["", "The same layers through the fp8 calls (moe_forward_fp8 / moe_backward_fp8: e4m3 row-wise expert",
          "products in the forward and both data gradients, bf16 weight gradients; the e4m3 weight copies are",
          "written once per weight update and timed on their own).  Layers whose hidden widths are not multiples",
          "of 128, or fp32 layers, have no fp8 calls.", ""]
    L.append(f"{'layer':<18s} {'fp8 ms/step':>11s} {'tokens/s':>11s} {'vs bf16':>8s} {'weight copies ms':>16s} "
             f"{'activation quant us':>19s}")
    for r in rows:
        f8 = r.get("fp8_layer")
        if not f8:
            continue
        q = f8["stages"].get("fp8_quantize", {})
        steps_q = q.get("launches", 0)
        L.append(f"{r['config']['workload'].split(':')[0]:<18s} {f8['ms_per_step']:11.3f} {f8['tokens_per_s']:11.0f} "
                 f"{f8['speedup_vs_bf16_step']:8.2f} {f8['weight_copies_ms']:16.3f} "
                 f"{q.get('us', 0.0) * steps_q / max(1, min(steps, 5)):19.1f}")
    ck = rows[0].get("mfma_ceiling") if rows else None
    if ck:
        L += ["", "Matrix-core ceiling measured on the same box (moe_mfma_ceiling: independent MFMAs on register "
              "operands, no memory traffic), TFLOP/s: " +
              ", ".join(f"{k} {v:.0f}" for k, v in ck["tflops"].items())]
    names = [r["config"]["workload"].split(":")[0] for r in rows]
    stages = []
    for r in rows:
        stages += [n for n in r["stages"] if n not in stages]
    L += ["", "Per-stage mean time (us) and rate (TFLOP/s for products, GB/s of algorithmic bytes otherwise):", ""]
    L.append(f"{'stage':<22s}" + "".join(f"{n:>22s}" for n in names))
    for st in stages:
        cells = []
        for r in rows:
            e = r["stages"].get(st)
            if e is None:
                cells.append(f"{'-':>22s}")
                continue
            rate = f"{e['tflops']:.0f} TF" if "tflops" in e and "gbs" not in e else (
                f"{e['gbs']:.0f} GB/s" if "gbs" in e else "")
            cells.append(f"{e['us']:10.1f} {rate:>11s}")
        L.append(f"{st:<22s}" + "".join(cells))
    with open(ALL_CONFIGS_FILE, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L), file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.trace_summarize:
        trace_summarize(args.trace_summarize)
        return
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
        return
    if args.pmc_report:
        pmc_report(args.pmc_report)
        return
    if args.all_configs_summarize:
        with open(args.all_configs_summarize) as fh:
            rows = [json.loads(ln) for ln in fh if ln.startswith("{")]
        write_all_configs(rows, rows[0]["steps"], rows[0]["warmup"])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this MoE layer build has no multi-GPU path "
              "(expert-parallel sharding is described in DESIGN.md but not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mixture_experts_layer_18_amd import _lib
    _lib.load()
    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    if args.all_configs:
        all_configs(args)
        return
    res = run_config(args, args.config, args.cpu_tokens, pmc_probe=args.pmc_probe)
    if res is not None:
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
