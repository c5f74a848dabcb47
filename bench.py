"""Benchmark of the MoE-layer forward on one MI355X.

One step = one moe_layer_forward (route, permute, expert up/down GEMMs,
combine) over the workload's S tokens, inputs resident in HBM.  Prints ONE
JSON line on stdout: MoE-layer tokens/s at the Mixtral-shape prefill workload
(S=4096, d=4096, d_ff=14336, E=8, K=2, bf16; median of per-step HIP-event
times), the roofline of the dominant kernel, and the other workloads' legs:
the same layer under a per-expert capacity, the DeepSeek-shape fp8-weight
layer with bf16 and with e4m3 activations (per-product rooflines), the
decode workload's HBM fraction, the Zipf-skewed layer; and the CPU oracle's
rate on a bounded sample of every workload.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-decode] [--no-capacity] [--no-w8a8]
       python bench.py --pmc-probe [--workload NAME] [--act-quant]   (under rocprofv3 --pmc)
       python bench.py --pmc-summary FETCH_DIR WRITE_DIR [--workload NAME]
       python bench.py --pmc-mfma-summary DIR [--workload NAME]
       python bench.py --pmc-mem-summary L2_DIR L1_DIR [--workload NAME]
       python bench.py --trace-table KERNELS_SUMMARY_MD   (rocpd2summary markdown -> this library's rows)
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # dense MFMA, MI355X
PEAK_GBS = 8000.0                                             # HBM3E
METRIC = "MoE-layer tokens/s at Mixtral shape; % MFMA peak (prefill), % HBM BW (decode)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-capacity", action="store_true")
    ap.add_argument("--no-w8a8", action="store_true")
    ap.add_argument("--no-skew", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="only launch a 1 GiB copy and the expert GEMMs (for rocprofv3 --pmc passes)")
    ap.add_argument("--act-quant", action="store_true",
                    help="with --pmc-probe: the fp8-activation (W8A8) products of the workload")
    ap.add_argument("--pmc-mfma-summary", metavar="DIR",
                    help="write profiles/mfma_*.md from a rocprofv3 --pmc pass over the MFMA counters")
    ap.add_argument("--trace-table", metavar="KERNELS_SUMMARY_MD",
                    help="print the rows of this library's kernels from a rocpd2summary kernel table")
    ap.add_argument("--pmc-mem-summary", nargs=2, metavar=("L2_DIR", "L1_DIR"),
                    help="write profiles/memory_path_*.md from the two memory-path counter passes")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_*.md from two rocprofv3 --pmc output directories")
    return ap.parse_args()


class Workload:
    """Device inputs, outputs and stage buffers of one configuration."""

    def __init__(self, cfg, D, M, torch):
        self.cfg, self.M, self.torch = cfg, M, torch
        dev = "cuda"
        t0 = time.time()
        self.inp = D.make_inputs(cfg, dev)
        torch.cuda.synchronize()
        log(f"[bench] {cfg.name}: inputs generated in {time.time() - t0:.1f}s")
        c = cfg
        self.p = M.make_problem(c.S, c.d, c.d_ff, c.E, c.K, c.act, c.w, c.n_groups, c.topk_groups, c.renormalize)
        act = torch.bfloat16 if c.act == "bf16" else torch.float32
        cap = M.moe_rows_capacity(self.p)
        i32 = dict(dtype=torch.int32, device=dev)
        self.y = torch.empty((c.S, c.d), dtype=act, device=dev)
        self.ws = M.workspace(self.p, M.STAGE_LAYER, dev)
        self.counts = torch.empty(c.E, **i32)
        # stage buffers
        self.idx = torch.empty((c.S, c.K), **i32)
        self.gate = torch.empty((c.S, c.K), dtype=torch.float32, device=dev)
        self.ws_route = M.workspace(self.p, M.STAGE_ROUTE, dev)
        self.ws_perm = M.workspace(self.p, M.STAGE_PERMUTE, dev)
        self.ws_ffn = M.workspace(self.p, M.STAGE_EXPERT_FFN, dev)
        self.offsets = torch.empty(c.E + 1, **i32)
        self.perm = torch.empty(c.S * c.K, **i32)
        self.inv = torch.empty(c.S * c.K, **i32)
        self.x_perm = torch.empty((cap, c.d), dtype=act, device=dev)
        self.h = torch.empty((cap, c.d_ff), dtype=act, device=dev)
        self.y_perm = torch.empty((cap, c.d), dtype=act, device=dev)
        self.y2 = torch.empty((c.S, c.d), dtype=act, device=dev)

    def layer(self):
        i, M = self.inp, self.M
        M.moe_layer_forward(self.p, i["x"], i["W_r"], i["W1"], i["b1"], i["W2"], i["b2"], i["router_bias"],
                            i["select_bias"], i["w1_scale"], i["w2_scale"], y=self.y,
                            expert_counts_out=self.counts, ws=self.ws)

    def stages(self):
        i, M, p = self.inp, self.M, self.p
        return {
            "route": lambda: M.moe_route(p, i["x"], i["W_r"], i["router_bias"], i["select_bias"],
                                         topk_idx=self.idx, topk_gate=self.gate, ws=self.ws_route),
            "permute": lambda: M.moe_permute(p, self.idx, i["x"], self.counts, self.offsets, self.perm,
                                             self.inv, self.x_perm, ws=self.ws_perm),
            "expert_up": lambda: M.moe_expert_up(p, self.x_perm, self.counts, self.offsets, i["W1"], i["b1"],
                                                 i["w1_scale"], h=self.h, ws=self.ws_ffn),
            "expert_down": lambda: M.moe_expert_down(p, self.h, self.counts, self.offsets, i["W2"], i["b2"],
                                                     i["w2_scale"], y_perm=self.y_perm, ws=self.ws_ffn),
            "combine": lambda: M.moe_combine(p, self.y_perm, self.inv, self.gate, y=self.y2),
        }


def time_calls(torch, fn, steps, warmup):
    """(mean, median) ms per call.  HIP events are recorded on the stream the
    library launches on (torch's current stream) between back-to-back calls,
    so each call's duration is the gap between two events and the durations
    add up to the whole timed region."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return sum(per) / steps, statistics.median(per)


def algorithmic(cfg, touched, a8=False):
    """Per-launch algorithmic flops and HBM bytes of the two expert GEMMs.

    Flops count only the S*K routed rows (no padding).  Bytes: each touched
    expert's weights (+ fp8 scales) and biases once, the routed activation
    rows in and out once (with fp8 activations, a8: e4m3 rows plus a float32
    scale per row in, bf16 out)."""
    a = 2 if cfg.act == "bf16" else 4
    a_in = 1 if a8 else a
    row_sc = 4 if a8 else 0
    w = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.w]
    rows = cfg.S * cfg.K
    fl = 2.0 * rows * cfg.d * cfg.d_ff
    sc = 4 if cfg.w == "fp8" else 0
    up = touched * (cfg.d * cfg.d_ff * w + cfg.d_ff * (a + sc)) + rows * (cfg.d * a_in + row_sc + cfg.d_ff * a)
    down = touched * (cfg.d_ff * cfg.d * w + cfg.d * (a + sc)) + rows * (cfg.d_ff * a_in + row_sc + cfg.d * a)
    return {"expert_up": (fl, up), "expert_down": (fl, down)}


def gemm_source_hash():
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "sparse_ffn_layer_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_path(kernel, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")


def traffic_for(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    path = traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            vals[k.strip("`")] = v.strip().strip("`")
    if vals.get("source_hash") != gemm_source_hash():
        return None
    try:
        return int(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_PROBE_BYTES = 1 << 30   # plain device copy of known size: scales the HBM counters


def pmc_probe(a, D, M, torch):
    """Launch only what the counter passes need: a plain 1 GiB device copy
    (three times) and the workload's two expert GEMM stages (three times
    each; with --act-quant the W8A8 products on rows quantised per row), so
    the counters per dispatch can be read off."""
    cfg = D.CONFIGS[a.workload]
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = Workload(cfg, D, M, torch)
    st = w.stages()
    st["route"]()
    st["permute"]()
    torch.cuda.synchronize()
    if a.act_quant:
        i = w.inp
        p8 = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                            cfg.renormalize, 1.0, 0, 1)
        x8, xs = M.moe_quantize_rows(w.x_perm)
        st["expert_up"]()
        h8, hs = M.moe_quantize_rows(w.h)
        for _ in range(3):
            M.moe_expert_up_a8(p8, x8, xs, w.counts, w.offsets, i["W1"], i["b1"], i["w1_scale"], h=w.h, ws=w.ws_ffn)
            M.moe_expert_down_a8(p8, h8, hs, w.counts, w.offsets, i["W2"], i["b2"], i["w2_scale"], y_perm=w.y_perm,
                                 ws=w.ws_ffn)
    else:
        for _ in range(3):
            st["expert_up"]()
            st["expert_down"]()
    torch.cuda.synchronize()
    log(f"[bench] pmc probe done: {cfg.name}{' (W8A8)' if a.act_quant else ''}")


def gemm_kernel_stage(k):
    """(stage, fp8 activations?) of an expert GEMM kernel name, or None.  The
    epilogue (0: bias + GeLU = expert_up, 1: bias = expert_down) is the only
    template argument of the eight-wave kernel and the eighth of the general
    one, whose eleventh says whether the activations are e4m3."""
    if "grouped_gemm_bf16" not in k or "fixup" in k or "<" not in k:
        return None
    args = [x.strip() for x in k.split("<", 1)[1].split(">", 1)[0].split(",")]
    epi = args[0] if "_w8_kernel" in k else args[7]
    if epi not in ("0", "1"):
        return None
    a8 = len(args) > 10 and args[10] == "true"
    return ("expert_up" if epi == "0" else "expert_down"), a8


def pmc_summary(a):
    """Turn the two counter passes (rocprofv3 --pmc FETCH_SIZE, then
    WRITE_SIZE, csv output) into profiles/traffic_<stage>_<workload>.md."""
    import csv
    import statistics

    def read(d):
        rows = []
        for root, _, files in os.walk(d):
            for f in files:
                if f.endswith("counter_collection.csv"):
                    rows += list(csv.DictReader(open(os.path.join(root, f))))
        return rows

    fetch, write = read(a.pmc_summary[0]), read(a.pmc_summary[1])

    def per_kernel(rows, counter):
        out = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fk, wk = per_kernel(fetch, "FETCH_SIZE"), per_kernel(write, "WRITE_SIZE")
    # the probe's three 1 GiB copies are by far the largest copy dispatches of
    # the run; each reads and writes COPY_PROBE_BYTES
    ck = next(k for k in fk if "copy" in k.lower() and len(fk[k]) >= 3
              and max(fk[k]) * 1024 > COPY_PROBE_BYTES / 4)
    f_scale = statistics.median(sorted(fk[ck])[-3:]) * 1024 / COPY_PROBE_BYTES
    w_scale = statistics.median(sorted(wk[ck])[-3:]) * 1024 / COPY_PROBE_BYTES
    stages = {}
    for k in fk:
        sa = gemm_kernel_stage(k)
        if sa is not None and len(fk[k]) >= 3:   # the probe launches each product three times
            stages[sa] = k
    for (stage, a8), k in stages.items():
        cfg_name = a.workload + ("_w8a8" if a8 else "")
        probe = " --act-quant" if a8 else ""
        fb = statistics.median(fk[k]) * 1024 / f_scale
        wb = statistics.median(wk[k]) * 1024 / w_scale
        path = traffic_path(stage, cfg_name)
        with open(path, "w") as f:
            f.write(f"# HBM traffic: `{stage}` GEMM, {cfg_name} workload\n\n")
            f.write("Commands (one MI355X, repository root; two counter passes, then this summary):\n\n```\n")
            f.write(f"rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o f --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {a.workload}{probe}\n")
            f.write(f"rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o w --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {a.workload}{probe}\n")
            f.write(f"python bench.py --workload {a.workload} --pmc-summary gpurun_out/pmc_fetch "
                    f"gpurun_out/pmc_write\n```\n\n")
            f.write(f"Kernel: `{k}` ({len(fk[k])} dispatches, median per dispatch).\n\n")
            f.write("| counter | raw (KiB per dispatch) | plain-copy scale (counter bytes / true bytes) | HBM bytes per launch |\n")
            f.write("|:--|--:|--:|--:|\n")
            f.write(f"| FETCH_SIZE | {statistics.median(fk[k]):.0f} | {f_scale:.4f} | {fb:.4g} |\n")
            f.write(f"| WRITE_SIZE | {statistics.median(wk[k]):.0f} | {w_scale:.4f} | {wb:.4g} |\n\n")
            f.write(f"The scale comes from a plain {COPY_PROBE_BYTES >> 20} MiB device copy in the same run "
                    f"(`{ck[:60]}`), which reads and writes exactly that many bytes.\n\n")
            f.write(f"- bytes_per_launch: {int(round(fb + wb))}\n")
            f.write(f"- fetch_bytes: {int(round(fb))}\n")
            f.write(f"- write_bytes: {int(round(wb))}\n")
            f.write(f"- source_hash: {gemm_source_hash()}\n")
        log(f"[bench] wrote {path}")


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE"  # one pass
MFMA_COUNTERS_F8 = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE"


def pmc_mfma_summary(a):
    """Turn one rocprofv3 --pmc pass over MFMA_COUNTERS (or MFMA_COUNTERS_F8
    for the fp8-activation products; csv output) into
    profiles/mfma_<stage>_<workload>.md: per expert GEMM dispatch, the MFMA
    busy fraction of all SIMDs, the shader clock, and the MFMA work executed
    (padding rows included) against the algorithmic work."""
    import csv
    import statistics

    rows = []
    for root, _, files in os.walk(a.pmc_mfma_summary):
        for f in files:
            if f.endswith("counter_collection.csv"):
                rows += list(csv.DictReader(open(os.path.join(root, f))))
    disp = {}
    for r in rows:
        k = r["Kernel_Name"]
        if gemm_kernel_stage(k) is None:
            continue
        d = disp.setdefault((k, r["Dispatch_Id"]), {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    import datagen as D
    cfg = D.CONFIGS[a.workload]
    alg = 2.0 * cfg.S * cfg.K * cfg.d * cfg.d_ff
    cus, simds, xccs = 256, 4, 8
    kernels = {}
    for (k, _), d in disp.items():
        kernels.setdefault(k, []).append(d)
    for k, ds in kernels.items():
        if len(ds) < 3:
            continue
        stage, a8 = gemm_kernel_stage(k)
        mops = next((c for c in ds[0] if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")), None)
        if mops is None:
            continue
        dt = mops.rsplit("_", 1)[1].lower()
        cfg_name = a.workload + ("_w8a8" if a8 else "")
        counters = MFMA_COUNTERS_F8 if a8 else MFMA_COUNTERS
        probe = " --act-quant" if a8 else ""
        peak = PEAK_TFLOPS["fp8" if a8 else "bf16"]
        med = lambda f: statistics.median(f(d) for d in ds)
        ghz = med(lambda d: d["GRBM_GUI_ACTIVE"] / xccs / d["ns"])
        busy = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / xccs * cus * simds))
        flops = med(lambda d: d[mops] * 512)
        ms = med(lambda d: d["ns"]) / 1e6
        path = os.path.join(ROOT, "profiles", f"mfma_{stage}_{cfg_name}.md")
        with open(path, "w") as f:
            f.write(f"# MFMA utilisation: `{stage}` GEMM, {cfg_name} workload\n\n")
            f.write("Commands (one MI355X, repository root; one counter pass, then this summary):\n\n```\n")
            f.write(f"rocprofv3 --pmc {counters} -d gpurun_out/pmc_mfma -o m --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {a.workload}{probe}\n")
            f.write(f"python bench.py --workload {a.workload} --pmc-mfma-summary gpurun_out/pmc_mfma\n```\n\n")
            f.write(f"Kernel: `{k}` ({len(ds)} dispatches, medians).  Counters are summed over the {xccs} XCCs "
                    f"and their SIMDs; shader cycles = GRBM_GUI_ACTIVE / {xccs}.\n\n")
            f.write("| quantity | value |\n|:--|--:|\n")
            f.write(f"| dispatch duration under counter collection | {ms:.3f} ms |\n")
            f.write(f"| shader clock (cycles / duration) | {ghz:.2f} GHz |\n")
            f.write(f"| MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {cus} CUs x {simds} SIMDs) | {100 * busy:.1f} % |\n")
            f.write(f"| {dt} MFMA work executed: 512 {mops} | {flops:.4g} flop |\n")
            f.write(f"| algorithmic work (2 d d_ff per routed row) | {alg:.4g} flop |\n")
            f.write(f"| executed / algorithmic (padding rows of partly filled tiles) | {flops / alg:.3f} |\n")
            f.write(f"| executed rate during the dispatch | {flops / (ms / 1e3) / 1e12:.0f} TFLOP/s |\n")
            f.write(f"| dense {'fp8' if a8 else 'bf16'} peak at the measured clock ({ghz:.2f} / 2.4 x "
                    f"{peak / 1000:.1f} PFLOP/s) | {peak * ghz / 2.4:.0f} TFLOP/s |\n\n")
            f.write(f"The fraction of the {peak / 1000:.1f} PFLOP/s peak that the algorithmic work reaches factors as "
                    "MFMA busy x (clock / 2.4 GHz) / (executed / algorithmic): "
                    f"{busy:.3f} x {ghz / 2.4:.3f} / {flops / alg:.3f} = {busy * ghz / 2.4 / (flops / alg):.3f} under "
                    "counter collection (the bench line's figure comes from uninstrumented launches, at a clock "
                    "that varies from box to box).\n\n")
            f.write(f"- source_hash: {gemm_source_hash()}\n")
        log(f"[bench] wrote {path}")


def trace_table(path):
    """The library's kernels (namespace sfl) from a rocpd2summary markdown
    kernel table (durations in ns), as a markdown table in microseconds,
    longest total time first."""
    import re
    rows = []
    for line in open(path):
        if "sfl::" not in line:
            continue
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        name = re.sub(r"\(.*$", "", re.sub(r"^void ", "", cells[0]))
        rows.append((float(cells[2]), name, int(cells[1]), float(cells[3]) / 1e3, float(cells[5]) / 1e3,
                     float(cells[6]) / 1e3))
    rows.sort(reverse=True)
    print("| kernel | calls | avg (us) | min (us) | max (us) |\n|:--|--:|--:|--:|--:|")
    for _, n, c, avg, mn, mx in rows:
        print(f"| `{n}` | {c} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")


MEM_COUNTERS_L2 = "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE"
MEM_COUNTERS_L1 = "TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum GRBM_GUI_ACTIVE"


def pmc_mem_summary(a):
    """Turn two rocprofv3 --pmc passes (MEM_COUNTERS_L2, then MEM_COUNTERS_L1;
    csv output) into profiles/memory_path_<stage>_<workload>.md: per expert
    GEMM, the L2 hit rate, the memory reads behind L2 (count, latency, how
    many are in flight on average) and the L1 -> L2 read requests (latency
    and the average in flight per CU, by Little's law: summed latency over
    elapsed cycles)."""
    import csv
    import statistics

    def read(d):
        disp = {}
        for root, _, files in os.walk(d):
            for f in files:
                if not f.endswith("counter_collection.csv"):
                    continue
                for r in csv.DictReader(open(os.path.join(root, f))):
                    k = r["Kernel_Name"]
                    if gemm_kernel_stage(k) is None:
                        continue
                    e = disp.setdefault(k, {}).setdefault(r["Dispatch_Id"], {
                        "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                    e[r["Counter_Name"]] = float(r["Counter_Value"])
        return disp

    l2, l1 = read(a.pmc_mem_summary[0]), read(a.pmc_mem_summary[1])
    cus, xccs = 256, 8
    for k in l2:
        if k not in l1 or len(l2[k]) < 3 or len(l1[k]) < 3:
            continue
        stage, a8 = gemm_kernel_stage(k)
        cfg_name = a.workload + ("_w8a8" if a8 else "")
        probe = " --act-quant" if a8 else ""
        A, B = list(l2[k].values()), list(l1[k].values())
        med = lambda ds, f: statistics.median(f(d) for d in ds)
        cyc = lambda d: d["GRBM_GUI_ACTIVE"] / xccs
        ms = med(A, lambda d: d["ns"]) / 1e6
        ghz = med(A, lambda d: cyc(d) / d["ns"])
        hit = med(A, lambda d: d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] + d["TCC_MISS_sum"]))
        rd = med(A, lambda d: d["TCC_EA0_RDREQ_sum"])
        rd_lat = med(A, lambda d: d["TCC_EA0_RDREQ_LEVEL_sum"] / d["TCC_EA0_RDREQ_sum"])
        rd_fly = med(A, lambda d: d["TCC_EA0_RDREQ_LEVEL_sum"] / cyc(d))
        rd_rate = med(A, lambda d: d["TCC_EA0_RDREQ_sum"] * 128 / (d["ns"] * 1e-9) / 1e12)
        q = med(B, lambda d: d["TCP_TCC_READ_REQ_sum"])
        q_lat = med(B, lambda d: d["TCP_TCC_READ_REQ_LATENCY_sum"] / d["TCP_TCC_READ_REQ_sum"])
        q_fly = med(B, lambda d: d["TCP_TCC_READ_REQ_LATENCY_sum"] / cyc(d) / cus)
        pend = med(B, lambda d: d["TCP_PENDING_STALL_CYCLES_sum"] / cyc(d) / cus)
        path = os.path.join(ROOT, "profiles", f"memory_path_{stage}_{cfg_name}.md")
        with open(path, "w") as f:
            f.write(f"# Memory path: `{stage}` GEMM, {cfg_name} workload\n\n")
            f.write("Commands (one MI355X, repository root; two counter passes, then this summary):\n\n```\n")
            f.write(f"rocprofv3 --pmc {MEM_COUNTERS_L2} -d gpurun_out/pmc_l2 -o a --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {a.workload}{probe}\n")
            f.write(f"rocprofv3 --pmc {MEM_COUNTERS_L1} -d gpurun_out/pmc_l1 -o b --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {a.workload}{probe}\n")
            f.write(f"python bench.py --workload {a.workload} --pmc-mem-summary gpurun_out/pmc_l2 gpurun_out/pmc_l1\n"
                    "```\n\n")
            f.write(f"Kernel: `{k}` ({len(A)} dispatches, medians).  Cycles = GRBM_GUI_ACTIVE / {xccs} "
                    f"(summed over the XCCs); {cus} CUs.\n\n")
            f.write("| quantity | value |\n|:--|--:|\n")
            f.write(f"| dispatch duration under counter collection | {ms:.3f} ms |\n")
            f.write(f"| shader clock | {ghz:.2f} GHz |\n")
            f.write(f"| L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS) | {100 * hit:.1f} % |\n")
            f.write(f"| memory reads behind L2: TCC_EA0_RDREQ | {rd:.4g} |\n")
            f.write(f"| their rate at 128 B each | {rd_rate:.2f} TB/s |\n")
            f.write(f"| memory read latency: TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ | {rd_lat:.0f} cycles |\n")
            f.write(f"| memory reads in flight on average: TCC_EA0_RDREQ_LEVEL / cycles | {rd_fly:.0f} |\n")
            f.write(f"| L1 -> L2 read requests: TCP_TCC_READ_REQ | {q:.4g} |\n")
            f.write(f"| L1 -> L2 read latency: TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ | {q_lat:.0f} cycles |\n")
            f.write(f"| L1 -> L2 reads in flight per CU: TCP_TCC_READ_REQ_LATENCY / cycles / {cus} | {q_fly:.1f} |\n")
            f.write(f"| L1 cycles stalled on pending L2 reads: TCP_PENDING_STALL_CYCLES / cycles / {cus} | "
                    f"{100 * pend:.0f} % |\n\n")
            f.write(f"- source_hash: {gemm_source_hash()}\n")
        log(f"[bench] wrote {path}")


def roofline(cfg, stage_ms, touched, workload, kernel=None, a8=False):
    """Roofline of one expert GEMM (the slower of the two unless `kernel` is
    named): algorithmic work per launch over its average launch duration,
    against the dense MFMA peak of its operand type or the HBM peak,
    whichever its arithmetic intensity makes binding."""
    alg = algorithmic(cfg, touched, a8)
    name = kernel or max(("expert_up", "expert_down"), key=lambda k: stage_ms[k])
    fl, by = alg[name]
    sec = stage_ms[name] / 1e3
    intensity = fl / by
    peak_f = PEAK_TFLOPS["fp8" if a8 else ("bf16" if cfg.act == "bf16" else "f32")]
    ridge = peak_f * 1e12 / (PEAK_GBS * 1e9)
    if intensity >= ridge:
        ach, peak, unit, bound = fl / sec / 1e12, peak_f, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = by / sec / 1e9, PEAK_GBS, "GB/s", "hbm"
    return {"kernel": name, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic_for(name, workload),
            "avg_launch_ms": round(stage_ms[name], 4), "algorithmic_flops": fl, "algorithmic_bytes": by,
            "mfma_frac": round(fl / sec / (peak_f * 1e12), 4), "hbm_frac": round(by / sec / (PEAK_GBS * 1e9), 4)}


def layer_fractions(cfg, ms, touched, mfma_dtype):
    """Layer-level fractions of the two roofs: algorithmic layer flops
    (4 S K d d_ff + 2 S d E) over the step time against the dense MFMA peak
    of mfma_dtype, and algorithmic layer bytes (x and y once, W_r, and every
    touched expert's weights, scales and biases once) against the HBM peak."""
    a = 2 if cfg.act == "bf16" else 4
    w = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.w]
    sc = 4 if cfg.w == "fp8" else 0
    fl = 4.0 * cfg.S * cfg.K * cfg.d * cfg.d_ff + 2.0 * cfg.S * cfg.d * cfg.E
    by = (2 * cfg.S * cfg.d * a + cfg.E * cfg.d * a
          + touched * (2 * cfg.d * cfg.d_ff * w + (cfg.d + cfg.d_ff) * (a + sc)))
    sec = ms / 1e3
    return {"algorithmic_flops": fl, "algorithmic_bytes": by,
            "mfma_frac": round(fl / sec / (PEAK_TFLOPS[mfma_dtype] * 1e12), 4), "mfma_peak_dtype": mfma_dtype,
            "hbm_frac": round(by / sec / (PEAK_GBS * 1e9), 4)}


def run_workload(name, steps, warmup, D, M, torch):
    """The layer step (mean and median ms) and each stage's mean and median
    launch time; the expert counts of the step."""
    cfg = D.CONFIGS[name]
    w = Workload(cfg, D, M, torch)
    ms, ms_med = time_calls(torch, w.layer, steps, warmup)
    counts = w.counts.cpu()
    touched = int((counts > 0).sum())
    st = {k: time_calls(torch, fn, steps, max(2, warmup // 2)) for k, fn in w.stages().items()}
    return cfg, w, (ms, ms_med), st, touched, counts


def stage_dicts(st):
    return ({k: v[0] for k, v in st.items()}, {k: round(v[1], 4) for k, v in st.items()})


def context_leg(w, torch, counts):
    """Context for the roofline, on the same box in the same run (never the
    measured figure): a plain 1 GiB device copy, and the vendor library's
    GEMM (torch.matmul -> hipBLASLt) on the expert-up work of the workload --
    once as one dense product over all routed rows, once as one product per
    expert at the routed counts, the library's way to run the same grouped
    work."""
    c = w.cfg
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    copy_ms = time_calls(torch, lambda: dst.copy_(src), 10, 3)[0]
    del src, dst
    gen = torch.Generator(device="cuda").manual_seed(0)
    rows = int(sum(int(n) for n in counts))
    # weights in the layout the expert products read them, [d_ff][d] (a
    # linear layer's [out][in]); a plain 2-D product with the transposed view
    a = torch.randn((rows, c.d), device="cuda", generator=gen).to(torch.bfloat16)
    wt = torch.randn((c.d_ff, c.d), device="cuda", generator=gen).to(torch.bfloat16)
    dense_ms = time_calls(torch, lambda: torch.mm(a, wt.t()), 10, 3)[0]
    ws = [torch.randn((c.d_ff, c.d), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(c.E)]
    offs = [0]
    for n in counts:
        offs.append(offs[-1] + int(n))

    def per_expert():
        for e in range(c.E):
            if offs[e + 1] > offs[e]:
                torch.mm(a[offs[e]:offs[e + 1]], ws[e].t())

    grouped_ms = time_calls(torch, per_expert, 10, 3)[0]
    fl = 2.0 * rows * c.d * c.d_ff
    out = {"copy_GBps_read_plus_write": round(2 * COPY_PROBE_BYTES / (copy_ms / 1e3) / 1e9, 1),
           "hipblaslt_dense_up_TFLOPs": round(fl / (dense_ms / 1e3) / 1e12, 1),
           "hipblaslt_per_expert_up_TFLOPs": round(fl / (grouped_ms / 1e3) / 1e12, 1),
           "rows": rows, "shape": f"[{rows} x {c.d}] x [{c.d} x {c.d_ff}] bf16"}
    del a, wt, ws
    torch.cuda.empty_cache()
    return out


def graph_leg(w, torch, steps, warmup):
    """The layer captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed: the same launches without the host's per-launch cost.  A
    separate figure, never the headline."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w.layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w.layer()
    ms, med = time_calls(torch, g.replay, steps, warmup)
    return {"ms_per_step": round(med, 4), "ms_per_step_mean": round(ms, 4),
            "tokens_per_s": round(w.cfg.S / (med / 1e3), 1)}


def capacity_leg(w, M, torch, factor, steps):
    """The workload with each expert limited to factor * S*K/E pairs: the
    layer step with the limit, and moe_apply_capacity alone on the routed
    indices (restored before every call, outside the timed region)."""
    c, i = w.cfg, w.inp
    cap = max(1, int(factor * c.S * c.K / c.E))
    p = M.make_problem(c.S, c.d, c.d_ff, c.E, c.K, c.act, c.w, c.n_groups, c.topk_groups, c.renormalize,
                       1.0, cap)
    ws = M.workspace(p, M.STAGE_LAYER, "cuda")
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    logits = torch.empty((c.S, c.E), dtype=torch.float32, device="cuda")
    y = torch.empty_like(w.y)

    def layer():
        M.moe_layer_forward(p, i["x"], i["W_r"], i["W1"], i["b1"], i["W2"], i["b2"], i["router_bias"],
                            i["select_bias"], i["w1_scale"], i["w2_scale"], y=y, expert_counts_out=counts,
                            logits_out=logits, ws=ws)

    layer_ms, layer_med = time_calls(torch, layer, steps, 3)
    M.moe_route(w.p, i["x"], i["W_r"], i["router_bias"], i["select_bias"], topk_idx=w.idx, topk_gate=w.gate,
                ws=w.ws_route)
    idx0 = w.idx.clone()
    ws_c = M.workspace(p, M.STAGE_CAPACITY, "cuda")
    dropped = torch.zeros(4, dtype=torch.int32, device="cuda")
    evs = []
    for k in range(steps + 3):
        w.idx.copy_(idx0)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        M.moe_apply_capacity(p, logits, w.idx, i["select_bias"], w.gate, dropped, ws=ws_c)
        e.record()
        if k >= 3:
            evs.append((s, e))
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in evs]
    nd = int(dropped.cpu()[0])
    moved = int((w.idx != idx0).sum().cpu()) - nd
    return {"factor": factor, "capacity": cap, "layer_ms_per_step": round(layer_med, 4),
            "layer_ms_per_step_mean": round(layer_ms, 4),
            "tokens_per_s": round(c.S / (layer_med / 1e3), 1), "apply_capacity_ms": round(statistics.median(per), 4),
            "rerouted_pairs": moved, "dropped_pairs": nd, "drop_rate": round(nd / (c.S * c.K), 5)}


def w8a8_leg(D, M, torch, steps, warmup, cpu_budget=0.0):
    """The DeepSeek-shape fp8-weight layer with bf16 activations (W8A16) and
    with e4m3 activations (W8A8), same inputs: the layer step, every stage
    alone (the W8A8 products through moe_expert_up_a8 / moe_expert_down_a8,
    the row quantisations through moe_quantize_rows), and the roofline of
    each expert product.  The products stream every touched expert's fp8
    weights once, so they are HBM-bound at their algorithmic intensity."""
    cfg = D.CONFIGS["dsv3_fp8"]
    w = Workload(cfg, D, M, torch)
    inp, out = w.inp, {"workload": cfg.name}
    ms16, med16 = time_calls(torch, w.layer, steps, warmup)
    counts = w.counts.cpu()
    touched = int((counts > 0).sum())
    st16 = {k: time_calls(torch, fn, steps, 2) for k, fn in w.stages().items()}
    # W8A8: the layer, then its stages one by one
    p8 = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                        cfg.renormalize, 1.0, 0, 1)
    ws8 = M.workspace(p8, M.STAGE_LAYER, "cuda")
    y8 = torch.empty_like(w.y)

    def layer8():
        M.moe_layer_forward(p8, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"], y=y8,
                            expert_counts_out=w.counts, ws=ws8)

    ms8, med8 = time_calls(torch, layer8, steps, warmup)
    cap = M.moe_rows_capacity(p8)
    x8 = torch.empty((cap, cfg.d), dtype=torch.uint8, device="cuda")
    xs = torch.empty(cap, dtype=torch.float32, device="cuda")
    h8 = torch.empty((cap, cfg.d_ff), dtype=torch.uint8, device="cuda")
    hs = torch.empty(cap, dtype=torch.float32, device="cuda")
    for fn in w.stages().values():   # routing, permutation and x_perm of this step
        fn()
    st8 = {
        "quantize_x": lambda: M.moe_quantize_rows(w.x_perm, x8, xs),
        "expert_up": lambda: M.moe_expert_up_a8(p8, x8, xs, w.counts, w.offsets, inp["W1"], inp["b1"],
                                                inp["w1_scale"], h=w.h, ws=w.ws_ffn),
        "quantize_h": lambda: M.moe_quantize_rows(w.h, h8, hs),
        "expert_down": lambda: M.moe_expert_down_a8(p8, h8, hs, w.counts, w.offsets, inp["W2"], inp["b2"],
                                                    inp["w2_scale"], y_perm=w.y_perm, ws=w.ws_ffn),
    }
    st8 = {k: time_calls(torch, fn, steps, 2) for k, fn in st8.items()}
    m16, d16 = stage_dicts(st16)
    m8, d8 = stage_dicts(st8)
    wbytes = touched * 2 * cfg.d * cfg.d_ff + touched * 4 * (cfg.d + cfg.d_ff)
    out.update({
        "ms_per_step_w8a8": round(med8, 4), "ms_per_step_w8a8_mean": round(ms8, 4),
        "ms_per_step_w8a16": round(med16, 4), "ms_per_step_w8a16_mean": round(ms16, 4),
        "tokens_per_s": round(cfg.S / (med8 / 1e3), 1), "tokens_per_s_w8a16": round(cfg.S / (med16 / 1e3), 1),
        "experts_touched": touched, "expert_weight_bytes": wbytes,
        "weight_stream_GBps": round(wbytes / (med8 / 1e3) / 1e9, 1), "hbm_peak_GBps": PEAK_GBS,
        "layer_w8a8": layer_fractions(cfg, med8, touched, "fp8"),
        "layer_w8a16": layer_fractions(cfg, med16, touched, "bf16"),
        "stage_ms_w8a16": {k: round(v, 4) for k, v in m16.items()}, "stage_ms_median_w8a16": d16,
        "stage_ms_w8a8": {k: round(v, 4) for k, v in m8.items()}, "stage_ms_median_w8a8": d8,
        "roofline_w8a16": {k: roofline(cfg, m16, touched, cfg.name, k) for k in ("expert_up", "expert_down")},
        "roofline_w8a8": {k: roofline(cfg, m8, touched, cfg.name + "_w8a8", k, a8=True)
                          for k in ("expert_up", "expert_down")},
    })
    if cpu_budget > 0:
        out["cpu_loops"] = cpu_loops_rate(cfg, inp, cpu_budget, torch, max_experts=100)
    del w, ws8, x8, h8
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ CPU oracle
def _host_decode(t, dt, torch, scale=None):
    """A device tensor of storage dtype `dt` -> float64 host array (fp8 times
    its per-output-channel scale)."""
    import numpy as np

    from oracle import cref
    t = t.detach().cpu()
    if dt == "bf16":
        v = cref.decode(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    elif dt == "fp8":
        v = cref.decode(t.view(torch.uint8).numpy(), "fp8")
    else:
        v = t.double().numpy()
    if scale is not None:
        v *= scale.detach().cpu().double().numpy()[:, None]
    return v


def cpu_loops_rate(cfg, inp, budget_s, torch, threads=None, n_tokens=None, repeats=1, max_experts=None):
    """The plain C++ loops of oracle/moe_oracle_ref.cpp (OpenMP over tokens,
    double precision) as they stand, on the first n tokens of the workload:
    n grows until one call costs about budget_s (or covers S, or touches more
    than max_experts experts), unless n_tokens fixes it.  Device inputs are
    copied and decoded to double beforehand, only for the experts the sample
    routes to (the other experts' weights are untouched zero pages); timed is
    the oracle_layer_forward call alone (scores, selection, gates, every
    routed pair's expert FFN, combine).  Returns tokens/s and what ran."""
    import numpy as np

    from oracle import cref
    if not os.path.exists(cref.LIB_PATH):
        return None
    default_threads = cref.threads()
    cref.set_threads(threads or default_threads)
    used_threads = cref.threads()
    E, d, d_ff = cfg.E, cfg.d, cfg.d_ff
    wr = _host_decode(inp["W_r"], cfg.act, torch)
    rb = None if inp["router_bias"] is None else inp["router_bias"].cpu().numpy()
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    b1, b2 = _host_decode(inp["b1"], cfg.act, torch), _host_decode(inp["b2"], cfg.act, torch)
    W1 = np.zeros((E, d_ff, d))      # zero pages until an expert is filled in
    W2 = np.zeros((E, d, d_ff))
    have = set()

    def sample(n):
        x = _host_decode(inp["x"][:n], cfg.act, torch)
        idx, _ = cref.route(cref.router_logits(x, wr, rb), cfg.K, sb, cfg.n_groups, cfg.topk_groups,
                            cfg.renormalize)
        used = sorted(set(int(e) for e in np.unique(idx)))
        for e in used:
            if e not in have:
                W1[e] = _host_decode(inp["W1"][e], cfg.w, torch, inp["w1_scale"][e] if cfg.w == "fp8" else None)
                W2[e] = _host_decode(inp["W2"][e], cfg.w, torch, inp["w2_scale"][e] if cfg.w == "fp8" else None)
                have.add(e)
        return x, len(used)

    def run(x):
        t0 = time.perf_counter()
        cref.layer_forward(x, wr, W1, b1, W2, b2, K=cfg.K, router_bias=rb, select_bias=sb, n_groups=cfg.n_groups,
                           topk_groups=cfg.topk_groups, renormalize=cfg.renormalize)
        return time.perf_counter() - t0

    try:
        if n_tokens is not None:
            n = min(cfg.S, n_tokens)
            x, ne = sample(n)
            ts = [run(x) for _ in range(repeats)]
            t = statistics.median(ts)
        else:
            n = min(cfg.S, 4)
            x, ne = sample(n)
            t = run(x)
            while t < 0.5 * budget_s and n < cfg.S:
                grow = 2.0 if max_experts is not None else min(8.0, max(2.0, budget_s / max(t, 1e-3)))
                n2 = int(min(cfg.S, n * grow))
                x2, ne2 = sample(n2)
                if max_experts is not None and ne2 > max_experts:
                    break
                n, x, ne = n2, x2, ne2
                t = run(x)
            ts = [t]
    finally:
        cref.set_threads(default_threads)
    return {"value": round(n / t, 3), "unit": "tokens/s", "tokens": n, "of": cfg.S, "experts_touched": ne,
            "seconds": round(t, 3), "runs": len(ts), "threads": used_threads}


def cpu_numpy_rate(cfg, w, target_s, torch):
    """The numpy oracle (oracle/moe_oracle.py, float64, BLAS products) as it
    stands on the first n tokens of the same workload."""
    import numpy as np

    import oracle as O
    from threadpoolctl import threadpool_info

    def raw(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()

    inp = w.inp
    host = {k: (None if v is None else raw(v)) for k, v in inp.items() if k not in ("W1", "W2")}
    W1 = {}
    W2 = {}

    def run(n):
        x = host["x"][:n]
        lg = O.router_logits(O.decode(x, cfg.act), O.decode(host["W_r"], cfg.act), host["router_bias"])
        used = np.unique(O.select_experts(lg, cfg.K, host["select_bias"], cfg.n_groups, cfg.topk_groups))
        for e in used:   # device -> host copies stay outside the timed region
            if int(e) not in W1:
                W1[int(e)], W2[int(e)] = raw(inp["W1"][int(e)]), raw(inp["W2"][int(e)])
        t0 = time.perf_counter()
        O.layer_forward(x, host["W_r"], W1, host["b1"], W2, host["b2"], K=cfg.K, act=cfg.act, w=cfg.w,
                        router_bias=host["router_bias"], select_bias=host["select_bias"],
                        n_groups=cfg.n_groups, topk_groups=cfg.topk_groups, renormalize=cfg.renormalize,
                        w1_scale=host["w1_scale"], w2_scale=host["w2_scale"])
        return time.perf_counter() - t0

    n = min(cfg.S, 32)
    t = run(n)
    while t < 0.5 * target_s and n < cfg.S:
        n = int(min(cfg.S, n * min(8.0, max(2.0, target_s / max(t, 1e-3)))))
        t = run(n)
    threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    return {"value": round(n / t, 2), "unit": "tokens/s", "blas_threads": threads, "tokens": n, "of": cfg.S,
            "seconds": round(t, 2)}


def host_cores():
    """Logical CPUs this process may run on, and the machine's count."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count()
    return aff, os.cpu_count()


def main():
    a = parse()
    if a.pmc_summary:
        pmc_summary(a)
        return
    if a.pmc_mfma_summary:
        pmc_mfma_summary(a)
        return
    if a.pmc_mem_summary:
        pmc_mem_summary(a)
        return
    if a.trace_table:
        trace_table(a.trace_table)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(json.dumps({"metric": METRIC, "error": "this MoE layer runs on exactly one GPU; "
                          f"--gpus {a.gpus} (WORLD_SIZE {world}) is not supported"}))
        sys.exit(2)
    import torch

    import datagen as D
    import sparse_ffn_layer_amd as M

    M.lib()   # raises if the HIP library is missing: there is no fallback
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if a.pmc_probe:
        pmc_probe(a, D, M, torch)
        return
    cpu = not a.no_cpu_baseline
    cpu_legs = {}
    cfg, w, (ms, med), st, touched, counts = run_workload(a.workload, a.steps, a.warmup, D, M, torch)
    stage_ms, stage_med = stage_dicts(st)
    mean = cfg.S * cfg.K / cfg.E
    out = {
        "metric": METRIC, "value": round(cfg.S / (med / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(med, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.act, "data": "synthetic",
        "config": {"workload": cfg.name, "S": cfg.S, "d": cfg.d, "d_ff": cfg.d_ff, "E": cfg.E, "K": cfg.K,
                   "weights": cfg.w, "max_over_mean_load": round(float(counts.max()) / mean, 3),
                   "experts_touched": touched},
        "statistic": "median of per-step HIP-event times (value, ms_per_step); mean in ms_per_step_mean",
        "ms_per_step_mean": round(ms, 4),
        "roofline": roofline(cfg, stage_ms, touched, cfg.name),
        "layer": layer_fractions(cfg, med, touched, "bf16" if cfg.act == "bf16" else "f32"),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()}, "stage_ms_median": stage_med,
        "layer_tflops": round(4.0 * cfg.S * cfg.K * cfg.d * cfg.d_ff / (med / 1e3) / 1e12, 2),
    }
    log(f"[bench] {cfg.name}: {med:.3f} ms/step (mean {ms:.3f}), stages {out['stage_ms']}")
    if cpu:
        cpu_legs[cfg.name] = cpu_loops_rate(cfg, w.inp, a.cpu_seconds / 2, torch)
        log(f"[bench] cpu loops {cfg.name}: {cpu_legs[cfg.name]}")
        one = cpu_loops_rate(cfg, w.inp, 0, torch, threads=1, n_tokens=4)
        log(f"[bench] cpu loops {cfg.name}, one thread: {one}")
    if not a.no_context and cfg.act == "bf16":
        out["context"] = context_leg(w, torch, counts.tolist())
        out["context"]["this_up_TFLOPs"] = out["roofline"]["achieved"] if out["roofline"]["kernel"] == "expert_up" \
            else None
        log(f"[bench] context: {out['context']}")
    if not a.no_capacity:
        out["capacity"] = capacity_leg(w, M, torch, 1.25, a.steps)
        log(f"[bench] capacity: {out['capacity']}")
    if cpu:
        out["cpu_numpy"] = cpu_numpy_rate(cfg, w, a.cpu_seconds / 2, torch)
    del w
    torch.cuda.empty_cache()
    if not a.no_w8a8:
        out["w8a8"] = w8a8_leg(D, M, torch, max(5, a.steps // 2), 3, a.cpu_seconds / 3 if cpu else 0.0)
        if cpu and out["w8a8"].get("cpu_loops"):
            cpu_legs["dsv3_fp8"] = out["w8a8"].pop("cpu_loops")
        log(f"[bench] w8a8: {out['w8a8']}")
    if not a.no_decode and cfg.name != "decode":
        dcfg, dw, (dms, dmed), dst, dtouched, _ = run_workload("decode", max(a.steps, 100), a.warmup, D, M, torch)
        dmean, dmedian = stage_dicts(dst)
        out["decode"] = {"workload": "decode", "tokens_per_s": round(dcfg.S / (dmed / 1e3), 1),
                         "ms_per_step": round(dmed, 4), "ms_per_step_mean": round(dms, 4),
                         "experts_touched": dtouched,
                         "roofline": roofline(dcfg, dmean, dtouched, "decode"),
                         "layer": layer_fractions(dcfg, dmed, dtouched, "bf16"),
                         "stage_ms": {k: round(v, 4) for k, v in dmean.items()}, "stage_ms_median": dmedian,
                         "graph": graph_leg(dw, torch, max(a.steps, 100), a.warmup)}
        if cpu:
            cpu_legs["decode"] = cpu_loops_rate(dcfg, dw.inp, 0, torch, n_tokens=dcfg.S)
        del dw
        torch.cuda.empty_cache()
    if not a.no_skew and cfg.name != "zipf_skew":
        zcfg, zw, (zms, zmed), zst, ztouched, zcounts = run_workload("zipf_skew", a.steps, a.warmup, D, M, torch)
        zmean, zmedian = stage_dicts(zst)
        gemm_ms = zmean["expert_up"] + zmean["expert_down"]
        ffn_flops = 4.0 * zcfg.S * zcfg.K * zcfg.d * zcfg.d_ff
        out["zipf_skew"] = {"workload": "zipf_skew", "tokens_per_s": round(zcfg.S / (zmed / 1e3), 1),
                            "ms_per_step": round(zmed, 4), "ms_per_step_mean": round(zms, 4),
                            "max_over_mean_load": round(float(zcounts.max()) / (zcfg.S * zcfg.K / zcfg.E), 3),
                            "empty_experts": zcfg.E - ztouched,
                            "roofline": roofline(zcfg, zmean, ztouched, "zipf_skew"),
                            "gemms_mfma_frac": round(ffn_flops / (gemm_ms / 1e3) / (PEAK_TFLOPS["bf16"] * 1e12), 4),
                            "layer": layer_fractions(zcfg, zmed, ztouched, "bf16"),
                            "stage_ms": {k: round(v, 4) for k, v in zmean.items()}, "stage_ms_median": zmedian}
        log(f"[bench] zipf_skew: {zmed:.3f} ms/step, stages {out['zipf_skew']['stage_ms']}")
        if cpu:
            cpu_legs["zipf_skew"] = cpu_loops_rate(zcfg, zw.inp, a.cpu_seconds / 3, torch)
        del zw
        torch.cuda.empty_cache()
    if cpu:
        tcfg = D.CONFIGS["tiny_f32"]
        tinp = D.make_inputs(tcfg, "cpu")
        cpu_legs["tiny_f32"] = cpu_loops_rate(tcfg, tinp, 0, torch, n_tokens=tcfg.S, repeats=10)
        tiny_one = cpu_loops_rate(tcfg, tinp, 0, torch, threads=1, n_tokens=tcfg.S, repeats=3)
        aff, ncpu = host_cores()
        gpu_rates = {cfg.name: out["value"], "decode": out.get("decode", {}).get("tokens_per_s"),
                     "zipf_skew": out.get("zipf_skew", {}).get("tokens_per_s"),
                     "dsv3_fp8": out.get("w8a8", {}).get("tokens_per_s_w8a16")}
        for k, v in cpu_legs.items():
            if v is not None and gpu_rates.get(k):
                v["gpu_tokens_per_s"] = gpu_rates[k]
        main_leg = cpu_legs[cfg.name]
        out["cpu_baseline"] = {
            "value": main_leg["value"], "unit": "tokens/s", "cores": main_leg["threads"], "kind": "oracle",
            "sample": f"first {main_leg['tokens']} of {cfg.S} tokens of {cfg.name}: the plain C++ loops of the "
                      f"oracle (double, OpenMP over tokens, {main_leg['threads']} threads), one call, "
                      f"{main_leg['seconds']}s; weights decoded beforehand",
            "host_cpus_available": aff, "host_cpus_total": ncpu,
            "single_thread": {"tiny_f32_64_tokens": tiny_one, cfg.name: one},
            "per_config": cpu_legs,
            "numpy_oracle": out.pop("cpu_numpy", None),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
