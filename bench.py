"""Benchmark of the MoE-layer forward on one MI355X.

One step = one moe_layer_forward (route, permute, expert up/down GEMMs,
combine) over the workload's S tokens, inputs resident in HBM.  Prints ONE
JSON line on stdout: MoE-layer tokens/s at the Mixtral-shape prefill workload
(S=4096, d=4096, d_ff=14336, E=8, K=2, bf16), the roofline of the dominant
kernel, the decode workload's HBM fraction, the same layer under a
per-expert capacity, the DeepSeek-shape fp8 layer with fp8 activations, and
the CPU oracle's rate on a bounded sample of the same workload.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-decode] [--no-capacity] [--no-w8a8]
       python bench.py --pmc-probe [--workload NAME]     (under rocprofv3 --pmc)
       python bench.py --pmc-summary FETCH_DIR WRITE_DIR [--workload NAME]
"""
import argparse
import hashlib
import json
import os
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
    ap.add_argument("--pmc-mfma-summary", metavar="DIR",
                    help="write profiles/mfma_*.md from a rocprofv3 --pmc pass over the MFMA counters")
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
    """Average ms per call, HIP events on the stream the library launches on."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def algorithmic(cfg, touched):
    """Per-launch algorithmic flops and HBM bytes of the two expert GEMMs.

    Flops count only the S*K routed rows (no padding).  Bytes: each touched
    expert's weights (+ fp8 scales) and biases once, the routed activation
    rows in and out once."""
    a = 2 if cfg.act == "bf16" else 4
    w = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.w]
    rows = cfg.S * cfg.K
    fl = 2.0 * rows * cfg.d * cfg.d_ff
    sc = 4 if cfg.w == "fp8" else 0
    up = touched * (cfg.d * cfg.d_ff * w + cfg.d_ff * (a + sc)) + rows * (cfg.d + cfg.d_ff) * a
    down = touched * (cfg.d_ff * cfg.d * w + cfg.d * (a + sc)) + rows * (cfg.d_ff + cfg.d) * a
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
    each), so FETCH_SIZE / WRITE_SIZE per dispatch can be read off."""
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
    for _ in range(3):
        st["expert_up"]()
        st["expert_down"]()
    torch.cuda.synchronize()
    log(f"[bench] pmc probe done: {cfg.name}")


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
    # the expert GEMM kernels: expert_up has epilogue 0 (bias+GeLU), expert_down
    # epilogue 1 (bias); the epilogue is the only template argument of the
    # four-wave kernel and the eighth of the general one
    stages = {}
    for k in fk:
        if "grouped_gemm_bf16" not in k or "fixup" in k:
            continue
        args = [x.strip() for x in k.split("<", 1)[1].split(">", 1)[0].split(",")]
        epi = args[0] if "_w4_kernel" in k else args[7]
        stages["expert_up" if epi == "0" else "expert_down"] = k
    cfg_name = a.workload
    for stage, k in stages.items():
        fb = statistics.median(fk[k]) * 1024 / f_scale
        wb = statistics.median(wk[k]) * 1024 / w_scale
        path = traffic_path(stage, cfg_name)
        with open(path, "w") as f:
            f.write(f"# HBM traffic: `{stage}` GEMM, {cfg_name} workload\n\n")
            f.write("Commands (one MI355X, repository root; two counter passes, then this summary):\n\n```\n")
            f.write(f"rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o f --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {cfg_name}\n")
            f.write(f"rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o w --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {cfg_name}\n")
            f.write(f"python bench.py --workload {cfg_name} --pmc-summary gpurun_out/pmc_fetch gpurun_out/pmc_write\n```\n\n")
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


def pmc_mfma_summary(a):
    """Turn one rocprofv3 --pmc pass over MFMA_COUNTERS (csv output) into
    profiles/mfma_<stage>_<workload>.md: per expert GEMM dispatch, the MFMA
    busy fraction of all SIMDs, the shader clock, and the bf16 MFMA work
    executed (padding rows included) against the algorithmic work."""
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
        if "grouped_gemm_bf16" not in k or "fixup" in k:
            continue
        d = disp.setdefault((k, r["Dispatch_Id"]), {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    cfg_name = a.workload
    import datagen as D
    cfg = D.CONFIGS[cfg_name]
    alg = 2.0 * cfg.S * cfg.K * cfg.d * cfg.d_ff
    cus, simds, xccs = 256, 4, 8
    for stage, epi in (("expert_up", "0"), ("expert_down", "1")):
        ds = [v for (k, _), v in disp.items()
              if [x.strip() for x in k.split("<", 1)[1].split(">", 1)[0].split(",")][0 if "_w4_kernel" in k else 7] == epi]
        if not ds:
            continue
        kname = next(k for (k, _) in disp if k.split("<", 1)[1].split(">", 1)[0].split(",")[0 if "_w4_kernel" in k else 7].strip() == epi)
        med = lambda f: statistics.median(f(d) for d in ds)
        gui = med(lambda d: d["GRBM_GUI_ACTIVE"] / xccs)          # shader cycles of the dispatch
        ghz = med(lambda d: d["GRBM_GUI_ACTIVE"] / xccs / d["ns"])
        busy = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / xccs * cus * simds))
        flops = med(lambda d: d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512)
        ms = med(lambda d: d["ns"]) / 1e6
        path = os.path.join(ROOT, "profiles", f"mfma_{stage}_{cfg_name}.md")
        with open(path, "w") as f:
            f.write(f"# MFMA utilisation: `{stage}` GEMM, {cfg_name} workload\n\n")
            f.write("Commands (one MI355X, repository root; one counter pass, then this summary):\n\n```\n")
            f.write(f"rocprofv3 --pmc {MFMA_COUNTERS} -d gpurun_out/pmc_mfma -o m --output-format csv -- "
                    f"python -u bench.py --pmc-probe --workload {cfg_name}\n")
            f.write(f"python bench.py --workload {cfg_name} --pmc-mfma-summary gpurun_out/pmc_mfma\n```\n\n")
            f.write(f"Kernel: `{kname}` ({len(ds)} dispatches, medians).  Counters are summed over the {xccs} XCCs "
                    f"and their SIMDs; shader cycles = GRBM_GUI_ACTIVE / {xccs}.\n\n")
            f.write("| quantity | value |\n|:--|--:|\n")
            f.write(f"| dispatch duration under counter collection | {ms:.3f} ms |\n")
            f.write(f"| shader clock (cycles / duration) | {ghz:.2f} GHz |\n")
            f.write(f"| MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {cus} CUs x {simds} SIMDs) | {100 * busy:.1f} % |\n")
            f.write(f"| bf16 MFMA work executed: 512 SQ_INSTS_VALU_MFMA_MOPS_BF16 | {flops:.4g} flop |\n")
            f.write(f"| algorithmic work (2 d d_ff per routed row) | {alg:.4g} flop |\n")
            f.write(f"| executed / algorithmic (padding rows of partly filled tiles) | {flops / alg:.3f} |\n")
            f.write(f"| executed rate during the dispatch | {flops / (ms / 1e3) / 1e12:.0f} TFLOP/s |\n")
            f.write(f"| dense bf16 peak at the measured clock ({ghz:.2f} / 2.4 x 2.5 PFLOP/s) | "
                    f"{2500 * ghz / 2.4:.0f} TFLOP/s |\n\n")
            f.write("The fraction of the 2.5 PFLOP/s peak that the algorithmic work reaches factors as MFMA busy x "
                    "(clock / 2.4 GHz) / (executed / algorithmic): "
                    f"{busy:.3f} x {ghz / 2.4:.3f} / {flops / alg:.3f} = {busy * ghz / 2.4 / (flops / alg):.3f} under "
                    "counter collection (the bench line's figure comes from uninstrumented launches, at a clock "
                    "that varies from box to box).\n\n")
            f.write(f"- source_hash: {gemm_source_hash()}\n")
        log(f"[bench] wrote {path}")


def roofline(cfg, stage_ms, touched, workload):
    alg = algorithmic(cfg, touched)
    name = max(("expert_up", "expert_down"), key=lambda k: stage_ms[k])
    fl, by = alg[name]
    sec = stage_ms[name] / 1e3
    intensity = fl / by
    peak_f = PEAK_TFLOPS["bf16" if cfg.act == "bf16" else "f32"]
    ridge = peak_f * 1e12 / (PEAK_GBS * 1e9)
    if intensity >= ridge:
        ach, peak, unit, bound = fl / sec / 1e12, peak_f, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = by / sec / 1e9, PEAK_GBS, "GB/s", "hbm"
    return {"kernel": name, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic_for(name, workload),
            "avg_launch_ms": round(stage_ms[name], 4), "algorithmic_flops": fl, "algorithmic_bytes": by}


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
    cfg = D.CONFIGS[name]
    w = Workload(cfg, D, M, torch)
    ms = time_calls(torch, w.layer, steps, warmup)
    counts = w.counts.cpu()
    touched = int((counts > 0).sum())
    stage_ms = {k: time_calls(torch, fn, steps, max(2, warmup // 2)) for k, fn in w.stages().items()}
    return cfg, w, ms, stage_ms, touched, counts


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
    copy_ms = time_calls(torch, lambda: dst.copy_(src), 10, 3)
    del src, dst
    gen = torch.Generator(device="cuda").manual_seed(0)
    rows = int(sum(int(n) for n in counts))
    # weights in the layout the expert products read them, [d_ff][d] (a
    # linear layer's [out][in]); a plain 2-D product with the transposed view
    a = torch.randn((rows, c.d), device="cuda", generator=gen).to(torch.bfloat16)
    wt = torch.randn((c.d_ff, c.d), device="cuda", generator=gen).to(torch.bfloat16)
    dense_ms = time_calls(torch, lambda: torch.mm(a, wt.t()), 10, 3)
    ws = [torch.randn((c.d_ff, c.d), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(c.E)]
    offs = [0]
    for n in counts:
        offs.append(offs[-1] + int(n))

    def per_expert():
        for e in range(c.E):
            if offs[e + 1] > offs[e]:
                torch.mm(a[offs[e]:offs[e + 1]], ws[e].t())

    grouped_ms = time_calls(torch, per_expert, 10, 3)
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
    ms = time_calls(torch, g.replay, steps, warmup)
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.cfg.S / (ms / 1e3), 1)}


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

    layer_ms = time_calls(torch, layer, steps, 3)
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
    apply_ms = sum(s.elapsed_time(e) for s, e in evs) / len(evs)
    nd = int(dropped.cpu()[0])
    moved = int((w.idx != idx0).sum().cpu()) - nd
    return {"factor": factor, "capacity": cap, "layer_ms_per_step": round(layer_ms, 4),
            "tokens_per_s": round(c.S / (layer_ms / 1e3), 1), "apply_capacity_ms": round(apply_ms, 4),
            "rerouted_pairs": moved, "dropped_pairs": nd, "drop_rate": round(nd / (c.S * c.K), 5)}


def w8a8_leg(D, M, torch, steps, warmup):
    """The DeepSeek-shape fp8-weight layer with e4m3 activations (W8A8)
    against the same layer with bf16 activations (W8A16), same inputs.  The
    expert products stream every touched expert's fp8 weights once, so the
    weight bytes over the step time are reported next to the HBM peak."""
    cfg = D.CONFIGS["dsv3_fp8"]
    inp = D.make_inputs(cfg, "cuda")
    torch.cuda.synchronize()
    y = torch.empty((cfg.S, cfg.d), dtype=torch.bfloat16, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    out = {"workload": cfg.name}
    for aq in (0, 1):
        p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                           cfg.renormalize, 1.0, 0, aq)
        ws = M.workspace(p, M.STAGE_LAYER, "cuda")

        def step():
            M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                                inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"], y=y,
                                expert_counts_out=counts, ws=ws)

        ms = time_calls(torch, step, steps, warmup)
        out["ms_per_step_w8a8" if aq else "ms_per_step_w8a16"] = round(ms, 4)
        del ws
    touched = int((counts > 0).sum().cpu())
    wbytes = touched * 2 * cfg.d * cfg.d_ff + touched * 4 * (cfg.d + cfg.d_ff)
    ms = out["ms_per_step_w8a8"]
    out.update({"tokens_per_s": round(cfg.S / (ms / 1e3), 1), "experts_touched": touched,
                "expert_weight_bytes": wbytes,
                "weight_stream_GBps": round(wbytes / (ms / 1e3) / 1e9, 1), "hbm_peak_GBps": PEAK_GBS,
                "layer_w8a8": layer_fractions(cfg, ms, touched, "fp8"),
                "layer_w8a16": layer_fractions(cfg, out["ms_per_step_w8a16"], touched, "bf16")})
    del inp
    torch.cuda.empty_cache()
    return out


def cpu_loops_baseline(cfg, w, target_s, torch):
    """The plain C++ loops of oracle/moe_oracle_ref.cpp (OpenMP over tokens,
    double precision) on the first n tokens of the same workload; the
    experts' weights are decoded to double before the timed call."""
    import numpy as np

    from oracle import cref
    if not os.path.exists(cref.LIB_PATH):
        return None

    def host(t, dt):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return cref.decode(t.view(torch.int16).numpy().view(np.uint16), "bf16")
        if t.dtype == torch.float8_e4m3fn:
            return cref.decode(t.view(torch.uint8).numpy(), "fp8")
        return t.double().numpy()

    inp = w.inp
    if cfg.w == "fp8":
        return None     # the loops take the fp8 scales folded in; measured on bf16 workloads only
    W1, W2 = host(inp["W1"], cfg.w), host(inp["W2"], cfg.w)
    b1, b2 = host(inp["b1"], cfg.act), host(inp["b2"], cfg.act)
    wr = host(inp["W_r"], cfg.act)
    rb = None if inp["router_bias"] is None else inp["router_bias"].cpu().numpy()
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    xall = host(inp["x"], cfg.act)

    def run(n):
        t0 = time.perf_counter()
        cref.layer_forward(xall[:n], wr, W1, b1, W2, b2, K=cfg.K, router_bias=rb, select_bias=sb,
                           n_groups=cfg.n_groups, topk_groups=cfg.topk_groups, renormalize=cfg.renormalize)
        return time.perf_counter() - t0

    n = min(cfg.S, 16)
    t = run(n)
    while t < 0.5 * target_s and n < cfg.S:
        n = int(min(cfg.S, n * min(8.0, max(2.0, target_s / max(t, 1e-3)))))
        t = run(n)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    return {"value": round(n / t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.S} tokens of {cfg.name}: plain C++ loops (double, OpenMP), "
                      f"weights decoded beforehand; {t:.1f}s", "seconds": round(t, 2)}


def cpu_baseline(cfg, w, target_s, torch):
    """The oracle, as it is, on the first n tokens of the same workload."""
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

    # grow the sample until it costs about target_s of CPU time (or covers S)
    n = min(cfg.S, 32)
    t = run(n)
    while t < 0.5 * target_s and n < cfg.S:
        n = int(min(cfg.S, n * min(8.0, max(2.0, target_s / max(t, 1e-3)))))
        t = run(n)
    threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    return {"value": round(n / t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.S} tokens of {cfg.name}: routing, every expert they touch "
                      f"(float64, weights decoded per expert), combine; {t:.1f}s",
            "seconds": round(t, 2)}


def main():
    a = parse()
    if a.pmc_summary:
        pmc_summary(a)
        return
    if a.pmc_mfma_summary:
        pmc_mfma_summary(a)
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
    cfg, w, ms, stage_ms, touched, counts = run_workload(a.workload, a.steps, a.warmup, D, M, torch)
    mean = cfg.S * cfg.K / cfg.E
    out = {
        "metric": METRIC, "value": round(cfg.S / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.act, "data": "synthetic",
        "config": {"workload": cfg.name, "S": cfg.S, "d": cfg.d, "d_ff": cfg.d_ff, "E": cfg.E, "K": cfg.K,
                   "weights": cfg.w, "max_over_mean_load": round(float(counts.max()) / mean, 3),
                   "experts_touched": touched},
        "roofline": roofline(cfg, stage_ms, touched, cfg.name),
        "layer": layer_fractions(cfg, ms, touched, "bf16" if cfg.act == "bf16" else "f32"),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "layer_tflops": round(4.0 * cfg.S * cfg.K * cfg.d * cfg.d_ff / (ms / 1e3) / 1e12, 2),
    }
    log(f"[bench] {cfg.name}: {ms:.3f} ms/step, stages {out['stage_ms']}")
    if not a.no_context and cfg.act == "bf16":
        out["context"] = context_leg(w, torch, counts.tolist())
        out["context"]["this_up_TFLOPs"] = out["roofline"]["achieved"] if out["roofline"]["kernel"] == "expert_up" \
            else None
        log(f"[bench] context: {out['context']}")
    if not a.no_capacity:
        out["capacity"] = capacity_leg(w, M, torch, 1.25, a.steps)
        log(f"[bench] capacity: {out['capacity']}")
    if not a.no_w8a8:
        out["w8a8"] = w8a8_leg(D, M, torch, max(5, a.steps // 2), 3)
        log(f"[bench] w8a8: {out['w8a8']}")
    if not a.no_decode and cfg.name != "decode":
        dcfg, dw, dms, dstage, dtouched, _ = run_workload("decode", max(a.steps, 100), a.warmup, D, M, torch)
        out["decode"] = {"workload": "decode", "tokens_per_s": round(dcfg.S / (dms / 1e3), 1),
                         "ms_per_step": round(dms, 4), "roofline": roofline(dcfg, dstage, dtouched, "decode"),
                         "layer": layer_fractions(dcfg, dms, dtouched, "bf16"),
                         "stage_ms": {k: round(v, 4) for k, v in dstage.items()},
                         "graph": graph_leg(dw, torch, max(a.steps, 100), a.warmup)}
        del dw
    if not a.no_skew and cfg.name != "zipf_skew":
        zcfg, zw, zms, zstage, ztouched, zcounts = run_workload("zipf_skew", a.steps, a.warmup, D, M, torch)
        gemm_ms = zstage["expert_up"] + zstage["expert_down"]
        ffn_flops = 4.0 * zcfg.S * zcfg.K * zcfg.d * zcfg.d_ff
        out["zipf_skew"] = {"workload": "zipf_skew", "tokens_per_s": round(zcfg.S / (zms / 1e3), 1),
                            "ms_per_step": round(zms, 4),
                            "max_over_mean_load": round(float(zcounts.max()) / (zcfg.S * zcfg.K / zcfg.E), 3),
                            "empty_experts": zcfg.E - ztouched,
                            "roofline": roofline(zcfg, zstage, ztouched, "zipf_skew"),
                            "gemms_mfma_frac": round(ffn_flops / (gemm_ms / 1e3) / (PEAK_TFLOPS["bf16"] * 1e12), 4),
                            "layer": layer_fractions(zcfg, zms, ztouched, "bf16"),
                            "stage_ms": {k: round(v, 4) for k, v in zstage.items()}}
        log(f"[bench] zipf_skew: {zms:.3f} ms/step, stages {out['zipf_skew']['stage_ms']}")
        del zw
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, w, a.cpu_seconds, torch)
        loops = cpu_loops_baseline(cfg, w, a.cpu_seconds / 2, torch)
        if loops is not None:
            out["cpu_baseline"]["cpp_loops"] = loops
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
