"""Benchmark of the NVFP4 block-scaled fused-MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the Qwen3-30B-A3B-shaped decode layer (H=2048, I=768, E=128,
top-8, NVFP4 weights, BF16 activations). One step runs the whole layer once for
each decode batch T in {1, 8, 32, 64} (105 tokens), each batch with its own
seeded weights, inputs and logits, so the 1.36 GB of weights the step streams
exceed the 256 MB Infinity Cache. Inputs are resident in HBM before timing;
W warmup steps, then exactly K timed steps between two device synchronisations.
The step is captured once in a HIP graph and replayed (the serving launch path);
the eager-launch time of the same step is reported beside it.

Prints one JSON line: tokens/s of the whole step (value), the per-step distribution of K
further replays (median, IQR, samples), plus
  roofline:     the dominant kernel (the gate/up grouped GEMM) timed with HIP
                events recorded on its launch stream over K further steps:
                algorithmic bytes per launch / mean launch time vs 8 TB/s HBM
                (decode) or algorithmic FLOPs / time vs 2.5 PFLOP/s bf16 MFMA
                (prefill workloads);
  cpu_baseline: the CPU oracle (FP64, OpenMP) on a bounded sample of the same
                workload, on this host's cores.
Other workloads (--workload qwen3-30b-a3b-prefill | deepseek-v3 | skewed-w4a4 |
skewed-w4a4-all (h quantised to NVFP4 too) | tiny) print the same line for that configuration, and so do the router/activation
variants deepseek-v4-flash-decode (256 experts, top-6, H=4096, I=1024, sqrt-softplus
scores with a selection bias, SwiGLU clamped at 10, one shared expert; T in
{1, 8, 32, 64}) and deepseek-v3-noaux (the DeepSeek-V3 layer with its grouped
sigmoid router, selection bias and routed scale 2.5), and deepseek-v4-flash-sharing (one
rank's routed V4-Flash MoE on the sharing workloads: T = 6 with 0, 20, .., 100% of the
(token, expert) picks reused across the batch, T = 4, 5, 8 at 40%; each batch line records
its expert row counts and useful weight bytes).

roofline.traffic is the HBM traffic of one gate/up launch measured by rocprofv3
counters (FETCH_SIZE and WRITE_SIZE runs, each scaled by the reading of a 1 GiB
device copy), taken from the record in profiles/ whose kernel-source hash matches
the sources built now (null otherwise). The records and the kernel-trace
summaries in profiles/ are made from rocprofv3 output by this script:

    python bench.py --trace-summary RESULTS_DB --title T --command C
    python bench.py --traffic-summary FETCH_CSV WRITE_CSV --workload W --title T --command C
    python bench.py --counter-summary PMC_CSV [PMC_CSV ...] --title T --command C
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
import nvfp4_block_scaled_router_amd as m  # noqa: E402
from nvfp4_block_scaled_router_amd.weights import quantize_projection  # noqa: E402

METRIC = "NVFP4 fused-MoE tokens/s; decode HBM GB/s and prefill TFLOP/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0        # dense fp8 MFMA (the W4A8 scaled MFMA: E2M1 x E4M3 operands)
NVFP4_BYTES_PER_WEIGHT = 0.5 + 1.0 / 16.0      # E2M1 nibble + one E4M3 byte per 16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def workload(name):
    if name == "qwen3-30b-a3b-decode":
        return [synth.qwen3_decode(T) for T in synth.DECODE_TOKENS], "hbm"
    if name == "qwen3-30b-a3b-prefill":
        return [synth.qwen3_prefill()], "mfma"
    if name == "deepseek-v3":
        return [synth.deepseek_v3()], "mfma"
    if name == "skewed-w4a4":
        return [synth.skewed_w4a4()], "hbm"
    if name == "skewed-w4a4-all":        # the same layer with h quantised to NVFP4 as well
        return [synth.skewed_w4a4_all()], "hbm"
    if name == "tiny":
        return [synth.tiny()], "hbm"
    # router / activation variants of the layer (sqrt-softplus + bias + clamped SwiGLU;
    # DeepSeek-V3's grouped sigmoid router with bias and routed scaling)
    if name == "deepseek-v4-flash-decode":
        return [synth.deepseek_v4_flash(T) for T in synth.DECODE_TOKENS], "hbm"
    # the V4-Flash layer in its W4A8 profile (MXFP8 x and h, the block-scaled MFMA)
    if name == "deepseek-v4-flash-w4a8-decode":
        return [synth.deepseek_v4_flash_w4a8(T) for T in synth.DECODE_TOKENS], "hbm"
    if name == "deepseek-v4-flash-w4a8-prefill":
        return [synth.deepseek_v4_flash_w4a8(8192)], "mfma"
    if name == "deepseek-v4-flash-prefill":           # the same batch in W4A16 (bf16 x, 16-bit MFMA)
        return [synth.deepseek_v4_flash(8192)], "mfma"
    if name == "deepseek-v3-noaux":
        return [synth.deepseek_v3_router(8192)], "mfma"
    # one rank's routed DeepSeek-V4-Flash MoE on the sharing workloads: T = 6 at 0..100%
    # reuse of (token, expert) picks, and T = 4, 5, 8 at 40%
    if name == "deepseek-v4-flash-sharing":
        return ([synth.deepseek_v4_flash_sharing(6, lv) for lv in synth.SHARING_LEVELS]
                + [synth.deepseek_v4_flash_sharing(T, 0.4) for T in (4, 5, 8)]), "hbm"
    raise SystemExit(f"unknown workload {name}")


class Batch:
    """One configuration resident on the GPU: packed weights, inputs, routing info."""

    def __init__(self, cfg, dev):
        self.cfg = cfg
        log(f"[bench] preparing {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
        projs = ["w1", "w2"] + (["ws1", "ws2"] if cfg.shared else [])
        W = []
        for w in projs:
            G = cfg.shared if w.startswith("ws") else cfg.E
            N, K = (2 * cfg.I, cfg.H) if w in ("w1", "ws1") else (cfg.H, cfg.I)
            if cfg.wfmt == "mxfp4":   # drawn directly in the boundary format
                codes, scales = synth.mxfp4_weights(cfg, w, 0, G)
                W.append((torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev), None))
            else:
                W.append(quantize_projection(G, N, K, lambda e0, c, w=w: synth.expert_weights_f32(cfg, w, e0, c),
                                             dev))
        self.layer = m.MoeLayer.from_config(cfg, device=dev)
        self.layer.pack(W[0], W[1], W[2] if cfg.shared else None, W[3] if cfg.shared else None)
        bias = synth.router_bias(cfg)
        if bias is not None:
            self.layer.pack_router_bias(torch.from_numpy(bias).to(dev))
        del W
        x = synth.activations(cfg)
        self.x = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.logits = torch.from_numpy(synth.logits(cfg)).to(dev)
        self.out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
        bufs, rout = self.layer.routing_buffers(cfg.T)
        self.layer(self.x, self.logits, out=self.out, routing=rout)
        torch.cuda.synchronize()
        counts = bufs["expert_counts"].cpu().numpy()
        self.touched = int((counts > 0).sum())
        self.expert_rows = sorted((int(c) for c in counts if c > 0), reverse=True)
        self.rows = cfg.T * cfg.k
        torch.cuda.synchronize()

    def run(self):
        self.layer(self.x, self.logits, out=self.out)

    def run_timed(self, events):
        L = self.layer
        m.moe_run_timed(L.plan, L.packed, self.cfg.T, self.x, self.logits, self.out, None, L.workspace,
                        L.workspace_bytes, None, events)

    # algorithmic work of the gate/up launch (the dominant kernel) and of the layer
    def weight_bytes(self, n: int) -> float:
        """Algorithmic bytes of n weights of one expert projection in the workload's format:
        NVFP4 4.5 bits + a 4-byte global scale, MXFP4 4.25 bits (E8M0 per 32, no global scale)."""
        if self.cfg.wfmt == "mxfp4":
            return n * (0.5 + 1.0 / 32)
        return n * NVFP4_BYTES_PER_WEIGHT + 4

    def gate_up_bytes(self):
        c = self.cfg
        w = (self.touched + c.shared) * self.weight_bytes(2 * c.I * c.H)
        act = c.T * c.H * {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32}.get(c.act, NVFP4_BYTES_PER_WEIGHT + 4.0 / c.H)
        h = (self.rows + c.shared * c.T) * c.I * (4 if c.act in ("nvfp4_all", "mxfp8") else 2)   # fp32 h / h16
        return w + act + h

    def gate_up_flops(self):
        c = self.cfg
        return 2.0 * (self.rows + c.shared * c.T) * 2 * c.I * c.H

    def layer_bytes(self):
        c = self.cfg
        w = (self.touched + c.shared) * (self.weight_bytes(2 * c.I * c.H) + self.weight_bytes(c.H * c.I))
        return w + c.T * c.H * 2 + c.T * c.E * 4 + c.T * c.H * 2

    def layer_flops(self):
        c = self.cfg
        return 6.0 * (self.rows + c.shared * c.T) * c.I * c.H


def cpu_baseline(cfgs, budget_s=6.0):
    """The CPU oracle, untouched, on a bounded sample: the largest decode batch of the
    workload (or 16 tokens of a prefill workload), repeated until budget_s has passed."""
    import oracle
    import oracle.moe as omoe
    o = oracle.default()
    cfg = max(cfgs, key=lambda c: c.T)
    tokens = np.arange(cfg.T, dtype=np.int32) if cfg.T <= 64 else synth.token_sample(cfg, 16)
    logits = synth.logits(cfg)
    ids, _ = omoe.route(cfg, logits, o)
    need = sorted(set(ids[tokens].reshape(-1).tolist()))
    log(f"[bench] cpu baseline: preparing the weights of {len(need)} experts for the oracle (untimed)")
    W1 = omoe.projection_weights(cfg, "w1", need)
    W2 = omoe.projection_weights(cfg, "w2", need)
    WS1 = omoe.projection_weights(cfg, "ws1") if cfg.shared else None
    WS2 = omoe.projection_weights(cfg, "ws2") if cfg.shared else None
    x = synth.activations(cfg)
    n_tok, t0, reps = 0, time.perf_counter(), 0
    while True:
        omoe.forward(cfg, x, logits, W1, W2, WS1, WS2, tokens=tokens, o=o)
        n_tok += len(tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": n_tok / el, "unit": "tokens/s", "cores": min(o.threads(), len(tokens)), "kind": "oracle",
            "sample": f"{cfg.name}: {len(tokens)} tokens (routing, {'activation quantisation, ' if cfg.act != 'bf16' else ''}"
                      f"FP64 expert MLPs of their {cfg.k} experts, combine) x {reps} repeats, {el:.1f} s; "
                      f"weight preparation untimed"}


# ------------------------------------------------------------ rocprofv3 summaries

STAGE_OF_MODE = {"0": "gate_up", "1": "gate_up", "3": "gate_up", "5": "gate_up", "2": "down", "4": "down", "6": "down"}
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("gemm.hip", "common.hpp", "kernels.hpp", "api.cpp")   # kernels + their launch choices


def kernel_source_hash():
    """sha256 over the GEMM kernel sources (a traffic record is valid only for these)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_stage(name):
    """Layer stage of a kernel name from the trace (gate_up / down / route / ...)."""
    import re
    mm = re.search(r"gemm_\w+_kernel<(\d+)", name)
    if mm:
        return STAGE_OF_MODE.get(mm.group(1), "gemm")
    for key, st in (("plan", "route"), ("route", "route"), ("combine", "combine"),
                    ("quant_rows_kernel<float>", "down"), ("mxfp8_rows_kernel<float>", "down"),   # h before down
                    ("quant", "quant"), ("mxfp8_rows", "quant"), ("rows_to_f16", "quant"), ("pack", "pack"),
                    ("group_gs", "pack")):
        if key in name:
            return st
    return "other"


def trace_summary(db, title, command):
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration), "
                       "max(grid_x), max(grid_y), max(workgroup_x), max(vgpr_count), max(accum_vgpr_count), "
                       "max(lds_size) from kernels group by name order by sum(duration) desc").fetchall()
    out = [f"# {title}", "", "Command (on one MI355X, from the repository root):", "", "```", command, "```", "",
           "| kernel | stage | calls | avg us | min us | max us | total ms | grid (x,y) | wg | vgpr/agpr | lds B |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    stage = {}
    for n, c, a, mn, mx, t, gx, gy, wg, v, ag, lds in rows:
        short = n.replace("nvmoe::", "").split("(")[0]
        st = kernel_stage(short)
        stage.setdefault(st, [0, 0.0])
        stage[st][0] += c
        stage[st][1] += t
        out.append(f"| `{short}` | {st} | {c} | {a / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {t / 1e6:.3f} | "
                   f"{gx},{gy} | {wg} | {v}/{ag} | {lds} |")
    out += ["", "Per stage (all launches of the stage's kernels):", "", "| stage | launches | avg us per launch |",
            "|---|---|---|"]
    for st, (c, t) in sorted(stage.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| {st} | {c} | {t / c / 1e3:.2f} |")
    return "\n".join(out)


def _pmc_per_dispatch(path, counter):
    """{dispatch_id: (kernel name, grid, value summed over the counter's instances)} from a rocprofv3 csv."""
    import csv
    res = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name = r["Kernel_Name"].replace("nvmoe::", "").split("(")[0]
        prev = res.get(d, (name, int(r["Grid_Size"]), 0.0))
        res[d] = (name, int(r["Grid_Size"]), prev[2] + float(r["Counter_Value"]))
    return res


def traffic_summary(fetch_csv, write_csv, workload_name, title, command):
    """HBM bytes per gate/up launch from FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch),
    each scaled by what the counter reads for the 1 GiB device copy of --copy-probe."""
    fetch = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)

    def copy_kib(d):
        big = [v for (n, g, v) in d.values() if "copy" in n.lower() or "elementwise" in n.lower()]
        return max(big) if big else None
    cf, cw = copy_kib(fetch), copy_kib(write)
    f_scale = gib_kib / cf if cf else 1.0
    w_scale = gib_kib / cw if cw else 1.0
    out = [f"# {title}", "", "Commands (on one MI355X, from the repository root):", "", "```", command, "```", "",
           f"Calibration: the 1 GiB device copy reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB, "
           f"so FETCH_SIZE is scaled by {f_scale:.3f} and WRITE_SIZE by {w_scale:.3f} (1 GiB = {gib_kib:.0f} KiB).",
           "", "| kernel | stage | grid | dispatches | FETCH MB (scaled) | WRITE MB (scaled) |", "|---|---|---|---|---|---|"]
    groups = {}
    for d, (n, g, v) in fetch.items():
        key = (n, g)
        wv = write.get(d, (n, g, None))[2]
        groups.setdefault(key, []).append((v * f_scale * 1024, None if wv is None else wv * w_scale * 1024))
    # the write run has its own dispatch ids; pair by (kernel, grid) and order
    wgroups = {}
    for d, (n, g, v) in sorted(write.items()):
        wgroups.setdefault((n, g), []).append(v * w_scale * 1024)
    gu = []
    for (n, g), lst in sorted(groups.items()):
        fb = [a for a, _ in lst]
        wb = wgroups.get((n, g), [])
        st = kernel_stage(n)
        fmean = sum(fb) / len(fb)
        wmean = sum(wb) / len(wb) if wb else float("nan")
        out.append(f"| `{n}` | {st} | {g} | {len(fb)} | {fmean / 1e6:.2f} | {wmean / 1e6:.2f} |")
        if st == "gate_up":
            gu.append((g, fmean, wmean))
    per_launch = sum(f + w for _, f, w in gu) / len(gu) if gu else None
    rec = {"workload": workload_name, "kernel": "gate_up", "bytes_per_launch": per_launch,
           "launches_averaged": len(gu), "source_sha256": kernel_source_hash()}
    out += ["", "Mean HBM traffic (FETCH + WRITE, scaled) per gate/up launch: "
            + ("n/a" if per_launch is None else f"{per_launch / 1e6:.2f} MB"), "",
            "traffic-record: " + json.dumps(rec)]
    return "\n".join(out)


def counter_summary(csvs, title, command):
    """Per-kernel means of every counter in one or more rocprofv3 --pmc runs (values summed
    over a dispatch's instances, then averaged over the kernel's dispatches of one grid),
    plus the derived figures the dequant route is judged by: VALU instructions per MFMA,
    MFMA-pipe busy share (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE / 8
    XCDs), the clock the kernel ran at (GRBM_GUI_ACTIVE / 8 / duration) and LDS
    instructions per MFMA."""
    import csv
    rows = {}
    for path in csvs:
        per = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].replace("nvmoe::", "").replace("void ", "").split("(")[0]
            key = (name, int(r["Grid_Size"]))
            d = (path, int(r["Dispatch_Id"]))
            c = r["Counter_Name"]
            e = per.setdefault(d, {"key": key, "dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            e[c] = e.get(c, 0.0) + float(r["Counter_Value"])
        for d, e in per.items():
            agg = rows.setdefault(e["key"], {})
            for c, v in e.items():
                if c != "key":
                    agg.setdefault(c, []).append(v)
    out = [f"# {title}", "", "Commands (on one MI355X, from the repository root):", "", "```", command, "```", "",
           "| kernel | stage | grid | dispatches | counter means per dispatch | VALU/MFMA | LDS/MFMA | MFMA busy | clock GHz |",
           "|---|---|---|---|---|---|---|---|---|"]
    for (n, g), agg in sorted(rows.items(), key=lambda kv: (kernel_stage(kv[0][0]), kv[0])):
        st = kernel_stage(n)
        if st not in ("gate_up", "down"):
            continue
        m = {c: sum(v) / len(v) for c, v in agg.items()}
        ndisp = max(len(v) for c, v in agg.items() if c != "dur")
        mf = m.get("SQ_INSTS_MFMA")
        ratio = lambda c: f"{m[c] / mf:.2f}" if mf and c in m else "-"
        gui = m.get("GRBM_GUI_ACTIVE")
        busy = (f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * gui / 8):.3f}"
                if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m else "-")
        clk = f"{gui / 8 / m['dur']:.2f}" if gui and m.get("dur") else "-"
        cs = ", ".join(f"{c.replace('SQ_', '')} {v:.4g}" for c, v in sorted(m.items()) if c != "dur")
        out.append(f"| `{n}` | {st} | {g} | {ndisp} | {cs} | {ratio('SQ_INSTS_VALU')} | {ratio('SQ_INSTS_LDS')} | "
                   f"{busy} | {clk} |")
    return "\n".join(out)


def traffic_record(workload_name):
    """The measured gate/up traffic per launch for this workload if its record matches the
    kernel sources built now, else None."""
    if not os.path.isdir(PROFILES):
        return None
    want = kernel_source_hash()
    for f in sorted(os.listdir(PROFILES)):
        if not f.endswith(".md"):
            continue
        for line in open(os.path.join(PROFILES, f)):
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
                if rec.get("workload") == workload_name and rec.get("source_sha256") == want:
                    return rec.get("bytes_per_launch")
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3-30b-a3b-decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration for --pmc runs)")
    ap.add_argument("--trace-summary", metavar="RESULTS_DB", help="summarise a rocprofv3 kernel trace and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise FETCH_SIZE / WRITE_SIZE counter runs and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_CSV",
                    help="tabulate the counters of rocprofv3 --pmc runs per GEMM kernel and exit")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.title, args.command))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary, args.title, args.command))
        return
    if args.traffic_summary:
        print(traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload, args.title,
                              args.command))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfgs, bound = workload(args.workload)
    batches = [Batch(c, dev) for c in cfgs]

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step():
        for b in batches:
            b.run()

    # eager launches
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # the same step captured once in a HIP graph and replayed (fixed pointers; the layer
    # enqueues no memset and never synchronises, so it is capturable as is)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    tokens = sum(c.T for c in cfgs)
    value = tokens / (ms / 1e3)
    # the per-step distribution: K more replays, each between two events on the replay stream
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for e0, e1 in step_ev:
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    step_samples = [e0.elapsed_time(e1) for e0, e1 in step_ev]

    # dominant kernel: gate/up GEMM, timed by HIP events recorded on its launch stream
    # (moe_run_timed records them around each stage on the stream moe_run uses)
    stage_tot = {b.cfg.name: [0.0] * m.MOE_NUM_STAGES for b in batches}
    all_ev = {b.cfg.name: [torch.cuda.Event(enable_timing=True) for _ in range(2 * m.MOE_NUM_STAGES)]
              for b in batches}
    for ev in all_ev.values():                  # materialise the HIP events before handing them over
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for b in batches:
            ev = all_ev[b.cfg.name]
            b.run_timed([e.cuda_event for e in ev])
        torch.cuda.synchronize()
        for b in batches:
            ev = all_ev[b.cfg.name]
            for s in range(m.MOE_NUM_STAGES):
                stage_tot[b.cfg.name][s] += ev[2 * s].elapsed_time(ev[2 * s + 1])
    per_launch = {n: [t / args.steps for t in v] for n, v in stage_tot.items()}
    gu_time = sum(v[m.MOE_STAGE_GATE_UP] for v in per_launch.values())          # ms per step
    if bound == "hbm":
        work = sum(b.gate_up_bytes() for b in batches)
        achieved = work / (gu_time / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    else:
        work = sum(b.gate_up_flops() for b in batches)
        achieved = work / (gu_time / 1e3) / 1e12
        peak = FP8_PEAK_TFLOPS if cfgs[0].act == "mxfp8" else BF16_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["kernel"] = "gate_up grouped GEMM (+SwiGLU)"
    roof["launch_ms"] = gu_time / len(batches)
    roof["algorithmic_bytes_per_launch"] = sum(b.gate_up_bytes() for b in batches) / len(batches)
    roof["traffic"] = traffic_record(args.workload)

    layer_bytes = sum(b.layer_bytes() for b in batches)
    layer_flops = sum(b.layer_flops() for b in batches)
    detail = {}
    for b in batches:
        st = per_launch[b.cfg.name]
        detail[b.cfg.name] = {
            "T": b.cfg.T, "touched_experts": b.touched,
            "stage_ms": {m.STAGE_NAMES[s]: round(st[s], 5) for s in range(m.MOE_NUM_STAGES)},
            "expert_rows": b.expert_rows,
            "useful_weight_bytes": (b.touched + b.cfg.shared) * (b.weight_bytes(2 * b.cfg.I * b.cfg.H)
                                                                 + b.weight_bytes(b.cfg.H * b.cfg.I)),
            "gate_up_GBps": b.gate_up_bytes() / (st[m.MOE_STAGE_GATE_UP] / 1e3) / 1e9,
            "gate_up_TFLOPs": b.gate_up_flops() / (st[m.MOE_STAGE_GATE_UP] / 1e3) / 1e12,
        }

    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8xfp4" if cfgs[0].act == "mxfp8" else "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "T": [c.T for c in cfgs], "H": cfgs[0].H, "I": cfgs[0].I,
                   "E": cfgs[0].E, "top_k": cfgs[0].k, "score": cfgs[0].score, "shared": cfgs[0].shared,
                   "activations": cfgs[0].act,
                   "weights": ("mxfp4 e2m1 + e8m0/32" if cfgs[0].wfmt == "mxfp4"
                               else "nvfp4 e2m1 + e4m3/16 + fp32 per expert")},
        "launch": "hip graph replay of the step (eager: %.4f ms/step)" % eager_ms,
        "eager_ms_per_step": eager_ms,
        "step_ms_median": float(np.median(step_samples)),
        "step_ms_iqr": [float(np.percentile(step_samples, 25)), float(np.percentile(step_samples, 75))],
        "step_ms_samples": [round(v, 5) for v in step_samples],
        "layer_GBps": layer_bytes / (ms / 1e3) / 1e9,
        "layer_TFLOPs": layer_flops / (ms / 1e3) / 1e12,
        "roofline": roof,
        "per_batch": detail,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfgs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
