"""Benchmark of the NVFP4 block-scaled fused-MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--headline-only]
                    [--no-cpu-baseline]

Default run: the Qwen3-30B-A3B-shaped decode layer (H=2048, I=768, E=128, top-8, NVFP4
weights, BF16 activations) as the headline. One step runs the whole layer once for each
decode batch T in {1, 8, 32, 64} (105 tokens), each batch with its own seeded weights,
inputs and logits, so the 1.36 GB of weights the step streams exceed the 256 MB Infinity
Cache. Beside it, in the same JSON line, the same measurement of the prefill
configurations (the Qwen3 shape at T=4096; the DeepSeek-V3-shaped layer, T=8192, H=7168,
I=2048, E=256, top-8 sigmoid router, one shared expert) under "prefill", and of the
skewed W4A4 layer (T=512, H=4096, I=1536, E=64, top-4, Zipf-biased router, NVFP4
row-quantised activations) under "skewed".

Order: every batch is prepared and run once; then the oracle leg (unless
--no-cpu-baseline) times the CPU oracle on a bounded sample and checks every batch's first
run against the oracle (routing bit-exact, output within the parity tests' bar: every token
of a decode batch, a seeded token sample of the prefill-sized ones); a mismatch prints the
parity record and exits with status 1 before anything is timed. Inputs are resident in HBM
before timing; each workload first runs untimed for one second (the GPU leaves its idle
clocks), then W warmup steps, then exactly K timed steps between two device
synchronisations, eager and as a replayed HIP graph (the serving launch path; after its
capture the graph replays untimed for another second, since the capture's idle time drops
the clocks again).

The JSON line holds: tokens/s of the headline step (value, graph replay), the per-step
distribution of K further replays (median, IQR, samples), the layer's HBM rate and its
fraction of 8 TB/s, plus
  roofline:     the dominant kernel (the gate/up grouped GEMM) timed with HIP
                events recorded on its launch stream over K further steps:
                algorithmic bytes per launch / mean launch time vs 8 TB/s HBM
                (decode) or algorithmic FLOPs / time vs 2.5 PFLOP/s bf16 MFMA
                (prefill workloads);
  prefill / skewed: per workload step time, tokens/s, the layer's TFLOP/s and GB/s against
                the MFMA and HBM peaks, and each grouped GEMM's (gate_up, down) rate and
                fractions from the same kernel-stamped events;
  parity:       the oracle checks the timing was gated on;
  host:         CPU model and threads, GPU name, clocks, power and use before timing;
  cpu_baseline: the CPU oracle (FP64, OpenMP) on a bounded sample of the headline
                workload, on this host's cores.
Other workloads (--workload qwen3-30b-a3b-prefill | deepseek-v3 | skewed-w4a4 |
skewed-w4a4-all (h quantised to NVFP4 too) | tiny) print the same line for that configuration, and so
do qwen3-30b-a3b-w4a8-decode / -prefill (the Qwen3 layer with x and h FP8 with one scale per
row on NVFP4 weights: T in {1, 8, 32, 64}, and T = 4096) and the router/activation
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
PEAK_SCLK_GHZ = 2.4                             # MI355X peak engine clock


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
    # the Qwen3 layer on the W4A8 path with NVFP4 weights (x and h FP8 with a per-row scale)
    if name == "qwen3-30b-a3b-w4a8-decode":
        return [synth.qwen3_w4a8(T) for T in synth.DECODE_TOKENS], "hbm"
    if name == "qwen3-30b-a3b-w4a8-prefill":
        return [synth.qwen3_w4a8(4096)], "mfma"
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
        # the first run's results, kept on the host for the parity gate
        self.first = {k: v.cpu().numpy() for k, v in bufs.items()}
        self.first_out = self.out.cpu()
        counts = self.first["expert_counts"]
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
        act = c.T * c.H * {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32, "fp8": 1.0 + 4.0 / c.H}.get(
            c.act, NVFP4_BYTES_PER_WEIGHT + 4.0 / c.H)
        h = (self.rows + c.shared * c.T) * c.I * (4 if c.act in ("nvfp4_all", "mxfp8", "fp8") else 2)   # fp32 h / h16
        return w + act + h

    def gate_up_flops(self):
        c = self.cfg
        return 2.0 * (self.rows + c.shared * c.T) * 2 * c.I * c.H

    def down_bytes(self):
        """Weights of the touched experts, the h rows read (h16 with its block exponents, or
        the NVFP4 / MXFP8 / FP8-row h codes and scales) and the y rows written (fp16 + exponents)."""
        c = self.cfg
        rows = self.rows + c.shared * c.T
        w = (self.touched + c.shared) * self.weight_bytes(c.H * c.I)
        h = rows * {"nvfp4_all": c.I * NVFP4_BYTES_PER_WEIGHT + 4, "mxfp8": c.I * (1 + 1.0 / 32),
                    "fp8": c.I + 4.0}.get(c.act, c.I * 2 + c.I / 16)
        return w + h + rows * (c.H * 2 + c.H / 16)

    def down_flops(self):
        c = self.cfg
        return 2.0 * (self.rows + c.shared * c.T) * c.H * c.I

    def layer_bytes(self):
        c = self.cfg
        w = (self.touched + c.shared) * (self.weight_bytes(2 * c.I * c.H) + self.weight_bytes(c.H * c.I))
        return w + c.T * c.H * 2 + c.T * c.E * 4 + c.T * c.H * 2

    def layer_flops(self):
        c = self.cfg
        return 6.0 * (self.rows + c.shared * c.T) * c.I * c.H


# Tokens of a prefill-sized batch the parity gate compares with the oracle (decode batches: all)
PARITY_SAMPLE = {"qwen3-30b-a3b-prefill": 48, "skewed-w4a4": 48, "skewed-w4a4-all": 48, "deepseek-v3": 4,
                 "deepseek-v3-noaux-t8192": 4, "deepseek-v4-flash-t8192": 8, "deepseek-v4-flash-w4a8-t8192": 8,
                 "qwen3-30b-a3b-w4a8-t4096": 48}
PARITY_REL_L2, PARITY_MAX_OVER_RMS, PARITY_W_ABS = 5e-3, 2e-2, 1e-6
PARITY_MAX_FLIPS = 2     # h codes per token that may lie on the other side of a rounding boundary


def _beyond_bf16(o, r, rms):
    """max(|o - r| - half a bf16 ulp of r) / rms: the error beyond the output's own rounding."""
    _, ex = np.frexp(r)
    half_ulp = np.where(r == 0, 0.0, np.ldexp(1.0, ex - 9))
    return float(max((np.abs(o - r) - half_ulp).max(), 0.0) / rms)


def _parity_check(b, ref, tokens, flips=None):
    """The first run of batch b against the oracle's result `ref` for `tokens`: routing ids,
    counts, offsets and permutation bit-exact, routing weights within 1e-6, quantised
    activations bit-exact, and the output within relL2 <= 5e-3 and a max error beyond the
    bf16 output rounding <= 2e-2 RMS (the parity tests' bar). For the variants that quantise
    h, `flips(t)` lists the output changes of the other rounding of token position t's h
    elements within a tiny distance of a code boundary (found on the oracle side): as in the
    parity tests, a token over the max bar may take up to two of them."""
    f = b.first
    routing_ok = (np.array_equal(f["topk_ids"], ref["ids"]) and np.array_equal(f["expert_counts"], ref["counts"])
                  and np.array_equal(f["expert_offsets"], ref["offsets"]) and np.array_equal(f["perm"], ref["perm"])
                  and float(np.abs(f["topk_weights"] - ref["w"]).max()) <= PARITY_W_ABS)
    act_ok = True
    if "xq" in ref and "act_packed" in f:
        act_ok = np.array_equal(f["act_packed"], ref["xq"])
        if "xs" in ref:
            act_ok = act_ok and np.array_equal(f["act_scales"], ref["xs"])
        if "xg" in ref:
            act_ok = act_ok and np.array_equal(f["act_global"].view(np.uint32), ref["xg"].view(np.uint32))
    o = b.first_out[torch.from_numpy(np.asarray(tokens, np.int64))].float().numpy().astype(np.float64)
    r = ref["out"]
    d = np.abs(o - r)
    rms = float(np.sqrt(np.mean(r * r)))
    _, ex = np.frexp(r)
    half_ulp = np.where(r == 0, 0.0, np.ldexp(1.0, ex - 9))
    rel = float(np.linalg.norm(o - r) / np.linalg.norm(r))
    beyond = float(max((d - half_ulp).max(), 0.0) / rms)
    used = 0
    if flips is not None and beyond > PARITY_MAX_OVER_RMS:
        worst = 0.0
        for t in range(r.shape[0]):
            alt = r[t].copy()
            if _beyond_bf16(o[t], alt, rms) > PARITY_MAX_OVER_RMS:
                cand = flips(t)
                for _ in range(PARITY_MAX_FLIPS):
                    if not cand or _beyond_bf16(o[t], alt, rms) <= PARITY_MAX_OVER_RMS:
                        break
                    best = min(range(len(cand)), key=lambda c: _beyond_bf16(o[t], alt + cand[c], rms))
                    alt = alt + cand.pop(best)
                    used += 1
            worst = max(worst, _beyond_bf16(o[t], alt, rms))
        beyond = worst
    ok = bool(routing_ok and act_ok and rel <= PARITY_REL_L2 and beyond <= PARITY_MAX_OVER_RMS and np.isfinite(o).all())
    res = {"batch": b.cfg.name, "tokens_checked": int(len(tokens)), "tokens": int(b.cfg.T),
           "routing_bit_exact": bool(routing_ok), "activation_codes_bit_exact": bool(act_ok) if "xq" in ref else None,
           "relL2": rel, "max_over_rms": float(d.max() / rms), "beyond_bf16_over_rms": beyond, "ok": ok}
    if used:
        res["h_codes_across_a_boundary"] = used
    return res


def cpu_baseline_and_parity(headline, extra, budget_s=6.0):
    """The CPU oracle, untouched, on a bounded sample (the largest batch of the headline
    workload: all its tokens if it has at most 64, else 16), repeated until budget_s has
    passed; then the parity gate: that result and the oracle's result for every other batch
    (every token of a decode batch, a seeded token sample of a prefill-sized one, evaluated
    one expert at a time) against each batch's first run on the GPU."""
    import oracle
    import oracle.moe as omoe
    o = oracle.default()

    def weights(cfg, need):
        W1 = omoe.projection_weights(cfg, "w1", need)
        W2 = omoe.projection_weights(cfg, "w2", need)
        WS1 = omoe.projection_weights(cfg, "ws1") if cfg.shared else None
        WS2 = omoe.projection_weights(cfg, "ws2") if cfg.shared else None
        return W1, W2, WS1, WS2

    big = max(headline, key=lambda b: b.cfg.T)
    cfg = big.cfg
    tokens = np.arange(cfg.T, dtype=np.int32) if cfg.T <= 64 else synth.token_sample(cfg, 16)
    logits = synth.logits(cfg)
    ids, _ = omoe.route(cfg, logits, o)
    need = sorted(set(ids[tokens].reshape(-1).tolist()))
    log(f"[bench] cpu baseline: preparing the weights of {len(need)} experts for the oracle (untimed)")
    W = weights(cfg, need)
    x = synth.activations(cfg)
    n_tok, t0, reps = 0, time.perf_counter(), 0
    while True:
        ref = omoe.forward(cfg, x, logits, *W, tokens=tokens, o=o)
        n_tok += len(tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    baseline = {"value": n_tok / el, "unit": "tokens/s", "cores": min(o.threads(), len(tokens)), "kind": "oracle",
                "sample": f"{cfg.name}: {len(tokens)} tokens (routing, "
                          f"{'activation quantisation, ' if cfg.act != 'bf16' else ''}"
                          f"FP64 expert MLPs of their {cfg.k} experts, combine) x {reps} repeats, {el:.1f} s; "
                          f"weight preparation untimed"}
    def flips(cfg, ref, W, tokens):
        if cfg.act not in omoe.HQ:                       # h is not quantised: no boundary to cross
            return None
        return lambda t: omoe.h_flip_candidates(cfg, ref, W, int(tokens[t]), o)

    checks = [_parity_check(big, ref, tokens, flips(cfg, ref, W, tokens))]
    log(f"[bench] parity {checks[-1]}")
    for b in [b for b in headline if b is not big] + list(extra):
        cfg = b.cfg
        n = PARITY_SAMPLE.get(cfg.name, 16)
        tokens = np.arange(cfg.T, dtype=np.int32) if cfg.T <= 64 else synth.token_sample(cfg, n)
        logits = synth.logits(cfg)
        ids, _ = omoe.route(cfg, logits, o)
        need = sorted(set(ids[tokens].reshape(-1).tolist()))
        log(f"[bench] parity: oracle for {len(tokens)} tokens of {cfg.name} ({len(need)} experts)")
        Wn = weights(cfg, need)
        ref = omoe.forward_by_expert(cfg, synth.activations(cfg), logits, *Wn, tokens=tokens, o=o)
        checks.append(_parity_check(b, ref, tokens, flips(cfg, ref, Wn, tokens)))
        log(f"[bench] parity {checks[-1]}")
    parity = {"status": "ok" if all(c["ok"] for c in checks) else "FAILED",
              "bar": "routing and activation codes bit-exact; relL2 <= 5e-3; max |d| beyond the bf16 output "
                     "rounding <= 2e-2 RMS (quantised-h variants: up to 2 h codes per token on the other side of "
                     "a rounding boundary they lie within 2e-5 of)", "checks": checks}
    return baseline, parity


def host_info():
    """CPU model and thread count of this host; GPU name, clocks, power and use before timing."""
    info = {"cpu_model": None, "cpu_threads": len(os.sched_getaffinity(0))}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["gpu"] = torch.cuda.get_device_properties(0).name
    try:
        import shutil
        import subprocess
        # rocm-smi is a Python script: run it with this interpreter as a child process (its
        # "#!/usr/bin/env python3" line would re-exec, which a profiled process must not do)
        smi = os.path.realpath(shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi")
        r = subprocess.run([sys.executable, smi, "--showclocks", "--showpower", "--showuse", "--showtemp", "--json"],
                           capture_output=True, text=True, timeout=30)
        card = next(iter(json.loads(r.stdout).values()))
        keep = ("sclk clock speed:", "mclk clock speed:", "GPU use (%)", "Temperature (Sensor junction) (C)")
        info["gpu_state"] = {k: v for k, v in card.items() if k in keep or "Power" in k}
    except Exception as exc:   # the state is a record, not a requirement
        info["gpu_state"] = f"unavailable: {type(exc).__name__}"
    return info


# ------------------------------------------------------------ rocprofv3 summaries

STAGE_OF_MODE = {"0": "gate_up", "1": "gate_up", "5": "gate_up", "2": "down", "4": "down", "6": "down"}
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
    if "down_persist" in name:    # the persistent prefill down GEMM (its first argument is not a mode)
        return "down"
    mm = re.search(r"gemm_\w+_kernel<(\d+)", name)
    if mm:
        return STAGE_OF_MODE.get(mm.group(1), "gemm")
    for key, st in (("plan", "route"), ("route", "route"), ("combine", "combine"),
                    ("quant_rows_kernel<float>", "h_prep"), ("mxfp8_rows_kernel<float>", "h_prep"),   # h before down
                    ("fp8_rows_kernel<float>", "h_prep"), ("h_rescale", "h_prep"),
                    ("quant", "quant"), ("mxfp8_rows", "quant"), ("fp8_rows", "quant"), ("pack", "pack"),
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
    LDS instructions per MFMA, and the MFMA-pipe busy share = SQ_VALU_MFMA_BUSY_CYCLES over
    (1024 SIMDs x the kernel's cycles). The kernel's cycles are its duration (dispatch
    timestamps) times its clock; the clock is GRBM_GUI_ACTIVE / 8 XCDs / duration where that
    is at most the 2.4 GHz peak. GRBM_GUI_ACTIVE counts over a window that can outlast a
    short kernel, so where it gives more than 2.4 GHz the clock is taken as 2.4 GHz (a lower
    bound on the busy share) and the row is flagged."""
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
        gui, dur = m.get("GRBM_GUI_ACTIVE"), m.get("dur")
        busy = clk = "-"
        if gui and dur:
            ghz = gui / 8 / dur
            capped = ghz > PEAK_SCLK_GHZ
            cycles = dur * min(ghz, PEAK_SCLK_GHZ)
            clk = f"{min(ghz, PEAK_SCLK_GHZ):.2f}" + (f" (GRBM window {ghz:.2f}: capped)" if capped else "")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                busy = f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cycles):.3f}" + (" (lower bound)" if capped else "")
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
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (the CPU baseline and the parity gate)")
    ap.add_argument("--headline-only", action="store_true",
                    help="default workload: time the decode headline only, not the prefill and skewed objects")
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
    host = host_info()
    cfgs, bound = workload(args.workload)
    batches = [Batch(c, dev) for c in cfgs]
    extras = []                                  # (object, workload name, batches, bound)
    if args.workload == DEFAULT_WORKLOAD and not args.headline_only:
        for kind, name in EXTRA_WORKLOADS:
            ecfgs, ebound = workload(name)
            extras.append((kind, name, [Batch(c, dev) for c in ecfgs], ebound))

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # parity first: no timing unless every batch's first run matched the oracle
    baseline = parity = None
    if not args.no_cpu_baseline:
        baseline, parity = cpu_baseline_and_parity(batches, [b for _, _, bs, _ in extras for b in bs])
        if parity["status"] != "ok":
            print(json.dumps({"metric": METRIC, "error": "parity check against the oracle failed", "parity": parity}),
                  flush=True)
            sys.exit(1)

    t = time_steps(batches, args.steps, args.warmup)
    ms = t["ms"]
    tokens = sum(c.T for c in cfgs)
    value = tokens / (ms / 1e3)
    per_launch = t["per_launch"]
    gu_time = sum(v[m.MOE_STAGE_GATE_UP] for v in per_launch.values())          # ms per step
    if bound == "hbm":
        work = sum(b.gate_up_bytes() for b in batches)
        achieved = work / (gu_time / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    else:
        work = sum(b.gate_up_flops() for b in batches)
        achieved = work / (gu_time / 1e3) / 1e12
        peak = mfma_peak(cfgs[0])
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["kernel"] = "gate_up grouped GEMM (+SwiGLU)"
    roof["launch_ms"] = gu_time / len(batches)
    roof["algorithmic_bytes_per_launch"] = sum(b.gate_up_bytes() for b in batches) / len(batches)
    roof["traffic"] = traffic_record(args.workload)

    layer_bytes = sum(b.layer_bytes() for b in batches)
    layer_flops = sum(b.layer_flops() for b in batches)
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"mxfp8": "fp8xfp4", "fp8": "f16"}.get(cfgs[0].act, "bf16"), "data": "synthetic",
        "config": {"workload": args.workload, "T": [c.T for c in cfgs], "H": cfgs[0].H, "I": cfgs[0].I,
                   "E": cfgs[0].E, "top_k": cfgs[0].k, "score": cfgs[0].score, "shared": cfgs[0].shared,
                   "activations": cfgs[0].act,
                   "weights": ("mxfp4 e2m1 + e8m0/32" if cfgs[0].wfmt == "mxfp4"
                               else "nvfp4 e2m1 + e4m3/16 + fp32 per expert")},
        "launch": "hip graph replay of the step (eager: %.4f ms/step)" % t["eager_ms"],
        "eager_ms_per_step": t["eager_ms"],
        "step_ms_median": float(np.median(t["samples"])),
        "step_ms_iqr": [float(np.percentile(t["samples"], 25)), float(np.percentile(t["samples"], 75))],
        "step_ms_samples": [round(v, 5) for v in t["samples"]],
        "layer_GBps": layer_bytes / (ms / 1e3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "layer_TFLOPs": layer_flops / (ms / 1e3) / 1e12,
        "roofline": roof,
        "per_batch": {b.cfg.name: batch_record(b, per_launch[b.cfg.name]) for b in batches},
    }
    for kind, name, bs, eb in extras:
        log(f"[bench] timing {name}")
        res.setdefault(kind, {})[name] = workload_record(bs, time_steps(bs, args.steps, args.warmup), eb)
    if parity is not None:
        res["parity"] = parity
    res["host"] = host
    if baseline is not None:
        res["cpu_baseline"] = baseline
    print(json.dumps(res), flush=True)


DEFAULT_WORKLOAD = "qwen3-30b-a3b-decode"
PRIME_S = 1.0       # untimed seconds of steps before a workload's warmup steps
# measured beside the decode headline in the default run: the prefill configurations (MFMA
# bound) and the skewed W4A4 layer (mixed)
EXTRA_WORKLOADS = (("prefill", "qwen3-30b-a3b-prefill"), ("prefill", "deepseek-v3"), ("skewed", "skewed-w4a4"))


def mfma_peak(cfg):
    return FP8_PEAK_TFLOPS if cfg.act == "mxfp8" else BF16_PEAK_TFLOPS


def time_steps(batches, steps, warmup):
    """Eager and HIP-graph timing of one step (every batch once), the per-step distribution
    of further replays, and each stage's kernel time per launch from moe_run_timed's events."""
    def step():
        for b in batches:
            b.run()

    # bring the GPU out of its idle clocks (the oracle leg before this keeps it idle for tens
    # of seconds): the step runs untimed for PRIME_S seconds before the warmup steps
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PRIME_S:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps

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
    # the capture leaves the GPU idle long enough to drop its clocks: replay untimed for
    # PRIME_S seconds again (without it the first replays of a prefill step ran ~15% slower,
    # eager steps after the same pause likewise)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PRIME_S:
        for _ in range(8):
            graph.replay()
        torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in step_ev:
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    samples = [e0.elapsed_time(e1) for e0, e1 in step_ev]
    del graph

    # stage times: HIP events recorded by moe_run_timed on the stream the layer launches on
    # (after the replays above, so at the same working clocks)
    stage_tot = {b.cfg.name: [0.0] * m.MOE_NUM_STAGES for b in batches}
    all_ev = {b.cfg.name: [torch.cuda.Event(enable_timing=True) for _ in range(2 * m.MOE_NUM_STAGES)]
              for b in batches}
    for ev in all_ev.values():                  # materialise the HIP events before handing them over
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    for _ in range(steps):
        for b in batches:
            b.run_timed([e.cuda_event for e in all_ev[b.cfg.name]])
        torch.cuda.synchronize()
        for b in batches:
            ev = all_ev[b.cfg.name]
            for s in range(m.MOE_NUM_STAGES):
                stage_tot[b.cfg.name][s] += ev[2 * s].elapsed_time(ev[2 * s + 1])
    per_launch = {n: [v / steps for v in tot] for n, tot in stage_tot.items()}
    return {"eager_ms": eager_ms, "ms": ms, "samples": samples, "per_launch": per_launch}


def batch_record(b, st):
    """Per-batch detail: stage times, rows per expert, the GEMMs' rates against their roofs."""
    c = b.cfg
    gu, dn = st[m.MOE_STAGE_GATE_UP], st[m.MOE_STAGE_DOWN]
    peak = mfma_peak(c)
    return {
        "T": c.T, "touched_experts": b.touched,
        "stage_ms": {m.STAGE_NAMES[s]: round(st[s], 5) for s in range(m.MOE_NUM_STAGES)},
        "expert_rows": b.expert_rows if len(b.expert_rows) <= 128 else b.expert_rows[:16] + ["..."],
        "useful_weight_bytes": (b.touched + c.shared) * (b.weight_bytes(2 * c.I * c.H) + b.weight_bytes(c.H * c.I)),
        "gate_up_GBps": b.gate_up_bytes() / (gu / 1e3) / 1e9,
        "gate_up_hbm_frac": b.gate_up_bytes() / (gu / 1e3) / 1e9 / HBM_PEAK_GBS,
        "gate_up_TFLOPs": b.gate_up_flops() / (gu / 1e3) / 1e12,
        "gate_up_mfma_frac": b.gate_up_flops() / (gu / 1e3) / 1e12 / peak,
        "down_GBps": b.down_bytes() / (dn / 1e3) / 1e9,
        "down_hbm_frac": b.down_bytes() / (dn / 1e3) / 1e9 / HBM_PEAK_GBS,
        "down_TFLOPs": b.down_flops() / (dn / 1e3) / 1e12,
        "down_mfma_frac": b.down_flops() / (dn / 1e3) / 1e12 / peak,
    }


def workload_record(batches, t, bound):
    """One extra workload of the default run: step time and rates, the layer's and each
    grouped GEMM's fraction of the MFMA peak (and of HBM bandwidth), per-batch detail."""
    ms = t["ms"]
    c = batches[0].cfg
    peak = mfma_peak(c)
    flops = sum(b.layer_flops() for b in batches)
    nbytes = sum(b.layer_bytes() for b in batches)
    gu = sum(v[m.MOE_STAGE_GATE_UP] for v in t["per_launch"].values())
    dn = sum(v[m.MOE_STAGE_DOWN] for v in t["per_launch"].values())
    gu_f, dn_f = sum(b.gate_up_flops() for b in batches), sum(b.down_flops() for b in batches)
    gu_b, dn_b = sum(b.gate_up_bytes() for b in batches), sum(b.down_bytes() for b in batches)
    return {
        "bound": bound, "T": [b.cfg.T for b in batches], "H": c.H, "I": c.I, "E": c.E, "top_k": c.k,
        "shared": c.shared, "activations": c.act,
        "ms_per_step": ms, "eager_ms_per_step": t["eager_ms"], "step_ms_median": float(np.median(t["samples"])),
        "tokens_per_s": sum(b.cfg.T for b in batches) / (ms / 1e3),
        "layer_TFLOPs": flops / (ms / 1e3) / 1e12, "layer_mfma_frac": flops / (ms / 1e3) / 1e12 / peak,
        "layer_GBps": nbytes / (ms / 1e3) / 1e9, "layer_hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "mfma_peak_TFLOPs": peak,
        "gate_up": {"ms": gu, "TFLOPs": gu_f / (gu / 1e3) / 1e12, "mfma_frac": gu_f / (gu / 1e3) / 1e12 / peak,
                    "GBps": gu_b / (gu / 1e3) / 1e9, "hbm_frac": gu_b / (gu / 1e3) / 1e9 / HBM_PEAK_GBS},
        "down": {"ms": dn, "TFLOPs": dn_f / (dn / 1e3) / 1e12, "mfma_frac": dn_f / (dn / 1e3) / 1e12 / peak,
                 "GBps": dn_b / (dn / 1e3) / 1e9, "hbm_frac": dn_b / (dn / 1e3) / 1e9 / HBM_PEAK_GBS},
        "per_batch": {b.cfg.name: batch_record(b, t["per_launch"][b.cfg.name]) for b in batches},
    }


if __name__ == "__main__":
    main()
