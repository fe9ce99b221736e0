"""Helpers shared by the GPU parity tests (inputs from synth, expected values from
the oracle, device results through the C ABI)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
import oracle
import oracle.moe as omoe
import nvfp4_block_scaled_router_amd as m
from nvfp4_block_scaled_router_amd.weights import quantize_projection

DEV = torch.device("cuda:0")

# Output tolerance of the layer (fixed for every configuration). The max bound applies to
# the error beyond rounding the exact result to the bf16 output format: half a bf16 ulp is
# up to 2^-8 |out|, which alone exceeds 2e-2 RMS wherever |out| > 5 RMS.
REL_L2 = 5e-3
MAX_OVER_RMS = 2e-2
W_ABS = 1e-6       # routing weights, fp32 vs fp64


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16(x_u16: np.ndarray) -> torch.Tensor:
    return up(x_u16.view(np.int16)).view(torch.bfloat16)


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |ref|: the largest error of rounding ref to
    the layer's bf16 output (8 significant bits, round to nearest even)."""
    _, ex = np.frexp(ref)                       # |ref| in [2^(ex-1), 2^ex)
    return np.where(ref == 0, 0.0, np.ldexp(1.0, ex - 9))


def out_metrics(o_gpu: torch.Tensor, ref: np.ndarray):
    """relL2, max|d|/RMS, and max(|d| - half bf16 ulp of ref)/RMS: the error beyond the
    output format's own rounding, which no bf16 result can avoid."""
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    d = np.abs(o - ref)
    rms = np.sqrt(np.mean(ref * ref))
    rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    return rel, d.max() / rms, max((d - bf16_half_ulp(ref)).max(), 0.0) / rms


# Variants that quantise h (NVFP4 or MXFP8 h rows) decide a code on an intermediate the two
# sides compute differently (FP32 accumulation vs FP64): an h value within FLIP_REL
# (relative) of a rounding boundary may round either way, and both results are correct. For a
# token over the max bound the check may take up to MAX_FLIPS such alternative roundings of
# its h elements, each found on the oracle side (its FP64 h and its quantiser), never from
# the device.
FLIP_REL = omoe.FLIP_REL
MAX_FLIPS = 2


def _beyond(g, r, rms):
    return max((np.abs(g - r) - bf16_half_ulp(r)).max(), 0.0) / rms


def check_out(o_gpu, ref, what="", flips=None):
    """flips: for quantised-h variants, a function token position -> list of output
    changes (one per alternative rounding of an h element near a boundary)."""
    rel, mx, beyond = out_metrics(o_gpu, ref)
    rms = np.sqrt(np.mean(ref * ref))
    g = o_gpu.float().cpu().numpy().astype(np.float64)
    used = 0
    if flips is not None and beyond > MAX_OVER_RMS:
        for t in range(ref.shape[0]):
            if _beyond(g[t], ref[t], rms) <= MAX_OVER_RMS:
                continue
            alt, cand = ref[t].copy(), flips(t)
            for _ in range(MAX_FLIPS):
                if not cand or _beyond(g[t], alt, rms) <= MAX_OVER_RMS:
                    break
                best = min(range(len(cand)), key=lambda c: _beyond(g[t], alt + cand[c], rms))
                alt = alt + cand.pop(best)
                used += 1
            assert _beyond(g[t], alt, rms) <= MAX_OVER_RMS, (what, "token", t, _beyond(g[t], alt, rms))
        beyond = max(_beyond(g[t], ref[t], rms) for t in range(ref.shape[0])) if used == 0 else beyond
    log(f"  {what} relL2 {rel:.3e} (<= {REL_L2}), max|d|/rms {mx:.3e}, "
        f"beyond bf16 rounding {beyond:.3e} (<= {MAX_OVER_RMS})"
        + (f"; {used} h code(s) taken on the other side of a rounding boundary" if used else ""))
    assert rel <= REL_L2 and (used > 0 or beyond <= MAX_OVER_RMS), (rel, mx, beyond)
    assert np.all(np.isfinite(g))


def h_flip_candidates(case, ref, t):
    """Output changes of the alternative roundings of token t's h elements that lie within
    FLIP_REL of a code boundary (MXFP8, FP8-row or NVFP4 h), from the oracle's FP64 h."""
    return omoe.h_flip_candidates(case.cfg, ref, case.W, int(case.tokens[t]), oracle.default())


def gpu_weights(cfg, which):
    """Weights quantised on the device by the library from the synth fp32 draws."""
    G = cfg.shared if which.startswith("ws") else cfg.E
    N, K = (2 * cfg.I, cfg.H) if which in ("w1", "ws1") else (cfg.H, cfg.I)
    return quantize_projection(G, N, K, lambda e0, c: synth.expert_weights_f32(cfg, which, e0, c), DEV,
                               progress=log)


def both_weights(cfg, which, experts=None):
    """Every expert of one projection quantised by the library's device quantiser (the GPU
    side's weights) and the experts in `experts` (all if None) from the same fp32 draws by the
    oracle's (the oracle's weights; the rest stay zero there). The two must agree byte for
    byte. Returns (oracle arrays, device tensors)."""
    o = oracle.default()
    G = cfg.shared if which.startswith("ws") else cfg.E
    N, K = (2 * cfg.I, cfg.H) if which in ("w1", "ws1") else (cfg.H, cfg.I)
    host = (np.zeros((G, N, K // 2), np.uint8), np.zeros((G, N, K // 16), np.uint8), np.zeros(G, np.float32))
    dev = (torch.empty((G, N, K // 2), dtype=torch.uint8, device=DEV),
           torch.empty((G, N, K // 16), dtype=torch.uint8, device=DEV), torch.empty(G, dtype=torch.float32, device=DEV))
    per = max(1, (1 << 30) // (4 * N * K))
    for e0 in range(0, G, per):
        cnt = min(per, G - e0)
        w = synth.expert_weights_f32(cfg, which, e0, cnt)
        m.moe_quantize_nvfp4_weights(torch.from_numpy(w).to(DEV), cnt, N, K, dev[0][e0:e0 + cnt],
                                     dev[1][e0:e0 + cnt], dev[2][e0:e0 + cnt])
        sel = [e for e in range(e0, e0 + cnt) if experts is None or e in experts]
        w = w.reshape(cnt, N, K)
        for e in sel:
            p, sc, g = o.quantize(w[e - e0], rows_per_gs=N)
            host[0][e], host[1][e], host[2][e] = p, sc, g[0]
            for a, d in zip(host, dev):
                assert np.array_equal(a[e], d[e].cpu().numpy()), \
                    f"device weight quantiser differs from the oracle's ({which}, expert {e})"
        log(f"  {which}: experts {e0}..{e0 + cnt - 1} of {G} quantised on the device, {len(sel)} of them also "
            f"by the oracle: bytes identical")
    return host, list(dev)


_WCACHE = {}


def oracle_weights(cfg, which, experts):
    """Oracle-quantised weights, cached per (config, projection, expert set)."""
    key = (cfg, which, None if experts is None else tuple(experts))
    if key not in _WCACHE:
        if len(_WCACHE) > 8:
            _WCACHE.clear()
        _WCACHE[key] = omoe.quantized_weights(cfg, which, experts)
    return _WCACHE[key]


class Case:
    """One configuration on both sides: oracle expectations and the device layer.

    weights: "oracle" -- the oracle's quantiser for both sides (with a token subset, only
    the experts those tokens use are filled; the rest are zero); "gpu" -- every expert
    quantised from the same draws by the library's device quantiser for the GPU side and
    by the oracle's for the oracle side, asserted byte-identical. by_expert: evaluate the
    oracle one expert at a time (oracle.moe.forward_by_expert), for full-size checks."""

    def __init__(self, cfg, tokens=None, weights="oracle", by_expert=False):
        self.cfg = cfg
        self.by_expert = by_expert
        self.x = synth.activations(cfg)
        self.logits = synth.logits(cfg)
        o = oracle.default()
        self.bias = synth.router_bias(cfg)
        self.ids_ref, self.w_ref = omoe.route(cfg, self.logits, o)
        self.tokens = np.arange(cfg.T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
        need = sorted(set(self.ids_ref[self.tokens].reshape(-1).tolist()))
        projs = ["w1", "w2"] + (["ws1", "ws2"] if cfg.shared else [])
        if cfg.wfmt == "mxfp4":   # drawn directly in the boundary format: one set serves both sides
            W = [tuple(synth.mxfp4_weights(cfg, w, 0, cfg.shared if w.startswith("ws") else cfg.E)) + (None,)
                 for w in projs]
            dev = [[up(Wi[0]), up(Wi[1]), None] for Wi in W]
        elif weights == "oracle":
            sel = need if tokens is not None else None
            W = [oracle_weights(cfg, w, sel if w in ("w1", "w2") else None) for w in projs]
            dev = [[up(a) for a in Wi] for Wi in W]
        else:  # every expert, device and oracle quantisers from the same draws
            sel = set(need) if tokens is not None else None
            W, dev = zip(*[both_weights(cfg, w, sel if w in ("w1", "w2") else None) for w in projs])
            W, dev = list(W), list(dev)
        self.W = W
        self.dev_w = dev
        self.need = need

    def reference(self):
        W1, W2 = self.W[0], self.W[1]
        WS1, WS2 = (self.W[2], self.W[3]) if self.cfg.shared else (None, None)
        if self.by_expert:
            return omoe.forward_by_expert(self.cfg, self.x, self.logits, W1, W2, WS1, WS2, tokens=self.tokens,
                                          progress=log)
        return omoe.forward(self.cfg, self.x, self.logits, W1, W2, WS1, WS2, tokens=self.tokens)

    def layer(self, max_tokens=None):
        L = m.MoeLayer.from_config(self.cfg, max_tokens=max_tokens, device=DEV)
        ws = self.dev_w
        L.pack(ws[0], ws[1], ws[2] if self.cfg.shared else None, ws[3] if self.cfg.shared else None)
        if self.bias is not None:
            L.pack_router_bias(up(self.bias))
        return L
