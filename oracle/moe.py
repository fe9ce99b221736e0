"""Oracle-side MoE layer: routing, activation quantisation, expert MLPs, combine.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). Composes the plain C
functions of ``oracle.c`` in the order the method runs them:

1. route the FP32 logits (top-k, renormalised weights; or the generalised router of the
   variant layers), then count/offset/permute;
2. activations: bf16 decoded exactly, or (W4A4) NVFP4 row-quantised with the
   binary32 quantizer and decoded exactly;
3. per token, the k expert SwiGLU MLPs in FP64 (act "nvfp4_all": h row-quantised the
   same way before the down projection; act "mxfp8": x and h MXFP8), weighted sum, plus
   the shared expert with weight 1.

Weights are the synth draws quantised per expert projection by the oracle's
own quantizer (one global scale per expert projection).
"""
from __future__ import annotations

import functools
from typing import Dict, Iterable, Optional

import numpy as np

import synth
from . import default, Oracle


def quantized_weights(cfg: synth.MoeConfig, which: str, experts: Optional[Iterable[int]] = None,
                      o: Optional[Oracle] = None):
    """(packed [G][N][K/2], scales [G][N][K/16], gs [G]) in the boundary layout.

    `which` in {"w1", "w2", "ws1", "ws2"}. With `experts` given, only those
    experts are quantised; the other slots stay zero (np.zeros pages are not
    touched, so a full-size array costs only what is filled)."""
    o = o or default()
    G = cfg.shared if which.startswith("ws") else cfg.E
    N, K = (2 * cfg.I, cfg.H) if which in ("w1", "ws1") else (cfg.H, cfg.I)
    packed = np.zeros((G, N, K // 2), np.uint8)
    scales = np.zeros((G, N, K // 16), np.uint8)
    gs = np.zeros(G, np.float32)
    sel = list(range(G)) if experts is None else sorted(set(int(e) for e in experts))
    chunk = max(1, (1 << 28) // (N * K))             # <= 1 GiB of fp32 draws at a time
    runs = []                                        # maximal runs of consecutive experts
    for e in sel:
        if runs and runs[-1][0] + runs[-1][1] == e and runs[-1][1] < chunk:
            runs[-1][1] += 1
        else:
            runs.append([e, 1])
    for e0, cnt in runs:
        w = synth.expert_weights_f32(cfg, which, e0, cnt)
        p, s, g = o.quantize(w, rows_per_gs=N)      # one global scale per expert projection
        packed[e0:e0 + cnt] = p.reshape(cnt, N, K // 2)
        scales[e0:e0 + cnt] = s.reshape(cnt, N, K // 16)
        gs[e0:e0 + cnt] = g
    return packed, scales, gs


def projection_weights(cfg: synth.MoeConfig, which: str, experts: Optional[Iterable[int]] = None,
                       o: Optional[Oracle] = None):
    """The configuration's weights of one projection as the oracle reads them: NVFP4
    (packed, scales, gs) quantised from the fp32 draws, or MXFP4 (packed, scales, None) as
    drawn. With `experts` given, only those experts are filled (the rest stay zero)."""
    if cfg.wfmt != "mxfp4":
        return quantized_weights(cfg, which, experts, o)
    G = cfg.shared if which.startswith("ws") else cfg.E
    N, K = (2 * cfg.I, cfg.H) if which in ("w1", "ws1") else (cfg.H, cfg.I)
    if experts is None:
        codes, scales = synth.mxfp4_weights(cfg, which, 0, G)
        return codes, scales, None
    codes = np.zeros((G, N, K // 2), np.uint8)
    scales = np.zeros((G, N, K // 32), np.uint8)
    for e in sorted(set(int(e) for e in experts)):
        c, sc = synth.mxfp4_weights(cfg, which, e, 1)
        codes[e], scales[e] = c[0], sc[0]
    return codes, scales, None


@functools.lru_cache(maxsize=4)
def cached_weights(cfg: synth.MoeConfig):
    """All routed and shared weights of a (small) configuration."""
    W1 = quantized_weights(cfg, "w1")
    W2 = quantized_weights(cfg, "w2")
    WS1 = quantized_weights(cfg, "ws1") if cfg.shared else None
    WS2 = quantized_weights(cfg, "ws2") if cfg.shared else None
    return W1, W2, WS1, WS2


def route(cfg: synth.MoeConfig, logits: np.ndarray, o: Optional[Oracle] = None):
    """ids [T][k] and FP64 weights of the configuration's router (plain or generalised)."""
    o = o or default()
    if cfg.variant_router:
        return o.route_general(logits, cfg.k, cfg.score, synth.router_bias(cfg), cfg.n_group, cfg.topk_group,
                               cfg.renorm, cfg.routed_scaling)
    return o.route(logits, cfg.k, cfg.score)


def forward(cfg: synth.MoeConfig, x_bf16: np.ndarray, logits: np.ndarray, W1, W2, WS1=None,
            WS2=None, tokens: Optional[np.ndarray] = None, o: Optional[Oracle] = None) -> Dict:
    """Layer output (FP64, never rounded) for `tokens` (all tokens if None).

    Returns a dict with out [n][H], ids [T][k], w [T][k] (FP64), counts [E],
    offsets [E+1], perm [T*k], inv [T*k], and for W4A4 the quantised
    activations xq [T][H/2], xs [T][H/16], xg [T]."""
    o = o or default()
    T = x_bf16.shape[0]
    tokens = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    ids, w = route(cfg, logits, o)
    counts, offsets, perm, inv = o.plan(ids, cfg.E)
    res = dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv, tokens=tokens)
    if cfg.act == "mxfp8":                               # W4A8: MXFP8 x (and h)
        xf = o.bf16_rows(x_bf16).astype(np.float32)       # exact: bf16 -> binary32
        xq, xs = o.mxfp8_quantize(xf)
        res.update(xq=xq, xs=xs)
        x_rows = o.mxfp8_rows(xq[tokens], xs[tokens])
    elif cfg.act in ("nvfp4", "nvfp4_all"):
        xf = o.bf16_rows(x_bf16).astype(np.float32)       # exact: bf16 -> binary32
        xq, xs, xg = o.quantize(xf, rows_per_gs=1)
        res.update(xq=xq, xs=xs, xg=xg)
        x_rows = o.dequant_rows(xq[tokens], xs[tokens], xg[tokens])
    else:
        x_rows = o.bf16_rows(x_bf16[tokens])
    hq = {"nvfp4_all": 1, "mxfp8": 2}.get(cfg.act, 0)
    res["out"] = o.moe_tokens(W1, W2, WS1, WS2, tokens, x_rows, ids, w, cfg.swiglu_limit, hq=hq)
    return res
