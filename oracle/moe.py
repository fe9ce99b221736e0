"""Oracle-side MoE layer: routing, activation quantisation, expert MLPs, combine.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). Composes the plain C
functions of ``oracle.c`` in the order the method runs them:

1. route the FP32 logits (top-k, renormalised weights; or the generalised router of the
   variant layers), then count/offset/permute;
2. activations: bf16 decoded exactly, or (W4A4) NVFP4 row-quantised with the
   binary32 quantizer and decoded exactly, or MXFP8 (act "mxfp8", MXFP4 weights), or FP8
   with one scale per row (act "fp8", NVFP4 weights: the W4A8 path on NVFP4);
3. per token, the k expert SwiGLU MLPs in FP64 (act "nvfp4_all": h row-quantised the
   same way before the down projection; "mxfp8" and "fp8": h in x's format), weighted
   sum, plus the shared expert with weight 1.

Weights are the synth draws quantised per expert projection by the oracle's
own quantizer (one global scale per expert projection).

``forward`` evaluates the MLPs per token in the C loops (weights decoded element by
element at every use); ``forward_by_expert`` evaluates the same definition one expert
at a time (each expert decoded once, FP64 matrix products as the library step) so that
full-size layers can be checked on every token. Both are pinned, the second against the
first and against a dense numpy layer (tests/pins.py).
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


def _prepare(cfg, x_bf16, logits, tokens, o):
    """forward()'s routing, plan and decoded activation rows (no expert MLP)."""
    T = x_bf16.shape[0]
    tokens = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    ids, w = route(cfg, logits, o)
    counts, offsets, perm, inv = o.plan(ids, cfg.E)
    res = dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv, tokens=tokens)
    if cfg.act == "mxfp8":
        xq, xs = o.mxfp8_quantize(o.bf16_rows(x_bf16).astype(np.float32))
        res.update(xq=xq, xs=xs)
        res["x_rows"] = o.mxfp8_rows(xq[tokens], xs[tokens])
    elif cfg.act == "fp8":                               # NVFP4 weights, FP8 x (and h) per row
        xq, xg = o.fp8_rows_quantize(o.bf16_rows(x_bf16).astype(np.float32))
        res.update(xq=xq, xg=xg)
        res["x_rows"] = o.fp8_rows(xq[tokens], xg[tokens])
    elif cfg.act in ("nvfp4", "nvfp4_all"):
        xq, xs, xg = o.quantize(o.bf16_rows(x_bf16).astype(np.float32), rows_per_gs=1)
        res.update(xq=xq, xs=xs, xg=xg)
        res["x_rows"] = o.dequant_rows(xq[tokens], xs[tokens], xg[tokens])
    else:
        res["x_rows"] = o.bf16_rows(x_bf16[tokens])
    return res


def forward(cfg: synth.MoeConfig, x_bf16: np.ndarray, logits: np.ndarray, W1, W2, WS1=None,
            WS2=None, tokens: Optional[np.ndarray] = None, o: Optional[Oracle] = None) -> Dict:
    """Layer output (FP64, never rounded) for `tokens` (all tokens if None).

    Returns a dict with out [n][H], ids [T][k], w [T][k] (FP64), counts [E],
    offsets [E+1], perm [T*k], inv [T*k], and for W4A4 the quantised
    activations xq [T][H/2], xs [T][H/16], xg [T]."""
    o = o or default()
    res = _prepare(cfg, x_bf16, logits, tokens, o)
    x_rows = res.pop("x_rows")
    hq = HQ.get(cfg.act, 0)
    res["out"] = o.moe_tokens(W1, W2, WS1, WS2, res["tokens"], x_rows, res["ids"], res["w"], cfg.swiglu_limit,
                              hq=hq)
    return res


# h quantisation of each activation format: NVFP4 rows (1), MXFP8 (2), per-row FP8 (3)
HQ = {"nvfp4_all": 1, "mxfp8": 2, "fp8": 3}


def _swiglu(g: np.ndarray, u: np.ndarray, limit: Optional[float]) -> np.ndarray:
    """silu(g) u, or with a limit L the clamped silu(min(g, L)) min(max(u, -L), L), FP64,
    as the oracle's per-token MLP evaluates it (g / (1 + exp(-g)) u)."""
    if limit is not None:
        g = np.minimum(g, limit)
        u = np.minimum(np.maximum(u, -limit), limit)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def _quantize_h(h: np.ndarray, hq: int, o: Oracle) -> np.ndarray:
    """h rows rounded to binary32 and quantised as forward()'s MLP does: NVFP4 with one
    global scale per row (hq 1), MXFP8 (hq 2) or FP8 with one scale per row (hq 3),
    returned as their exact FP64 decode."""
    h32 = h.astype(np.float32)
    if hq == 3:
        return o.fp8_rows(*o.fp8_rows_quantize(h32))
    if hq == 2:
        return o.mxfp8_rows(*o.mxfp8_quantize(h32))
    return o.dequant_rows(*o.quantize(h32, rows_per_gs=1))


def forward_by_expert(cfg: synth.MoeConfig, x_bf16: np.ndarray, logits: np.ndarray, W1, W2, WS1=None,
                      WS2=None, tokens: Optional[np.ndarray] = None, o: Optional[Oracle] = None,
                      progress=None) -> Dict:
    """forward()'s result evaluated one expert at a time (for full-size checks).

    The layer output out_t = sum_j w_tj FFN_{ids_tj}(x_t) (+ FFN_shared(x_t)) is a sum of
    one term per (token, pick). Here each expert's two projections are decoded once to FP64
    by the oracle's element decode (``decode_projection``) and its FFN is applied to every
    row routed to it with FP64 matrix products as the library step: g = X Wg^T, u = X Wu^T,
    h = SwiGLU(g, u) (quantised first for the h-quantised variants), y = h W2^T. The terms
    of a token are then summed in pick order, the shared expert last, as forward() sums
    them. Routing, the activation rows and every formula are forward()'s; only the order of
    the FP64 roundings inside each dot product differs (relative differences near 1e-16)."""
    o = o or default()
    res = _prepare(cfg, x_bf16, logits, tokens, o)
    tokens = res["tokens"]
    ids, w, counts, offsets, perm = res["ids"], res["w"], res["counts"], res["offsets"], res["perm"]
    T, k = ids.shape
    H, I = cfg.H, cfg.I
    x_rows = res.pop("x_rows")                            # decoded inputs of `tokens`, in that order
    pos = np.full(T, -1, np.int64)                        # token -> its row in x_rows / out
    pos[tokens] = np.arange(len(tokens))
    hq = HQ.get(cfg.act, 0)
    routed_limit = cfg.swiglu_limit

    def ffn(Wa, Wb, g, X, limit):
        A = o.decode_projection(Wa, g)                    # [2I][H]: gate rows, then up rows
        h = _swiglu(X @ A[:I].T, X @ A[I:].T, limit)
        del A
        if hq:
            h = _quantize_h(h, hq, o)
        return h @ o.decode_projection(Wb, g).T           # [rows][H]

    Y = np.zeros((len(tokens), k, H), np.float64)         # one term per (token, pick)
    for e in range(cfg.E):
        rows = perm[offsets[e]:offsets[e + 1]]
        t_of, j_of = rows // k, rows % k
        keep = pos[t_of] >= 0
        if not keep.any():
            continue
        t_of, j_of = pos[t_of[keep]], j_of[keep]
        Y[t_of, j_of] = ffn(W1, W2, e, x_rows[t_of], routed_limit)
        if progress and (e % 32 == 31 or e == cfg.E - 1):
            progress(f"oracle by expert: experts 0..{e} of {cfg.E} done")
    out = np.zeros((len(tokens), H), np.float64)
    wt = w[tokens]
    for j in range(k):                                    # picks in order
        out += wt[:, j:j + 1] * Y[:, j]
    del Y
    for s in range(cfg.shared):                           # shared expert(s) last, weight 1
        out += ffn(WS1, WS2, s, x_rows, None)
    res["out"] = out
    return res


# Variants that quantise h (NVFP4, MXFP8 or per-row FP8 h) decide each h code on an
# intermediate that the device computes in binary32 arithmetic and the oracle in FP64: an h
# value within FLIP_REL (relative) of a rounding boundary may take either neighbouring code,
# and both results are correct. A parity check may take such alternative roundings, each found
# here on the oracle side (its FP64 h, rounded to binary32 as its own quantiser does, and its
# quantiser), never from the device.
FLIP_REL = 2e-5


def h_flip_candidates(cfg: synth.MoeConfig, ref: Dict, W, tok: int, o: Optional[Oracle] = None):
    """Output changes of the alternative roundings of token tok's h elements that lie within
    FLIP_REL of a code boundary: for each such element of each of the token's experts (its
    routed picks, then the shared expert), w_j D2[:, i] sign (q' - q) step, with q, q' the
    element's code value and its neighbour across the boundary and step the element's scale.
    W = (W1, W2) or, with a shared expert, (W1, W2, WS1, WS2) as forward() takes them; ref is
    forward()'s result (its quantised activation rows cover every token)."""
    o = o or default()
    W1, W2 = W[0], W[1]
    WS1, WS2 = (W[2], W[3]) if cfg.shared else (None, None)
    if cfg.act == "mxfp8":
        x_t = o.mxfp8_rows(ref["xq"][tok:tok + 1], ref["xs"][tok:tok + 1])[0]
    elif cfg.act == "fp8":
        x_t = o.fp8_rows(ref["xq"][tok:tok + 1], ref["xg"][tok:tok + 1])[0]
    else:
        x_t = o.dequant_rows(ref["xq"][tok:tok + 1], ref["xs"][tok:tok + 1], ref["xg"][tok:tok + 1])[0]
    experts = [(W1, W2, int(e), float(wj), cfg.swiglu_limit) for e, wj in zip(ref["ids"][tok], ref["w"][tok])]
    if cfg.shared:
        experts.append((WS1, WS2, 0, 1.0, None))
    e4 = np.array([o.e4m3fn(c) for c in range(0x7F)])        # E4M3 magnitudes of codes 0x00..0x7E
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])                 # E2M1 magnitudes
    out = []
    for Wa, Wb, e, wj, lim in experts:
        h32 = o.expert_h(Wa, Wb, e, x_t, lim).astype(np.float32)
        D2 = o.decode_projection(Wb, e)                        # [H][I]
        if cfg.act in ("mxfp8", "fp8"):
            codes, sc = o.mxfp8_quantize(h32[None]) if cfg.act == "mxfp8" else o.fp8_rows_quantize(h32[None])
            for i in range(h32.size):
                c = int(codes[0, i]) & 0x7F
                step = np.ldexp(1.0, int(sc[0, i // 32]) - 127) if cfg.act == "mxfp8" else float(sc[0])
                v = abs(float(h32[i])) / step
                for c2 in (c - 1, c + 1):
                    if 0 <= c2 <= 0x7E and v > 0 and abs(v - (e4[c] + e4[c2]) / 2) <= FLIP_REL * v:
                        sgn = -1.0 if h32[i] < 0 else 1.0
                        out.append(wj * D2[:, i] * sgn * (e4[c2] - e4[c]) * step)
        else:
            packed, scales, gs = o.quantize(h32[None], rows_per_gs=1)
            for i in range(h32.size):
                c = (int(packed[0, i // 2]) >> (4 * (i & 1))) & 7
                d = float(np.float32(np.float32(o.e4m3fn(int(scales[0, i // 16]))) * gs[0]))
                if d == 0:
                    continue
                v = abs(float(h32[i])) / d
                for c2 in (c - 1, c + 1):
                    if 0 <= c2 <= 7 and v > 0 and abs(v - (e2[c] + e2[c2]) / 2) <= FLIP_REL * v:
                        sgn = -1.0 if h32[i] < 0 else 1.0
                        out.append(wj * D2[:, i] * sgn * (e2[c2] - e2[c]) * d)
    return out
