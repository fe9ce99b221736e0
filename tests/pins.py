"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees with an independent source:
hand tables from ``tests/golden/`` (constants the pages state), PyTorch's own
float8_e4m3fn / bfloat16 decoders, numpy/scipy library routines (stable
argsort, matmul, softmax, expit), brute force on tiny inputs, closed forms and
invariants. ``tests/test_oracle_mutation.py`` plants mistakes in copies of
``oracle.c`` and requires that some pin fails for each.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------ independent decoders

def e2m1_table() -> np.ndarray:
    """E2M1 code -> value from the hand-written golden table."""
    t = np.zeros(16)
    for code, val in _read_golden("e2m1_codes.txt"):
        t[int(code)] = float(val)
    return t


def e4m3_table_torch() -> np.ndarray:
    """E4M3fn byte -> value via PyTorch's float8_e4m3fn decoder (NaN for 0x7F/0xFF)."""
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return b.to(torch.float64).numpy()


def e4m3_encode_torch(v: np.ndarray) -> np.ndarray:
    """float32 -> E4M3fn byte by PyTorch's round-to-nearest-even conversion."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def decode_nvfp4(packed: np.ndarray, scales: np.ndarray, gs) -> np.ndarray:
    """[..., N, K/2] codes + [..., N, K/16] scales (+ scalar gs) -> FP64 [..., N, K]."""
    e2 = e2m1_table()
    e4 = e4m3_table_torch()
    lo = e2[packed & 15]
    hi = e2[packed >> 4]
    q = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    s = np.repeat(e4[scales], 16, axis=-1)
    return q * s * np.float64(gs)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def silu(z):
    return z / (1.0 + np.exp(-z))


# ------------------------------------------------------------------ codecs

def pin_e2m1_table(o):
    t = e2m1_table()
    for c in range(16):
        assert o.e2m1(c) == t[c] and math.copysign(1, o.e2m1(c)) == math.copysign(1, t[c]), c


def pin_e4m3_points(o):
    for b, v in _read_golden("e4m3fn_points.txt"):
        got = o.e4m3fn(int(b, 16))
        if v == "nan":
            assert math.isnan(got), b
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), (b, got, v)


def pin_e4m3_exhaustive(o):
    ref = e4m3_table_torch()
    for b in range(256):
        got = o.e4m3fn(b)
        if math.isnan(ref[b]):
            assert math.isnan(got), b
        else:
            assert got == ref[b], (b, got, ref[b])


def pin_bf16(o):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, 4000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite patterns
    ref = bf16_to_f64(bits)
    got = o.bf16_rows(bits)
    assert np.array_equal(got, ref)


def pin_weight_decode(o):
    # nibble order by hand: byte 0x21 holds k=0 -> code 1 (0.5), k=1 -> code 2 (1.0)
    packed = np.zeros((1, 8), np.uint8)
    packed[0, 0] = 0x21
    scales = np.full((1, 1), 0x38, np.uint8)      # E4M3 1.0
    assert o.weight(packed, scales, 1.0, 0, 0) == 0.5
    assert o.weight(packed, scales, 1.0, 0, 1) == 1.0
    # random tensor vs the independent decoder
    rng = np.random.default_rng(7)
    N, K = 6, 64
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)  # finite, non-negative
    gs = np.float32(0.0123)
    ref = decode_nvfp4(packed, scales, gs)
    for n in range(N):
        for k in range(K):
            assert o.weight(packed, scales, gs, n, k) == ref[n, k], (n, k)


def pin_layout_sizes(o):
    lim = {k: int(v) for k, v in _read_golden("nvfp4_limits.txt")}
    x = np.linspace(-1, 1, 512, dtype=np.float32).reshape(1, 512)
    p, s, g = o.quantize(x)
    assert p.shape == (1, 512 // lim["packed_cols_div"]) and s.shape == (1, 512 // lim["scale_cols_div"])
    assert p.nbytes + s.nbytes == lim["row512_bytes"]


# --------------------------------------------------------------- encoders

def pin_e4m3_encode(o):
    lim = {k: int(v) for k, v in _read_golden("nvfp4_limits.txt")}
    vals = e4m3_table_torch()[:0x7F]
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        mid = np.float32((a + b) / 2)
        pts += [np.float32(a), mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    rng = np.random.default_rng(11)
    pts += list((np.exp(rng.uniform(math.log(1e-5), math.log(447.9), 3000))).astype(np.float32))
    pts = np.array([p for p in pts if 0 < p < lim["e4m3_max"]], np.float32)
    ref = e4m3_encode_torch(pts)
    got = np.array([o.e4m3_encode(float(p)) for p in pts], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(ref[i])) for i in bad[:5]]
    assert o.e4m3_encode(0.0) == 0
    for v in (448.0, 460.0, 464.0, 1e30, float("inf")):
        assert o.e4m3_encode(v) == 0x7E, v                # saturates to the E4M3 max
    # survey example: 7.5 * 2^-9 is the midpoint of 0x07 and 0x08 -> even code 0x08
    assert o.e4m3_encode(7.5 * 2 ** -9) == 0x08


def pin_e2m1_encode(o):
    for r, code in _read_golden("e2m1_rounding.txt"):
        assert o.e2m1_encode(float(np.float32(float(r)))) == int(code), r


# -------------------------------------------------------------- quantizer

def quant_rows_fixture():
    rng = np.random.default_rng(13)
    rows = [rng.standard_normal(64).astype(np.float32) for _ in range(6)]
    rows.append(np.zeros(64, np.float32))                          # all zero
    r = np.zeros(64, np.float32); r[37] = -3.5; rows.append(r)      # one non-zero
    r = np.full(64, -0.0, np.float32); r[5] = 1e-3; rows.append(r)  # negative zeros
    rows.append((rng.standard_normal(64) * 1e4).astype(np.float32))  # large
    rows.append((rng.standard_normal(64) * 1e-6).astype(np.float32))  # small
    r = rng.standard_normal(64).astype(np.float32); r[:16] *= 1e-6; rows.append(r)  # underflowing block
    return np.stack(rows)


def pin_quantize(o):
    lim = {k: int(v) for k, v in _read_golden("nvfp4_limits.txt")}
    e2 = e2m1_table()
    e4 = e4m3_table_torch()
    x = quant_rows_fixture()
    p, s, g = o.quantize(x, rows_per_gs=1)
    for i, row in enumerate(x):
        A = np.float32(np.max(np.abs(row)))
        gs = A / np.float32(lim["gs_divisor"])                   # the page's formula, binary32
        assert g[i] == gs, (i, g[i], gs)
        codes = np.stack([p[i] & 15, p[i] >> 4], -1).reshape(-1)
        for b in range(row.size // 16):
            blk = row[16 * b:16 * b + 16]
            ab = np.float32(np.max(np.abs(blk)))
            if gs == 0:
                exp_s = 0
            else:
                ratio = ab / (np.float32(6.0) * gs)
                exp_s = 0x7E if ratio >= lim["e4m3_max"] else int(e4m3_encode_torch(np.array([ratio]))[0])
            assert s[i, b] == exp_s, (i, b, s[i, b], exp_s)
            d = np.float32(np.float32(e4[s[i, b]]) * gs)
            for j in range(16):
                v = blk[j]
                c = int(codes[16 * b + j])
                assert (c >> 3) == int(np.signbit(v)), (i, b, j)
                if d == 0:
                    assert (c & 7) == 0
                    continue
                r = np.float32(abs(v) / d)
                # brute-force optimality of the magnitude code on the binary32 ratio, ties to even
                dist = np.abs(e2[:8] - np.float64(r))
                best = np.flatnonzero(dist == dist.min())
                want = int(best[0]) if best.size == 1 else int([c_ for c_ in best if c_ % 2 == 0][0])
                assert (c & 7) == want, (i, b, j, float(r), c & 7, want)
    # the row maximum lands on the largest code with the largest scale
    i = 0
    k = int(np.argmax(np.abs(x[i])))
    code = (p[i, k // 2] >> (4 * (k & 1))) & 7
    assert s[i, k // 16] == 0x7E and code == 7


def pin_quantize_error_bound(o):
    """|x - x_hat| <= half the E2M1 spacing times d (no clipping inside the range)."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    p, s, g = o.quantize(x)
    xh = decode_nvfp4(p, s, 1.0) * g[:, None].astype(np.float64)
    e4 = e4m3_table_torch()
    d = np.repeat(e4[s] * g[:, None].astype(np.float64), 16, axis=1)
    r = np.abs(x) / d
    half = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0))
    assert np.all(np.abs(x - xh) <= half * d * (1 + 1e-6))


def pin_quantize_groups(o):
    """rows_per_gs = N: one global scale for the whole matrix (per expert weight tensor)."""
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((8, 32)) * 0.02).astype(np.float32)
    p, s, g = o.quantize(w, rows_per_gs=8)
    assert g.shape == (1,) and g[0] == np.float32(np.max(np.abs(w))) / np.float32(2688)
    p1, s1, g1 = o.quantize(w, rows_per_gs=1)
    assert np.all(g1 <= g[0]) and g1.max() == g[0]


# ----------------------------------------------------------------- routing

def route_fixture():
    rng = np.random.default_rng(23)
    l = rng.standard_normal((40, 16)).astype(np.float32)
    l[0] = 0.25                                    # all equal -> ids 0..k-1
    l[1] = np.round(l[1] * 4) / 4                  # many ties
    l[2, :] = -1.0; l[2, 9] = 0.0; l[2, 3] = -0.0  # -0 == +0 -> lower index first
    l[3] = np.round(l[3])
    return l


def pin_route_sort(o):
    l = route_fixture()
    for k in (1, 2, 5, 16):
        ids, w = o.route(l, k, "softmax")
        for t in range(l.shape[0]):
            order = sorted(range(l.shape[1]), key=lambda e: (-float(l[t, e]), e))
            assert list(ids[t]) == order[:k], (t, k, list(ids[t]), order[:k])
    ids, _ = o.route(l, 4, "softmax")
    assert list(ids[0]) == [0, 1, 2, 3]
    assert list(ids[2][:2]) == [3, 9]


def pin_route_softmax(o):
    l = route_fixture()
    ids, w = o.route(l, 16, "softmax")              # k = E: plain softmax over all experts
    ref = torch.softmax(torch.from_numpy(l.astype(np.float64)), dim=1).numpy()
    for t in range(l.shape[0]):
        assert np.allclose(w[t], ref[t, ids[t]], rtol=1e-13, atol=0)
    ids, w = o.route(l, 3, "softmax")
    for t in range(l.shape[0]):
        sel = l[t, ids[t]].astype(np.float64)
        ref = torch.softmax(torch.from_numpy(sel), 0).numpy()
        assert np.allclose(w[t], ref, rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1) < 1e-14 and np.all(np.diff(w[t]) <= 0)
    _, w1 = o.route(l, 1, "softmax")
    assert np.all(w1 == 1.0)


def pin_route_sigmoid(o):
    from scipy.special import expit
    l = route_fixture()
    ids, w = o.route(l, 4, "sigmoid")
    ids_s, _ = o.route(l, 4, "softmax")
    assert np.array_equal(ids, ids_s)               # selection does not depend on the score
    for t in range(l.shape[0]):
        sg = expit(l[t, ids[t]].astype(np.float64))
        assert np.allclose(w[t], sg / sg.sum(), rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1) < 1e-14


# ------------------------------------------------ generalised router (variants)

def _scores_library(l64: np.ndarray, score: str) -> np.ndarray:
    """FP64 router scores by library routines: torch softmax / sigmoid / softplus."""
    t = torch.from_numpy(l64)
    if score == "softmax":
        return torch.softmax(t, dim=-1).numpy()
    if score == "sigmoid":
        return torch.sigmoid(t).numpy()
    return torch.sqrt(torch.nn.functional.softplus(t)).numpy()


def _brute_topk(keys: np.ndarray, cand, k: int):
    """The k-subset of `cand` every member of which beats every non-member under the order
    (key desc, id asc), found by trying all subsets; returned in that order."""
    import itertools
    better = lambda a, b: (keys[a] > keys[b]) or (keys[a] == keys[b] and a < b)
    found = [S for S in itertools.combinations(cand, k)
             if all(better(a, b) for a in S for b in cand if b not in S)]
    assert len(found) == 1
    return sorted(found[0], key=lambda e: (-keys[e], e))


def _brute_route(l: np.ndarray, k: int, score: str, bias, n_group: int, topk_group: int,
                 renorm: bool, scaling: float):
    T, E = l.shape
    gsz = E // n_group
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        s = _scores_library(l[t].astype(np.float64), score)
        keys = s.astype(np.float32)
        if bias is not None:
            keys = (keys + bias.astype(np.float32)).astype(np.float32)
        gsc = np.zeros(n_group, np.float32)
        for q in range(n_group):
            top = sorted(keys[q * gsz:(q + 1) * gsz].tolist(), reverse=True)[:2]
            gsc[q] = np.float32(top[0]) if len(top) == 1 else np.float32(top[0]) + np.float32(top[1])
        groups = _brute_topk(gsc, list(range(n_group)), topk_group)
        cand = [e for e in range(E) if e // gsz in groups]
        ids[t] = _brute_topk(keys, cand, k)
        sel = s[ids[t]]
        w[t] = (sel / sel.sum() if renorm else sel) * scaling
    return ids, w


def route_general_fixture(T=24, E=16, seed=47):
    rng = np.random.default_rng(seed)
    l = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    return l, bias


def pin_route_general_bruteforce(o):
    """Every score function, with and without the selection bias and the group step, against
    library scores and an all-subsets search; weights from the unbiased scores."""
    l, bias = route_general_fixture()
    cases = [("sqrt_softplus", None, 1, 1, True, 1.0), ("sqrt_softplus", bias, 1, 1, True, 1.0),
             ("sigmoid", bias, 4, 2, True, 2.5), ("softmax", bias, 8, 3, True, 1.0),
             ("sigmoid", None, 4, 3, False, 1.5), ("softmax", None, 2, 1, False, 1.0),
             ("sqrt_softplus", bias, 16, 5, True, 1.0)]
    for score, b, ng, tg, rn, sc in cases:
        k = 3
        ids, w = o.route_general(l, k, score, b, ng, tg, rn, sc)
        rids, rw = _brute_route(l, k, score, b, ng, tg, rn, sc)
        assert np.array_equal(ids, rids), (score, ng, tg)
        assert np.allclose(w, rw, rtol=1e-12, atol=0), (score, ng, tg)


def pin_route_general_bias_selection_only(o):
    """The bias changes which experts are picked but never their weights: the weight of a
    pick is its unbiased score share, the same as without the bias when the picks agree."""
    l, bias = route_general_fixture(T=64, seed=53)
    big = bias * 4
    ids_b, w_b = o.route_general(l, 4, "sigmoid", big)
    ids_n, w_n = o.route_general(l, 4, "sigmoid")
    assert np.any(ids_b != ids_n)                      # the bias matters for selection
    for t in range(l.shape[0]):
        s = _scores_library(l[t].astype(np.float64), "sigmoid")[ids_b[t]]
        assert np.allclose(w_b[t], s / s.sum(), rtol=1e-13, atol=0)
        if np.array_equal(np.sort(ids_b[t]), np.sort(ids_n[t])):
            order = np.argsort(ids_n[t])
            assert np.allclose(np.sort(w_b[t]), np.sort(w_n[t]), rtol=1e-13, atol=0)
    zero = np.zeros(l.shape[1], np.float32)
    assert np.array_equal(o.route_general(l, 4, "sigmoid", zero)[0], ids_n)


def pin_route_general_special_cases(o):
    """Reductions to simpler routers: all groups kept = no group step; one expert per group
    with k groups kept = plain top-k on the keys; the plain router's picks and weights when
    no variant is on; weights summing to the routed scale; un-renormalised softmax weights
    = the full softmax; equal keys -> lower ids."""
    l, bias = route_general_fixture(T=40, seed=59)
    E, k = l.shape[1], 4
    for score in ("softmax", "sigmoid", "sqrt_softplus"):
        a = o.route_general(l, k, score, bias, 4, 4)
        b = o.route_general(l, k, score, bias, 1, 1)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        c = o.route_general(l, k, score, bias, E, k)
        assert np.array_equal(c[0], b[0])
    for score in ("softmax", "sigmoid"):
        ids_p, w_p = o.route(l, k, score)
        ids_g, w_g = o.route_general(l, k, score)
        assert np.array_equal(ids_p, ids_g)
        assert np.allclose(w_p, w_g, rtol=1e-13, atol=0)
    _, w = o.route_general(l, k, "sigmoid", bias, 2, 1, True, 2.5)
    assert np.allclose(w.sum(axis=1), 2.5, rtol=1e-14, atol=0)
    ids, w = o.route_general(l, k, "softmax", None, 1, 1, False, 1.0)
    full = _scores_library(l.astype(np.float64), "softmax")
    assert np.allclose(w, np.take_along_axis(full, ids, axis=1), rtol=1e-13, atol=0)
    eq = np.full((3, 8), 0.5, np.float32)
    ids, _ = o.route_general(eq, 3, "sqrt_softplus", np.zeros(8, np.float32), 4, 2)
    assert np.all(ids == np.array([0, 1, 2]))


def pin_plan(o):
    rng = np.random.default_rng(29)
    l = rng.standard_normal((37, 12)).astype(np.float32)
    ids, _ = o.route(l, 3, "softmax")
    counts, offsets, perm, inv = o.plan(ids, 12)
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=12))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(inv, np.argsort(perm, kind="stable"))
    assert counts.sum() == ids.size and all(len(set(r)) == 3 for r in ids)


# -------------------------------------------------------------------- MLP

def random_weights(rng, G, N, K, sigma=0.02):
    """A small random NVFP4 projection set [G][N][K] via the oracle-independent route:
    raw codes and scales drawn directly (finite, non-negative scales)."""
    packed = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x48, (G, N, K // 16), dtype=np.uint8)
    gs = (rng.uniform(0.5, 2.0, G) * sigma / 6).astype(np.float32)
    return packed, scales, gs


def pin_ffn_textbook(o):
    """E=1, k=1: the textbook SwiGLU MLP W2 (silu(Wg x) * (Wu x)) with numpy matmuls."""
    rng = np.random.default_rng(31)
    H, I = 64, 32
    W1 = random_weights(rng, 1, 2 * I, H)
    W2 = random_weights(rng, 1, H, I)
    x = rng.standard_normal(H)
    y = o.expert_ffn(W1, W2, 0, x)
    D1 = decode_nvfp4(W1[0][0], W1[1][0], W1[2][0])
    D2 = decode_nvfp4(W2[0][0], W2[1][0], W2[2][0])
    ref = D2 @ (silu(D1[:I] @ x) * (D1[I:] @ x))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())
    h = silu(D1[:I] @ x) * (D1[I:] @ x)                  # the first half alone (orc_expert_h)
    assert np.allclose(o.expert_h(W1, W2, 0, x), h, rtol=1e-12, atol=1e-15 * np.abs(h).max())


def pin_ffn_hand(o):
    g = {k: float(v) for k, v in _read_golden("hand_ffn.txt")}
    H, I = int(g["H"]), int(g["I"])
    W1 = (np.full((1, 2 * I, H // 2), 0x22, np.uint8), np.full((1, 2 * I, H // 16), 0x38, np.uint8),
          np.ones(1, np.float32))
    W2 = (np.full((1, H, I // 2), 0x22, np.uint8), np.full((1, H, I // 16), 0x38, np.uint8),
          np.ones(1, np.float32))
    y = o.expert_ffn(W1, W2, 0, np.ones(H))
    assert np.allclose(y, g["y"], rtol=1e-14, atol=0)


def _hand_weights(H, I):
    W1 = (np.full((1, 2 * I, H // 2), 0x22, np.uint8), np.full((1, 2 * I, H // 16), 0x38, np.uint8),
          np.ones(1, np.float32))
    W2 = (np.full((1, H, I // 2), 0x22, np.uint8), np.full((1, H, I // 16), 0x38, np.uint8),
          np.ones(1, np.float32))
    return W1, W2


def pin_ffn_clamped_hand(o):
    """The hand-worked clamped examples: both clamp sides, the unclamped side of the gate,
    and a zero limit zeroing the expert."""
    g = {k: float(v) for k, v in _read_golden("hand_ffn_clamped.txt")}
    H, I, L = int(g["H"]), int(g["I"]), g["L"]
    W1, W2 = _hand_weights(H, I)
    y = o.expert_ffn(W1, W2, 0, np.ones(H), swiglu_limit=L)
    assert np.allclose(y, g["y_pos"], rtol=1e-14, atol=0)
    y = o.expert_ffn(W1, W2, 0, -np.ones(H), swiglu_limit=L)
    assert np.allclose(y, g["y_neg"], rtol=1e-12, atol=0)
    for x in (np.ones(H), -np.ones(H), np.linspace(-3, 3, H)):
        assert np.all(o.expert_ffn(W1, W2, 0, x, swiglu_limit=0.0) == 0.0)


def pin_ffn_clamped_textbook(o):
    """Random weights: the clamped MLP equals W2 (silu(min(Wg x, L)) * clip(Wu x, -L, L)) with
    numpy matmuls and np.minimum / np.clip, and a limit above every |g|, |u| gives the plain MLP."""
    rng = np.random.default_rng(37)
    H, I = 64, 32
    W1 = random_weights(rng, 1, 2 * I, H, sigma=2.0)
    W2 = random_weights(rng, 1, H, I)
    D1 = decode_nvfp4(W1[0][0], W1[1][0], W1[2][0])
    D2 = decode_nvfp4(W2[0][0], W2[1][0], W2[2][0])
    for trial in range(4):
        x = rng.standard_normal(H) * 3
        gv, uv = D1[:I] @ x, D1[I:] @ x
        L = float(np.median(np.abs(np.concatenate([gv, uv]))))     # clamps about half of them
        ref = D2 @ (silu(np.minimum(gv, L)) * np.clip(uv, -L, L))
        y = o.expert_ffn(W1, W2, 0, x, swiglu_limit=L)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max())
        big = o.expert_ffn(W1, W2, 0, x, swiglu_limit=1e300)
        assert np.array_equal(big, o.expert_ffn(W1, W2, 0, x))


def pin_moe_clamp_routed_only(o):
    """The clamp reaches the routed experts and leaves the shared one plain: with a zero
    limit the layer output is the shared expert's output alone."""
    rng = np.random.default_rng(41)
    W1, W2, WS1, WS2, x, l = moe_small(rng, shared=1)
    ids, w = o.route(l, 2, "softmax")
    T = x.shape[0]
    toks = np.arange(T, dtype=np.int32)
    out = o.moe_tokens(W1, W2, WS1, WS2, toks, x, ids, w, swiglu_limit=0.0)
    ref = np.stack([o.expert_ffn(WS1, WS2, 0, x[t]) for t in range(T)])
    assert np.array_equal(out, ref)


def quantize_row_brute(row: np.ndarray) -> np.ndarray:
    """The NVFP4 row quantiser written from its definition, independently of the oracle:
    binary32 gs = A / 2688, each block's E4M3 scale by PyTorch's round-to-nearest-even
    float8 conversion (saturating at 448), each magnitude the nearest E2M1 value by a
    search over all 8 (ties to the even code); returns the exact FP64 decode."""
    lim = {k: int(v) for k, v in _read_golden("nvfp4_limits.txt")}
    e2 = e2m1_table()
    e4 = e4m3_table_torch()
    row = np.asarray(row, np.float32)
    gs = np.float32(np.max(np.abs(row))) / np.float32(lim["gs_divisor"])
    out = np.zeros(row.size, np.float64)
    for b in range(row.size // 16):
        blk = row[16 * b:16 * b + 16]
        if gs == 0:
            continue
        ratio = np.float32(np.max(np.abs(blk))) / (np.float32(6.0) * gs)
        s = 0x7E if ratio >= lim["e4m3_max"] else int(e4m3_encode_torch(np.array([ratio]))[0])
        d = np.float32(np.float32(e4[s]) * gs)
        if d == 0:
            continue
        for j in range(16):
            r = np.float64(np.float32(abs(blk[j]) / d))
            dist = np.abs(e2[:8] - r)
            best = np.flatnonzero(dist == dist.min())
            c = int(best[0]) if best.size == 1 else int([q for q in best if q % 2 == 0][0])
            out[16 * b + j] = np.copysign(e2[c] * float(e4[s]) * float(gs), blk[j])
    return out


def pin_ffn_hq_textbook(o):
    """W4A4 down: the MLP equals W2 . Q(fp32(h)) with h the textbook SwiGLU (numpy matmuls)
    and Q the row quantiser written from its definition above; every h row gets its own
    global scale, and h far from quantisation (hq off) is the plain MLP."""
    rng = np.random.default_rng(43)
    H, I = 64, 64
    W1 = random_weights(rng, 1, 2 * I, H, sigma=0.5)
    W2 = random_weights(rng, 1, H, I)
    D1 = decode_nvfp4(W1[0][0], W1[1][0], W1[2][0])
    D2 = decode_nvfp4(W2[0][0], W2[1][0], W2[2][0])
    for trial in range(3):
        x = rng.standard_normal(H) * (1.0 + trial)
        h = silu(D1[:I] @ x) * (D1[I:] @ x)
        hq = quantize_row_brute(h.astype(np.float32))
        assert np.max(np.abs(hq - h)) > 1e-3 * np.max(np.abs(h))     # the quantisation is visible
        ref = D2 @ hq
        y = o.expert_ffn(W1, W2, 0, x, hq=True)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max()), np.abs(y - ref).max()
        yc = o.expert_ffn(W1, W2, 0, x, swiglu_limit=0.5, hq=True)
        hc = silu(np.minimum(D1[:I] @ x, 0.5)) * np.clip(D1[I:] @ x, -0.5, 0.5)
        refc = D2 @ quantize_row_brute(hc.astype(np.float32))
        assert np.allclose(yc, refc, rtol=1e-12, atol=1e-14 * np.abs(refc).max())


def pin_moe_hq_every_expert(o):
    """h quantisation reaches the routed and the shared experts: the layer output equals
    sum_j w_j FFN_q(e_j) + FFN_q(shared), each FFN_q the textbook MLP on the quantised h."""
    rng = np.random.default_rng(47)
    W1, W2, WS1, WS2, x, l = moe_small(rng, T=6, shared=1)
    ids, w = o.route(l, 2, "softmax")
    T = x.shape[0]
    I = W2[0].shape[-1] * 2

    def ffn(Wa, Wb, e, xt):
        D1 = decode_nvfp4(Wa[0][e], Wa[1][e], Wa[2][e])
        D2 = decode_nvfp4(Wb[0][e], Wb[1][e], Wb[2][e])
        return D2 @ quantize_row_brute((silu(D1[:I] @ xt) * (D1[I:] @ xt)).astype(np.float32))

    out = o.moe_tokens(W1, W2, WS1, WS2, np.arange(T, dtype=np.int32), x, ids, w, hq=True)
    for t in range(T):
        ref = sum(w[t, j] * ffn(W1, W2, ids[t, j], x[t]) for j in range(2)) + ffn(WS1, WS2, 0, x[t])
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def quantize_mxfp8_brute(row: np.ndarray):
    """MXFP8 row quantiser written from its definition, independently of the oracle:
    per 32 consecutive k, X = floor(log2 amax) - 8 from numpy's frexp (clamped to
    [-127, 127], -127 for an all-zero block), elements by PyTorch's round-to-nearest-even
    float8_e4m3fn conversion of |x| 2^-X (saturating at 448), sign kept; returns
    (codes, scale bytes, exact FP64 decode)."""
    row = np.asarray(row, np.float32)
    K = row.size
    codes = np.zeros(K, np.uint8)
    sc = np.zeros(K // 32, np.uint8)
    e4 = e4m3_table_torch()
    for b in range(K // 32):
        blk = row[32 * b:32 * b + 32]
        A = float(np.max(np.abs(blk)))
        X = -127
        if A > 0:
            X = int(np.frexp(np.float32(A))[1]) - 1 - 8
            X = max(-127, min(127, X))
        sc[b] = X + 127
        r = np.ldexp(np.abs(blk).astype(np.float64), -X).astype(np.float32)   # exact power-of-two scaling
        enc = np.where(r >= 448, 0x7E, e4m3_encode_torch(np.minimum(r, np.float32(448))))
        codes[32 * b:32 * b + 32] = enc.astype(np.uint8) | np.where(np.signbit(blk), 0x80, 0).astype(np.uint8)
    dec = np.array([e4[c & 0x7F] * (-1.0 if c & 0x80 else 1.0) for c in codes]) * np.repeat(
        np.ldexp(1.0, sc.astype(np.int64) - 127), 32)
    return codes, sc, dec


def mxfp8_fixture():
    rng = np.random.default_rng(53)
    rows = [rng.standard_normal(64).astype(np.float32) for _ in range(4)]
    rows.append(np.zeros(64, np.float32))                                   # all zero: scale byte 0
    r = np.zeros(64, np.float32); r[40] = -3.5; r[3] = 1e-30; rows.append(r)  # one non-zero per block
    r = rng.standard_normal(64).astype(np.float32); r[0] = 500.0; r[1] = 448.0; rows.append(r)  # clipping
    r = np.full(64, -0.0, np.float32); r[33] = 2.0 ** -120; rows.append(r)  # negative zeros, tiny block
    rows.append((rng.standard_normal(64) * 1e30).astype(np.float32))       # large
    rows.append((rng.standard_normal(64) * 1e-20).astype(np.float32))      # small
    return np.stack(rows)


def pin_mxfp8_quantize(o):
    """Codes and scale bytes bit-exact against the definition written in the test; the row
    maximum of a block with max 2^e lands on E4M3 256 (0x78) at scale 2^(e-8)."""
    x = mxfp8_fixture()
    codes, sc = o.mxfp8_quantize(x)
    for i, row in enumerate(x):
        c, s, _ = quantize_mxfp8_brute(row)
        assert np.array_equal(sc[i], s), (i, sc[i], s)
        assert np.array_equal(codes[i], c), (i, np.flatnonzero(codes[i] != c))
    one = np.zeros((1, 32), np.float32)
    one[0, 5] = 4.0
    c, s = o.mxfp8_quantize(one)
    assert s[0, 0] == 127 + 2 - 8 and c[0, 5] == 0x78
    assert sc[4, 0] == 0 and not codes[4].any()                              # zero block
    assert codes[6, 0] == 0x7E and codes[6, 1] == 0x7E                       # 500 and 448 saturate / exact


def pin_mxfp8_decode(o):
    """Every E4M3 code times E8M0 scales against PyTorch's float8_e4m3fn decoder."""
    e4 = e4m3_table_torch()
    for s in (0, 1, 100, 120, 127, 130, 200, 254):
        for c in range(256):
            if (c & 0x7F) == 0x7F:
                continue
            want = e4[c] * 2.0 ** (s - 127)
            assert o.mxfp8(c, s) == want, (c, s)


def pin_ffn_mxfp8_textbook(o):
    """W4A8 MLP: MXFP4 weights, the input and h MXFP8: W2 . Q8(fp32(silu(Wg x) (Wu x)))
    with Q8 the quantiser written in the test, plain and clamped."""
    rng = np.random.default_rng(59)
    H, I = 64, 64
    W1 = random_mx_weights(rng, 1, 2 * I, H)
    W2 = random_mx_weights(rng, 1, H, I)
    D1 = decode_mxfp4(W1[0][0], W1[1][0])
    D2 = decode_mxfp4(W2[0][0], W2[1][0])
    for trial in range(3):
        x = (rng.standard_normal(H) * 4.0 ** trial).astype(np.float32)
        _, _, xh = quantize_mxfp8_brute(x)
        for lim in (None, 0.05):
            gv, uv = D1[:I] @ xh, D1[I:] @ xh
            if lim is not None:
                gv, uv = np.minimum(gv, lim), np.clip(uv, -lim, lim)
            h = silu(gv) * uv
            _, _, hh = quantize_mxfp8_brute(h.astype(np.float32))
            assert np.max(np.abs(hh - h)) > 1e-4 * np.max(np.abs(h))          # the quantisation is visible
            ref = D2 @ hh
            y = o.expert_ffn((W1[0], W1[1], None), (W2[0], W2[1], None), 0, xh, swiglu_limit=lim, hq=2)
            assert np.allclose(y, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max()), np.abs(y - ref).max()


# ------------------------------------------- FP8 rows with a per-row scale (W4A8 on NVFP4)

def quantize_fp8_row_brute(row: np.ndarray):
    """Per-row FP8 quantiser written from its definition, independently of the oracle:
    s = float32(max|x|) / 448 in float32, codes by PyTorch's round-to-nearest-even
    float8_e4m3fn conversion of float32(|x| / s) (ratios of 448 and above: 0x7E), sign kept,
    all codes 0 when s is 0; returns (codes, s, exact FP64 decode)."""
    row = np.asarray(row, np.float32)
    A = np.float32(np.max(np.abs(row))) if row.size else np.float32(0)
    s = np.float32(A / np.float32(448.0))
    if s == 0:
        codes = np.where(np.signbit(row), 0x80, 0).astype(np.uint8)
    else:
        r = (np.abs(row) / s).astype(np.float32)
        enc = np.where(r >= 448, 0x7E, e4m3_encode_torch(np.minimum(r, np.float32(448))))
        codes = enc.astype(np.uint8) | np.where(np.signbit(row), 0x80, 0).astype(np.uint8)
    e4 = e4m3_table_torch()
    return codes, s, e4[codes] * np.float64(s)


def fp8_rows_fixture():
    rng = np.random.default_rng(61)
    rows = [rng.standard_normal(96).astype(np.float32) for _ in range(4)]
    rows.append(np.zeros(96, np.float32))                                    # all zero: s = 0
    r = np.full(96, -0.0, np.float32); rows.append(r)                        # negative zeros
    r = np.zeros(96, np.float32); r[17] = -3.0; r[50] = 1e-6; rows.append(r)  # tiny next to the max
    rows.append((rng.standard_normal(96) * 1e30).astype(np.float32))         # large
    rows.append((rng.standard_normal(96) * 1e-30).astype(np.float32))        # small (s subnormal-free)
    r = rng.standard_normal(96).astype(np.float32); r[3] = 7.0; r[4] = -7.0; rows.append(r)  # tied maxima
    rows.append(np.ldexp(1.0, rng.integers(-12, 4, 96)).astype(np.float32) * rng.choice([-1, 1], 96))  # powers of 2
    r = rng.standard_normal(96).astype(np.float32); r[0] = 5.0; r[-1] = -9.0; rows.append(r)  # max at either end
    return np.stack(rows)


def pin_fp8_rows_quantize(o):
    """Codes and scales bit-exact against the definition written in the test; the row's
    largest magnitude always encodes as 448 (0x7E), and a zero row has scale 0."""
    x = fp8_rows_fixture()
    codes, s = o.fp8_rows_quantize(x)
    for i, row in enumerate(x):
        c, si, _ = quantize_fp8_row_brute(row)
        assert s[i] == si, (i, s[i], si)
        assert np.array_equal(codes[i], c), (i, np.flatnonzero(codes[i] != c))
        if si > 0:
            assert (codes[i][np.abs(row) == np.abs(row).max()] & 0x7F == 0x7E).all(), i
    assert s[4] == 0 and not codes[4].any()
    assert s[5] == 0 and (codes[5] == 0x80).all()


def pin_fp8_rows_decode_and_bound(o):
    """The decode is E4M3 (PyTorch's decoder) times the row scale, and it lies within E4M3's
    rounding bound of x: relative 2^-4 for |x| >= 2^-6 s, absolute 2^-10 s below that."""
    x = fp8_rows_fixture()
    codes, s = o.fp8_rows_quantize(x)
    dec = o.fp8_rows(codes, s)
    e4 = e4m3_table_torch()
    assert np.array_equal(dec, e4[codes] * s[:, None].astype(np.float64))
    for i in range(x.shape[0]):
        si = float(s[i])
        xi = x[i].astype(np.float64)
        big = np.abs(xi) >= si * 2.0 ** -6
        err = np.abs(dec[i] - xi)
        tol_rel = 2.0 ** -4 * np.abs(xi) * (1 + 1e-6)
        assert (err[big] <= tol_rel[big] + 1e-300).all(), i
        assert (err[~big] <= si * 2.0 ** -10 * (1 + 1e-6)).all(), i


def pin_ffn_fp8_textbook(o):
    """W4A8 on NVFP4 weights: the input and h quantised to FP8 per row,
    W2 . Q(fp32(silu(Wg x) (Wu x))) with Q the quantiser written in the test, plain and
    clamped, NVFP4 weights decoded by the test's own decoder."""
    rng = np.random.default_rng(67)
    H, I = 64, 96
    W1 = random_weights(rng, 1, 2 * I, H)
    W2 = random_weights(rng, 1, H, I)
    D1 = decode_nvfp4(W1[0][0], W1[1][0], W1[2][0])
    D2 = decode_nvfp4(W2[0][0], W2[1][0], W2[2][0])
    for trial in range(3):
        x = (rng.standard_normal(H) * 4.0 ** trial).astype(np.float32)
        _, _, xh = quantize_fp8_row_brute(x)
        for lim in (None, 0.05):
            gv, uv = D1[:I] @ xh, D1[I:] @ xh
            if lim is not None:
                gv, uv = np.minimum(gv, lim), np.clip(uv, -lim, lim)
            h = silu(gv) * uv
            _, _, hh = quantize_fp8_row_brute(h.astype(np.float32))
            assert np.max(np.abs(hh - h)) > 1e-4 * np.max(np.abs(h))          # the quantisation is visible
            ref = D2 @ hh
            y = o.expert_ffn(W1, W2, 0, xh, swiglu_limit=lim, hq=3)
            assert np.allclose(y, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max()), np.abs(y - ref).max()


def pin_moe_fp8_layer(o):
    """The layer with act "fp8" equals, per token, the textbook sum over its picks with x
    and h quantised by the test's FP8 quantiser (routing ids and weights from the result)."""
    import synth
    import oracle.moe as omoe
    cfg = synth.MoeConfig("pin-w4a8-nvfp4", T=10, H=64, I=64, E=6, k=2, shared=1, act="fp8", seed=209)
    x, lg = synth.activations(cfg), synth.logits(cfg)
    W1, W2, WS1, WS2 = _layer_weights(cfg, o)
    res = omoe.forward(cfg, x, lg, W1, W2, WS1, WS2, o=o)
    I = cfg.I

    def mlp(Wa, Wb, e, v):
        A = decode_nvfp4(Wa[0][e], Wa[1][e], Wa[2][e])
        B = decode_nvfp4(Wb[0][e], Wb[1][e], Wb[2][e])
        h = silu(A[:I] @ v) * (A[I:] @ v)
        return B @ quantize_fp8_row_brute(h.astype(np.float32))[2]
    X = bf16_to_f64(x).astype(np.float32)
    for t in range(cfg.T):
        xt = quantize_fp8_row_brute(X[t])[2]
        ref = sum(res["w"][t, j] * mlp(W1, W2, res["ids"][t, j], xt) for j in range(cfg.k)) + mlp(WS1, WS2, 0, xt)
        assert np.allclose(res["out"][t], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max()), t


# ------------------------------------------------------------ MXFP4 weights

def e8m0_table_torch() -> np.ndarray:
    """E8M0 byte -> value via PyTorch's float8_e8m0fnu decoder (NaN for 0xFF)."""
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu)
    return b.to(torch.float64).numpy()


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., N, K/2] codes + [..., N, K/32] E8M0 scales -> FP64 [..., N, K]."""
    e2 = e2m1_table()
    lo = e2[packed & 15]
    hi = e2[packed >> 4]
    q = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    return q * np.repeat(e8m0_table_torch()[scales], 32, axis=-1)


def random_mx_weights(rng, G, N, K):
    """Raw MXFP4 codes and E8M0 scales drawn directly (scales 2^-10 .. 2^-3)."""
    packed = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    scales = rng.integers(117, 125, (G, N, K // 32), dtype=np.uint8)
    return packed, scales, None


def pin_e8m0(o):
    ref = e8m0_table_torch()
    for b in range(256):
        v = o.e8m0(b)
        assert (math.isnan(v) and math.isnan(ref[b])) or v == ref[b], (b, v, ref[b])


def pin_mx_weight_decode(o):
    rng = np.random.default_rng(61)
    packed, scales, _ = random_mx_weights(rng, 1, 8, 96)
    ref = decode_mxfp4(packed[0], scales[0])
    for n in range(8):
        for k in range(96):
            assert o.weight_mx(packed[0], scales[0], n, k) == ref[n, k], (n, k)


def pin_mx_ffn_textbook(o):
    """MXFP4 expert MLP = the textbook SwiGLU MLP on the library-decoded weights."""
    rng = np.random.default_rng(67)
    H, I = 64, 64
    W1 = random_mx_weights(rng, 2, 2 * I, H)
    W2 = random_mx_weights(rng, 2, H, I)
    x = rng.standard_normal(H)
    for g in range(2):
        y = o.expert_ffn(W1, W2, g, x)
        D1 = decode_mxfp4(W1[0][g], W1[1][g])
        D2 = decode_mxfp4(W2[0][g], W2[1][g])
        ref = D2 @ (silu(D1[:I] @ x) * (D1[I:] @ x))
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


def pin_mx_unit_scales_equal_nvfp4(o):
    """MXFP4 with every scale 2^0 is the NVFP4 tensor with every block scale 1.0 and
    global scale 1.0: identical expert outputs."""
    rng = np.random.default_rng(71)
    H, I = 64, 32
    p1 = rng.integers(0, 256, (1, 2 * I, H // 2), dtype=np.uint8)
    p2 = rng.integers(0, 256, (1, H, I // 2), dtype=np.uint8)
    mx1 = (p1, np.full((1, 2 * I, H // 32), 127, np.uint8), None)
    mx2 = (p2, np.full((1, H, I // 32), 127, np.uint8), None)
    nv1 = (p1, np.full((1, 2 * I, H // 16), 0x38, np.uint8), np.ones(1, np.float32))
    nv2 = (p2, np.full((1, H, I // 16), 0x38, np.uint8), np.ones(1, np.float32))
    x = rng.standard_normal(H)
    assert np.array_equal(o.expert_ffn(mx1, mx2, 0, x), o.expert_ffn(nv1, nv2, 0, x))


def moe_small(rng, T=12, H=32, I=16, E=6, k=2, shared=0):
    W1 = random_weights(rng, E, 2 * I, H)
    W2 = random_weights(rng, E, H, I)
    WS1 = random_weights(rng, shared, 2 * I, H) if shared else None
    WS2 = random_weights(rng, shared, H, I) if shared else None
    x = rng.standard_normal((T, H))
    l = rng.standard_normal((T, E)).astype(np.float32)
    return W1, W2, WS1, WS2, x, l


def pin_moe_dense(o):
    """All experts on every token with a dense gate matrix (zeros off-route):
    out = sum_e G[t, e] * MLP_e(x_t) (+ shared), by numpy matmuls."""
    rng = np.random.default_rng(37)
    for score, shared in (("softmax", 0), ("sigmoid", 1)):
        T, H, I, E, k = 12, 32, 16, 6, 2
        W1, W2, WS1, WS2, x, l = moe_small(rng, T, H, I, E, k, shared)
        ids, w = o.route(l, k, score)
        out = o.moe_tokens(W1, W2, WS1, WS2, np.arange(T), x, ids, w)
        G = np.zeros((T, E))
        for t in range(T):
            G[t, ids[t]] = w[t]
        ref = np.zeros((T, H))
        for e in range(E):
            D1 = decode_nvfp4(W1[0][e], W1[1][e], W1[2][e])
            D2 = decode_nvfp4(W2[0][e], W2[1][e], W2[2][e])
            Y = (silu(x @ D1[:I].T) * (x @ D1[I:].T)) @ D2.T
            ref += G[:, e:e + 1] * Y
        for s in range(shared):
            D1 = decode_nvfp4(WS1[0][s], WS1[1][s], WS1[2][s])
            D2 = decode_nvfp4(WS2[0][s], WS2[1][s], WS2[2][s])
            ref += (silu(x @ D1[:I].T) * (x @ D1[I:].T)) @ D2.T
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def pin_moe_invariance(o):
    """Expert relabelling and token subsets do not change a token's output."""
    rng = np.random.default_rng(41)
    T, H, I, E, k = 10, 32, 16, 6, 3
    W1, W2, _, _, x, l = moe_small(rng, T, H, I, E, k)
    ids, w = o.route(l, k, "softmax")
    out = o.moe_tokens(W1, W2, None, None, np.arange(T), x, ids, w)
    P = rng.permutation(E)                       # new label P[e] for old expert e
    W1p = tuple(a[np.argsort(P)] for a in W1)
    W2p = tuple(a[np.argsort(P)] for a in W2)
    lp = np.empty_like(l)
    lp[:, P] = l
    ids_p, w_p = o.route(lp, k, "softmax")
    out_p = o.moe_tokens(W1p, W2p, None, None, np.arange(T), x, ids_p, w_p)
    assert np.allclose(out, out_p, rtol=1e-13, atol=1e-15)
    sub = np.array([7, 2])
    out_s = o.moe_tokens(W1, W2, None, None, sub, x[sub], ids, w)
    assert np.array_equal(out_s, out[sub])


def pin_dequant_rows(o):
    rng = np.random.default_rng(43)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    p, s, g = o.quantize(x)
    got = o.dequant_rows(p, s, g)
    ref = decode_nvfp4(p, s, 1.0) * g[:, None].astype(np.float64)
    assert np.array_equal(got, ref)


# ---------------------------------------------- per-expert evaluation of the layer

def _by_expert_configs():
    import synth
    return [
        synth.MoeConfig("bx-plain", T=24, H=128, I=128, E=8, k=2, seed=201),
        synth.MoeConfig("bx-shared-sigmoid", T=20, H=256, I=128, E=16, k=4, score="sigmoid", shared=1, seed=202),
        synth.MoeConfig("bx-w4a4-clamp", T=16, H=128, I=128, E=8, k=2, act="nvfp4", swiglu_limit=0.05, shared=1,
                        seed=203),
        synth.MoeConfig("bx-h-nvfp4", T=16, H=128, I=128, E=8, k=2, act="nvfp4_all", shared=1, seed=204),
        synth.MoeConfig("bx-w4a8", T=16, H=128, I=128, E=8, k=2, act="mxfp8", wfmt="mxfp4", seed=205),
        synth.MoeConfig("bx-w4a8-nvfp4", T=16, H=128, I=128, E=8, k=2, act="fp8", shared=1, swiglu_limit=0.05,
                        seed=207),
        synth.MoeConfig("bx-mx-general", T=16, H=128, I=128, E=16, k=4, wfmt="mxfp4", score="sqrt_softplus",
                        bias_sigma=0.3, seed=206),
    ]


def _layer_weights(cfg, o):
    import oracle.moe as omoe
    W = [omoe.projection_weights(cfg, w, o=o) for w in ("w1", "w2")]
    S = [omoe.projection_weights(cfg, w, o=o) for w in ("ws1", "ws2")] if cfg.shared else [None, None]
    return W + S


def pin_moe_by_expert_equals_per_token(o):
    """forward_by_expert (each expert decoded once, FP64 matrix products, terms summed per
    token in pick order) against forward (per token, per element, the C loops) on small
    layers of every variant: plain, shared + sigmoid, NVFP4 x + clamp, NVFP4 h, MXFP8 x and h
    on MXFP4 weights, the generalised router; and on a token subset given out of order."""
    import synth
    import oracle.moe as omoe
    for cfg in _by_expert_configs():
        x, lg = synth.activations(cfg), synth.logits(cfg)
        W1, W2, WS1, WS2 = _layer_weights(cfg, o)
        a = omoe.forward(cfg, x, lg, W1, W2, WS1, WS2, o=o)["out"]
        b = omoe.forward_by_expert(cfg, x, lg, W1, W2, WS1, WS2, o=o)["out"]
        rms = np.sqrt(np.mean(a * a))
        assert rms > 0 and np.abs(a - b).max() <= 1e-12 * rms, (cfg.name, np.abs(a - b).max() / rms)
        sub = np.array([5, 0, cfg.T - 1, 3], np.int32)
        c = omoe.forward_by_expert(cfg, x, lg, W1, W2, WS1, WS2, tokens=sub, o=o)["out"]
        assert np.abs(c - a[sub]).max() <= 1e-12 * rms, cfg.name


def pin_moe_by_expert_dense_numpy(o):
    """forward_by_expert against a dense numpy layer built from the library decoders (torch's
    float8 decoders for the weights and bf16 inputs): per token, the sum over its picks of
    w_j W2_e (silu(Wg_e x) * (Wu_e x)), plus the shared expert. Routing ids and weights are
    taken from the result (they are pinned on their own)."""
    import synth
    import oracle.moe as omoe
    for cfg in _by_expert_configs():
        if cfg.act not in ("bf16",):
            continue
        x, lg = synth.activations(cfg), synth.logits(cfg)
        W1, W2, WS1, WS2 = _layer_weights(cfg, o)
        res = omoe.forward_by_expert(cfg, x, lg, W1, W2, WS1, WS2, o=o)
        dec = (lambda W, e: decode_mxfp4(W[0][e], W[1][e])) if cfg.wfmt == "mxfp4" else \
            (lambda W, e: decode_nvfp4(W[0][e], W[1][e], W[2][e]))
        X = bf16_to_f64(x)
        I = cfg.I

        def mlp(Wa, Wb, e, v):
            A, B = dec(Wa, e), dec(Wb, e)
            return B @ (silu(A[:I] @ v) * (A[I:] @ v))
        ref = np.zeros((cfg.T, cfg.H))
        for t in range(cfg.T):
            for j in range(cfg.k):
                ref[t] += res["w"][t, j] * mlp(W1, W2, res["ids"][t, j], X[t])
            for s in range(cfg.shared):
                ref[t] += mlp(WS1, WS2, s, X[t])
        rms = np.sqrt(np.mean(ref * ref))
        assert np.abs(ref - res["out"]).max() <= 1e-12 * rms, cfg.name


ALL_PINS = [v for k, v in dict(globals()).items() if k.startswith("pin_")]
