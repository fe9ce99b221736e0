"""GPU parity of the whole layer against the CPU oracle (through the C ABI)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_util import Case, DEV, bf16, check_out, h_flip_candidates, log, up, W_ABS

pytestmark = pytest.mark.gpu


def _run_and_check(case: Case):
    cfg = case.cfg
    covered = len(set(case.ids_ref[case.tokens].reshape(-1).tolist()))
    touched = len(set(case.ids_ref.reshape(-1).tolist()))
    log(f"[{cfg.name}] T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} act={cfg.act} shared={cfg.shared} "
        f"checked tokens {len(case.tokens)} / {cfg.T}, covering {covered} of the {touched} routed experts used")
    ref = case.reference()
    L = case.layer()
    x = bf16(case.x)
    lg = up(case.logits)
    bufs, rout = L.routing_buffers(cfg.T)
    out = L(x, lg, routing=rout)
    torch.cuda.synchronize()
    assert np.array_equal(bufs["topk_ids"].cpu().numpy(), ref["ids"]), "topk ids"
    assert np.abs(bufs["topk_weights"].cpu().numpy() - ref["w"]).max() <= W_ABS, "topk weights"
    assert np.array_equal(bufs["expert_counts"].cpu().numpy(), ref["counts"]), "counts"
    assert np.array_equal(bufs["expert_offsets"].cpu().numpy(), ref["offsets"]), "offsets"
    assert np.array_equal(bufs["perm"].cpu().numpy(), ref["perm"]), "perm"
    if cfg.act == "mxfp8":
        assert np.array_equal(bufs["act_packed"].cpu().numpy(), ref["xq"]), "MXFP8 activation codes"
        assert np.array_equal(bufs["act_scales"].cpu().numpy(), ref["xs"]), "MXFP8 activation scales"
    if cfg.act == "fp8":
        assert np.array_equal(bufs["act_packed"].cpu().numpy(), ref["xq"]), "FP8 activation codes"
        assert np.array_equal(bufs["act_global"].cpu().numpy().view(np.uint32), ref["xg"].view(np.uint32)), \
            "FP8 activation row scales"
    if cfg.act in ("nvfp4", "nvfp4_all"):
        assert np.array_equal(bufs["act_packed"].cpu().numpy(), ref["xq"]), "quantised activation codes"
        assert np.array_equal(bufs["act_scales"].cpu().numpy(), ref["xs"]), "quantised activation scales"
        assert np.array_equal(bufs["act_global"].cpu().numpy().view(np.uint32), ref["xg"].view(np.uint32))
    flips = (lambda t: h_flip_candidates(case, ref, t)) if cfg.act in ("mxfp8", "nvfp4_all", "fp8") else None
    check_out(out[torch.from_numpy(case.tokens).long().to(DEV)], ref["out"], cfg.name, flips=flips)
    return L, x, lg, out


SMALL = [
    synth.tiny(),
    synth.with_tokens(synth.tiny(), 13, "tiny-t13"),
    synth.with_tokens(synth.tiny(), 200, "tiny-prefill-t200"),
    synth.with_tokens(synth.skewed_w4a4(), 48, "skewed-w4a4-t48"),
    synth.with_tokens(synth.qwen3_prefill(), 300, "qwen3-prefill-t300"),
    synth.MoeConfig("one-expert", T=5, H=128, I=128, E=1, k=1, seed=11),
    synth.MoeConfig("all-experts", T=40, H=256, I=128, E=8, k=8, score="sigmoid", seed=12),
    synth.MoeConfig("shared-small", T=70, H=256, I=256, E=16, k=4, score="sigmoid", shared=1, seed=13),
    synth.MoeConfig("shared-small-w4a4", T=150, H=512, I=128, E=8, k=2, shared=1, act="nvfp4", seed=14),
    # small bf16 decode batches: a shared expert, 256 experts (16 per lane of a routing
    # row), a single pick, one token
    synth.MoeConfig("decode-shared", T=7, H=256, I=128, E=16, k=4, shared=1, seed=17),
    synth.MoeConfig("decode-e256-k1", T=64, H=256, I=128, E=256, k=1, seed=18),
    synth.MoeConfig("decode-e200-t1", T=1, H=384, I=256, E=200, k=8, score="sigmoid", seed=19),
    # decode-regime batches over 64 tokens with at least 256 routed rows (fp16 or NVFP4 x): the
    # conversion runs as its own launch beside the per-token router, or in the general router's
    # launch
    synth.MoeConfig("decode-wide-f16", T=100, H=256, I=128, E=64, k=4, seed=20),
    synth.MoeConfig("decode-wide-w4a4", T=100, H=256, I=128, E=64, k=4, act="nvfp4", seed=30),
    synth.MoeConfig("decode-wide-general", T=90, H=256, I=128, E=64, k=4, score="sqrt_softplus", bias_sigma=0.5,
                    seed=29),
    # small decode grids load all K chunks of a wave at once: 2 chunks per wave (bf16 x),
    # 3 per wave with one wave's range across an 8-chunk scale group, fp16 x (256 rows)
    synth.MoeConfig("decode-pf-h1024", T=5, H=1024, I=256, E=16, k=4, seed=34),
    synth.MoeConfig("decode-pf-h1536", T=6, H=1536, I=256, E=16, k=4, score="sigmoid", seed=35),
    synth.MoeConfig("decode-pf-f16", T=64, H=1024, I=128, E=64, k=4, seed=36),
    # hidden 128 / 384: the prefill down launch cannot use its widest workgroup and narrows
    synth.MoeConfig("prefill-h128", T=260, H=128, I=256, E=4, k=2, seed=15),
    synth.MoeConfig("prefill-h384-w4a4", T=300, H=384, I=128, E=4, k=2, act="nvfp4", seed=16),
    # prefill down with at most 8 K chunks runs as resident workgroups over (tile, column
    # block) items: 2 and 8 chunks, one and two column blocks, tile counts that leave XCDs
    # without items, ragged last tiles, h16 rows (row exponent) and FP8 rows (row scale)
    synth.MoeConfig("prefill-persist-kc2", T=700, H=512, I=256, E=8, k=2, seed=31),
    synth.MoeConfig("prefill-persist-kc8", T=500, H=256, I=1024, E=4, k=2, shared=1, seed=32),
    synth.MoeConfig("prefill-persist-fp8", T=600, H=512, I=512, E=8, k=2, act="fp8", seed=33),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small(cfg):
    _run_and_check(Case(cfg))


def _random_configs(n, seed=20261203):
    """Seeded layer shapes across the regimes (decode / skewed / prefill tiles, persistent and
    one-item down, 1-2 column blocks), activation formats and routers; every token is checked.
    T is capped so that the FP64 oracle stays within about a second per case."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([128, 256, 384, 512, 768, 1024, 2048]))
        I = int(rng.choice([128, 256, 384, 512, 768, 1024]))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(8, E) + 1))
        act = str(rng.choice(["bf16", "bf16", "nvfp4", "nvfp4_all", "fp8", "mxfp8"]))
        wfmt = "mxfp4" if act == "mxfp8" else "nvfp4"
        T = int(rng.integers(1, 2001))
        T = max(1, min(T, int(3e8 // (k * H * I))))
        out.append(synth.MoeConfig(f"rand{i}-T{T}-H{H}-I{I}-E{E}-k{k}-{act}", T=T, H=H, I=I, E=E, k=k,
                                   score=str(rng.choice(["softmax", "sigmoid"])), shared=int(rng.integers(0, 2)),
                                   act=act, wfmt=wfmt, seed=700 + i))
    return out


@pytest.mark.parametrize("cfg", _random_configs(32), ids=lambda c: c.name)
def test_random_shapes(cfg):
    _run_and_check(Case(cfg))


def _random_variant_configs(n, seed=20261204):
    """Seeded layers with the router and activation variants drawn at random: sqrt-softplus
    scores, a selection-only bias, the group step, routed scaling, no renormalisation, a
    clamped SwiGLU, MXFP4 weights; every token is checked."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([128, 256, 512, 1024]))
        I = int(rng.choice([128, 256, 384, 512]))
        n_group = int(rng.choice([1, 1, 2, 4, 8]))
        E = n_group * int(rng.integers(max(1, 4 // n_group), 65 // n_group + 1))
        topk_group = int(rng.integers(1, n_group + 1))
        k = int(rng.integers(1, min(8, topk_group * (E // n_group)) + 1))
        act = str(rng.choice(["bf16", "nvfp4", "nvfp4_all", "fp8", "mxfp8"]))
        wfmt = "mxfp4" if act == "mxfp8" or rng.random() < 0.3 else "nvfp4"
        if act == "fp8":
            wfmt = "nvfp4"
        T = int(rng.integers(1, 1201))
        T = max(1, min(T, int(3e8 // (k * H * I))))
        out.append(synth.MoeConfig(
            f"rvar{i}-T{T}-H{H}-I{I}-E{E}-k{k}-{act}-{wfmt}", T=T, H=H, I=I, E=E, k=k,
            score=str(rng.choice(["softmax", "sigmoid", "sqrt_softplus"])), shared=int(rng.integers(0, 2)),
            act=act, wfmt=wfmt, seed=800 + i,
            bias_sigma=float(rng.choice([0.0, 0.0, 0.3])), n_group=n_group, topk_group=topk_group,
            renorm=bool(rng.random() < 0.8), routed_scaling=float(rng.choice([1.0, 1.0, 2.5])),
            swiglu_limit=(None if rng.random() < 0.6 else float(rng.choice([0.0, 0.05, 7.0])))))
    return out


@pytest.mark.parametrize("cfg", _random_variant_configs(16), ids=lambda c: c.name)
def test_random_variants(cfg):
    _run_and_check(Case(cfg))


# router and activation variants: sqrt-softplus scores, selection-only bias, the group step,
# routed scaling, un-renormalised weights, clamped SwiGLU (routed experts only)
VARIANTS = [
    synth.MoeConfig("v-sqrtsoftplus-bias-clamp", T=40, H=256, I=128, E=16, k=4, score="sqrt_softplus",
                    shared=1, seed=21, bias_sigma=0.3, swiglu_limit=0.05),
    synth.MoeConfig("v-groups-scaled", T=300, H=256, I=256, E=32, k=4, score="sigmoid", seed=22,
                    bias_sigma=0.05, n_group=8, topk_group=3, routed_scaling=2.5),
    synth.MoeConfig("v-softmax-norenorm", T=24, H=128, I=128, E=64, k=6, seed=23, renorm=False,
                    n_group=4, topk_group=2),
    synth.MoeConfig("v-clamp-zero", T=33, H=256, I=128, E=8, k=2, shared=1, seed=24, swiglu_limit=0.0),
    synth.MoeConfig("v-w4a4-wide-e", T=130, H=256, I=128, E=600, k=8, act="nvfp4", score="sqrt_softplus",
                    seed=25, bias_sigma=0.2, n_group=6, topk_group=4),
    synth.deepseek_v4_flash(8),
    # MXFP4 weights (E8M0 per 32, no global scale): decode, prefill with a shared expert, W4A4
    synth.MoeConfig("mx-decode", T=8, H=256, I=128, E=16, k=4, seed=41, wfmt="mxfp4"),
    synth.MoeConfig("mx-prefill-shared", T=300, H=512, I=256, E=8, k=2, shared=1, seed=42, wfmt="mxfp4"),
    # (uniform random E2M1 codes give heavy output tails: max|out| is 6-8 RMS here, where
    # the bf16 rounding of the exact output alone reaches 2e-2 RMS)
    synth.MoeConfig("mx-w4a4", T=100, H=512, I=256, E=8, k=2, act="nvfp4", seed=45, wfmt="mxfp4"),
    # sharing workloads (a fraction of the picks reused across the batch)
    synth.MoeConfig("share40-small", T=6, H=256, I=128, E=64, k=6, score="sqrt_softplus", seed=27,
                    bias_sigma=0.5, wfmt="mxfp4", sharing=0.4),
    synth.deepseek_v4_flash_sharing(6, 0.8),
]


@pytest.mark.parametrize("cfg", VARIANTS, ids=lambda c: c.name)
def test_router_activation_variants(cfg):
    _run_and_check(Case(cfg))


def test_deepseek_v4_flash_t64():
    cfg = synth.deepseek_v4_flash(64)
    _run_and_check(Case(cfg, by_expert=True))


def test_deepseek_v3_router_sampled():
    cfg = synth.deepseek_v3_router(1024)
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 3), weights="gpu"))


@pytest.mark.parametrize("T", synth.DECODE_TOKENS)
def test_qwen3_decode(T):
    _run_and_check(Case(synth.qwen3_decode(T)))


# The full-size workloads, every token against the oracle (evaluated one expert at a time),
# every expert with its real weights on both sides.
def test_qwen3_prefill_full():
    _run_and_check(Case(synth.qwen3_prefill(), by_expert=True))


def test_skewed_w4a4_full():
    _run_and_check(Case(synth.skewed_w4a4(), by_expert=True))


def test_deepseek_v3_full():
    """8192 tokens x 7168 outputs; the GPU side's weights come from the library's device
    quantiser, asserted byte-identical to the oracle's for every expert."""
    _run_and_check(Case(synth.deepseek_v3(), weights="gpu", by_expert=True))


def test_deterministic_and_graph_replay():
    """Byte-identical repeats, and HIP-graph replays equal to the eager result."""
    cfg = synth.with_tokens(synth.qwen3_prefill(), 300, "qwen3-prefill-t300")
    case = Case(cfg)
    L = case.layer()
    x, lg = bf16(case.x), up(case.logits)
    a = L(x, lg).clone()
    b = L(x, lg).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    out = torch.empty_like(a)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L(x, lg, out=out)                       # warm on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L(x, lg, out=out)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), a.view(torch.int16)), f"replay {i}"
        c = L(x, lg).clone()                    # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), a.view(torch.int16))


def test_token_counts_within_capacity():
    """One plan (T_max = 300) serves smaller live T (both kernel regimes); T = 0 enqueues nothing."""
    cfg = synth.with_tokens(synth.qwen3_prefill(), 300, "qwen3-prefill-t300")
    case = Case(cfg)
    ref = case.reference()["out"]
    L = case.layer()
    x, lg = bf16(case.x), up(case.logits)
    for T in (1, 17, 129, 300):
        part = L(x[:T], lg[:T])
        torch.cuda.synchronize()
        check_out(part, ref[:T], f"T={T} of capacity 300")   # a token's output depends on that token only
    sentinel = torch.full((1, cfg.H), 7.0, dtype=torch.bfloat16, device=DEV)
    import nvfp4_block_scaled_router_amd as m
    m.moe_run(L.plan, L.packed, 0, x, lg, sentinel, None, L.workspace, L.workspace_bytes)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_w4a8_token_counts_and_graph_replay():
    """W4A8: one plan (T_max = 300) at live T in both regimes (h quantised in the decode
    epilogue at small T, by the row kernel after the prefill GEMM at large T), and a HIP graph
    of the prefill-regime run replayed between eager runs."""
    cfg = synth.MoeConfig("w4a8-capacity", T=300, H=256, I=256, E=8, k=2, shared=1, act="mxfp8", wfmt="mxfp4",
                          seed=77)
    case = Case(cfg)
    full = case.reference()
    ref = full["out"]
    L = case.layer()
    x, lg = bf16(case.x), up(case.logits)
    for T in (1, 7, 64, 300):
        part = L(x[:T], lg[:T])
        torch.cuda.synchronize()
        check_out(part, ref[:T], f"W4A8 T={T} of capacity 300", flips=lambda t: h_flip_candidates(case, full, t))
    a = L(x, lg).clone()
    out = torch.empty_like(a)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L(x, lg, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L(x, lg, out=out)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), a.view(torch.int16)), f"replay {i}"
        c = L(x[:7], lg[:7]).clone()            # an eager decode-regime run between replays
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), L(x[:7], lg[:7]).view(torch.int16))


@pytest.mark.parametrize("T", [8, 300])
def test_run_timed_matches_run(T):
    """moe_run_timed gives moe_run's bytes and a positive time for every stage that runs
    kernels (decode regime at T = 8, prefill regime at T = 300)."""
    import nvfp4_block_scaled_router_amd as m
    cfg = synth.with_tokens(synth.qwen3_prefill(), T, f"qwen3-t{T}")
    case = Case(cfg)
    L = case.layer()
    x, lg = bf16(case.x), up(case.logits)
    a = L(x, lg).clone()
    out = torch.empty_like(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * m.MOE_NUM_STAGES)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    m.moe_run_timed(L.plan, L.packed, T, x, lg, out, None, L.workspace, L.workspace_bytes, None,
                    [e.cuda_event for e in ev])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), a.view(torch.int16))
    for s in (m.MOE_STAGE_ROUTE, m.MOE_STAGE_GATE_UP, m.MOE_STAGE_DOWN, m.MOE_STAGE_COMBINE):
        t = ev[2 * s].elapsed_time(ev[2 * s + 1])
        log(f"T={T} stage {m.STAGE_NAMES[s]}: {t * 1e3:.1f} us")
        assert 0.0 < t < 1000.0


# W4A4 down: h of every expert row quantised to NVFP4 before the down GEMM (decode and
# prefill regimes, a shared expert, skewed routing with the 16-row cold list, clamped SwiGLU,
# MXFP4 weights, the widest intermediate size)
W4A4_ALL = [
    synth.MoeConfig("all-decode", T=8, H=256, I=128, E=16, k=4, act="nvfp4_all", seed=61),
    synth.MoeConfig("all-prefill-shared", T=300, H=512, I=256, E=8, k=2, shared=1, act="nvfp4_all", seed=62),
    synth.MoeConfig("all-skewed-cold", T=200, H=256, I=256, E=32, k=4, act="nvfp4_all", zipf_s=1.2, seed=63),
    synth.MoeConfig("all-clamp-sigmoid", T=100, H=256, I=128, E=16, k=4, score="sigmoid", shared=1,
                    act="nvfp4_all", swiglu_limit=0.05, seed=64),
    synth.MoeConfig("all-mx", T=64, H=512, I=256, E=8, k=2, act="nvfp4_all", wfmt="mxfp4", seed=65),
    synth.MoeConfig("all-max-inter", T=40, H=128, I=16384, E=4, k=2, shared=1, act="nvfp4_all", seed=66),
]


@pytest.mark.parametrize("cfg", W4A4_ALL, ids=lambda c: c.name)
def test_w4a4_down(cfg):
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 24) if cfg.I > 4096 else None))


def test_skewed_w4a4_down_full():
    _run_and_check(Case(synth.skewed_w4a4_all(), by_expert=True))


# W4A8: MXFP4 weights with MXFP8 x and h through the block-scaled MFMA (decode-sized and
# larger batches, a shared expert, the V4-Flash router and clamp, the V4-Flash shape, the
# widest intermediate size). The x quantisation of decode-regime batches rides on the routing
# launch: the one-workgroup plan (w4a8-decode), the general router (w4a8-v4-router-clamp), or
# its own launch beside the per-token router for more than 64 tokens (w4a8-decode-wide).
W4A8 = [
    synth.MoeConfig("w4a8-decode", T=8, H=256, I=128, E=16, k=4, act="mxfp8", wfmt="mxfp4", seed=71),
    synth.MoeConfig("w4a8-decode-wide", T=120, H=256, I=128, E=64, k=2, act="mxfp8", wfmt="mxfp4", seed=77),
    synth.MoeConfig("w4a8-prefill-shared", T=300, H=512, I=256, E=8, k=2, shared=1, act="mxfp8", wfmt="mxfp4",
                    seed=72),
    synth.MoeConfig("w4a8-v4-router-clamp", T=64, H=512, I=256, E=32, k=6, shared=1, score="sqrt_softplus",
                    bias_sigma=0.5, swiglu_limit=10.0, act="mxfp8", wfmt="mxfp4", seed=73),
    dataclasses.replace(synth.deepseek_v4_flash(8), name="w4a8-deepseek-v4-flash-t8", act="mxfp8"),
    synth.MoeConfig("w4a8-max-inter", T=40, H=128, I=16384, E=4, k=2, shared=1, act="mxfp8", wfmt="mxfp4",
                    seed=74),
    synth.MoeConfig("w4a8-skewed-cold", T=256, H=256, I=256, E=32, k=4, zipf_s=1.2, act="mxfp8", wfmt="mxfp4",
                    seed=75),
    synth.MoeConfig("w4a8-prefill-ragged", T=777, H=384, I=384, E=8, k=2, score="sigmoid", act="mxfp8",
                    wfmt="mxfp4", seed=76),
]


@pytest.mark.parametrize("cfg", W4A8, ids=lambda c: c.name)
def test_w4a8_mx(cfg):
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 24) if cfg.I > 4096 else None))


# W4A8 on NVFP4 weights: x and h FP8 with one scale per row, through the fp16 GEMMs (decode
# and prefill regimes, the skewed split launch, a shared expert, clamped SwiGLU, MXFP4
# weights, the widest intermediate size, a ragged prefill batch)
W4A8_NVFP4 = [
    synth.MoeConfig("fp8-decode", T=8, H=256, I=128, E=16, k=4, act="fp8", seed=91),
    synth.MoeConfig("fp8-decode-t1", T=1, H=384, I=256, E=32, k=8, score="sigmoid", shared=1, act="fp8", seed=92),
    synth.MoeConfig("fp8-decode-wide", T=120, H=256, I=128, E=64, k=2, act="fp8", seed=93),
    synth.MoeConfig("fp8-prefill-shared", T=300, H=512, I=256, E=8, k=2, shared=1, act="fp8", seed=94),
    synth.MoeConfig("fp8-skewed-split", T=256, H=256, I=256, E=32, k=4, zipf_s=1.2, act="fp8", seed=95),
    synth.MoeConfig("fp8-clamp-general", T=64, H=512, I=256, E=32, k=6, shared=1, score="sqrt_softplus",
                    bias_sigma=0.5, swiglu_limit=0.05, act="fp8", seed=96),
    synth.MoeConfig("fp8-mx-weights", T=64, H=512, I=256, E=8, k=2, act="fp8", wfmt="mxfp4", seed=97),
    synth.MoeConfig("fp8-max-inter", T=40, H=128, I=16384, E=4, k=2, shared=1, act="fp8", seed=98),
    synth.MoeConfig("fp8-prefill-ragged", T=777, H=384, I=384, E=8, k=2, score="sigmoid", act="fp8", seed=99),
]


@pytest.mark.parametrize("cfg", W4A8_NVFP4, ids=lambda c: c.name)
def test_w4a8_nvfp4(cfg):
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 24) if cfg.I > 4096 else None))


@pytest.mark.parametrize("T", [64, 4096])
def test_w4a8_nvfp4_qwen3_full(T):
    """The Qwen3-30B-A3B layer on the NVFP4-weight W4A8 path, decode (64 tokens) and prefill
    (4096 tokens), every token against the oracle."""
    _run_and_check(Case(synth.qwen3_w4a8(T), by_expert=True))


# the descriptor's limits: hidden and intermediate 16384 (128 K chunks), 65536 tokens
MAX_SIZES = [
    synth.MoeConfig("max-hidden-decode", T=16, H=16384, I=128, E=4, k=2, seed=31),
    synth.MoeConfig("max-hidden-prefill-w4a4", T=200, H=16384, I=128, E=4, k=2, act="nvfp4", seed=32),
    synth.MoeConfig("max-inter-prefill", T=40, H=128, I=16384, E=4, k=2, shared=1, seed=33),
    synth.MoeConfig("max-inter-decode", T=3, H=256, I=16384, E=8, k=2, score="sigmoid", seed=35),
]


@pytest.mark.parametrize("cfg", MAX_SIZES, ids=lambda c: c.name)
def test_max_sizes(cfg):
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 16)))


def test_max_tokens_sampled():
    """T = 65536 = the token limit: the whole routing (ids, weights, counts, offsets,
    permutation of 524288 rows) bit-exact, sampled outputs."""
    cfg = synth.MoeConfig("max-tokens", T=65536, H=128, I=128, E=64, k=8, seed=34)
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 24)))


def test_h16_past_4gib_sampled():
    """h16 beyond 4 GiB: 20000 tokens x (8 of 8 experts + a shared one) x I = 16384 gives
    180000 h rows (5.9 GB of h16); every token has rows past byte 2^32 (the later experts' and
    the shared expert's), which the GEMMs, the rescale and the combine address from 64-bit row
    bases. Sampled tokens against the oracle."""
    cfg = synth.MoeConfig("h16-past-4gib", T=20000, H=128, I=16384, E=8, k=8, shared=1, seed=36)
    assert (cfg.T * cfg.k + cfg.T) * cfg.I * 2 > 2 ** 32
    _run_and_check(Case(cfg, tokens=synth.token_sample(cfg, 16)))


def test_mxfp4_span_too_wide_is_loud():
    """An MXFP4 expert whose E8M0 bytes span more than the NVFP4 form holds exactly (here one
    byte 20 binades under the expert's largest) is rejected by the host validation, and if
    packed anyway every output that reads it is NaN; the other tokens still match the oracle."""
    import nvfp4_block_scaled_router_amd as m
    cfg = synth.MoeConfig("mx-wide-span", T=40, H=256, I=128, E=4, k=1, seed=81, wfmt="mxfp4")
    case = Case(cfg)
    W1 = case.W[0]
    codes, scales = W1[0].copy(), W1[1].copy()
    scales[0, 3, 2] = int(scales[0].max()) - 20
    desc = m.make_desc(cfg.H, cfg.I, cfg.E, cfg.k, cfg.T, weights="mxfp4")
    t = m.nvfp4_tensor(codes.ctypes.data, scales.ctypes.data, None)
    assert m.moe_validate_weights_host(desc, t, 0) == m.MOE_ERR_WEIGHT
    case.dev_w[0] = [up(codes), up(scales), None]
    L = case.layer()
    out = L(bf16(case.x), up(case.logits))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    on0 = case.ids_ref[:, 0] == 0
    assert on0.any() and (~on0).any()
    assert np.isnan(o[on0]).all(), "outputs of the too-wide expert must be NaN"
    ref = case.reference()
    check_out(out[torch.from_numpy(np.where(~on0)[0]).long().to(DEV)], ref["out"][~on0], cfg.name + " other experts")
