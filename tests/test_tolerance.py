"""The output check's allowance for the bf16 output format: half a bf16 ulp at the exact
value bounds the error of rounding it to bf16 (round to nearest even), and is reached."""
import numpy as np
import torch

from gpu_util import bf16_half_ulp


def test_half_ulp_bounds_bf16_rounding():
    rng = np.random.default_rng(7)
    # float32 values, so torch's conversion rounds once (a double goes through float32)
    r = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    r = r.astype(np.float64)
    err = np.abs(torch.from_numpy(r).to(torch.bfloat16).double().numpy() - r)
    a = bf16_half_ulp(r)
    assert np.all(err <= a)
    assert np.max(err / a) > 0.999          # the bound is tight


def test_half_ulp_values():
    # 1.0 has ulp 2^-7 in bf16; 1.5 the same; 2.0 has 2^-6; 0 gets no allowance
    r = np.array([1.0, 1.5, 1.999, 2.0, -3.0, 0.0, 2.0 ** -10])
    np.testing.assert_array_equal(bf16_half_ulp(r),
                                  [2.0 ** -8, 2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 0.0, 2.0 ** -18])
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: RNE gives 1, an error of exactly the allowance
    x = np.array([1.0 + 2.0 ** -8])
    assert torch.from_numpy(x).to(torch.bfloat16).double().item() == 1.0


def _w4a8_case():
    """The oracle side of a W4A8 case (no device): T=300 with a shared expert."""
    import synth
    from gpu_util import Case
    cfg = synth.MoeConfig("w4a8-capacity", T=300, H=256, I=256, E=8, k=2, shared=1, act="mxfp8", wfmt="mxfp4",
                          seed=77)
    case = Case.__new__(Case)
    case.cfg, case.x, case.logits = cfg, synth.activations(cfg), synth.logits(cfg)
    case.by_expert = False
    case.tokens = np.arange(cfg.T, dtype=np.int32)
    case.W = [tuple(synth.mxfp4_weights(cfg, w, 0, cfg.shared if w.startswith("ws") else cfg.E)) + (None,)
              for w in ("w1", "w2", "ws1", "ws2")]
    return case, case.reference()


def test_requant_flip_allowance():
    """The max check of quantised-h variants accepts an output that differs from the oracle by
    the other rounding of an h element within FLIP_REL of a code boundary (token 129's shared
    expert holds one: h = -9.5000483 at scale 2^-5, next to the -9 / -10 midpoint), rejects the
    same output without the allowance, and rejects a planted error."""
    import pytest
    from gpu_util import check_out, h_flip_candidates
    case, full = _w4a8_case()
    ref = full["out"]
    cand = h_flip_candidates(case, full, 129)
    assert len(cand) >= 1
    flips = lambda t: h_flip_candidates(case, full, t)   # noqa: E731
    rms = np.sqrt(np.mean(ref * ref))
    big = [c for c in cand if np.abs(c).max() > 0.05 * rms]   # the shared expert's element
    assert len(big) == 1
    for c in cand:                                       # every boundary element may round either way
        flipped = ref.copy()
        flipped[129] += c
        out = torch.from_numpy(flipped.astype(np.float32)).to(torch.bfloat16)
        check_out(out, ref, "one boundary flip", flips=flips)
    flipped = ref.copy()
    flipped[129] += big[0]
    with pytest.raises(AssertionError):                 # the same output without the allowance
        check_out(torch.from_numpy(flipped.astype(np.float32)).to(torch.bfloat16), ref, "without the allowance")
    bad = ref.copy()
    bad[5, 17] += 0.05 * rms
    with pytest.raises(AssertionError):
        check_out(torch.from_numpy(bad.astype(np.float32)).to(torch.bfloat16), ref, "planted error", flips=flips)


def test_flip_candidates_without_shared_expert():
    """A quantised-h layer without a shared expert holds two projection sets only; the
    candidate search takes them and finds boundary elements (oracle side, no device)."""
    import synth
    import oracle.moe as omoe
    from gpu_util import Case
    cfg = synth.MoeConfig("w4a8-noshared", T=40, H=256, I=256, E=8, k=2, shared=0, act="mxfp8", wfmt="mxfp4",
                          seed=78)
    case = Case.__new__(Case)
    case.cfg, case.x, case.logits = cfg, synth.activations(cfg), synth.logits(cfg)
    case.by_expert = False
    case.tokens = np.arange(cfg.T, dtype=np.int32)
    case.W = [tuple(synth.mxfp4_weights(cfg, w, 0, cfg.E)) + (None,) for w in ("w1", "w2")]
    full = case.reference()
    assert sum(len(omoe.h_flip_candidates(cfg, full, case.W, t)) for t in range(cfg.T)) > 0
