"""GPU NVFP4 quantisers against the oracle's binary32 quantiser: bit-exact bytes."""
import numpy as np
import pytest
import torch

import synth
import oracle
import pins
import nvfp4_block_scaled_router_amd as m
from gpu_util import DEV, bf16, log, up

pytestmark = pytest.mark.gpu


def _gpu_rows(x_u16):
    rows, K = x_u16.shape
    p = torch.empty((rows, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, K // 16), dtype=torch.uint8, device=DEV)
    g = torch.empty(rows, dtype=torch.float32, device=DEV)
    m.moe_quantize_nvfp4_rows(bf16(x_u16), rows, K, p, s, g)
    torch.cuda.synchronize()
    return p.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy()


def _bf16_bits(xf: np.ndarray) -> np.ndarray:
    return torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _check(x_u16, what):
    o = oracle.default()
    xf = o.bf16_rows(x_u16).astype(np.float32)
    rp, rs, rg = o.quantize(xf, rows_per_gs=1)
    gp, gsc, gg = _gpu_rows(x_u16)
    log(f"  {what}: rows {x_u16.shape[0]} K {x_u16.shape[1]}")
    assert np.array_equal(gg.view(np.uint32), rg.view(np.uint32)), "row global scales"
    assert np.array_equal(gsc, rs), "block scales"
    assert np.array_equal(gp, rp), "codes"


def test_rows_skewed_workload_activations():
    cfg = synth.skewed_w4a4()
    _check(synth.activations(cfg), "skewed-w4a4 x [512][4096]")


def test_rows_edge_cases():
    x = pins.quant_rows_fixture()                      # zeros, single value, -0, large, small, underflow
    _check(_bf16_bits(x), "edge rows")


def test_rows_ties_and_saturation():
    rng = np.random.default_rng(3)
    # values on E2M1 decision boundaries relative to the block scale, and blocks whose
    # ratio a_b/(6 gs) sits on E4M3 midpoints
    base = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0], size=(64, 128))
    sign = rng.choice([-1.0, 1.0], size=base.shape)
    scale = 2.0 ** rng.integers(-8, 8, size=(64, 1))
    _check(_bf16_bits(base * sign * scale), "boundary values")


def test_rows_tiny_magnitudes():
    """Rows whose global scale is a binary32 subnormal."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((8, 64)) * 1e-36).astype(np.float32)
    _check(_bf16_bits(x), "subnormal global scale")


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_weight_quantiser(which):
    cfg = synth.qwen3_decode(8)
    import oracle.moe as omoe
    from gpu_util import gpu_weights
    ref = omoe.quantized_weights(cfg, which, experts=range(8))
    G = cfg.E
    N, K = (2 * cfg.I, cfg.H) if which == "w1" else (cfg.H, cfg.I)
    from nvfp4_block_scaled_router_amd.weights import quantize_projection
    dev = quantize_projection(8, N, K, lambda e0, c: synth.expert_weights_f32(cfg, which, e0, c), DEV)
    for a, d in zip(ref, dev):
        assert np.array_equal(a[:8], d.cpu().numpy()), which


# ---------------------------------------------- FP8 rows with a per-row scale (W4A8 on NVFP4)

def _check_fp8(x_u16, what):
    o = oracle.default()
    rows, K = x_u16.shape
    rc, rs = o.fp8_rows_quantize(o.bf16_rows(x_u16).astype(np.float32))
    c = torch.empty((rows, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, dtype=torch.float32, device=DEV)
    m.moe_quantize_fp8_rows(bf16(x_u16), rows, K, c, s)
    torch.cuda.synchronize()
    log(f"  {what}: rows {rows} K {K}")
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "row scales"
    assert np.array_equal(c.cpu().numpy(), rc), "codes"


def test_fp8_rows_workload_activations():
    _check_fp8(synth.activations(synth.qwen3_w4a8(4096)), "qwen3 w4a8 x [4096][2048]")


def test_fp8_rows_edge_cases():
    _check_fp8(_bf16_bits(pins.fp8_rows_fixture()), "edge rows")


def test_fp8_rows_ties_and_saturation():
    """Rows whose maximum is 448 2^j (scale exactly 2^j) and whose other values sit on E4M3
    rounding midpoints (ties to the even code), on codes, and between them."""
    rng = np.random.default_rng(5)
    e4 = pins.e4m3_table_torch()[:0x7F]
    mids = (e4[:-1] + e4[1:]) / 2
    vals = np.concatenate([mids, e4, mids * (1 + 2.0 ** -6)])
    base = rng.choice(vals, size=(64, 256))
    base[:, 0] = 448.0
    sign = rng.choice([-1.0, 1.0], size=base.shape)
    scale = 2.0 ** rng.integers(-10, 10, size=(64, 1))
    _check_fp8(_bf16_bits(base * sign * scale), "E4M3 midpoints")


def test_fp8_rows_tiny_magnitudes():
    """Rows whose scale max|x| / 448 is a binary32 subnormal."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((8, 64)) * 1e-37).astype(np.float32)
    _check_fp8(_bf16_bits(x), "subnormal row scale")
