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
