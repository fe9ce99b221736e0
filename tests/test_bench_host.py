"""Host-side logic of bench.py: the stage a traced kernel is booked under, and the one-GPU guard.

No GPU is touched: the stage map reads kernel names only, and `--gpus N` with N > 1 exits
before any device call.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("name, stage", [
    # GEMM kernels: the first template argument is the GEMM mode
    ("void nvmoe::gemm_prefill_kernel<0, 2, 6, 3, 8, 4>(nvmoe::GemmArgs)", "gate_up"),
    ("void nvmoe::gemm_prefill_kernel<2, 2, 6, 3, 8, 4>(nvmoe::GemmArgs)", "down"),
    ("void nvmoe::gemm_decode_kernel<0, 2, 4>(nvmoe::GemmArgs)", "gate_up"),
    ("void nvmoe::gemm_decode_kernel<4, 2, 4>(nvmoe::GemmArgs)", "down"),
    ("void nvmoe::gemm_prefill_mx8_kernel<5, 2, 4, 2, 96>(nvmoe::GemmArgs)", "gate_up"),
    ("void nvmoe::gemm_split_kernel<2, 4, 4, 4>(nvmoe::GemmArgs, nvmoe::GemmArgs, int, int, int)", "down"),
    # the persistent down kernel's first argument is a tile count, not a mode
    ("void nvmoe::gemm_prefill_down_persist_kernel<2, 6, 3, 8, 4>(nvmoe::GemmArgs, int)", "down"),
    ("void nvmoe::gemm_prefill_down_persist_kernel<1, 6, 3, 8, 4>(nvmoe::GemmArgs, int)", "down"),
    # routing and plan, h preparation, combine, weight packing
    ("void nvmoe::route_row_kernel<8>(nvmoe::RouteArgs)", "route"),
    ("nvmoe::plan_count_kernel(nvmoe::PlanArgs, int*, int*)", "route"),
    ("nvmoe::h_rescale_kernel(unsigned short*, signed char const*, int const*)", "h_prep"),
    ("void nvmoe::quant_rows_kernel<float>(float const*)", "h_prep"),
    ("nvmoe::combine_kernel(nvmoe::CombineArgs)", "combine"),
    ("nvmoe::pack_fp4_kernel(unsigned char const*)", "pack"),
    ("__amd_rocclr_copyBuffer", "other"),
])
def test_kernel_stage(name, stage):
    assert bench.kernel_stage(name) == stage


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_parity_gate_h_boundary_allowance():
    """bench.py's parity gate on a quantised-h variant (oracle side only, no device): an output
    that takes the other rounding of an h element lying next to a code boundary passes with
    the allowance and fails without it; a planted error fails either way."""
    import types
    import numpy as np
    import torch
    import oracle
    import oracle.moe as omoe
    from test_tolerance import _w4a8_case
    case, full = _w4a8_case()
    ref = full["out"]
    tokens = case.tokens
    o = oracle.default()
    flips = lambda t: omoe.h_flip_candidates(case.cfg, full, case.W, int(tokens[t]), o)   # noqa: E731
    rms = np.sqrt(np.mean(ref * ref))
    big = [c for c in flips(129) if np.abs(c).max() > 0.05 * rms]    # the shared expert's boundary element
    assert len(big) == 1

    def batch(out):
        b = types.SimpleNamespace(cfg=case.cfg)
        b.first = {"topk_ids": full["ids"], "expert_counts": full["counts"], "expert_offsets": full["offsets"],
                   "perm": full["perm"], "topk_weights": full["w"]}
        b.first_out = torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16)
        return b

    flipped = ref.copy()
    flipped[129] += big[0]
    with_allowance = bench._parity_check(batch(flipped), full, tokens, flips)
    assert with_allowance["ok"] and with_allowance["h_codes_across_a_boundary"] == 1
    assert not bench._parity_check(batch(flipped), full, tokens)["ok"]
    bad = ref.copy()
    bad[5, 17] += 0.05 * rms
    assert not bench._parity_check(batch(bad), full, tokens, flips)["ok"]
    assert bench._parity_check(batch(ref), full, tokens, flips)["ok"]
