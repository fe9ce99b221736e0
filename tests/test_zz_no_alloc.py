"""moe_run_no_alloc (the library's static device scratch as the workspace, no allocation)
against moe_run on the same inputs: output and every routing output byte-identical, two
calls in a row with the second smaller, on a decode-regime and a prefill-regime layer and
a W4A4 layer with a shared expert (each later call finds the scratch holding the previous
layer's values)."""
import pytest
import torch

import synth
import nvfp4_block_scaled_router_amd as m
from gpu_util import Case, DEV, bf16, log, up

pytestmark = pytest.mark.gpu


def _both(case, L, T):
    x, lg = bf16(case.x[:T]), up(case.logits[:T])
    bufs_a, rout_a = L.routing_buffers(T)
    a = torch.empty((T, case.cfg.H), dtype=torch.bfloat16, device=DEV)
    m.moe_run(L.plan, L.packed, T, x, lg, a, rout_a, L.workspace, L.workspace_bytes)
    bufs_b, rout_b = L.routing_buffers(T)
    for v in bufs_b.values():
        v.fill_(0x5A if v.dtype == torch.uint8 else 7)
    b = torch.full_like(a, 7.0)
    m.moe_run_no_alloc(L.plan, L.packed, T, x, lg, b, rout_b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (case.cfg.name, T)
    for k in bufs_a:
        assert torch.equal(bufs_a[k], bufs_b[k]), (case.cfg.name, T, k)
    log(f"  {case.cfg.name} T={T}: moe_run_no_alloc == moe_run (output and routing outputs)")


CASES = [
    (synth.qwen3_decode(64), (64, 8)),
    (synth.with_tokens(synth.qwen3_prefill(), 300, "qwen3-prefill-t300"), (300, 129)),
    (synth.MoeConfig("shared-w4a4-no-alloc", T=150, H=512, I=128, E=8, k=2, shared=1, act="nvfp4", seed=14),
     (150, 13)),
]


def test_no_alloc_matches_run():
    for cfg, Ts in CASES:
        case = Case(cfg)
        L = case.layer()
        assert L.workspace_bytes <= m.MOE_STATIC_SCRATCH_BYTES
        for T in Ts:
            _both(case, L, T)
        del L
