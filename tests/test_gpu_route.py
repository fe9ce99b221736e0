"""GPU routing (top-k ids, weights, counts, offsets, permutation) against the oracle."""
import numpy as np
import pytest
import torch

import synth
import oracle
import nvfp4_block_scaled_router_amd as m
from gpu_util import DEV, W_ABS, log, up

pytestmark = pytest.mark.gpu


def _route_on_gpu(cfg, logits):
    """Run the whole layer (tiny H, I) and read back the routing outputs."""
    L = m.MoeLayer(128, 128, cfg.E, cfg.k, cfg.T, cfg.score, "bf16", 0, DEV)
    z = lambda *s: torch.zeros(s, dtype=torch.uint8, device=DEV)
    W1 = (z(cfg.E, 256, 64), torch.full((cfg.E, 256, 8), 0x38, dtype=torch.uint8, device=DEV),
          torch.ones(cfg.E, device=DEV))
    W2 = (z(cfg.E, 128, 64), torch.full((cfg.E, 128, 8), 0x38, dtype=torch.uint8, device=DEV),
          torch.ones(cfg.E, device=DEV))
    L.pack(W1, W2)
    x = torch.zeros((cfg.T, 128), dtype=torch.bfloat16, device=DEV)
    bufs, rout = L.routing_buffers(cfg.T)
    out = L(x, up(logits), routing=rout)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    return {k: v.cpu().numpy() for k, v in bufs.items()}


def _check(cfg, logits):
    o = oracle.default()
    ids, w = o.route(logits, cfg.k, cfg.score)
    counts, offsets, perm, inv = o.plan(ids, cfg.E)
    got = _route_on_gpu(cfg, logits)
    log(f"  {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k} {cfg.score}")
    assert np.array_equal(got["topk_ids"], ids)
    assert np.abs(got["topk_weights"] - w).max() <= W_ABS
    assert np.array_equal(got["expert_counts"], counts)
    assert np.array_equal(got["expert_offsets"], offsets)
    assert np.array_equal(got["perm"], perm)


@pytest.mark.parametrize("cfg", synth.all_configs(), ids=lambda c: c.name)
def test_route_workloads(cfg):
    _check(cfg, synth.logits(cfg))


@pytest.mark.parametrize("E,k,T", [(1024, 8, 300), (512, 16, 1500), (64, 64, 7), (256, 8, 1), (8, 1, 2000)])
def test_route_shapes(E, k, T):
    cfg = synth.MoeConfig(f"route-e{E}-k{k}-t{T}", T=T, H=128, I=128, E=E, k=k, seed=900 + E + k)
    _check(cfg, synth.logits(cfg))


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_route_ties(score):
    cfg = synth.MoeConfig("ties", T=333, H=128, I=128, E=128, k=8, score=score, seed=77)
    lg = np.round(synth.logits(cfg) * 2) / 2                  # many equal logits
    lg[0] = 0.5                                                # all equal: ids 0..k-1
    lg[1] = -0.0
    lg[1, 5] = 0.0                                             # -0 == +0
    _check(cfg, lg.astype(np.float32))
