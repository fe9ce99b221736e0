"""GPU routing (top-k ids, weights, counts, offsets, permutation) against the oracle."""
import numpy as np
import pytest
import torch

import synth
import oracle
import nvfp4_block_scaled_router_amd as m
from gpu_util import DEV, W_ABS, log, up

pytestmark = pytest.mark.gpu


def _route_on_gpu(cfg, logits, bias=None):
    """Run the whole layer (tiny H, I) and read back the routing outputs."""
    L = m.MoeLayer(128, 128, cfg.E, cfg.k, cfg.T, cfg.score, "bf16", 0, DEV, use_bias=bias is not None,
                   n_group=cfg.n_group, topk_group=cfg.topk_group, renormalize=cfg.renorm,
                   routed_scaling=cfg.routed_scaling)
    z = lambda *s: torch.zeros(s, dtype=torch.uint8, device=DEV)
    W1 = (z(cfg.E, 256, 64), torch.full((cfg.E, 256, 8), 0x38, dtype=torch.uint8, device=DEV),
          torch.ones(cfg.E, device=DEV))
    W2 = (z(cfg.E, 128, 64), torch.full((cfg.E, 128, 8), 0x38, dtype=torch.uint8, device=DEV),
          torch.ones(cfg.E, device=DEV))
    L.pack(W1, W2)
    if bias is not None:
        L.pack_router_bias(up(bias))
    x = torch.zeros((cfg.T, 128), dtype=torch.bfloat16, device=DEV)
    bufs, rout = L.routing_buffers(cfg.T)
    out = L(x, up(logits), routing=rout)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    return {k: v.cpu().numpy() for k, v in bufs.items()}


def _check(cfg, logits, bias=None):
    o = oracle.default()
    if cfg.variant_router or bias is not None:
        ids, w = o.route_general(logits, cfg.k, cfg.score, bias, cfg.n_group, cfg.topk_group, cfg.renorm,
                                 cfg.routed_scaling)
    else:
        ids, w = o.route(logits, cfg.k, cfg.score)
    counts, offsets, perm, inv = o.plan(ids, cfg.E)
    got = _route_on_gpu(cfg, logits, bias)
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


# generalised router: every score, bias on/off, group step, both plan paths (T*k <= 4096 in
# one workgroup, larger through the count/scan/scatter kernels), up to 1024 experts
@pytest.mark.parametrize("E,k,T,score,bias,ng,tg,renorm,scale", [
    (128, 8, 64, "sqrt_softplus", 0.5, 1, 1, True, 1.0),
    (256, 8, 2000, "sigmoid", 0.05, 8, 4, True, 2.5),
    (256, 6, 7, "sqrt_softplus", 0.5, 1, 1, True, 1.0),
    (64, 4, 513, "softmax", 0.0, 4, 2, False, 1.0),
    (1024, 16, 300, "sigmoid", 0.1, 64, 8, True, 1.5),
    (72, 3, 100, "softmax", 0.2, 36, 5, True, 1.0),
    (8, 8, 40, "sqrt_softplus", 1.0, 2, 2, False, 3.0),
])
def test_route_general(E, k, T, score, bias, ng, tg, renorm, scale):
    cfg = synth.MoeConfig(f"route-gen-e{E}-k{k}-t{T}", T=T, H=128, I=128, E=E, k=k, score=score,
                          seed=950 + E + k + T, bias_sigma=bias, n_group=ng, topk_group=tg, renorm=renorm,
                          routed_scaling=scale)
    _check(cfg, synth.logits(cfg), synth.router_bias(cfg))


@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrt_softplus"])
def test_route_general_ties(score):
    """Equal keys everywhere (equal logits, no or equal bias): lower ids win, groups too."""
    cfg = synth.MoeConfig("gen-ties", T=200, H=128, I=128, E=64, k=6, score=score, seed=78, n_group=8,
                          topk_group=3, routed_scaling=2.0)
    lg = np.round(synth.logits(cfg) * 2) / 2
    lg[0] = 0.5
    lg[1] = -0.0
    lg[1, 5] = 0.0
    _check(cfg, lg.astype(np.float32), np.zeros(64, np.float32))
    _check(cfg, lg.astype(np.float32), np.full(64, 0.25, np.float32))
