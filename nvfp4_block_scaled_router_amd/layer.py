"""Torch-side plumbing around one planned layer: owns the plan handle and the two
device buffers (packed weights, workspace) the C ABI asks the caller for."""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (make_desc, moe_pack_router_bias, moe_pack_weights, moe_plan, moe_plan_destroy, moe_run, nvfp4_tensor,
               routing_out)


class MoeLayer:
    """One NVFP4 fused-MoE layer: ``moe_plan`` + packed weights + workspace.

    Weights are given per projection as ``(packed u8 [G][N][K/2], scales u8
    [G][N][K/16], global_scale f32 [G])`` device tensors in the boundary layout
    (gate_up: N = 2I, rows 0..I-1 gate; down: N = H)."""

    def __init__(self, hidden: int, inter: int, num_experts: int, top_k: int, max_tokens: int,
                 score: str = "softmax", act: str = "bf16", num_shared: int = 0, device="cuda", **variants):
        self.desc = make_desc(hidden, inter, num_experts, top_k, max_tokens, score, act, num_shared, **variants)
        self.plan, self.packed_bytes, self.workspace_bytes = moe_plan(self.desc)
        self.device = torch.device(device)
        self.packed = torch.empty(self.packed_bytes, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)
        self.H, self.I, self.E, self.k, self.max_tokens = hidden, inter, num_experts, top_k, max_tokens
        self.S = num_shared

    @classmethod
    def from_config(cls, cfg, max_tokens: Optional[int] = None, device="cuda") -> "MoeLayer":
        return cls(cfg.H, cfg.I, cfg.E, cfg.k, max_tokens or cfg.T, cfg.score, cfg.act, cfg.shared, device,
                   use_bias=cfg.bias_sigma > 0, n_group=cfg.n_group, topk_group=cfg.topk_group,
                   renormalize=cfg.renorm, routed_scaling=cfg.routed_scaling, swiglu_limit=cfg.swiglu_limit,
                   weights=cfg.wfmt)

    def pack_router_bias(self, bias: torch.Tensor, stream=None) -> None:
        """The per-expert selection bias (device f32 [E]) of a layer declared with use_bias."""
        moe_pack_router_bias(self.plan, bias, self.packed, self.packed_bytes, stream)

    def pack(self, w1: Sequence[torch.Tensor], w2: Sequence[torch.Tensor], ws1: Optional[Sequence] = None,
             ws2: Optional[Sequence] = None, stream=None) -> None:
        t = [nvfp4_tensor(*w1), nvfp4_tensor(*w2)]
        s1 = nvfp4_tensor(*ws1) if ws1 is not None else None
        s2 = nvfp4_tensor(*ws2) if ws2 is not None else None
        moe_pack_weights(self.plan, t[0], t[1], s1, s2, self.packed, self.packed_bytes, stream)

    def __call__(self, x: torch.Tensor, logits: torch.Tensor, out: Optional[torch.Tensor] = None,
                 routing=None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=x.device)
        moe_run(self.plan, self.packed, T, x, logits, out, routing, self.workspace, self.workspace_bytes, stream)
        return out

    def routing_buffers(self, T: int):
        """Device tensors for every optional routing output, and the struct pointing at them."""
        dev = self.device
        bufs = dict(
            topk_ids=torch.empty((T, self.k), dtype=torch.int32, device=dev),
            topk_weights=torch.empty((T, self.k), dtype=torch.float32, device=dev),
            expert_counts=torch.empty(self.E, dtype=torch.int32, device=dev),
            expert_offsets=torch.empty(self.E + 1, dtype=torch.int32, device=dev),
            perm=torch.empty(T * self.k, dtype=torch.int32, device=dev),
        )
        if self.desc.act_format == 3:       # MXFP8: E4M3 codes and E8M0 scales per 32
            bufs.update(act_packed=torch.empty((T, self.H), dtype=torch.uint8, device=dev),
                        act_scales=torch.empty((T, self.H // 32), dtype=torch.uint8, device=dev))
        elif self.desc.act_format == 4:     # FP8 rows: E4M3 codes and one scale per row
            bufs.update(act_packed=torch.empty((T, self.H), dtype=torch.uint8, device=dev),
                        act_global=torch.empty(T, dtype=torch.float32, device=dev))
        elif self.desc.act_format in (1, 2):
            bufs.update(act_packed=torch.empty((T, self.H // 2), dtype=torch.uint8, device=dev),
                        act_scales=torch.empty((T, self.H // 16), dtype=torch.uint8, device=dev),
                        act_global=torch.empty(T, dtype=torch.float32, device=dev))
        return bufs, routing_out(**bufs)

    def __del__(self):
        try:
            if self.plan:
                moe_plan_destroy(self.plan)
                self.plan = None
        except Exception:
            pass
