"""Python binding of libnvfp4moe.so: the NVFP4 block-scaled fused-MoE layer on MI355X.

Thin ctypes marshalling over the C ABI in ``include/nvfp4_moe.h``; every step of
the layer runs in the library's HIP kernels. PyTorch only supplies device memory
(tensors, passed by ``data_ptr()``) and streams. Functions keep the C names and
raise ``RuntimeError`` with ``moe_strerror`` on a non-zero return code. There is
no fallback: if the library is missing, importing the binding works but the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4moe.so")

MOE_ABI_VERSION = 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SQRT_SOFTPLUS = 0, 1, 2
MOE_ACT_BF16, MOE_ACT_NVFP4_ROWQ, MOE_ACT_NVFP4_ALL, MOE_ACT_MXFP8, MOE_ACT_FP8_ROW = 0, 1, 2, 3, 4
MOE_WEIGHTS_NVFP4, MOE_WEIGHTS_MXFP4 = 0, 1
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_SIZE, MOE_ERR_TOKENS = 0, -1, -2, -3, -4
MOE_ERR_ALIGN, MOE_ERR_ABI, MOE_ERR_ENUM, MOE_ERR_WEIGHT, MOE_ERR_SCRATCH = -5, -6, -7, -8, -9
MOE_STATIC_SCRATCH_BYTES = 64 << 20

MOE_STAGE_QUANT, MOE_STAGE_ROUTE, MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_COMBINE = 0, 1, 2, 3, 4
MOE_NUM_STAGES = 5
STAGE_NAMES = ("h_prep", "route", "gate_up", "down", "combine")   # h_prep: MOE_STAGE_QUANT

EXPORTED = ("moe_plan", "moe_plan_destroy", "moe_pack_weights", "moe_pack_router_bias", "moe_run", "moe_run_timed",
            "moe_run_no_alloc",
            "moe_quantize_nvfp4_rows", "moe_quantize_fp8_rows", "moe_quantize_nvfp4_weights", "moe_validate_weights_host", "moe_strerror",
            "moe_abi_version")

_i32, _u32, _sz, _vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p


class moe_desc(ctypes.Structure):
    _fields_ = [("abi_version", _u32), ("hidden", _i32), ("inter", _i32), ("num_experts", _i32),
                ("top_k", _i32), ("max_tokens", _i32), ("score_fn", _i32), ("renormalize", _i32),
                ("act_format", _i32), ("num_shared", _i32),
                # since ABI 2
                ("use_bias", _i32), ("n_group", _i32), ("topk_group", _i32), ("swiglu_clamp", _i32),
                ("routed_scaling", ctypes.c_float), ("swiglu_limit", ctypes.c_float), ("weight_format", _i32)]


class moe_nvfp4_tensor(ctypes.Structure):
    _fields_ = [("packed", _vp), ("scales", _vp), ("global_scale", _vp)]


class moe_routing_out(ctypes.Structure):
    _fields_ = [("topk_ids", _vp), ("topk_weights", _vp), ("expert_counts", _vp), ("expert_offsets", _vp),
                ("perm", _vp), ("act_packed", _vp), ("act_scales", _vp), ("act_global", _vp)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_plan.restype = _i32
        L.moe_plan.argtypes = [ctypes.POINTER(moe_desc), ctypes.POINTER(_vp), ctypes.POINTER(_sz),
                               ctypes.POINTER(_sz)]
        L.moe_plan_destroy.restype = None
        L.moe_plan_destroy.argtypes = [_vp]
        T = ctypes.POINTER(moe_nvfp4_tensor)
        L.moe_pack_weights.restype = _i32
        L.moe_pack_weights.argtypes = [_vp, T, T, T, T, _vp, _sz, _vp]
        L.moe_pack_router_bias.restype = _i32
        L.moe_pack_router_bias.argtypes = [_vp, _vp, _vp, _sz, _vp]
        L.moe_run.restype = _i32
        L.moe_run.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.POINTER(moe_routing_out), _vp, _sz, _vp]
        L.moe_run_timed.restype = _i32
        L.moe_run_timed.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.POINTER(moe_routing_out), _vp, _sz, _vp,
                                    ctypes.POINTER(_vp)]
        L.moe_run_no_alloc.restype = _i32
        L.moe_run_no_alloc.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.POINTER(moe_routing_out), _vp]
        L.moe_quantize_nvfp4_rows.restype = _i32
        L.moe_quantize_nvfp4_rows.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp]
        L.moe_quantize_fp8_rows.restype = _i32
        L.moe_quantize_fp8_rows.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp]
        L.moe_quantize_nvfp4_weights.restype = _i32
        L.moe_quantize_nvfp4_weights.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]
        L.moe_validate_weights_host.restype = _i32
        L.moe_validate_weights_host.argtypes = [ctypes.POINTER(moe_desc), T, _i32]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [_i32]
        L.moe_abi_version.restype = _u32
        L.moe_abi_version.argtypes = []
        if L.moe_abi_version() != MOE_ABI_VERSION:
            raise RuntimeError("libnvfp4moe.so ABI version does not match the binding")
        _lib = L
    return _lib


def moe_strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def _check(rc: int):
    if rc != 0:
        raise RuntimeError(f"libnvfp4moe: {moe_strerror(rc)} (code {rc})")


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL); ints are taken as raw addresses."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(hidden: int, inter: int, num_experts: int, top_k: int, max_tokens: int, score: str = "softmax",
              act: str = "bf16", num_shared: int = 0, abi_version: int = MOE_ABI_VERSION, *,
              use_bias: bool = False, n_group: int = 1, topk_group: int = 1, renormalize: bool = True,
              routed_scaling: float = 1.0, swiglu_limit: Optional[float] = None,
              weights: str = "nvfp4") -> moe_desc:
    """Layer descriptor; the keyword arguments select the router and activation variants
    (all off by default: the plain layer)."""
    d = moe_desc()
    d.abi_version = abi_version
    d.hidden, d.inter, d.num_experts, d.top_k, d.max_tokens = hidden, inter, num_experts, top_k, max_tokens
    d.score_fn = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID,
                  "sqrt_softplus": MOE_SCORE_SQRT_SOFTPLUS}.get(score, score)
    d.renormalize = 1 if renormalize else 0
    d.act_format = {"bf16": MOE_ACT_BF16, "nvfp4": MOE_ACT_NVFP4_ROWQ, "nvfp4_all": MOE_ACT_NVFP4_ALL,
                    "mxfp8": MOE_ACT_MXFP8, "fp8": MOE_ACT_FP8_ROW}.get(act, act)
    d.num_shared = num_shared
    d.use_bias = 1 if use_bias else 0
    d.n_group, d.topk_group = n_group, topk_group
    d.routed_scaling = routed_scaling
    d.swiglu_clamp = 0 if swiglu_limit is None else 1
    d.swiglu_limit = 0.0 if swiglu_limit is None else swiglu_limit
    d.weight_format = {"nvfp4": MOE_WEIGHTS_NVFP4, "mxfp4": MOE_WEIGHTS_MXFP4}.get(weights, weights)
    return d


def moe_plan(desc: moe_desc):
    """-> (plan handle, packed_bytes, workspace_bytes); raises on a rejected descriptor."""
    plan, pb, wb = _vp(), _sz(), _sz()
    _check(lib().moe_plan(ctypes.byref(desc), ctypes.byref(plan), ctypes.byref(pb), ctypes.byref(wb)))
    return plan.value, pb.value, wb.value


def moe_plan_destroy(plan) -> None:
    lib().moe_plan_destroy(plan)


def nvfp4_tensor(packed, scales, global_scale) -> moe_nvfp4_tensor:
    t = moe_nvfp4_tensor()
    t.packed, t.scales, t.global_scale = _ptr(packed), _ptr(scales), _ptr(global_scale)
    return t


def _tref(t: Optional[moe_nvfp4_tensor]):
    return None if t is None else ctypes.byref(t)


def moe_pack_router_bias(plan, bias, packed, packed_bytes: int, stream=None) -> None:
    """Copy the per-expert selection bias (device f32 [E]) into the packed buffer."""
    _check(lib().moe_pack_router_bias(plan, _ptr(bias), _ptr(packed), packed_bytes, _stream(stream)))


def moe_pack_weights(plan, gate_up: moe_nvfp4_tensor, down: moe_nvfp4_tensor,
                     shared_gate_up: Optional[moe_nvfp4_tensor], shared_down: Optional[moe_nvfp4_tensor],
                     packed, packed_bytes: int, stream=None) -> None:
    _check(lib().moe_pack_weights(plan, _tref(gate_up), _tref(down), _tref(shared_gate_up), _tref(shared_down),
                                  _ptr(packed), packed_bytes, _stream(stream)))


def routing_out(topk_ids=None, topk_weights=None, expert_counts=None, expert_offsets=None, perm=None,
                act_packed=None, act_scales=None, act_global=None) -> moe_routing_out:
    r = moe_routing_out()
    r.topk_ids, r.topk_weights = _ptr(topk_ids), _ptr(topk_weights)
    r.expert_counts, r.expert_offsets, r.perm = _ptr(expert_counts), _ptr(expert_offsets), _ptr(perm)
    r.act_packed, r.act_scales, r.act_global = _ptr(act_packed), _ptr(act_scales), _ptr(act_global)
    return r


def moe_run(plan, packed, T: int, x, router_logits, out, routing: Optional[moe_routing_out], workspace,
            workspace_bytes: int, stream=None) -> None:
    _check(lib().moe_run(plan, _ptr(packed), T, _ptr(x), _ptr(router_logits), _ptr(out),
                         None if routing is None else ctypes.byref(routing), _ptr(workspace), workspace_bytes,
                         _stream(stream)))


def moe_run_timed(plan, packed, T: int, x, router_logits, out, routing: Optional[moe_routing_out], workspace,
                  workspace_bytes: int, stream, stage_events) -> None:
    """stage_events: sequence of 2*MOE_NUM_STAGES raw hipEvent_t handles (int or None)."""
    arr = (_vp * (2 * MOE_NUM_STAGES))(*[e or None for e in stage_events])
    _check(lib().moe_run_timed(plan, _ptr(packed), T, _ptr(x), _ptr(router_logits), _ptr(out),
                               None if routing is None else ctypes.byref(routing), _ptr(workspace),
                               workspace_bytes, _stream(stream), arr))


def moe_run_no_alloc(plan, packed, T: int, x, router_logits, out, routing: Optional[moe_routing_out],
                     stream=None) -> None:
    """moe_run with the library's static device scratch as the workspace (no allocation)."""
    _check(lib().moe_run_no_alloc(plan, _ptr(packed), T, _ptr(x), _ptr(router_logits), _ptr(out),
                                  None if routing is None else ctypes.byref(routing), _stream(stream)))


def moe_quantize_nvfp4_rows(x, rows: int, K: int, packed, scales, row_global, stream=None) -> None:
    _check(lib().moe_quantize_nvfp4_rows(_ptr(x), rows, K, _ptr(packed), _ptr(scales), _ptr(row_global),
                                         _stream(stream)))


def moe_quantize_fp8_rows(x, rows: int, K: int, codes, row_scale, stream=None) -> None:
    _check(lib().moe_quantize_fp8_rows(_ptr(x), rows, K, _ptr(codes), _ptr(row_scale), _stream(stream)))


def moe_quantize_nvfp4_weights(w, groups: int, rows_per_group: int, K: int, packed, scales, group_global,
                               stream=None) -> None:
    _check(lib().moe_quantize_nvfp4_weights(_ptr(w), groups, rows_per_group, K, _ptr(packed), _ptr(scales),
                                            _ptr(group_global), _stream(stream)))


def moe_validate_weights_host(desc: moe_desc, host_copy: moe_nvfp4_tensor, which: int) -> int:
    """Returns the code (0 or MOE_ERR_*) rather than raising: it is a check."""
    return int(lib().moe_validate_weights_host(ctypes.byref(desc), ctypes.byref(host_copy), which))


from .layer import MoeLayer  # noqa: E402  (torch-side plumbing around the C calls)
