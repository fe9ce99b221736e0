"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and its host-side validation returns the documented codes before
anything is enqueued (no call here reaches a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import nvfp4_block_scaled_router_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moe_[a-z0-9_]+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(m.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = m.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert m.moe_abi_version() == m.MOE_ABI_VERSION


def desc(**kw):
    base = dict(hidden=256, inter=128, num_experts=8, top_k=2, max_tokens=16)
    base.update(kw)
    return m.make_desc(**base)


def plan_rc(d):
    plan, pb, wb = ctypes.c_void_p(), ctypes.c_size_t(), ctypes.c_size_t()
    rc = m.lib().moe_plan(ctypes.byref(d), ctypes.byref(plan), ctypes.byref(pb), ctypes.byref(wb))
    if rc == 0:
        m.moe_plan_destroy(plan.value)
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(), m.MOE_OK),
    (dict(abi_version=7), m.MOE_ERR_ABI),
    (dict(hidden=200), m.MOE_ERR_SHAPE),
    (dict(hidden=0), m.MOE_ERR_SHAPE),
    (dict(inter=96), m.MOE_ERR_SHAPE),
    (dict(num_experts=0), m.MOE_ERR_SHAPE),
    (dict(num_experts=1025), m.MOE_ERR_SHAPE),
    (dict(top_k=9), m.MOE_ERR_SHAPE),
    (dict(top_k=0), m.MOE_ERR_SHAPE),
    (dict(max_tokens=0), m.MOE_ERR_SHAPE),
    (dict(num_shared=2), m.MOE_ERR_SHAPE),
    (dict(score=5), m.MOE_ERR_ENUM),
    (dict(act=5), m.MOE_ERR_ENUM),
    (dict(act=-1), m.MOE_ERR_ENUM),
    (dict(act="mxfp8"), m.MOE_ERR_SHAPE),                   # MXFP8 activations need MXFP4 weights
    (dict(act="mxfp8", weights="mxfp4"), m.MOE_OK),
    (dict(act="fp8"), m.MOE_OK),                            # FP8 rows: NVFP4 weights ...
    (dict(act="fp8", weights="mxfp4"), m.MOE_OK),           # ... or MXFP4 ones
    # router / activation variants (ABI 2)
    (dict(score="sqrt_softplus", use_bias=True, n_group=4, topk_group=2, routed_scaling=2.5,
          swiglu_limit=10.0), m.MOE_OK),
    (dict(renormalize=False), m.MOE_OK),
    (dict(swiglu_limit=0.0), m.MOE_OK),
    (dict(n_group=3), m.MOE_ERR_SHAPE),                    # does not divide E = 8
    (dict(n_group=8, topk_group=1), m.MOE_ERR_SHAPE),      # 1 group of 1 expert < k = 2
    (dict(n_group=4, topk_group=5), m.MOE_ERR_SHAPE),
    (dict(n_group=4, topk_group=0), m.MOE_ERR_SHAPE),
    (dict(routed_scaling=0.0), m.MOE_ERR_SHAPE),
    (dict(routed_scaling=float("inf")), m.MOE_ERR_SHAPE),
    (dict(swiglu_limit=-1.0), m.MOE_ERR_SHAPE),
    (dict(swiglu_limit=float("nan")), m.MOE_ERR_SHAPE),
    (dict(score=3), m.MOE_ERR_ENUM),
    (dict(weights="mxfp4"), m.MOE_OK),
    (dict(weights=2), m.MOE_ERR_ENUM),
])
def test_plan_validation(kw, code):
    assert plan_rc(desc(**kw)) == code


class moe_desc_v1(ctypes.Structure):
    """The version-1 descriptor: the current one without the fields added in ABI 2."""
    _fields_ = m.moe_desc._fields_[:10]


def test_plan_accepts_version1_descriptor():
    d2 = desc()
    d1 = moe_desc_v1()
    for name, _ in moe_desc_v1._fields_:
        setattr(d1, name, getattr(d2, name))
    d1.abi_version = 1
    as_desc = lambda d: ctypes.cast(ctypes.pointer(d), ctypes.POINTER(m.moe_desc))
    sizes = []
    for d in (d1, d2):
        plan, pb, wb = ctypes.c_void_p(), ctypes.c_size_t(), ctypes.c_size_t()
        assert m.lib().moe_plan(as_desc(d), ctypes.byref(plan), ctypes.byref(pb), ctypes.byref(wb)) == 0
        m.moe_plan_destroy(plan.value)
        sizes.append((pb.value, wb.value))
    assert sizes[0] == sizes[1]
    d1.renormalize = 0                                       # version 1 has no un-renormalised weights
    plan = ctypes.c_void_p()
    assert m.lib().moe_plan(as_desc(d1), ctypes.byref(plan), None, None) == m.MOE_ERR_SHAPE


def test_pack_router_bias_validation():
    fake = 1 << 20
    plain, pb, _ = m.moe_plan(desc())
    biased, pb2, _ = m.moe_plan(desc(use_bias=True))
    L = m.lib()
    try:
        assert pb2 >= pb + 8 * 4
        assert L.moe_pack_router_bias(plain, fake, fake, pb, None) == m.MOE_ERR_SHAPE    # no bias declared
        assert L.moe_pack_router_bias(biased, None, fake, pb2, None) == m.MOE_ERR_NULL
        assert L.moe_pack_router_bias(biased, fake, fake, pb2 - 1, None) == m.MOE_ERR_SIZE
        assert L.moe_pack_router_bias(biased, fake + 2, fake, pb2, None) == m.MOE_ERR_ALIGN
    finally:
        m.moe_plan_destroy(plain)
        m.moe_plan_destroy(biased)


def test_plan_sizes_cover_the_layout():
    # deepseek-v3-shaped layer: packed bytes are 0.5625 B per weight plus small tile padding
    d = desc(hidden=7168, inter=2048, num_experts=256, top_k=8, max_tokens=8192, score="sigmoid", num_shared=1)
    plan, pb, wb = m.moe_plan(d)
    m.moe_plan_destroy(plan)
    weights = 257 * 3 * 2048 * 7168
    assert weights * 0.5625 <= pb <= weights * 0.5625 * 1.01
    rows = 8192 * 9
    # h16 with its block exponents and row minimum, y16 with its block exponents
    assert wb >= rows * (2048 * 2 + 2048 // 16 + 4 + 7168 * 2 + 7168 // 16)
    # NVFP4 h: fp32 rows, codes, block scales and a global scale per row instead of h16
    d4 = desc(hidden=7168, inter=2048, num_experts=256, top_k=8, max_tokens=8192, score="sigmoid",
              num_shared=1, act="nvfp4_all")
    plan, pb4, wb4 = m.moe_plan(d4)
    m.moe_plan_destroy(plan)
    assert pb4 == pb
    assert wb4 >= rows * (2048 * 4 + 2048 // 2 + 2048 // 16 + 4 + 4 + 7168 * 2 + 7168 // 16) + 8192 * (7168 // 2)


def test_fp8_rows_workspace():
    """FP8 rows: the fp32 h rows, their fp16 decode and one scale per row; no block exponents."""
    kw = dict(hidden=2048, inter=768, num_experts=128, top_k=8, max_tokens=4096)
    plan, _, wb = m.moe_plan(desc(**kw))
    m.moe_plan_destroy(plan)
    plan, _, wb8 = m.moe_plan(desc(act="fp8", **kw))
    m.moe_plan_destroy(plan)
    rows = 4096 * 8
    assert wb8 >= rows * (768 * 4 + 768 * 2 + 4 + 4 + 2048 * 2 + 2048 // 16) + 4096 * 2048 * 2
    assert wb8 - wb >= rows * (768 * 4 + 4 - 768 // 16)


def test_quantize_fp8_rows_rejects():
    L = m.lib()
    fake = 1 << 20
    assert L.moe_quantize_fp8_rows(None, 4, 64, fake, fake, None) == m.MOE_ERR_NULL
    assert L.moe_quantize_fp8_rows(fake, 4, 60, fake, fake, None) == m.MOE_ERR_SHAPE
    assert L.moe_quantize_fp8_rows(fake, -1, 64, fake, fake, None) == m.MOE_ERR_SHAPE
    assert L.moe_quantize_fp8_rows(fake, 4, 16384 + 16, fake, fake, None) == m.MOE_ERR_SHAPE
    assert L.moe_quantize_fp8_rows(fake + 2, 4, 64, fake, fake, None) == m.MOE_ERR_ALIGN
    assert L.moe_quantize_fp8_rows(fake, 4, 64, fake + 4, fake, None) == m.MOE_ERR_ALIGN
    assert L.moe_quantize_fp8_rows(fake, 4, 64, fake, fake + 2, None) == m.MOE_ERR_ALIGN


def test_run_rejects_before_enqueue():
    plan, pb, wb = m.moe_plan(desc())
    L = m.lib()
    fake = 1 << 20        # 16-byte aligned addresses that are never dereferenced
    try:
        assert L.moe_run(None, fake, 4, fake, fake, fake, None, fake, wb, None) == m.MOE_ERR_NULL
        assert L.moe_run(plan, fake, 17, fake, fake, fake, None, fake, wb, None) == m.MOE_ERR_TOKENS
        assert L.moe_run(plan, fake, -1, fake, fake, fake, None, fake, wb, None) == m.MOE_ERR_TOKENS
        assert L.moe_run(plan, fake, 4, fake, fake, fake, None, fake, wb - 1, None) == m.MOE_ERR_SIZE
        assert L.moe_run(plan, fake + 2, 4, fake, fake, fake, None, fake, wb, None) == m.MOE_ERR_ALIGN
        assert L.moe_run(plan, fake, 4, fake, fake, fake, None, fake + 8, wb, None) == m.MOE_ERR_ALIGN
        assert L.moe_run(plan, fake, 0, fake, fake, fake, None, fake, wb, None) == m.MOE_OK   # nothing to do
        r = m.routing_out(topk_ids=fake + 2)
        assert L.moe_run(plan, fake, 4, fake, fake, fake, ctypes.byref(r), fake, wb, None) == m.MOE_ERR_ALIGN
        t = m.nvfp4_tensor(fake, fake, fake)
        assert L.moe_pack_weights(plan, ctypes.byref(t), ctypes.byref(t), None, None, fake, pb - 1, None) == m.MOE_ERR_SIZE
        assert L.moe_pack_weights(plan, ctypes.byref(t), None, None, None, fake, pb, None) == m.MOE_ERR_NULL
        assert L.moe_run_no_alloc(None, fake, 4, fake, fake, fake, None, None) == m.MOE_ERR_NULL
        assert L.moe_quantize_nvfp4_rows(fake, 4, 40, fake, fake, fake, None) == m.MOE_ERR_SHAPE
        assert L.moe_quantize_nvfp4_rows(fake + 4, 4, 64, fake, fake, fake, None) == m.MOE_ERR_ALIGN
        assert L.moe_quantize_nvfp4_weights(fake, 1, 0, 64, fake, fake, fake, None) == m.MOE_ERR_SHAPE
    finally:
        m.moe_plan_destroy(plan)
    with pytest.raises(RuntimeError, match="token count"):
        p2, _, w2 = m.moe_plan(desc())
        try:
            m.moe_run(p2, fake, 99, fake, fake, fake, None, fake, w2, stream=0)
        finally:
            m.moe_plan_destroy(p2)


def test_no_alloc_rejects_oversize_plan():
    """A plan whose workspace exceeds the static scratch is rejected on the host, before
    any HIP call; a plan within it is not (checked here up to the first HIP call only
    through sizes)."""
    plan, pb, wb = m.moe_plan(desc(hidden=2048, inter=768, num_experts=128, top_k=8, max_tokens=4096))
    fake = 1 << 20
    try:
        assert wb > m.MOE_STATIC_SCRATCH_BYTES
        assert m.lib().moe_run_no_alloc(plan, fake, 4, fake, fake, fake, None, None) == m.MOE_ERR_SCRATCH
    finally:
        m.moe_plan_destroy(plan)
    plan, pb, wb = m.moe_plan(desc(hidden=2048, inter=768, num_experts=128, top_k=8, max_tokens=64))
    m.moe_plan_destroy(plan)
    assert wb <= m.MOE_STATIC_SCRATCH_BYTES
    with pytest.raises(RuntimeError, match="static scratch"):
        p2, _, _ = m.moe_plan(desc(hidden=2048, inter=768, num_experts=128, top_k=8, max_tokens=4096))
        try:
            m.moe_run_no_alloc(p2, fake, 4, fake, fake, fake, None, stream=0)
        finally:
            m.moe_plan_destroy(p2)


def test_validate_weights_host():
    d = desc()
    G, N, K = 8, 256, 256
    packed = np.zeros((G, N, K // 2), np.uint8)
    scales = np.full((G, N, K // 16), 0x38, np.uint8)
    gs = np.ones(G, np.float32)
    t = m.nvfp4_tensor(packed.ctypes.data, scales.ctypes.data, gs.ctypes.data)
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_OK
    scales[3, 7, 2] = 0x7F                              # E4M3fn NaN
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_ERR_WEIGHT
    scales[3, 7, 2] = 0xB8                              # negative scale
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_ERR_WEIGHT
    scales[3, 7, 2] = 0x38
    gs[5] = np.inf
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_ERR_WEIGHT
    gs[5] = 1.0
    assert m.moe_validate_weights_host(d, t, 4) == m.MOE_ERR_ENUM


def test_strerror_covers_every_code():
    for code in range(-9, 1):
        assert m.moe_strerror(code) and m.moe_strerror(code) != "unknown error"


def test_validate_mxfp4_weights_host():
    d = desc(weights="mxfp4")
    G, N, K = 8, 256, 256
    packed = np.zeros((G, N, K // 2), np.uint8)
    scales = np.full((G, N, K // 32), 120, np.uint8)
    t = m.nvfp4_tensor(packed.ctypes.data, scales.ctypes.data, None)     # no global scale
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_OK
    scales[2, 5, 1] = 120 - 17                         # the widest exact span
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_OK
    scales[2, 5, 1] = 120 - 18
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_ERR_WEIGHT
    d8 = desc(weights="mxfp4", act="mxfp8")            # native E8M0 for the scaled MFMA: any span
    assert m.moe_validate_weights_host(d8, t, 0) == m.MOE_OK
    scales[2, 5, 1] = 0xFF                             # E8M0 NaN
    assert m.moe_validate_weights_host(d, t, 0) == m.MOE_ERR_WEIGHT
    assert m.moe_validate_weights_host(d8, t, 0) == m.MOE_ERR_WEIGHT
    scales[2, 5, 1] = 120
    t_nv = m.nvfp4_tensor(packed.ctypes.data, scales.ctypes.data, None)
    assert m.moe_validate_weights_host(desc(), t_nv, 0) == m.MOE_ERR_NULL   # NVFP4 needs its global scale
