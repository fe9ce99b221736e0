"""CPU oracle for the NVFP4 block-scaled fused-MoE layer (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP path (``nvfp4_block_scaled_router_amd``); both take their inputs
from ``synth``.

Every function cites, in ``oracle.c``, the page passage it follows; the pins
that check it against something other than itself are in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_vp = ctypes.c_void_p
_i32, _i64, _u32, _f32, _f64, _u16 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                      ctypes.c_float, ctypes.c_double, ctypes.c_uint16)


class ProjSet(ctypes.Structure):
    _fields_ = [("w1_packed", _vp), ("w1_scales", _vp), ("w1_gs", _vp),
                ("w2_packed", _vp), ("w2_scales", _vp), ("w2_gs", _vp), ("mx", ctypes.c_int32)]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class Oracle:
    """One loaded copy of the oracle library (tests also load planted mutants)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        L.orc_threads.restype = _i32
        L.orc_e2m1.restype = _f64
        L.orc_e2m1.argtypes = [_u32]
        L.orc_e4m3fn.restype = _f64
        L.orc_e4m3fn.argtypes = [_u32]
        L.orc_bf16.restype = _f64
        L.orc_bf16.argtypes = [_u16]
        L.orc_weight.restype = _f64
        L.orc_weight.argtypes = [_vp, _vp, _f32, _i32, _i32, _i32]
        L.orc_e8m0.restype = _f64
        L.orc_e8m0.argtypes = [_u32]
        L.orc_weight_mx.restype = _f64
        L.orc_weight_mx.argtypes = [_vp, _vp, _i32, _i32, _i32]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [_f32]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e2m1_encode.argtypes = [_f32]
        L.orc_quantize.argtypes = [_vp, _i64, _i32, _i64, _vp, _vp, _vp]
        L.orc_mxfp8_quantize.argtypes = [_vp, _i64, _i32, _vp, _vp]
        L.orc_mxfp8.restype = ctypes.c_double
        L.orc_mxfp8.argtypes = [_u32, _u32]
        L.orc_mxfp8_rows.argtypes = [_vp, _vp, _i64, _i32, _vp]
        L.orc_route.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp]
        L.orc_plan.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]
        L.orc_route_general.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _f64, _vp, _vp]
        L.orc_expert_ffn.argtypes = [ctypes.POINTER(ProjSet), _i32, _i32, _i32, _vp, _vp]
        L.orc_expert_ffn_clamp.argtypes = [ctypes.POINTER(ProjSet), _i32, _i32, _i32, _vp, _vp, _i32, _f64]
        L.orc_expert_ffn_q.argtypes = [ctypes.POINTER(ProjSet), _i32, _i32, _i32, _vp, _vp, _i32, _f64, _i32]
        L.orc_expert_h.argtypes = [ctypes.POINTER(ProjSet), _i32, _i32, _i32, _vp, _vp, _i32, _f64]
        L.orc_moe_tokens_clamp.argtypes = [ctypes.POINTER(ProjSet), ctypes.POINTER(ProjSet), _i32, _i32,
                                           _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _f64]
        L.orc_moe_tokens_q.argtypes = [ctypes.POINTER(ProjSet), ctypes.POINTER(ProjSet), _i32, _i32,
                                       _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _f64, _i32]
        L.orc_dequant_rows.argtypes = [_vp, _vp, _vp, _i64, _i32, _vp]
        L.orc_bf16_rows.argtypes = [_vp, _i64, _vp]
        L.orc_decode_proj.argtypes = [ctypes.POINTER(ProjSet), _i32, _i32, _i32, _i32, _vp]
        L.orc_fp8_rows_quantize.argtypes = [_vp, _i64, _i32, _vp, _vp]
        L.orc_fp8_rows.argtypes = [_vp, _vp, _i64, _i32, _vp]
        self.L = L
        self.path = path

    # ---------------------------------------------------------------- scalars
    def threads(self) -> int:
        return self.L.orc_threads()

    def e2m1(self, nib: int) -> float:
        return self.L.orc_e2m1(nib)

    def e4m3fn(self, b: int) -> float:
        return self.L.orc_e4m3fn(b)

    def bf16(self, b: int) -> float:
        return self.L.orc_bf16(b)

    def e4m3_encode(self, v: float) -> int:
        return int(self.L.orc_e4m3_encode(v))

    def e2m1_encode(self, r: float) -> int:
        return int(self.L.orc_e2m1_encode(r))

    # ---------------------------------------------------------------- arrays
    def quantize(self, x: np.ndarray, rows_per_gs: int = 1):
        """x float32 [rows][K] -> (packed u8 [rows][K/2], scales u8 [rows][K/16], gs f32 [rows/rows_per_gs])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        rows, K = x.shape
        assert K % 16 == 0 and rows % rows_per_gs == 0
        packed = np.zeros((rows, K // 2), np.uint8)
        scales = np.zeros((rows, K // 16), np.uint8)
        gs = np.zeros(rows // rows_per_gs, np.float32)
        self.L.orc_quantize(x.ctypes.data, rows, K, rows_per_gs, packed.ctypes.data,
                            scales.ctypes.data, gs.ctypes.data)
        return packed, scales, gs

    def mxfp8_quantize(self, x: np.ndarray):
        """float32 [rows][K] -> (codes u8 [rows][K], E8M0 scales u8 [rows][K/32])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        rows, K = x.shape
        codes = np.zeros((rows, K), np.uint8)
        scales = np.zeros((rows, K // 32), np.uint8)
        self.L.orc_mxfp8_quantize(x.ctypes.data, rows, K, codes.ctypes.data, scales.ctypes.data)
        return codes, scales

    def fp8_rows_quantize(self, x: np.ndarray):
        """float32 [rows][K] -> (E4M3 codes u8 [rows][K], per-row FP32 scales [rows])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        rows, K = x.shape
        codes = np.zeros((rows, K), np.uint8)
        scale = np.zeros(rows, np.float32)
        self.L.orc_fp8_rows_quantize(x.ctypes.data, rows, K, codes.ctypes.data, scale.ctypes.data)
        return codes, scale

    def fp8_rows(self, codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
        """Exact FP64 decode of per-row-scaled FP8 rows."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        rows, K = codes.shape
        out = np.empty((rows, K), np.float64)
        self.L.orc_fp8_rows(codes.ctypes.data, scale.ctypes.data, rows, K, out.ctypes.data)
        return out

    def mxfp8(self, code: int, scale: int) -> float:
        return self.L.orc_mxfp8(code, scale)

    def mxfp8_rows(self, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
        """Exact FP64 decode of MXFP8 rows."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        rows, K = codes.shape
        out = np.empty((rows, K), np.float64)
        self.L.orc_mxfp8_rows(codes.ctypes.data, scales.ctypes.data, rows, K, out.ctypes.data)
        return out

    def weight(self, packed, scales, gs, n, k) -> float:
        K = packed.shape[-1] * 2
        return self.L.orc_weight(packed.ctypes.data, scales.ctypes.data, float(gs), K, n, k)

    def route(self, logits: np.ndarray, k: int, score: str = "softmax"):
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        ids = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float64)
        self.L.orc_route(logits.ctypes.data, T, E, k, 0 if score == "softmax" else 1,
                         ids.ctypes.data, w.ctypes.data)
        return ids, w

    SCORES = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}

    def route_general(self, logits: np.ndarray, k: int, score: str = "sigmoid",
                      bias: Optional[np.ndarray] = None, n_group: int = 1, topk_group: int = 1,
                      renorm: bool = True, scaling: float = 1.0):
        """Generalised router (score functions, selection-only bias, group step, routed
        scaling): ids [T][k] int32 and FP64 weights [T][k]."""
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        assert E % n_group == 0 and 1 <= topk_group <= n_group and topk_group * (E // n_group) >= k
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        ids = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float64)
        self.L.orc_route_general(logits.ctypes.data, T, E, k, self.SCORES[score], _ptr(b), n_group,
                                 topk_group, int(bool(renorm)), float(scaling), ids.ctypes.data,
                                 w.ctypes.data)
        return ids, w

    def plan(self, ids: np.ndarray, E: int):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, k = ids.shape
        counts = np.zeros(E, np.int32)
        offsets = np.zeros(E + 1, np.int32)
        perm = np.zeros(T * k, np.int32)
        inv = np.zeros(T * k, np.int32)
        self.L.orc_plan(ids.ctypes.data, T, E, k, counts.ctypes.data, offsets.ctypes.data,
                        perm.ctypes.data, inv.ctypes.data)
        return counts, offsets, perm, inv

    def dequant_rows(self, packed, scales, gs) -> np.ndarray:
        rows, K2 = packed.shape
        out = np.zeros((rows, K2 * 2), np.float64)
        self.L.orc_dequant_rows(packed.ctypes.data, scales.ctypes.data, gs.ctypes.data, rows,
                                K2 * 2, out.ctypes.data)
        return out

    def bf16_rows(self, b: np.ndarray) -> np.ndarray:
        b = np.ascontiguousarray(b, dtype=np.uint16)
        out = np.zeros(b.shape, np.float64)
        self.L.orc_bf16_rows(b.ctypes.data, b.size, out.ctypes.data)
        return out

    def e8m0(self, b: int) -> float:
        return self.L.orc_e8m0(b)

    def weight_mx(self, packed, scales, n, k) -> float:
        K = packed.shape[-1] * 2
        return self.L.orc_weight_mx(packed.ctypes.data, scales.ctypes.data, K, n, k)

    def decode_projection(self, W, g: int) -> np.ndarray:
        """Expert g of one projection W = (packed [G][N][K/2], scales, gs or None) decoded to
        FP64 [N][K] by the oracle's element decode (NVFP4, or MXFP4 when gs is None)."""
        N, K = W[0].shape[1], W[0].shape[2] * 2
        ps = self._projset(W, W)
        out = np.empty((N, K), np.float64)
        self.L.orc_decode_proj(ctypes.byref(ps), 0, g, N, K, out.ctypes.data)
        return out

    @staticmethod
    def _projset(W1, W2):
        """W = (packed, scales, gs) for NVFP4, (packed, scales, None) for MXFP4 (the format is
        told by the scale width: K/16 vs K/32 bytes per row)."""
        ps = ProjSet()
        ps.w1_packed, ps.w1_scales, ps.w1_gs = _ptr(W1[0]), _ptr(W1[1]), _ptr(W1[2])
        ps.w2_packed, ps.w2_scales, ps.w2_gs = _ptr(W2[0]), _ptr(W2[1]), _ptr(W2[2])
        ps.mx = 1 if W1[2] is None else 0
        return ps

    def expert_ffn(self, W1, W2, g: int, x: np.ndarray, swiglu_limit: Optional[float] = None,
                   hq: int = 0) -> np.ndarray:
        """W1 = (packed [G][2I][H/2], scales [G][2I][H/16], gs [G]); W2 likewise [G][H][I/..].
        swiglu_limit: None for the plain SwiGLU, else the clamp limit L >= 0; hq: the down
        projection takes h row-quantised to NVFP4 (True / 1), MXFP8 (2) or per-row FP8 (3)."""
        H = W1[0].shape[-1] * 2
        I = W2[0].shape[-1] * 2
        x = np.ascontiguousarray(x, dtype=np.float64)
        y = np.zeros(H, np.float64)
        ps = self._projset(W1, W2)
        clamp = swiglu_limit is not None
        self.L.orc_expert_ffn_q(ctypes.byref(ps), g, H, I, x.ctypes.data, y.ctypes.data, int(clamp),
                                float(swiglu_limit) if clamp else 0.0, int(hq))
        return y

    def expert_h(self, W1, W2, g: int, x: np.ndarray, swiglu_limit: Optional[float] = None) -> np.ndarray:
        """h = SwiGLU(W1_g x) in FP64, before any quantisation."""
        H = W1[0].shape[-1] * 2
        I = W2[0].shape[-1] * 2
        x = np.ascontiguousarray(x, dtype=np.float64)
        h = np.zeros(I, np.float64)
        ps = self._projset(W1, W2)
        clamp = swiglu_limit is not None
        self.L.orc_expert_h(ctypes.byref(ps), g, H, I, x.ctypes.data, h.ctypes.data, int(clamp),
                            float(swiglu_limit) if clamp else 0.0)
        return h

    def moe_tokens(self, W1, W2, WS1, WS2, tokens, x_rows, ids, w,
                   swiglu_limit: Optional[float] = None, hq: bool = False) -> np.ndarray:
        """FP64 layer output for `tokens` (x_rows: their decoded inputs [n][H]); the clamp
        (swiglu_limit not None) applies to the routed experts, hq (h row-quantised to NVFP4
        before the down projection) to every expert."""
        H = W1[0].shape[-1] * 2
        I = W2[0].shape[-1] * 2
        T, k = ids.shape
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        x_rows = np.ascontiguousarray(x_rows, dtype=np.float64)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        out = np.zeros((len(tokens), H), np.float64)
        routed = self._projset(W1, W2)
        num_shared = 0 if WS1 is None else WS1[0].shape[0]
        shared = self._projset(WS1, WS2) if num_shared else ProjSet()
        clamp = swiglu_limit is not None
        self.L.orc_moe_tokens_q(ctypes.byref(routed), ctypes.byref(shared), num_shared, H, I, k,
                                len(tokens), tokens.ctypes.data, x_rows.ctypes.data, ids.ctypes.data,
                                w.ctypes.data, out.ctypes.data, int(clamp),
                                float(swiglu_limit) if clamp else 0.0, int(hq))
        return out


@functools.lru_cache(maxsize=1)
def default() -> Oracle:
    return Oracle()
