"""Seeded synthetic workloads for the NVFP4 block-scaled fused-MoE layer.

This package is the one module that both sides of every check share: the CPU
oracle (``oracle/``) and the HIP path (``nvfp4_block_scaled_router_amd``) get
their inputs from here and from nowhere else. It draws random numbers only and
holds none of the method's arithmetic.

Workload shapes follow the configurations the pages' models imply (b12x
README, "What's in here" / ``moe`` and "DeepSeek V4 Flash 0731 MoE
reproduction"; vllm.cpp STATUS capability table, Qwen3 MoE rows; megamoe
README, "MoE kernel"). Recipe, per tensor:

* activations ``x``   : bf16(N(0, 1))                         stream 1
* router logits       : f32(N(0, 1) [+ Zipf bias])             stream 2
* routed gate_up W1   : f32(N(0, 0.02)), [E][2I][H]            stream 3
* routed down W2      : f32(N(0, 0.02)), [E][H][I]             stream 4
* shared gate_up/down : same, 1 expert                          streams 5, 6
* Zipf rank permutation (skewed workload)                       stream 7
* router selection bias (variant routers)   : f32(N(0, sigma)) stream 8
* sharing workloads: a seeded expert pool order                 stream 9
  (token t's k picks are pool[(t k + j) mod U], U = max(k, round(T k (1 - sharing)))
  distinct experts in all; their logits are set to 20 - j / 4, above every N(0, 1) draw)
* MXFP4 weights (second weight format), drawn directly in the boundary format:
  E2M1 code bytes uniform over 0..255 and E8M0 scales uniform over 117..124
  (2^-10 .. 2^-3)                                         streams 20 + 2p, 21 + 2p
  (p = 0 w1, 1 w2, 2 ws1, 3 ws2)

The generator is counter based (see ``synth.c``): element ``i`` of a stream
depends only on (seed, stream, i).
"""
from __future__ import annotations

import ctypes
import math
import os
import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

STREAM_X, STREAM_LOGITS, STREAM_W1, STREAM_W2, STREAM_WS1, STREAM_WS2, STREAM_ZIPF = 1, 2, 3, 4, 5, 6, 7
STREAM_BIAS = 8
STREAM_SHARE = 9
WEIGHT_SIGMA = 0.02

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, i32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_bits.restype = u64
        L.synth_bits.argtypes = [u64, u64, u64]
        L.synth_normal.restype = f64
        L.synth_normal.argtypes = [u64, u64, u64]
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, f64, f64, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, i64, f64, vp]
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_logits.argtypes = [u64, u64, u64, i32, i32, vp, vp]
        L.synth_bytes.argtypes = [u64, u64, u64, i64, ctypes.c_uint32, ctypes.c_uint32, vp]
        _lib = L
    return _lib


@dataclass(frozen=True)
class MoeConfig:
    """One workload: layer shape, router, activation format and seed."""
    name: str
    T: int                  # tokens in the batch
    H: int                  # hidden size
    I: int                  # expert intermediate size
    E: int                  # routed experts
    k: int                  # experts per token
    score: str = "softmax"  # "softmax" | "sigmoid" | "sqrt_softplus"
    shared: int = 0         # always-on shared experts (0 or 1), intermediate size I
    act: str = "bf16"       # "bf16" (W4A16) | "nvfp4" (row-quantised x, W4A4) | "nvfp4_all" (x and h)
                            # | "mxfp8" (x and h MXFP8, with MXFP4 weights: W4A8)
                            # | "fp8" (x and h FP8 with a per-row scale, NVFP4 weights: W4A8)
    zipf_s: float = 0.0     # > 0: add -s*ln(rank_e) to every logit of expert e
    seed: int = 0
    # router / activation variants (the defaults are the plain layer)
    bias_sigma: float = 0.0         # > 0: a per-expert selection bias N(0, sigma) (stream 8)
    n_group: int = 1                # group step: E in n_group groups, topk_group of them kept
    topk_group: int = 1
    renorm: bool = True             # weights renormalised over the k picks
    routed_scaling: float = 1.0     # factor on the routed weights
    swiglu_limit: Optional[float] = None   # clamped SwiGLU limit (routed experts), None = plain
    wfmt: str = "nvfp4"             # weight format: "nvfp4" (quantised fp32 draws) | "mxfp4" (drawn directly)
    sharing: float = -1.0           # >= 0: the fraction of (token, expert) picks reused across the batch

    @property
    def variant_router(self) -> bool:
        """True when the router is not the plain top-k (needs the generalised router)."""
        return (self.score == "sqrt_softplus" or self.bias_sigma > 0 or self.n_group > 1
                or not self.renorm or self.routed_scaling != 1.0)

    @property
    def rows(self) -> int:
        return self.T * self.k


def tiny() -> MoeConfig:
    return MoeConfig("tiny", T=16, H=256, I=128, E=8, k=2, seed=101)


DECODE_TOKENS = (1, 8, 32, 64)


def qwen3_decode(T: int) -> MoeConfig:
    assert T in DECODE_TOKENS
    return MoeConfig(f"qwen3-30b-a3b-decode-t{T}", T=T, H=2048, I=768, E=128, k=8, seed=200 + T)


def qwen3_prefill() -> MoeConfig:
    return MoeConfig("qwen3-30b-a3b-prefill", T=4096, H=2048, I=768, E=128, k=8, seed=301)


def deepseek_v3() -> MoeConfig:
    return MoeConfig("deepseek-v3", T=8192, H=7168, I=2048, E=256, k=8, score="sigmoid",
                     shared=1, seed=401)


def skewed_w4a4() -> MoeConfig:
    return MoeConfig("skewed-w4a4", T=512, H=4096, I=1536, E=64, k=4, act="nvfp4",
                     zipf_s=1.2, seed=501)


def skewed_w4a4_all() -> MoeConfig:
    """The skewed W4A4 layer with h quantised to NVFP4 as well (W4A4 down GEMM)."""
    return dataclasses.replace(skewed_w4a4(), name="skewed-w4a4-all", act="nvfp4_all")


def deepseek_v3_router(T: int = 256) -> MoeConfig:
    """DeepSeek-V3's router on the DeepSeek-V3 layer shape: sigmoid scores, a selection
    bias, 8 groups of 32 experts with 4 kept, routed scaling 2.5."""
    return MoeConfig(f"deepseek-v3-noaux-t{T}", T=T, H=7168, I=2048, E=256, k=8, score="sigmoid",
                     shared=1, seed=411, bias_sigma=0.05, n_group=8, topk_group=4, routed_scaling=2.5)


def deepseek_v4_flash(T: int = 64) -> MoeConfig:
    """DeepSeek-V4-Flash routed layer at one rank's share of a 2-way split of each expert's
    intermediate width: 256 experts, top 6, hidden 4096, intermediate 1024, MXFP4 weights,
    sqrt-softplus scores with a selection bias, SwiGLU clamped at 10, one shared expert."""
    return MoeConfig(f"deepseek-v4-flash-t{T}", T=T, H=4096, I=1024, E=256, k=6, score="sqrt_softplus",
                     shared=1, seed=421, bias_sigma=0.5, swiglu_limit=10.0, wfmt="mxfp4")


def deepseek_v4_flash_w4a8(T: int = 64) -> MoeConfig:
    """The DeepSeek-V4-Flash layer in its W4A8 profile: MXFP4 weights with MXFP8 activations
    (x and h)."""
    return dataclasses.replace(deepseek_v4_flash(T), name=f"deepseek-v4-flash-w4a8-t{T}", act="mxfp8")


def qwen3_w4a8(T: int) -> MoeConfig:
    """The Qwen3-30B-A3B layer on the W4A8 path with NVFP4 weights: x and h FP8 with one
    scale per row."""
    return MoeConfig(f"qwen3-30b-a3b-w4a8-t{T}", T=T, H=2048, I=768, E=128, k=8, act="fp8", seed=600 + T % 97)


SHARING_LEVELS = (0.0, 0.2, 0.4, 0.6, 0.8, 1.0)


def deepseek_v4_flash_sharing(T: int, sharing: float) -> MoeConfig:
    """One rank's routed DeepSeek-V4-Flash MoE (no shared expert) on a sharing workload:
    the fraction `sharing` of the T x 6 (token, expert) picks reuses experts across the
    batch (at T = 6: 36, 29, 22, 14, 7, 6 distinct experts for 0 .. 100%)."""
    level = int(round(sharing * 100))
    return MoeConfig(f"deepseek-v4-flash-t{T}-shared{level}", T=T, H=4096, I=1024, E=256, k=6,
                     score="sqrt_softplus", shared=0, seed=440 + 10 * T + level // 20, bias_sigma=0.5,
                     swiglu_limit=10.0, wfmt="mxfp4", sharing=sharing)


def all_configs():
    return [tiny()] + [qwen3_decode(t) for t in DECODE_TOKENS] + [qwen3_prefill(), deepseek_v3(), skewed_w4a4()]


def with_tokens(cfg: MoeConfig, T: int, name: Optional[str] = None) -> MoeConfig:
    """Same layer and seed, another batch size (for bounded samples and edge cases)."""
    d = dict(cfg.__dict__)
    d["T"] = T
    d["name"] = name or f"{cfg.name}-t{T}"
    return MoeConfig(**d)


# --------------------------------------------------------------------------- draws

def normal_f32(seed: int, stream: int, offset: int, n: int, sigma: float, mean: float = 0.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        lib().synth_normal_f32(seed, stream, offset, n, mean, sigma, out.ctypes.data)
    return out


def normal_bf16(seed: int, stream: int, offset: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma) draws."""
    out = np.empty(n, dtype=np.uint16)
    if n:
        lib().synth_normal_bf16(seed, stream, offset, n, sigma, out.ctypes.data)
    return out


def zipf_bias(cfg: MoeConfig) -> Optional[np.ndarray]:
    """Per-expert logit bias -s*ln(r_e), r_e a seeded permutation of 1..E (None if s == 0)."""
    if cfg.zipf_s <= 0:
        return None
    ranks = np.empty(cfg.E, dtype=np.int32)
    lib().synth_permutation(cfg.seed, STREAM_ZIPF, cfg.E, ranks.ctypes.data)
    return np.array([-cfg.zipf_s * math.log(int(r)) for r in ranks], dtype=np.float64)


MX_SCALE_LO, MX_SCALE_SPAN = 117, 8
_MX_PROJ = {"w1": 0, "w2": 1, "ws1": 2, "ws2": 3}


def mxfp4_weights(cfg: MoeConfig, which: str, first: int, count: int):
    """MXFP4 projection of experts first..first+count-1 in the boundary layout: codes
    u8 [count][N][K/2] (element 2i in the low nibble), E8M0 scales u8 [count][N][K/32]."""
    N, K = _proj_shape(cfg, which)
    p = _MX_PROJ[which]
    codes = np.empty(count * N * K // 2, np.uint8)
    scales = np.empty(count * N * K // 32, np.uint8)
    if codes.size:
        lib().synth_bytes(cfg.seed, 20 + 2 * p, first * N * K // 2, codes.size, 0, 256, codes.ctypes.data)
        lib().synth_bytes(cfg.seed, 21 + 2 * p, first * N * K // 32, scales.size, MX_SCALE_LO, MX_SCALE_SPAN,
                          scales.ctypes.data)
    return codes.reshape(count, N, K // 2), scales.reshape(count, N, K // 32)


def router_bias(cfg: MoeConfig) -> Optional[np.ndarray]:
    """Per-expert selection bias, float32 [E] (None if bias_sigma == 0)."""
    if cfg.bias_sigma <= 0:
        return None
    return normal_f32(cfg.seed, STREAM_BIAS, 0, cfg.E, cfg.bias_sigma)


def activations(cfg: MoeConfig) -> np.ndarray:
    """x as bf16 bit patterns, shape [T][H]."""
    return normal_bf16(cfg.seed, STREAM_X, 0, cfg.T * cfg.H).reshape(cfg.T, cfg.H)


def sharing_experts(cfg: MoeConfig) -> np.ndarray:
    """The designated picks [T][k] of a sharing workload: U = max(k, round(T k (1 - sharing)))
    experts of a seeded pool, token t taking pool[(t k + j) mod U] (k distinct per token)."""
    A = cfg.T * cfg.k
    U = min(cfg.E, max(cfg.k, int(round(A * (1.0 - cfg.sharing)))))
    ranks = np.empty(cfg.E, dtype=np.int32)
    lib().synth_permutation(cfg.seed, STREAM_SHARE, cfg.E, ranks.ctypes.data)
    pool = np.argsort(ranks, kind="stable")[:U]
    idx = (np.arange(cfg.T)[:, None] * cfg.k + np.arange(cfg.k)[None, :]) % U
    return pool[idx].astype(np.int32)


def logits(cfg: MoeConfig) -> np.ndarray:
    """Router logits, float32 [T][E]."""
    out = np.empty(cfg.T * cfg.E, dtype=np.float32)
    bias = zipf_bias(cfg)
    bptr = bias.ctypes.data if bias is not None else None
    lib().synth_logits(cfg.seed, STREAM_LOGITS, 0, cfg.T, cfg.E, bptr, out.ctypes.data)
    out = out.reshape(cfg.T, cfg.E)
    if cfg.sharing >= 0:
        picks = sharing_experts(cfg)
        for j in range(cfg.k):
            out[np.arange(cfg.T), picks[:, j]] = np.float32(20.0 - 0.25 * j)
    return out


def _proj_shape(cfg: MoeConfig, which: str):
    if which in ("w1", "ws1"):
        return 2 * cfg.I, cfg.H
    if which in ("w2", "ws2"):
        return cfg.H, cfg.I
    raise ValueError(which)


_STREAM_OF = {"w1": STREAM_W1, "w2": STREAM_W2, "ws1": STREAM_WS1, "ws2": STREAM_WS2}


def expert_weight_f32(cfg: MoeConfig, which: str, expert: int) -> np.ndarray:
    """Unquantised fp32 weights of one expert: w1/ws1 -> [2I][H] (rows 0..I-1 gate,
    I..2I-1 up); w2/ws2 -> [H][I]."""
    N, K = _proj_shape(cfg, which)
    n = N * K
    return normal_f32(cfg.seed, _STREAM_OF[which], expert * n, n, WEIGHT_SIGMA).reshape(N, K)


def expert_weights_f32(cfg: MoeConfig, which: str, first: int, count: int) -> np.ndarray:
    """Experts first..first+count-1 stacked: [count*N][K] (one generator call)."""
    N, K = _proj_shape(cfg, which)
    n = N * K
    return normal_f32(cfg.seed, _STREAM_OF[which], first * n, count * n, WEIGHT_SIGMA).reshape(count * N, K)


def token_sample(cfg: MoeConfig, count: int, salt: int = 0) -> np.ndarray:
    """A seeded, sorted sample of distinct token indices (first and last token always in)."""
    if count >= cfg.T:
        return np.arange(cfg.T, dtype=np.int32)
    picks = {0, cfg.T - 1}
    i = 0
    while len(picks) < count:
        picks.add(int(lib().synth_bits(cfg.seed, 1000 + salt, i) % cfg.T))
        i += 1
    return np.array(sorted(picks), dtype=np.int32)
