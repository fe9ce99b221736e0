"""Device-side NVFP4 weight preparation with the library's quantiser.

``quantize_projection`` turns fp32 expert weights, supplied chunk by chunk from the
host, into the boundary operand layout (packed [G][N][K/2], scales [G][N][K/16],
global [G]) with one global scale per expert projection, using
``moe_quantize_nvfp4_weights`` on the GPU.
"""
from __future__ import annotations

from typing import Callable, Tuple

import numpy as np
import torch

from . import moe_quantize_nvfp4_weights


def quantize_projection(G: int, N: int, K: int, draw: Callable[[int, int], np.ndarray], device,
                        chunk_bytes: int = 1 << 30, progress: Callable[[str], None] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """draw(first, count) -> fp32 [count*N][K] weights of experts first..first+count-1."""
    packed = torch.empty((G, N, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((G, N, K // 16), dtype=torch.uint8, device=device)
    gs = torch.empty(G, dtype=torch.float32, device=device)
    per = max(1, chunk_bytes // (4 * N * K))
    for e0 in range(0, G, per):
        cnt = min(per, G - e0)
        w = torch.from_numpy(draw(e0, cnt)).to(device)
        moe_quantize_nvfp4_weights(w, cnt, N, K, packed[e0:e0 + cnt], scales[e0:e0 + cnt], gs[e0:e0 + cnt])
        torch.cuda.current_stream().synchronize()
        del w
        if progress:
            progress(f"quantized experts {e0}..{e0 + cnt - 1} of {G} ({N}x{K})")
    return packed, scales, gs
