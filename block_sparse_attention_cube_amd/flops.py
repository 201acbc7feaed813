"""Work accounting for VSA calls (host-side arithmetic, used by the bench).

The fine stage executes, per (query cube, selected key cube) pair, two 64x64xd
products (Q K^T and P V): 4 * 64 * 64 * d FLOPs.  Sparsity 1 - K/C therefore
cuts attention FLOPs by C/K -- 8x at 87.5% (the 410M scaling experiment in
the results section "一张卡，秒生视频" of the FastWan/VSA re-post).
"""
from __future__ import annotations

from typing import Sequence

BLOCK = 64

# MI355X published dense peaks (no structured sparsity)
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2       # 256 CU x 2.4 GHz x 8192 FLOP/clk
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0


def fine_forward_flops(B: int, H: int, C: int, K: int, d: int) -> int:
    """FLOPs the 64x64-block fine kernel executes (pad slots included)."""
    return 4 * d * BLOCK * BLOCK * B * H * C * K


def fine_backward_flops(B: int, H: int, C: int, K: int, d: int) -> int:
    """Backward of the fine stage: 5 block products (S recompute, dV, dP, dQ, dK)
    against 2 in the forward, i.e. 2.5x."""
    return fine_forward_flops(B, H, C, K, d) * 5 // 2


def dense_flops(B: int, H: int, n_tokens: int, d: int) -> int:
    """Dense attention over n_tokens queries and keys."""
    return 4 * d * n_tokens * n_tokens * B * H


def useful_fine_flops(B: int, H: int, d: int, n_valid: Sequence[int], idx) -> int:
    """Valid x valid FLOPs: 4 d sum_i n_i sum_{j in idx[i]} n_j, summed over (b, h).

    idx: array-like [B, H, C, K] of selected cubes; n_valid[c] the valid slot count."""
    import numpy as np
    n = np.asarray(n_valid, dtype=np.int64)
    sel = np.asarray(idx, dtype=np.int64)
    per_row = n[sel].sum(axis=-1)                  # [B, H, C]
    return int(4 * d * (per_row * n[None, None, :]).sum())


def executed_fine_flops(B: int, H: int, K: int, d: int, t_extent: Sequence[int]) -> int:
    """FLOPs the bf16 fine kernel executes: each query cube's four 16-row
    waves hold time slices 0..3, and a wave whose slice lies past the cube's
    t extent (t_extent[c], 1..4) computes nothing, so a cube costs
    min(t_extent, 4) / 4 of its 64x64-block FLOPs."""
    import numpy as np
    nt = np.minimum(np.asarray(t_extent, dtype=np.int64), 4)
    return int(4 * d * BLOCK * BLOCK * B * H * K * nt.sum() // 4)


def reorder_bytes(B: int, H: int, N: int, Np: int, d: int, elem: int, tensors: int = 3) -> int:
    """HBM bytes of the raster -> cube reorder: read N rows, write Np rows."""
    return tensors * B * H * (N + Np) * d * elem
