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


def query_wave_rows(T: int, Hh: int, Ww: int) -> str:
    """Which 16-slot rows the bf16 fine kernel's four query waves hold on a
    token grid: "h" (h-rows) where that idles more waves over the cube grid
    than time slices do ("t"), as its launcher decides."""
    ct, ch, cw = -(-T // 4), -(-Hh // 4), -(-Ww // 4)
    t_idle = (4 * ct - T) * ch * cw
    h_idle = (4 * ch - Hh) * ct * cw
    return "h" if h_idle > t_idle else "t"


def executed_fine_flops(grid: Sequence[int], d: int, idx) -> int:
    """FLOPs the bf16 fine kernel executes on a token grid (T, Hh, Ww) with
    block lists idx [B, H, C, K]: 4 * 64 * 64 * d per (query cube, selected
    cube) pair, scaled by
      * the query cube's active waves / 4: a wave whose 16 query slots (a
        time slice, or an h-row, see query_wave_rows) lie past the cube's
        extent computes nothing;
      * 1/2 for a selected cube at most two time slices deep: its empty
        second half is neither staged nor computed."""
    import numpy as np
    T, Hh, Ww = grid
    ct, ch, cw = -(-T // 4), -(-Hh // 4), -(-Ww // 4)
    nt = np.array([min(4, T - 4 * t) for t in range(ct) for _ in range(ch) for _ in range(cw)])
    nh = np.array([min(4, Hh - 4 * h) for _ in range(ct) for h in range(ch) for _ in range(cw)])
    waves = nh if query_wave_rows(T, Hh, Ww) == "h" else nt           # active waves per query cube
    halves = np.where(nt <= 2, 1, 2)                                    # key halves per key cube
    sel = np.asarray(idx, dtype=np.int64)
    per_query = halves[sel].sum(axis=-1)                                # [B, H, C]
    return int(BLOCK * BLOCK * d * (per_query * waves[None, None, :]).sum() // 2)


def reorder_bytes(B: int, H: int, N: int, Np: int, d: int, elem: int, tensors: int = 3) -> int:
    """HBM bytes of the raster -> cube reorder: read N rows, write Np rows."""
    return tensors * B * H * (N + Np) * d * elem
