"""The five workloads VSA is checked and measured on.

Each entry fixes a token grid, head count, head dimension, element type and
top-K.  Shapes follow the video-DiT workloads on the FastWan / VSA write-up
("一张卡，秒生视频" results section: the 410M scaling DiT with latent
(16,32,32), Wan-1.3B fine-tuned on 16x28x52 latents; and the Wan2.1-14B 720p
case of more than 80k tokens in the section on the two bottlenecks).  Latents
are patchified 1x2x2, so (16,32,32) -> 16x16x16 tokens and 16x28x52 ->
16x14x26 tokens.

This module only describes shapes; it holds no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    Hh: int
    Ww: int
    d: int
    dtype: str            # "f32" or "bf16"
    topk: int
    structure: str        # "offset" (per-cube shared offset) or "field" (smooth field)
    alpha: float          # offset / field amplitude added to q and k
    backward: bool = False
    # oracle sampling for shapes the fp64 oracle cannot finish in seconds
    sample_heads: Optional[Tuple[int, ...]] = None
    sample_qcubes: int = 0

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.Ww

    @property
    def cube_grid(self) -> Tuple[int, int, int]:
        return (-(-self.T // 4), -(-self.Hh // 4), -(-self.Ww // 4))

    @property
    def C(self) -> int:
        ct, ch, cw = self.cube_grid
        return ct * ch * cw

    @property
    def Np(self) -> int:
        return 64 * self.C

    def with_topk(self, k: int) -> "Workload":
        return replace(self, topk=k, name=f"{self.name}-k{k}")


def topk_from_ratio(ratio: float, C: int) -> int:
    """K = max(1, round(ratio * C)); 0.2/0.1/0.03 of 112 cubes give 22/11/3."""
    return max(1, int(round(ratio * C)))


TINY_F32 = Workload("tiny-f32", B=1, H=2, T=8, Hh=8, Ww=8, d=64, dtype="f32",
                    topk=2, structure="offset", alpha=1.0)
DIT_410M = Workload("dit410m", B=1, H=16, T=16, Hh=16, Ww=16, d=64, dtype="bf16",
                    topk=8, structure="offset", alpha=0.5)
WAN_1_3B = Workload("wan1.3b-480p", B=1, H=12, T=16, Hh=14, Ww=26, d=128, dtype="bf16",
                    topk=14, structure="field", alpha=0.5)
WAN_14B = Workload("wan14b-720p", B=1, H=40, T=21, Hh=45, Ww=80, d=128, dtype="bf16",
                   topk=144, structure="field", alpha=0.5,
                   sample_heads=None, sample_qcubes=16)
SWEEP_RATIOS = (0.2, 0.1, 0.03)
SWEEP = tuple(
    replace(WAN_1_3B, name=f"wan1.3b-sweep-r{r}", topk=topk_from_ratio(r, WAN_1_3B.C),
            backward=True)
    for r in SWEEP_RATIOS
)

ALL = (TINY_F32, DIT_410M, WAN_1_3B, WAN_14B) + SWEEP
BY_NAME = {w.name: w for w in ALL}
