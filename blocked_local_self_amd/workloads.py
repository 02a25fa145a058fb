"""The five synthetic halo-attention workloads and their accounting.

Shapes follow the HaloNet stages described in "Scaling Local Self-Attention
for Parameter Efficient Visual Backbones": 16 channels per head and 8 heads in
the later stages (section 2.3, appendix C.1), b=8/h=3 giving 14x14 windows
(sections 2.3 and 4.6), windows up to 18x18 (section 2.3; b=12 as in the
384-pixel transfer setting of appendix E), 64x64 and 32x32 maps from 256-pixel
inputs, and stride-2 attention downsampling (section 2.2, Figure 2); plus the
larger-window settings: b=32/h=3 from the detection study (section 4.6) and
global attention over a 16x16 map (section 2.2).

Accounting conventions (per launch):
  flops     = 4 * d * r^2 per (query, head): q.k and p.v over the full
              (b+2h)^2 window; relative-term and softmax work excluded.
  tokens    = B * (H/s) * (W/s) output positions (all heads of a position).
  alg_bytes = e * d * B*heads * (2*H*W + 2*(H/s)*(W/s)): k and v read once,
              q read at query pixels only, out written once (tables ignored).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    heads: int
    H: int
    W: int
    d: int
    block: int
    halo: int
    stride: int = 1

    @property
    def r(self) -> int:
        return self.block + 2 * self.halo

    @property
    def Ho(self) -> int:
        return self.H // self.stride

    @property
    def Wo(self) -> int:
        return self.W // self.stride

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def nblocks(self) -> int:
        nbh = -(-self.H // self.block)
        nbw = -(-self.W // self.block)
        return self.B * self.heads * nbh * nbw

    @property
    def flops(self) -> int:
        return 4 * self.d * self.r * self.r * self.B * self.heads * self.Ho * self.Wo

    @property
    def tokens(self) -> int:
        return self.B * self.Ho * self.Wo

    @property
    def alg_bytes(self) -> int:
        bh = self.B * self.heads
        return self.elem_bytes * self.d * bh * (2 * self.H * self.W + 2 * self.Ho * self.Wo)

    def shape(self) -> tuple:
        return (self.B, self.heads, self.H, self.W, self.d)

    def out_shape(self) -> tuple:
        return (self.B, self.heads, self.Ho, self.Wo, self.d)

    def describe(self) -> dict:
        return {"workload": self.name, "dtype": self.dtype, "B": self.B, "heads": self.heads,
                "H": self.H, "W": self.W, "d": self.d, "block": self.block, "halo": self.halo,
                "query_stride": self.stride, "window": f"{self.r}x{self.r}"}


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny_fp32_16x16_d16_b4h1", "fp32", 1, 2, 16, 16, 16, 4, 1, 1),
        Workload("early_stage_bf16_64x64_d16_b8h3", "bf16", 32, 8, 64, 64, 16, 8, 3, 1),
        Workload("mid_stage_bf16_32x32_d32_b8h3", "bf16", 64, 8, 32, 32, 32, 8, 3, 1),
        Workload("strided_bf16_64x64_d16_b8h3_s2", "bf16", 32, 8, 64, 64, 16, 8, 3, 2),
        Workload("large_bf16_128x128_d32_b12h3", "bf16", 8, 8, 128, 128, 32, 12, 3, 1),
        # larger windows: the detection setting with b=32, h=3 (section 4.6;
        # 38x38 windows, 1444 keys), and whole-map attention at the smallest
        # resolution (section 2.2, last paragraph: one block covers the map)
        Workload("detection_bf16_64x64_d16_b32h3", "bf16", 8, 8, 64, 64, 16, 32, 3, 1),
        Workload("global_bf16_16x16_d16_b16h0", "bf16", 64, 8, 16, 16, 16, 16, 0, 1),
    )
}

# Workload of the benchmark's headline line: the largest single-GPU shape
# (18x18 windows on 128x128 maps).
BENCH_WORKLOAD = "large_bf16_128x128_d32_b12h3"
# The HaloNet-stage shapes the headline line also reports, one entry each.
STAGE_WORKLOADS = ("early_stage_bf16_64x64_d16_b8h3", "mid_stage_bf16_32x32_d32_b8h3",
                   "strided_bf16_64x64_d16_b8h3_s2", "large_bf16_128x128_d32_b12h3")
# Default workload of the backward and whole-layer passes.
PASS_WORKLOAD = "early_stage_bf16_64x64_d16_b8h3"


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
