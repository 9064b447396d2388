"""Seeded synthetic inputs for the packed-ternary x INT8-activation matmul.

This module is the only thing the CPU oracle and the HIP path share.  It
holds none of the method's arithmetic: it draws random code bytes, random
fp16 block scales and random activations, and lays the raw 34-byte blocks out
(scale bytes first, then 32 code bytes, the block format given on the page
"Kernel experiments: recorded evidence", section A / Diagram 1).  The four
2-bit fields of every code byte are drawn independently from the same
distribution, so the generator makes no statement about which field is which
weight; the decode (the method's business) lives separately in the oracle and
in the kernels.

Workloads (the shapes and value distributions the pages' decode and prefill
projections use; no dataset or trained weights are involved):

  tiny    K=512,   N=1024,  M=1          codes ternary + 1% code 3, seed 0
  qkv     K=5120,  N=10240, M=1..4       codes as tiny; N(0,1) activations with
                                         0.1% outliers at +-20, seed 2
  up      K=5120,  N=17408, M=1..4, 8    codes uniform {0,1,2}, seed 3
  down    K=17408, N=5120,  M=1,2,4,16   codes as tiny; Laplace(0, 0.5)
                                         activations, seed 4
  prefill K=5120,  N=6144 / 17408, M=256, 512, 1024; codes uniform {0,1,2};
          N(0,1) activations, seed 5 (gate) / 6 (up)

Block scales are U[0.005, 0.05] rounded to fp16 (round to nearest even) in
every workload.  Activations are drawn once at [max M][K] per workload; a
smaller M uses the first M rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

GROUP = 128
BLOCK_BYTES = 34


@dataclass(frozen=True)
class Workload:
    name: str
    k: int
    n: int
    ms: tuple
    seed: int
    codes: str        # "ternary" (uniform 0,1,2) or "ternary+3" (1% code 3)
    act: str          # "normal", "normal+outliers" or "laplace"

    @property
    def groups(self) -> int:
        return self.k // GROUP

    def weight_bytes(self) -> int:
        return self.n * self.groups * BLOCK_BYTES


WORKLOADS = {
    "tiny": Workload("tiny", 512, 1024, (1,), 0, "ternary+3", "normal"),
    "qkv": Workload("qkv", 5120, 10240, (1, 2, 3, 4), 2, "ternary+3", "normal+outliers"),
    "up": Workload("up", 5120, 17408, (1, 2, 3, 4, 8), 3, "ternary", "normal"),
    "down": Workload("down", 17408, 5120, (1, 2, 4, 16), 4, "ternary+3", "laplace"),
    "prefill_gate": Workload("prefill_gate", 5120, 6144, (256, 512, 1024), 5, "ternary", "normal"),
    "prefill_up": Workload("prefill_up", 5120, 17408, (256, 512, 1024), 6, "ternary", "normal"),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _draw_codes(gen: torch.Generator, count: int, dist: str) -> torch.Tensor:
    """`count` independent 2-bit codes (uint8 in 0..3)."""
    codes = torch.randint(0, 3, (count,), generator=gen, dtype=torch.uint8)
    if dist == "ternary+3":
        rare = torch.randint(0, 100, (count,), generator=gen, dtype=torch.uint8) == 0
        codes[rare] = 3
    elif dist != "ternary":
        raise ValueError(dist)
    return codes


def make_raw_weights(n: int, k: int, seed: int, codes: str = "ternary",
                     row_pad: int = 0) -> np.ndarray:
    """Raw PQ2 rows: uint8 [n][k/128*34 + row_pad] (pad bytes are 0xEE)."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 128")
    gen = _gen(seed)
    groups = k // GROUP
    fields = _draw_codes(gen, n * groups * 32 * 4, codes).view(n, groups, 32, 4)
    code_bytes = (fields[..., 0] | (fields[..., 1] << 2) | (fields[..., 2] << 4)
                  | (fields[..., 3] << 6))
    scales = (torch.rand((n, groups), generator=gen, dtype=torch.float32) * 0.045 + 0.005)
    scale_bytes = scales.to(torch.float16).contiguous().view(torch.uint8).view(n, groups, 2)
    blocks = torch.cat([scale_bytes, code_bytes], dim=2).reshape(n, groups * BLOCK_BYTES)
    if row_pad:
        pad = torch.full((n, row_pad), 0xEE, dtype=torch.uint8)
        blocks = torch.cat([blocks, pad], dim=1)
    return blocks.contiguous().numpy()


def make_activations(m: int, k: int, seed: int, dist: str = "normal") -> torch.Tensor:
    """bf16 activations [m][k] (CPU tensor), rounded to nearest even from FP32."""
    gen = _gen(seed + 1000)
    if dist in ("normal", "normal+outliers"):
        x = torch.randn((m, k), generator=gen, dtype=torch.float32)
        if dist == "normal+outliers":
            hit = torch.rand((m, k), generator=gen) < 0.001
            sign = torch.randint(0, 2, (m, k), generator=gen).to(torch.float32) * 2 - 1
            x = torch.where(hit, 20.0 * sign, x)
    elif dist == "laplace":
        # Inverse CDF of Laplace(0, b=0.5) on an open-interval uniform.
        v = torch.randint(1, 1 << 24, (m, k), generator=gen).to(torch.float64) / float(1 << 24)
        u = v - 0.5
        x = (-0.5 * torch.sign(u) * torch.log1p(-2.0 * u.abs())).to(torch.float32)
    else:
        raise ValueError(dist)
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 CPU tensor."""
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def workload_inputs(name: str, m: int | None = None, row_pad: int = 0):
    """(raw weights uint8 [n][stride], bf16 activations [m][k]) for a workload."""
    w = WORKLOADS[name]
    m = max(w.ms) if m is None else m
    raw = make_raw_weights(w.n, w.k, w.seed, w.codes, row_pad=row_pad)
    x = make_activations(max(w.ms), w.k, w.seed, w.act)[:m].contiguous()
    return raw, x
