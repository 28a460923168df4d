"""Seeded synthetic inputs for the attention workloads.

This module holds no part of the method's arithmetic: it only draws random
tensors, scales them and rounds them to the storage type, so the same bytes
can be handed to the GPU path and, widened to fp64, to the CPU oracle.

Recipe: ``numpy.random.Generator(PCG64(seed)).standard_normal(shape,
float32)``, drawn in the order Q, K, V, each in C order ``[b, s, H, d]``,
multiplied by its scale in fp32, then (bf16 workloads) rounded to bfloat16
by round-to-nearest-even.
"""
from dataclasses import dataclass, field
import math
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16" storage/compute type of Q, K, V
    b: int
    s: int
    hq: int
    hkv: int
    d: int
    cp: int
    seed: int
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    rope_theta: Optional[float] = None
    note: str = field(default="", compare=False)

    @property
    def c(self) -> int:
        return self.s // (2 * self.cp)

    @property
    def rank(self) -> int:
        """The measured rank: the middle one, max(cp/2 - 1, 0).

        Every rank has the same causal work; this one runs both kinds of
        non-causal step (cp/2 - 1 KV-first-half and cp/2 Q-second-half).
        """
        return max(self.cp // 2 - 1, 0)

    def rank_flops(self) -> int:
        """Causal-effective FLOPs of one rank's share: 4*d per visible pair."""
        c = self.c
        pairs = c * (2 * c + 1) + (self.cp - 1) * 2 * c * c
        return 4 * self.d * self.b * self.hq * pairs


WORKLOADS = {
    w.name: w for w in [
        Workload("fp32_mha_s512_cp2", "f32", 1, 512, 4, 4, 64, 2, seed=0,
                 note="fp32 debug path, all ranks, all rows"),
        Workload("bf16_gqa_s8k_cp4", "bf16", 1, 8192, 32, 8, 128, 4, seed=1,
                 q_scale=0.5, k_scale=0.5, v_scale=0.5),
        Workload("bf16_gqa_s32k_cp8", "bf16", 1, 32768, 64, 8, 128, 8, seed=2,
                 q_scale=0.5, k_scale=0.5, v_scale=0.5,
                 note="headline: one rank's share, all cp steps plus merge"),
        Workload("bf16_mha_s16k_cp4_widelogits", "bf16", 2, 16384, 16, 16, 128, 4,
                 seed=3, q_scale=math.sqrt(5.0), k_scale=math.sqrt(5.0),
                 v_scale=1.0,
                 note="logit std 5, extremes near +-30: stresses the LSE merge"),
        Workload("bf16_gqa_s128k_cp16_rope", "bf16", 1, 131072, 32, 8, 128, 16,
                 seed=4, q_scale=0.5, k_scale=0.5, v_scale=0.5,
                 rope_theta=10000.0,
                 note="one rank's 8192 rows vs all keys, RoPE at global positions"),
    ]
}
HEADLINE = "bf16_gqa_s32k_cp8"
SMALL = "fp32_mha_s512_cp2"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def make_inputs(w: Workload, b=None, s=None):
    """Returns (q, k, v) for workload ``w`` (optionally at another b or s).

    fp32 workloads: float32 arrays.  bf16 workloads: uint16 arrays holding
    the bfloat16 bits.  Shapes: q [b, s, hq, d], k and v [b, s, hkv, d].
    """
    b = w.b if b is None else b
    s = w.s if s is None else s
    rng = np.random.Generator(np.random.PCG64(w.seed))
    out = []
    for h, scale in ((w.hq, w.q_scale), (w.hkv, w.k_scale), (w.hkv, w.v_scale)):
        x = rng.standard_normal((b, s, h, w.d), dtype=np.float32)
        x *= np.float32(scale)
        out.append(f32_to_bf16_bits(x) if w.dtype == "bf16" else x)
    return tuple(out)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Exact fp32 value of an input array (bf16 bits widened, fp32 as is)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, np.float32)
