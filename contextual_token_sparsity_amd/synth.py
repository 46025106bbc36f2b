"""Seeded synthetic inputs for the token-elimination hot path.

This module only draws random numbers and converts them to bf16 bit patterns.
It holds none of the scoring, selection or movement arithmetic, so both the
CPU oracle (through the tests) and the HIP library can be fed from it without
sharing any of the method's code.

Recipe (the pages train on RedPajama / LongAlign / PG19 text with OPT and
Llama weights; none of that is available, so Gaussian stand-ins of the same
shapes take their place):

* ``rng = numpy.random.Generator(PCG64(seed))``; draws happen in a fixed order:
  X ~ N(0, 1) float32 ``[N][d]``; the planted block set (``choice`` without
  replacement); ``g ~ N(0, I_d)`` giving the unit direction ``u = g/|g|``;
  Wq, Wk ~ N(0, 1/d); U_q, V_q, U_k, V_k ~ N(0, 1/fan_in); the stand-in layer
  output Y ~ N(0, 1) ``[N][d]``; the MLP activation A ~ N(0, 1) ``[N][w]``.
* Planted "informative" blocks: every row of ``round(p * nb)`` chosen blocks
  gets ``+3u`` before rounding to bf16.
* Every stored tensor is rounded to bf16 (round to nearest even) by torch's
  float32 -> bfloat16 conversion and kept as raw ``uint16`` bits.
* Q = bf16(X Wq), K = bf16(X Wk), the product taken in float32 by torch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (torch's RNE conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """Shape of one synthetic layer (sizes follow the models the pages fine-tune)."""
    name: str
    n_tokens: int
    d_model: int
    block: int
    seed: int
    n_heads: int = 0            # 0: no exact-path Q/K for this workload
    head_dim: int = 0
    rank: int = 0               # 0: no predictor weights
    mlp_width: int = 0          # 0: no MLP activation
    planted_frac: float = 0.1
    keep_pct: tuple = ()        # per-layer keep ratios in percent (TOPK); () = MEAN
    n_layers: int = 1

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // self.block


# Shapes used by the tests and the benchmark.  Model widths: OPT-1.3B d=2048
# (32 heads of 64), Llama2-7B d=4096 (32 x 128, MLP 11008), Llama2-13B d=5120.
WORKLOADS = {
    "tiny": Workload("tiny", 1024, 512, 64, 20251115, n_heads=4, head_dim=128,
                     planted_frac=0.20, keep_pct=(50,)),
    "opt1.3b-n4k": Workload("opt1.3b-n4k", 4096, 2048, 64, 20252115, n_heads=32,
                            head_dim=64, planted_frac=0.15, keep_pct=(40,)),
    "llama2-7b-n8k-exact": Workload("llama2-7b-n8k-exact", 8192, 4096, 64, 20253115,
                                    n_heads=32, head_dim=128, planted_frac=0.10,
                                    keep_pct=(30,)),
    "llama2-7b-n16k": Workload("llama2-7b-n16k", 16384, 4096, 64, 20254115,
                               n_heads=32, head_dim=128, rank=128, mlp_width=11008,
                               planted_frac=0.10),
    "llama2-13b-n32k-4layer": Workload("llama2-13b-n32k-4layer", 32768, 5120, 128, 20255115,
                                       rank=256, planted_frac=0.10,
                                       keep_pct=(60, 45, 35, 25), n_layers=4),
}


@dataclass
class LayerInputs:
    """bf16 bit patterns (uint16) of one synthetic layer."""
    x: np.ndarray
    planted_blocks: np.ndarray
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    u_q: Optional[np.ndarray] = None
    v_q: Optional[np.ndarray] = None
    u_k: Optional[np.ndarray] = None
    v_k: Optional[np.ndarray] = None
    y: Optional[np.ndarray] = None
    act: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make_layer(n_tokens: int, d_model: int, block: int, seed: int, *,
               n_heads: int = 0, head_dim: int = 0, rank: int = 0,
               mlp_width: int = 0, planted_frac: float = 0.1,
               with_y: bool = True, proj_device: str = "cpu") -> LayerInputs:
    """Draw one synthetic layer.  ``proj_device`` only picks where the float32
    Q/K projection runs (a large product is slow on the host); the draw itself
    is always on the host and seeded."""
    if n_tokens % block:
        raise ValueError("n_tokens must be a multiple of block")
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = n_tokens // block
    x = _normal(rng, (n_tokens, d_model))
    n_planted = int(np.floor(planted_frac * nb + 0.5))
    planted = np.sort(rng.choice(nb, size=n_planted, replace=False)) if n_planted else np.zeros(0, np.int64)
    g = rng.standard_normal(size=d_model)
    u = (g / np.linalg.norm(g)).astype(np.float32)
    for blk in planted:
        x[blk * block:(blk + 1) * block] += np.float32(3.0) * u
    out = LayerInputs(x=to_bf16_bits(x), planted_blocks=planted)
    if n_heads:
        if n_heads * head_dim != d_model:
            raise ValueError("n_heads * head_dim must equal d_model")
        wq = _normal(rng, (d_model, d_model), 1.0 / np.sqrt(d_model))
        wk = _normal(rng, (d_model, d_model), 1.0 / np.sqrt(d_model))
        xt = torch.from_numpy(x).to(proj_device)
        for name, w in (("q", wq), ("k", wk)):
            p = (xt @ torch.from_numpy(w).to(proj_device)).to(torch.bfloat16)
            setattr(out, name, p.cpu().view(torch.int16).numpy().view(np.uint16))
        del xt
    if rank:
        out.u_q = to_bf16_bits(_normal(rng, (d_model, rank), 1.0 / np.sqrt(d_model)))
        out.v_q = to_bf16_bits(_normal(rng, (rank, rank), 1.0 / np.sqrt(rank)))
        out.u_k = to_bf16_bits(_normal(rng, (d_model, rank), 1.0 / np.sqrt(d_model)))
        out.v_k = to_bf16_bits(_normal(rng, (rank, rank), 1.0 / np.sqrt(rank)))
    if with_y:
        out.y = to_bf16_bits(_normal(rng, (n_tokens, d_model)))
    if mlp_width:
        out.act = to_bf16_bits(_normal(rng, (n_tokens, mlp_width)))
    return out


def make_workload(w: Workload, layer: int = 0, **kw) -> LayerInputs:
    return make_layer(w.n_tokens, w.d_model, w.block, w.seed + layer,
                      n_heads=w.n_heads, head_dim=w.head_dim, rank=w.rank,
                      mlp_width=w.mlp_width, planted_frac=w.planted_frac, **kw)


def random_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """Small helper for tests: N(0, std^2) values rounded to bf16 bits."""
    return to_bf16_bits(_normal(rng, shape, std))


def keep_count(keep_pct: int, n_blocks: int) -> int:
    """Number of blocks a keep ratio in whole percent asks for: ceil(pct*nb/100)
    in integer arithmetic."""
    return (keep_pct * n_blocks + 99) // 100
