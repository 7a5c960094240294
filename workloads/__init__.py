"""Seeded synthetic inputs for the GPT-OSS MXFP4 mixture-of-experts layer.

This module is the only code shared by the CPU oracle's tests and the GPU path's
tests and benchmark. It draws random numbers and packs them into the storage
formats the layer consumes; it performs none of the layer's arithmetic (no
dequantisation, no routing, no matmul).

Storage formats (ZeroModels GPT-OSS page, "MXFP4 experts": experts stay packed
as uint8 nibble blocks plus e8m0 scales; "Precision": dense weights in bf16):

* bf16 tensors are numpy ``uint16`` arrays holding the bf16 bit patterns. Float
  draws are made in float32 and rounded to bf16 with round-to-nearest-even.
* packed expert blocks are ``uint8`` arrays ``[E, rows, cols/2]``; every byte is
  drawn uniformly in 0..255, i.e. both nibbles are uniform 4-bit codes.
* scales are ``uint8`` arrays ``[E, rows, cols/32]``; each byte is ``127 + x``
  with the exponent ``x`` uniform over the config's integer range.

Random streams: ``numpy.random.Generator(PCG64(SeedSequence([cfg_id, tensor_id,
seed])))`` with fixed tensor ids, so each tensor of each config is reproducible
on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Tuple

import numpy as np

__all__ = ["MoeConfig", "CONFIGS", "TENSOR_IDS", "ALL_PARTS", "make_inputs", "bf16_bits_from_f32",
           "f32_from_bf16_bits", "shape_of"]

TENSOR_IDS = {
    "x": 0, "router_w": 1, "router_b": 2, "gu_blocks": 3, "gu_scales": 4,
    "gu_bias": 5, "dn_blocks": 6, "dn_scales": 7, "dn_bias": 8, "expert_offset": 9,
    "norm_w": 10,
}


@dataclass(frozen=True)
class MoeConfig:
    """One synthetic workload: layer shape plus value distributions."""
    name: str
    cfg_id: int
    T: int
    H: int
    I: int
    E: int
    k: int
    router_w_std: float = 0.02
    router_b_std: float = 0.02
    expert_offset_std: float = 0.0   # per-expert N(0, std) added to the router bias
    norm_w_std: float = 0.1          # RMSNorm weights 1 + N(0, std)
    scale_exp_lo: int = -8           # e8m0 exponent range, inclusive
    scale_exp_hi: int = -3
    bias_std: float = 0.02
    alpha: float = 1.702
    limit: float = 7.0

    def with_(self, **kw) -> "MoeConfig":
        return replace(self, **kw)


# The workloads: a tiny layer for exhaustive parity, GPT-OSS-20B / 120B shaped layers
# (embed_dim = mlp_dim = 2880, 32 or 128 experts, top-4; ZeroModels GPT-OSS page, "API"
# table) at decode and prefill token counts, and one GPU's shard of the 20B layer.
CONFIGS: Dict[str, MoeConfig] = {
    "tiny": MoeConfig("tiny", 0, T=8, H=64, I=64, E=4, k=2, router_b_std=0.01,
                      scale_exp_lo=-6, scale_exp_hi=-2),
    "decode_20b": MoeConfig("decode_20b", 1, T=1, H=2880, I=2880, E=32, k=4),
    "batched_decode_20b": MoeConfig("batched_decode_20b", 2, T=64, H=2880, I=2880, E=32, k=4,
                                    expert_offset_std=1.0),
    "prefill_20b": MoeConfig("prefill_20b", 3, T=4096, H=2880, I=2880, E=32, k=4),
    "prefill_120b": MoeConfig("prefill_120b", 4, T=2048, H=2880, I=2880, E=128, k=4),
    # One GPU's share of the 20B layer on eight GPUs, at its real shape. Tensor-parallel decode:
    # every expert's I sliced eight ways on 32-element block boundaries (90 blocks: shards of 11
    # or 12 blocks; the larger, I = 384, sets the step), the router and x replicated.
    # Expert-parallel prefill: four local experts receiving 2048 routed rows (a quarter each)
    # of the 4096-token batch, drawn here as 2048 tokens routed top-1 over those four experts.
    "decode_20b_tp8": MoeConfig("decode_20b_tp8", 5, T=1, H=2880, I=384, E=32, k=4),
    "batched_decode_20b_tp8": MoeConfig("batched_decode_20b_tp8", 6, T=64, H=2880, I=384, E=32, k=4,
                                        expert_offset_std=1.0),
    "prefill_20b_ep8": MoeConfig("prefill_20b_ep8", 7, T=2048, H=2880, I=2880, E=4, k=1),
}


def shape_of(cfg: MoeConfig) -> Tuple[int, int, int, int, int]:
    return cfg.T, cfg.H, cfg.I, cfg.E, cfg.k


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(cfg: MoeConfig, tensor: str, seed: int) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.cfg_id, TENSOR_IDS[tensor], seed])
    return np.random.Generator(np.random.PCG64(ss))


def _normal_bf16(cfg, tensor, seed, shape, std) -> np.ndarray:
    draw = _rng(cfg, tensor, seed).standard_normal(size=shape, dtype=np.float32)
    return bf16_bits_from_f32(draw * np.float32(std))


def _bytes(cfg, tensor, seed, shape) -> np.ndarray:
    return _rng(cfg, tensor, seed).integers(0, 256, size=shape, dtype=np.uint8)


def _scales(cfg, tensor, seed, shape) -> np.ndarray:
    e = _rng(cfg, tensor, seed).integers(cfg.scale_exp_lo, cfg.scale_exp_hi + 1, size=shape,
                                         dtype=np.int16)
    return (127 + e).astype(np.uint8)


ALL_PARTS = ("x", "router_w", "router_b", "gu_blocks", "gu_scales", "gu_bias", "dn_blocks",
             "dn_scales", "dn_bias", "norm_w")


def make_inputs(cfg: MoeConfig, seed: int = 0, T: int | None = None,
                parts=ALL_PARTS) -> Dict[str, np.ndarray]:
    """Draw the input tensors of ``cfg`` (host numpy arrays).

    ``T`` overrides the token count (the weights do not depend on it; ``x`` is
    drawn for that many tokens). ``parts`` selects which tensors to draw; each
    tensor has its own random stream, so a subset has the same values as in the
    full set.
    """
    T = cfg.T if T is None else T
    H, I, E = cfg.H, cfg.I, cfg.E
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of the 32-element scale block")

    def router_bias():
        b = _rng(cfg, "router_b", seed).standard_normal(size=(E,), dtype=np.float32)
        b = b * np.float32(cfg.router_b_std)
        if cfg.expert_offset_std:
            off = _rng(cfg, "expert_offset", seed).standard_normal(size=(E,), dtype=np.float32)
            b = b + off * np.float32(cfg.expert_offset_std)
        return bf16_bits_from_f32(b)

    makers = {
        "x": lambda: _normal_bf16(cfg, "x", seed, (T, H), 1.0),
        "router_w": lambda: _normal_bf16(cfg, "router_w", seed, (E, H), cfg.router_w_std),
        "router_b": router_bias,
        "gu_blocks": lambda: _bytes(cfg, "gu_blocks", seed, (E, 2 * I, H // 2)),
        "gu_scales": lambda: _scales(cfg, "gu_scales", seed, (E, 2 * I, H // 32)),
        "gu_bias": lambda: _normal_bf16(cfg, "gu_bias", seed, (E, 2 * I), cfg.bias_std),
        "dn_blocks": lambda: _bytes(cfg, "dn_blocks", seed, (E, H, I // 2)),
        "dn_scales": lambda: _scales(cfg, "dn_scales", seed, (E, H, I // 32)),
        "dn_bias": lambda: _normal_bf16(cfg, "dn_bias", seed, (E, H), cfg.bias_std),
        # the pre-MoE RMSNorm's weights (used by the Pre-LN block entry point only)
        "norm_w": lambda: bf16_bits_from_f32(
            np.float32(1.0) + _rng(cfg, "norm_w", seed).standard_normal(size=(H,), dtype=np.float32)
            * np.float32(cfg.norm_w_std)),
    }
    unknown = set(parts) - set(makers)
    if unknown:
        raise ValueError(f"unknown input tensors {sorted(unknown)}")
    return {name: makers[name]() for name in ALL_PARTS if name in parts}
