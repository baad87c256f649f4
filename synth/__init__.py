"""Seeded synthetic KV-cache inputs shared by the oracle tests, the GPU tests and bench.py.

This module only draws random numbers and rounds them to the stored element type.  It holds
none of the codec's or the attention's arithmetic, and imports neither the oracle nor the HIP
library.  No model weights or datasets exist here; these distributions stand in for the model
KV states the GAAC page measures on (per-channel exponent concentration, §3.1).

Recipe (per layer, numpy PCG64, seed = (config index, layer)):
  1. per KV head h, in order: sK = lognormal(0, 1, D); sK[choice(D, n_outlier, no replace)] *= 20;
     sV = lognormal(0, 0.5, D).  Scales are a property of the layer, shared by all sequences.
  2. each call to ``tokens(n)`` draws K = N(0,1)[n][Hkv][D] * sK, then V likewise with sV,
     in float32, then rounds to BF16 (round-to-nearest-even), optionally then to FP8.
Queries: q = N(0,1)[n_seqs][Hq][D] -> BF16, seed = (config index, 7919, step).
Rotated keys (``rope_keys``): a model caches keys after its rotary position embedding; these
are the BF16 keys above rotated at their positions (pairs (c, c + D/2), inverse frequencies
theta^(-2i/D), Qwen3's theta = 1e6) in float32 and rounded back to BF16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BF16, E5M2, E4M3 = 0, 1, 2


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    n_seqs: int
    Hkv: int
    Hq: int
    D: int
    context: tuple          # per-sequence context length
    T: int                  # tokens per block
    G: int = 16             # tokens per exponent group
    n_outlier: int = 4      # outlier key channels per head
    n_cal: int = 256        # calibration tokens (first tokens of sequence 0)
    fmt: int = BF16
    appends: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


def _cfg3_lengths() -> tuple:
    rng = np.random.default_rng(3)
    return tuple(int(x) for x in rng.integers(4096, 32768, endpoint=True, size=32))


def config(index: int, fmt: int = BF16) -> Config:
    """The five workloads: 0 tiny CPU-seconds case, 1 Qwen3-0.6B-like layer, 2 the 64K
    Qwen3-8B-like headline layer, 3 the 32-sequence paged serving mix, 4 = 2 in FP8."""
    if index == 0:
        return Config(0, "tiny-2kv4q-d64-1k", 1, 2, 4, 64, (1024,), 64, n_outlier=2)
    if index == 1:
        return Config(1, "qwen3-0.6b-like-8k", 1, 8, 16, 128, (8192,), 64, appends=64)
    if index == 2:
        return Config(2, "qwen3-8b-like-64k", 1, 8, 32, 128, (65536,), 64)
    if index == 3:
        return Config(3, "paged-mix-32seq", 32, 8, 32, 128, _cfg3_lengths(), 16)
    if index == 4:
        return Config(4, "qwen3-8b-like-64k-fp8", 1, 8, 32, 128, (65536,), 64, fmt=fmt if fmt != BF16 else E5M2)
    raise ValueError(index)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def bf16_bits_to_fp8_bits(b: np.ndarray, fmt: int) -> np.ndarray:
    """BF16 values -> OCP FP8 bits (RNE).  E4M3 saturates finite values to +-448 first."""
    x = torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float32)
    if fmt == E4M3:
        fin = torch.isfinite(x)
        x = torch.where(fin, x.clamp(-448.0, 448.0), x)
        y = x.to(torch.float8_e4m3fn)
    elif fmt == E5M2:
        y = x.to(torch.float8_e5m2)
    else:
        raise ValueError(fmt)
    return y.view(torch.uint8).numpy().astype(np.uint16)


class LayerGen:
    """Token stream of one layer.  ``tokens(n)`` continues the same seeded stream."""

    def __init__(self, cfg: Config, layer: int = 0):
        self.cfg = cfg
        self.rng = np.random.default_rng([cfg.index, layer])
        H, D = cfg.Hkv, cfg.D
        self.sK = np.empty((H, D), np.float64)
        self.sV = np.empty((H, D), np.float64)
        for h in range(H):
            s = self.rng.lognormal(0.0, 1.0, D)
            s[self.rng.choice(D, cfg.n_outlier, replace=False)] *= 20.0
            self.sK[h] = s
            self.sV[h] = self.rng.lognormal(0.0, 0.5, D)
        self._sK32 = self.sK.astype(np.float32)
        self._sV32 = self.sV.astype(np.float32)

    def tokens(self, n: int):
        """Next n tokens: (K, V) element bits [n][Hkv][D] (uint16; FP8 bits in the low byte)."""
        H, D = self.cfg.Hkv, self.cfg.D
        k = self.rng.standard_normal((n, H, D), dtype=np.float32) * self._sK32
        v = self.rng.standard_normal((n, H, D), dtype=np.float32) * self._sV32
        kb, vb = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        if self.cfg.fmt != BF16:
            kb, vb = bf16_bits_to_fp8_bits(kb, self.cfg.fmt), bf16_bits_to_fp8_bits(vb, self.cfg.fmt)
        return kb, vb


def rope_keys(k_bits: np.ndarray, theta: float = 1.0e6, first_pos: int = 0) -> np.ndarray:
    """Keys [n][Hkv][D] (BF16 bits) rotated by rotary position embedding at positions
    first_pos .. first_pos + n - 1: channel pair (i, i + D/2) turns by angle pos * theta^(-2i/D)."""
    n, H, D = k_bits.shape
    half = D // 2
    x = bf16_bits_to_f32(k_bits).reshape(n, H, D)
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = (first_pos + np.arange(n, dtype=np.float64))[:, None] * inv[None, :]
    c = np.cos(ang).astype(np.float32)[:, None, :]
    s = np.sin(ang).astype(np.float32)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return f32_to_bf16_bits(np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1))


def sequence_tokens(cfg: Config, layer: int = 0):
    """All context tokens of every sequence of one layer, drawn in sequence order from one
    stream: list of (K, V) [L_s][Hkv][D]."""
    g = LayerGen(cfg, layer)
    return g, [g.tokens(L) for L in cfg.context]


def queries(cfg: Config, step: int = 0) -> np.ndarray:
    """Decode-step queries [n_seqs][Hq][D] as BF16 bits."""
    rng = np.random.default_rng([cfg.index, 7919, step])
    return f32_to_bf16_bits(rng.standard_normal((cfg.n_seqs, cfg.Hq, cfg.D), dtype=np.float32))
