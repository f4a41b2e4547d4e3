"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws random inputs and describes shapes; it holds none of the
quantizer's or the attention's arithmetic, so both the HIP path and the CPU oracle can be
fed from it without sharing any method code.

The shapes mirror the pages' synthetic decode benchmark (B=1, H=32, D=128, b=2, g=32,
S_q=1, S_kv from 512 to 65536; "Changelog", v0.42.0 "Added") and model-shaped batches
(Llama-3-8B-like GQA, Mistral-7B-like 32-layer stack). The pages measure on real model
activations that are not available here; these seeded normal draws with a few x10 outlier
key channels stand in for them.

Draw order for one workload (numpy PCG64, ``default_rng(seed)``):

1. ragged batches only: per-sequence lengths ``rng.integers(lo, hi + 1, size=B)``;
2. the outlier key channels, one set shared by every batch row and head:
   ``rng.choice(D, n_outlier, replace=False)``;
3. for each sequence b in order: ``K_b`` then ``V_b`` as
   ``rng.standard_normal((H_kv, S_b, D), float32)``; the outlier channels of ``K_b`` are
   multiplied by 10 in float32; both are then rounded to float16;
4. ``q = (rng.standard_normal((B, H_q, D), float32) / sqrt(D))`` rounded to float16;
5. tokens for appends continue the same stream: per step ``k`` then ``v`` as
   ``rng.standard_normal((B, H_kv, D), float32)`` (outliers x10 on k), rounded to float16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    key_bits: int
    value_bits: int
    seq_len: int | None  # fixed length, or None for a ragged batch
    ragged: tuple[int, int] | None  # inclusive length range for ragged batches
    n_outlier: int
    seed: int
    group: int = 32
    residual: int = 32
    layers: int = 1

    def describe(self) -> str:
        s = f"S={self.seq_len}" if self.seq_len else f"S~U[{self.ragged[0]},{self.ragged[1]}]"
        lay = f"{self.layers}x " if self.layers > 1 else ""
        return (f"{lay}B={self.batch} Hq={self.n_q_heads} Hkv={self.n_kv_heads} D={self.head_dim} "
                f"{s} bk={self.key_bits} bv={self.value_bits} g={self.group} R={self.residual}")


WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 8, 64, 2, 2, 256, None, 4, 101),
    "short": Workload("short", 1, 32, 32, 128, 2, 2, 512, None, 8, 102),
    "long": Workload("long", 1, 32, 32, 128, 2, 2, 65536, None, 8, 103),
    "gqa": Workload("gqa", 16, 32, 8, 128, 2, 4, None, (1024, 16384), 5, 104),
    "full32": Workload("full32", 8, 32, 8, 128, 2, 2, 32768, None, 8, 105, layers=32),
}


class Draw:
    """The arrays of one workload (one layer), drawn in the documented order."""

    def __init__(self, wl: Workload, layer: int = 0, seq_lens=None, heads=None):
        seed = wl.seed if wl.layers == 1 else [wl.seed, layer]
        self.rng = np.random.default_rng(seed)
        self.wl = wl
        D = wl.head_dim
        if wl.ragged is not None:
            lens = self.rng.integers(wl.ragged[0], wl.ragged[1] + 1, size=wl.batch)
        else:
            lens = np.full(wl.batch, wl.seq_len)
        if seq_lens is not None:  # caller override (small parity cases); the draw order is unchanged
            lens = np.asarray(seq_lens)
        self.seq_lens = [int(x) for x in lens]
        self.outliers = self.rng.choice(D, wl.n_outlier, replace=False)
        self.K, self.V = [], []
        for b in range(wl.batch):
            self.K.append(self._keys((wl.n_kv_heads, self.seq_lens[b], D)))
            self.V.append(self.rng.standard_normal((wl.n_kv_heads, self.seq_lens[b], D), np.float32)
                          .astype(np.float16))
        self.q = (self.rng.standard_normal((wl.batch, wl.n_q_heads, D), np.float32)
                  / np.float32(math.sqrt(D))).astype(np.float16)

    def _keys(self, shape):
        k = self.rng.standard_normal(shape, np.float32)
        k[..., self.outliers] *= np.float32(10.0)
        return k.astype(np.float16)

    def next_token(self):
        """(k, v) for one append step, each float16 [B, H_kv, D]."""
        wl = self.wl
        shape = (wl.batch, wl.n_kv_heads, wl.head_dim)
        k = self._keys(shape)
        v = self.rng.standard_normal(shape, np.float32).astype(np.float16)
        return k, v

    def padded(self):
        """K, V as float16 [B, H_kv, max_S, D] (zero padded) plus the length list."""
        wl = self.wl
        S = max(self.seq_lens)
        K = np.zeros((wl.batch, wl.n_kv_heads, S, wl.head_dim), np.float16)
        V = np.zeros_like(K)
        for b in range(wl.batch):
            K[b, :, : self.seq_lens[b]] = self.K[b]
            V[b, :, : self.seq_lens[b]] = self.V[b]
        return K, V, list(self.seq_lens)


def custom(name="custom", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64, key_bits=2, value_bits=2,
           seq_len=256, n_outlier=2, seed=7, residual=32, ragged=None) -> Workload:
    """A small workload of arbitrary shape for parity cases, with the same draw recipe."""
    return Workload(name, batch, n_q_heads, n_kv_heads, head_dim, key_bits, value_bits,
                    None if ragged else seq_len, ragged, n_outlier, seed, residual=residual)
