"""Seeded synthetic workloads for chunked GRPO log-probabilities and loss.

The shapes, value distributions and length mixes follow the long-context GRPO
workloads described on the Unsloth pages ("Reinforcement Learning GRPO mit 7x
laengerem Kontext", section on flattened sequence-length chunking: batch and
context flattened into one token stream and cut into chunks).  No dataset,
tokenizer or trained weights are involved: hidden states are N(0, 1), the
lm_head weight is N(0, 0.02^2), target ids are uniform over the vocabulary.

Recipe (identical bits on every machine, independent of thread count):
  * every draw comes from numpy's PCG64 seeded by a SeedSequence of
    ``(seed, stream, block)``: stream 0 holds the small per-sequence and
    per-token draws in a fixed order (lengths, rewards, targets, old-policy
    noise, reference-policy noise), stream 1 the hidden states and stream 2
    the lm_head weight, each in blocks of 4096 rows, one generator per block,
    so blocks can be drawn in parallel threads;
  * bf16 tensors are fp32 draws rounded to nearest-even by bit arithmetic and
    kept as their uint16 bit patterns; fp32 workloads keep the fp32 draws.

The module only draws and rounds numbers.  The old-policy and reference
log-probabilities of a case are built by the caller as ``logp + noise`` from
whatever log-probabilities it has.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 4096

# The five workloads.  ``chunk`` is the number of flattened tokens per chunk.
CONFIGS = {
    0: dict(workload="tiny-fp32 D=64 V=512 1x4x32 tokens", dtype="f32", D=64, V=512,
            G=4, lengths=("fixed", 4, 32), rewards=("bernoulli", 0.5), chunk=32),
    1: dict(workload="qwen2.5-1.5b-shaped D=1536 V=151936 8x8 completions U[256,1024]",
            dtype="bf16", D=1536, V=151936, G=8, lengths=("uniform", 64, 256, 1024),
            rewards=("uniform",), chunk=4096),
    2: dict(workload="llama-3.1-8b-shaped D=4096 V=128256 1x4x5120 tokens", dtype="bf16",
            D=4096, V=128256, G=4, lengths=("fixed", 4, 5120), rewards=("bernoulli", 0.3),
            chunk=2048),
    3: dict(workload="qwen3-8b-shaped D=4096 V=151936 1x2x55000 tokens (110000)",
            dtype="bf16", D=4096, V=151936, G=2, lengths=("fixed", 2, 55000),
            rewards=("bernoulli", 0.5), chunk=8192),
    4: dict(workload="gpt-oss-20b-shaped D=2880 V=201088 4 completions summing to 380000",
            dtype="bf16", D=2880, V=201088, G=4, lengths=("composition", 4, 380000),
            rewards=("bernoulli", 0.5), chunk=8192),
}

OLD_NOISE_STD = 0.01
REF_NOISE_STD = 0.05


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs are finite draws; NaN is not
    special-cased.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += b
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, stream: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, block])))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_matrix(seed: int, stream: int, rows: int, cols: int, scale: float, dtype: str):
    """rows x cols matrix of N(0, scale^2) draws in 4096-row blocks."""
    out = np.empty((rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def fill(b):
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        x = _rng(seed, stream, b).standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[r0:r1] = bf16_bits_from_f32(x) if dtype == "bf16" else x

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _lengths(rng: np.random.Generator, spec) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        return np.full(spec[1], spec[2], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[2], spec[3] + 1, size=spec[1]).astype(np.int64)
    if kind == "composition":
        # n parts >= 1 summing to total: n-1 distinct cut points in [1, total-1]
        n, total = spec[1], spec[2]
        cuts = np.sort(rng.choice(np.arange(1, total), size=n - 1, replace=False))
        return np.diff(np.concatenate([[0], cuts, [total]])).astype(np.int64)
    if kind == "list":
        return np.asarray(spec[1], dtype=np.int64)
    raise ValueError(f"unknown length spec {spec}")


def _rewards(rng: np.random.Generator, spec, S: int) -> np.ndarray:
    kind = spec[0]
    if kind == "bernoulli":
        return (rng.random(S) < spec[1]).astype(np.float32)
    if kind == "uniform":
        return rng.random(S).astype(np.float32)
    if kind == "normal":
        return rng.standard_normal(S).astype(np.float32)
    raise ValueError(f"unknown reward spec {spec}")


@dataclass
class Case:
    """One synthetic workload.  Arrays live on the host."""
    name: str
    dtype: str              # "bf16" (H, W are uint16 bit patterns) or "f32"
    D: int
    V: int
    G: int
    chunk: int
    lengths: np.ndarray     # int64 [S]
    cu: np.ndarray          # int32 [S+1], cu[0] = 0, cu[S] = T
    H: np.ndarray           # [T, D]
    W: np.ndarray           # [V, D]
    targets: np.ndarray     # int32 [T]
    rewards: np.ndarray     # float32 [S]
    mask: np.ndarray        # uint8 [T]
    noise_old: np.ndarray   # float64 [T]
    noise_ref: np.ndarray   # float64 [T]
    params: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.cu[-1])

    @property
    def S(self) -> int:
        return int(self.lengths.shape[0])


def make_case(seed: int, *, D: int, V: int, G: int, lengths, dtype: str = "bf16",
              rewards=("bernoulli", 0.5), chunk: int = 4096, w_std: float = 0.02,
              h_std: float = 1.0, name: str = "custom", with_H: bool = True) -> Case:
    """Draw a workload.  ``lengths`` is a spec tuple or an explicit list of lengths."""
    if not isinstance(lengths, tuple):
        lengths = ("list", list(lengths))
    rng = _rng(seed, 0)
    L = _lengths(rng, lengths)
    S = int(L.shape[0])
    cu = np.zeros(S + 1, dtype=np.int64)
    np.cumsum(L, out=cu[1:])
    T = int(cu[-1])
    r = _rewards(rng, rewards, S)
    targets = rng.integers(0, V, size=T).astype(np.int32)
    n_old = rng.normal(0.0, OLD_NOISE_STD, size=T)
    n_ref = rng.normal(0.0, REF_NOISE_STD, size=T)
    H = _draw_matrix(seed, 1, T, D, h_std, dtype) if with_H else None
    W = _draw_matrix(seed, 2, V, D, w_std, dtype)
    return Case(name=name, dtype=dtype, D=D, V=V, G=G, chunk=chunk, lengths=L,
                cu=cu.astype(np.int32), H=H, W=W, targets=targets, rewards=r,
                mask=np.ones(T, dtype=np.uint8), noise_old=n_old, noise_ref=n_ref,
                params=dict(clip_eps_low=0.2, clip_eps_high=0.2, beta=0.001,
                            temperature=1.0, adv_eps=1e-4))


def make_config(cfg: int, *, with_H: bool = True) -> Case:
    c = CONFIGS[cfg]
    return make_case(1000 + cfg, D=c["D"], V=c["V"], G=c["G"], lengths=c["lengths"],
                     dtype=c["dtype"], rewards=c["rewards"], chunk=c["chunk"],
                     name=c["workload"], with_H=with_H)
