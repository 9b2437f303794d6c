"""Seeded synthetic inputs for the GPT-2 training step: initial parameters and token batches.

This module is shared by the HIP path's tests/bench and by the oracle's tests. It holds none
of the model's arithmetic: only a counter-based random generator, the parameter layout sizes
needed to place the draws, and the recipe that turns draws into fp32 parameters and int32
tokens.

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) used as a counter-based hash, ``x_i = mix(seed + (i+1)*golden)``.
It is chosen over the xorshift* generator of the llm.c pages (llm.c annotated, section 1.33
random_u32) because a counter-based stream vectorises in numpy, so a 774M-parameter init
takes seconds rather than hours. Normal draws use the Box-Muller transform (Box & Muller,
1958) on pairs of uniforms.

Recipe (no initialisation is given on the pages; they load a checkpoint, llm.c annotated
section 1.22):
- every weight matrix and both embeddings ~ N(0, 0.02), rounded to fp32;
- all linear and LayerNorm biases are 0, LayerNorm gains are 1;
- when ``scale_residual`` is set, the two residual projections (attprojw, fcprojw) use
  std 0.02/sqrt(2L);
- tokens are uniform in [0, V); in "stream" mode one stream of B*T+1 tokens gives
  inputs = s[0:BT] and targets = s[1:BT+1] (the DataLoader's shift by one, llm.c annotated
  section 1.29); in "independent" mode targets are a second independent draw.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# order and names of the 16 parameter tensors (llm.c annotated, section 1.16 ParameterTensors)
PARAM_NAMES = ("wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
               "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb")


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream for ``seed`` (uint64)."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    """float64 uniforms in [0, 1) from the top 53 bits of each draw."""
    z = splitmix64(seed, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(seed: int, start: int, count: int) -> np.ndarray:
    """float64 N(0,1) draws; element i uses uniforms 2i and 2i+1 of the stream (Box-Muller)."""
    u = uniform01(seed, 2 * start, 2 * count)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))  # 1-u1 is in (0, 1]
    return r * np.cos(2.0 * math.pi * u2)


_BIASES = ("ln1b", "qkvb", "attprojb", "ln2b", "fcb", "fcprojb", "lnfb")


def param_sizes(L: int, C: int, V: int, maxT: int) -> list[int]:
    """Element counts of the 16 tensors, in flat order (llm.c annotated, section 1.22)."""
    return [V * C, maxT * C, L * C, L * C, L * 3 * C * C, L * 3 * C, L * C * C, L * C,
            L * C, L * C, L * 4 * C * C, L * 4 * C, L * C * 4 * C, L * C, C, C]


@dataclass(frozen=True)
class ModelShape:
    L: int
    C: int
    H: int
    V: int
    maxT: int


def init_params(shape: ModelShape, seed: int, scale_residual: bool,
                std: float = 0.02, chunk: int = 1 << 24) -> np.ndarray:
    """Flat fp32 parameter vector in the 16-tensor order.

    The normal draw for flat element ``i`` is stream element ``i`` regardless of the tensor
    it lands in, so any slice can be regenerated on its own.
    """
    sizes = param_sizes(shape.L, shape.C, shape.V, shape.maxT)
    out = np.empty(sum(sizes), dtype=np.float32)
    resid_std = std / math.sqrt(2.0 * shape.L) if scale_residual else std
    jobs = []  # (first flat element, count, std) of each chunk of normal draws
    off = 0
    for name, n in zip(PARAM_NAMES, sizes):
        if name in ("ln1w", "ln2w", "lnfw"):
            out[off:off + n] = 1.0
        elif name in _BIASES:
            out[off:off + n] = 0.0
        else:
            s = resid_std if name in ("attprojw", "fcprojw") else std
            jobs += [(off + c0, min(chunk, n - c0), s) for c0 in range(0, n, chunk)]
        off += n

    def fill(job):
        start, count, s = job
        out[start:start + count] = (normal(seed, start, count) * s).astype(np.float32)

    # chunks are independent slices of the counter-based stream; numpy releases the GIL
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, jobs))
    return out


def tokens_uniform(seed: int, start: int, count: int, V: int) -> np.ndarray:
    """int32 tokens uniform in [0, V) (multiply-shift of the high 32 bits)."""
    z = splitmix64(seed, start, count)
    hi = (z >> np.uint64(32)).astype(np.uint64)
    with np.errstate(over="ignore"):
        return ((hi * np.uint64(V)) >> np.uint64(32)).astype(np.int32)


_ZIPF_CDF: dict = {}


def tokens_zipf(seed: int, start: int, count: int, V: int, exponent: float = 1.0) -> np.ndarray:
    """int32 tokens in [0, V) with P(k) proportional to 1/(k+1)^exponent (Zipf's law, the
    rank-frequency shape of word and sub-word counts in text; token k is the k-th most
    frequent), by inverting the cumulative distribution at the stream's uniforms."""
    key = (V, exponent)
    if key not in _ZIPF_CDF:
        w = 1.0 / np.arange(1, V + 1, dtype=np.float64) ** exponent
        cdf = np.cumsum(w)
        _ZIPF_CDF[key] = cdf / cdf[-1]
    u = uniform01(seed, start, count)
    return np.minimum(np.searchsorted(_ZIPF_CDF[key], u, side="right"), V - 1).astype(np.int32)


def batch(seed: int, B: int, T: int, V: int, step: int = 0,
          mode: str = "stream") -> tuple[np.ndarray, np.ndarray]:
    """(inputs, targets), each int32 (B, T).

    mode "stream": the token stream advances by B*T per step and targets are the inputs
    shifted by one; mode "independent": inputs and targets are separate uniform draws;
    mode "zipf": as "stream" with Zipf-distributed tokens (exponent 1) in place of uniform
    ones, the skew of real text (many repeats of the frequent tokens in every batch).
    """
    n = B * T
    if mode == "stream":
        s = tokens_uniform(seed, step * n, n + 1, V)
        return s[:n].reshape(B, T).copy(), s[1:].reshape(B, T).copy()
    if mode == "zipf":
        s = tokens_zipf(seed, step * n, n + 1, V)
        return s[:n].reshape(B, T).copy(), s[1:].reshape(B, T).copy()
    if mode == "independent":
        s = tokens_uniform(seed, step * 2 * n, 2 * n, V)
        return s[:n].reshape(B, T).copy(), s[n:].reshape(B, T).copy()
    raise ValueError(f"unknown token mode {mode!r}")


@dataclass(frozen=True)
class Workload:
    """One named training-step workload: model shape, batch, dtype and input recipe."""
    name: str
    shape: ModelShape
    B: int
    T: int
    dtype: str          # "fp32", "bf16" or "fp16"
    scale_residual: bool
    token_mode: str
    seed: int
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


# The workloads: a tiny model, GPT-2 124M at two batch sizes (and on Zipf-distributed tokens),
# 350M, and 774M in bf16 and in fp16.
WORKLOADS = {
    "tiny": Workload("tiny L1 C16 H4 V27 B4 T16 fp32", ModelShape(1, 16, 4, 27, 16), 4, 16,
                     "fp32", False, "independent", seed=1337),
    "gpt2_124m_b4_t64": Workload("gpt2-124M B4 T64 fp32", ModelShape(12, 768, 12, 50257, 1024),
                                 4, 64, "fp32", True, "stream", seed=1338),
    "gpt2_124m_b16_t1024": Workload("gpt2-124M B16 T1024 fp32",
                                    ModelShape(12, 768, 12, 50257, 1024), 16, 1024, "fp32",
                                    True, "stream", seed=1339),
    # the same step on Zipf-distributed tokens (the token skew of real text)
    "gpt2_124m_b16_t1024_zipf": Workload("gpt2-124M B16 T1024 fp32, Zipf tokens",
                                         ModelShape(12, 768, 12, 50257, 1024), 16, 1024, "fp32",
                                         True, "zipf", seed=1339),
    "gpt2_350m_b8_t1024": Workload("gpt2-350M B8 T1024 fp32",
                                   ModelShape(24, 1024, 16, 50257, 1024), 8, 1024, "fp32",
                                   True, "stream", seed=1340),
    "gpt2_774m_b8_t1024_bf16": Workload("gpt2-774M B8 T1024 bf16",
                                        ModelShape(36, 1280, 20, 50257, 1024), 8, 1024,
                                        "bf16", True, "stream", seed=1341),
    # the same shape and inputs in fp16 with loss scaling (the pages' "fp16 or lower")
    "gpt2_774m_b8_t1024_fp16": Workload("gpt2-774M B8 T1024 fp16",
                                        ModelShape(36, 1280, 20, 50257, 1024), 8, 1024,
                                        "fp16", True, "stream", seed=1341),
}
