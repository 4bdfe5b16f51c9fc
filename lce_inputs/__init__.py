"""Seeded synthetic inputs for the chunked linear-cross-entropy workloads.

This module holds no loss arithmetic. It only draws random numbers, rounds
the drawn float32 values to bfloat16 (round-to-nearest-even on the bit
pattern), and lists the workload shapes. The oracle's tests, the GPU parity
tests and the benchmark all take their inputs from here, so both sides see
the same bits.

Workload recipe (shapes follow the Qwen3 heads the pages train: Qwen3-0.6B
with a 2048-token cutoff in the LlamaFactory chunk-loss yaml example, Qwen3-4B
at 32k and 160k tokens in the TRL long-context guide's "chunking" section,
and Qwen3-8B at one GPU's eighth of a 1M-token sequence in that guide's
"run" section):

* one ``numpy.random.Generator(PCG64(seed))``; draw order hidden, weight,
  bias, labels, ignore mask;
* hidden ``standard_normal((N, H), float32)``; for the "rms" workloads each
  row is divided by ``sqrt(mean(x**2) + 1e-6)`` (computed in float64);
* weight ``weight_std * standard_normal((V, H))``; bias, when present,
  ``bias_std * standard_normal(V)``;
* labels uniform on ``[0, V)`` or Zipf(s) over ranks ``1..V`` (finite
  support, inverse CDF by ``searchsorted``), label = rank - 1;
* ignore rows set to ``IGNORE_INDEX``: exactly ``floor(p*N)`` rows picked by
  ``permutation(N)`` ("random"), the first ``floor(p*N)`` rows ("prefix",
  a masked prompt), or none.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace

import numpy as np

# The ignore label of the pages' per-token cross-entropy (LlamaFactory's
# IGNORE_INDEX constant, -100).
IGNORE_INDEX = -100


@dataclass(frozen=True)
class Workload:
    name: str
    n_rows: int
    hidden: int
    vocab: int
    hidden_dist: str = "normal"      # "normal" | "rms"
    weight_std: float = 0.02
    bias_std: float | None = None
    labels: str = "uniform"          # "uniform" | "zipf"
    zipf_s: float = 1.1
    ignore: str = "random"           # "random" | "prefix" | "none"
    ignore_frac: float = 0.0
    chunk_rows: int = 256
    reduction: str = "sum"
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def n_ignored(self) -> int:
        if self.ignore == "none":
            return 0
        return int(math.floor(self.ignore_frac * self.n_rows))


WORKLOADS: dict[str, Workload] = {
    "tiny": Workload("tiny", 512, 256, 4096, ignore="random", ignore_frac=0.10),
    "qwen3_0p6b_head": Workload("qwen3_0p6b_head", 2048, 1024, 151936,
                                ignore="prefix", ignore_frac=0.30),
    "qwen3_4b_32k": Workload("qwen3_4b_32k", 32768, 2560, 151936, hidden_dist="rms",
                             labels="zipf", ignore="random", ignore_frac=0.05),
    "qwen3_4b_160k": Workload("qwen3_4b_160k", 163840, 2560, 151936, hidden_dist="rms",
                              labels="zipf", ignore="none"),
    "qwen3_8b_1m_shard": Workload("qwen3_8b_1m_shard", 131072, 4096, 151936,
                                  bias_std=0.01, labels="zipf", ignore="random",
                                  ignore_frac=0.02),
}
WORKLOAD_ORDER = ["tiny", "qwen3_0p6b_head", "qwen3_4b_32k", "qwen3_4b_160k",
                  "qwen3_8b_1m_shard"]


def bf16_bits_reference(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even,
    on the bit pattern: add 0x7FFF plus the lowest kept bit, drop 16 bits.
    Inputs here are finite draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Same rounding as bf16_bits_reference, through torch's vectorised
    float32 -> bfloat16 conversion (round to nearest even) when available."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        return bf16_bits_reference(x)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exactly equal float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    workload: Workload
    hidden_bits: np.ndarray          # uint16 [N, H]
    weight_bits: np.ndarray          # uint16 [V, H]
    bias_bits: np.ndarray | None     # uint16 [V]
    labels: np.ndarray               # int64 [N]

    def hidden_f32(self) -> np.ndarray:
        return bits_to_f32(self.hidden_bits)

    def weight_f32(self) -> np.ndarray:
        return bits_to_f32(self.weight_bits)

    def bias_f32(self) -> np.ndarray | None:
        return None if self.bias_bits is None else bits_to_f32(self.bias_bits)

    def digest(self) -> str:
        """sha256 over all input bits: pins stored expected values to these inputs."""
        h = hashlib.sha256()
        for a in (self.hidden_bits, self.weight_bits, self.bias_bits, self.labels):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def _normal_bits(gen: np.random.Generator, shape, scale: float, rms: bool = False,
                 block_rows: int = 8192) -> np.ndarray:
    """Draw standard normals row block by row block (same stream as one big
    draw would give, since rows are drawn in order) and round to bf16."""
    n, h = shape
    out = np.empty((n, h), dtype=np.uint16)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        x = gen.standard_normal((r1 - r0, h), dtype=np.float32)
        if rms:
            x64 = x.astype(np.float64)
            x = (x64 / np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True) + 1e-6)).astype(np.float32)
        elif scale != 1.0:
            x = x * np.float32(scale)
        out[r0:r1] = bf16_bits(x)
    return out


def zipf_cdf(vocab: int, s: float) -> np.ndarray:
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    return cdf / cdf[-1]


def make_inputs(w: Workload) -> Inputs:
    gen = np.random.Generator(np.random.PCG64(w.seed))
    hidden = _normal_bits(gen, (w.n_rows, w.hidden), 1.0, rms=(w.hidden_dist == "rms"))
    weight = _normal_bits(gen, (w.vocab, w.hidden), w.weight_std)
    bias = None
    if w.bias_std is not None:
        bias = bf16_bits(np.float32(w.bias_std) * gen.standard_normal(w.vocab, dtype=np.float32))
    if w.labels == "uniform":
        labels = gen.integers(0, w.vocab, w.n_rows, dtype=np.int64)
    elif w.labels == "zipf":
        u = gen.random(w.n_rows)
        labels = np.minimum(np.searchsorted(zipf_cdf(w.vocab, w.zipf_s), u, side="right"),
                            w.vocab - 1).astype(np.int64)
    else:
        raise ValueError(f"unknown label distribution {w.labels!r}")
    k = w.n_ignored
    if w.ignore == "random" and k > 0:
        labels[gen.permutation(w.n_rows)[:k]] = IGNORE_INDEX
    elif w.ignore == "prefix" and k > 0:
        labels[:k] = IGNORE_INDEX
    elif w.ignore not in ("random", "prefix", "none"):
        raise ValueError(f"unknown ignore mode {w.ignore!r}")
    return Inputs(w, hidden, weight, bias, labels)


def make_case(n_rows: int, hidden: int, vocab: int, *, seed: int = 0, bias_std: float | None = None,
              labels: str = "uniform", ignore: str = "random", ignore_frac: float = 0.1,
              hidden_dist: str = "normal", weight_std: float = 0.02, chunk_rows: int = 256,
              reduction: str = "sum") -> Inputs:
    """A small ad-hoc workload with the same recipe (tests use many shapes)."""
    w = Workload(f"case_{n_rows}x{hidden}x{vocab}_s{seed}", n_rows, hidden, vocab,
                 hidden_dist=hidden_dist, weight_std=weight_std, bias_std=bias_std,
                 labels=labels, ignore=ignore, ignore_frac=ignore_frac,
                 chunk_rows=chunk_rows, reduction=reduction, seed=seed)
    return make_inputs(w)


def sample_rows(w: Workload, labels: np.ndarray, count: int = 256, seed: int = 1) -> np.ndarray:
    """Seeded row subset for full-size checks: random rows, the first and last
    rows of the first, middle and last chunk, ignored rows and rows whose
    label is the most frequent id."""
    gen = np.random.Generator(np.random.PCG64(seed))
    n, c = w.n_rows, w.chunk_rows
    t = (n + c - 1) // c
    picks = list(gen.choice(n, size=min(count, n), replace=False))
    for k in (0, t // 2, t - 1):
        picks += [k * c, min(n, (k + 1) * c) - 1]
    ign = np.flatnonzero(labels == IGNORE_INDEX)
    if ign.size:
        picks += list(ign[:8])
    valid = labels[labels != IGNORE_INDEX]
    if valid.size:
        hot = np.bincount(valid, minlength=w.vocab).argmax()
        picks += list(np.flatnonzero(labels == hot)[:8])
    return np.unique(np.asarray(picks, dtype=np.int64))


def sample_cols(w: Workload, labels: np.ndarray, count: int = 256, seed: int = 2) -> np.ndarray:
    """Seeded vocabulary subset: random ids, the 10 most frequent labels and
    the last 128 ids (the ragged end of the vocabulary)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    v = w.vocab
    picks = list(gen.choice(v, size=min(count, v), replace=False))
    valid = labels[labels != IGNORE_INDEX]
    if valid.size:
        picks += list(np.argsort(-np.bincount(valid, minlength=v), kind="stable")[:10])
    picks += list(range(max(0, v - 128), v))
    return np.unique(np.asarray(picks, dtype=np.int64))
