"""Seeded synthetic inputs for the SharQ linear-layer hot path.

This module is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It holds none of the method's arithmetic: it only
draws random activations, RMSNorm weights, linear weights and MoE routings with
the shapes of the models the SharQ pages evaluate (Llama-3.1-8B, Qwen2.5-7B,
Qwen3-30B-A3B layer shapes), and rounds them to the storage type (bf16 or fp32).

Draw order (numpy ``default_rng(seed)``, PCG64; every draw is float32 unless
stated):

* activation ``X`` (T x K): standard normal; then a fixed set of
  ``max(1, round(frac_ch * K))`` channels (drawn without replacement) is scaled
  by ``U(lo, hi)`` (one factor per channel, same for every token); then, per
  token, ``max(1, round(frac_tok * K))`` positions (drawn without replacement
  through random keys) are scaled by ``tok_mult``.  Overlaps multiply.
  The result is rounded to the storage dtype (bf16: round-to-nearest-even).
* ``gamma`` (K): ``U(0.5, 1.5)`` (or all ones).
* ``W`` (K x D): normal with std 0.02, rounded to the storage dtype.

The synthetic inputs stand in for the pages' models and datasets, which are not
available: only the layer shapes are taken from them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "ActSpec", "LinearCase", "MoECase",
    "tiny_case", "decode_cases", "prefill_case", "nvfp4_cases", "moe_case",
    "draw_activation", "draw_weight", "draw_gamma", "draw_routing",
]


# ----------------------------------------------------------------------------
# storage-type rounding (input representation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class ActSpec:
    """Outlier model of an activation tensor."""
    frac_ch: float = 0.005      # share of fixed outlier channels
    ch_lo: float = 30.0         # channel multiplier ~ U(ch_lo, ch_hi)
    ch_hi: float = 100.0
    frac_tok: float = 0.001     # share of random per-token positions
    tok_mult: float = 20.0
    fixed_cols: tuple = ()      # explicit outlier columns (tiny case)
    fixed_mult: float = 1.0


LLAMA_OUTLIERS = ActSpec()
QWEN_OUTLIERS = ActSpec(frac_ch=0.01, ch_lo=20.0, ch_hi=200.0)


def _count(frac: float, K: int) -> int:
    return max(1, int(round(frac * K)))


def draw_activation(rng: np.random.Generator, T: int, K: int, spec: ActSpec) -> np.ndarray:
    """float32 activation before storage rounding (see module docstring)."""
    X = rng.standard_normal((T, K), dtype=np.float32)
    if spec.fixed_cols:
        X[:, list(spec.fixed_cols)] *= np.float32(spec.fixed_mult)
        return X
    n_ch = _count(spec.frac_ch, K)
    ch = rng.choice(K, size=n_ch, replace=False)
    mult = rng.uniform(spec.ch_lo, spec.ch_hi, size=n_ch).astype(np.float32)
    X[:, ch] *= mult[None, :]
    n_tok = _count(spec.frac_tok, K)
    keys = rng.random((T, K), dtype=np.float32)
    pos = np.argpartition(keys, n_tok - 1, axis=1)[:, :n_tok]
    rows = np.repeat(np.arange(T), n_tok)
    X[rows, pos.reshape(-1)] *= np.float32(spec.tok_mult)
    return X


def draw_gamma(rng: np.random.Generator, K: int, ones: bool = False) -> np.ndarray:
    if ones:
        return np.ones(K, dtype=np.float32)
    return rng.uniform(0.5, 1.5, size=K).astype(np.float32)


def draw_weight(rng: np.random.Generator, K: int, D: int) -> np.ndarray:
    """float32 weight K x D, N(0, 0.02^2), before storage rounding."""
    W = rng.standard_normal((K, D), dtype=np.float32)
    W *= np.float32(0.02)
    return W


def draw_routing(rng: np.random.Generator, n_tokens: int, n_experts: int, top_k: int):
    """Each token picks ``top_k`` distinct experts uniformly at random.  Routed
    rows are sorted by (expert, token).  Returns ``(group_offsets, row_index)``:
    rows ``group_offsets[e]:group_offsets[e+1]`` belong to expert ``e`` and row
    ``r`` reads token ``row_index[r]``."""
    keys = rng.random((n_tokens, n_experts))
    experts = np.argpartition(keys, top_k - 1, axis=1)[:, :top_k]          # (tokens, top_k)
    tok = np.repeat(np.arange(n_tokens), top_k)
    exp = experts.reshape(-1)
    order = np.lexsort((tok, exp))
    row_index = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=n_experts)
    group_offsets = np.zeros(n_experts + 1, dtype=np.int32)
    group_offsets[1:] = np.cumsum(counts)
    return group_offsets, row_index


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------
@dataclass
class LinearCase:
    """One SharQ linear: X (T x K) -> Y (T x D).  ``x`` and ``w`` hold storage
    patterns: float32 arrays when ``dtype == 'f32'``, uint16 bf16 patterns when
    ``dtype == 'bf16'``."""
    name: str
    fmt: str                    # "mxfp4" | "nvfp4"
    dtype: str                  # "f32" | "bf16"
    T: int
    K: int
    D: int
    x: np.ndarray
    gamma: Optional[np.ndarray]
    w: np.ndarray
    eps: float = 1e-6

    def x_f32(self) -> np.ndarray:
        return self.x if self.dtype == "f32" else bf16_bits_to_f32(self.x)

    def w_f32(self) -> np.ndarray:
        return self.w if self.dtype == "f32" else bf16_bits_to_f32(self.w)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32) if dtype == "f32" else f32_to_bf16_bits(a)


def tiny_case(seed: int = 0) -> LinearCase:
    """Tiny MXFP4 linear: T=16, K=256, D=256, fp32; X ~ N(0,1) with channels 7
    and 130 scaled by 40; gamma = 1; W ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    X = draw_activation(rng, 16, 256, ActSpec(fixed_cols=(7, 130), fixed_mult=40.0))
    W = draw_weight(rng, 256, 256)
    return LinearCase("tiny", "mxfp4", "f32", 16, 256, 256, X, np.ones(256, np.float32), W)


def _llama_like(name, fmt, T, K, D, spec, seed) -> LinearCase:
    rng = np.random.default_rng(seed)
    X = draw_activation(rng, T, K, spec)
    g = draw_gamma(rng, K)
    W = draw_weight(rng, K, D)
    return LinearCase(name, fmt, "bf16", T, K, D, _store(X, "bf16"), g, _store(W, "bf16"))


DECODE_SHAPES = ((4096, 4096), (4096, 14336), (14336, 4096))


def decode_case(i: int, seed: int = 0, T: int = 8) -> LinearCase:
    """Llama-3.1-8B decode linear number i of DECODE_SHAPES (T=8), MXFP4, bf16."""
    K, D = DECODE_SHAPES[i]
    return _llama_like(f"decode_{K}x{D}", "mxfp4", T, K, D, LLAMA_OUTLIERS, seed)


def decode_cases(seed: int = 0, T: int = 8):
    """All three Llama-3.1-8B decode linears (T=8), MXFP4, bf16 storage."""
    return [decode_case(i, seed, T) for i in range(len(DECODE_SHAPES))]


def prefill_case(seed: int = 0, T: int = 4096, K: int = 4096, D: int = 14336) -> LinearCase:
    """Llama-3.1-8B prefill linear 4096 x 4096 x 14336, MXFP4, bf16 storage."""
    return _llama_like(f"prefill_{T}x{K}x{D}", "mxfp4", T, K, D, LLAMA_OUTLIERS, seed)


NVFP4_SHAPES = ((3584, 18944), (18944, 3584))


def nvfp4_cases(seed: int = 0, T: int = 2048, shapes=NVFP4_SHAPES):
    """Qwen2.5-7B linears (T=2048), emulated NVFP4, 1% outlier channels x U(20,200)."""
    return [_llama_like(f"nvfp4_{T}x{K}x{D}", "nvfp4", T, K, D, QWEN_OUTLIERS, seed)
            for K, D in shapes]


@dataclass
class MoECase:
    """Grouped (MoE) SharQ linear.  ``x`` holds the activation rows fed to the
    prepare step (``n_rows`` x K); routed row ``r`` of expert ``e`` reads
    activation row ``row_index[r]`` (``row_index is None``: row r itself)."""
    name: str
    n_experts: int
    K: int
    D: int
    x: np.ndarray               # bf16 patterns (n_rows x K)
    gamma: np.ndarray
    w: np.ndarray               # bf16 patterns (E x K x D)
    group_offsets: np.ndarray   # int32 (E+1)
    row_index: Optional[np.ndarray]
    eps: float = 1e-6
    fmt: str = "mxfp4"
    dtype: str = "bf16"

    @property
    def total_rows(self) -> int:
        return int(self.group_offsets[-1])

    def x_f32(self):
        return bf16_bits_to_f32(self.x)

    def w_f32(self):
        return bf16_bits_to_f32(self.w)


def moe_case(proj: str, seed: int = 0, n_tokens: int = 4096, n_experts: int = 128,
             top_k: int = 8, hidden: int = 2048, inter: int = 768) -> MoECase:
    """Qwen3-30B-A3B-shaped expert linears.  ``proj == 'up'``: K=hidden,
    D=inter, the token activations are prepared once and gathered per expert;
    ``proj == 'down'``: K=inter, D=hidden over n_tokens*top_k expert-sorted rows
    drawn independently.  Both use the Llama outlier model."""
    rng = np.random.default_rng(seed)
    group_offsets, row_index = draw_routing(rng, n_tokens, n_experts, top_k)
    if proj == "up":
        K, D, n_rows = hidden, inter, n_tokens
    elif proj == "down":
        K, D, n_rows = inter, hidden, n_tokens * top_k
    else:
        raise ValueError(proj)
    X = draw_activation(rng, n_rows, K, LLAMA_OUTLIERS)
    g = draw_gamma(rng, K)
    W = np.empty((n_experts, K, D), dtype=np.uint16)
    for e in range(n_experts):
        W[e] = f32_to_bf16_bits(draw_weight(rng, K, D))
    return MoECase(f"moe_{proj}_{n_experts}x{K}x{D}", n_experts, K, D, f32_to_bf16_bits(X), g, W,
                   group_offsets, row_index if proj == "up" else None)


def random_case(seed: int, T: int, K: int, D: int, fmt: str = "mxfp4", dtype: str = "bf16",
                spec: ActSpec = LLAMA_OUTLIERS, gamma: bool = True) -> LinearCase:
    """Small parity case of arbitrary shape with the Llama outlier model."""
    rng = np.random.default_rng(seed)
    X = draw_activation(rng, T, K, spec)
    g = draw_gamma(rng, K) if gamma else None
    W = draw_weight(rng, K, D)
    return LinearCase(f"rand_{fmt}_{T}x{K}x{D}", fmt, dtype, T, K, D, _store(X, dtype), g, _store(W, dtype))
