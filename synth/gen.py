"""Seeded generators for the five MoE-FFN workloads and for small test shapes.

Every tensor comes from its own NumPy ``Generator(PCG64(SeedSequence([seed, tag,
layer, expert, matrix])))`` stream, so any expert of any layer can be regenerated
on its own (the oracle does that for the few experts a sampled token touches).

Distributions (the Hy4 layer shape is the Hy4-preview Flash-MoE STQ1_0 package
table: hidden 6144, MoE intermediate 2048, 256 routed experts, 8 selected, one
shared expert):

* activations: bf16 round-to-nearest-even of fp32 N(0, 1);
* router and shared-expert weights: bf16 of fp32 N(0, 0.02);
* STQ1_0 expert matrices: every group of four weights independently takes one of
  the 32 (zero lane, three signs) patterns with equal probability.  In the packed
  layout each group's 5-bit pattern number is spread over a 4-bit nibble and one
  high bit, and all 32 values are valid patterns, so uniform random code bytes are
  exactly uniform patterns.  The per-256-weight scale is the fp16 (round to nearest
  even) of |N(0, 0.02)|;
* MXFP4 expert matrices: every 4-bit E2M1 code uniform over its 16 values (so two
  codes per byte make a uniform byte), every group-32 UE8M0 scale byte uniform over
  127 + {-8, ..., -4};
* skewed routing: a Zipf(s = 1.1) prior over a seeded ranking of the experts,
  added to the router logits as ``-s * ln(rank)``;
* prefill logits: i.i.d. fp32 N(0, 1).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "LayerCfg", "CONFIGS", "cfg", "rng", "f32_to_bf16_bits", "bf16_normal",
    "fp16_abs_normal", "stq1_codes_bytes", "stq1_matrix", "stq1_family",
    "stq1_pattern_fields", "mxfp4_matrix", "mxfp4_family", "zipf_bias",
    "prefill_logits", "activations", "router_weights", "shared_weights",
    "sample_tokens", "mxfp8_matrix", "shared_weights_mxfp8",
    "STQ_BLOCK", "STQ_CODE_BYTES", "MAT_GATE", "MAT_UP", "MAT_DOWN",
]

STQ_BLOCK = 256          # weights per STQ1_0 block
STQ_CODE_BYTES = 40      # pattern bytes per block (scale stored separately)
MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2

# stream tags
_T_X, _T_ROUTER, _T_RANK, _T_LOGITS = 1, 2, 3, 4
_T_STQ_CODES, _T_STQ_SCALES, _T_STQ_Z, _T_STQ_S = 10, 11, 12, 13
_T_MX_CODES, _T_MX_SCALES = 20, 21
_T_SHARED, _T_SAMPLE = 30, 40
_T_SH8_CODES, _T_SH8_SCALES = 31, 32


@dataclass(frozen=True)
class LayerCfg:
    name: str
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    k: int            # experts per token
    shared: bool      # one bf16 shared expert
    fmt: str          # "stq1" or "mxfp4"
    zipf: bool        # Zipf(1.1) logit bias
    logits_given: bool  # router logits drawn directly (no router GEMV)
    layers: int
    seed: int


CONFIGS = {
    0: LayerCfg("tiny-stq1-h256-i128-e8-top2-t4", 4, 256, 128, 8, 2, False, "stq1",
                False, False, 1, 0),
    1: LayerCfg("hy4-stq1-decode-t1", 1, 6144, 2048, 256, 8, True, "stq1",
                False, False, 1, 1),
    2: LayerCfg("hy4-stq1-decode-t64-zipf", 64, 6144, 2048, 256, 8, True, "stq1",
                True, False, 1, 2),
    3: LayerCfg("hy4-mxfp4-prefill-t4096", 4096, 6144, 2048, 256, 8, True, "mxfp4",
                False, True, 1, 3),
    4: LayerCfg("hy4-stq1-stack29-t16-zipf", 16, 6144, 2048, 256, 8, True, "stq1",
                True, False, 29, 7),
}


def cfg(i: int) -> LayerCfg:
    return CONFIGS[i]


def rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, tags)])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of finite fp32 values, round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_normal(seed: int, tags: tuple, shape, std: float) -> np.ndarray:
    g = rng(seed, *tags)
    v = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v).reshape(shape)


def fp16_abs_normal(g: np.random.Generator, n: int, std: float) -> np.ndarray:
    """fp16 bit patterns (round to nearest even from fp64) of |N(0, std)|."""
    v = np.abs(g.standard_normal(n)) * std
    return v.astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------- STQ1_0
def stq1_codes_bytes(n_weights: int) -> int:
    assert n_weights % STQ_BLOCK == 0
    return n_weights // STQ_BLOCK * STQ_CODE_BYTES


def stq1_matrix(seed: int, layer: int, expert: int, mat: int, n_weights: int,
                out_codes: np.ndarray | None = None, out_scales: np.ndarray | None = None):
    """Pattern bytes [n_blk*40] (uniform) and fp16 scale bits [n_blk] of one matrix."""
    n_blk = n_weights // STQ_BLOCK
    assert n_blk * STQ_BLOCK == n_weights
    gc = rng(seed, _T_STQ_CODES, layer, expert, mat)
    codes = gc.integers(0, 256, n_blk * STQ_CODE_BYTES, dtype=np.uint8)
    gs = rng(seed, _T_STQ_SCALES, layer, expert, mat)
    scales = fp16_abs_normal(gs, n_blk, 0.02)
    if out_codes is not None:
        out_codes[...] = codes
        out_scales[...] = scales
        return out_codes, out_scales
    return codes, scales


def stq1_family(seed: int, layer: int, mat: int, E: int, n_weights: int, experts=None):
    """Expert-major codes [E, n_blk*40] and scales [E, n_blk] of one weight family."""
    n_blk = n_weights // STQ_BLOCK
    codes = np.empty((E, n_blk * STQ_CODE_BYTES), dtype=np.uint8)
    scales = np.empty((E, n_blk), dtype=np.uint16)
    todo = range(E) if experts is None else experts
    if experts is not None:
        codes[...] = 0
        scales[...] = 0
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda e: stq1_matrix(seed, layer, e, mat, n_weights, codes[e], scales[e]), todo))
    return codes, scales


def stq1_pattern_fields(seed: int, layer: int, expert: int, mat: int, n_groups: int):
    """Independent (zero lane in 0..3, three sign bits in 0..7) per group, for the
    packing parity checks."""
    z = rng(seed, _T_STQ_Z, layer, expert, mat).integers(0, 4, n_groups, dtype=np.uint8)
    s = rng(seed, _T_STQ_S, layer, expert, mat).integers(0, 8, n_groups, dtype=np.uint8)
    d = fp16_abs_normal(rng(seed, _T_STQ_SCALES, layer, expert, mat), n_groups // 64, 0.02)
    return z, s, d


# ----------------------------------------------------------------------------- MXFP4
def mxfp4_matrix(seed: int, layer: int, expert: int, mat: int, N: int, K: int,
                 out_codes: np.ndarray | None = None, out_scales: np.ndarray | None = None):
    """E2M1 code bytes [N, K/2] (uniform) and UE8M0 scale bytes [N, K/32] in 119..123."""
    assert K % 32 == 0
    codes = rng(seed, _T_MX_CODES, layer, expert, mat).integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = (127 + rng(seed, _T_MX_SCALES, layer, expert, mat).integers(
        -8, -3, (N, K // 32), dtype=np.int16)).astype(np.uint8)
    if out_codes is not None:
        out_codes[...] = codes
        out_scales[...] = scales
        return out_codes, out_scales
    return codes, scales


def mxfp4_family(seed: int, layer: int, mat: int, E: int, N: int, K: int):
    codes = np.empty((E, N, K // 2), dtype=np.uint8)
    scales = np.empty((E, N, K // 32), dtype=np.uint8)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda e: mxfp4_matrix(seed, layer, e, mat, N, K, codes[e], scales[e]), range(E)))
    return codes, scales


# ----------------------------------------------------------------------------- routing inputs
def zipf_bias(seed: int, layer: int, E: int, s: float = 1.1) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank), rank = 1 + a seeded permutation of 0..E-1."""
    rank = 1 + rng(seed, _T_RANK, layer).permutation(E)
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def prefill_logits(seed: int, layer: int, T: int, E: int) -> np.ndarray:
    return rng(seed, _T_LOGITS, layer).standard_normal((T, E), dtype=np.float32)


def activations(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    return bf16_normal(seed, (_T_X, layer), (T, H), 1.0)


def router_weights(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    return bf16_normal(seed, (_T_ROUTER, layer), (E, H), 0.02)


def shared_weights(seed: int, layer: int, I: int, H: int):
    """bf16 gate [I, H], up [I, H], down [H, I] of the shared expert."""
    return (bf16_normal(seed, (_T_SHARED, layer, MAT_GATE), (I, H), 0.02),
            bf16_normal(seed, (_T_SHARED, layer, MAT_UP), (I, H), 0.02),
            bf16_normal(seed, (_T_SHARED, layer, MAT_DOWN), (H, I), 0.02))


def mxfp8_matrix(seed: int, layer: int, mat: int, N: int, K: int):
    """MXFP8 weights of the shared expert: E4M3 code bytes [N, K] uniform over the 254
    finite codes, UE8M0 scale bytes [N, K/32] in 113..116 (|w| up to about 0.05)."""
    assert K % 32 == 0
    g = rng(seed, _T_SH8_CODES, layer, mat)
    codes = g.integers(0, 254, (N, K), dtype=np.int16)
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)   # skip 0x7F and 0xFF (NaN)
    scales = (127 + rng(seed, _T_SH8_SCALES, layer, mat).integers(-14, -10, (N, K // 32),
                                                                   dtype=np.int16)).astype(np.uint8)
    return codes, scales


def shared_weights_mxfp8(seed: int, layer: int, I: int, H: int):
    """MXFP8 (codes, scales) of the shared expert's gate [I, H], up [I, H], down [H, I]."""
    return (mxfp8_matrix(seed, layer, MAT_GATE, I, H), mxfp8_matrix(seed, layer, MAT_UP, I, H),
            mxfp8_matrix(seed, layer, MAT_DOWN, H, I))


def sample_tokens(seed: int, T: int, n: int) -> np.ndarray:
    return np.sort(rng(seed, _T_SAMPLE).choice(T, size=n, replace=False))
