"""Seeded synthetic inputs shaped like the expert layers of an MXFP4 MoE.

This module only draws random numbers and lays them out.  It holds none of
the quantization arithmetic, so both the GPU library's tests/bench and the
CPU oracle can take their inputs from here.

The pages ("Training an MoE LLM in MXFP4: How We Closed the Gap to BF16",
Abstract) train GPT-OSS-20B, a 20B-parameter MoE, on the MLPerf Small MoE
benchmark with C4.  None of that data is used: the tensors below only take
the shapes of its expert layers (d_model 2880, 32 experts, top-4 routing,
expert FFN 2880) and stand in for activations, weights and gradients.

bf16 tensors are returned as their uint16 bit patterns, rounded from fp32 to
nearest-even.
"""
from __future__ import annotations

import numpy as np

D_MODEL = 2880
D_FF2 = 5760          # gate+up fused output width of the first expert linear
N_EXPERTS = 32
TOP_K = 4
N_TOKENS = 16384


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# config 1: fp32 256x512, N(0,1), 0.1% of entries scaled by 50 (outliers)
# ---------------------------------------------------------------------------
def outlier_matrix(rows=256, cols=512, frac=0.001, factor=50.0, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    n_out = int(round(frac * rows * cols))
    pos = rng.choice(rows * cols, size=n_out, replace=False)
    flat = x.reshape(-1)
    flat[pos] *= factor
    return x.astype(np.float32), np.sort(pos)


# ---------------------------------------------------------------------------
# config 2 / 4 / 5 activations: N(0,1) x per-column log-uniform[0.1, 10]
# ---------------------------------------------------------------------------
def channel_scaled_activations(rows=N_TOKENS, cols=D_MODEL, seed=1, lo=0.1, hi=10.0):
    rng = np.random.default_rng(seed)
    c = np.exp(rng.uniform(np.log(lo), np.log(hi), size=cols))
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    return f32_to_bf16_bits(z * c.astype(np.float32)[None, :])


def normal_bf16(shape, std, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(std))


# ---------------------------------------------------------------------------
# Zipf(1.1) routing counts over 32 experts, 65,536 assignments
# ---------------------------------------------------------------------------
def zipf_counts(n_assign=N_TOKENS * TOP_K, n_experts=N_EXPERTS, s=1.1, seed=4,
                cap=N_TOKENS):
    """Bounded Zipf over ranks 1..E (p_k ~ k^-s), one multinomial draw, then
    each expert is capped at `cap` (a token picks an expert at most once in
    top-k) with the excess spread over the uncapped experts in proportion to
    p.  Expert e takes rank e+1."""
    rng = np.random.default_rng(seed)
    k = np.arange(1, n_experts + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    counts = rng.multinomial(n_assign, p).astype(np.int64)
    while counts.max() > cap:
        over = counts > cap
        excess = int((counts[over] - cap).sum())
        counts[over] = cap
        free = ~over & (counts < cap)
        w = p * free
        share = excess * w / w.sum()
        base = np.floor(share).astype(np.int64)
        rem = excess - int(base.sum())
        order = np.argsort(-(share - base), kind="stable")
        base[order[:rem]] += 1
        counts += base
    assert counts.sum() == n_assign
    return counts


def offsets_from_counts(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def routing_row_index(counts, n_tokens=N_TOKENS) -> np.ndarray:
    """Assignment j (in expert order) reads token j mod n_tokens; with counts
    capped at n_tokens the tokens of one expert are distinct."""
    total = int(np.sum(counts))
    return (np.arange(total, dtype=np.int64) % n_tokens).astype(np.int32)


# ---------------------------------------------------------------------------
# small helpers for tests
# ---------------------------------------------------------------------------
def random_group_counts(total, groups, seed, min_count=0):
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, total + 1, size=groups - 1))
    counts = np.diff(np.concatenate([[0], cuts, [total]]))
    return np.maximum(counts, min_count).astype(np.int64)
