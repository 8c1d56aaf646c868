"""Seeded synthetic inputs for decode attention over a rotated, quantized, paged KV cache.

This module only draws random numbers and fixes the workload shapes.  It holds
none of the method's arithmetic (no rotation, clipping, quantization, packing
or attention): the CPU oracle and the GPU path both receive the arrays made
here and nothing else is shared between them.

The workloads follow the shapes of the pages' serving experiments (GQA 32/8 or
64/8, head dim 128, 4k..131k contexts, batch 1..32).  The pages measure on
public suites with real models; these seeded caches stand in for them in shape
only (channel outliers like real keys, decaying channel spectra).

bf16 data are made by truncating float32 draws to their top 16 bits: that is a
way of producing bf16 test data, not the cache's rounding rule.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

HEAD_DIM = 128

# stream tags so each tensor draws from its own independent seed sequence
_TAG = {"k": 1, "v": 2, "q": 3, "outlier": 4, "rot_k": 5, "rot_v": 6,
        "sign_k": 7, "sign_v": 8, "pages": 9, "lens": 10, "step": 11}


@dataclass(frozen=True)
class Workload:
    """Shape, scheme and input recipe of one synthetic workload."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    scheme: str                 # "int2_channel" (per channel, 128-token groups) | "int2_token" | "int4_token"
    n_sink: int
    n_recent: int
    clip_k: float
    clip_v: float
    src_dtype: str              # "f32" | "bf16"
    seq_len: int                # context length (max for ragged)
    seq_len_min: Optional[int] = None   # ragged lengths U{min..seq_len}, seeded
    outlier_channels: int = 0   # per (kv head, K or V)
    outlier_scale: float = 1.0
    spectrum: str = "flat"      # "flat" | "decay" (sigma_c = (c+1)^-0.5)
    identity_pages: bool = False
    page_tokens: int = 64
    group_tokens: int = 128
    split_tokens: int = 512
    rotation: str = "oscar"     # "oscar" (QR·H·P_br) | "saw" (diag(sign)·H)
    key_only: bool = False      # rotate K only; V quantized in its own frame
    hadamard_block: int = 128   # block order h of the randomized Hadamard ("saw" rotation)
    seed: int = 1000
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def gq(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny_1h_4k": Workload(
        name="tiny_1h_4k", batch=1, n_q_heads=1, n_kv_heads=1, scheme="int2_channel",
        n_sink=4, n_recent=128, clip_k=0.96, clip_v=0.92, src_dtype="f32", seq_len=4096,
        outlier_channels=4, outlier_scale=10.0, identity_pages=True, seed=1001),
    "gqa_b1_32k": Workload(
        name="gqa_b1_32k", batch=1, n_q_heads=32, n_kv_heads=8, scheme="int2_channel",
        n_sink=4, n_recent=128, clip_k=0.96, clip_v=0.92, src_dtype="bf16", seq_len=32768,
        outlier_channels=3, outlier_scale=8.0, seed=1002),
    "batch32_8k_32k": Workload(
        name="batch32_8k_32k", batch=32, n_q_heads=32, n_kv_heads=8, scheme="int2_channel",
        n_sink=4, n_recent=128, clip_k=0.96, clip_v=0.92, src_dtype="bf16", seq_len=32768,
        seq_len_min=8192, outlier_channels=3, outlier_scale=8.0, seed=1003),
    # the headline point: every sequence at 32k
    "batch32_32k": Workload(
        name="batch32_32k", batch=32, n_q_heads=32, n_kv_heads=8, scheme="int2_channel",
        n_sink=4, n_recent=128, clip_k=0.96, clip_v=0.92, src_dtype="bf16", seq_len=32768,
        outlier_channels=3, outlier_scale=8.0, seed=1003),
    "saw_int4_b16_16k": Workload(
        name="saw_int4_b16_16k", batch=16, n_q_heads=32, n_kv_heads=8, scheme="int4_token",
        n_sink=0, n_recent=0, clip_k=1.0, clip_v=1.0, src_dtype="bf16", seq_len=16384,
        rotation="saw", seed=1004, extra={"prefill_chunk": 8192}),
    "long_b4_131k": Workload(
        name="long_b4_131k", batch=4, n_q_heads=64, n_kv_heads=8, scheme="int2_channel",
        n_sink=4, n_recent=256, clip_k=0.96, clip_v=0.92, src_dtype="bf16", seq_len=131072,
        spectrum="decay", seed=1005),
}


def scaled(wl: Workload, **changes) -> Workload:
    """Same recipe with some fields changed (smaller sizes for CPU-feasible parity)."""
    return replace(wl, **changes)


def _rng(wl: Workload, tag: str, *idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.seed, _TAG[tag], *idx]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Truncate float32 draws to bf16 bit patterns (test-data construction)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def seq_lens(wl: Workload) -> np.ndarray:
    if wl.seq_len_min is None:
        return np.full(wl.batch, wl.seq_len, dtype=np.int32)
    r = _rng(wl, "lens")
    return r.integers(wl.seq_len_min, wl.seq_len + 1, size=wl.batch).astype(np.int32)


def outlier_channels(wl: Workload, kv_head: int, which: str) -> np.ndarray:
    """Seeded outlier channel indices for one (kv head, K|V)."""
    if wl.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(wl, "outlier", kv_head, 0 if which == "k" else 1)
    return np.sort(r.choice(HEAD_DIM, size=wl.outlier_channels, replace=False))


def channel_gain(wl: Workload, which: str) -> np.ndarray:
    """[n_kv, 128] per-channel multiplier: outliers and/or decaying spectrum."""
    g = np.ones((wl.n_kv_heads, HEAD_DIM), dtype=np.float32)
    if wl.spectrum == "decay":
        g *= (np.arange(1, HEAD_DIM + 1, dtype=np.float64) ** -0.5).astype(np.float32)[None, :]
    for h in range(wl.n_kv_heads):
        ch = outlier_channels(wl, h, which)
        g[h, ch] *= np.float32(wl.outlier_scale)
    return g


def kv_tokens(wl: Workload, seq: int, start: int, count: int, which: str) -> np.ndarray:
    """Source K or V for tokens [start, start+count) of sequence `seq`.

    Returns float32 [count, n_kv, 128] for f32 workloads and bf16 bit patterns
    (uint16) of the same shape otherwise.  Tokens are drawn in blocks of 1024
    from per-(seq, block) streams, so any token range can be regenerated
    without drawing the whole sequence.
    """
    assert which in ("k", "v")
    blk = 1024
    out = np.empty((count, wl.n_kv_heads, HEAD_DIM), dtype=np.float32)
    gain = channel_gain(wl, which)
    t = start
    while t < start + count:
        b = t // blk
        r = _rng(wl, which, seq, b)
        block = r.standard_normal((blk, wl.n_kv_heads, HEAD_DIM), dtype=np.float32)
        lo = t - b * blk
        hi = min(blk, start + count - b * blk)
        out[t - start:t - start + (hi - lo)] = block[lo:hi]
        t += hi - lo
    out *= gain[None]
    if wl.src_dtype == "bf16":
        return to_bf16_bits(out)
    return out


def queries(wl: Workload, step: int = 0) -> np.ndarray:
    """Decode queries [batch, n_q, 128]: float32 or bf16 bits like the cache source."""
    r = _rng(wl, "q", step)
    q = r.standard_normal((wl.batch, wl.n_q_heads, HEAD_DIM), dtype=np.float32)
    return to_bf16_bits(q) if wl.src_dtype == "bf16" else q


def prefill_queries(wl: Workload, seq: int, start: int, count: int) -> np.ndarray:
    """Queries of chunk positions start .. start + count - 1 of sequence `seq`: [count, n_q, 128], float32 or
    bf16 bits like the cache source (one seeded stream per position, so any chunking draws the same rows)."""
    rows = []
    for p in range(start, start + count):
        r = _rng(wl, "q", 7919, seq, p)
        rows.append(r.standard_normal((wl.n_q_heads, HEAD_DIM), dtype=np.float32))
    q = np.stack(rows) if rows else np.zeros((0, wl.n_q_heads, HEAD_DIM), np.float32)
    return to_bf16_bits(q) if wl.src_dtype == "bf16" else q


def rotation_gaussian(wl: Workload, which: str) -> np.ndarray:
    """Seeded 128x128 N(0,1) float64 matrix whose QR factor stands in for a calibrated eigenbasis."""
    r = _rng(wl, "rot_k" if which == "k" else "rot_v")
    return r.standard_normal((HEAD_DIM, HEAD_DIM))


def calibration_activations(n: int, seed: int, n_keys: int = 256):
    """Seeded calibration data for the covariance-built rotation: queries q [n][128] with a correlated,
    decaying spectrum (q = z diag(g) G, g_c = (c+1)^-0.5, z and G standard normal), values [n_keys][128]
    of the same kind, and row-stochastic attention scores [n][n_keys] (softmax of N(0, 2^2) logits).
    Returns (q, v, scores) as float32."""
    r = np.random.default_rng(np.random.SeedSequence([0xCA11B, seed]))
    g = (np.arange(HEAD_DIM) + 1.0) ** -0.5
    mix_q = g[:, None] * r.standard_normal((HEAD_DIM, HEAD_DIM))
    mix_v = g[:, None] * r.standard_normal((HEAD_DIM, HEAD_DIM))
    q = r.standard_normal((n, HEAD_DIM)) @ mix_q
    v = r.standard_normal((n_keys, HEAD_DIM)) @ mix_v
    logits = 2.0 * r.standard_normal((n, n_keys))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    scores = e / e.sum(axis=1, keepdims=True)
    return q.astype(np.float32), v.astype(np.float32), scores.astype(np.float32)


def sign_vector(wl: Workload, which: str) -> np.ndarray:
    """Seeded random signs (+1/-1, int8) of the randomized Hadamard transform."""
    r = _rng(wl, "sign_k" if which == "k" else "sign_v")
    return np.where(r.integers(0, 2, size=HEAD_DIM) == 1, 1, -1).astype(np.int8)


def step_tokens(wl: Workload, step: int, which: str) -> np.ndarray:
    """One appended token per sequence for decode step `step`: [batch, n_kv, 128]."""
    r = _rng(wl, "step", step, 0 if which == "k" else 1)
    x = r.standard_normal((wl.batch, wl.n_kv_heads, HEAD_DIM), dtype=np.float32)
    x *= channel_gain(wl, which)[None]
    return to_bf16_bits(x) if wl.src_dtype == "bf16" else x
