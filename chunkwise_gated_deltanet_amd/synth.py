"""Seeded synthetic inputs for the WY/UT preparation step.

This module only draws inputs; it holds none of the method's arithmetic.  The same host arrays
feed the HIP path (after a host-to-device copy) and the CPU oracle.

Recipe (one numpy PCG64 generator per workload, seeded with the workload's seed):
  1. packed workloads only: draw the sequence lengths (integers, uniform in [lo, hi]); any
     length that is a multiple of C is redrawn, so every sequence ends in a short chunk;
  2. k ~ N(0, 1) in float32, shape [B, T, Hq, dk], drawn in slices of 4096 tokens, then
     divided by its own L2 norm per (token, head), in float32;
  3. v ~ N(0, 1) in float32, shape [B, T, Hv, dv], drawn the same way;
  4. z ~ N(0, 1) in float32, shape [B, T, Hv]; beta = sigmoid(sigma * z) in float32;
  5. bf16 workloads: k and v rounded to bf16 (round to nearest, ties to even).  bf16 data is
     carried as uint16 bit patterns on the host;
  6. gated inputs only: y ~ N(0, 1) in float32, shape [B, T, Hv], and the log gate
     g = log sigmoid(mu + y) = -log(1 + exp(-(mu + y))) in float32, so every decay
     alpha = exp(g) lies in (0, 1).  mu = 4 puts alpha near 0.98 (0.88 .. 0.9975 within two
     standard deviations): a chunk of 64 tokens decays by about e^-1.6, and 6-8 chunks by
     e^-10 or more, the regime in which the FlashQLA page reports its gate warm-up working.
     Drawn after beta, so k, v and beta do not depend on whether gates are drawn;
  7. forward inputs only: q ~ N(0, 1) in float32, shape [B, T, Hq, dk], drawn like k and
     L2-normalised per (token, head) like k, then rounded to bf16 (bf16 workloads).  Drawn
     last.

Workload shapes follow the head configurations the pages benchmark GDN on (value heads 64 down
to 8 at d_k = d_v = 128) and the page's chunk sizes C in {32, 64, 128}.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SLICE_TOKENS = 4096


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite, so NaN payloads need no special case.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


@dataclass
class Workload:
    name: str
    batch: int
    seqlen: int          # per batch row; total packed tokens when seqlens is given
    num_qk_heads: int
    num_v_heads: int
    head_dim_k: int
    head_dim_v: int
    chunk_size: int
    dtype: str           # "bf16" or "f32" (k, v, W, U)
    beta_sigma: float
    seed: int
    seq_range: tuple | None = None   # (lo, hi, count) for packed sequences
    gate_mu: float | None = None     # None: no gates; else g = log sigmoid(gate_mu + N(0,1))
    with_q: bool = False             # also draw the queries q (the chunked forward's input)
    note: str = ""
    extra: dict = field(default_factory=dict)


def workloads() -> dict:
    """The five seeded workloads (sizes as stated by the hot path's target), and a sixth that
    stresses the packed-sequence work map: 1024 short sequences of 1..65 tokens."""
    return {
        1: Workload("tiny fp32: B=1 T=256 H=2/2 C=32", 1, 256, 2, 2, 128, 128, 32, "f32", 1.0, 1),
        2: Workload("B=1 T=8192 H=16/16 C=64 bf16", 1, 8192, 16, 16, 128, 128, 64, "bf16", 1.5,
                    2),
        3: Workload("B=4 T=4096 H=32/32 C=64 bf16", 4, 4096, 32, 32, 128, 128, 64, "bf16", 1.0,
                    3),
        4: Workload("B=1 T=32768 H=8/8 C=128 bf16", 1, 32768, 8, 8, 128, 128, 128, "bf16", 1.0,
                    4),
        5: Workload("packed 8 seqs U[300,16384] Hq=16 Hv=64 C=64 bf16", 1, 0, 16, 64, 128, 128,
                    64, "bf16", 1.0, 5, seq_range=(300, 16384, 8)),
        6: Workload("packed 1024 seqs U[1,65] Hq=16 Hv=16 C=64 bf16", 1, 0, 16, 16, 128, 128, 64,
                    "bf16", 1.0, 6, seq_range=(1, 65, 1024)),
    }


def workload(idx: int, chunk_size: int | None = None, **overrides) -> Workload:
    w = workloads()[idx]
    if chunk_size is not None:
        w.chunk_size = chunk_size
        w.name = w.name.replace(f"C={workloads()[idx].chunk_size}", f"C={chunk_size}")
    for key, val in overrides.items():
        setattr(w, key, val)
    return w


def _draw_normal(rng, shape):
    """N(0,1) float32 draws, slice by slice along the token axis (axis 1)."""
    out = np.empty(shape, np.float32)
    T = shape[1]
    for t0 in range(0, T, SLICE_TOKENS):
        t1 = min(T, t0 + SLICE_TOKENS)
        out[:, t0:t1] = rng.standard_normal((shape[0], t1 - t0) + tuple(shape[2:]),
                                            dtype=np.float32)
    return out


def draw_seqlens(rng, lo, hi, count, chunk_size):
    lens = rng.integers(lo, hi + 1, size=count)
    while True:
        bad = (lens % chunk_size) == 0
        if not bad.any():
            break
        lens[bad] = rng.integers(lo, hi + 1, size=int(bad.sum()))
    return lens.astype(np.int64)


def generate(w: Workload) -> dict:
    """Draws the inputs of a workload.

    Returns a dict with k, v (uint16 bf16 bits or float32), beta (float32 [B,T,Hv]),
    cu_seqlens (int32 [N+1] or None) and the shape fields.
    """
    rng = np.random.default_rng(w.seed)
    cu = None
    B, T = w.batch, w.seqlen
    if w.seq_range is not None:
        lo, hi, count = w.seq_range
        lens = draw_seqlens(rng, lo, hi, count, w.chunk_size)
        cu = np.zeros(count + 1, np.int64)
        cu[1:] = np.cumsum(lens)
        B, T = 1, int(cu[-1])
        cu = cu.astype(np.int32)
    k = _draw_normal(rng, (B, T, w.num_qk_heads, w.head_dim_k))
    norm = np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    k = (k / norm).astype(np.float32)
    v = _draw_normal(rng, (B, T, w.num_v_heads, w.head_dim_v))
    z = rng.standard_normal((B, T, w.num_v_heads), dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-np.float32(w.beta_sigma) * z, dtype=np.float32))).astype(
        np.float32)
    g = None
    if w.gate_mu is not None:
        y = rng.standard_normal((B, T, w.num_v_heads), dtype=np.float32)
        g = (-np.logaddexp(np.float32(0), -(np.float32(w.gate_mu) + y))).astype(np.float32)
    q = None
    if w.with_q:
        q = _draw_normal(rng, (B, T, w.num_qk_heads, w.head_dim_k))
        qn = np.sqrt(np.sum(q * q, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
        q = (q / qn).astype(np.float32)
    if w.dtype == "bf16":
        k = f32_to_bf16_bits(k)
        v = f32_to_bf16_bits(v)
        q = None if q is None else f32_to_bf16_bits(q)
    elif w.dtype != "f32":
        raise ValueError(w.dtype)
    return dict(k=k, v=v, beta=beta, g=g, q=q, cu_seqlens=cu, batch=B, seqlen=T,
                chunk_size=w.chunk_size, num_qk_heads=w.num_qk_heads,
                num_v_heads=w.num_v_heads, dtype=w.dtype, name=w.name)


def custom(batch, seqlen, num_qk_heads, num_v_heads, chunk_size, dtype="bf16", seed=0,
           beta_sigma=1.0, seqlens=None, head_dim=128, gate_mu=None, with_q=False) -> dict:
    """Inputs for an arbitrary shape, same recipe.  `seqlens` (list) makes a packed batch;
    `gate_mu` (float) adds log gates g; `with_q` adds queries q."""
    w = Workload("custom", batch, seqlen, num_qk_heads, num_v_heads, head_dim, head_dim,
                 chunk_size, dtype, beta_sigma, seed, gate_mu=gate_mu, with_q=with_q)
    if seqlens is not None:
        rng_lens = np.asarray(seqlens, np.int64)
        w.batch, w.seqlen = 1, int(rng_lens.sum())
        out = generate(w)
        cu = np.zeros(len(rng_lens) + 1, np.int64)
        cu[1:] = np.cumsum(rng_lens)
        out["cu_seqlens"] = cu.astype(np.int32)
        return out
    return generate(w)
