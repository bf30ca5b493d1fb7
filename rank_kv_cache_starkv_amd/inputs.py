"""Seeded synthetic inputs for the STAR-KV decode path.

This module is the only code shared by the CPU oracle side (tests, the CPU
baseline in ``bench.py``) and the GPU side.  It draws random numbers and shapes
them like the workloads the STAR-KV pages evaluate on; it holds none of the
method's arithmetic (no rank selection, no factor build, no quantisation, no
attention).

What it produces, per workload and layer:

* per key head ``g`` a projection ``W_k^g = U_g diag(sigma) V_g^T`` given by its
  factors: ``U_g`` (d x d_h, orthonormal columns from the QR of a Gaussian),
  ``V_g`` (d_h x d_h orthogonal) and the spectrum ``sigma_i = i^-p``;
* the joint value projection ``W_v`` the same way, with ``n_keep`` leading
  singular triplets (the method only ever keeps a prefix of them);
* per head thresholds ``tau_g`` placed at the geometric mean of
  ``sigma_{r_g}`` and ``sigma_{r_g+1}``, so that the adaptive rank each head
  ends up with is known by construction (STAR-KV page, Methodology section 1:
  thresholds are learnt per block and per head, and applied to the singular
  values);
* hidden states ``X ~ N(0, 1)``, queries ``q ~ N(0, 1)`` and context lengths.

Random streams are independent per (workload, layer, purpose, index), so a
sequence's prefill can be regenerated in pieces without drawing the others.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

SEED_ROOT = 2606_08382  # the arXiv id of the STAR-KV paper, used as a fixed seed

_PURPOSE = {
    "w_k": 1,
    "w_v": 2,
    "ranks": 3,
    "x_prefill": 4,
    "x_cal": 5,
    "x_new": 6,
    "q": 7,
    "lens": 8,
    "misc": 9,
    "W_q": 10,
    "x_q": 11,
}


def rng_for(cfg_id: int, layer: int, purpose: str, index: int = 0) -> np.random.Generator:
    """Independent generator for one (workload, layer, purpose, index)."""
    return np.random.default_rng(
        np.random.SeedSequence([SEED_ROOT, int(cfg_id), int(layer), _PURPOSE[purpose], int(index)])
    )


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload (one decoder layer)."""

    cfg_id: int
    name: str
    B: int
    H_q: int
    H_kv: int
    d_h: int
    d: int
    n_q: int
    latent: str  # "f32", "bf16", "mix84" (int8 lead / int4 rest), "had43" (rotated 4-bit / 3-bit) or
    #              "had43p" (the same codes packed to 4 / 3 bits)
    dtype: str  # "f32" or "bf16": X, q, factors, out
    p: float  # spectrum exponent: sigma_i = i^-p
    r_v: int  # value latent rank (joint decomposition)
    key_ranks: Optional[Tuple[int, ...]] = None  # explicit per-KV-head ranks
    rank_lo: int = 0
    rank_hi: int = 0
    rank_sum: int = 0
    T: int = 0  # context length at decode (fixed-length workloads)
    T_lo: int = 0  # ragged workloads: context drawn from U{T_lo..T_hi} before the append
    T_hi: int = 0
    n_cal: int = 0  # calibration tokens for the per-channel scales
    n_append: int = 0  # tokens per sequence appended by compress_append before decode

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def ragged(self) -> bool:
        return self.T_hi > 0


# The workloads.  Sizes follow the pages' evaluation setting: a 7B-class layer at
# a 4K context (the LongBench/RULER length), a GQA layer at long context, and a
# high-batch 13B-class serving step with a speculative-style chunk of 4 queries.
# Workload 5 is the 7B-class quantised layer with the block-rotated 4-bit/3-bit
# quantiser instead of the int8/int4 split; workload 6 is the same layer with those
# codes packed to their own widths (3.2 bits per channel).
WORKLOADS: Dict[int, Workload] = {
    0: Workload(0, "tiny-f32", B=1, H_q=4, H_kv=4, d_h=64, d=256, n_q=1, latent="f32", dtype="f32",
                p=0.7, r_v=64, key_ranks=(16, 24, 32, 16), T=256),
    1: Workload(1, "llama2-7b-bf16-latent", B=8, H_q=32, H_kv=32, d_h=128, d=4096, n_q=1,
                latent="bf16", dtype="bf16", p=0.5, r_v=1024, rank_lo=16, rank_hi=64, rank_sum=1024,
                T=4096),
    2: Workload(2, "llama2-7b-mix84", B=8, H_q=32, H_kv=32, d_h=128, d=4096, n_q=1,
                latent="mix84", dtype="bf16", p=0.5, r_v=1024, rank_lo=16, rank_hi=64, rank_sum=1024,
                T=4096, n_cal=512, n_append=128),
    3: Workload(3, "llama3-8b-gqa-32k-mix84", B=1, H_q=32, H_kv=8, d_h=128, d=4096, n_q=1,
                latent="mix84", dtype="bf16", p=0.5, r_v=512, rank_lo=32, rank_hi=96, rank_sum=512,
                T=32768, n_cal=512),
    4: Workload(4, "llama2-13b-b64-ragged-nq4-mix84", B=64, H_q=40, H_kv=40, d_h=128, d=5120, n_q=4,
                latent="mix84", dtype="bf16", p=0.5, r_v=1280, rank_lo=16, rank_hi=64, rank_sum=1280,
                T_lo=1024, T_hi=8192, n_cal=512, n_append=4),
    5: Workload(5, "llama2-7b-had43", B=8, H_q=32, H_kv=32, d_h=128, d=4096, n_q=1,
                latent="had43", dtype="bf16", p=0.5, r_v=1024, rank_lo=16, rank_hi=64, rank_sum=1024,
                T=4096, n_cal=512, n_append=128),
    6: Workload(6, "llama2-7b-had43p", B=8, H_q=32, H_kv=32, d_h=128, d=4096, n_q=1,
                latent="had43p", dtype="bf16", p=0.5, r_v=1024, rank_lo=16, rank_hi=64, rank_sum=1024,
                T=4096, n_cal=512, n_append=128),
}


def spectrum(n: int, p: float) -> np.ndarray:
    """sigma_i = i^-p for i = 1..n, as float32."""
    i = np.arange(1, n + 1, dtype=np.float64)
    return (i ** (-float(p))).astype(np.float32)


def orthonormal_columns(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Q factor of a Gaussian rows x cols matrix (orthonormal columns), float64."""
    g = rng.standard_normal((rows, cols))
    q, r = np.linalg.qr(g)
    # fix the column signs so the draw does not depend on the LAPACK sign convention
    sgn = np.sign(np.diag(r))
    sgn[sgn == 0] = 1.0
    return q * sgn


def draw_ranks(rng: np.random.Generator, H: int, lo: int, hi: int, total: int) -> np.ndarray:
    """Per-head ranks in [lo, hi] that sum to ``total``, with at least one odd rank.

    Starts from the mean and applies seeded transfers between random pairs of
    heads that keep every rank in range and the sum fixed.
    """
    if not (lo * H <= total <= hi * H):
        raise ValueError("rank bounds cannot reach the requested total")
    r = np.full(H, total // H, dtype=np.int64)
    r[: total - int(r.sum())] += 1
    for _ in range(8 * H):
        i, j = rng.integers(0, H, size=2)
        if i == j:
            continue
        amt = int(rng.integers(1, max(2, (hi - lo) // 2)))
        amt = min(amt, int(r[i]) - lo, hi - int(r[j]))
        if amt > 0:
            r[i] -= amt
            r[j] += amt
    if not np.any(r % 2 == 1):
        # move one unit between two heads that both have room: both become odd
        for i in range(H):
            j = (i + 1) % H
            if r[i] > lo and r[j] < hi:
                r[i] -= 1
                r[j] += 1
                break
    assert int(r.sum()) == total and r.min() >= lo and r.max() <= hi
    return r.astype(np.int32)


def threshold_between(s32: np.ndarray, rank: int) -> np.float32:
    """A float32 threshold strictly between s[rank-1] and s[rank] (1-based sigma_r, sigma_{r+1}).

    ``rank == len(s)`` gives half the smallest value; ``rank == 0`` gives twice the largest.
    """
    n = len(s32)
    if rank <= 0:
        t = np.float32(2.0 * float(s32[0]))
    elif rank >= n:
        t = np.float32(0.5 * float(s32[n - 1]))
    else:
        t = np.float32(math.sqrt(float(s32[rank - 1]) * float(s32[rank])))
    if rank > 0:
        assert s32[rank - 1] > t
    if rank < n:
        assert not (s32[rank] > t)
    return t


@dataclasses.dataclass
class LayerFactors:
    """SVD factors and thresholds of one layer's key and value projections (host, float32)."""

    U_k: np.ndarray  # [H_kv, d, d_h]
    s_k: np.ndarray  # [H_kv, d_h]
    V_k: np.ndarray  # [H_kv, d_h, d_h]
    tau_k: np.ndarray  # [H_kv]
    U_v: np.ndarray  # [d, n_keep]
    s_v: np.ndarray  # [n_keep]
    V_v: np.ndarray  # [H_kv * d_h, n_keep]
    tau_v: np.float32
    target_key_ranks: np.ndarray  # [H_kv] int32, the ranks tau was placed for
    target_r_v: int


def layer_spectra(w: Workload, layer: int = 0, n_keep_extra: int = 64):
    """Spectra and thresholds only (no bases): (s_k [H_kv, d_h], tau_k [H_kv], s_v, tau_v, ranks)."""
    s = spectrum(w.d_h, w.p)
    s_k = np.tile(s, (w.H_kv, 1))
    if w.key_ranks is not None:
        ranks = np.asarray(w.key_ranks, dtype=np.int32)
    else:
        ranks = draw_ranks(rng_for(w.cfg_id, layer, "ranks"), w.H_kv, w.rank_lo, w.rank_hi, w.rank_sum)
    tau_k = np.array([threshold_between(s_k[g], int(ranks[g])) for g in range(w.H_kv)], dtype=np.float32)
    n_full = min(w.d, w.H_kv * w.d_h)
    n_keep = min(n_full, w.r_v + n_keep_extra)
    s_v = spectrum(n_full, w.p)[:n_keep].copy()
    tau_v = threshold_between(s_v, w.r_v)
    return s_k, tau_k, s_v, tau_v, ranks


def layer_factors(w: Workload, layer: int = 0, n_keep_extra: int = 64) -> LayerFactors:
    """Synthetic SVD factors for one layer of workload ``w``."""
    s_k, tau_k, s_v, tau_v, ranks = layer_spectra(w, layer, n_keep_extra)
    rk = rng_for(w.cfg_id, layer, "w_k")
    U_k = np.empty((w.H_kv, w.d, w.d_h), dtype=np.float32)
    V_k = np.empty((w.H_kv, w.d_h, w.d_h), dtype=np.float32)
    for g in range(w.H_kv):
        U_k[g] = orthonormal_columns(rk, w.d, w.d_h).astype(np.float32)
        V_k[g] = orthonormal_columns(rk, w.d_h, w.d_h).astype(np.float32)
    n_keep = len(s_v)
    rv = rng_for(w.cfg_id, layer, "w_v")
    U_v = orthonormal_columns(rv, w.d, n_keep).astype(np.float32)
    V_v = orthonormal_columns(rv, w.H_kv * w.d_h, n_keep).astype(np.float32)
    return LayerFactors(U_k, s_k, V_k, tau_k, U_v, s_v, V_v, tau_v, ranks, w.r_v)


def context_lengths(w: Workload) -> np.ndarray:
    """Context length per sequence *before* the decode step's own append.

    Fixed-length workloads hold ``T - n_append`` prefilled tokens so that the
    decode sees ``T``; the ragged workload draws ``U{T_lo..T_hi}``.
    """
    if w.ragged:
        return rng_for(w.cfg_id, 0, "lens").integers(w.T_lo, w.T_hi + 1, size=w.B).astype(np.int32)
    return np.full(w.B, w.T - w.n_append, dtype=np.int32)


def gaussian(rng: np.random.Generator, shape: Sequence[int]) -> np.ndarray:
    return rng.standard_normal(tuple(shape), dtype=np.float32)


def x_prefill(w: Workload, b: int, t0: int, t1: int, layer: int = 0) -> np.ndarray:
    """Hidden states of sequence ``b``, tokens [t0, t1) (float32, N(0,1)).

    The stream of sequence ``b`` is drawn in order, so any token range is
    reproducible (tokens before t0 are drawn and discarded).
    """
    rng = rng_for(w.cfg_id, layer, "x_prefill", b)
    if t0 > 0:
        skip = t0
        while skip > 0:
            n = min(skip, 4096)
            rng.standard_normal((n, w.d), dtype=np.float32)
            skip -= n
    return gaussian(rng, (t1 - t0, w.d))


def x_prefill_chunks(w: Workload, b: int, T: int, chunk: int, layer: int = 0):
    """Yield (t0, t1, X[t0:t1]) over tokens [0, T) of sequence ``b`` from one stream
    (the same values :func:`x_prefill` gives for any range)."""
    rng = rng_for(w.cfg_id, layer, "x_prefill", b)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        yield t0, t1, gaussian(rng, (t1 - t0, w.d))


def x_calibration(w: Workload, layer: int = 0) -> np.ndarray:
    return gaussian(rng_for(w.cfg_id, layer, "x_cal"), (w.n_cal, w.d))


def x_new(w: Workload, n_new: int, layer: int = 0, step: int = 0) -> np.ndarray:
    """Hidden states of the tokens appended in one step: [B, n_new, d]."""
    return gaussian(rng_for(w.cfg_id, layer, "x_new", step), (w.B, n_new, w.d))


def query_weights(w: Workload, layer: int = 0) -> np.ndarray:
    """Synthetic query projection W_q [d, H_q * d_h] (q = x W_q), Gaussian / sqrt(d)."""
    g = gaussian(rng_for(w.cfg_id, layer, "W_q"), (w.d, w.H_q * w.d_h))
    return (g / np.float32(math.sqrt(w.d))).astype(np.float32)


def query_hidden(w: Workload, layer: int = 0, step: int = 0) -> np.ndarray:
    """Hidden states of the decode queries [B, n_q, d]."""
    return gaussian(rng_for(w.cfg_id, layer, "x_q", step), (w.B, w.n_q, w.d))


def queries(w: Workload, layer: int = 0, step: int = 0, scale: float = 1.0) -> np.ndarray:
    """Decode queries [B, n_q, H_q, d_h] (scale > 1 stresses the softmax max)."""
    return gaussian(rng_for(w.cfg_id, layer, "q", step), (w.B, w.n_q, w.H_q, w.d_h)) * np.float32(scale)


# ---------------------------------------------------------------------------
# dtype handling of inputs (the host side of the boundary carries bf16 as raw bits)

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-half-to-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the workload dtype, returned as float32 values."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(to_bf16_bits(x))
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# exact-latent conditioning: inputs on grids that make X @ A exact in fp32

def snap_hidden(x: np.ndarray) -> np.ndarray:
    """Round to multiples of 2^-4 with |x| <= 255/16 (exactly representable in bf16)."""
    y = np.rint(np.asarray(x, dtype=np.float64) * 16.0)
    y = np.clip(y, -255.0, 255.0)
    return (y / 16.0).astype(np.float32)


def snap_columns(a_cols: np.ndarray) -> np.ndarray:
    """Round each row of ``a_cols`` (one latent channel's column of A) to 8 significant
    bits relative to that channel's max: a <- rint(a / g) * g with g = 2^(floor(log2 max|a|) - 7).
    Returned values are exactly representable in bf16.  Zero channels stay zero.
    """
    a = np.asarray(a_cols, dtype=np.float64)
    out = np.zeros_like(a)
    for c in range(a.shape[0]):
        m = float(np.max(np.abs(a[c]))) if a.shape[1] else 0.0
        if m == 0.0:
            continue
        g = 2.0 ** (math.floor(math.log2(m)) - 7)
        out[c] = np.rint(a[c] / g) * g
    return out.astype(np.float32)


def snap_grid_units(a_cols: np.ndarray) -> np.ndarray:
    """Per channel, the grid step g used by :func:`snap_columns` (0 for zero channels)."""
    a = np.asarray(a_cols, dtype=np.float64)
    g = np.zeros(a.shape[0])
    for c in range(a.shape[0]):
        m = float(np.max(np.abs(a[c]))) if a.shape[1] else 0.0
        if m > 0:
            g[c] = 2.0 ** (math.floor(math.log2(m)) - 7)
    return g
