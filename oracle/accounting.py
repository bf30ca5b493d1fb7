"""Closed-form accounting of the compressed cache (bits, ratios, reconstruction cost).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Sources (STAR-KV summary page):
* Methodology section 3: an outlier block of 20% of the latent channels at a
  higher bit width (4 bits in the example) and the inlier 80% at a lower one
  (3 bits); Key Results: this "3.2-bit" quantiser combined with up to 75%
  low-rank compression gives up to 20x overall cache reduction.
* Methodology section 2: joint decomposition costs h times (h = number of heads)
  the reconstruction compute of head-wise decomposition.
"""

from __future__ import annotations


def mean_bits(frac_hi: float, bits_hi: float, bits_lo: float) -> float:
    """Average bits per latent channel of a two-block mixed-precision quantiser."""
    return frac_hi * bits_hi + (1.0 - frac_hi) * bits_lo


def reduction(low_rank_compression: float, bits: float, base_bits: float = 16.0) -> float:
    """Overall cache reduction: keep (1 - c) of the channels, each at ``bits`` instead of 16."""
    return (1.0 / (1.0 - low_rank_compression)) * (base_bits / bits)


def reconstruction_flops_per_token(total_rank: int, heads: int, d_h: int, joint: bool) -> int:
    """Flops to rebuild one token's keys of all heads from the latent.

    Joint: one latent of rank R feeds every head's d_h outputs: 2 R (H d_h).
    Head-wise at equal total rank: head h has rank R/H and d_h outputs: H * 2 (R/H) d_h.
    """
    if joint:
        return 2 * total_rank * heads * d_h
    return 2 * total_rank * d_h

