"""STAR-KV decode path, step by step, on the CPU (NumPy, fp64 unless a step fixes
another precision).  TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Sources (the STAR-KV summary page, "STAR-KV: Low-Rank KV Cache Compression via
Soft Thresholding for Adaptive Rank Control"):

* Methodology section 1, Adaptive Rank Selection: thresholds act on the singular
  values of the key and value projections, one threshold per block and head; at
  inference the thresholds become hard and the projections are truncated.
  -> :func:`select_rank`, :func:`kept_spectrum`, :func:`factor_pair`.
* Methodology section 2, Hybrid Decomposition: keys are factored head by head
  (HD), values jointly over the concatenated heads (JD); the reconstruction
  matrices are fused by reordering the operations.
  -> :func:`build_layer`, :func:`reconstruct`, :func:`attention`,
  :func:`attention_latent`.
* Methodology section 3, Low-Rank-Aware Mixed-Precision Quantisation: leading
  (outlier) channels of the latent get more bits than the rest; the abstract adds
  that the quantiser uses data statistics.
  -> :func:`channel_qmax`, :func:`calibrate_scales`, :func:`quantize`.
  The same section's block-wise Hadamard: the outlier block (20% of the channels)
  and the inlier block (the rest) each get an independent Hadamard rotation that
  is folded into the factors, then 4-bit outlier and 3-bit inlier codes
  (``latent="had43"``).  -> :func:`sylvester`, :func:`pow2_blocks`,
  :func:`block_hadamard`, :func:`factor_pair`.
* Problem Statement: the cache holds the projected hidden states (the latent)
  instead of K and V.  -> :func:`latent`, the cache byte format.

Readings where the pages are silent (each also listed in the design notes):
the kept singular values are shrunk by tau (``shrink=True``) or kept as they
are (``shrink=False``); a channel survives only if ``s > tau`` (strict); the
singular values live in the down-projection ``A = U diag(s')``, ``B = V^T``; the
leading ceil(r/4) channels of each latent segment are int8 (qmax 127), the rest
int4 (qmax 7); quantisation is symmetric with per-channel fp16 scales
``fp16(fp32(absmax)/qmax)`` from calibration tokens, ``code = clamp(rne(x/s))``
with an IEEE fp32 division, and a zero scale gives code 0; the latent is the
fp32 accumulator value; the softmax scale is ``1/sqrt(d_h)``; query ``j`` of a
chunk of ``n_q`` sees the tokens at positions ``<= T - n_q + j``; query head
``h`` reads KV head ``h // (H_q/H_kv)``; there is no positional rotation.
For ``had43``: the outlier block is the leading ceil(r/5) channels of each
segment; a block whose size is not a power of two is rotated by Sylvester
Hadamards on the power-of-two pieces of its binary decomposition (largest
first); the +-1 matrix R goes into ``A`` and ``R^T / n`` (n = the piece's
order) into ``B``, so that ``A B`` is unchanged; codes are clamped to +-7
(outlier) and +-3 (inlier) and stored in the int8 and int4 regions of the
mix84 byte format.  ``had43p`` holds the same codes packed to their own widths:
the outlier block as 4-bit nibbles and the inlier block as 3-bit fields in bit
planes (the layout is :class:`CacheFormat`'s), which is how the codes reach the
3.2 bits per channel of the summary page's Key Results.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np

LOG2E = math.log2(math.e)
TT = 32  # tokens per value tile in the cache byte format


# ---------------------------------------------------------------------------
# precision helpers (the oracle's own; nothing shared with the GPU side)

def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    keep = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & 1) == 1))
    r = ((keep + up.astype(np.uint64)) << 16).astype(np.uint32)
    return r.view(np.float32).reshape(np.shape(x))


def round_dtype(x, dtype: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    if dtype == "bf16":
        return round_bf16(x32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# O1: rank selection (Methodology section 1: hard threshold at inference)

def select_rank(s, tau) -> int:
    """Number of singular values strictly above the threshold, compared in fp32."""
    s32 = np.asarray(s, dtype=np.float32)
    return int(np.count_nonzero(s32 > np.float32(tau)))


def kept_spectrum(s, tau, shrink: bool = True) -> np.ndarray:
    """Singular values that the truncated factors carry (fp32).

    shrink=True: the soft threshold ``max(s - tau, 0)`` (one fp32 subtraction);
    shrink=False: the values themselves (plain truncation).
    """
    s32 = np.asarray(s, dtype=np.float32)
    if not shrink:
        return s32.copy()
    return np.maximum(s32 - np.float32(tau), np.float32(0.0)).astype(np.float32)


# ---------------------------------------------------------------------------
# O2: factor build (truncated SVD factors; singular values in the down-projection)

def factor_pair(U, s, V, tau, shrink: bool = True, dtype: str = "f32", rotate: bool = False):
    """W = U diag(s) V^T  ->  A (d x r) = U[:, :r] diag(s'[:r]),  B (r x n) = V[:, :r]^T.

    A is one fp32 multiply per element, then rounded to ``dtype``; B is V^T rounded.
    rotate=True (Methodology section 3, block-wise Hadamard folded into the factors):
    A' = A R and B' = D^-1 R^T B with the +-1 block-diagonal R of
    :func:`block_hadamard` over the outlier and inlier blocks of this segment and D
    its piece orders; the products are summed in fp64 from the fp32 values, then
    rounded to fp32 and to ``dtype``.
    """
    r = select_rank(s, tau)
    sp = kept_spectrum(s, tau, shrink)[:r]
    U32 = np.asarray(U, dtype=np.float32)[:, :r]
    A32 = U32 * sp[None, :]
    B32 = np.asarray(V, dtype=np.float32)[:, :r].T
    if not rotate:
        return round_dtype(A32, dtype), round_dtype(B32, dtype)
    R, n = block_hadamard(r, had43_split(r)[0])
    A = A32.astype(np.float64) @ R
    B = (R.T @ B32.astype(np.float64)) / n[:, None]
    return round_dtype(A.astype(np.float32), dtype), round_dtype(B.astype(np.float32), dtype)


# ---------------------------------------------------------------------------
# block-wise Hadamard rotation (Methodology section 3)

def sylvester(n: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order n (a power of two): H_1 = [1],
    H_2m = [[H_m, H_m], [H_m, -H_m]].  Entries +-1 (int64)."""
    if n < 1 or n & (n - 1):
        raise ValueError(f"Sylvester order must be a power of two, got {n}")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def pow2_blocks(n: int) -> List[int]:
    """The powers of two that sum to n, largest first (its binary decomposition)."""
    return [1 << b for b in range(int(n).bit_length() - 1, -1, -1) if (int(n) >> b) & 1]


def block_hadamard(r: int, n_hi: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rotation of one latent segment of rank r whose leading n_hi channels are the
    outlier block: R (r x r, entries 0/+-1) is block-diagonal with one Sylvester
    Hadamard per power-of-two piece of the outlier block, then of the inlier block
    (pieces in the order of :func:`pow2_blocks`); n (length r) holds, per channel, the
    order of the piece it belongs to, so that R diag(1/n) R^T = I."""
    R = np.zeros((r, r), dtype=np.float64)
    n = np.zeros(r, dtype=np.float64)
    c = 0
    for size in pow2_blocks(n_hi) + pow2_blocks(r - n_hi):
        R[c: c + size, c: c + size] = sylvester(size)
        n[c: c + size] = size
        c += size
    assert c == r
    return R, n


@dataclasses.dataclass
class Layer:
    ranks: np.ndarray  # [H_kv] key ranks
    r_v: int
    A_cat: np.ndarray  # [d, sum(ranks) + r_v]  (natural channel order: key heads, then value)
    B_k: np.ndarray  # [sum(ranks), d_h]       (rows of head g at key offset of g)
    B_v: np.ndarray  # [r_v, H_kv * d_h]
    H_q: int
    H_kv: int
    d_h: int
    latent: str
    dtype: str

    @property
    def key_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.ranks)]).astype(np.int64)

    @property
    def n_key(self) -> int:
        return int(np.sum(self.ranks))

    @property
    def n_lat(self) -> int:
        return self.n_key + self.r_v


def build_layer(U_k, s_k, V_k, tau_k, U_v, s_v, V_v, tau_v, H_q: int, latent: str,
                dtype: str, shrink: bool = True) -> Layer:
    """Hybrid decomposition: per-head (HD) key factors, joint (JD) value factors."""
    H_kv, d, d_h = np.shape(U_k)
    As, Bs, ranks = [], [], []
    rot = latent in ROTATED
    for g in range(H_kv):
        A, B = factor_pair(U_k[g], s_k[g], V_k[g], tau_k[g], shrink, dtype, rotate=rot)
        As.append(A)
        Bs.append(B)
        ranks.append(A.shape[1])
    A_v, B_v = factor_pair(U_v, s_v, V_v, tau_v, shrink, dtype, rotate=rot)
    A_cat = np.concatenate(As + [A_v], axis=1)
    B_k = np.concatenate(Bs, axis=0) if Bs else np.zeros((0, d_h), np.float32)
    return Layer(np.asarray(ranks, dtype=np.int64), A_v.shape[1], A_cat, B_k, B_v,
                 H_q, H_kv, d_h, latent, dtype)


# ---------------------------------------------------------------------------
# mixed precision split (Methodology section 3; leading channels get more bits)

QUANTIZED = ("mix84", "had43", "had43p")
ROTATED = ("had43", "had43p")  # the block-rotated 4-bit/3-bit quantiser (byte regions / packed)


def is_quantized(latent: str) -> bool:
    return latent in QUANTIZED


def mix84_split(r: int) -> Tuple[int, int]:
    """(int8 channels, int4 channels) of a latent segment of rank r: the leading
    ceil(r/4) channels are int8, the rest int4."""
    n8 = -(-int(r) // 4)
    return n8, int(r) - n8


def had43_split(r: int) -> Tuple[int, int]:
    """(outlier channels, inlier channels) of a segment of rank r for the rotated
    quantiser: the leading ceil(r/5) channels (20%) are the outlier block."""
    n_hi = -(-int(r) // 5)
    return n_hi, int(r) - n_hi


def precision_split(r: int, latent: str) -> Tuple[int, int]:
    """(channels in the high-precision block, channels in the low one)."""
    return had43_split(r) if latent in ROTATED else mix84_split(r)


def code_limits(latent: str) -> Tuple[int, int]:
    """qmax of the high and the low block: int8/int4 (127, 7) for mix84; 4-bit and
    3-bit symmetric codes (7, 3) for had43 / had43p."""
    return (7, 3) if latent in ROTATED else (127, 7)


def channel_qmax(layer: Layer) -> np.ndarray:
    """qmax per latent channel in natural order."""
    q = []
    qhi, qlo = code_limits(layer.latent)
    for r in list(layer.ranks) + [layer.r_v]:
        nhi, nlo = precision_split(int(r), layer.latent)
        q += [qhi] * nhi + [qlo] * nlo
    return np.asarray(q, dtype=np.int64)


# ---------------------------------------------------------------------------
# O3 / O4 / O5: calibration, latent projection, quantisation

def latent(X, A_cat) -> np.ndarray:
    """The latent the cache stores before rounding: fp32 of the exact product X @ A."""
    return (np.asarray(X, np.float64) @ np.asarray(A_cat, np.float64)).astype(np.float32)


def calibrate_scales(X_cal, A_cat, qmax) -> np.ndarray:
    """Per-channel fp16 scale from calibration statistics: fp16(fp32(absmax) / qmax)."""
    L = np.asarray(X_cal, np.float64) @ np.asarray(A_cat, np.float64)
    amax = np.max(np.abs(L), axis=0).astype(np.float32) if L.shape[0] else np.zeros(L.shape[1], np.float32)
    return (amax / np.asarray(qmax, dtype=np.float32)).astype(np.float16)


def quantize(x32, scales_f16, qmax) -> np.ndarray:
    """code = clamp(rne(x / s), -qmax, qmax) with an fp32 IEEE division; s == 0 gives 0."""
    x32 = np.asarray(x32, dtype=np.float32)
    s32 = np.asarray(scales_f16, dtype=np.float16).astype(np.float32)
    qm = np.asarray(qmax, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x32 / s32
    c = np.clip(np.rint(y), -qm, qm)
    c = np.where(s32 == 0, 0.0, c)
    return c.astype(np.int64)


def dequantize(codes, scales_f16) -> np.ndarray:
    """x_hat = code * s (fp64)."""
    return np.asarray(codes, np.float64) * np.asarray(scales_f16, dtype=np.float16).astype(np.float64)


def stored_latent(x32, latent_kind: str) -> np.ndarray:
    """Unquantised cache value: the fp32 latent itself or its bf16 rounding (float32 out)."""
    if latent_kind == "f32":
        return np.asarray(x32, dtype=np.float32).copy()
    if latent_kind == "bf16":
        return round_bf16(x32)
    raise ValueError(latent_kind)


# ---------------------------------------------------------------------------
# O6: the cache byte format (as the library header documents it)

def _ceil_to(x: int, m: int) -> int:
    return -(-int(x) // m) * m


@dataclasses.dataclass
class CacheFormat:
    """Byte layout of one layer's cache.

    mix84 key row (one per token): an int8 region of K8 bytes holding, head after
    head, the leading ceil(r_g/4) channels of each head's key latent (two's
    complement), zero-padded to a multiple of 16; then an int4 region of K4/2
    bytes holding, head after head, the remaining channels, two per byte (the
    even-indexed one in the low nibble, two's complement nibbles), zero-padded
    to a multiple of 32 nibbles.
    mix84 value tile (32 tokens): V8 byte-rows, one per int8 channel (zero-padded
    to a multiple of 32 rows), then V4/2 byte-rows, one per pair of int4 channels
    (low nibble = even channel, padded to a multiple of 64 channels); byte t of a
    row is token t of the tile.
    had43 uses the same regions, with the outlier block (ceil(r/5) channels) in
    the int8 region and the inlier block in the int4 region.
    had43p key row: a nibble region of K4/2 bytes holding, head after head, each
    head's outlier channels as two's complement nibbles (low nibble first),
    zero-padded to a multiple of 64 nibbles; then a 3-bit region holding, head
    after head, the inlier channels in groups of 32: a group is three little-endian
    32-bit words P0, P1, P2, where bit j of Pb is bit b of (code + 4) of the
    group's channel j (a field of 1..7; padding channels are 0); the region is
    padded to a multiple of 64 channels and the row to a multiple of 16 bytes.
    had43p value tile: one byte-row per outlier channel pair (low nibble = even
    channel, padded to a multiple of 64 channels), then the inlier channels as a
    byte stream laid over 32-byte rows (stream byte k in row V4/2 + k // 32,
    column k % 32): 12 bytes per channel, three little-endian words P0, P1, P2
    over the tile's 32 tokens, token t at bit 8 (t >> 3) + 4 (t & 1) + ((t >> 1) & 3)
    of each word holding bit b of (code + 4); the stream is padded to a multiple
    of 64 channels and the rows to a multiple of 32.
    f32/bf16: key row = the key latent in channel order, padded to 16 bytes;
    value tile = r_v (padded to a multiple of 32) element-rows of 32 tokens.
    """

    latent: str
    ranks: Tuple[int, ...]
    r_v: int

    @property
    def elem(self) -> int:
        return {"f32": 4, "bf16": 2, "mix84": 1, "had43": 1, "had43p": 1}[self.latent]

    @property
    def quantized(self) -> bool:
        return is_quantized(self.latent)

    @property
    def packed(self) -> bool:
        """Codes at their own widths (had43p): 4-bit nibbles and 3-bit planes."""
        return self.latent == "had43p"

    def split(self, r: int) -> Tuple[int, int]:
        """Channels of a rank-r segment in the int8 region and in the int4 region."""
        return precision_split(r, self.latent)

    # key side
    @property
    def n8(self) -> List[int]:
        return [self.split(r)[0] for r in self.ranks]

    @property
    def n4(self) -> List[int]:
        return [self.split(r)[1] for r in self.ranks]

    @property
    def K8(self) -> int:
        """Byte positions of the int8 region (none when packed)."""
        return 0 if self.packed else _ceil_to(sum(self.n8), 16)

    @property
    def K4(self) -> int:
        """Nibble positions of the 4-bit region: the int4 block, or the packed outlier block."""
        if self.packed:
            return _ceil_to(sum(self.n8), 64)
        return _ceil_to(sum(self.n4), 32)

    @property
    def K3(self) -> int:
        """Channel positions of the packed 3-bit region (0 unless packed)."""
        return _ceil_to(sum(self.n4), 64) if self.packed else 0

    @property
    def k_row_bytes(self) -> int:
        if self.packed:
            return _ceil_to(self.K4 // 2 + 3 * self.K3 // 8, 16)
        if self.quantized:
            return self.K8 + self.K4 // 2
        return _ceil_to(sum(self.ranks) * self.elem, 16)

    # value side
    @property
    def V8(self) -> int:
        return 0 if self.packed else _ceil_to(self.split(self.r_v)[0], 32)

    @property
    def V4(self) -> int:
        """Channels of the nibble-pair rows: the int4 block, or the packed outlier block."""
        return _ceil_to(self.split(self.r_v)[0 if self.packed else 1], 64)

    @property
    def V3(self) -> int:
        """Channels of the packed 3-bit stream (0 unless packed)."""
        return _ceil_to(self.split(self.r_v)[1], 64) if self.packed else 0

    @property
    def v_rows(self) -> int:
        """Rows of a value tile (byte-rows when quantised, element-rows otherwise)."""
        if self.packed:
            return _ceil_to(self.V4 // 2 + 3 * self.V3 // 8, 32)
        if self.quantized:
            return self.V8 + self.V4 // 2
        return _ceil_to(self.r_v, 32)

    @property
    def v_tile_bytes(self) -> int:
        return self.v_rows * TT * self.elem


def token_bit3(t: int) -> int:
    """Bit of token t (0..31) in a packed value plane word: 8 (t >> 3) + 4 (t & 1) + ((t >> 1) & 3)."""
    return 8 * (t >> 3) + 4 * (t & 1) + ((t >> 1) & 3)


def _planes(fields) -> np.ndarray:
    """Bit planes of 3-bit fields [..., 32] -> little-endian words [..., 3] (bit j of word b is
    bit b of field j)."""
    f = np.asarray(fields, dtype=np.uint64)
    w = np.zeros(f.shape[:-1] + (3,), dtype=np.uint64)
    for b in range(3):
        for j in range(32):
            w[..., b] |= ((f[..., j] >> np.uint64(b)) & np.uint64(1)) << np.uint64(j)
    return w.astype(np.uint32)


def _unplanes(words) -> np.ndarray:
    """Inverse of :func:`_planes`: words [..., 3] -> fields [..., 32]."""
    w = np.asarray(words, dtype=np.uint64)
    f = np.zeros(w.shape[:-1] + (32,), dtype=np.int64)
    for b in range(3):
        for j in range(32):
            f[..., j] |= (((w[..., b] >> np.uint64(j)) & np.uint64(1)) << np.uint64(b)).astype(np.int64)
    return f


def _pack_key_rows_packed(vals, fmt: CacheFormat) -> np.ndarray:
    T = vals.shape[0]
    out = np.zeros((T, fmt.k_row_bytes), dtype=np.uint8)
    koff = np.concatenate([[0], np.cumsum(fmt.ranks)])
    nh = [fmt.split(r)[0] for r in fmt.ranks]
    nl = [fmt.split(r)[1] for r in fmt.ranks]
    oh = np.concatenate([[0], np.cumsum(nh)])
    ol = np.concatenate([[0], np.cumsum(nl)])
    fields = np.zeros((T, fmt.K3), dtype=np.int64)  # padding channels: 0
    for g, r in enumerate(fmt.ranks):
        seg = vals[:, koff[g]: koff[g] + r].astype(np.int64)
        for k in range(nh[g]):
            u = oh[g] + k
            out[:, u // 2] |= ((seg[:, k] & 0xF) << (4 * (u % 2))).astype(np.uint8)
        fields[:, ol[g]: ol[g] + nl[g]] = seg[:, nh[g]:] + 4
    words = _planes(fields.reshape(T, fmt.K3 // 32, 32))  # [T, groups, 3]
    b3 = fmt.K4 // 2
    out[:, b3: b3 + 3 * fmt.K3 // 8] = np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(T, -1)
    return out


def _unpack_key_rows_packed(rows, fmt: CacheFormat) -> np.ndarray:
    T = rows.shape[0]
    out = np.zeros((T, sum(fmt.ranks)), dtype=np.int64)
    koff = np.concatenate([[0], np.cumsum(fmt.ranks)])
    nh = [fmt.split(r)[0] for r in fmt.ranks]
    nl = [fmt.split(r)[1] for r in fmt.ranks]
    oh = np.concatenate([[0], np.cumsum(nh)])
    ol = np.concatenate([[0], np.cumsum(nl)])
    b3 = fmt.K4 // 2
    words = np.ascontiguousarray(rows[:, b3: b3 + 3 * fmt.K3 // 8]).view("<u4").reshape(T, fmt.K3 // 32, 3)
    fields = _unplanes(words).reshape(T, fmt.K3)
    for g in range(len(fmt.ranks)):
        for k in range(nh[g]):
            u = oh[g] + k
            nib = (rows[:, u // 2].astype(np.int64) >> (4 * (u % 2))) & 0xF
            out[:, koff[g] + k] = np.where(nib >= 8, nib - 16, nib)
        out[:, koff[g] + nh[g]: koff[g] + nh[g] + nl[g]] = fields[:, ol[g]: ol[g] + nl[g]] - 4
    return out


def _pack_value_tiles_packed(vals, fmt: CacheFormat, n_tiles: int) -> np.ndarray:
    T = vals.shape[0]
    nh, nl = fmt.split(fmt.r_v)
    c = np.zeros((n_tiles * TT, fmt.r_v), dtype=np.int64)
    c[:T] = vals
    out = np.zeros((n_tiles, fmt.v_rows, TT), dtype=np.uint8)
    for k in range(nh):
        nib = (c[:, k] & 0xF).astype(np.uint8).reshape(n_tiles, TT)
        out[:, k // 2, :] |= nib if k % 2 == 0 else (nib << 4)
    # fields [tile, channel, bit position]: token t of the tile at position token_bit3(t);
    # tokens past T and padding channels hold 0
    fields = np.zeros((n_tiles, fmt.V3, 32), dtype=np.int64)
    valid = (np.arange(n_tiles * TT) < T).reshape(n_tiles, TT)
    perm = [token_bit3(t) for t in range(TT)]
    for k in range(nl):
        f = (c[:, nh + k] + 4).reshape(n_tiles, TT)
        fields[:, k, perm] = np.where(valid, f, 0)
    stream = np.ascontiguousarray(_planes(fields).astype("<u4")).view(np.uint8).reshape(n_tiles, -1)
    r3 = fmt.V4 // 2
    flat = out.reshape(n_tiles, -1)
    flat[:, r3 * TT: r3 * TT + stream.shape[1]] = stream
    return out


def _unpack_value_tiles_packed(tiles, fmt: CacheFormat, T: int) -> np.ndarray:
    n_tiles = tiles.shape[0]
    nh, nl = fmt.split(fmt.r_v)
    out = np.zeros((n_tiles * TT, fmt.r_v), dtype=np.int64)
    for k in range(nh):
        nib = (tiles[:, k // 2, :].astype(np.int64) >> (4 * (k % 2))) & 0xF
        out[:, k] = np.where(nib >= 8, nib - 16, nib).reshape(-1)
    r3 = fmt.V4 // 2
    flat = tiles.reshape(n_tiles, -1)
    stream = np.ascontiguousarray(flat[:, r3 * TT: r3 * TT + 12 * fmt.V3])
    fields = _unplanes(stream.view("<u4").reshape(n_tiles, fmt.V3, 3))  # [tile, channel, position]
    perm = [token_bit3(t) for t in range(TT)]
    for k in range(nl):
        out[:, nh + k] = (fields[:, k, perm] - 4).reshape(-1)
    return out[:T]


def pack_key_rows(vals, fmt: CacheFormat) -> np.ndarray:
    """Key latent rows [T, sum(r)] (codes when quantised, values otherwise) -> bytes [T, k_row_bytes]."""
    vals = np.asarray(vals)
    T = vals.shape[0]
    if fmt.packed:
        return _pack_key_rows_packed(vals, fmt)
    out = np.zeros((T, fmt.k_row_bytes), dtype=np.uint8)
    if not fmt.quantized:
        if fmt.latent == "f32":
            raw = np.ascontiguousarray(vals, dtype=np.float32).view(np.uint8).reshape(T, -1)
        else:
            raw = (round_bf16(vals).view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(T, -1)
        out[:, : raw.shape[1]] = raw
        return out
    koff = np.concatenate([[0], np.cumsum(fmt.ranks)])
    o8 = np.concatenate([[0], np.cumsum(fmt.n8)])
    o4 = np.concatenate([[0], np.cumsum(fmt.n4)])
    for g, r in enumerate(fmt.ranks):
        n8, n4 = fmt.n8[g], fmt.n4[g]
        seg = vals[:, koff[g]: koff[g] + r].astype(np.int64)
        out[:, o8[g]: o8[g] + n8] = (seg[:, :n8] & 0xFF).astype(np.uint8)
        for k in range(n4):
            u = o4[g] + k
            nib = (seg[:, n8 + k] & 0xF).astype(np.uint8)
            col = fmt.K8 + u // 2
            out[:, col] |= nib if u % 2 == 0 else (nib << 4)
    return out


def unpack_key_rows(rows, fmt: CacheFormat) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    T = rows.shape[0]
    if fmt.packed:
        return _unpack_key_rows_packed(rows, fmt)
    nk = sum(fmt.ranks)
    if fmt.latent == "f32":
        return rows[:, : nk * 4].copy().view(np.float32).reshape(T, nk)
    if fmt.latent == "bf16":
        b = rows[:, : nk * 2].copy().view(np.uint16).reshape(T, nk)
        return (b.astype(np.uint32) << 16).view(np.float32)
    out = np.zeros((T, nk), dtype=np.int64)
    koff = np.concatenate([[0], np.cumsum(fmt.ranks)])
    o8 = np.concatenate([[0], np.cumsum(fmt.n8)])
    o4 = np.concatenate([[0], np.cumsum(fmt.n4)])
    for g, r in enumerate(fmt.ranks):
        n8, n4 = fmt.n8[g], fmt.n4[g]
        out[:, koff[g]: koff[g] + n8] = rows[:, o8[g]: o8[g] + n8].view(np.int8)
        for k in range(n4):
            u = o4[g] + k
            byte = rows[:, fmt.K8 + u // 2].astype(np.int64)
            nib = (byte >> (4 * (u % 2))) & 0xF
            out[:, koff[g] + n8 + k] = np.where(nib >= 8, nib - 16, nib)
    return out


def pack_value_tiles(vals, fmt: CacheFormat, n_tiles: int) -> np.ndarray:
    """Value latent [T, r_v] -> tiles [n_tiles, v_rows, 32 * elem] (tokens >= T are zero)."""
    vals = np.asarray(vals)
    T = vals.shape[0]
    if fmt.packed:
        return _pack_value_tiles_packed(vals, fmt, n_tiles)
    out = np.zeros((n_tiles, fmt.v_rows, TT * fmt.elem), dtype=np.uint8)
    if not fmt.quantized:
        if fmt.latent == "f32":
            ev = np.zeros((n_tiles * TT, fmt.v_rows), dtype=np.float32)
            ev[:T, : fmt.r_v] = vals
            raw = ev.reshape(n_tiles, TT, fmt.v_rows).transpose(0, 2, 1).copy().view(np.uint8)
        else:
            ev = np.zeros((n_tiles * TT, fmt.v_rows), dtype=np.uint16)
            ev[:T, : fmt.r_v] = (round_bf16(vals).view(np.uint32) >> 16).astype(np.uint16)
            raw = ev.reshape(n_tiles, TT, fmt.v_rows).transpose(0, 2, 1).copy().view(np.uint8)
        return raw.reshape(n_tiles, fmt.v_rows, TT * fmt.elem)
    n8, n4 = fmt.split(fmt.r_v)
    c = np.zeros((n_tiles * TT, fmt.r_v), dtype=np.int64)
    c[:T] = vals
    byrow = np.zeros((n_tiles * TT, fmt.v_rows), dtype=np.uint8)
    byrow[:, :n8] = (c[:, :n8] & 0xFF).astype(np.uint8)
    for k in range(n4):
        nib = (c[:, n8 + k] & 0xF).astype(np.uint8)
        byrow[:, fmt.V8 + k // 2] |= nib if k % 2 == 0 else (nib << 4)
    return byrow.reshape(n_tiles, TT, fmt.v_rows).transpose(0, 2, 1).copy()


def unpack_value_tiles(tiles, fmt: CacheFormat, T: int) -> np.ndarray:
    tiles = np.asarray(tiles, dtype=np.uint8)
    n_tiles = tiles.shape[0]
    if fmt.packed:
        return _unpack_value_tiles_packed(tiles, fmt, T)
    if fmt.latent == "f32":
        v = tiles.copy().view(np.float32).reshape(n_tiles, fmt.v_rows, TT)
        return v.transpose(0, 2, 1).reshape(n_tiles * TT, fmt.v_rows)[:T, : fmt.r_v].copy()
    if fmt.latent == "bf16":
        v = tiles.copy().view(np.uint16).reshape(n_tiles, fmt.v_rows, TT)
        v = v.transpose(0, 2, 1).reshape(n_tiles * TT, fmt.v_rows)[:T, : fmt.r_v]
        return (v.astype(np.uint32) << 16).view(np.float32)
    n8, n4 = fmt.split(fmt.r_v)
    by = tiles.transpose(0, 2, 1).reshape(n_tiles * TT, fmt.v_rows)[:T]
    out = np.zeros((T, fmt.r_v), dtype=np.int64)
    out[:, :n8] = by[:, :n8].view(np.int8)
    for k in range(n4):
        nib = (by[:, fmt.V8 + k // 2].astype(np.int64) >> (4 * (k % 2))) & 0xF
        out[:, n8 + k] = np.where(nib >= 8, nib - 16, nib)
    return out


# ---------------------------------------------------------------------------
# O7: reconstruct dense K and V from the (dequantised) latent

def reconstruct(xk_hat, xv_hat, layer: Layer) -> Tuple[np.ndarray, np.ndarray]:
    """K_g = L_g B_g (head-wise), V = C_v B_v (joint) -> both [T, H_kv, d_h] fp64."""
    xk_hat = np.asarray(xk_hat, np.float64)
    T = xk_hat.shape[0]
    K = np.zeros((T, layer.H_kv, layer.d_h))
    off = layer.key_offsets
    Bk = np.asarray(layer.B_k, np.float64)
    for g in range(layer.H_kv):
        K[:, g, :] = xk_hat[:, off[g]: off[g + 1]] @ Bk[off[g]: off[g + 1]]
    V = (np.asarray(xv_hat, np.float64) @ np.asarray(layer.B_v, np.float64)).reshape(T, layer.H_kv, layer.d_h)
    return K, V


# ---------------------------------------------------------------------------
# O8: dense attention of the decode queries over the reconstructed cache

def attention(q, K, V, n_q: int) -> np.ndarray:
    """q [n_q, H_q, d_h]; K, V [T, H_kv, d_h]; causal over the last n_q positions.

    Query j sits at position T - n_q + j and sees positions <= that; query head h
    reads KV head h // (H_q / H_kv); scores are scaled by 1/sqrt(d_h).
    """
    q = np.asarray(q, np.float64)
    T, H_kv, d_h = K.shape
    H_q = q.shape[1]
    G = H_q // H_kv
    out = np.zeros((n_q, H_q, d_h))
    for j in range(n_q):
        pos = T - n_q + j
        for h in range(H_q):
            g = h // G
            s = (K[: pos + 1, g, :] @ q[j, h]) / math.sqrt(d_h)
            p = np.exp(s - np.max(s))
            out[j, h] = (p @ V[: pos + 1, g, :]) / np.sum(p)
    return out


# ---------------------------------------------------------------------------
# Rotary position embedding of the reconstructed keys and of the queries.  The pages evaluate
# Llama-family models, whose attention rotates keys and queries by their positions after the
# key projection; a latent cache then holds the keys before the rotation, which the attention
# applies to each reconstructed key (Problem Statement: the reconstruction cost; Methodology
# section 2: head-wise key factors keep it per head).

def rope(x, positions, theta: float, rotary_dim: int) -> np.ndarray:
    """x [T, ..., d] at integer positions [T] (fp64): for i < rotary_dim / 2 the pair
    (x[..., i], x[..., i + rotary_dim / 2]) is rotated by the angle
    positions[t] * theta^(-2 i / rotary_dim); dimensions from rotary_dim on are unchanged."""
    x = np.asarray(x, np.float64)
    half = rotary_dim // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / rotary_dim)
    ang = np.asarray(positions, np.float64)[:, None] * inv[None, :]  # [T, half]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, sn = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    out = x.copy()
    a, b = x[..., :half], x[..., half:rotary_dim]
    out[..., :half] = a * c - b * sn
    out[..., half:rotary_dim] = a * sn + b * c
    return out


# ---------------------------------------------------------------------------
# O9: the same attention computed in the latent space (operations reordered)

def attention_latent(q, xk_hat, xv_hat, layer: Layer, n_q: int) -> np.ndarray:
    """q is projected into each key head's latent (q B_g^T), scored against the latent
    keys; the probabilities weight the joint value latent, which is then up-projected
    per head with the head's slice of B_v."""
    q = np.asarray(q, np.float64)
    xk_hat = np.asarray(xk_hat, np.float64)
    xv_hat = np.asarray(xv_hat, np.float64)
    T = xk_hat.shape[0]
    G = layer.H_q // layer.H_kv
    off = layer.key_offsets
    Bk = np.asarray(layer.B_k, np.float64)
    Bv = np.asarray(layer.B_v, np.float64)
    d_h = layer.d_h
    out = np.zeros((n_q, layer.H_q, d_h))
    for j in range(n_q):
        pos = T - n_q + j
        for h in range(layer.H_q):
            g = h // G
            qt = Bk[off[g]: off[g + 1]] @ q[j, h]
            s = (xk_hat[: pos + 1, off[g]: off[g + 1]] @ qt) / math.sqrt(d_h)
            p = np.exp(s - np.max(s))
            z = p @ xv_hat[: pos + 1]
            out[j, h] = (z @ Bv[:, g * d_h: (g + 1) * d_h]) / np.sum(p)
    return out


# ---------------------------------------------------------------------------
# split-K over the context: partial softmax states and their log-sum-exp merge

def partial_state(s, values) -> Tuple[float, float, np.ndarray]:
    """(max, sum of exp(s - max), sum of exp(s - max) * values) over one token range."""
    s = np.asarray(s, np.float64)
    m = float(np.max(s))
    e = np.exp(s - m)
    return m, float(np.sum(e)), e @ np.asarray(values, np.float64)


def lse_merge(parts: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Merge partial states: m = max m_i, l = sum e^(m_i - m) l_i, acc likewise; -> acc / l."""
    m = max(p[0] for p in parts)
    l = sum(math.exp(p[0] - m) * p[1] for p in parts)
    acc = sum(math.exp(p[0] - m) * p[2] for p in parts)
    return acc / l


# ---------------------------------------------------------------------------
# the whole path for one sequence

@dataclasses.dataclass
class SequenceCache:
    """The oracle's cache of one sequence: integer codes (mix84, had43, had43p) or stored values."""

    key: np.ndarray  # [T, sum(r)]
    value: np.ndarray  # [T, r_v]


def compress(X, layer: Layer, scales=None) -> SequenceCache:
    """Project hidden states X [T, d] into the latent and quantise / round it."""
    x = latent(X, layer.A_cat)
    nk = layer.n_key
    if is_quantized(layer.latent):
        codes = quantize(x, scales, channel_qmax(layer))
        return SequenceCache(codes[:, :nk], codes[:, nk:])
    v = stored_latent(x, layer.latent)
    return SequenceCache(v[:, :nk], v[:, nk:])


def dequantized(cache: SequenceCache, layer: Layer, scales=None) -> Tuple[np.ndarray, np.ndarray]:
    nk = layer.n_key
    if is_quantized(layer.latent):
        s = np.asarray(scales, dtype=np.float16)
        return dequantize(cache.key, s[:nk]), dequantize(cache.value, s[nk:])
    return np.asarray(cache.key, np.float64), np.asarray(cache.value, np.float64)


def query_from_hidden(x, W_q, H_q: int, d_h: int) -> np.ndarray:
    """Queries of hidden states x [n_q, d] through the query projection W_q [d, H_q d_h]:
    q[j, h] = x[j] W_q[:, h d_h:(h + 1) d_h], in fp64 (the product the absorbed factors
    W_q^h B_g^T fold into the key latent; Methodology section 2)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W_q, np.float64)
    return (x @ W).reshape(x.shape[0], H_q, d_h)


def decode(q, cache: SequenceCache, layer: Layer, n_q: int, scales=None, mode: str = "reconstruct",
           rope_theta: float = 0.0, rotary_dim: int = 0) -> np.ndarray:
    """Decode attention of one sequence; ``mode`` = "reconstruct" (O7 + O8) or "latent" (O9).
    With ``rope_theta`` > 0 the reconstructed keys (position t) and the queries (position
    T - n_q + j) are rotated first; the latent order does not apply then (the rotation depends
    on the position, so B_g cannot move past it)."""
    xk, xv = dequantized(cache, layer, scales)
    if rope_theta > 0:
        if mode != "reconstruct":
            raise ValueError("rotary keys need the reconstruct order")
        K, V = reconstruct(xk, xv, layer)
        T = K.shape[0]
        K = rope(K, np.arange(T), rope_theta, rotary_dim)
        q = rope(np.asarray(q, np.float64), np.arange(T - n_q, T), rope_theta, rotary_dim)
        return attention(q, K, V, n_q)
    if mode == "latent":
        return attention_latent(q, xk, xv, layer, n_q)
    K, V = reconstruct(xk, xv, layer)
    return attention(q, K, V, n_q)
