"""Counter-based random numbers and samplers for the synthetic DLRM inputs.

Nothing here computes any step of the recommendation model: these are the
seeded input generators that the GPU path and the CPU oracle both consume.

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the n-th output of a generator whose state starts
  at ``s`` is ``fmix(s + n * GAMMA)``.  Embedding-table values use it as a
  counter-based generator so that the GPU can fill 200 GB of tables in place
  while the host regenerates only the rows a test touches.
* A keyed Feistel bijection with cycle walking (Black & Rogaway, "Ciphers with
  arbitrary finite domains", CT-RSA 2002) maps Zipf ranks to rows, so the hot
  rows land at scattered addresses without materialising a permutation.
* Truncated Zipf by inverse transform over the exact cumulative table.
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def fmix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def fmix_int(z: int) -> int:
    """Scalar SplitMix64 output function on a Python int (mod 2**64)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def splitmix64_stream(state: int, count: int) -> np.ndarray:
    """First ``count`` outputs of a SplitMix64 generator seeded with ``state``."""
    n = np.arange(1, count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return fmix(np.uint64(state & _MASK64) + n * GAMMA)


def table_key(seed: int, table: int) -> int:
    """Per-table SplitMix64 state for the embedding-table value stream."""
    base = fmix_int((seed + int(GAMMA)) & _MASK64)
    return fmix_int((base + (table + 1) * int(GAMMA)) & _MASK64)


def table_scale(rows: int) -> np.float32:
    """Half-width a_k of the uniform table init U(-a_k, a_k), a_k = 1/sqrt(m_k)."""
    return np.float32(1.0 / math.sqrt(float(rows)))


def table_rows(seed: int, table: int, rows: int, row_ids: np.ndarray, d: int) -> np.ndarray:
    """Values of the listed rows of table ``table`` (``rows`` rows of width ``d``).

    Element (r, c) is ``a * (2u - 1)`` with ``u = (h >> 40) * 2**-24`` and
    ``h`` the ``(r*d + c + 1)``-th SplitMix64 output of the table's state.
    ``2u - 1`` is exact in fp32, so the product with ``a`` is the only
    rounding; the device fill computes the same value bit for bit.
    """
    row_ids = np.asarray(row_ids, dtype=np.int64)
    key = np.uint64(table_key(seed, table))
    e = (row_ids[:, None] * d + np.arange(d, dtype=np.int64)[None, :]).astype(np.uint64)
    with np.errstate(over="ignore"):
        h = fmix(key + (e + np.uint64(1)) * GAMMA)
    top = (h >> np.uint64(40)).astype(np.int64)  # 24 random bits
    t = (top * 2 - (1 << 24)).astype(np.float32) * np.float32(2.0 ** -24)
    return (table_scale(rows) * t).astype(np.float32)


def table_rows_bf16(seed: int, table: int, rows: int, row_ids: np.ndarray, d: int) -> np.ndarray:
    """bf16 table rows (uint16 bit patterns): the high half of each fp32
    value of ``table_rows``."""
    return (table_rows(seed, table, rows, row_ids, d).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def scale_bias_key(seed: int, table: int) -> int:
    """State of the per-row (scale, bias) stream of an int8 table."""
    return fmix_int(table_key(seed, table) ^ 0xD6E8FEB86659FD93)


def table_rows_i8(seed: int, table: int, rows: int, row_ids: np.ndarray, d: int):
    """int8 table rows and their fp32 (scale, bias) pairs.

    q(r, c) is the top byte, as a signed value, of output ``r*d + c + 1`` of
    the table's state.  Row r's scale is ``a * ((0.5 + u1) * 2**-7)`` and its
    bias ``a * ((2 u2 - 1) * 2**-3)``, u1 = (h1 >> 41) 2**-23 and
    u2 = (h2 >> 40) 2**-24 from outputs 2r + 1 and 2r + 2 of the row-parameter
    state: the factors after ``a`` are exact, so each is one fp32 rounding,
    as in the device fill.
    """
    row_ids = np.asarray(row_ids, dtype=np.int64)
    key = np.uint64(table_key(seed, table))
    e = (row_ids[:, None] * d + np.arange(d, dtype=np.int64)[None, :]).astype(np.uint64)
    with np.errstate(over="ignore"):
        h = fmix(key + (e + np.uint64(1)) * GAMMA)
    q = (h >> np.uint64(56)).astype(np.uint8).view(np.int8)
    k2 = np.uint64(scale_bias_key(seed, table))
    r = row_ids.astype(np.uint64)
    with np.errstate(over="ignore"):
        h1 = fmix(k2 + (np.uint64(2) * r + np.uint64(1)) * GAMMA)
        h2 = fmix(k2 + (np.uint64(2) * r + np.uint64(2)) * GAMMA)
    u1 = (h1 >> np.uint64(41)).astype(np.float32) * np.float32(2.0 ** -23)
    f1 = (np.float32(0.5) + u1) * np.float32(2.0 ** -7)
    top = (h2 >> np.uint64(40)).astype(np.int64)
    f2 = (top * 2 - (1 << 24)).astype(np.float32) * np.float32(2.0 ** -27)
    a = table_scale(rows)
    sb = np.stack([a * f1, a * f2], axis=1).astype(np.float32)
    return np.ascontiguousarray(q), sb


class FeistelPermutation:
    """Seeded bijection of [0, m) built from a 4-round balanced Feistel network
    on the smallest even bit width covering m, with cycle walking."""

    ROUNDS = 4

    def __init__(self, m: int, key: int):
        if m < 1:
            raise ValueError("empty domain")
        self.m = int(m)
        bits = max(2, int(math.ceil(math.log2(max(m, 2)))))
        bits += bits & 1
        self.half = bits // 2
        self.mask = np.uint64((1 << self.half) - 1)
        self.keys = [np.uint64(fmix_int(key + (i + 1) * int(GAMMA))) for i in range(self.ROUNDS)]

    def _network(self, x: np.ndarray) -> np.ndarray:
        half = np.uint64(self.half)
        left = x >> half
        right = x & self.mask
        for k in self.keys:
            with np.errstate(over="ignore"):
                f = fmix(right + k) & self.mask
            left, right = right, left ^ f
        return (left << half) | right

    def __call__(self, x) -> np.ndarray:
        y = self._network(np.asarray(x, dtype=np.uint64))
        m = np.uint64(self.m)
        bad = y >= m
        while bad.any():
            y[bad] = self._network(y[bad])
            bad = y >= m
        return y.astype(np.int64)


_ZIPF_CDF_CACHE: dict = {}


def zipf_cdf(m: int, alpha: float) -> np.ndarray:
    """Cumulative distribution of P(k) proportional to k**-alpha on k = 1..m."""
    key = (int(m), float(alpha))
    cdf = _ZIPF_CDF_CACHE.get(key)
    if cdf is None:
        w = np.arange(1, m + 1, dtype=np.float64)
        np.power(w, -alpha, out=w)
        np.cumsum(w, out=w)
        w /= w[-1]
        if sum(c.size for c in _ZIPF_CDF_CACHE.values()) + m > 3e8:
            _ZIPF_CDF_CACHE.clear()
        _ZIPF_CDF_CACHE[key] = cdf = w
    return cdf


def zipf_ranks(rng: np.random.Generator, m: int, alpha: float, size: int) -> np.ndarray:
    """Zero-based Zipf ranks (0 is the most frequent) by inverse transform."""
    cdf = zipf_cdf(m, alpha)
    u = rng.random(size)
    r = np.searchsorted(cdf, u, side="right")
    return np.minimum(r, m - 1).astype(np.int64)


def stream_rng(master: int, *stream) -> np.random.Generator:
    """Independent numpy PCG64 stream for (master seed, stream id...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(master), *map(int, stream)])))
