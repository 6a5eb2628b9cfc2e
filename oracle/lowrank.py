"""Low-rank anchor storage (KVCMAS, "what differs": base caches and delta
corrections kept as truncated SVDs, Z ~ U_r S_r R_r^T = A R^T, rank r = 32 and
V = 10 anchors per slot by default; "how it is used": the correction for a
target is a weighted sum of the stored low-rank factors, added to the aligned
source cache to materialise the full-width target cache).

TEST INFRASTRUCTURE, like the rest of this package (see oracle/__init__.py).

A matrix Z here is one layer's K or V of one cache: T rows (tokens) by H*d
columns (heads x channels), read from the cache layout [H][T][d]. Factors
are stored as bf16, both row-major: A = U_r S_r (T x r) and R = R_r
(H*d x r), so that Z ~ A R^T. Everything is computed in binary64 (numpy's
SVD, a library primitive, for the factorisation) and rounded once to bf16
where a bf16 is stored.
"""

import numpy as np

from . import f64_to_bf16


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 (exact: the bits become the top half)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x):
    """binary64 array -> bf16 bits, each value rounded once to nearest, ties
    to even. In the bf16 normal range the binary64 significand is cut at its
    7th fraction bit by integer arithmetic (a carry into the exponent is the
    correct result); other values (zero, subnormal, beyond the range) go
    through the scalar routine."""
    x = np.ascontiguousarray(x, np.float64)
    u = x.view(np.uint64)
    e = (u >> np.uint64(52)) & np.uint64(0x7FF)
    normal = (e >= np.uint64(1023 - 126)) & (e < np.uint64(1023 + 128))
    low = u & np.uint64((1 << 45) - 1)
    keep = u >> np.uint64(45)
    half = np.uint64(1 << 44)
    up = (low > half) | ((low == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    y = ((keep + up.astype(np.uint64)) << np.uint64(45)).view(np.float64)
    with np.errstate(over="ignore"):
        out = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    for i in np.flatnonzero(~normal):
        out.flat[i] = f64_to_bf16(float(x.flat[i]))
    return out


def as_matrix(cache_layer):
    """[H][T][d] bf16 bits -> T x (H*d) matrix view (copy), column h*d + c."""
    H, T, d = cache_layer.shape
    return np.ascontiguousarray(np.transpose(cache_layer, (1, 0, 2)).reshape(T, H * d))


def from_matrix(m, H, d):
    T = m.shape[0]
    return np.ascontiguousarray(np.transpose(m.reshape(T, H, d), (1, 0, 2)))


def factor(z_bits, r):
    """Truncated SVD of the T x D matrix z (bf16 bits): returns (A, R) bf16
    bits, A = U_r S_r (T x r), R = R_r (D x r), and the singular values."""
    z = bf16_bits_to_f32(z_bits).astype(np.float64)
    u, s, vt = np.linalg.svd(z, full_matrices=False)
    a = u[:, :r] * s[:r]
    rr = vt[:r, :].T
    return round_bf16(a), round_bf16(rr), s


def materialize(src_bits, a_bits, r_bits, w):
    """bf16(src + sum_v w_v A_v R_v^T) for src T x D, A [V][T][r],
    R [V][D][r], w [V] (binary32 weights), in binary64, rounded once."""
    src = bf16_bits_to_f32(src_bits).astype(np.float64)
    acc = src.copy()
    for v in range(len(w)):
        av = bf16_bits_to_f32(a_bits[v]).astype(np.float64)
        rv = bf16_bits_to_f32(r_bits[v]).astype(np.float64)
        acc += float(np.float32(w[v])) * (av @ rv.T)
    return round_bf16(acc)


def materialize_cache(src, a, r, w):
    """The whole cache: src bf16 bits [L][H][T][d] (one of K or V), factors
    A [L][V][T][r] and R [L][V][H*d][r], weights [L][V]; per layer the
    matrix view materialised, back in the cache layout."""
    L, H, T, d = src.shape
    out = np.empty_like(src)
    for l in range(L):
        out[l] = from_matrix(materialize(as_matrix(src[l]), a[l], r[l], w[l]), H, d)
    return out
