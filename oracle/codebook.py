"""Lloyd-Max codebook for the standard normal density (3 bits, 8 levels).

TEST INFRASTRUCTURE. This module belongs to the CPU oracle: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it. The
GPU library carries its own constants and is checked against this derivation.

What it follows: PolyKV (gist.science/ko/paper/2604.24971), section 2.B,
item 2 ("TurboQuant MSE"): after the Walsh-Hadamard rotation the coordinates
are close to N(0,1), and each is mapped to the nearest of a precomputed set of
Lloyd-Max centroids optimised for N(0,1). The pages give neither the number
nor the values of the centroids beyond "3 bits"; the levels are derived here
from the density by Lloyd's iteration, in float64:

  * boundaries are the midpoints of neighbouring levels;
  * each level is the conditional mean of N(0,1) over its cell,
        c_k = (phi(b_k) - phi(b_{k+1})) / (Phi(b_{k+1}) - Phi(b_k)),
    with the tail probabilities taken from erfc so the outer cells keep full
    relative precision.

Codec table (a reading of ours, stated in the design notes): the stored
levels are the converged levels rounded to the nearest multiple of 2**-15, and
the decision thresholds are the exact midpoints of neighbouring stored levels
(multiples of 2**-16, hence exact in float32). On that grid the inverse
transform of any code vector of length <= 128 is exact in float32, and the
encoder's threshold rule is exactly nearest-level for the stored table.
"""

import math

GRID_BITS = 15          # stored levels are integers / 2**GRID_BITS
LEVELS = 8


def _phi(x):
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper_tail(x):
    """P(X >= x) for X ~ N(0,1), accurate in both tails."""
    if x == math.inf:
        return 0.0
    if x == -math.inf:
        return 1.0
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def cell_probability(lo, hi):
    """P(lo <= X < hi) for X ~ N(0,1)."""
    if lo >= 0.0:
        return _upper_tail(lo) - _upper_tail(hi)
    if hi <= 0.0:
        return _upper_tail(-hi) - _upper_tail(-lo)
    return 1.0 - _upper_tail(hi) - _upper_tail(-lo)


def cell_mean(lo, hi):
    """E[X | lo <= X < hi] for X ~ N(0,1)."""
    return (_phi(lo) - _phi(hi)) / cell_probability(lo, hi)


def boundaries_of(levels):
    """Decision boundaries b_1..b_{n-1}: midpoints of neighbouring levels."""
    return [0.5 * (levels[i] + levels[i + 1]) for i in range(len(levels) - 1)]


def lloyd_max_gaussian(n=LEVELS, tol=1e-14, max_iter=100000):
    """Lloyd's iteration on the N(0,1) density.

    Returns (levels, boundaries, iterations); levels ascending, float64.
    """
    # symmetric, evenly spread start
    levels = [(-1.0 + (2.0 * i + 1.0) / n) * 2.0 for i in range(n)]
    for it in range(1, max_iter + 1):
        b = boundaries_of(levels)
        edges = [-math.inf] + b + [math.inf]
        new = [cell_mean(edges[i], edges[i + 1]) for i in range(n)]
        delta = max(abs(a - c) for a, c in zip(new, levels))
        levels = new
        if delta < tol:
            return levels, boundaries_of(levels), it
    raise RuntimeError("Lloyd iteration did not converge")


def distortion(levels, boundaries):
    """Mean squared error E[(X - Q(X))^2] of the quantiser on N(0,1).

    Uses E[X^2 1{cell}] = P - x phi(x) |_lo^hi for the second moment.
    """
    edges = [-math.inf] + list(boundaries) + [math.inf]
    total = 0.0
    for k, c in enumerate(levels):
        lo, hi = edges[k], edges[k + 1]
        p = cell_probability(lo, hi)
        m1 = _phi(lo) - _phi(hi)
        xlo = 0.0 if math.isinf(lo) else lo * _phi(lo)
        xhi = 0.0 if math.isinf(hi) else hi * _phi(hi)
        m2 = p + xlo - xhi
        total += m2 - 2.0 * c * m1 + c * c * p
    return total


def codec_table():
    """The table the codec uses: (levels, thresholds), both exact float32 values.

    levels: 8 ascending values, each an integer multiple of 2**-15.
    thresholds: 7 ascending midpoints of neighbouring levels.
    """
    levels, _, _ = lloyd_max_gaussian()
    q = [round(c * (1 << GRID_BITS)) / float(1 << GRID_BITS) for c in levels]
    return q, boundaries_of(q)


def codec_table_integers():
    """Stored levels as integers in units of 2**-15 (ascending)."""
    q, _ = codec_table()
    return [int(round(c * (1 << GRID_BITS))) for c in q]
