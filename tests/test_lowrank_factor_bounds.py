"""Where the factorisation's parity bounds come from: a float64 mirror of the
randomized truncated SVD that kvc_lowrank_factor computes (range finder on a
48-column Gaussian sketch, one power iteration, CholeskyQR with dependent
columns dropped, Rayleigh-Ritz through the eigenvectors of the projected
Gram matrix; Halko, Martinsson and Tropp 2011), with its factors stored as
bf16, run on the inputs of the GPU tests and held to the bounds those tests
use:
  - residual ||Z - A R^T||_F <= 1.02 x the optimal rank-32 residual;
  - where sigma_32 / sigma_33 >= 3: singular values within 2e-3 sigma_1,
    ||A R^T - A_o R_o^T||_F <= 2^-6 ||A_o R_o^T||_F, R orthonormal within 2^-5.
Where the spectrum has a gap the mirror reaches each with room to spare
(checked below against tighter bounds), so most of each bound is left for
the GPU's binary32 products and binary64 small-matrix work; without a gap
the residual ratio is the sketch's own approximation (about 1.013 here),
and 1.02 adds a small margin to it. The reference is the oracle's exact SVD
(numpy, binary64)."""

import numpy as np
import pytest

from agent_handoff_amd import synth
from oracle import lowrank

SKETCH = 48


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def cholesky_qr(Y, drop=1e-12):
    """Q with orthonormal (or zero) columns spanning Y's, by Cholesky of the
    Gram matrix; a pivot at most drop x the largest diagonal entry drops its
    column (Q's column zero), so rank-deficient inputs give no NaNs."""
    G = Y.T @ Y
    n = G.shape[0]
    Lm = np.zeros_like(G)
    keep = np.zeros(n, bool)
    top = max(float(np.max(np.diag(G))), 0.0)
    for j in range(n):
        piv = G[j, j] - np.dot(Lm[j, :j], Lm[j, :j])
        if top == 0.0 or piv <= drop * top:
            continue
        keep[j] = True
        Lm[j, j] = np.sqrt(piv)
        for i in range(j + 1, n):
            Lm[i, j] = (G[i, j] - np.dot(Lm[i, :j], Lm[j, :j])) / Lm[j, j]
    Q = np.zeros_like(Y)
    idx = np.flatnonzero(keep)
    if idx.size:
        Rk = Lm[np.ix_(idx, idx)].T       # upper triangular on the kept columns
        Q[:, idx] = Y[:, idx] @ np.linalg.inv(Rk)
    return Q


def randomized_svd(Z, omega, r=32):
    Q = cholesky_qr(Z @ omega)
    W = cholesky_qr(Z.T @ Q)
    Q = cholesky_qr(Z @ W)
    W = Z.T @ Q                           # B^T with B = Q^T Z
    lam, U = np.linalg.eigh(W.T @ W)
    order = np.argsort(lam)[::-1][:r]
    lam, U = np.maximum(lam[order], 0.0), U[:, order]
    s = np.sqrt(lam)
    inv = np.where(s > 0, 1.0 / np.where(s > 0, s, 1.0), 0.0)
    A = (Q @ U) * s
    R = (W @ U) * inv
    return lowrank.round_bf16(A), lowrank.round_bf16(R), s


@pytest.mark.parametrize("shape,rank,noise,gapped", [
    ((2, 3, 300, 128), 32, 0.01, True),
    ((1, 2, 1000, 64), 20, 0.01, False),
    ((3, 1, 50, 128), 32, 0.005, True),
    ((1, 2, 40, 128), 32, 0.02, False),
    ((2, 8, 512, 128), 32, 0.01, True),
])
def test_mirror_meets_the_gpu_bounds_with_room(shape, rank, noise, gapped):
    z = synth.lowrank_caches(3, 8, *shape, rank=rank, noise=noise)
    omega = synth.sketch(0, 7, shape[1] * shape[3]).astype(np.float64)
    for l in range(shape[0]):
        zm = lowrank.as_matrix(z[l])
        Z = _f(zm)
        a_o, r_o, s_o = lowrank.factor(zm, 32)
        a_m, r_m, s_m = randomized_svd(Z, omega)
        Pm, Po = _f(a_m) @ _f(r_m).T, _f(a_o) @ _f(r_o).T
        em, eo = np.linalg.norm(Z - Pm), np.linalg.norm(Z - Po)
        # The bound is 1.02. With a gap at 32 the mirror stays within 1.005
        # (room for the GPU's rounding); without one the sketch's own
        # approximation sets the ratio (about 1.013 on the rank-20 input),
        # and 1.02 is that plus a margin.
        assert em <= (1.005 if gapped else 1.016) * eo, (shape, l, em / eo)
        assert np.all(np.diff(s_m) <= 1e-12 * s_m[0])
        if gapped:
            assert s_o[31] / s_o[32] >= 3
            # bounds 2e-3 sigma_1, 2^-6 and 2^-5; the mirror within a quarter
            assert np.max(np.abs(s_m - s_o[:32])) <= 5e-4 * s_o[0], (shape, l)
            assert np.linalg.norm(Pm - Po) <= 2.0 ** -8 * np.linalg.norm(Po), (shape, l)
            Rm = _f(r_m)
            assert np.max(np.abs(Rm.T @ Rm - np.eye(32))) <= 2.0 ** -7, (shape, l)


def test_bf16_storage_alone_explains_the_product_bound():
    """The exact factors rounded to bf16 (each entry within 2^-9 relative)
    already move A R^T by about 2^-9 of its norm: the 2^-6 bound leaves a
    factor 8 for the randomized approximation and the GPU's arithmetic."""
    z = synth.lowrank_caches(3, 8, 1, 8, 512, 128, rank=32, noise=0.01)
    Z = _f(lowrank.as_matrix(z[0]))
    u, s, vt = np.linalg.svd(Z, full_matrices=False)
    P = (u[:, :32] * s[:32]) @ vt[:32]
    a, r, _ = lowrank.factor(lowrank.as_matrix(z[0]), 32)
    rel = np.linalg.norm(_f(a) @ _f(r).T - P) / np.linalg.norm(P)
    assert 2.0 ** -12 < rel < 2.0 ** -8
