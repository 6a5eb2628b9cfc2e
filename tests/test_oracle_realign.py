"""Pins of the key re-alignment oracle (KVCMAS procedure: key positions of a
shared segment re-aligned to the target's; QKVShare item 2: the card
carries the source position offset). Rotary keys at position p hold channel
pair j rotated by p * f_j; re-aligning by delta rotates each pair by
delta * f_j more. Checked against complex multiplication, the group
property of rotations, the shift invariance that rotary positions exist
for, the relation between the two pairings, and the identities at zero."""

import numpy as np
import pytest

import oracle
from agent_handoff_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits


def _ulp(x):
    """bf16 ulp at each value of x (leading-bit weight / 2^7, normal range)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - 1, -126) - 7)


def _freqs(d, base=500000.0):
    return (base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)).astype(np.float32)


def _keys(shape, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits((rng.standard_normal(shape) * np.exp(rng.standard_normal(shape[-1]))).astype(np.float32))


@pytest.mark.parametrize("pairing", [0, 1])
def test_zero_shift_and_zero_frequency_are_identities(pairing):
    k = _keys((2, 2, 9, 64), 0)
    assert np.array_equal(oracle.realign_keys(k, 0, _freqs(64), pairing), k)
    assert np.array_equal(oracle.realign_keys(k, 123457, np.zeros(32, np.float32), pairing), k)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_equals_complex_multiplication(d):
    """Pair (j, j + d/2) as the complex number a + ib, times exp(i delta f_j)."""
    k = _keys((1, 3, 40, d), 1)
    f = _freqs(d)
    for delta in (1, -7, 4096, 2 ** 31 + 5):
        got = oracle.realign_keys(k, delta, f, 0)
        x = bf16_bits_to_f32(k).astype(np.float64)
        z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * (float(delta) * f.astype(np.float64)))
        want = np.concatenate([z.real, z.imag], axis=-1)
        g = bf16_bits_to_f32(got).astype(np.float64)
        ulp = _ulp(want)
        assert np.all(np.abs(g - want) <= 0.5 * ulp * (1 + 1e-6) + 1e-300), delta


def test_shifts_compose():
    k = _keys((1, 2, 30, 128), 2)
    f = _freqs(128)
    two = oracle.realign_keys(oracle.realign_keys(k, 300, f), -1200, f)
    one = oracle.realign_keys(k, -900, f)
    a, b = bf16_bits_to_f32(two).astype(np.float64), bf16_bits_to_f32(one).astype(np.float64)
    x = bf16_bits_to_f32(k).astype(np.float64)
    mag = np.sqrt(x[..., :64] ** 2 + x[..., 64:] ** 2)
    mag = np.concatenate([mag, mag], axis=-1)
    assert np.all(np.abs(a - b) <= 2 ** -6 * mag + 1e-30)


def test_dot_products_are_shift_invariant():
    """What rotary positions are for: moving queries and keys by the same
    delta leaves every query-key dot product unchanged."""
    d = 128
    q = _keys((1, 1, 16, d), 3)
    k = _keys((1, 1, 16, d), 4)
    f = _freqs(d)
    qs, ks = oracle.realign_keys(q, 777, f), oracle.realign_keys(k, 777, f)
    Q, K = bf16_bits_to_f32(q[0, 0]).astype(np.float64), bf16_bits_to_f32(k[0, 0]).astype(np.float64)
    Qs, Ks = bf16_bits_to_f32(qs[0, 0]).astype(np.float64), bf16_bits_to_f32(ks[0, 0]).astype(np.float64)
    scale = np.outer(np.linalg.norm(Q, axis=1), np.linalg.norm(K, axis=1))
    assert np.all(np.abs(Qs @ Ks.T - Q @ K.T) <= 2 ** -6 * scale)


def test_adjacent_pairing_is_the_halves_pairing_permuted():
    d = 64
    k = _keys((2, 1, 11, d), 5)
    f = _freqs(d)
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2           # adjacent position 2j holds halves channel j, 2j+1 holds j+d/2
    adj = np.ascontiguousarray(k[..., perm])
    got = oracle.realign_keys(adj, 55, f, 1)
    want = oracle.realign_keys(k, 55, f, 0)[..., perm]
    assert np.array_equal(got, want)
