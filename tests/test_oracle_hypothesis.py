"""The CPU oracle on random tiny shapes and value mixes (hypothesis draws
them) against the brute-force references of tests/brute.py and the
properties any correct encoder has:

- keys: per-layer int8 codes equal float64 rint(x * 127 / m) away from a
  half-integer; the scale is m / 127;
- values: fp16 RMS scales and 3-bit codes equal the float64 pipeline
  (scipy's dense Hadamard matrix, nearest level) away from a decision
  boundary; the code section unpacks with numpy to the same codes; the
  decode is within half a bf16 ulp of the float64 reconstruction;
- CacheCard (groups whose step is a normal fp16 number): width 16 is the
  identity, each group's minimum decodes to
  itself, the group maximum gets the top code, every value is within half a
  step plus half a bf16 ulp of its input.

Value mixes include exact key ties (integers and halves at scale 1), zero
vectors, signed zeros, outlier channels and a wide dynamic range."""

import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from agent_handoff_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
from brute import (bf16_ulp, card_record_size, k_codes_brute, unpack_v_codes, v_codes_brute,
                   v_decode_brute)
from oracle import codebook

LEVELS, THRESH = codebook.codec_table()

shapes = st.tuples(st.integers(1, 3), st.integers(1, 3), st.integers(1, 40), st.sampled_from([64, 128]))
mixes = st.sampled_from(["normal", "ties", "zeros", "outliers", "wide"])


def _values(shape, mix, seed, wide_exp=20):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if mix == "ties":
        # integers and halves with |x| <= 127 and one 127 per layer: scale 1,
        # so x * 127 / m lands exactly on half-integers
        x = (np.rint(x * 20) / 2).astype(np.float32)
        x = np.clip(x, -126.5, 126.5)
        x.reshape(shape[0], -1)[:, 0] = 127.0
    elif mix == "zeros":
        x[..., ::3, :] = 0.0
        x[..., 1::5, :] = -0.0
    elif mix == "outliers":
        x[..., rng.integers(shape[3])] *= 30.0
        x[..., 0, :] *= 50.0
    elif mix == "wide":
        x *= np.exp2(rng.integers(-wide_exp, wide_exp, size=shape[:3] + (1,))).astype(np.float32)
    return f32_to_bf16_bits(x)


def _sections(pool, shape):
    L, H, T, d = shape
    off = oracle.pool_layout(L, H, T, d)
    k_scale = pool[off[0]:off[0] + 4 * L].view(np.float32)
    k_codes = pool[off[1]:off[1] + L * H * T * d].view(np.int8).reshape(L, H, T, d)
    v_scale = pool[off[2]:off[2] + 2 * L * H * T].view(np.uint16).reshape(L, H, T)
    return k_scale, k_codes, v_scale, pool[off[3]:off[4]]


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shape=shapes, kmix=mixes, vmix=mixes, seed=st.integers(0, 2 ** 31 - 1))
def test_pool_oracle_against_brute_on_random_shapes(shape, kmix, vmix, seed):
    L, H, T, d = shape
    k = _values(shape, kmix, seed)
    v = _values(shape, vmix, seed + 1)
    pool = oracle.pool_encode(k, v)
    assert pool.size == oracle.pool_bytes(*shape)
    k_scale, k_codes, v_scale, v_sec = _sections(pool, shape)

    ref_k, ref_scale, near_tie = k_codes_brute(k)
    np.testing.assert_allclose(k_scale, ref_scale, rtol=2 ** -23)
    assert np.all(k_codes[~near_tie] == ref_k[~near_tie])
    if kmix == "ties":
        # exact ties: the oracle rounds half-integers to even
        x = bf16_bits_to_f32(k).astype(np.float64)
        tie = (np.abs(x - np.floor(x)) == 0.5)
        np.testing.assert_array_equal(k_codes[tie], (2 * np.rint(x[tie] / 2)).astype(np.int8))

    ref_codes, ref_vs, near = v_codes_brute(v, LEVELS, THRESH)
    vec_near = near.any(axis=-1)
    np.testing.assert_array_equal(v_scale[~vec_near], ref_vs[~vec_near])
    codes = unpack_v_codes(v_sec, L, H, T, d)
    np.testing.assert_array_equal(codes, oracle.pool_v_codes(pool, shape))
    assert np.all(codes[~near] == ref_codes[~near])

    ko, vo = oracle.pool_decode(pool, shape)
    y = v_decode_brute(codes, v_scale, LEVELS)
    got = bf16_bits_to_f32(vo).astype(np.float64)
    ulp = np.vectorize(bf16_ulp)(y)
    assert np.all(np.abs(got - y) <= 0.5 * ulp * (1 + 1e-9))
    kx = k_codes.astype(np.float64) * k_scale.astype(np.float64)[:, None, None, None]
    kg = bf16_bits_to_f32(ko).astype(np.float64)
    kulp = np.vectorize(bf16_ulp)(kx)
    assert np.all(np.abs(kg - kx) <= 0.5 * kulp * (1 + 1e-9))


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shape=shapes, mix=mixes, seed=st.integers(0, 2 ** 31 - 1), data=st.data())
def test_card_oracle_properties_on_random_shapes(shape, mix, seed, data):
    L, H, T, d = shape
    # a group's step (max - min) / (2^b - 1) stays a normal fp16 number
    # (2^-14 .. 65504) for vectors scaled by 2^-6 .. 2^6
    k = _values(shape, mix, seed, wide_exp=6)
    v = _values(shape, mix, seed + 7, wide_exp=6)
    widths = np.array(data.draw(st.lists(st.sampled_from([2, 4, 8, 16]), min_size=T, max_size=T)), np.uint8)
    card = oracle.card_pack(k, v, widths, b"hyp", seed % 1000)
    assert card.size == oracle.card_bytes(L, H, T, d, widths)
    ko, vo = oracle.card_unpack(card, shape)
    sizes = np.array([card_record_size(d, int(b)) for b in widths], np.int64)
    off = np.concatenate([[0], np.cumsum(sizes)])
    payload = -(-(256 + T) // 256) * 256
    S = int(-(-off[-1] // 256) * 256)
    G = d // 32
    for src, out, kv in ((k, ko, 0), (v, vo, 1)):
        x = bf16_bits_to_f32(src).astype(np.float64)
        y = bf16_bits_to_f32(out).astype(np.float64)
        for l in range(L):
            for h in range(H):
                base = payload + ((2 * l + kv) * H + h) * S
                for t in range(T):
                    b = int(widths[t])
                    if b == 16:
                        np.testing.assert_array_equal(out[l, h, t], src[l, h, t])
                        continue
                    rec = card[base + off[t]: base + off[t + 1]]
                    s16 = rec[:2 * G].view("<f2").astype(np.float64)
                    codes = np.unpackbits(rec[4 * G:4 * G + d * b // 8], bitorder="little").reshape(d, b)
                    q = (codes * (1 << np.arange(b))).sum(axis=1)
                    for g in range(G):
                        xg, yg, qg = x[l, h, t, 32 * g:32 * g + 32], y[l, h, t, 32 * g:32 * g + 32], q[32 * g:32 * g + 32]
                        assert yg[np.argmin(xg)] == xg.min()
                        if xg.max() > xg.min():
                            assert qg[np.argmax(xg)] == 2 ** b - 1
                        tol = 0.5 * s16[g] * (1 + 2 ** -10) + 0.5 * np.array([bf16_ulp(u) for u in yg])
                        assert np.all(np.abs(xg - yg) <= tol + 1e-30)
    assert math.isfinite(float(np.sum(bf16_bits_to_f32(ko))))
