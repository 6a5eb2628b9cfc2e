"""GPU parity of low-rank anchor materialisation (kvc_lowrank_materialize,
called through the C ABI) against the CPU oracle, which forms
src + sum_v w_v A_v R_v^T in binary64 and rounds once to bf16.

Tolerance (derived from the arithmetic, stated in the library's header):
the products of two bf16 values are exact in binary32; the matrix core adds
r of them per anchor (r - 1 additions, counted twice in case it truncates),
each anchor is folded in with one fused multiply-add and src with one
addition, so the binary32 value is within (2r + V + 1) * 2^-24 * S of the
exact one, S = |src| + sum_v |w_v| sum_k |A_vk R_vk|, to first order; the
final rounding adds at most one bf16 ulp. Beyond the bound, most values
must be bit-identical to the oracle's and none may be off by more than one
ulp unless the bound allows it (heavy cancellation)."""

import numpy as np
import pytest
import torch

from agent_handoff_amd import kvcodec as kv
from agent_handoff_amd import synth
from gpu_util import DEV, say, to_dev, to_host, ulp_distance
from oracle import lowrank

pytestmark = pytest.mark.gpu


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _ulp(x):
    """bf16 ulp at |x| (binary64 array), the subnormal step below 2^-126."""
    m = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(m)) - 7)


def _bound(src_rows, a_rows, r_mat, w, r):
    """(2r + V + 1) 2^-24 S per element of a T' x D matrix view."""
    V = len(w)
    s = np.abs(_f(src_rows))
    for v in range(V):
        s = s + abs(float(w[v])) * (np.abs(_f(a_rows[v])) @ np.abs(_f(r_mat[v])).T)
    return (2 * r + V + 1) * 2.0 ** -24 * s * 1.001


def check_matrix(got_rows, src_rows, a_rows, r_mat, w, r, what):
    """Compare T' x D rows of one matrix (bf16 bits) with the oracle."""
    ref = lowrank.materialize(src_rows, a_rows, r_mat, w)
    g, e = _f(got_rows), _f(ref)
    d = ulp_distance(got_rows, ref)
    tol = _ulp(np.maximum(np.abs(g), np.abs(e))) + _bound(src_rows, a_rows, r_mat, w, r)
    bad = np.abs(g - e) > tol
    assert not bad.any(), f"{what}: {np.count_nonzero(bad)} values beyond the bound, max ulp {d.max()}"
    over1 = d > 1
    if over1.any():
        # only where the binary32 error bound itself exceeds half an ulp
        b = _bound(src_rows, a_rows, r_mat, w, r)
        assert np.all(b[over1] > 0.5 * _ulp(e[over1])), f"{what}: {np.count_nonzero(over1)} values > 1 ulp"
    return float(np.mean(d == 0))


def run(shape, V, r, seed, weights=None, in_place=False, cfg=3):
    L, H, T, d = shape
    src = synth.tensor_bits(synth.WORKLOADS[cfg], seed, synth.K_TENSOR, shape=shape)
    A, R, w = synth.anchor_factors(seed, 6, L, V, T, H * d, r)
    if weights is not None:
        w = np.asarray(weights, np.float32).reshape(L, V)
    sd = to_dev(src)
    out = sd if in_place else torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    say("lowrank", shape, "V", V, "r", r, "seed", seed, "in_place", in_place)
    kv.kvc_lowrank_materialize(shape, r, V, sd, to_dev(A), to_dev(R), torch.from_numpy(w).to(DEV), out)
    torch.cuda.synchronize()
    got = to_host(out)
    exact = []
    for l in range(L):
        exact.append(check_matrix(lowrank.as_matrix(got[l]), lowrank.as_matrix(src[l]), A[l], R[l], w[l], r,
                                  f"{shape} V={V} r={r} layer {l}"))
    return got, src, A, R, w, float(np.mean(exact))


@pytest.mark.parametrize("shape,V,r", [
    ((2, 3, 300, 128), 3, 32),     # ragged tail: 300 = 2 tiles of 128 + 2 blocks of 16 + 12
    ((1, 2, 40, 64), 2, 64),       # d = 64, r = 64, less than one tile
    ((9, 1, 17, 128), 1, 32),      # 9 matrices over 8 XCD groups, one anchor
    ((3, 2, 513, 128), 16, 32),    # most anchors at d = 128, r = 32
    ((2, 2, 64, 64), 32, 32),      # most anchors at d = 64 (one weight per lane)
    ((1, 1, 16, 128), 8, 64),      # most anchors at d = 128, r = 64
    ((2, 8, 1024, 128), 10, 32),   # the pages' defaults, Llama-3-8B heads
    ((16, 8, 700, 64), 3, 32),     # chunks of three tiles per workgroup (a staging buffer reused), ragged last tile
    ((1, 2, 200, 128), 11, 32),    # the most anchors with store waves at d = 128, r = 32
    ((1, 2, 200, 128), 12, 32),    # one more: two blocks per wave, no store waves
])
def test_materialize_matches_oracle(shape, V, r):
    *_, exact = run(shape, V, r, seed=11)
    assert exact > 0.9, f"only {exact:.3f} of values bit-identical"


def test_zero_weights_give_the_source_back_exactly():
    shape, V = (2, 2, 100, 128), 4
    got, src, *_ = run(shape, V, 32, seed=3, weights=np.zeros(2 * V))
    assert np.array_equal(got, src)


def test_signed_weights_and_in_place():
    shape, V = (2, 3, 77, 128), 5
    w = np.array([[1.5, -2.0, 0.0, 0.25, -0.75], [-1.0, 1.0, -1.0, 1.0, 3.0]], np.float32)
    got, *_ = run(shape, V, 32, seed=5, weights=w)
    again, *_ = run(shape, V, 32, seed=5, weights=w, in_place=True)
    assert np.array_equal(got, again)


def test_cancellation_of_two_equal_anchors():
    """Anchors 0 and 1 identical with weights +1 and -1: the two products are
    bit-identical in binary32, so the correction is exactly zero."""
    shape, V, r = (1, 2, 48, 128), 2, 32
    L, H, T, d = shape
    src = synth.tensor_bits(synth.WORKLOADS[3], 8, synth.K_TENSOR, shape=shape)
    A, R, _ = synth.anchor_factors(8, 6, L, V, T, H * d, r)
    A[:, 1] = A[:, 0]
    R[:, 1] = R[:, 0]
    w = np.array([[1.0, -1.0]], np.float32)
    out = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    kv.kvc_lowrank_materialize(shape, r, V, to_dev(src), to_dev(A), to_dev(R), torch.from_numpy(w).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), src)


def test_materialize_full_size_sampled():
    """Llama-3-8B at 4096 tokens (32 layers of K, 8 KV heads, d = 128) with
    V = 10 anchors of rank 32, the launch the benchmark times; the oracle
    checks sampled token rows of sampled layers."""
    w8 = synth.WORKLOADS[3]
    L, H, T, d = w8.shape
    V, r = 10, 32
    kd, _ = synth.kv_tensors_torch(w8, 0, DEV)
    A, R, wt = synth.anchor_factors_torch(0, 6, L, V, T, H * d, r, device=DEV)
    out = torch.empty_like(kd)
    say("lowrank full size", w8.shape, V, r)
    kv.kvc_lowrank_materialize(w8.shape, r, V, kd, A, R, wt, out)
    torch.cuda.synchronize()
    first = to_host(out)
    kv.kvc_lowrank_materialize(w8.shape, r, V, kd, A, R, wt, out)      # deterministic
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), first)
    g = np.random.default_rng(0)
    wh = wt.cpu().numpy()
    for l in (0, 13, 31):
        rows = np.sort(g.choice(T, 96, replace=False))
        rows[:2] = [0, T - 1]
        src_m = lowrank.as_matrix(to_host(kd[l]))[rows]
        got_m = lowrank.as_matrix(first[l])[rows]
        a_rows = to_host(A[l])[:, rows]
        check_matrix(got_m, src_m, a_rows, to_host(R[l]), wh[l], r, f"full size layer {l}")


def test_materialize_back_to_back_calls_agree():
    """Eight calls queued back to back at the benchmark's launch (compute
    waves handing staged blocks to store waves through LDS flags), each into
    its own output, with no synchronisation between them: all eight are
    byte-identical to a call made alone, and its rows match the oracle."""
    w8 = synth.WORKLOADS[3]
    L, H, T, d = w8.shape
    shape = (4, H, T, d)
    V, r = 10, 32
    kd, _ = synth.kv_tensors_torch(w8, 1, DEV)
    kd = kd[:4].contiguous()
    A, R, wt = synth.anchor_factors_torch(1, 6, 4, V, T, H * d, r, device=DEV)
    alone = torch.empty_like(kd)
    say("lowrank back to back", shape, V, r)
    kv.kvc_lowrank_materialize(shape, r, V, kd, A, R, wt, alone)
    torch.cuda.synchronize()
    outs = [torch.full_like(kd, float("nan")) for _ in range(8)]
    for o in outs:
        kv.kvc_lowrank_materialize(shape, r, V, kd, A, R, wt, o)
    torch.cuda.synchronize()
    ref = to_host(alone)
    for i, o in enumerate(outs):
        assert np.array_equal(to_host(o), ref), f"call {i}"
    g = np.random.default_rng(1)
    rows = np.sort(g.choice(T, 64, replace=False))
    rows[:2] = [0, T - 1]
    check_matrix(lowrank.as_matrix(ref[2])[rows], lowrank.as_matrix(to_host(kd[2]))[rows],
                 to_host(A[2])[:, rows], to_host(R[2]), wt.cpu().numpy()[2], r, "back to back layer 2")
