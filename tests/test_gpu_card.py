"""GPU parity of the CacheCard codec (cachecard_pack / cachecard_unpack,
called through the C ABI) against the CPU oracle: card bytes bit-exact,
unpacked bf16 within 1 ulp, device-side errors reported in the status word."""

import numpy as np
import pytest
import torch

import oracle
from agent_handoff_amd import kvcodec as kv
from agent_handoff_amd import synth
from gpu_util import DEV, assert_decode_close, dev_bytes, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def gpu_pack(shape, k, v, widths, model=b"llama-3.1-8b", pos=0, capacity=None):
    kd, vd = to_dev(k), to_dev(v)
    wd = torch.from_numpy(np.ascontiguousarray(widths, np.uint8)).to(DEV)
    cap = kv.cachecard_max_bytes(shape) if capacity is None else capacity
    card = dev_bytes(cap, fill=0xA5)
    ws = dev_bytes(kv.cachecard_workspace_bytes(shape), fill=0x5A)
    nbytes = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.cachecard_pack(shape, kd, vd, wd, card, ws, model, pos, nbytes, status)
    torch.cuda.synchronize()
    return card, int(nbytes.item()), int(status.item())


def gpu_unpack(shape, card, n):
    ws = dev_bytes(kv.cachecard_workspace_bytes(shape))
    ko = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    vo = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.cachecard_unpack(shape, card, ko, vo, ws, card_bytes=n, dev_status=status)
    torch.cuda.synchronize()
    return ko, vo, int(status.item())


CASES = [((1, 2, 37, 128), "mixed"), ((2, 3, 70, 64), "mixed"), ((1, 1, 1, 128), "mixed"),
         ((2, 2, 64, 128), "all2"), ((1, 2, 33, 64), "all16"), ((3, 1, 50, 128), "runs")]


def _widths(kind, T, seed):
    rng = np.random.default_rng(seed)
    if kind == "mixed":
        return rng.choice(np.array([2, 4, 8, 16], np.uint8), T)
    if kind == "all2":
        return np.full(T, 2, np.uint8)
    if kind == "all16":
        return np.full(T, 16, np.uint8)
    return synth.card_widths(synth.WORKLOADS[4], seed, T=T)


@pytest.mark.parametrize("shape,kind", CASES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_bit_exact_and_unpack_within_one_ulp(shape, kind, seed):
    say("card", shape, kind, seed)
    k, v = synth.kv_bits(synth.WORKLOADS[4], seed, shape=shape)
    widths = _widths(kind, shape[2], seed)
    card, n, st = gpu_pack(shape, k, v, widths, pos=-5 + seed)
    ref = oracle.card_pack(k, v, widths, b"llama-3.1-8b", -5 + seed)
    assert st == 0 and n == ref.size
    got = card[:n].cpu().numpy()
    if not np.array_equal(got, ref):
        idx = np.nonzero(got != ref)[0]
        raise AssertionError(f"{idx.size} card bytes differ, first at {idx[0]}: got {got[idx[0]]} want {ref[idx[0]]}")
    # unpack the oracle's card (decode tested on its own)
    ko, vo, st = gpu_unpack(shape, torch.from_numpy(ref).to(DEV), n)
    assert st == 0
    rk, rv = oracle.card_unpack(ref, shape)
    assert_decode_close(to_host(ko), rk, "K")
    assert_decode_close(to_host(vo), rv, "V")


def test_full_size_cachecard_workload():
    w = synth.WORKLOADS[4]
    say("full-size card workload", w.name)
    k, v = synth.kv_bits(w, 0)
    widths = synth.card_widths(w, 0)
    card, n, st = gpu_pack(w.shape, k, v, widths, pos=4096)
    ref = oracle.card_pack(k, v, widths, b"llama-3.1-8b", 4096)
    assert st == 0 and n == ref.size == kv.cachecard_bytes_host(w.shape, widths)
    assert np.array_equal(card[:n].cpu().numpy(), ref)
    ko, vo, st = gpu_unpack(w.shape, card, n)
    assert st == 0
    rk, rv = oracle.card_unpack(ref, w.shape)
    n1 = assert_decode_close(to_host(ko), rk, "K") + assert_decode_close(to_host(vo), rv, "V")
    say("  values at 1 ulp:", n1)


def test_bad_width_is_reported():
    shape = (1, 2, 20, 128)
    k, v = synth.kv_bits(synth.WORKLOADS[4], 0, shape=shape)
    widths = np.full(20, 4, np.uint8)
    widths[7] = 5
    card, n, st = gpu_pack(shape, k, v, widths)
    assert st & kv.KVC_DEV_BAD_WIDTH
    assert torch.all(card == 0xA5)     # nothing written


def test_small_capacity_is_reported_with_needed_size():
    shape = (1, 2, 20, 128)
    k, v = synth.kv_bits(synth.WORKLOADS[4], 0, shape=shape)
    widths = np.full(20, 8, np.uint8)
    need = kv.cachecard_bytes_host(shape, widths)
    card, n, st = gpu_pack(shape, k, v, widths, capacity=need - 256)
    assert st == kv.KVC_DEV_CAPACITY and n == need
    assert torch.all(card == 0xA5)


def test_unpack_rejects_bad_header_and_widths():
    shape = (1, 2, 20, 64)
    k, v = synth.kv_bits(synth.WORKLOADS[4], 0, shape=shape)
    widths = np.full(20, 4, np.uint8)
    ref = oracle.card_pack(k, v, widths)
    for pos, val, flag in [(0, 0, kv.KVC_DEV_BAD_HEADER), (16, 21, kv.KVC_DEV_BAD_HEADER),
                           (256 + 3, 3, kv.KVC_DEV_BAD_WIDTH), (256 + 4, 16, kv.KVC_DEV_BAD_HEADER)]:
        bad = ref.copy()
        bad[pos] = val
        ko, vo, st = gpu_unpack(shape, torch.from_numpy(bad).to(DEV), ref.size)
        assert st & flag, (pos, st)
        assert torch.isnan(ko.float()).all() and torch.isnan(vo.float()).all()
