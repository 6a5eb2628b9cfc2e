"""GPU parity of key position re-alignment (kvc_realign_keys, called
through the C ABI) against the CPU oracle's binary64 rotation: bit-exact
(both sides form each value in binary64 in the same operation order and
round it once to bf16), in place and out of place."""

import numpy as np
import pytest
import torch

import oracle
from agent_handoff_amd import kvcodec as kv
from agent_handoff_amd import synth
from gpu_util import DEV, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _freqs(d, base=500000.0):
    return (base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)).astype(np.float32)


@pytest.mark.parametrize("shape", [(1, 2, 37, 128), (2, 3, 20, 64), (1, 1, 1, 128), (3, 8, 512, 128)])
@pytest.mark.parametrize("pairing", [kv.KVC_ROPE_HALVES, kv.KVC_ROPE_ADJACENT])
def test_realign_bit_exact(shape, pairing):
    k, _ = synth.kv_bits(synth.WORKLOADS[3], 2, shape=shape)
    f = _freqs(shape[3])
    for delta in (1, -4096, 123457, 2 ** 33 + 7):
        say("realign", shape, pairing, delta)
        kd = to_dev(k)
        out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        kv.kvc_realign_keys(shape, kd, out, delta, f, pairing)
        torch.cuda.synchronize()
        ref = oracle.realign_keys(k, delta, f, pairing)
        got = to_host(out)
        assert np.array_equal(got, ref), f"delta {delta}: {np.count_nonzero(got != ref)} values differ"
        kv.kvc_realign_keys(shape, kd, kd, delta, f, pairing)      # in place
        torch.cuda.synchronize()
        assert torch.equal(kd.view(torch.int16), out.view(torch.int16))


def test_zero_shift_is_exact_identity():
    shape = (2, 2, 33, 128)
    k, _ = synth.kv_bits(synth.WORKLOADS[3], 4, shape=shape)
    kd = to_dev(k)
    out = torch.empty_like(kd)
    kv.kvc_realign_keys(shape, kd, out, 0, _freqs(128))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), k)


def test_realign_full_size_keys():
    """The Llama-3-8B 4K key cache moved by 4096 positions (a card made at
    offset 0 landing after a 4096-token prompt)."""
    w = synth.WORKLOADS[3]
    kd, _ = synth.kv_tensors_torch(w, 0, DEV)
    f = _freqs(w.shape[3])
    out = torch.empty_like(kd)
    kv.kvc_realign_keys(w.shape, kd, out, 4096, f)
    torch.cuda.synchronize()
    k = to_host(kd)
    got, ref = to_host(out), oracle.realign_keys(k, 4096, f)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} values differ"
