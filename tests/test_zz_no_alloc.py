"""kvpool_encode_noalloc (the encode for callers that cannot allocate: its
workspace is the library's per-GPU scratch array) against kvpool_encode with
a caller workspace, called through the C ABI on the same seeded inputs.

Bar: the two pools are byte-identical (codes, scales, header, padding), on
two calls in a row, the second with a smaller input; the first call takes
the layered path (a layer larger than one round of the single-pass grid),
the second the single pass, so the second also shows that what the first
left in the scratch does not leak into it."""

import numpy as np
import pytest
import torch

from agent_handoff_amd import kvcodec as kv
from agent_handoff_amd import synth
from gpu_util import DEV, dev_bytes, say, to_dev

pytestmark = pytest.mark.gpu


def _pool_both_ways(shape, cfg, seed):
    k, v = synth.kv_bits(synth.WORKLOADS[cfg], seed, shape=shape)
    kd, vd = to_dev(k), to_dev(v)
    ref = dev_bytes(kv.kvpool_bytes(shape), fill=0xA5)
    ws = dev_bytes(kv.kvpool_workspace_bytes(shape), fill=0)
    kv.kvpool_encode(shape, kd, vd, ref, ws)
    got = dev_bytes(kv.kvpool_bytes(shape), fill=0x3C)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.kvpool_encode_noalloc(shape, kd, vd, got, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_encode_equals_workspace_encode():
    # d = 128, 8 heads x 4200 tokens: 2104 blocks per layer, more than a
    # round of 256 workgroups x 8 slots holds -> layered path
    calls = [((2, 8, 4200, 128), 3, 11), ((3, 4, 300, 64), 2, 12)]
    for shape, cfg, seed in calls:
        say("noalloc encode", shape, "recipe", cfg, "seed", seed)
        got, ref = _pool_both_ways(shape, cfg, seed)
        assert got.size == ref.size == kv.kvpool_bytes(shape)
        diff = np.nonzero(got != ref)[0]
        assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[0]}"
