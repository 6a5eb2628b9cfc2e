"""The object wrappers SharedKVPool and CacheCard (allocation and calls
only) give the same bytes as the C-ABI calls they wrap, and as the
oracle."""

import numpy as np
import pytest
import torch

import oracle
from agent_handoff_amd import kvcodec as kv
from agent_handoff_amd import synth
from gpu_util import DEV, assert_pool_equal, dev_bytes, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_shared_pool_encode_and_decode_layers():
    shape = (3, 2, 100, 128)
    k, v = synth.kv_bits(synth.WORKLOADS[3], 4, shape=shape)
    pool = kv.SharedKVPool.encode(to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert_pool_equal(pool.pool.cpu().numpy(), oracle.pool_encode(k, v), shape)
    ko, vo = pool.decode_layers(1, 3, n_agents=2)
    ref_k = [torch.empty((2,) + shape[1:], dtype=torch.bfloat16, device=DEV)]
    ref_v = [torch.empty_like(ref_k[0])]
    kv.kvpool_decode(shape, pool.pool, 1, 3, ref_k, ref_v)
    torch.cuda.synchronize()
    for a in range(2):
        assert np.array_equal(to_host(ko[a]), to_host(ref_k[0]))
        assert np.array_equal(to_host(vo[a]), to_host(ref_v[0]))


def test_cache_card_pack_unpack_transcode():
    shape = (2, 2, 70, 128)
    k, v = synth.kv_bits(synth.WORKLOADS[4], 5, shape=shape)
    w = synth.card_widths(synth.WORKLOADS[4], 5, T=shape[2])
    w2 = synth.card_widths(synth.WORKLOADS[4], 6, T=shape[2])
    card = kv.CacheCard.pack(to_dev(k), to_dev(v), w, model_id="llama-3.1-8b", position_offset=17)
    ref = oracle.card_pack(k, v, w, b"llama-3.1-8b", 17)
    assert card.status() == 0 and card.nbytes == ref.size
    assert np.array_equal(card.card.cpu().numpy()[:card.nbytes], ref)
    # unpack through the wrapper and through the call it wraps
    ko, vo = card.unpack()
    k_ref, v_ref = torch.empty_like(ko), torch.empty_like(vo)
    kv.cachecard_unpack(shape, card.card, k_ref, v_ref, dev_bytes(kv.cachecard_workspace_bytes(shape)), card.nbytes)
    torch.cuda.synchronize()
    assert card.status() == 0
    assert np.array_equal(to_host(ko), to_host(k_ref)) and np.array_equal(to_host(vo), to_host(v_ref))
    # one hop: the oracle's pack of the unpacked values at the new widths
    hop = card.transcode(w2)
    assert hop.status() == 0
    assert np.array_equal(hop.card.cpu().numpy()[:hop.nbytes],
                          oracle.card_pack(to_host(ko), to_host(vo), w2, b"llama-3.1-8b", 17))
