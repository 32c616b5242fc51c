"""Pins of the paged-cache part of the oracle, CPU only.

``attention_fp64_kv_cache`` (queries at the end of the sequence) and
``attention_fp64_paged`` (sequences gathered through block tables) are checked
against ``attention_fp64`` and ``attention_fp64_key_range`` (pinned in
test_oracle.py), against their special cases, and against invariances of the
paged layout.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import (attention_fp64, attention_fp64_key_range, attention_fp64_kv_cache,
                    attention_fp64_paged, gather_paged)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_full_cache_equals_top_left_causal_and_full_attention():
    q, k, v = _rand((4, 50, 16), 1), _rand((2, 50, 16), 2), _rand((2, 50, 16), 3)
    for causal in (False, True):
        o, lse = attention_fp64_kv_cache(q, k, v, 0.3, causal)
        ro, rl = attention_fp64(q[None], k[None], v[None], 0.3, causal)
        assert np.allclose(o, ro[0], rtol=0, atol=1e-13) and np.allclose(lse, rl[0], rtol=0, atol=1e-13)


def test_bottom_right_rows_equal_prefix_attention():
    """Query i of N_q sees exactly the keys 0 .. N - N_q + i."""
    N, Nq = 40, 7
    q, k, v = _rand((2, Nq, 8), 4), _rand((1, N, 8), 5), _rand((1, N, 8), 6)
    o, lse = attention_fp64_kv_cache(q, k, v, 0.4, True)
    for i in range(Nq):
        ro, rl = attention_fp64_key_range(q[None, :, i:i + 1], k[None], v[None], 0.4, False, 0,
                                          N - Nq + i + 1)
        assert np.allclose(o[:, i], ro[0, :, 0], rtol=0, atol=1e-13)
        assert np.allclose(lse[:, i], rl[0, :, 0], rtol=0, atol=1e-13)
    # the last query sees every key: the same as without the mask
    on, ln = attention_fp64_kv_cache(q, k, v, 0.4, False)
    assert np.allclose(o[:, -1], on[:, -1], rtol=0, atol=1e-13)


def test_rows_without_keys():
    q, k, v = _rand((2, 5, 8), 7), _rand((1, 3, 8), 8), _rand((1, 3, 8), 9)
    o, lse = attention_fp64_kv_cache(q, k, v, 0.5, True)   # N_q = 5 > N = 3: rows 0, 1 see nothing
    assert np.all(o[:, :2] == 0) and np.all(np.isneginf(lse[:, :2]))
    assert np.all(np.isfinite(lse[:, 2:]))
    o0, l0 = attention_fp64_kv_cache(q, k[:, :0], v[:, :0], 0.5, False)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


@pytest.mark.parametrize("bs", [16, 32])
def test_paged_equals_dense(bs):
    q, k, v = workloads.make_inputs(3, 4, 2, 2, 100, 16, "f32", seed=10)
    lens = [100, 37, 1]
    kc, vc, tab, sl = workloads.paginate(k, v, lens, bs, seed=11)
    for causal in (False, True):
        o, lse = attention_fp64_paged(q.double().numpy(), kc.double().numpy(), vc.double().numpy(),
                                      tab.numpy(), sl.numpy(), 0.25, causal)
        for b, n in enumerate(lens):
            ro, rl = attention_fp64_kv_cache(q[b].double().numpy(), k[b, :, :n].double().numpy(),
                                             v[b, :, :n].double().numpy(), 0.25, causal)
            assert np.array_equal(o[b], ro) and np.array_equal(lse[b], rl)


def test_gather_reads_only_the_sequence_and_block_order_does_not_matter():
    _, k, v = workloads.make_inputs(2, 2, 2, 1, 70, 8, "f32", seed=12)
    kc, vc, tab, sl = workloads.paginate(k, v, [70, 33], 16, seed=13)
    for b, n in enumerate([70, 33]):
        g = gather_paged(kc.numpy(), tab[b].numpy(), n)
        assert np.array_equal(g, k[b, :, :n].numpy())          # no NaN slot was read
    kc2, vc2, tab2, _ = workloads.paginate(k, v, [70, 33], 16, seed=14)   # another pool order
    assert not np.array_equal(tab.numpy(), tab2.numpy())
    q = _rand((2, 2, 1, 8), 15)
    a = attention_fp64_paged(q, kc.numpy(), vc.numpy(), tab.numpy(), sl.numpy(), 0.3, False)
    c = attention_fp64_paged(q, kc2.numpy(), vc2.numpy(), tab2.numpy(), sl.numpy(), 0.3, False)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_paginate_layout():
    _, k, v = workloads.make_inputs(2, 2, 3, 1, 40, 8, "bf16", seed=16)
    kc, vc, tab, sl = workloads.paginate(k, v, [40, 17], 16, seed=17, spare_blocks=3)
    assert kc.shape == (3 + 2 + 3, 16, 3, 8) and kc.dtype == torch.bfloat16
    assert tab.dtype == torch.int32 and tab.shape == (2, 3) and sl.tolist() == [40, 17]
    assert tab[1, 2].item() == -1 and sorted(tab[tab >= 0].tolist()) == sorted(set(tab[tab >= 0].tolist()))
    # key 20 of sequence 0: block tab[0][1], slot 4, all heads
    assert torch.equal(kc[tab[0, 1], 4], k[0, :, 20])
    # unused slots are NaN
    assert torch.isnan(kc[tab[1, 1], 1:]).all() and torch.isnan(kc[tab[0, 2], 8:]).all()
