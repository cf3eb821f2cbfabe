"""Host checks of the block-mask input generators (CPU): FlexAttention-style
causal block lists reproduce the causal element mask through the oracle, and
random lists keep their junk outside the valid block range."""

import numpy as np

import oracle as ORC
import workloads as W


def test_causal_block_lists_reproduce_causal_mask():
    for q_lens, kv_lens, qb, kb in (([300, 200, 129], [300, 200, 129], 128, 128),
                                    ([70, 260], [400, 520], 32, 128), ([5], [900], 64, 64),
                                    ([1], [1], 32, 64)):
        kn, ki, fn, fi = W.causal_block_mask(q_lens, kv_lens, qb, kb)
        for b in range(len(q_lens)):
            elem = ORC.visibility(q_lens[b], kv_lens[b], ORC.MASK_CAUSAL)
            vis = ORC.block_visibility(elem, qb, kb, kn[b, 0], ki[b, 0], fn[b, 0], fi[b, 0])
            assert np.array_equal(vis, elem)
            # full blocks need no element mask: dropping it changes nothing
            free = ORC.block_visibility(np.ones_like(elem), qb, kb, np.zeros_like(kn[b, 0]),
                                        ki[b, 0], fn[b, 0], fi[b, 0])
            assert not np.any(free & ~elem)


def test_random_lists_junk_out_of_range():
    rng = np.random.default_rng(5)
    q_lens, kv_lens = [100, 7], [300, 64]
    kn, ki, fn, fi = W.random_block_mask(rng, q_lens, kv_lens, 32, 64, 2)
    for b, kl in enumerate(kv_lens):
        nk = -(-kl // 64)
        for num, idx in ((kn, ki), (fn, fi)):
            for h in range(2):
                for q in range(num.shape[2]):
                    n = num[b, h, q]
                    assert np.all((idx[b, h, q, :n] >= 0) & (idx[b, h, q, :n] < nk))
                    assert np.all((idx[b, h, q, n:] < 0) | (idx[b, h, q, n:] >= nk))
