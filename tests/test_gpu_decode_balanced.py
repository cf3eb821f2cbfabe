"""The decode's balanced split schedule against the fp64 oracle.

The (sequence, group of 4, 2 or 1 adjacent kv heads) units' tile runs are
laid end to end and cut into equal workgroup shares, so a share may hold many
short units, a long unit may be cut into many shares, and a share may begin
in the middle of a unit.  Each case is built so that one of these happens,
with empty sequences between the units, and is held to the oracle with the
default schedule and with forced shares of split_tokens keys; the kv head
counts cover every grouping (8, 4, 12: four heads per unit; 2, 6: two; 3:
one).
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import (ATOL_16, REL_16, banner, compare, gpu_cache, gpu_decode,
                        gpu_decode_fp8kv, lib_module, oracle_decode, oracle_decode_fp8kv,
                        requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _check(A, w, what, splits, fp8=False):
    banner(f"balanced decode {what}: {len(w.kv_lens)} sequences, {int(w.kv_lens.sum())} keys, "
           f"{w.num_heads}/{w.num_kv_heads} heads")
    cache = gpu_cache(w, A, poison=0x7F) if fp8 else gpu_cache(w, A)
    ref_o, ref_l = oracle_decode_fp8kv(w) if fp8 else oracle_decode(w)
    run = gpu_decode_fp8kv if fp8 else gpu_decode
    for st in splits:
        out, lse = run(w, A, split_tokens=st, cache=cache)
        compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"{what} split={st}")


def test_many_short_units_per_workgroup(A):
    """400 sequences of 0-70 keys, 8 kv heads: by default each share holds
    16 tiles, most of them several units."""
    rng = np.random.default_rng(601)
    lens = rng.integers(0, 71, 400)
    lens[::37] = 0
    w = W.make_decode("bal_short", 602, "bf16", lens, 32, 8, 128, 16)
    _check(A, w, "many_short", (0, 256))


def test_one_unit_over_many_workgroups(A):
    """A 40,000-key sequence among short and empty ones, 2 kv heads: each of
    its units is cut into about 80 shares of the default grid."""
    w = W.make_decode("bal_long", 603, "bf16", [3, 40000, 0, 77, 0], 8, 2, 128, 32)
    _check(A, w, "one_long", (0, 1024, 8192))


def test_shares_start_inside_units_d64_f16(A):
    """Unit lengths that are not multiples of a share: 1,000-3,000 keys at
    head size 64, fp16, forced shares of 256 and 768 keys."""
    rng = np.random.default_rng(604)
    lens = rng.integers(1000, 3001, 9)
    w = W.make_decode("bal_mid", 605, "f16", lens, 12, 3, 64, 16)
    _check(A, w, "mid_unit_d64", (0, 256, 768))


def test_fp8_cache_balanced(A):
    """The fp8-cache decode on the same schedule: long and short units and an
    empty one, block size 64."""
    w = W.to_fp8_cache(W.make_decode("bal_fp8", 606, "bf16", [20000, 1, 0, 333, 9000], 32, 8,
                                     128, 64))
    _check(A, w, "fp8_cache", (0, 512, 8192), fp8=True)


@pytest.mark.parametrize("hq,hkv", [(16, 4), (24, 6), (12, 12)])
def test_head_groups(A, hq, hkv):
    """Four kv heads (one unit of 4 per sequence), six (three units of 2) and
    twelve with one query head each (three units of 4, G = 1), ragged lengths
    with an empty sequence, forced shares cutting units mid-way."""
    w = W.make_decode(f"bal_groups_{hkv}", 607 + hkv, "bf16", [700, 0, 2500, 33, 4100], hq, hkv,
                      128, 16)
    _check(A, w, f"head_groups_{hq}_{hkv}", (0, 256, 1280))
