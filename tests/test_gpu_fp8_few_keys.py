"""fp8 rows that see few keys, held to the fp8 bar (max-abs 6e-2).

The fp8 method of the pytorch commit "[FlexAttention] Enforce Q,K,V memory
layouts for fp8 flex attention to avoid perf degradation" (Context: "FP8
GEMM softmax_scores @ v") rounds the probabilities to e4m3, a relative error
of up to 2^-4 per weight.  Rows with many visible keys average that out;
rows with a handful do not, and the kernel carries their probabilities as
two e4m3 terms.  These cases put many rows in that regime: narrow local
windows, short documents, the first rows of causal sequences and very short
key sequences, on real N(0, 1) data.
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import (ATOL_FP8, LSE_ATOL_FP8, banner, compare, gpu_fp8, lib_module,
                        oracle_fp8, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _run(A, w, what, window=0):
    banner(f"fp8 few keys {what}: q={w.q_lens.tolist()[:6]} kv={w.kv_lens.tolist()[:6]} "
           f"flags={w.mask_flags} window={window}")
    out, lse = gpu_fp8(w, A, window=window)
    ref_o, ref_l = oracle_fp8(w, window=window)
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what=f"fp8_{what}", lse_atol=LSE_ATOL_FP8)


@pytest.mark.parametrize("window", [1, 2, 5, 16, 40])
def test_fp8_narrow_windows(A, window):
    lens = [300, 77, 513]
    w = W.make_fp8("fw", 401, lens, lens, 8, 2, 128, W.MASK_CAUSAL)
    _run(A, w, f"window{window}", window=window)


def test_fp8_short_documents(A):
    """Documents of 1 to 12 tokens packed into two sequences."""
    rng = np.random.default_rng(402)
    lens = [400, 333]
    ids = []
    for n in lens:
        doc_lens = rng.integers(1, 13, n)
        ids.append(np.repeat(np.arange(n), doc_lens)[:n].astype(np.int32))
    ids = np.concatenate(ids)
    for flags in (W.MASK_DOCUMENT | W.MASK_CAUSAL, W.MASK_DOCUMENT):
        w = W.make_fp8("fd", 403, lens, lens, 8, 2, 128, flags, q_ids=ids, kv_ids=ids)
        _run(A, w, f"short_documents_{flags}")


def test_fp8_short_key_sequences(A):
    """Cross attention without a mask over 1 to 15 keys."""
    q_lens = [100, 50, 37, 64, 9]
    kv_lens = [1, 5, 15, 2, 9]
    w = W.make_fp8("fk", 404, q_lens, kv_lens, 8, 2, 128, W.MASK_NONE)
    _run(A, w, "short_keys")


def test_fp8_first_rows_many_sequences(A):
    """Sixty causal sequences of 1 to 40 tokens: every row sees at most 40 keys."""
    rng = np.random.default_rng(405)
    lens = rng.integers(1, 41, 60)
    w = W.make_fp8("ff", 406, lens, lens, 16, 16, 128, W.MASK_CAUSAL)
    _run(A, w, "first_rows")
