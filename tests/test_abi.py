"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from attention_cu_seqlens_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_cu_seqlens.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libattn_cu_seqlens.so is not built (python -m attention_cu_seqlens_amd.build_lib)")
    return _lib.load()


def test_header_declares_the_five_entry_points():
    names = _declared()
    for n in ("attn_cu_seqlens", "attn_reshape_and_cache", "attn_paged_prefill_fwd",
              "attn_paged_decode_fwd", "attn_fp8_fwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(_lib.SIGNATURES), "binding signatures out of sync with header"


def test_abi_version_and_status_strings(lib):
    assert lib.attn_abi_version() == 4
    for code in range(7):
        assert lib.attn_status_string(code)
    assert lib.attn_status_string(99) == b"unknown status"


P = ctypes.c_void_p(16)   # never dereferenced: every call below fails its host checks


def test_cu_seqlens_host_checks(lib):
    assert lib.attn_cu_seqlens(None, P, 3, None) == 1
    assert lib.attn_cu_seqlens(P, P, -1, None) == 2
    assert lib.attn_cu_seqlens(P, P, 0, None) == 0     # nothing to do, no GPU touched


def test_reshape_and_cache_host_checks(lib):
    f = lib.attn_reshape_and_cache
    ok = [P, P, P, P, P, 4, P, P, 2, 10, 2, 64, 16, 8, 1, None]
    bad = list(ok); bad[0] = None
    assert f(*bad) == 1
    bad = list(ok); bad[12] = 24                        # block_size not a power of two
    assert f(*bad) == 2
    bad = list(ok); bad[10], bad[11], bad[14] = 1, 4, 2  # 4 fp8 bytes per row: not 16-byte rows
    assert f(*bad) == 2
    bad = list(ok); bad[14] = 7
    assert f(*bad) == 3
    bad = list(ok); bad[9] = 0                          # no tokens: no-op
    assert f(*bad) == 0


def test_rotary_cache_host_checks(lib):
    f = lib.attn_rotary_reshape_and_cache

    def call(**kw):
        a = dict(qkv=P, q=None, k=None, v=None, cos=P, sin=P, maxpos=64, rd=64, inter=0, qout=P,
                 kc=P, vc=P, bt=P, mbps=4, cun=P, cukv=P, batch=2, total=10, mskv=64, hq=8, hkv=2,
                 d=128, bs=16, nb=8, dtype=1, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(batch=0) == 0
    assert call(total=0, rd=0, cos=None, sin=None) == 0
    assert call(batch=0, qkv=None, k=P, v=P, qout=None) == 0   # K/V only, no query
    assert call(dtype=2) == 3                                  # fp8: no rotary arithmetic
    assert call(rd=24) == 2                                    # not a multiple of 16
    assert call(rd=144) == 2                                   # above head_size
    assert call(inter=2) == 2
    assert call(cos=None) == 1
    assert call(maxpos=63) == 2                                # table shorter than the longest kv
    assert call(qkv=None, k=P, v=P) == 1                       # q_out without q
    assert call(qkv=None, q=P, k=None, v=P) == 1
    assert call(kc=None) == 1
    assert call(d=100) == 2
    assert call(bs=24) == 2
    assert call(mskv=65) == 2                                  # table too narrow
    assert call(qout=ctypes.c_void_p(24)) == 2                 # misaligned


def test_varlen_bwd_host_checks(lib):
    ws = lib.attn_varlen_bwd_workspace_bytes
    assert ws(100, 8) == 3328            # 3200 rounded up to 256
    assert ws(-1, 8) == 0 and ws(10, 0) == 0
    f = lib.attn_varlen_bwd

    def call(**kw):
        a = dict(q=P, k=P, v=P, out=P, dout=P, lse=P, cuq=P, cukv=P, batch=2, tq=100, tkv=100,
                 msq=64, mskv=64, hq=8, hkv=2, d=128, scale=0.1, mask=1, qids=None, kvids=None,
                 window=0, softcap=0.0, dtype=1, dq=P, dk=P, dv=P, ws=ctypes.c_void_p(256), wsb=3328,
                 stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(batch=0) == 0
    assert call(lse=None) == 1
    assert call(dk=None) == 1
    assert call(d=96) == 3
    assert call(dtype=2) == 3
    assert call(hq=6, hkv=4) == 2
    assert call(window=-1) == 2
    assert call(softcap=-1.0) == 2
    assert call(softcap=float("nan")) == 2
    assert call(batch=0, softcap=30.0) == 0
    assert call(scale=float("inf")) == 2
    assert call(mask=2) == 1                      # DOCUMENT needs both id arrays
    assert call(wsb=3327) == 6
    assert call(ws=None) == 6
    assert call(ws=ctypes.c_void_p(128)) == 6     # not 256-byte aligned
    assert call(dq=ctypes.c_void_p(24)) == 2      # misaligned
    # empty tensors may be NULL: query side when total_q is 0, key side when
    # total_kv is 0 (both empty: nothing to do); still required otherwise
    none_q = dict(q=None, out=None, dout=None, lse=None, dq=None)
    none_kv = dict(k=None, v=None, dk=None, dv=None)
    assert call(tq=0, tkv=0, msq=0, mskv=0, **none_q, **none_kv) == 0
    assert call(tq=0, tkv=0, msq=0, mskv=0, **none_q) == 0
    assert call(tkv=0, **none_q) == 1             # total_q > 0 needs the query side
    assert call(tq=0, **none_kv) == 1             # total_kv > 0 needs the key side


def _prefill_args(**kw):
    a = dict(q=P, kc=P, vc=P, bt=P, mbps=8, cuq=P, cukv=P, batch=2, total_q=100, msq=64, mskv=64,
             hq=8, hkv=2, d=128, bs=16, nb=32, scale=0.1, mask=1, qids=None, kvids=None, window=0,
             softcap=0.0, dtype=1, out=P, lse=None, stream=None)
    a.update(kw)
    return list(a.values())


def test_prefill_host_checks(lib):
    f = lib.attn_paged_prefill_fwd
    assert f(*_prefill_args(q=None)) == 1
    assert f(*_prefill_args(d=96)) == 3
    assert f(*_prefill_args(hq=6, hkv=4)) == 2
    assert f(*_prefill_args(bs=8)) == 3
    assert f(*_prefill_args(dtype=2)) == 3
    assert f(*_prefill_args(mask=2)) == 1               # DOCUMENT needs both id arrays
    assert f(*_prefill_args(mask=4)) == 1               # PATCH needs q_ids
    assert f(*_prefill_args(mask=6, qids=P, kvids=P)) == 3
    assert f(*_prefill_args(mask=8)) == 3
    assert f(*_prefill_args(mskv=129)) == 2             # table too narrow for the longest kv
    assert f(*_prefill_args(scale=float("nan"))) == 2
    assert f(*_prefill_args(window=-1)) == 2
    assert f(*_prefill_args(softcap=-1.0)) == 2
    assert f(*_prefill_args(softcap=float("inf"))) == 2
    assert f(*_prefill_args(softcap=float("nan"))) == 2
    assert f(*_prefill_args(batch=0, window=64, softcap=50.0)) == 0
    assert f(*_prefill_args(batch=0)) == 0
    assert f(*_prefill_args(total_q=0)) == 0


def _sparse_args(**kw):
    a = dict(q=P, kc=P, vc=P, bt=P, mbps=8, cuq=P, cukv=P, batch=2, total_q=100, msq=64, mskv=64,
             hq=8, hkv=2, d=128, bs=16, nb=32, scale=0.1, mask=1, qids=None, kvids=None, window=0,
             softcap=0.0, qblk=128, kvblk=128, mheads=2, nqb=1, cap=1, knum=P, kidx=P, fnum=None,
             fidx=None, dtype=1, out=P, lse=None, stream=None)
    a.update(kw)
    return list(a.values())


def test_block_sparse_prefill_host_checks(lib):
    f = lib.attn_paged_prefill_block_sparse_fwd
    assert f(*_sparse_args(batch=0)) == 0
    assert f(*_sparse_args(batch=0, mheads=1, fnum=P, fidx=P)) == 0
    assert f(*_sparse_args(batch=0, mheads=8)) == 0      # one list per query head
    assert f(*_sparse_args(knum=None)) == 1
    assert f(*_sparse_args(kidx=None)) == 1
    assert f(*_sparse_args(fnum=P)) == 1                 # half of the full pair
    assert f(*_sparse_args(qblk=96)) == 3                # not a power of two
    assert f(*_sparse_args(qblk=16)) == 3                # below 32 rows
    assert f(*_sparse_args(kvblk=32)) == 3               # below 64 keys
    assert f(*_sparse_args(kvblk=(1 << 31) - 1)) == 3   # not a power of two
    assert f(*_sparse_args(batch=0, qblk=1 << 30, kvblk=1 << 30)) == 0
    assert f(*_sparse_args(mheads=4)) == 2               # neither 1, Hkv nor Hq
    assert f(*_sparse_args(nqb=0)) == 2
    assert f(*_sparse_args(msq=129, nqb=1)) == 2         # too few query blocks for 129 rows
    assert f(*_sparse_args(cap=0)) == 2
    # LDS state: 256 rows / 4 heads packed = 64 tokens -> 2 blocks of 32 rows;
    # 2 x 8192 key blocks of 64 keys fit, 2 x 8193 do not
    assert f(*_sparse_args(batch=0, qblk=32, kvblk=64, nqb=2, mskv=8192 * 64,
                              mbps=8192 * 4)) == 0
    assert f(*_sparse_args(qblk=32, kvblk=64, nqb=2, mskv=8193 * 64,
                              mbps=8193 * 4)) == 3
    # the element-mask checks of the plain prefill still apply
    assert f(*_sparse_args(mask=2)) == 1
    assert f(*_sparse_args(window=-1)) == 2


def test_decode_host_checks(lib):
    ws = lib.attn_paged_decode_workspace_bytes
    assert ws(64, 32, 8, 128, 32768, 0, 0) > 0
    assert ws(64, 32, 8, 128, 32768, 0, 100) == 0       # split not a multiple of 256
    assert ws(64, 32, 8, 128, 32768, 0, 8448) == 0      # split above 8192
    assert ws(64, 32, 8, 128, 32768, -1, 0) == 0        # negative window
    assert ws(0, 32, 8, 128, 1, 0, 0) == 0
    def layout(units, rows_per_slot, d, grid):
        # partial slots (units + grid), one row per query head of a unit: O
        # rows, then (m, l), each rounded up to 256 bytes; then two ints per unit
        rows = (units + grid) * rows_per_slot
        up = lambda n: (n + 255) // 256 * 256
        return up(rows * d * 4) + up(rows * 2 * 4) + units * 2 * 4

    need = ws(4, 8, 2, 128, 1000, 0, 256)
    # 2 kv heads form one unit per sequence (8 query rows): 4 units of at most
    # 32 tiles, 8 tiles (256 keys) per workgroup -> 16 workgroups
    assert need == layout(4, 8, 128, 16)
    # a window of 300 keys: a unit spans at most 300 + 31 keys -> 11 tiles
    assert ws(4, 8, 2, 128, 1000, 300, 256) == layout(4, 8, 128, 6)
    # by default: segments of at least 16 tiles over at most 1024 workgroups
    assert ws(4, 8, 2, 128, 1000, 0, 0) == layout(4, 8, 128, 8)
    # 8 kv heads: units of 4 heads (16 query rows), 2 per sequence
    assert ws(64, 32, 8, 128, 32768, 0, 0) == layout(128, 16, 128, 1024)
    # 3 kv heads: one head per unit
    assert ws(4, 6, 3, 64, 1000, 0, 256) == layout(12, 2, 64, 48)
    # tile lists longer than 2^30 are refused
    assert ws(1 << 14, 64, 64, 128, 1 << 20, 0, 0) == 0

    def call(**kw):
        a = dict(q=P, kc=P, vc=P, bt=P, mbps=64, cukv=P, batch=4, mskv=1000, hq=8, hkv=2, d=128,
                 bs=16, nb=300, scale=0.1, window=0, softcap=0.0, split=256, dtype=1, out=P, lse=None,
                 ws=ctypes.c_void_p(256), wsb=need, stream=None)
        a.update(kw)
        return lib.attn_paged_decode_fwd(*a.values())

    assert call(q=None) == 1
    assert call(wsb=need - 1) == 6
    assert call(ws=None) == 6
    assert call(ws=ctypes.c_void_p(128)) == 6             # not 256-byte aligned
    assert call(hq=66, hkv=1) == 3                      # group above 32
    assert call(split=300) == 2
    assert call(split=8448) == 2                        # above 8192
    assert call(window=-5) == 2
    assert call(softcap=float("nan")) == 2
    assert call(batch=0) == 0


def test_decode_noalloc_host_checks(lib):
    """The allocation-free decode takes the decode checks and refuses, on the
    host, sizes whose split partials exceed its fixed scratch."""
    ws = lib.attn_paged_decode_workspace_bytes

    def call(**kw):
        a = dict(q=P, kc=P, vc=P, bt=P, mbps=4096, cukv=P, batch=4, mskv=1000, hq=8, hkv=2, d=128,
                 bs=16, nb=300, scale=0.1, window=0, softcap=0.0, split=256, dtype=1, out=P,
                 lse=None, stream=None)
        a.update(kw)
        return lib.attn_paged_decode_fwd_noalloc(*a.values())

    assert call(q=None) == 1
    assert call(split=300) == 2
    assert call(hq=66, hkv=1) == 3
    assert call(batch=0) == 0
    # 256 sequences x 64 heads in splits of 256 keys: over 500 MiB of partials
    big = dict(batch=256, hq=64, hkv=8, mskv=16384, split=256)
    assert ws(256, 64, 8, 128, 16384, 0, 256) > _lib.ATTN_DECODE_SCRATCH_BYTES
    assert call(**big) == 6
    # the decode workload's shape fits
    assert ws(64, 32, 8, 128, 32768, 0, 0) <= _lib.ATTN_DECODE_SCRATCH_BYTES


def test_decode_fp8kv_host_checks(lib):
    f = lib.attn_paged_decode_fp8kv_fwd
    ws = lib.attn_paged_decode_workspace_bytes
    need = ws(4, 8, 2, 128, 1000, 0, 256)

    def call(**kw):
        a = dict(q=P, kc=P, vc=P, ds=P, bt=P, mbps=64, cukv=P, batch=4, mskv=1000, hq=8, hkv=2,
                 d=128, bs=16, nb=300, scale=0.1, window=0, softcap=0.0, split=256, dtype=1,
                 out=P, lse=None, ws=ctypes.c_void_p(256), wsb=need, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(ds=None) == 1                           # descales required
    assert call(kc=None) == 1
    assert call(dtype=2) == 3                           # q must be fp16 / bf16
    assert call(wsb=need - 1) == 6
    assert call(window=-1) == 2
    assert call(batch=0) == 0


def test_fp8_host_checks(lib):
    f = lib.attn_fp8_fwd

    def call(**kw):
        a = dict(q=P, k=P, v=P, ds=P, cuq=P, cukv=P, batch=2, tq=10, tkv=10, msq=5, mskv=5, hq=4,
                 hkv=4, d=128, scale=0.1, mask=1, qids=None, kvids=None, window=0, softcap=0.0,
                 out=P, lse=None, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(d=64) == 3
    assert call(ds=None) == 1
    assert call(hq=6) == 2
    assert call(window=-1) == 2
    assert call(softcap=-0.5) == 2
    assert call(tkv=(1 << 27) + 16) == 2                # V^T offsets of one wave must fit 32 bits
    assert call(tq=0) == 0
