"""C-ABI checks that need no GPU: the library loads, exports every function
include/csa2.h declares, and rejects invalid arguments on the host before
anything is launched.  No call here reaches a kernel launch: every call has at
least one argument that fails validation."""
import ctypes
import os
import re

import pytest

import fp4_compressed_sparse_e2m1_amd as csa2
from fp4_compressed_sparse_e2m1_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000          # an aligned, non-null address that is never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function():
    lib = csa2.load()
    names = declared_functions()
    assert {"csa2_quantize_fp4", "csa2_index_full", "csa2_index_reindex", "csa2_sparse_attn",
            "csa2_swa_merge", "csa2_index_scan", "csa2_index_scan_append", "csa2_index_pool"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in csa2.h but not exported"


def test_status_strings_and_version():
    lib = csa2.load()
    for s in range(5):
        assert lib.csa2_status_string(s).decode().startswith("CSA2_")
    assert "gfx950" in csa2.version()


def test_workspace_size_rules():
    lib = csa2.load()
    assert lib.csa2_workspace_size(1, 8, 1 << 20, 2048, 512) > 8 * (1 << 17) * 4
    assert lib.csa2_workspace_size(9, 8, 100, 10, 10) == 0          # unknown op
    assert lib.csa2_workspace_size(1, 0, 100, 10, 10) == 0          # no rows
    assert lib.csa2_workspace_size(1, 1, 100, 5000, 10) == 0        # k_blocks too large
    assert lib.csa2_workspace_size(2, 1, 100, 0, 0) == 0            # k_pos < 1
    # flat mode needs the per-entry keys of every row
    assert lib.csa2_workspace_size(1, 4, 1000, 0, 16) >= 4 * 1000 * 4


def cache_struct(cap=100, n_seq=1, null_ik=False):
    return B._CacheStruct(FAKE, FAKE, 0 if null_ik else FAKE, FAKE, cap, n_seq)


def test_quantize_validation():
    lib = csa2.load()
    f = lib.csa2_quantize_fp4
    assert f(FAKE, -1, 512, 16, None, FAKE, FAKE, 4, None) == INVALID
    assert f(FAKE, 4, 512, 8, None, FAKE, FAKE, 4, None) == UNSUPPORTED
    assert f(FAKE, 4, 520, 16, None, FAKE, FAKE, 4, None) == UNSUPPORTED
    assert f(FAKE, 4, 16, 16, None, FAKE, FAKE, 4, None) == UNSUPPORTED
    assert f(None, 4, 512, 16, None, FAKE, FAKE, 4, None) == INVALID
    assert f(FAKE + 4, 4, 512, 16, None, FAKE, FAKE, 4, None) == INVALID     # misaligned x
    assert f(FAKE, 4, 512, 16, None, FAKE, FAKE, 3, None) == INVALID         # planes too short
    assert f(FAKE, 4, 512, 16, None, FAKE, FAKE, -1, None) == INVALID
    assert f(FAKE, 0, 512, 16, None, None, None, 0, None) == OK              # nothing to do


def test_cache_append_validation():
    lib = csa2.load()
    f = lib.csa2_cache_append
    c = cache_struct()
    assert f(ctypes.byref(c), FAKE, FAKE, -1, FAKE, None) == INVALID           # n < 0
    assert f(None, FAKE, FAKE, 4, FAKE, None) == INVALID                       # no cache
    cn = cache_struct(null_ik=True)
    assert f(ctypes.byref(cn), FAKE, FAKE, 4, FAKE, None) == INVALID           # missing plane
    assert f(ctypes.byref(c), None, FAKE, 4, FAKE, None) == INVALID            # no latent
    assert f(ctypes.byref(c), FAKE, FAKE, 4, None, None) == INVALID            # dst_rows required
    assert f(ctypes.byref(c), FAKE + 4, FAKE, 4, FAKE, None) == INVALID        # misaligned latent
    assert f(ctypes.byref(c), FAKE, FAKE + 8, 4, FAKE, None) == INVALID        # misaligned ikey
    assert f(ctypes.byref(c), None, None, 0, None, None) == OK                 # nothing to do


def test_index_full_noalloc_validation():
    """The no-workspace variant checks its arguments like csa2_index_full and
    rejects sizes whose scratch exceeds its static array, all before touching
    the device."""
    lib = csa2.load()
    c = cache_struct(cap=1 << 20)
    f = lib.csa2_index_full_noalloc

    def call(R=8, max_nvis=1 << 20, kb=2048, kp=512, pool=FAKE, npool=FAKE, cache=None, q=FAKE):
        return f(cache if cache is not None else ctypes.byref(c), q, FAKE, FAKE, FAKE, R, max_nvis,
                 kb, kp, pool, npool, FAKE, FAKE, None)

    assert call(max_nvis=(1 << 20) + 1) == INVALID          # beyond cap
    assert call(R=0) == INVALID
    assert call(kp=0) == INVALID
    assert call(q=FAKE + 2) == INVALID
    assert call(pool=None) == INVALID
    assert call(kb=4097) == UNSUPPORTED
    assert call(cache=ctypes.byref(cache_struct(null_ik=True))) == INVALID
    # 8 decode rows at 2^20 entries fit in the static scratch; 4,096 flat rows do not
    assert lib.csa2_workspace_size(1, 8, 1 << 20, 2048, 512) <= B.NOALLOC_SCRATCH_BYTES
    assert lib.csa2_workspace_size(1, 4096, 32768, 0, 512) > B.NOALLOC_SCRATCH_BYTES
    assert call(R=4096, max_nvis=32768, kb=0, pool=None, npool=None) == UNSUPPORTED
    assert call(R=64, max_nvis=1 << 20) == UNSUPPORTED


def test_index_validation():
    lib = csa2.load()
    c = cache_struct()
    full = lib.csa2_index_full
    args = lambda **kw: dict(dict(cache=ctypes.byref(c), q=FAKE, w=FAKE, seq=FAKE, nvis=FAKE, R=2,
                                  max_nvis=100, kb=8, kp=16, pool=FAKE, npool=FAKE, topk=FAKE,
                                  ntopk=FAKE, ws=FAKE, wsb=0, st=None), **kw)

    def call(**kw):
        a = args(**kw)
        return full(a["cache"], a["q"], a["w"], a["seq"], a["nvis"], a["R"], a["max_nvis"], a["kb"],
                    a["kp"], a["pool"], a["npool"], a["topk"], a["ntopk"], a["ws"], a["wsb"], a["st"])

    assert call(wsb=0) == WORKSPACE                       # everything else valid
    assert call(max_nvis=101) == INVALID                  # beyond cap
    assert call(R=0) == INVALID
    assert call(kp=0) == INVALID
    assert call(kb=-1) == INVALID
    assert call(kb=4097) == UNSUPPORTED
    assert call(kp=5000) == UNSUPPORTED
    assert call(q=FAKE + 2) == INVALID                    # misaligned q_idx
    assert call(pool=None) == INVALID                     # block mode needs pool outputs
    assert call(pool=None, npool=None, kb=0, wsb=0) == WORKSPACE   # flat mode: pool unused
    assert call(cache=ctypes.byref(cache_struct(null_ik=True))) == INVALID
    assert call(cache=None) == INVALID
    need = lib.csa2_workspace_size(1, 2, 100, 8, 16)
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=FAKE + 8, wsb=need) == WORKSPACE       # workspace must be 256-B aligned
    scan = lib.csa2_index_scan
    assert scan(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 100, None, None) == INVALID
    assert scan(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 101, FAKE, None) == INVALID
    sa = lib.csa2_index_scan_append
    c4 = cache_struct(n_seq=4)

    def sa_call(cache=None, lat=FAKE, ik=FAKE, R=2, max_nvis=100, keys=FAKE):
        return sa(ctypes.byref(cache if cache is not None else c4), lat, ik, FAKE, FAKE, FAKE, FAKE, R,
                  max_nvis, keys, None)

    assert sa_call(R=5) == INVALID                        # more rows than sequences
    assert sa_call(cache=c, R=2) == INVALID               # (c holds one sequence)
    assert sa_call(keys=None) == INVALID
    assert sa_call(lat=None) == INVALID
    assert sa_call(ik=FAKE + 4) == INVALID                # misaligned indexer keys
    assert sa_call(max_nvis=101) == INVALID               # beyond cap
    assert sa_call(R=0) == INVALID
    assert sa_call(cache=B._CacheStruct(0, 0, FAKE, FAKE, 100, 4)) == INVALID   # no latent planes
    pool = lib.csa2_index_pool
    assert pool(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 100, FAKE, 0, 16, FAKE, FAKE, FAKE,
                FAKE, FAKE, 1 << 30, None) == INVALID     # pool stage needs k_blocks >= 1
    assert pool(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 100, None, 8, 16, FAKE, FAKE, FAKE,
                FAKE, FAKE, 1 << 30, None) == INVALID     # no block keys
    assert pool(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 100, FAKE, 8, 16, FAKE, FAKE, FAKE,
                FAKE, FAKE, 0, None) == WORKSPACE
    assert lib.csa2_workspace_size(3, 2, 100, 0, 16) == 0
    assert 0 < lib.csa2_workspace_size(3, 2, 100, 8, 16) < lib.csa2_workspace_size(1, 2, 100, 8, 16)
    re_ = lib.csa2_index_reindex
    assert re_(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 100, FAKE, None, 8, 16, FAKE, FAKE,
               FAKE, 1 << 30, None) == INVALID            # pool without counts
    assert re_(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 2, 100, FAKE, FAKE, 0, 16, FAKE, FAKE,
               FAKE, 1 << 30, None) == INVALID            # pool with k_blocks 0


def test_attention_validation():
    lib = csa2.load()
    c = cache_struct()
    f = lib.csa2_sparse_attn
    base = [ctypes.byref(c), FAKE, 16, FAKE, 4, FAKE, FAKE, 512, 0.04, None, FAKE, FAKE, None, 0, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(2, 24) == UNSUPPORTED                     # heads not a multiple of 16
    assert call(2, 128) == UNSUPPORTED
    assert call(2, 48) == UNSUPPORTED
    assert call(7, 0) == INVALID                          # k_pos
    assert call(8, float("inf")) == INVALID               # scale
    assert call(1, FAKE + 2) == INVALID                   # misaligned q
    assert call(10, FAKE + 4) == INVALID                  # o not 16-B aligned (vector stores)
    assert call(5, None) == INVALID                       # topk
    assert call(4, -1) == INVALID
    bad_swa = B._SwaStruct(FAKE, 128, FAKE, 2048)         # window too long
    assert call(9, ctypes.byref(bad_swa)) == INVALID
    m = lib.csa2_swa_merge
    good_swa = B._SwaStruct(FAKE, 128, FAKE, 128)
    assert m(FAKE, 16, FAKE, 4, None, 1, 0.04, FAKE, FAKE, None, 0, None) == INVALID
    assert m(FAKE, 16, FAKE, 4, ctypes.byref(good_swa), 0, 0.04, FAKE, FAKE, None, 0, None) == INVALID
    assert m(FAKE, 20, FAKE, 4, ctypes.byref(good_swa), 1, 0.04, FAKE, FAKE, None, 0, None) == UNSUPPORTED
    assert m(FAKE, 16, FAKE, 0, ctypes.byref(good_swa), 1, 0.04, FAKE, FAKE, None, 0, None) == OK
    assert m(FAKE, 16, FAKE, 4, ctypes.byref(good_swa), 1, 0.04, FAKE + 8, FAKE, None, 0, None) == INVALID
    # flat mode's workspace is bounded (rows go in passes)
    assert lib.csa2_workspace_size(1, 4096, 32768, 0, 512) <= 256 << 20
    assert lib.csa2_workspace_size(1, 1, 32768, 0, 512) >= 32768 * 4
    # a split needs its workspace: given but too small is an error, NULL is not
    ws = lib.csa2_attn_workspace_size(8, 64, 512, 128)
    assert ws >= 8 * 2 * 64 * 514 * 4
    # counters, then the partials of several splits per row
    assert lib.csa2_attn_workspace_size(8, 16, 512, 128) >= 16384 + 8 * 2 * 16 * 512 * 4
    assert lib.csa2_attn_workspace_size(100, 16, 512, 128) > 0     # 16 heads, few rows: channel quarters
    # sized for every call of up to n_rows rows (rows past 191 never split)
    sizes = [lib.csa2_attn_workspace_size(n, 16, 512, 128) for n in range(1, 260)]
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    assert sizes[255] == sizes[190] > 0
    assert lib.csa2_attn_workspace_size(0, 16, 512, 128) == 0
    assert lib.csa2_attn_workspace_size(8, 24, 512, 128) == 0        # invalid heads
    a = list(base)
    a[2] = 64
    a[12], a[13] = FAKE, 64                                           # split planned, 64 B given
    assert f(*a) == WORKSPACE
    a[12] = FAKE + 8
    a[13] = 1 << 30
    assert f(*a) == WORKSPACE                                         # misaligned workspace


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 512)
    codes = torch.zeros(4, 256, dtype=torch.uint8)
    scales = torch.zeros(4, 32, dtype=torch.uint8)
    with pytest.raises(ValueError):
        csa2.csa2_quantize_fp4(x, 16, codes, scales)


def test_cache_record_validation():
    """Export / import reject bad ranges and buffers before any launch; an
    empty range is a no-op."""
    lib = csa2.load()
    for f in (lib.csa2_cache_export, lib.csa2_cache_import):
        cs = cache_struct(cap=100, n_seq=2)
        assert f(ctypes.byref(cs), 0, 0, 0, None, None) == OK            # nothing to copy
        assert f(ctypes.byref(cs), 2, 0, 1, FAKE, None) == INVALID       # sequence out of range
        assert f(ctypes.byref(cs), -1, 0, 1, FAKE, None) == INVALID
        assert f(ctypes.byref(cs), 0, -1, 1, FAKE, None) == INVALID      # negative first
        assert f(ctypes.byref(cs), 0, 90, 11, FAKE, None) == INVALID     # past cap
        assert f(ctypes.byref(cs), 0, 101, 0, FAKE, None) == INVALID
        assert f(ctypes.byref(cs), 0, 0, -1, FAKE, None) == INVALID
        assert f(ctypes.byref(cs), 0, 0, 5, None, None) == INVALID       # no buffer
        assert f(ctypes.byref(cs), 0, 0, 5, FAKE + 2, None) == INVALID   # misaligned buffer
        assert f(ctypes.byref(cache_struct(null_ik=True)), 0, 0, 5, FAKE, None) == INVALID
        assert f(None, 0, 0, 5, FAKE, None) == INVALID
