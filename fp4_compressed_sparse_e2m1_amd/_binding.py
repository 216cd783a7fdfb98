"""Thin ctypes binding of libcsa2 (include/csa2.h).

Argument marshalling only: every function checks dtypes, shapes and devices
of the torch tensors it receives, passes their device pointers and the
current HIP stream to the C function of the same name, and raises
``Csa2Error`` on a non-OK status.  All computation happens in the HIP
kernels of libcsa2.so; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

CSA2_OK = 0
CSA2_OP_INDEX_FULL = 1
CSA2_OP_INDEX_REINDEX = 2
CSA2_OP_INDEX_POOL = 3

_lib = None
_lock = threading.Lock()


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class _CacheStruct(ctypes.Structure):
    _fields_ = [("kv_codes", ctypes.c_void_p), ("kv_scales", ctypes.c_void_p),
                ("ik_codes", ctypes.c_void_p), ("ik_scales", ctypes.c_void_p),
                ("cap", ctypes.c_int64), ("n_seq", ctypes.c_int32)]


class _SwaStruct(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("len", ctypes.c_int64),
                ("row_end", ctypes.c_void_p), ("window", ctypes.c_int32)]


def load():
    """Load libcsa2.so, building it first only if no built library exists."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.csa2_quantize_fp4.argtypes = [P, i64, i32, i32, P, P, P, i64, P]
        lib.csa2_quantize_fp4.restype = ctypes.c_int
        lib.csa2_cache_append.argtypes = [P, P, P, i64, P, P]
        lib.csa2_cache_append.restype = ctypes.c_int
        lib.csa2_cache_export.argtypes = [P, i32, i64, i64, P, P]
        lib.csa2_cache_export.restype = ctypes.c_int
        lib.csa2_cache_import.argtypes = [P, i32, i64, i64, P, P]
        lib.csa2_cache_import.restype = ctypes.c_int
        lib.csa2_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        lib.csa2_workspace_size.restype = sz
        lib.csa2_index_full.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
        lib.csa2_index_full.restype = ctypes.c_int
        lib.csa2_index_full_noalloc.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P, P, P, P, P]
        lib.csa2_index_full_noalloc.restype = ctypes.c_int
        lib.csa2_index_scan.argtypes = [P, P, P, P, P, i32, i32, P, P]
        lib.csa2_index_scan.restype = ctypes.c_int
        lib.csa2_index_scan_append.argtypes = [P, P, P, P, P, P, P, i32, i32, P, P]
        lib.csa2_index_scan_append.restype = ctypes.c_int
        lib.csa2_index_pool.argtypes = [P, P, P, P, P, i32, i32, P, i32, i32, P, P, P, P, P, sz, P]
        lib.csa2_index_pool.restype = ctypes.c_int
        lib.csa2_index_reindex.argtypes = [P, P, P, P, P, i32, i32, P, P, i32, i32, P, P, P, sz, P]
        lib.csa2_index_reindex.restype = ctypes.c_int
        lib.csa2_sparse_attn.argtypes = [P, P, i32, P, i32, P, P, i32, ctypes.c_float, P, P, P, P,
                                         sz, P]
        lib.csa2_sparse_attn.restype = ctypes.c_int
        lib.csa2_swa_merge.argtypes = [P, i32, P, i32, P, i32, ctypes.c_float, P, P, P, sz, P]
        lib.csa2_swa_merge.restype = ctypes.c_int
        lib.csa2_attn_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.csa2_attn_workspace_size.restype = sz
        lib.csa2_status_string.argtypes = [ctypes.c_int]
        lib.csa2_status_string.restype = ctypes.c_char_p
        lib.csa2_version.argtypes = []
        lib.csa2_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(fn: str, status: int):
    if status != CSA2_OK:
        raise Csa2Error(fn, status, load().csa2_status_string(status).decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, dtype, name, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


class Cache:
    """Device planes of one Full layer's global cache (356 B per entry).

    kv_codes [n_seq, cap, 256], kv_scales [n_seq, cap, 32],
    ik_codes [n_seq, cap, 64], ik_scales [n_seq, cap, 4], all uint8."""

    def __init__(self, n_seq: int, cap: int, device="cuda", planes=None):
        self.n_seq, self.cap = int(n_seq), int(cap)
        if planes is None:
            mk = lambda w: torch.zeros((self.n_seq, self.cap, w), dtype=torch.uint8, device=device)
            planes = (mk(256), mk(32), mk(64), mk(4))
        self.kv_codes, self.kv_scales, self.ik_codes, self.ik_scales = planes
        for t, wdt, nm in zip(planes, (256, 32, 64, 4), ("kv_codes", "kv_scales", "ik_codes", "ik_scales")):
            _ptr(t, torch.uint8, nm, (self.n_seq, self.cap, wdt))

    def struct(self) -> _CacheStruct:
        return _CacheStruct(self.kv_codes.data_ptr(), self.kv_scales.data_ptr(),
                            self.ik_codes.data_ptr(), self.ik_scales.data_ptr(),
                            self.cap, self.n_seq)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.kv_codes, self.kv_scales, self.ik_codes, self.ik_scales))


class Swa:
    """SWA branch: E4M3FN bytes [n_seq, len, 512], per-row window end, window."""

    def __init__(self, kv: torch.Tensor, row_end: torch.Tensor, window: int = 128):
        if kv.dim() != 3 or kv.shape[2] != 512:
            raise ValueError("swa kv must be [n_seq, len, 512] uint8")
        _ptr(kv, torch.uint8, "swa.kv")
        _ptr(row_end, torch.int32, "swa.row_end")
        self.kv, self.row_end, self.window = kv, row_end, int(window)

    def struct(self) -> _SwaStruct:
        return _SwaStruct(self.kv.data_ptr(), self.kv.shape[1], self.row_end.data_ptr(), self.window)


def csa2_workspace_size(op: int, n_rows: int, max_nvis: int, k_blocks: int, k_pos: int) -> int:
    return int(load().csa2_workspace_size(op, n_rows, max_nvis, k_blocks, k_pos))


def workspace(op: int, n_rows: int, max_nvis: int, k_blocks: int, k_pos: int, device="cuda"):
    """Indexer workspace, zero-filled (its block-selection counters must be
    zero before first use)."""
    n = csa2_workspace_size(op, n_rows, max_nvis, k_blocks, k_pos)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def csa2_quantize_fp4(x, group, codes, scales, dst_rows=None, stream=None):
    """x fp32 [n, dim] -> codes (uint8, rows of dim/2 bytes) and scales (uint8,
    rows of dim/group bytes); row r goes to plane row dst_rows[r] (int64)."""
    n, dim = x.shape
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("codes and scales must be uint8")
    if codes.numel() % (dim // 2) or scales.numel() % (dim // group):
        raise ValueError("plane sizes do not match dim/group")
    rows = codes.numel() // (dim // 2)
    if scales.numel() // (dim // group) != rows:
        raise ValueError("codes and scales planes have different row counts")
    if dst_rows is None and n > rows:
        raise ValueError("more input rows than plane rows")
    lib = load()
    st = lib.csa2_quantize_fp4(_ptr(x, torch.float32, "x"), n, dim, group,
                               _ptr(dst_rows, torch.int64, "dst_rows", (n,), allow_none=True),
                               _ptr(codes, torch.uint8, "codes"), _ptr(scales, torch.uint8, "scales"),
                               rows, _stream(stream))
    _check("csa2_quantize_fp4", st)


def csa2_cache_append(cache: Cache, latent, ikey, dst_rows, stream=None):
    """Encodes latent fp32 [n, 512] and ikey fp32 [n, 128] into the cache's four
    planes at plane rows dst_rows (int64 [n], seq * cap + position), one launch."""
    n = latent.shape[0]
    lib = load()
    cs = cache.struct()
    st = lib.csa2_cache_append(ctypes.byref(cs), _ptr(latent, torch.float32, "latent", (n, 512)),
                               _ptr(ikey, torch.float32, "ikey", (n, 128)), n,
                               _ptr(dst_rows, torch.int64, "dst_rows", (n,)), _stream(stream))
    _check("csa2_cache_append", st)


RECORD_BYTES = 356


def csa2_cache_export(cache: Cache, seq: int, first: int, count: int, records, stream=None):
    """Entries first .. first + count - 1 of sequence seq as count records of
    356 bytes (uint8 device tensor [count, 356]; kv codes, kv scales, indexer
    codes, indexer scales)."""
    lib = load()
    cs = cache.struct()
    rp = _ptr(records, torch.uint8, "records", (count, RECORD_BYTES)) if count > 0 else None
    _check("csa2_cache_export", lib.csa2_cache_export(ctypes.byref(cs), seq, first, count, rp,
                                                      _stream(stream)))


def csa2_cache_import(cache: Cache, seq: int, first: int, count: int, records, stream=None):
    """Writes count records (uint8 device tensor [count, 356]) into entries
    first .. first + count - 1 of sequence seq."""
    lib = load()
    cs = cache.struct()
    rp = _ptr(records, torch.uint8, "records", (count, RECORD_BYTES)) if count > 0 else None
    _check("csa2_cache_import", lib.csa2_cache_import(ctypes.byref(cs), seq, first, count, rp,
                                                      _stream(stream)))


def csa2_index_full(cache: Cache, q_idx, w, row_seq, row_nvis, max_nvis, k_blocks, k_pos,
                    pool_blocks, n_pool, topk, n_topk, workspace, stream=None):
    R = row_seq.shape[0]
    cs = cache.struct()
    st = load().csa2_index_full(
        ctypes.byref(cs), _ptr(q_idx, torch.bfloat16, "q_idx", (R, 8, 128)),
        _ptr(w, torch.float32, "w", (R, 8)), _ptr(row_seq, torch.int32, "row_seq", (R,)),
        _ptr(row_nvis, torch.int32, "row_nvis", (R,)), R, int(max_nvis), int(k_blocks), int(k_pos),
        _ptr(pool_blocks, torch.int32, "pool_blocks", (R, k_blocks), allow_none=k_blocks == 0),
        _ptr(n_pool, torch.int32, "n_pool", (R,), allow_none=k_blocks == 0),
        _ptr(topk, torch.int32, "topk", (R, k_pos)), _ptr(n_topk, torch.int32, "n_topk", (R,)),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check("csa2_index_full", st)


def csa2_index_full_noalloc(cache: Cache, q_idx, w, row_seq, row_nvis, max_nvis, k_blocks, k_pos,
                            pool_blocks, n_pool, topk, n_topk, stream=None):
    """csa2_index_full with the library's static per-device scratch instead of
    a workspace (for callers that cannot allocate)."""
    R = row_seq.shape[0]
    cs = cache.struct()
    st = load().csa2_index_full_noalloc(
        ctypes.byref(cs), _ptr(q_idx, torch.bfloat16, "q_idx", (R, 8, 128)),
        _ptr(w, torch.float32, "w", (R, 8)), _ptr(row_seq, torch.int32, "row_seq", (R,)),
        _ptr(row_nvis, torch.int32, "row_nvis", (R,)), R, int(max_nvis), int(k_blocks), int(k_pos),
        _ptr(pool_blocks, torch.int32, "pool_blocks", (R, k_blocks), allow_none=k_blocks == 0),
        _ptr(n_pool, torch.int32, "n_pool", (R,), allow_none=k_blocks == 0),
        _ptr(topk, torch.int32, "topk", (R, k_pos)), _ptr(n_topk, torch.int32, "n_topk", (R,)),
        _stream(stream))
    _check("csa2_index_full_noalloc", st)


NOALLOC_SCRATCH_BYTES = 16 << 20


def block_keys_buffer(n_rows: int, max_nvis: int, device="cuda"):
    """uint32 block-score keys [n_rows, max(1, ceil(max_nvis / 8))] (held as int32)."""
    return torch.empty((n_rows, max(1, (max_nvis + 7) // 8)), dtype=torch.int32, device=device)


def csa2_index_scan(cache: Cache, q_idx, w, row_seq, row_nvis, max_nvis, block_keys, stream=None):
    R = row_seq.shape[0]
    cs = cache.struct()
    st = load().csa2_index_scan(
        ctypes.byref(cs), _ptr(q_idx, torch.bfloat16, "q_idx", (R, 8, 128)),
        _ptr(w, torch.float32, "w", (R, 8)), _ptr(row_seq, torch.int32, "row_seq", (R,)),
        _ptr(row_nvis, torch.int32, "row_nvis", (R,)), R, int(max_nvis),
        _ptr(block_keys, torch.int32, "block_keys", (R, max(1, (max_nvis + 7) // 8))), _stream(stream))
    _check("csa2_index_scan", st)


def csa2_index_scan_append(cache: Cache, latent, ikey, q_idx, w, row_seq, row_nvis, max_nvis, block_keys,
                           stream=None):
    """Appends row r's latent [R, 512] / ikey [R, 128] at entry min(row_nvis[r], max_nvis) - 1 of
    sequence row_seq[r] (rows name distinct sequences), then scans as csa2_index_scan, one launch."""
    R = row_seq.shape[0]
    cs = cache.struct()
    st = load().csa2_index_scan_append(
        ctypes.byref(cs), _ptr(latent, torch.float32, "latent", (R, 512)),
        _ptr(ikey, torch.float32, "ikey", (R, 128)), _ptr(q_idx, torch.bfloat16, "q_idx", (R, 8, 128)),
        _ptr(w, torch.float32, "w", (R, 8)), _ptr(row_seq, torch.int32, "row_seq", (R,)),
        _ptr(row_nvis, torch.int32, "row_nvis", (R,)), R, int(max_nvis),
        _ptr(block_keys, torch.int32, "block_keys", (R, max(1, (max_nvis + 7) // 8))), _stream(stream))
    _check("csa2_index_scan_append", st)


def csa2_index_pool(cache: Cache, q_idx, w, row_seq, row_nvis, max_nvis, block_keys, k_blocks, k_pos,
                    pool_blocks, n_pool, topk, n_topk, workspace, stream=None):
    R = row_seq.shape[0]
    cs = cache.struct()
    st = load().csa2_index_pool(
        ctypes.byref(cs), _ptr(q_idx, torch.bfloat16, "q_idx", (R, 8, 128)),
        _ptr(w, torch.float32, "w", (R, 8)), _ptr(row_seq, torch.int32, "row_seq", (R,)),
        _ptr(row_nvis, torch.int32, "row_nvis", (R,)), R, int(max_nvis),
        _ptr(block_keys, torch.int32, "block_keys", (R, max(1, (max_nvis + 7) // 8))),
        int(k_blocks), int(k_pos), _ptr(pool_blocks, torch.int32, "pool_blocks", (R, k_blocks)),
        _ptr(n_pool, torch.int32, "n_pool", (R,)), _ptr(topk, torch.int32, "topk", (R, k_pos)),
        _ptr(n_topk, torch.int32, "n_topk", (R,)), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check("csa2_index_pool", st)


def csa2_index_reindex(cache: Cache, q_idx, w, row_seq, row_nvis, max_nvis, pool_blocks, n_pool,
                       k_blocks, k_pos, topk, n_topk, workspace, stream=None):
    R = row_seq.shape[0]
    cs = cache.struct()
    flat = pool_blocks is None
    st = load().csa2_index_reindex(
        ctypes.byref(cs), _ptr(q_idx, torch.bfloat16, "q_idx", (R, 8, 128)),
        _ptr(w, torch.float32, "w", (R, 8)), _ptr(row_seq, torch.int32, "row_seq", (R,)),
        _ptr(row_nvis, torch.int32, "row_nvis", (R,)), R, int(max_nvis),
        _ptr(pool_blocks, torch.int32, "pool_blocks", None if flat else (R, k_blocks), allow_none=True),
        _ptr(n_pool, torch.int32, "n_pool", None if flat else (R,), allow_none=True),
        int(k_blocks), int(k_pos), _ptr(topk, torch.int32, "topk", (R, k_pos)),
        _ptr(n_topk, torch.int32, "n_topk", (R,)), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check("csa2_index_reindex", st)


def csa2_attn_workspace_size(n_rows: int, n_heads: int, k_pos: int, swa_window: int) -> int:
    return int(load().csa2_attn_workspace_size(n_rows, n_heads, k_pos, swa_window))


def attn_workspace(n_rows: int, n_heads: int, k_pos: int, swa_window: int, device="cuda"):
    """Workspace for the split attention path (zero-filled, as its counters
    must be before first use), or None when no split is used."""
    n = csa2_attn_workspace_size(n_rows, n_heads, k_pos, swa_window)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, torch.uint8, "workspace"), workspace.numel()


def csa2_sparse_attn(cache: Cache, q, row_seq, topk, n_topk, scale, o, lse, swa: Swa = None,
                     workspace=None, stream=None):
    R, H, D = q.shape
    if D != 512:
        raise ValueError("q must be [n_rows, n_heads, 512]")
    cs = cache.struct()
    ss = swa.struct() if swa is not None else None
    wp, wb = _ws(workspace)
    st = load().csa2_sparse_attn(
        ctypes.byref(cs), _ptr(q, torch.bfloat16, "q"), H, _ptr(row_seq, torch.int32, "row_seq", (R,)),
        R, _ptr(topk, torch.int32, "topk"), _ptr(n_topk, torch.int32, "n_topk", (R,)),
        topk.shape[1], float(scale), ctypes.byref(ss) if ss is not None else None,
        _ptr(o, torch.float32, "o", (R, H, 512)), _ptr(lse, torch.float32, "lse", (R, H)),
        wp, wb, _stream(stream))
    _check("csa2_sparse_attn", st)


def csa2_swa_merge(q, row_seq, swa: Swa, scale, o, lse, workspace=None, stream=None):
    R, H, D = q.shape
    ss = swa.struct()
    wp, wb = _ws(workspace)
    st = load().csa2_swa_merge(
        _ptr(q, torch.bfloat16, "q"), H, _ptr(row_seq, torch.int32, "row_seq", (R,)), R,
        ctypes.byref(ss), swa.kv.shape[0], float(scale), _ptr(o, torch.float32, "o", (R, H, 512)),
        _ptr(lse, torch.float32, "lse", (R, H)), wp, wb, _stream(stream))
    _check("csa2_swa_merge", st)


def version() -> str:
    return load().csa2_version().decode()
