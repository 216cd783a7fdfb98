"""CSA2 reference oracle (TEST INFRASTRUCTURE ONLY).

Plain CPU implementation, in fp64, of what the CSA2 hot path computes: FP4
E2M1 encoding with E4M3 scales, the Full-mode indexer with its hierarchical
block pool, Reindex-mode Top-K, and sparse attention merged with the SWA
branch.  The arithmetic lives in ``csa2_oracle.c`` (plain C, built with gcc);
this module only marshals numpy arrays.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path and
never imports it.

The pipeline helpers at the bottom follow the steps in the order the pages give
them (P1 "무엇과 다른가"; P3 "레이어 40개 가운데 4개만 전역 캐시를 만듭니다"):
the first decoder Full layer scores every visible entry, keeps up to 2,048
blocks of 8 as the candidate pool and picks Top-512 inside it; a Reindex layer
re-scores the pool with its own indexer query; every layer attends over its
Top-512 plus its 128-token SWA window.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ATTN_DIM = 512        # main-KV latent channels
IDX_DIM = 128         # indexer key dims
IDX_HEADS = 8         # indexer heads
KV_GROUP = 16         # channels per E4M3 scale in the main latent
IK_GROUP = 32         # channels per E4M3 scale in the indexer key (68-B reading)
BLOCK = 8             # positions per indexer block


def build() -> str:
    """Compile ``liboracle.so`` with gcc (plain fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-shared", "-fPIC", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_e2m1_value.argtypes = [i32]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [i32]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_quantize.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_dequantize.argtypes = [P, P, i64, i32, i32, P]
    lib.oracle_index_scores.argtypes = [P, P, P, P, P, i64, P]
    lib.oracle_block_pool.argtypes = [P, i64, i64, P, P]
    lib.oracle_block_pool.restype = i64
    lib.oracle_pool_entries.argtypes = [P, i64, i64, P]
    lib.oracle_pool_entries.restype = i64
    lib.oracle_topk.argtypes = [P, P, i64, i64, P]
    lib.oracle_topk.restype = i64
    lib.oracle_attention.argtypes = [P, i32, P, i64, ctypes.c_double, P, P]
    lib.oracle_lse_merge.argtypes = [P, P, P, P, i32, i32, P, P]
    lib.oracle_decode_e4m3_rows.argtypes = [P, i64, i32, P]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ formats
def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


# ----------------------------------------------------------------- encoding
def quantize(x: np.ndarray, group: int):
    """fp32 [n, dim] -> (codes uint8 [n, dim/2], scales uint8 [n, dim/group])."""
    x = _c(x, np.float32)
    n, dim = x.shape
    assert dim % group == 0 and group % 2 == 0
    codes = np.zeros((n, dim // 2), np.uint8)
    scales = np.zeros((n, dim // group), np.uint8)
    _load().oracle_quantize(_p(x), n, dim, group, _p(codes), _p(scales))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    n, half = codes.shape
    out = np.zeros((n, 2 * half), np.float64)
    _load().oracle_dequantize(_p(codes), _p(scales), n, 2 * half, group, _p(out))
    return out


def decode_e4m3(rows: np.ndarray) -> np.ndarray:
    """E4M3FN bytes (any shape) -> fp64 values of the same shape."""
    rows = _c(rows, np.uint8)
    flat = rows.reshape(1, -1)
    out = np.zeros(flat.shape, np.float64)
    _load().oracle_decode_e4m3_rows(_p(flat), 1, flat.shape[1], _p(out))
    return out.reshape(rows.shape)


# ------------------------------------------------------------------ indexer
def index_scores(q_idx_bits: np.ndarray, w: np.ndarray, ik_codes: np.ndarray,
                 ik_scales: np.ndarray, entries: np.ndarray) -> np.ndarray:
    """q_idx_bits: uint16 bf16 bits [8, 128]; w: float32 [8]; planes of one
    sequence; entries: int64 candidate ids.  Returns fp64 scores."""
    q = _c(q_idx_bits, np.uint16)
    w = _c(w, np.float32)
    ikc, iks = _c(ik_codes, np.uint8), _c(ik_scales, np.uint8)
    ent = _c(entries, np.int64)
    out = np.zeros(len(ent), np.float64)
    _load().oracle_index_scores(_p(q), _p(w), _p(ikc), _p(iks), _p(ent), len(ent), _p(out))
    return out


def block_pool(entry_scores: np.ndarray, k_blk: int):
    """Returns (pool_blocks int32 ascending, block_scores fp64)."""
    s = _c(entry_scores, np.float64)
    n_vis = len(s)
    nb = (n_vis + BLOCK - 1) // BLOCK
    pool = np.zeros(max(min(k_blk, nb), 1), np.int32)
    bs = np.zeros(max(nb, 1), np.float64)
    m = _load().oracle_block_pool(_p(s), n_vis, k_blk, _p(pool), _p(bs))
    return pool[:m].copy(), bs[:nb].copy()


def pool_entries(pool_blocks: np.ndarray, n_vis: int) -> np.ndarray:
    pb = _c(pool_blocks, np.int32)
    out = np.zeros(max(BLOCK * len(pb), 1), np.int64)
    m = _load().oracle_pool_entries(_p(pb), len(pb), n_vis, _p(out))
    return out[:m].copy()


def topk(scores: np.ndarray, cand: np.ndarray, k: int):
    """Returns (topk int32 [k] ascending with -1 pad, count)."""
    s = _c(scores, np.float64)
    c = _c(cand, np.int64)
    out = np.full(k, -1, np.int32)
    m = _load().oracle_topk(_p(s), _p(c), len(c), k, _p(out))
    return out, int(m)


# ---------------------------------------------------------------- attention
def attention(q_bits: np.ndarray, keys: np.ndarray, scale: float):
    """q_bits: uint16 bf16 [H, 512]; keys fp64 [n, 512].  Returns (o [H,512], lse [H])."""
    q = _c(q_bits, np.uint16)
    H = q.shape[0]
    k = _c(keys, np.float64).reshape(-1, ATTN_DIM)
    o = np.zeros((H, ATTN_DIM), np.float64)
    lse = np.zeros(H, np.float64)
    _load().oracle_attention(_p(q), H, _p(k), k.shape[0], float(scale), _p(o), _p(lse))
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    o_a, o_b = _c(o_a, np.float64), _c(o_b, np.float64)
    lse_a, lse_b = _c(lse_a, np.float64), _c(lse_b, np.float64)
    H, dim = o_a.shape
    o = np.zeros_like(o_a)
    lse = np.zeros_like(lse_a)
    _load().oracle_lse_merge(_p(o_a), _p(lse_a), _p(o_b), _p(lse_b), H, dim, _p(o), _p(lse))
    return o, lse


# ------------------------------------------------------- pipeline helpers
def full_layer_select(q_idx_bits, w, ik_codes, ik_scales, n_vis, k_blk, k_pos):
    """Decoder Full layer, indexer part, for one query row.

    Scores every visible entry, keeps the top ``k_blk`` blocks of 8 (pool),
    re-scores the pool and keeps the top ``k_pos`` positions.  With
    ``k_blk == 0`` (flat mode, no pool) the candidates are all visible entries.
    Returns a dict with the block scores, pool, candidate scores and Top-K.
    """
    vis = np.arange(n_vis, dtype=np.int64)
    scores = index_scores(q_idx_bits, w, ik_codes, ik_scales, vis)
    out = {"entry_scores": scores}
    if k_blk > 0:
        pool, bscores = block_pool(scores, k_blk)
        cand = pool_entries(pool, n_vis)
        cscores = index_scores(q_idx_bits, w, ik_codes, ik_scales, cand)
        out.update(pool=pool, block_scores=bscores)
    else:
        cand, cscores = vis, scores
    tk, n = topk(cscores, cand, k_pos)
    out.update(cand=cand, cand_scores=cscores, topk=tk, n_topk=n)
    return out


def reindex_select(q_idx_bits, w, ik_codes, ik_scales, n_vis, pool, k_pos):
    """Reindex layer for one query row: re-score the inherited pool with this
    layer's indexer query and keep the top ``k_pos`` positions.  ``pool=None``
    means flat mode (all visible entries are candidates)."""
    if pool is None:
        cand = np.arange(n_vis, dtype=np.int64)
    else:
        cand = pool_entries(pool, n_vis)
    cscores = index_scores(q_idx_bits, w, ik_codes, ik_scales, cand)
    tk, n = topk(cscores, cand, k_pos)
    return {"cand": cand, "cand_scores": cscores, "topk": tk, "n_topk": n}


def attend_row(q_bits, kv_codes, kv_scales, topk_ids, swa_rows, scale):
    """One query row: softmax attention over the Top-K latents (exact fp64
    decode of the FP4 entries) together with the SWA rows (E4M3 bytes
    [n, 512]).  Returns (o_g, lse_g) over the global keys alone and (o, lse)
    over the union of both key sets, the latter by its plain definition (one
    softmax over all keys)."""
    sel = np.asarray(topk_ids)
    sel = sel[sel >= 0].astype(np.int64)
    g_keys = dequantize(kv_codes[sel], kv_scales[sel], KV_GROUP) if len(sel) else \
        np.zeros((0, ATTN_DIM))
    swa = np.asarray(swa_rows, np.uint8).reshape(-1, ATTN_DIM)
    s_keys = decode_e4m3(swa) if len(swa) else np.zeros((0, ATTN_DIM))
    o_g, lse_g = attention(q_bits, g_keys, scale)
    o, lse = attention(q_bits, np.concatenate([g_keys, s_keys], axis=0), scale)
    return {"o_g": o_g, "lse_g": lse_g, "o": o, "lse": lse}


def parallel_map(fn, items, threads: int):
    """Run ``fn`` over ``items`` on ``threads`` host threads (the C calls
    release the GIL); used to time the oracle on several cores."""
    if threads <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))
