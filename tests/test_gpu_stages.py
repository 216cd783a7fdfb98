"""GPU parity, stage by stage, at sizes the oracle finishes in seconds.

Every case feeds the HIP path and the oracle the same seeded inputs; where a
stage consumes an upstream result, the GPU stage receives the oracle's
result (never the other way round), so each stage is compared on its own.
Sizes span several tiles and ragged tails; edge cases cover empty rows,
n_vis below K, scale ties, subnormal scales and invalid ids.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_attention, check_full_row, check_topk

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_compressed_sparse_e2m1_amd as m
    m.load()
    return m


def dev(x, dtype=None):
    t = torch.as_tensor(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def build_cache(csa2, lat_list, ik_list, cap):
    """Quantise per-sequence fp32 rows into a fresh cache with the GPU kernel;
    returns the cache and the oracle's codes for the same rows."""
    S = len(lat_list)
    cache = csa2.Cache(S, cap)
    ora = []
    for s, (lat, ik) in enumerate(zip(lat_list, ik_list)):
        n = lat.shape[0]
        dst = torch.arange(n, dtype=torch.int64, device="cuda") + s * cap
        csa2.csa2_quantize_fp4(dev(lat), 16, cache.kv_codes, cache.kv_scales, dst_rows=dst)
        csa2.csa2_quantize_fp4(dev(ik), 32, cache.ik_codes, cache.ik_scales, dst_rows=dst)
        kvc, kvs = oracle.quantize(lat, 16)
        ikc, iks = oracle.quantize(ik, 32)
        ora.append((kvc, kvs, ikc, iks))
    torch.cuda.synchronize()
    return cache, ora


# ---------------------------------------------------------------- S1 codec
@pytest.mark.parametrize("dim,group", [(512, 16), (128, 32)])
def test_quantize_bit_exact_random_and_edges(csa2, dim, group):
    x = W.rms_rows(997, dim, seed=100 + dim).numpy()
    x[1] *= 1e-3
    x[2] *= 3e-5                      # subnormal scales
    x[3] = 0.0                        # zero groups
    x[4] *= 60.0
    x[5, :group] = -1e-6              # scale underflow, negative zeros -> 0x8
    x[6, 0] = -0.0
    # a group fixing the scale at 0.5 with every E2M1 midpoint in it
    x[7, :] = 0.0
    x[7, 0] = 3.0
    for i, t in enumerate([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]):
        x[7, 1 + i] = 0.5 * t
        if group > 8 + i:
            x[7, 8 + i] = -0.5 * t
    # scale ties: amax/6 halfway between two E4M3 values
    x[8, :group] = 0.0
    x[8, 0] = 6 * (0.5 + 0.5625) / 2
    n = x.shape[0]
    codes = torch.zeros((n, dim // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((n, dim // group), dtype=torch.uint8, device="cuda")
    csa2.csa2_quantize_fp4(dev(x), group, codes, scales)
    rc, rs = oracle.quantize(x, group)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_quantize_scatter_rows(csa2):
    x = W.rms_rows(33, 512, seed=7).numpy()
    dst = np.random.default_rng(0).choice(200, size=33, replace=False).astype(np.int64)
    codes = torch.zeros((200, 256), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((200, 32), dtype=torch.uint8, device="cuda")
    csa2.csa2_quantize_fp4(dev(x), 16, codes, scales, dst_rows=dev(dst))
    rc, rs = oracle.quantize(x, 16)
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(c[dst], rc)
    np.testing.assert_array_equal(s[dst], rs)
    untouched = np.setdiff1d(np.arange(200), dst)
    assert not c[untouched].any() and not s[untouched].any()


def test_cache_append_both_planes(csa2):
    """One launch encodes both planes exactly as the oracle (and as the
    per-plane calls) would; rows aimed outside the planes are skipped."""
    n_seq, cap, n = 3, 50, 21
    lat = W.rms_rows(n, 512, seed=41).numpy()
    ik = W.rms_rows(n, 128, seed=42).numpy()
    lat[0] = 0.0                                   # zero groups
    lat[1] *= 3e-5                                 # subnormal scales
    ik[2] *= 60.0                                  # saturating scales
    ik[3, :32] = -1e-6                             # scale underflow, negative zeros
    rng = np.random.default_rng(5)
    dst = rng.choice(n_seq * cap, size=n, replace=False).astype(np.int64)
    dst[4], dst[5] = -1, n_seq * cap               # outside: skipped
    cache = csa2.Cache(n_seq, cap)
    csa2.csa2_cache_append(cache, dev(lat), dev(ik), dev(dst))
    torch.cuda.synchronize()
    kvc, kvs = oracle.quantize(lat, 16)
    ikc, iks = oracle.quantize(ik, 32)
    planes = [t.reshape(n_seq * cap, -1).cpu().numpy()
              for t in (cache.kv_codes, cache.kv_scales, cache.ik_codes, cache.ik_scales)]
    ok = (dst >= 0) & (dst < n_seq * cap)
    for got, ref in zip(planes, (kvc, kvs, ikc, iks)):
        np.testing.assert_array_equal(got[dst[ok]], ref[ok])
        untouched = np.setdiff1d(np.arange(n_seq * cap), dst[ok])
        assert not got[untouched].any()


def test_index_scan_append_matches_append_then_scan(csa2):
    """The one-launch append + scan writes the planes and block keys that the
    append at entry min(n_vis, max_nvis) - 1 followed by the scan write, byte
    for byte, and the appended bytes are the oracle's encoding.  The new
    entries sit at the start, the middle and the end of a 512-entry scan
    chunk, at entry 0, and past max_nvis (clamped); rows with n_vis 0 or an
    invalid sequence append nothing."""
    n_seq, cap, max_nvis = 8, 2600, 2500
    seqs = np.array([3, 0, 7, 1, 4, -1, 6, 2], np.int32)
    nvis = np.array([513, 1024, 1, 2100, 0, 300, 2599, 777], np.int32)
    R = len(seqs)
    g = torch.Generator(device="cpu").manual_seed(12)
    planes = [torch.randint(0, 256, (n_seq, cap, 256), generator=g, dtype=torch.uint8),
              torch.randint(0, 0x7F, (n_seq, cap, 32), generator=g, dtype=torch.uint8),
              torch.randint(0, 256, (n_seq, cap, 64), generator=g, dtype=torch.uint8),
              torch.randint(0, 0x7F, (n_seq, cap, 4), generator=g, dtype=torch.uint8)]
    ca = csa2.Cache(n_seq, cap, planes=[p.cuda() for p in planes])
    cb = csa2.Cache(n_seq, cap, planes=[p.cuda() for p in planes])
    lat = W.rms_rows(R, 512, seed=91).numpy()
    ik = W.rms_rows(R, 128, seed=92).numpy()
    lat[2] *= 3e-5                                  # subnormal scales
    ik[3] *= 60.0                                   # saturating scales
    q_idx = W.bf16_normal((R, 8, 128), 93, device="cuda")
    w = W.uniform01((R, 8), 94, device="cuda")
    n_eff = np.minimum(nvis, max_nvis)
    ok = (seqs >= 0) & (seqs < n_seq) & (n_eff >= 1)
    dst = np.where(ok, seqs.astype(np.int64) * cap + n_eff - 1, -1)
    ka = csa2.block_keys_buffer(R, max_nvis).fill_(0x5A5A5A5A)
    kb = csa2.block_keys_buffer(R, max_nvis).fill_(0x5A5A5A5A)
    csa2.csa2_cache_append(ca, dev(lat), dev(ik), dev(dst))
    csa2.csa2_index_scan(ca, q_idx, w, dev(seqs), dev(nvis), max_nvis, ka)
    csa2.csa2_index_scan_append(cb, dev(lat), dev(ik), q_idx, w, dev(seqs), dev(nvis), max_nvis, kb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kb.cpu().numpy(), ka.cpu().numpy())
    kvc, kvs = oracle.quantize(lat, 16)
    ikc, iks = oracle.quantize(ik, 32)
    for a, b, ref in ((ca.kv_codes, cb.kv_codes, kvc), (ca.kv_scales, cb.kv_scales, kvs),
                      (ca.ik_codes, cb.ik_codes, ikc), (ca.ik_scales, cb.ik_scales, iks)):
        bh = b.reshape(n_seq * cap, -1).cpu().numpy()
        np.testing.assert_array_equal(bh, a.reshape(n_seq * cap, -1).cpu().numpy())
        np.testing.assert_array_equal(bh[dst[ok]], ref[ok])
    # an n_vis-0 row and an invalid sequence left their planes alone
    for p_ref, b in zip(planes, (cb.kv_codes, cb.kv_scales, cb.ik_codes, cb.ik_scales)):
        assert torch.equal(b[4].cpu(), p_ref[4]) and torch.equal(b[5].cpu(), p_ref[5])


def test_cache_records_export_import(csa2):
    """Entry records (356 B: kv codes, kv scales, indexer codes, indexer
    scales) equal the oracle's encoding of the same rows laid out in that
    order, and a range exported from one cache and imported into another
    (different sequence and offset) reproduces the planes byte for byte
    without touching the entries around it."""
    n, cap = 1000, 1200
    lat = W.rms_rows(n, 512, seed=61).numpy()
    ik = W.rms_rows(n, 128, seed=62).numpy()
    src = csa2.Cache(2, cap)
    dst_rows = torch.arange(n, dtype=torch.int64, device="cuda") + cap + 100      # sequence 1, from 100
    csa2.csa2_cache_append(src, dev(lat), dev(ik), dst_rows)
    first, count = 137, 777
    rec = torch.full((count, 356), 0xAB, dtype=torch.uint8, device="cuda")
    csa2.csa2_cache_export(src, 1, 100 + first, count, rec)
    kvc, kvs = oracle.quantize(lat[first:first + count], 16)
    ikc, iks = oracle.quantize(ik[first:first + count], 32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rec.cpu().numpy(), np.concatenate([kvc, kvs, ikc, iks], axis=1))
    dst = csa2.Cache(3, 900)
    for plane in (dst.kv_codes, dst.kv_scales, dst.ik_codes, dst.ik_scales):
        plane.fill_(0x5A)
    csa2.csa2_cache_import(dst, 2, 900 - count, count, rec)
    csa2.csa2_cache_export(dst, 2, 0, 0, None)                                  # empty range: no-op
    torch.cuda.synchronize()
    for a, b in ((dst.kv_codes, src.kv_codes), (dst.kv_scales, src.kv_scales),
                 (dst.ik_codes, src.ik_codes), (dst.ik_scales, src.ik_scales)):
        np.testing.assert_array_equal(a[2, 900 - count:].cpu().numpy(),
                                      b[1, 100 + first:100 + first + count].cpu().numpy())
        assert torch.all(a[2, :900 - count] == 0x5A) and torch.all(a[:2] == 0x5A)


# ------------------------------------------------------------- S2-S4 index
def make_index_case(csa2, n_list, cap, seed, k_rows=None):
    lat = [W.rms_rows(n, 512, seed=seed + 10 * i).numpy() for i, n in enumerate(n_list)]
    ik = [W.rms_rows(n, 128, seed=seed + 10 * i + 1).numpy() for i, n in enumerate(n_list)]
    cache, ora = build_cache(csa2, lat, ik, cap)
    return cache, ora


def run_full(csa2, cache, qidx, w, row_seq, row_nvis, max_nvis, k_blk, k_pos):
    R = len(row_seq)
    pool = torch.full((R, max(k_blk, 1)), -7, dtype=torch.int32, device="cuda")
    npool = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    topk = torch.full((R, k_pos), -7, dtype=torch.int32, device="cuda")
    ntopk = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_FULL, R, max_nvis, k_blk, k_pos)
    csa2.csa2_index_full(cache, qidx, w, dev(row_seq, torch.int32), dev(row_nvis, torch.int32),
                         max_nvis, k_blk, k_pos, pool if k_blk else None, npool if k_blk else None,
                         topk, ntopk, ws)
    torch.cuda.synchronize()
    return pool.cpu().numpy(), npool.cpu().numpy(), topk.cpu().numpy(), ntopk.cpu().numpy()


@pytest.mark.parametrize("case", ["decode_small", "ragged", "multilevel"])
def test_index_full_block_mode(csa2, case):
    if case == "decode_small":        # the tiny-decode shape: 4,096 entries, 64 blocks -> 512
        n_list, rows, k_blk, k_pos = [4096], [(0, 4096)], 64, 512
    elif case == "ragged":            # several sequences, ragged tails, empty and tiny rows
        n_list = [5003, 77, 2000]
        rows = [(0, 5003), (1, 77), (2, 1999), (0, 4096), (2, 0), (0, 9), (5, 100)]
        k_blk, k_pos = 100, 64
    else:                             # >16,384 blocks: two selection levels
        n_list, rows, k_blk, k_pos = [140001], [(0, 140001), (0, 131072)], 2048, 512
    cap = max(n_list) + 3
    seeds = {"decode_small": 101, "ragged": 202, "multilevel": 303}
    cache, ora = make_index_case(csa2, n_list, cap, seed=seeds[case])
    R = len(rows)
    qidx = W.bf16_normal((R, 8, 128), seed=5)
    w = W.uniform01((R, 8), seed=6)
    row_seq = [s for s, _ in rows]
    row_nvis = [n for _, n in rows]
    max_nvis = max(row_nvis)
    qd, wd = dev(qidx), dev(w)
    pool, npool, topk, ntopk = run_full(csa2, cache, qd, wd, row_seq, row_nvis, max_nvis, k_blk, k_pos)
    qb = W.bf16_bits(qidx)
    wn = w.numpy()
    for r, (s, nv) in enumerate(rows):
        if s >= len(n_list):          # out-of-range sequence id -> empty row
            assert npool[r] == 0 and ntopk[r] == 0
            assert np.all(topk[r] == -1) and np.all(pool[r] == -1)
            continue
        _, _, ikc, iks = ora[s]
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nv, k_blk, k_pos)
        check_full_row(csa2, cache, qd[r:r + 1], wd[r:r + 1], s, nv, pool[r], npool[r], topk[r],
                       ntopk[r], ref, k_blk, k_pos, f"row {r}")


def test_index_full_block_mode_tied_blocks(csa2):
    """Four thousand blocks with one and the same top score, straddling the
    boundary between the two first-level chunks of a 17,501-block row, around
    the 2,048th place: the pool keeps the lowest-numbered tied blocks and the
    Top-512 the lowest-numbered tied entries, exactly as the oracle ranks
    (descending score, ties to the lower index) -- compared for equality, not
    within the tie tolerance."""
    n = 140001
    base = W.rms_rows(n, 128, seed=81).numpy()
    qidx = W.bf16_normal((1, 8, 128), seed=82)
    w = W.uniform01((1, 8), seed=83)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    ikc0, iks0 = oracle.quantize(base, 32)
    s0 = oracle.index_scores(qb[0], wn[0], ikc0, iks0, np.arange(n))
    ik = base.copy()
    ik[100000:132000] = 2.0 * base[int(np.argmax(s0))]     # blocks 12,500 .. 16,499, all tied
    lat = W.rms_rows(n, 512, seed=84).numpy()
    cache, ora = build_cache(csa2, [lat], [ik], n)
    _, _, ikc, iks = ora[0]
    pool, npool, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [0], [n], n, 2048, 512)
    ref = oracle.full_layer_select(qb[0], wn[0], ikc, iks, n, 2048, 512)
    assert list(ref["pool"][:3]) == [12500, 12501, 12502] and ref["pool"][-1] == 12500 + 2047
    assert npool[0] == len(ref["pool"]) and np.array_equal(pool[0][:npool[0]], ref["pool"])
    assert ntopk[0] == ref["n_topk"] == 512 and np.array_equal(topk[0], ref["topk"])


@pytest.mark.parametrize("n_tied", [40, 70])
def test_index_flat_tied_threshold(csa2, n_tied):
    """n_tied entries with one and the same score straddle the 512th place of
    a 10,000-entry flat selection: 40 leave the threshold's bin small enough to
    be ranked directly, 70 send it through the refining digits.  The Top-512
    must take exactly the lowest-numbered tied entries the oracle takes."""
    n, k = 10000, 512
    base = W.rms_rows(n, 128, seed=91).numpy()
    qidx = W.bf16_normal((1, 8, 128), seed=92)
    w = W.uniform01((1, 8), seed=93)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    slots = np.arange(1000, 1000 + 97 * n_tied, 97)[:n_tied]      # spread over the row
    c0, s0 = oracle.quantize(base, 32)
    order = np.argsort(-oracle.index_scores(qb[0], wn[0], c0, s0, np.arange(n)), kind="stable")
    for rank in range(480, 520):        # copy the rank-th entry's key into the slots
        ik = base.copy()
        ik[slots] = base[int(order[rank])]
        c1, s1 = oracle.quantize(ik, 32)
        sc = oracle.index_scores(qb[0], wn[0], c1, s1, np.arange(n))
        above = int((sc > sc[slots[0]]).sum())
        if above < k <= above + n_tied and above + n_tied - k >= 4 and k - above >= 4:
            break
    assert above < k <= above + n_tied, "no straddling tie found"
    lat = W.rms_rows(n, 512, seed=94).numpy()
    cache, ora = build_cache(csa2, [lat], [ik], n)
    _, _, ikc, iks = ora[0]
    _, _, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [0], [n], n, 0, k)
    ref = oracle.full_layer_select(qb[0], wn[0], ikc, iks, n, 0, k)
    assert ntopk[0] == ref["n_topk"] == k and np.array_equal(topk[0], ref["topk"])
    kept = np.intersect1d(topk[0], slots)
    assert len(kept) == k - above and np.array_equal(kept, slots[:k - above])


@pytest.mark.parametrize("n_vis_rows", [[4096, 1000, 1], [20000, 16385, 300], [32768, 32767, 16385],
                                        [40000, 32769, 5], [140001, 70000]])
def test_index_full_flat_mode(csa2, n_vis_rows):
    n = max(n_vis_rows)
    cache, ora = make_index_case(csa2, [n], n, seed=17)
    R = len(n_vis_rows)
    qidx = W.bf16_normal((R, 8, 128), seed=8)
    w = W.uniform01((R, 8), seed=9)
    _, _, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [0] * R, n_vis_rows, n, 0, 512)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    _, _, ikc, iks = ora[0]
    for r, nv in enumerate(n_vis_rows):
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nv, 0, 512)
        check_topk(topk[r], ntopk[r], ref, "flat")


def test_index_flat_rows_in_passes(csa2):
    """Flat mode with more rows than one 256-MiB pass holds (433 rows of up to
    140,001 entries: 416 rows per pass): the workspace stays bounded and the
    rows on both sides of the pass boundary match the oracle."""
    n, R = 140001, 433
    cache, ora = make_index_case(csa2, [n], n, seed=47)
    nvis = [n - (R - 1 - r) for r in range(R)]
    need = csa2.csa2_workspace_size(csa2.CSA2_OP_INDEX_FULL, R, n, 0, 512)
    # (one pass of every row would need 4 B per entry and two 9-chunk
    # selection buffers per row)
    assert need <= 256 << 20 < R * (n * 4 + 2 * 9 * 512 * 8)
    qidx = W.bf16_normal((R, 8, 128), seed=48)
    w = W.uniform01((R, 8), seed=49)
    _, _, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [0] * R, nvis, n, 0, 512)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    _, _, ikc, iks = ora[0]
    for r in (0, 415, 416, R - 1):
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nvis[r], 0, 512)
        check_topk(topk[r], ntopk[r], ref, f"row {r}")


def test_index_flat_many_rows(csa2):
    """Flat scoring of many rows at once (the prefill shape: consecutive query
    tokens of one sequence, n_vis growing by one per row), with work-groups
    whose rows mix sequences, an empty row, an out-of-range sequence id, a
    one-entry row and a row count that is not a multiple of the row group."""
    n_list = [5000, 3001]
    cache, ora = make_index_case(csa2, n_list, 5000, seed=41)
    rows = [(0, 4970 + i) for i in range(30)]
    rows[12] = (1, 3001)
    rows[13] = (1, 2999)
    rows += [(1, 3001), (0, 0), (7, 100), (1, 1), (0, 4999), (0, 512), (0, 513)]
    R, k_pos = len(rows), 512
    qidx = W.bf16_normal((R, 8, 128), seed=42)
    w = W.uniform01((R, 8), seed=43)
    _, _, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [s for s, _ in rows],
                                 [n for _, n in rows], max(n for _, n in rows), 0, k_pos)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    for r, (s, nv) in enumerate(rows):
        if s >= len(n_list) or nv == 0:
            assert ntopk[r] == 0 and np.all(topk[r] == -1), r
            continue
        _, _, ikc, iks = ora[s]
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nv, 0, k_pos)
        check_topk(topk[r], ntopk[r], ref, f"row {r}")


@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("per_seq", [3, 6])
@pytest.mark.parametrize("k_blk", [300, 0])
def test_index_multi_query_rows(csa2, per_seq, k_blk, interleave):
    """Several query rows per sequence (multi-query decode: draft tokens whose
    n_vis grow by one, checked together), in block mode (pool, then Top-K)
    and flat mode: rows share key tiles in the many-row scoring kernel (4 rows
    per work-group at 3 rows per sequence, 8 at 6), laid out sequence by
    sequence or interleaved (each work-group then scores several sequences in
    turn).  Also an out-of-range sequence id, an empty row, and rows of one
    sequence split across work-groups."""
    n_list = [6000, 4100, 9001]
    cache, ora = make_index_case(csa2, n_list, 9001, seed=51 + per_seq)
    rows = []
    for s, n in enumerate(n_list):
        rows += [(s, n - per_seq + 1 + i) for i in range(per_seq)]
    if interleave:              # sequences alternate row by row: several passes per work-group
        rows = [rows[per_seq * (i % 3) + i // 3] for i in range(len(rows))]
    rows += [(5, 100), (1, 0), (2, 8193)]
    R, k_pos = len(rows), 256
    qidx = W.bf16_normal((R, 8, 128), seed=52)
    w = W.uniform01((R, 8), seed=53)
    qd, wd = dev(qidx), dev(w)
    pool, npool, topk, ntopk = run_full(csa2, cache, qd, wd, [s for s, _ in rows],
                                        [n for _, n in rows], max(n for _, n in rows), k_blk, k_pos)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    for r, (s, nv) in enumerate(rows):
        if s >= len(n_list) or nv == 0:
            assert ntopk[r] == 0 and np.all(topk[r] == -1), r
            if k_blk:
                assert npool[r] == 0 and np.all(pool[r] == -1), r
            continue
        _, _, ikc, iks = ora[s]
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nv, k_blk, k_pos)
        if k_blk == 0:
            check_topk(topk[r], ntopk[r], ref, f"flat row {r}")
            continue
        check_full_row(csa2, cache, qd[r:r + 1], wd[r:r + 1], s, nv, pool[r], npool[r], topk[r],
                       ntopk[r], ref, k_blk, k_pos, f"row {r}")


@pytest.mark.parametrize("kind", ["outlier", "tied_block", "narrow_spread"])
def test_index_flat_selection_regimes(csa2, kind):
    """Score distributions that steer the selection off its common case:
    a few outliers far above the rest (the k-th score lies far below the
    maximum), thousands of identical top scores (a tie block larger than any
    candidate list), and scores that all lie within one octave."""
    n, k_pos = 20000, 512
    base = W.rms_rows(n, 128, seed=71).numpy()
    qidx = W.bf16_normal((2, 8, 128), seed=72)
    w = W.uniform01((2, 8), seed=73)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    ikc0, iks0 = oracle.quantize(base, 32)
    s0 = oracle.index_scores(qb[0], wn[0], ikc0, iks0, np.arange(n))
    ik = base.copy()
    if kind == "outlier":
        ik[:10] *= 200.0
    elif kind == "tied_block":
        ik[3000:9000] = 2.0 * base[int(np.argmax(s0))]
    else:
        med = np.median(s0[s0 > 0])
        band = np.flatnonzero((s0 > med) & (s0 < 1.6 * med))
        ik = base[band[np.arange(n) % len(band)]]
    lat = W.rms_rows(n, 512, seed=74).numpy()
    cache, ora = build_cache(csa2, [lat], [ik], n)
    _, _, ikc, iks = ora[0]
    _, _, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [0, 0], [n, n - 7], n, 0, k_pos)
    for r, nv in enumerate([n, n - 7]):
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nv, 0, k_pos)
        check_topk(topk[r], ntopk[r], ref, kind)


def test_index_reindex_on_oracle_pool(csa2):
    n_list = [9000, 3001]
    cache, ora = make_index_case(csa2, n_list, 9000, seed=23)
    rows = [(0, 9000), (1, 3001), (0, 8191), (1, 5)]
    R, k_blk, k_pos = len(rows), 300, 128
    q_full = W.bf16_normal((R, 8, 128), seed=31)
    w_full = W.uniform01((R, 8), seed=32)
    q_re = W.bf16_normal((R, 8, 128), seed=33)
    w_re = W.uniform01((R, 8), seed=34)
    pools = np.full((R, k_blk), -1, np.int32)
    npools = np.zeros(R, np.int32)
    refs = []
    for r, (s, nv) in enumerate(rows):
        _, _, ikc, iks = ora[s]
        f = oracle.full_layer_select(W.bf16_bits(q_full)[r], w_full.numpy()[r], ikc, iks, nv, k_blk, k_pos)
        pools[r, :len(f["pool"])] = f["pool"]
        npools[r] = len(f["pool"])
        refs.append(oracle.reindex_select(W.bf16_bits(q_re)[r], w_re.numpy()[r], ikc, iks, nv,
                                          f["pool"], k_pos))
    topk = torch.full((R, k_pos), -7, dtype=torch.int32, device="cuda")
    ntopk = torch.zeros(R, dtype=torch.int32, device="cuda")
    max_nvis = max(n for _, n in rows)
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_REINDEX, R, max_nvis, k_blk, k_pos)
    csa2.csa2_index_reindex(cache, dev(q_re), dev(w_re), dev([s for s, _ in rows], torch.int32),
                            dev([n for _, n in rows], torch.int32), max_nvis, dev(pools), dev(npools),
                            k_blk, k_pos, topk, ntopk, ws)
    torch.cuda.synchronize()
    topk, ntopk = topk.cpu().numpy(), ntopk.cpu().numpy()
    for r in range(R):
        check_topk(topk[r], ntopk[r], refs[r], "reindex")
    # flat reindex (no pool): every visible entry is a candidate
    ws2 = csa2.workspace(csa2.CSA2_OP_INDEX_REINDEX, R, max_nvis, 0, k_pos)
    topk_t = torch.full((R, k_pos), -7, dtype=torch.int32, device="cuda")
    ntopk_t = torch.zeros(R, dtype=torch.int32, device="cuda")
    csa2.csa2_index_reindex(cache, dev(q_re), dev(w_re), dev([s for s, _ in rows], torch.int32),
                            dev([n for _, n in rows], torch.int32), max_nvis, None, None, 0, k_pos,
                            topk_t, ntopk_t, ws2)
    torch.cuda.synchronize()
    for r, (s, nv) in enumerate(rows):
        _, _, ikc, iks = ora[s]
        ref = oracle.reindex_select(W.bf16_bits(q_re)[r], w_re.numpy()[r], ikc, iks, nv, None, k_pos)
        check_topk(topk_t.cpu().numpy()[r], ntopk_t.cpu().numpy()[r], ref, "reindex-flat")


def test_index_reindex_flat_many_rows(csa2):
    """Prefill Reindex: flat re-scoring of all visible entries for many query
    rows of a few sequences (no pool: the encoder keeps none), the rows of a
    sequence sharing key tiles in the many-row kernel."""
    n_list = [7000, 2500]
    cache, ora = make_index_case(csa2, n_list, 7000, seed=81)
    rows = [(0, 6980 + i) for i in range(20)] + [(1, 2490 + i) for i in range(11)] + [(0, 5), (1, 0)]
    R, k_pos = len(rows), 384
    q_re = W.bf16_normal((R, 8, 128), seed=82)
    w_re = W.uniform01((R, 8), seed=83)
    max_nvis = max(n for _, n in rows)
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_REINDEX, R, max_nvis, 0, k_pos)
    topk = torch.full((R, k_pos), -7, dtype=torch.int32, device="cuda")
    ntopk = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    csa2.csa2_index_reindex(cache, dev(q_re), dev(w_re), dev([s for s, _ in rows], torch.int32),
                            dev([n for _, n in rows], torch.int32), max_nvis, None, None, 0, k_pos,
                            topk, ntopk, ws)
    torch.cuda.synchronize()
    topk, ntopk = topk.cpu().numpy(), ntopk.cpu().numpy()
    qb, wn = W.bf16_bits(q_re), w_re.numpy()
    for r, (s, nv) in enumerate(rows):
        _, _, ikc, iks = ora[s]
        ref = oracle.reindex_select(qb[r], wn[r], ikc, iks, nv, None, k_pos)
        check_topk(topk[r], ntopk[r], ref, f"row {r}")


# ------------------------------------------------------------ S5-S6 attention
def attn_case(csa2, H, n_vis_list, topk_rows, swa_ends, seed=0, swa_len=200, window=128):
    S = len(n_vis_list)
    cap = max(n_vis_list)
    lat = [W.rms_rows(n, 512, seed=seed + i).numpy() for i, n in enumerate(n_vis_list)]
    ik = [np.zeros((n, 128), np.float32) for n in n_vis_list]
    cache, ora = build_cache(csa2, lat, ik, cap)
    swa = W.swa_rows_e4m3(S * swa_len, 512, seed=seed + 99).reshape(S, swa_len, 512)
    R = len(topk_rows)
    q = W.bf16_normal((R, H, 512), seed=seed + 7)
    k_pos = max(1, max(len(t) for t, _ in topk_rows))
    topk = np.full((R, k_pos), -1, np.int32)
    ntopk = np.zeros(R, np.int32)
    row_seq = np.zeros(R, np.int32)
    for r, (ids, s) in enumerate(topk_rows):
        topk[r, :len(ids)] = ids
        ntopk[r] = len(ids)
        row_seq[r] = s
    return dict(cache=cache, ora=ora, swa=swa, q=q, topk=topk, ntopk=ntopk, row_seq=row_seq,
                swa_end=np.asarray(swa_ends, np.int32), window=window, H=H)


def oracle_attn(c, r, q=None, scale=SCALE):
    s = int(c["row_seq"][r])
    kvc, kvs, _, _ = c["ora"][s]
    end = int(min(max(c["swa_end"][r], 0), c["swa"].shape[1]))
    rows = c["swa"][s, max(0, end - c["window"]):end].numpy()
    q = c["q"] if q is None else q
    return oracle.attend_row(W.bf16_bits(q[r]), kvc, kvs, c["topk"][r][:c["ntopk"][r]], rows, scale)


def pow2_bf16(x, e):
    """bf16 tensor x times 2^e (e broadcast against x), exact while the
    results stay bf16 normals."""
    return (x.double() * torch.pow(2.0, torch.as_tensor(e, dtype=torch.float64))).to(torch.bfloat16)


@pytest.mark.parametrize("split", [False, True], ids=["one_wg_per_row", "split_rows"])
@pytest.mark.parametrize("H", [16, 64])
def test_sparse_attn_global_fused_and_merge(csa2, H, split):
    rng = np.random.default_rng(H)
    nv = [3000, 700]
    rows = [(np.sort(rng.choice(3000, 512, replace=False)), 0),      # full Top-512
            (np.sort(rng.choice(700, 300, replace=False)), 1),       # ragged count
            (np.array([], np.int64), 0),                             # no global keys
            (np.sort(rng.choice(3000, 45, replace=False)), 0),
            (np.array([5, -1, 17, 699, -1]), 1)]                     # invalid ids skipped
    c = attn_case(csa2, H, nv, rows, swa_ends=[200, 128, 60, 0, 3], seed=H)
    R = len(rows)
    cache = c["cache"]
    q = dev(c["q"])
    row_seq = dev(c["row_seq"])
    topk = dev(c["topk"])
    ntopk = dev(c["ntopk"])
    swa = csa2.Swa(dev(c["swa"]), dev(c["swa_end"]), c["window"])
    refs = [oracle_attn(c, r) for r in range(R)]      # the oracle skips -1 ids as well
    k_pos = c["topk"].shape[1]
    ws_g = csa2.attn_workspace(R, H, k_pos, 0) if split else None
    ws_m = csa2.attn_workspace(R, H, 0, 128) if split else None
    ws_f = csa2.attn_workspace(R, H, k_pos, 128) if split else None
    if split:                  # few rows: every branch spreads over work-groups
        assert ws_g is not None and ws_m is not None and ws_f is not None
    # global branch only
    o = torch.empty((R, H, 512), device="cuda")
    lse = torch.empty((R, H), device="cuda")
    csa2.csa2_sparse_attn(cache, q, row_seq, topk, ntopk, SCALE, o, lse, workspace=ws_g)
    torch.cuda.synchronize()
    check_attention(o.cpu().numpy(), lse.cpu().numpy(), np.stack([x["o_g"] for x in refs]),
                    np.stack([x["lse_g"] for x in refs]), "global")
    # then the SWA branch merged onto it
    csa2.csa2_swa_merge(q, row_seq, swa, SCALE, o, lse, workspace=ws_m)
    torch.cuda.synchronize()
    check_attention(o.cpu().numpy(), lse.cpu().numpy(), np.stack([x["o"] for x in refs]),
                    np.stack([x["lse"] for x in refs]), "merged")
    # fused: both branches in one softmax
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    csa2.csa2_sparse_attn(cache, q, row_seq, topk, ntopk, SCALE, o2, lse2, swa=swa, workspace=ws_f)
    torch.cuda.synchronize()
    check_attention(o2.cpu().numpy(), lse2.cpu().numpy(), np.stack([x["o"] for x in refs]),
                    np.stack([x["lse"] for x in refs]), "fused")


@pytest.mark.parametrize("H,n_rows,k_pos,window,split", [
    (32, 3, 97, 100, True),       # 32 heads; Top-K and window not multiples of the tile
    (32, 3, 1000, 100, True),     # the same with a long Top-K list
    (32, 3, 97, 100, False),
    (16, 1, 2048, 1024, True),    # 96 tiles over 48 work-groups: the merge's loop past 16 splits
    (64, 200, 64, 32, True),      # 200 rows: no split even with a workspace given
    (16, 5, 33, 1, True),         # one-row window, a 1-key second tile
    (16, 5, 1100, 1, True),       # a long Top-K list, a one-row window
    (16, 100, 512, 128, True),    # 100 rows: a few splits per row
    (32, 40, 300, 70, True),      # 32 heads x 40 rows: splits of two head groups
    (16, 200, 200, 128, True),    # 200 rows of 16 heads: one work-group per row
    (16, 300, 200, 128, False),   # 300 rows, an odd number of Top-K tiles per row
    (32, 130, 97, 100, True),     # 32 heads x 130 rows, split
    (16, 1100, 512, 128, False),  # many rows (Top-512 + 128 SWA rows)
    (32, 520, 97, 100, True),     # 32 heads x 520 rows, ragged
], ids=["h32_ragged_split", "h32_long_split", "h32_ragged", "h16_2048_1024_48splits", "h64_200rows",
        "h16_tiny_tiles", "h16_long_tiny_window", "h16_100rows", "h32_40rows", "h16_200rows", "h16_300rows",
        "h32_130rows", "h16_1100rows", "h32_520rows"])
def test_sparse_attn_shapes(csa2, H, n_rows, k_pos, window, split):
    rng = np.random.default_rng(k_pos + window)
    n_vis = max(3000, k_pos + 10)
    rows = []
    for r in range(n_rows):
        cnt = k_pos if r % 3 == 0 else int(rng.integers(0, k_pos + 1))
        rows.append((np.sort(rng.choice(n_vis, cnt, replace=False)), 0))
    swa_len = window + 50
    ends = [swa_len if r % 2 == 0 else int(rng.integers(0, swa_len + 1)) for r in range(n_rows)]
    c = attn_case(csa2, H, [n_vis], rows, swa_ends=ends, seed=H + window, swa_len=swa_len, window=window)
    assert c["topk"].shape[1] == k_pos
    ws = csa2.attn_workspace(n_rows, H, k_pos, window) if split else None
    if split:
        assert ws is not None      # rows past 191 ignore it
    swa = csa2.Swa(dev(c["swa"]), dev(c["swa_end"]), window)
    o = torch.empty((n_rows, H, 512), device="cuda")
    lse = torch.empty((n_rows, H), device="cuda")
    csa2.csa2_sparse_attn(c["cache"], dev(c["q"]), dev(c["row_seq"]), dev(c["topk"]), dev(c["ntopk"]),
                          SCALE, o, lse, swa=swa, workspace=ws)
    torch.cuda.synchronize()
    refs = [oracle_attn(c, r) for r in range(n_rows)]
    check_attention(o.cpu().numpy(), lse.cpu().numpy(), np.stack([x["o"] for x in refs]),
                    np.stack([x["lse"] for x in refs]), f"H{H} k{k_pos} w{window}")
    # the same result as global attention followed by the SWA merge
    ws_g = csa2.attn_workspace(n_rows, H, k_pos, 0) if split else None
    ws_m = csa2.attn_workspace(n_rows, H, 0, window) if split else None
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    csa2.csa2_sparse_attn(c["cache"], dev(c["q"]), dev(c["row_seq"]), dev(c["topk"]), dev(c["ntopk"]),
                          SCALE, o2, lse2, workspace=ws_g)
    csa2.csa2_swa_merge(dev(c["q"]), dev(c["row_seq"]), swa, SCALE, o2, lse2, workspace=ws_m)
    torch.cuda.synchronize()
    check_attention(o2.cpu().numpy(), lse2.cpu().numpy(), np.stack([x["o"] for x in refs]),
                    np.stack([x["lse"] for x in refs]), f"H{H} k{k_pos} w{window} merged")


@pytest.mark.parametrize("H", [16, 32])
def test_attention_quarters_reuse_one_workspace(csa2, H):
    """Very few rows split over key ranges and channel quarters count the
    arrivals of their work-groups in the workspace's first 16 KiB, and every
    call leaves those counters at zero: one zero-filled workspace then serves
    calls of other row counts in turn, with and without the SWA merge (which
    counts a second time for its lse)."""
    rng = np.random.default_rng(41 + H)
    n_max = 16 // (H // 16)
    rows = [(np.sort(rng.choice(3000, int(rng.integers(1, 513)), replace=False)), 0) for _ in range(n_max)]
    c = attn_case(csa2, H, [3000], rows, swa_ends=[200 - 7 * r for r in range(n_max)], seed=5 + H)
    k_pos = c["topk"].shape[1]
    ws = csa2.attn_workspace(n_max, H, k_pos, 128)
    assert ws is not None
    swa = csa2.Swa(dev(c["swa"]), dev(c["swa_end"]), c["window"])
    refs = [oracle_attn(c, r) for r in range(n_max)]
    for n in (n_max, 2, n_max - 1, 1):
        assert csa2.csa2_attn_workspace_size(n, H, k_pos, 128) <= ws.numel()
        sl = slice(0, n)
        o = torch.empty((n, H, 512), device="cuda")
        lse = torch.empty((n, H), device="cuda")
        csa2.csa2_sparse_attn(c["cache"], dev(c["q"][sl]), dev(c["row_seq"][sl]), dev(c["topk"][sl]),
                              dev(c["ntopk"][sl]), SCALE, o, lse, swa=swa, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ws[:16384] == 0), f"counters left set after {n} rows"
        check_attention(o.cpu().numpy(), lse.cpu().numpy(), np.stack([x["o"] for x in refs[:n]]),
                        np.stack([x["lse"] for x in refs[:n]]), f"H{H} {n} rows")
        # global keys first, then the SWA rows merged in, on the same workspace
        o2 = torch.empty_like(o)
        lse2 = torch.empty_like(lse)
        csa2.csa2_sparse_attn(c["cache"], dev(c["q"][sl]), dev(c["row_seq"][sl]), dev(c["topk"][sl]),
                              dev(c["ntopk"][sl]), SCALE, o2, lse2, workspace=ws)
        csa2.csa2_swa_merge(dev(c["q"][sl]), dev(c["row_seq"][sl]), swa, SCALE, o2, lse2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ws[:16384] == 0), f"counters left set after the merge of {n} rows"
        check_attention(o2.cpu().numpy(), lse2.cpu().numpy(), np.stack([x["o"] for x in refs[:n]]),
                        np.stack([x["lse"] for x in refs[:n]]), f"H{H} {n} rows merged")


@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("split", [False, True])
def test_attention_empty_everything(csa2, split, H):
    rows = [(np.array([], np.int64), 0), (np.array([-1, -1], np.int64), 0)]
    c = attn_case(csa2, H, [100], rows, swa_ends=[0, -5], seed=3)
    o = torch.full((2, H, 512), 5.0, device="cuda")
    lse = torch.zeros((2, H), device="cuda")
    swa = csa2.Swa(dev(c["swa"]), dev(c["swa_end"]), 128)
    ws = csa2.attn_workspace(2, H, c["topk"].shape[1], 128) if split else None
    csa2.csa2_sparse_attn(c["cache"], dev(c["q"]), dev(c["row_seq"]), dev(c["topk"]),
                          dev(c["ntopk"]), SCALE, o, lse, swa=swa, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("split", [False, True], ids=["one_wg_per_row", "split_rows"])
@pytest.mark.parametrize("H", [16, 64])
def test_attention_q_range(csa2, H, split):
    """Q anywhere in the finite bf16 range.  (a) q * 2^e with the softmax
    scale times 2^-e has the same logits, for e from -80 (a head's largest
    |q| near 2^-78) to 120 (near the largest finite bf16); (b) the heads of
    one row 2^-80 .. 2^60 apart, so flat and one-hot softmaxes sit side by
    side.  Against the oracle on the very same inputs."""
    rng = np.random.default_rng(11 + H)
    rows = [(np.sort(rng.choice(3000, 300, replace=False)), 0),
            (np.sort(rng.choice(3000, 77, replace=False)), 0)]
    c = attn_case(csa2, H, [3000], rows, swa_ends=[200, 90], seed=31 + H)
    R, k_pos = len(rows), c["topk"].shape[1]
    swa = csa2.Swa(dev(c["swa"]), dev(c["swa_end"]), c["window"])
    ws = csa2.attn_workspace(R, H, k_pos, c["window"]) if split else None
    if split:
        assert ws is not None

    def check(q, scale, what):
        o = torch.empty((R, H, 512), device="cuda")
        lse = torch.empty((R, H), device="cuda")
        csa2.csa2_sparse_attn(c["cache"], dev(q), dev(c["row_seq"]), dev(c["topk"]), dev(c["ntopk"]),
                              scale, o, lse, swa=swa, workspace=ws)
        torch.cuda.synchronize()
        refs = [oracle_attn(c, r, q, scale) for r in range(R)]
        check_attention(o.cpu().numpy(), lse.cpu().numpy(), np.stack([x["o"] for x in refs]),
                        np.stack([x["lse"] for x in refs]), what)

    for e in (-80, -30, 40, 120):
        q = pow2_bf16(c["q"], e)
        assert torch.all(torch.isfinite(q.float()))
        check(q, SCALE * 2.0 ** -e, f"q * 2^{e}")
    e_head = np.array([-80, -40, 0, 30, 60])[np.arange(H) % 5]
    check(pow2_bf16(c["q"], e_head[None, :, None]), SCALE, "heads 2^-80 .. 2^60")


@pytest.mark.parametrize("shape", ["rows_one_per_wg", "many_rows_flat", "many_rows_block"])
def test_index_q_range(csa2, shape):
    """q_idx anywhere in the finite bf16 range: a row's (or one head's) q_idx
    times 2^e with its weight times 2^-e, for e from -80 to 120, and a row
    whose eight heads lie 2^-80 .. 2^110 apart.  The selection must match the
    oracle's on the very same inputs (the scores stay of order one, so the
    tie tolerance is meaningful).  Rows of distinct sequences are scored one
    per work-group, many rows of one sequence by the many-row kernel."""
    n = 4096
    cache, ora = make_index_case(csa2, [n], n, seed=61)
    exps = [-80, -30, 0, 30, 90, 120]
    mixed = [-80, -50, -20, 0, 20, 50, 80, 110]
    if shape == "rows_one_per_wg":
        R, k_blk = 7, 64
        nvis = [n, n - 5, 3000, n, 1000, n, n - 1]
    else:
        R, k_blk = 16, (0 if shape == "many_rows_flat" else 64)
        nvis = [n - 15 + r for r in range(R)]
    E = np.array([[exps[r % len(exps)]] * 8 for r in range(R)], np.float64)
    E[R - 1] = mixed
    if R > 8:
        E[5] = mixed[::-1]
    qidx = pow2_bf16(W.bf16_normal((R, 8, 128), seed=62), E[:, :, None])
    assert torch.all(torch.isfinite(qidx.float()))
    w = (W.uniform01((R, 8), seed=63).double() * torch.from_numpy(np.power(2.0, -E))).float()
    k_pos = 512
    qd, wd = dev(qidx), dev(w)
    pool, npool, topk, ntopk = run_full(csa2, cache, qd, wd, [0] * R, nvis, max(nvis), k_blk, k_pos)
    qb, wn = W.bf16_bits(qidx), w.numpy()
    _, _, ikc, iks = ora[0]
    for r in range(R):
        ref = oracle.full_layer_select(qb[r], wn[r], ikc, iks, nvis[r], k_blk, k_pos)
        if k_blk:
            check_full_row(csa2, cache, qd[r:r + 1], wd[r:r + 1], 0, nvis[r], pool[r], npool[r], topk[r],
                           ntopk[r], ref, k_blk, k_pos, f"row {r} e {E[r].tolist()}")
        else:
            check_topk(topk[r], ntopk[r], ref, f"row {r} e {E[r].tolist()}")


# ------------------------------------------------------------- one layer e2e
def test_tiny_full_decode_end_to_end(csa2):
    """The tiny Full-mode decode (batch 1, 4,096 entries, 64 blocks -> 512,
    16 heads, SWA 128): quantise, index, attend + merge, all on the GPU,
    compared with the oracle pipeline on the same fp32 inputs."""
    wl = W.WORKLOADS[0]
    T = wl.ctx
    lat = W.rms_rows(T, 512, seed=W.seed_for(wl.seed, W.T_LATENT)).numpy()
    ik = W.rms_rows(T, 128, seed=W.seed_for(wl.seed, W.T_IKEY)).numpy()
    cache, ora = build_cache(csa2, [lat], [ik], T)
    kvc, kvs, ikc, iks = ora[0]
    np.testing.assert_array_equal(cache.ik_codes[0].cpu().numpy(), ikc)
    np.testing.assert_array_equal(cache.kv_scales[0].cpu().numpy(), kvs)
    qidx = W.bf16_normal((1, 8, 128), seed=W.seed_for(wl.seed, W.T_QIDX))
    w = W.uniform01((1, 8), seed=W.seed_for(wl.seed, W.T_W))
    q = W.bf16_normal((1, wl.heads, 512), seed=W.seed_for(wl.seed, W.T_Q))
    swa = W.swa_rows_e4m3(wl.swa, 512, seed=W.seed_for(wl.seed, W.T_SWA)).reshape(1, wl.swa, 512)
    pool, npool, topk, ntopk = run_full(csa2, cache, dev(qidx), dev(w), [0], [T], T, wl.k_blk, wl.k_pos)
    ref = oracle.full_layer_select(W.bf16_bits(qidx)[0], w.numpy()[0], ikc, iks, T, wl.k_blk, wl.k_pos)
    check_full_row(csa2, cache, dev(qidx), dev(w), 0, T, pool[0], npool[0], topk[0], ntopk[0], ref,
                   wl.k_blk, wl.k_pos, "tiny decode")
    assert ntopk[0] == 512
    if not np.array_equal(topk[0], ref["topk"]):
        # an accepted tie swap: attention is compared on the oracle's list
        topk, ntopk = ref["topk"][None], np.array([ref["n_topk"]], np.int32)
    o = torch.empty((1, wl.heads, 512), device="cuda")
    lse = torch.empty((1, wl.heads), device="cuda")
    sw = csa2.Swa(dev(swa), dev(np.array([wl.swa], np.int32)), wl.swa)
    csa2.csa2_sparse_attn(cache, dev(q), dev(np.array([0], np.int32)), dev(topk), dev(ntopk),
                          SCALE, o, lse, swa=sw)
    torch.cuda.synchronize()
    r = oracle.attend_row(W.bf16_bits(q)[0], kvc, kvs, ref["topk"], swa[0].numpy(), SCALE)
    check_attention(o.cpu().numpy()[0], lse.cpu().numpy()[0], r["o"], r["lse"], "tiny decode")
