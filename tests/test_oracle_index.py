"""Pins for the oracle's indexer, hierarchical pool and Top-K (CPU only).

  * index scores against an independent numpy fp64 computation (keys decoded
    through torch's float8_e4m3fn and the OCP E2M1 table, then matmul, ReLU,
    weighted sum over heads);
  * block pool and Top-K against the properties that define a ranking
    selection uniquely (count, every kept value >= every dropped value, ties at
    the boundary resolved to the lower index, ascending output);
  * the pages' constant candidate bound: at most 2,048 blocks x 8 = 16,384
    candidates per query at any context length (P3 '레이어 40개 가운데 4개만
    전역 캐시를 만듭니다'; P1 '무엇과 다른가');
  * the hierarchy invariant: with block max aggregation and k_blk >= k_pos,
    Top-K inside the pool equals Top-K over every visible entry.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "pages_numbers.json")) as f:
    PAGES = json.load(f)
with open(os.path.join(GOLD, "ocp_e2m1_values.json")) as f:
    E2M1 = np.array(json.load(f)["magnitudes"])


def decode_keys_independently(codes, scales, group):
    """FP4 planes -> fp64 via the OCP E2M1 table and torch's E4M3 decode."""
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    s = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).double().numpy()
    return mag * np.repeat(s, group, axis=1)


def make_index_inputs(n, seed):
    keys = workloads.rms_rows(n, 128, seed=seed).numpy()
    ikc, iks = oracle.quantize(keys, oracle.IK_GROUP)
    q = workloads.bf16_normal((8, 128), seed=seed + 1)
    w = workloads.uniform01((8,), seed=seed + 2).numpy()
    return ikc, iks, workloads.bf16_bits(q), q.double().numpy(), w


def check_ranking_selection(values, kept, k):
    """`kept` (ascending positions) must be the unique top-k of `values`
    under (value descending, position ascending)."""
    n = len(values)
    kept = np.asarray(kept, np.int64)
    assert len(kept) == min(k, n)
    assert np.all(np.diff(kept) > 0)
    if len(kept) == n:
        return
    mask = np.zeros(n, bool)
    mask[kept] = True
    kmin = values[mask].min()
    dmax = values[~mask].max()
    assert kmin >= dmax
    if kmin == dmax:
        tied_kept = np.where(mask & (values == kmin))[0]
        tied_drop = np.where(~mask & (values == kmin))[0]
        assert tied_kept.max() < tied_drop.min()


def test_index_scores_match_numpy_fp64():
    ikc, iks, qbits, q, w = make_index_inputs(300, seed=21)
    ent = np.arange(300, dtype=np.int64)[::-1].copy()        # any order of candidates
    got = oracle.index_scores(qbits, w, ikc, iks, ent)
    k = decode_keys_independently(ikc, iks, oracle.IK_GROUP)[ent]
    ref = np.maximum(q @ k.T, 0.0).T @ w.astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_index_scores_relu_drops_negative_heads():
    # all-negative head products contribute nothing; a single positive head
    # contributes w_h * d_h exactly.
    keys = np.zeros((1, 128), np.float32)
    keys[0, 0] = 6.0                            # decodes to exactly 6 (scale 1)
    ikc, iks = oracle.quantize(keys, 32)
    q = torch.zeros(8, 128, dtype=torch.bfloat16)
    q[:, 0] = -1.0
    q[3, 0] = 2.0
    w = np.linspace(0.1, 0.8, 8).astype(np.float32)
    got = oracle.index_scores(workloads.bf16_bits(q), w, ikc, iks, np.array([0], np.int64))
    assert got[0] == pytest.approx(float(w[3]) * 12.0, rel=0, abs=1e-12)


@pytest.mark.parametrize("n_vis,k_blk", [(1, 4), (13, 2), (4096, 64), (5003, 100), (640, 2048)])
def test_block_pool_properties(n_vis, k_blk):
    rng = np.random.default_rng(n_vis)
    scores = rng.integers(0, 50, size=n_vis).astype(np.float64)   # many exact ties
    pool, bscores = oracle.block_pool(scores, k_blk)
    nb = (n_vis + 7) // 8
    padded = np.full(nb * 8, -np.inf)
    padded[:n_vis] = scores
    np.testing.assert_array_equal(bscores, padded.reshape(nb, 8).max(axis=1))
    check_ranking_selection(bscores, pool, k_blk)


@pytest.mark.parametrize("n_vis", [8, 1000, 16384, 16391, 131072, 1 << 20])
def test_candidate_pool_is_bounded_by_16384(n_vis):
    k_blk = PAGES["pool_blocks"]["value"]
    bound = PAGES["pool_candidates"]["value"]
    assert k_blk * PAGES["block_positions"]["value"] == bound
    scores = np.random.default_rng(n_vis).random(n_vis)
    pool, _ = oracle.block_pool(scores, k_blk)
    cand = oracle.pool_entries(pool, n_vis)
    assert len(cand) <= bound
    if n_vis <= bound:
        assert len(cand) == n_vis
    elif n_vis % 8 == 0:
        assert len(cand) == bound
    assert np.all(cand < n_vis) and np.all(np.diff(cand) > 0)


@pytest.mark.parametrize("n,k", [(0, 5), (3, 5), (10, 10), (1000, 512), (777, 64)])
def test_topk_properties(n, k):
    rng = np.random.default_rng(n + k)
    scores = rng.integers(0, 20, size=n).astype(np.float64)
    cand = np.sort(rng.choice(10 * n + 1, size=n, replace=False)).astype(np.int64)
    tk, m = oracle.topk(scores, cand, k)
    assert m == min(n, k)
    assert np.all(tk[m:] == -1)
    pos = np.searchsorted(cand, tk[:m])
    assert np.array_equal(cand[pos], tk[:m])
    check_ranking_selection(scores, pos, k)


def test_hierarchy_equals_direct_topk_under_max_pooling():
    ikc, iks, qbits, _, w = make_index_inputs(4096, seed=31)
    hier = oracle.full_layer_select(qbits, w, ikc, iks, 4096, k_blk=64, k_pos=48)
    flat = oracle.full_layer_select(qbits, w, ikc, iks, 4096, k_blk=0, k_pos=48)
    assert hier["n_topk"] == flat["n_topk"] == 48
    assert np.array_equal(hier["topk"], flat["topk"])
    # and the pool's re-scores equal the scan's scores of the same entries
    np.testing.assert_array_equal(hier["cand_scores"], hier["entry_scores"][hier["cand"]])


def test_tiny_decode_keeps_the_whole_pool():
    # 64 blocks of 8 = 512 candidates, Top-512 keeps all of them
    ikc, iks, qbits, _, w = make_index_inputs(4096, seed=41)
    r = oracle.full_layer_select(qbits, w, ikc, iks, 4096, k_blk=64, k_pos=512)
    assert r["n_topk"] == 512
    assert np.array_equal(r["topk"].astype(np.int64), r["cand"])


def test_reindex_rescoring_is_confined_to_the_pool():
    ikc, iks, qbits, _, w = make_index_inputs(3000, seed=51)
    full = oracle.full_layer_select(qbits, w, ikc, iks, 3000, k_blk=40, k_pos=64)
    q2 = workloads.bf16_bits(workloads.bf16_normal((8, 128), seed=77))
    w2 = workloads.uniform01((8,), seed=78).numpy()
    re = oracle.reindex_select(q2, w2, ikc, iks, 3000, full["pool"], 64)
    assert set(re["topk"][:re["n_topk"]]) <= set(full["cand"].tolist())
    assert len(re["cand"]) == 320
