"""Comparison rules shared by the GPU parity tests.

  * FP4 codes and scales: bit-exact.
  * Top-K / pool index sets: every GPU id must be a valid candidate (inside
    the row's block range, or one of its candidate entries) before anything
    else is looked at; then the sets must be equal, except that an index may
    be swapped for another whose oracle score lies within
    1e-5 * max(1, |s_k|) of the oracle's k-th score s_k (fp32 on the GPU vs
    fp64 in the oracle).
  * Attention: per (row, head), max |o - o_ref| <= 2e-3 * max |o_ref|; the
    log-sum-exp within 2e-3 * max(1, |lse_ref|).
"""
import numpy as np

TIE_REL = 1e-5
ATTN_REL = 2e-3


def check_selection(gpu_ids, gpu_n, ora_ids, ora_n, ora_score_of, what="topk", *, valid):
    """gpu_ids / ora_ids: int arrays (ascending, -1 padded); ora_score_of(id)
    returns the oracle's fp64 score of an id.  ``valid`` names the ids a
    selection may return: an int n (ids 0 .. n-1) or an array of candidate
    ids.  Returns the number of accepted tie swaps."""
    gpu_ids = np.asarray(gpu_ids)
    ora_ids = np.asarray(ora_ids)
    assert 0 <= int(gpu_n) <= len(gpu_ids), f"{what}: count {gpu_n} outside [0, {len(gpu_ids)}]"
    assert int(gpu_n) == int(ora_n), f"{what}: count {gpu_n} != oracle {ora_n}"
    n = int(ora_n)
    g = gpu_ids[:n].astype(np.int64)
    assert np.all(gpu_ids[n:] == -1), f"{what}: padding is not -1"
    if isinstance(valid, (int, np.integer)):
        bad = g[(g < 0) | (g >= int(valid))]
        assert bad.size == 0, f"{what}: ids {bad[:8].tolist()} outside [0, {int(valid)})"
    else:
        bad = g[~np.isin(g, np.asarray(valid, np.int64))]
        assert bad.size == 0, f"{what}: ids {bad[:8].tolist()} are not candidates"
    assert np.all(np.diff(g) > 0), f"{what}: not strictly ascending"
    if n == 0:
        return 0
    o = ora_ids[:n]
    k_score = min(ora_score_of(int(j)) for j in o)
    tol = TIE_REL * max(1.0, abs(k_score))
    diff = set(g.tolist()) ^ set(o.tolist())
    for j in diff:
        s = ora_score_of(int(j))
        assert abs(s - k_score) <= tol, (
            f"{what}: id {j} differs with oracle score {s!r}, k-th score {k_score!r}")
    return len(diff) // 2


def check_pool(gpu_pool, gpu_n, ref, what="pool"):
    """Block pool of one row against an oracle ``full_layer_select`` result
    (block ids in [0, #visible blocks), ranked by block score)."""
    bs = ref["block_scores"]
    k = len(gpu_pool)
    ora = np.full(k, -1, np.int64)
    ora[:len(ref["pool"])] = ref["pool"]
    return check_selection(gpu_pool, gpu_n, ora, len(ref["pool"]), lambda b: bs[b], what,
                           valid=len(bs))


def check_topk(gpu_ids, gpu_n, ref, what="topk"):
    """Top-K of one row against an oracle selection result (``cand`` /
    ``cand_scores`` / ``topk`` / ``n_topk``): ids must be candidates."""
    sc = dict(zip(ref["cand"].tolist(), ref["cand_scores"].tolist()))
    return check_selection(gpu_ids, gpu_n, ref["topk"], ref["n_topk"], lambda j: sc[j], what,
                           valid=ref["cand"])


def check_attention(o, lse, o_ref, lse_ref, what="attention"):
    """o: [H, 512] or [R, H, 512]; compared per (row, head)."""
    o = np.asarray(o, np.float64).reshape(-1, o_ref.shape[-1])
    o_ref = np.asarray(o_ref, np.float64).reshape(-1, o_ref.shape[-1])
    lse = np.asarray(lse, np.float64).reshape(-1)
    lse_ref = np.asarray(lse_ref, np.float64).reshape(-1)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty-set rows differ"
    assert np.all(o[empty] == 0), f"{what}: empty rows must be zero"
    ne = ~empty
    if not ne.any():
        return 0.0
    assert np.all(np.isfinite(o[ne])) and np.all(np.isfinite(lse[ne])), f"{what}: non-finite output"
    err = np.abs(o[ne] - o_ref[ne]).max(axis=1)
    ref = np.abs(o_ref[ne]).max(axis=1)
    rel = err / np.maximum(ref, 1e-30)
    worst = float(rel.max())
    assert worst <= ATTN_REL, f"{what}: max relative error {worst:.3e} > {ATTN_REL}"
    lerr = np.abs(lse[ne] - lse_ref[ne]) / np.maximum(1.0, np.abs(lse_ref[ne]))
    assert float(lerr.max()) <= ATTN_REL, f"{what}: lse error {float(lerr.max()):.3e}"
    return worst


def reindex_row(csa2, cache, q_idx_row, w_row, seq, n_vis, pool, k_blk, k_pos):
    """Runs csa2_index_reindex for one row on the given pool (block ids) and
    returns its (topk, n_topk) on the host.  q_idx_row / w_row: device
    tensors [1, 8, 128] bf16 / [1, 8] fp32."""
    import torch

    dev = q_idx_row.device
    pool = np.asarray(pool, np.int32)
    pb = torch.full((1, k_blk), -1, dtype=torch.int32, device=dev)
    if len(pool):
        pb[0, :len(pool)] = torch.from_numpy(pool).to(dev)
    npb = torch.tensor([len(pool)], dtype=torch.int32, device=dev)
    tk = torch.full((1, k_pos), -7, dtype=torch.int32, device=dev)
    nt = torch.full((1,), -7, dtype=torch.int32, device=dev)
    i32 = lambda v: torch.tensor([int(v)], dtype=torch.int32, device=dev)
    nv = int(n_vis)
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_REINDEX, 1, nv, k_blk, k_pos, device=dev)
    csa2.csa2_index_reindex(cache, q_idx_row.contiguous(), w_row.contiguous(), i32(seq), i32(nv), nv,
                            pb, npb, k_blk, k_pos, tk, nt, ws)
    torch.cuda.synchronize()
    return tk.cpu().numpy()[0], int(nt.cpu()[0])


def check_reindex_row(csa2, cache, q_idx_row, w_row, seq, n_vis, gpu_pool, gpu_npool, gpu_topk,
                      gpu_ntopk, ref, oracle_pool, k_blk, k_pos, what="reindex"):
    """Top-K of one row re-scored inside a pool.  ``ref`` is the oracle's
    selection inside ``oracle_pool``.  When the GPU's own pool equals the
    oracle's, the GPU's Top-K is checked as it stands; when it differs (an
    accepted tie swap upstream), the same stage is re-run on the oracle's pool
    (csa2_index_reindex with the same query: the same re-scoring and
    selection kernels) and that result is checked.  No row goes unchecked."""
    if np.array_equal(np.asarray(gpu_pool)[:int(gpu_npool)], np.asarray(oracle_pool)):
        return check_topk(gpu_topk, gpu_ntopk, ref, what)
    tk, n = reindex_row(csa2, cache, q_idx_row, w_row, seq, n_vis, oracle_pool, k_blk, k_pos)
    return check_topk(tk, n, ref, f"{what} (on the oracle's pool)")


def check_full_row(csa2, cache, q_idx_row, w_row, seq, n_vis, gpu_pool, gpu_npool, gpu_topk,
                   gpu_ntopk, ref, k_blk, k_pos, what="full"):
    """Full-layer block mode, one row: the pool, then the Top-K inside it
    (re-run on the oracle's pool when the pools differ by tie swaps)."""
    check_pool(gpu_pool, gpu_npool, ref, f"{what} pool")
    return check_reindex_row(csa2, cache, q_idx_row, w_row, seq, n_vis, gpu_pool, gpu_npool,
                             gpu_topk, gpu_ntopk, ref, ref["pool"], k_blk, k_pos, f"{what} topk")
