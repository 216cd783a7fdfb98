"""Comparison rules shared by the GPU parity tests.

  * FP4 codes and scales: bit-exact.
  * Top-K / pool index sets: equal, except that an index may be swapped for
    another whose oracle score lies within 1e-5 * max(1, |s_k|) of the
    oracle's k-th score s_k (fp32 on the GPU vs fp64 in the oracle).
  * Attention: per (row, head), max |o - o_ref| <= 2e-3 * max |o_ref|; the
    log-sum-exp within 2e-3 * max(1, |lse_ref|).
"""
import numpy as np

TIE_REL = 1e-5
ATTN_REL = 2e-3


def check_selection(gpu_ids, gpu_n, ora_ids, ora_n, ora_score_of, what="topk"):
    """gpu_ids / ora_ids: int arrays (ascending, -1 padded); ora_score_of(id)
    returns the oracle's fp64 score of an id."""
    gpu_ids = np.asarray(gpu_ids)
    ora_ids = np.asarray(ora_ids)
    assert int(gpu_n) == int(ora_n), f"{what}: count {gpu_n} != oracle {ora_n}"
    n = int(ora_n)
    g = gpu_ids[:n]
    assert np.all(gpu_ids[n:] == -1), f"{what}: padding is not -1"
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
    err = np.abs(o[ne] - o_ref[ne]).max(axis=1)
    ref = np.abs(o_ref[ne]).max(axis=1)
    rel = err / np.maximum(ref, 1e-30)
    worst = float(rel.max())
    assert worst <= ATTN_REL, f"{what}: max relative error {worst:.3e} > {ATTN_REL}"
    lerr = np.abs(lse[ne] - lse_ref[ne]) / np.maximum(1.0, np.abs(lse_ref[ne]))
    assert float(lerr.max()) <= ATTN_REL, f"{what}: lse error {float(lerr.max()):.3e}"
    return worst
