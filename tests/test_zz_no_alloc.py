"""csa2_index_full_noalloc (static per-device scratch, no workspace) against
csa2_index_full (caller workspace) through the C ABI: two calls in a row, the
second on a smaller input, each compared with the workspace entry point on
the same inputs.  Both run the same kernels in the same order, so pools and
Top-K lists must be identical (stronger than the tie rule); the first call
also runs the oracle on a sampled row, so the shared path stays pinned."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_full_row

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_compressed_sparse_e2m1_amd as m
    m.load()
    return m


def _case(csa2, n_list, rows, k_blk, k_pos, seed):
    cap = max(n_list) + 5
    cache = csa2.Cache(len(n_list), cap)
    ora = []
    for s, n in enumerate(n_list):
        ik = W.rms_rows(n, 128, seed=seed + s).numpy()
        dst = torch.arange(n, dtype=torch.int64, device="cuda") + s * cap
        csa2.csa2_quantize_fp4(torch.from_numpy(ik).cuda(), 32, cache.ik_codes, cache.ik_scales,
                               dst_rows=dst)
        ora.append(oracle.quantize(ik, 32))
    R = len(rows)
    q = W.bf16_normal((R, 8, 128), seed=seed + 100).cuda()
    w = W.uniform01((R, 8), seed=seed + 101).cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    seqs, nvis = i32([s for s, _ in rows]), i32([n for _, n in rows])
    max_nvis = max(n for _, n in rows)

    def outputs():
        return (torch.full((R, k_blk), -7, dtype=torch.int32, device="cuda"),
                torch.full((R,), -7, dtype=torch.int32, device="cuda"),
                torch.full((R, k_pos), -7, dtype=torch.int32, device="cuda"),
                torch.full((R,), -7, dtype=torch.int32, device="cuda"))

    ref = outputs()
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_FULL, R, max_nvis, k_blk, k_pos)
    csa2.csa2_index_full(cache, q, w, seqs, nvis, max_nvis, k_blk, k_pos, *ref, ws)
    got = outputs()
    csa2.csa2_index_full_noalloc(cache, q, w, seqs, nvis, max_nvis, k_blk, k_pos, *got)
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("pool", "n_pool", "topk", "n_topk")):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy(), err_msg=name)
    return cache, ora, q, w, [t.cpu().numpy() for t in got]


def test_noalloc_matches_workspace_entry_point_twice(csa2):
    # first call: two selection levels for the block pool (17,501 blocks)
    # over three sequences, ragged rows, an empty row
    rows = [(0, 140001), (1, 99999), (2, 5003), (0, 131072), (1, 0)]
    cache, ora, q, w, (pool, npool, topk, ntopk) = _case(
        csa2, [140001, 99999, 5003], rows, 2048, 512, seed=900)
    ikc, iks = ora[2]
    ref = oracle.full_layer_select(W.bf16_bits(q)[2], w.cpu().numpy()[2], ikc, iks, 5003, 2048, 512)
    check_full_row(csa2, cache, q[2:3], w[2:3], 2, 5003, pool[2], npool[2], topk[2], ntopk[2], ref,
                   2048, 512, "noalloc row 2")
    assert npool[4] == 0 and ntopk[4] == 0
    # second call, smaller: one level, fewer rows, other k values; the scratch
    # still holds the first call's contents
    _case(csa2, [3000, 777], [(1, 777), (0, 2999)], 100, 64, seed=901)


def test_noalloc_rejects_sizes_beyond_its_scratch(csa2):
    cache = csa2.Cache(1, 40000)
    R, nv = 200, 40000                      # flat mode: 200 x 40,000 x 4 B > 16 MiB
    assert csa2.csa2_workspace_size(csa2.CSA2_OP_INDEX_FULL, R, nv, 0, 512) > csa2.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((R, 8, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((R, 8), dtype=torch.float32, device="cuda")
    seqs = torch.zeros(R, dtype=torch.int32, device="cuda")
    nvis = torch.full((R,), nv, dtype=torch.int32, device="cuda")
    topk = torch.full((R, 512), -7, dtype=torch.int32, device="cuda")
    ntopk = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(csa2.Csa2Error) as ei:
        csa2.csa2_index_full_noalloc(cache, q, w, seqs, nvis, nv, 0, 512, None, None, topk, ntopk)
    assert ei.value.status == 2             # CSA2_E_UNSUPPORTED, nothing launched
    torch.cuda.synchronize()
    assert torch.all(topk == -7) and torch.all(ntopk == -7)
