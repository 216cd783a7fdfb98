"""GPU parity at the full workload sizes, on sampled rows.

Each test builds the workload at its real size on the GPU (the decode test
uses the benchmark's own build and step, so it checks the launch
configuration that bench.py times), then recomputes a few sampled rows with
the oracle from the same fp32 generator output and compares:
  * the FP4 planes bit-exactly (the whole indexer plane of a sampled 1M-entry
    sequence, the gathered latent rows);
  * pools and Top-K lists under the tie rule;
  * attention outputs to 2e-3 relative, attending over the oracle's Top-K
    (the GPU stage is given the oracle's list for the sampled rows).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_attention, check_full_row, check_reindex_row, check_topk

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_compressed_sparse_e2m1_amd as m
    m.load()
    return m


def i32(a):
    return torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")


def oracle_rows_of(gen_rows, ids):
    """Quantise (oracle) the fp32 rows `ids` of a device tensor."""
    sel = gen_rows[torch.from_numpy(np.asarray(ids, np.int64)).cuda()].cpu().numpy()
    return oracle.quantize(sel, oracle.KV_GROUP)


def attend_check(csa2, cache, q_all, row_seq, topk_rows, swa, sample, lat_for_seq, H, label,
                 workspace=None):
    """Run GPU attention for all rows with the given Top-K lists, compare the
    sampled rows with the oracle (keys quantised by the oracle from the same
    fp32 rows)."""
    R = q_all.shape[0]
    topk = i32(np.stack(topk_rows))
    ntopk = i32([int((t >= 0).sum()) for t in topk_rows])
    o = torch.empty((R, H, 512), device="cuda")
    lse = torch.empty((R, H), device="cuda")
    csa2.csa2_sparse_attn(cache, q_all, row_seq, topk, ntopk, SCALE, o, lse, swa=swa,
                          workspace=workspace)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    qb = W.bf16_bits(q_all)
    seqs = row_seq.cpu().numpy()
    ends = swa.row_end.cpu().numpy()
    for r in sample:
        ids = topk_rows[r][topk_rows[r] >= 0]
        kvc, kvs = oracle_rows_of(lat_for_seq(int(seqs[r])), ids)
        end = int(min(max(ends[r], 0), swa.kv.shape[1]))
        rows = swa.kv[int(seqs[r]), max(0, end - swa.window):end].cpu().numpy()
        ref = oracle.attend_row(qb[r], kvc, kvs, np.arange(len(ids), dtype=np.int32), rows, SCALE)
        check_attention(o[r], lse[r], ref["o"], ref["lse"], f"{label} row {r}")


# --------------------------------------------------------- 1M-context decode
def test_decode_b8_1m_full_reindex_reuse(csa2):
    """The benchmark's step as it times it: captured as HIP graphs and
    replayed (onto poisoned outputs), then every checked output is the
    replay's."""
    import bench

    c = bench.build()
    bench.step(c)
    torch.cuda.synchronize()
    graphs = bench.capture(c)
    for t in c["topk"] + c["n_topk"] + [c["pool"], c["n_pool"]]:
        t.fill_(-7)
    c["o"].fill_(float("nan"))
    c["lse"].fill_(float("nan"))
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    wl, T, B, H = c["wl"], c["T"], c["B"], c["H"]
    seed = wl.seed
    pool = c["pool"].cpu().numpy()
    npool = c["n_pool"].cpu().numpy()
    topk = [t.cpu().numpy() for t in c["topk"]]
    ntopk = [t.cpu().numpy() for t in c["n_topk"]]
    qi = [W.bf16_bits(x) for x in c["q_idx"]]
    wv = [x.cpu().numpy() for x in c["w"]]
    sample = [0, 5]

    def ik_rows(s):
        ik = W.rms_rows(T - 1, 128, W.seed_for(seed, W.T_IKEY, 0, s), device="cuda")
        return torch.cat([ik, c["new_ik"][s:s + 1]])

    def lat_rows(s):
        lat = W.rms_rows(T - 1, 512, W.seed_for(seed, W.T_LATENT, 0, s), device="cuda")
        return torch.cat([lat, c["new_lat"][s:s + 1]])

    planes = {s: oracle.quantize(ik_rows(s).cpu().numpy(), oracle.IK_GROUP) for s in sample}
    refs = oracle.parallel_map(
        lambda s: oracle.full_layer_select(qi[0][s], wv[0][s], *planes[s], T, wl.k_blk, wl.k_pos),
        sample, len(sample))
    oracle_topk = {}
    for s, f in zip(sample, refs):
        ikc, iks = planes[s]
        # the whole 1M-entry indexer plane of this sequence, bit for bit
        np.testing.assert_array_equal(c["cache"].ik_codes[s].cpu().numpy(), ikc)
        np.testing.assert_array_equal(c["cache"].ik_scales[s].cpu().numpy(), iks)
        check_full_row(csa2, c["cache"], c["q_idx"][0][s:s + 1], c["w"][0][s:s + 1], s, T, pool[s],
                       npool[s], topk[0][s], ntopk[0][s], f, wl.k_blk, wl.k_pos, f"full row {s}")
        oracle_topk[(s, 0)] = f["topk"]
        for l, mode in enumerate(wl.layers):
            if mode != "reindex":
                continue
            ref = oracle.reindex_select(qi[l][s], wv[l][s], ikc, iks, T, f["pool"], wl.k_pos)
            oracle_topk[(s, l)] = ref["topk"]
            check_reindex_row(csa2, c["cache"], c["q_idx"][l][s:s + 1], c["w"][l][s:s + 1], s, T,
                              pool[s], npool[s], topk[l][s], ntopk[l][s], ref, f["pool"], wl.k_blk,
                              wl.k_pos, f"reindex layer {l} row {s}")
    # the last layer's output as the replay left it, where the replay's
    # Top-K (of the layer it inherits) equals the oracle's
    srcs, src = [], None
    for l, mode in enumerate(wl.layers):
        src = l if mode != "reuse" else src
        srcs.append(src)
    last, src = len(wl.layers) - 1, srcs[-1]
    o_rep, lse_rep = c["o"].cpu().numpy(), c["lse"].cpu().numpy()
    qb_last = W.bf16_bits(c["q"][last])
    direct = 0
    for s in sample:
        g_ids = topk[src][s][:ntopk[src][s]]
        if set(g_ids.tolist()) != set(oracle_topk[(s, src)][oracle_topk[(s, src)] >= 0].tolist()):
            continue                  # a tie swap: covered by the checks below
        ids = np.sort(g_ids)
        kvc, kvs = oracle_rows_of(lat_rows(s), ids)
        end = int(min(max(c["swa"][last].row_end[s].item(), 0), c["swa"][last].kv.shape[1]))
        rows = c["swa"][last].kv[s, max(0, end - c["swa"][last].window):end].cpu().numpy()
        ref = oracle.attend_row(qb_last[s], kvc, kvs, np.arange(len(ids), dtype=np.int32), rows, SCALE)
        check_attention(o_rep[s], lse_rep[s], ref["o"], ref["lse"], f"replayed layer {last} row {s}")
        direct += 1
    assert direct >= 1
    # attention of a Full, a Reindex and a Reuse layer over the oracle's lists
    for l in (0, 2, 10):
        src = l if wl.layers[l] != "reuse" else 4
        rows = [topk[src][r] for r in range(B)]
        for s in sample:
            rows[s] = oracle_topk[(s, src)]
        attend_check(csa2, c["cache"], c["q"][l], c["row_seq"], rows, c["swa"][l], sample, lat_rows,
                     H, f"layer {l}", workspace=c["ws_attn"])
    # the appended entry (this step's S1) against the oracle
    for s in sample:
        kc, ks = oracle.quantize(c["new_lat"][s:s + 1].cpu().numpy(), 16)
        np.testing.assert_array_equal(c["cache"].kv_codes[s, T - 1].cpu().numpy(), kc[0])
        np.testing.assert_array_equal(c["cache"].kv_scales[s, T - 1].cpu().numpy(), ks[0])


# ------------------------------------------- multi-query decode at 1M context
def test_multi_query_scan_1m(csa2):
    """The multi-query scan as bench.py times it (8 sequences x 4 queries on
    the 1M-entry cache, rows sequence by sequence, n_vis = T - 3 .. T), then
    the pool and Top-512 of those rows; sampled rows against the oracle."""
    import bench

    c = bench.build()
    bench._append(c)
    wl, T, B = c["wl"], c["T"], c["B"]
    q = 4
    R = B * q
    seqs = torch.arange(B, dtype=torch.int32, device="cuda").repeat_interleave(q)
    nvis = (torch.arange(q, dtype=torch.int32, device="cuda") + (T - q + 1)).repeat(B)
    q_idx = W.bf16_normal((R, 8, 128), W.seed_for(wl.seed, W.T_QIDX, 99), device="cuda")
    w = W.uniform01((R, 8), W.seed_for(wl.seed, W.T_W, 99), device="cuda")
    keys = csa2.block_keys_buffer(R, T)
    csa2.csa2_index_scan(c["cache"], q_idx, w, seqs, nvis, T, keys)
    pool = torch.empty((R, wl.k_blk), dtype=torch.int32, device="cuda")
    npool = torch.empty(R, dtype=torch.int32, device="cuda")
    topk = torch.empty((R, wl.k_pos), dtype=torch.int32, device="cuda")
    ntopk = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_POOL, R, T, wl.k_blk, wl.k_pos)
    csa2.csa2_index_pool(c["cache"], q_idx, w, seqs, nvis, T, keys, wl.k_blk, wl.k_pos, pool, npool,
                         topk, ntopk, ws)
    torch.cuda.synchronize()
    qi, wv = W.bf16_bits(q_idx), w.cpu().numpy()
    pool_h, npool_h = pool.cpu().numpy(), npool.cpu().numpy()
    topk_h, ntopk_h = topk.cpu().numpy(), ntopk.cpu().numpy()
    nvis_h = nvis.cpu().numpy()
    sample = {0: [1, 3], 5: [20, 22]}           # sequence -> rows (n_vis T - 2, T; T - 3, T - 1)

    def ik_rows(s):
        ik = W.rms_rows(T - 1, 128, W.seed_for(wl.seed, W.T_IKEY, 0, s), device="cuda")
        return torch.cat([ik, c["new_ik"][s:s + 1]]).cpu().numpy()

    planes = {s: oracle.quantize(ik_rows(s), oracle.IK_GROUP) for s in sample}
    jobs = [(s, r) for s, rows in sample.items() for r in rows]
    refs = oracle.parallel_map(
        lambda sr: oracle.full_layer_select(qi[sr[1]], wv[sr[1]], *planes[sr[0]], int(nvis_h[sr[1]]),
                                            wl.k_blk, wl.k_pos), jobs, len(jobs))
    for (s, r), f in zip(jobs, refs):
        check_full_row(csa2, c["cache"], q_idx[r:r + 1], w[r:r + 1], s, int(nvis_h[r]), pool_h[r],
                       npool_h[r], topk_h[r], ntopk_h[r], f, wl.k_blk, wl.k_pos, f"row {r}")


# ------------------------------------------------------ 128K decode, 18 Reindex
def test_decode_b32_128k_full_18_reindex(csa2):
    wl = W.WORKLOADS[2]
    B, T, H, seed = wl.batch, wl.ctx, wl.heads, wl.seed
    cache = csa2.Cache(B, T)
    for s in range(B):
        dst = torch.arange(T, dtype=torch.int64, device="cuda") + s * T
        lat = W.rms_rows(T, 512, W.seed_for(seed, W.T_LATENT, 0, s), device="cuda")
        csa2.csa2_quantize_fp4(lat, 16, cache.kv_codes, cache.kv_scales, dst_rows=dst)
        ik = W.rms_rows(T, 128, W.seed_for(seed, W.T_IKEY, 0, s), device="cuda")
        csa2.csa2_quantize_fp4(ik, 32, cache.ik_codes, cache.ik_scales, dst_rows=dst)
    L = len(wl.layers)
    q_idx = [W.bf16_normal((B, 8, 128), W.seed_for(seed, W.T_QIDX, l), device="cuda") for l in range(L)]
    w = [W.uniform01((B, 8), W.seed_for(seed, W.T_W, l), device="cuda") for l in range(L)]
    seqs, nvis = i32(range(B)), i32([T] * B)
    pool = torch.empty((B, wl.k_blk), dtype=torch.int32, device="cuda")
    npool = torch.empty(B, dtype=torch.int32, device="cuda")
    topk = [torch.empty((B, wl.k_pos), dtype=torch.int32, device="cuda") for _ in range(L)]
    ntopk = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(L)]
    csa2.csa2_index_full(cache, q_idx[0], w[0], seqs, nvis, T, wl.k_blk, wl.k_pos, pool, npool,
                         topk[0], ntopk[0], csa2.workspace(csa2.CSA2_OP_INDEX_FULL, B, T, wl.k_blk, wl.k_pos))
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_REINDEX, B, T, wl.k_blk, wl.k_pos)
    for l in range(1, L):
        csa2.csa2_index_reindex(cache, q_idx[l], w[l], seqs, nvis, T, pool, npool, wl.k_blk,
                                wl.k_pos, topk[l], ntopk[l], ws)
    torch.cuda.synchronize()
    sample = [0, 17, 31]
    qi = [W.bf16_bits(x) for x in q_idx]
    wv = [x.cpu().numpy() for x in w]
    pool_h, npool_h = pool.cpu().numpy(), npool.cpu().numpy()
    topk_h = [t.cpu().numpy() for t in topk]
    ntopk_h = [t.cpu().numpy() for t in ntopk]
    for s in sample:
        ik = W.rms_rows(T, 128, W.seed_for(seed, W.T_IKEY, 0, s), device="cuda").cpu().numpy()
        ikc, iks = oracle.quantize(ik, 32)
        np.testing.assert_array_equal(cache.ik_codes[s].cpu().numpy(), ikc)
        f = oracle.full_layer_select(qi[0][s], wv[0][s], ikc, iks, T, wl.k_blk, wl.k_pos)
        assert len(oracle.pool_entries(f["pool"], T)) == 16384      # the constant candidate bound
        check_full_row(csa2, cache, q_idx[0][s:s + 1], w[0][s:s + 1], s, T, pool_h[s], npool_h[s],
                       topk_h[0][s], ntopk_h[0][s], f, wl.k_blk, wl.k_pos, f"full row {s}")
        for l in range(1, L):
            ref = oracle.reindex_select(qi[l][s], wv[l][s], ikc, iks, T, f["pool"], wl.k_pos)
            check_reindex_row(csa2, cache, q_idx[l][s:s + 1], w[l][s:s + 1], s, T, pool_h[s],
                              npool_h[s], topk_h[l][s], ntopk_h[l][s], ref, f["pool"], wl.k_blk,
                              wl.k_pos, f"reindex layer {l} row {s}")


# ----------------------------------------------------- encoder prefill chunk
def test_encoder_prefill_4k_rows_64k_ctx(csa2):
    wl = W.WORKLOADS[1]
    seed, H = wl.seed, wl.heads
    n_ent = wl.ctx // wl.entry_ratio                       # 32,768 entries (2 tokens -> 1)
    t = np.arange(wl.ctx - wl.chunk, wl.ctx)               # query tokens 61,440 .. 65,535
    n_vis = (t + 1) // 2                                   # entry j visible iff 2j + 1 <= t
    R = len(t)
    cache = csa2.Cache(1, n_ent)
    lat = W.rms_rows(n_ent, 512, W.seed_for(seed, W.T_LATENT), device="cuda")
    ik = W.rms_rows(n_ent, 128, W.seed_for(seed, W.T_IKEY), device="cuda")
    csa2.csa2_quantize_fp4(lat, 16, cache.kv_codes, cache.kv_scales)
    csa2.csa2_quantize_fp4(ik, 32, cache.ik_codes, cache.ik_scales)
    q_idx = W.bf16_normal((R, 8, 128), W.seed_for(seed, W.T_QIDX), device="cuda")
    w = W.uniform01((R, 8), W.seed_for(seed, W.T_W), device="cuda")
    seqs, nvis = i32([0] * R), i32(n_vis)
    topk = torch.empty((R, wl.k_pos), dtype=torch.int32, device="cuda")
    ntopk = torch.empty(R, dtype=torch.int32, device="cuda")
    csa2.csa2_index_full(cache, q_idx, w, seqs, nvis, int(n_vis.max()), 0, wl.k_pos, None, None, topk,
                         ntopk, csa2.workspace(csa2.CSA2_OP_INDEX_FULL, R, int(n_vis.max()), 0, wl.k_pos))
    torch.cuda.synchronize()
    ikc, iks = oracle.quantize(ik.cpu().numpy(), 32)
    np.testing.assert_array_equal(cache.ik_codes[0].cpu().numpy(), ikc)
    qi, wv = W.bf16_bits(q_idx), w.cpu().numpy()
    tk, nt = topk.cpu().numpy(), ntopk.cpu().numpy()
    sample = [0, 1, 2, 777, 2048, 4094, 4095]
    refs = {}
    for r in sample:
        f = oracle.full_layer_select(qi[r], wv[r], ikc, iks, int(n_vis[r]), 0, wl.k_pos)
        check_topk(tk[r], nt[r], f, f"row {r}")
        refs[r] = f["topk"]
    # attention + SWA over the last 128 tokens of each query (rows of the chunk's SWA buffer)
    swa_first = int(t[0]) - (wl.swa - 1)
    swa_kv = W.swa_rows_e4m3(int(t[-1]) - swa_first + 1, 512, W.seed_for(seed, W.T_SWA),
                             device="cuda").reshape(1, -1, 512)
    swa = csa2.Swa(swa_kv, i32(t - swa_first + 1), wl.swa)
    q = W.bf16_normal((R, H, 512), W.seed_for(seed, W.T_Q), device="cuda")
    rows = [tk[r] for r in range(R)]
    for r in sample:
        rows[r] = refs[r]
    attend_check(csa2, cache, q, seqs, rows, swa, sample, lambda s: lat, H, "prefill")


# ------------------------------------------------------ reuse-mode attention
def test_reuse_b256_h64_ragged_contexts(csa2):
    wl = W.WORKLOADS[4]
    B, H, seed = wl.batch, wl.heads, wl.seed
    lens = W.lengths_uniform(B, wl.ctx_min, wl.ctx, W.seed_for(seed, W.T_LEN))
    cap = int(lens.max())
    cache = csa2.Cache(B, cap)
    for s in range(B):
        n = int(lens[s])
        lat = W.rms_rows(n, 512, W.seed_for(seed, W.T_LATENT, 0, s), device="cuda")
        dst = torch.arange(n, dtype=torch.int64, device="cuda") + s * cap
        csa2.csa2_quantize_fp4(lat, 16, cache.kv_codes, cache.kv_scales, dst_rows=dst)
    topk_rows = [W.topk_uniform(int(lens[s]), wl.k_pos, W.seed_for(seed, W.T_TOPK, 0, s)) for s in range(B)]
    swa_kv = W.swa_rows_e4m3(B * wl.swa, 512, W.seed_for(seed, W.T_SWA), device="cuda").reshape(B, wl.swa, 512)
    swa = csa2.Swa(swa_kv, i32([wl.swa] * B), wl.swa)
    q = W.bf16_normal((B, H, 512), W.seed_for(seed, W.T_Q), device="cuda")
    sample = [0, 1, 100, 254, 255]

    def lat_rows(s):
        return W.rms_rows(int(lens[s]), 512, W.seed_for(seed, W.T_LATENT, 0, s), device="cuda")

    attend_check(csa2, cache, q, i32(range(B)), topk_rows, swa, sample, lat_rows, H, "reuse",
                 workspace=csa2.attn_workspace(B, H, wl.k_pos, wl.swa))
