#!/usr/bin/env python3
"""Benchmark of the CSA2 hot path on one MI355X.

A step is one decode step of the 1M-context stack: batch 8, 1,048,576 visible
entries per sequence, 20 CSA2 layers (1 Full, 4 Reindex, 15 Reuse), each
with its own 16-head query and its own 128-row FP8 SWA window
(P3 "레이어 40개 가운데 4개만 전역 캐시를 만듭니다"; P1 "무엇과 다른가").
  Full    : append the step's new entry (FP4 quantise, both planes), scan all
            1M entries, keep 2,048 blocks of 8, re-score the pool, Top-512,
            sparse attention with the SWA branch in the same softmax;
  Reindex : re-score the Full layer's pool with its own indexer query, Top-512,
            attention + SWA;
  Reuse   : attention + SWA over the last Reindex layer's Top-512.
Inputs are seeded synthetic tensors already resident in HBM; the cache
(8 x 1M entries x 356 B) is built before timing, and the timed steps cycle
through four input sets (each layer's queries, indexer weights and SWA rows).

The timed steps launch every kernel from Python (the GPU, not the host, is
the limit: replaying the step as HIP graphs measured no faster); --graph
replays it as two HIP graphs (the scan with its append, everything after it),
after checking that a replay reproduces the eager step's outputs bit for bit.

Output: one JSON line.  value = query tokens per second per CSA2 layer
(= batch x layers / step time); roofline = the Full-layer scan kernel,
timed with HIP events recorded between the graph launches on the stream
they run on; cpu_baseline = the oracle on a bounded sample of the same step.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
IK_BYTES = 68                  # indexer key bytes per entry (64 codes + 4 scales)
BLOCK_KEY_BYTES = 4            # the scan writes one 4-B key per block of 8 entries
APPEND_BYTES = 4 * (512 + 128) + 356   # per row: the fp32 latent and indexer key read, one entry written


def scan_bytes_per_launch(T, B):
    """Algorithmic HBM bytes of one scan-with-append launch: every visible
    entry's indexer key once, plus each row's append."""
    return IK_BYTES * T * B + APPEND_BYTES * B

# HBM bytes per scan launch from two rocprofv3 counter runs of this bench
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same
# counter reads for a plain 512-MiB device copy.  They describe the scan kernel
# as built from these sources; once the sources differ the figure is dropped.
SCAN_COUNTERS = {
    "sources": ["fp4_compressed_sparse_e2m1_amd/csrc/index.hip",
                "fp4_compressed_sparse_e2m1_amd/csrc/encode.h",
                "fp4_compressed_sparse_e2m1_amd/csrc/device.h",
                "fp4_compressed_sparse_e2m1_amd/csrc/internal.h"],
    "sha256": "5806cde2822378fe79fd25c60858aa567afaa7fa4120b704b2d0029100f96226",
    "fetch_kib": 278742.177, "fetch_scale": 524288 / 262166.625,
    "write_kib": 4099.052, "write_scale": 524288 / 524288.0,
}


# The same two counters for the 64-head attention at batch 256 (bench.py
# --attention-only --copy-calibration 512: 23 launches), scaled by the copy
# run first in the same process.
ATTN64_COUNTERS = {
    "sources": ["fp4_compressed_sparse_e2m1_amd/csrc/attention64.hip",
                "fp4_compressed_sparse_e2m1_amd/csrc/device.h",
                "fp4_compressed_sparse_e2m1_amd/csrc/internal.h"],
    "sha256": "5adf8767c29c7dc4c1b8cbdaeeb42e3230534d38717e042d6bb430d64c02df9a",
    "fetch_kib": 45558.027, "fetch_scale": 524288 / 262166.25,
    "write_kib": 32924.391, "write_scale": 524288 / 524288.0,
}


def counter_traffic_bytes(c):
    """Counter-measured HBM bytes per launch, or None when the kernel's
    sources changed since the counters were taken."""
    h = hashlib.sha256()
    for f in c["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != c["sha256"]:
        return None
    return int(round((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024))


def scan_traffic_bytes():
    """Counter-measured HBM bytes per scan launch, or None when the scan's
    sources changed since the counters were taken."""
    return counter_traffic_bytes(SCAN_COUNTERS)
SCALE = 1.0 / math.sqrt(512)
# input sets the timed steps cycle through (queries, indexer weights, SWA rows)
N_INPUT_SETS = 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=8,
                    help="query rows of the step the oracle runs for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attention-roofline", action="store_true",
                    help="skip the batch-256, 64-head attention bandwidth measurement")
    ap.add_argument("--attention-only", action="store_true",
                    help="run only the batch-256, 64-head attention measurement and print its object "
                         "(for profiling that kernel; not the benchmark line)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the encoder prefill chunk measurement and print its object "
                         "(for profiling those kernels; not the benchmark line)")
    ap.add_argument("--ctx", type=int, default=None, help="override the context (testing only)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, copy a MIB-MiB buffer once with a plain device copy "
                         "(a known-size kernel for scaling hardware byte counters)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (tiny decode, prefill chunk, batch-32 128K decode) "
                         "and the 4K-context run of the step")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as HIP graphs instead of launching every kernel from Python")
    return ap.parse_args()


def build(ctx_override=None, wid=3):
    """Builds a decode workload (the 1M-context stack by default): its FP4
    cache of T - 1 entries per sequence, the step's new entries, and every
    layer's queries, SWA windows and outputs."""
    import torch

    import fp4_compressed_sparse_e2m1_amd as csa2
    import workloads as W

    wl = W.WORKLOADS[wid]
    B, T, H = wl.batch, ctx_override or wl.ctx, wl.heads
    dev = "cuda"
    seed = wl.seed
    cache = csa2.Cache(B, T, device=dev)
    # bulk build of entries 0 .. T-2 (untimed); entry T-1 is the step's append
    for s in range(B):
        dst = torch.arange(T - 1, dtype=torch.int64, device=dev) + s * T
        lat = W.rms_rows(T - 1, 512, W.seed_for(seed, W.T_LATENT, 0, s), device=dev)
        csa2.csa2_quantize_fp4(lat, 16, cache.kv_codes, cache.kv_scales, dst_rows=dst)
        del lat
        ik = W.rms_rows(T - 1, 128, W.seed_for(seed, W.T_IKEY, 0, s), device=dev)
        csa2.csa2_quantize_fp4(ik, 32, cache.ik_codes, cache.ik_scales, dst_rows=dst)
        del ik, dst
    torch.cuda.synchronize()
    L = len(wl.layers)
    new_lat = W.rms_rows(B, 512, W.seed_for(seed, W.T_LATENT, 0, 1 << 20), device=dev)
    new_ik = W.rms_rows(B, 128, W.seed_for(seed, W.T_IKEY, 0, 1 << 20), device=dev)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    ctx = dict(
        csa2=csa2, wl=wl, B=B, T=T, H=H, L=L, cache=cache, new_lat=new_lat, new_ik=new_ik,
        new_dst=torch.arange(B, dtype=torch.int64, device=dev) * T + (T - 1),
        row_seq=i32(list(range(B))), row_nvis=i32([T] * B),
        block_keys=csa2.block_keys_buffer(B, T),
        pool=torch.empty((B, wl.k_blk), dtype=torch.int32, device=dev),
        n_pool=torch.empty(B, dtype=torch.int32, device=dev),
        topk=[torch.empty((B, wl.k_pos), dtype=torch.int32, device=dev) for _ in range(L)],
        n_topk=[torch.empty(B, dtype=torch.int32, device=dev) for _ in range(L)],
        ws_pool=csa2.workspace(csa2.CSA2_OP_INDEX_POOL, B, T, wl.k_blk, wl.k_pos),
        ws_re=csa2.workspace(csa2.CSA2_OP_INDEX_REINDEX, B, T, wl.k_blk, wl.k_pos),
        ws_attn=csa2.attn_workspace(B, H, wl.k_pos, wl.swa),
        o=torch.empty((B, H, 512), dtype=torch.float32, device=dev),
        lse=torch.empty((B, H), dtype=torch.float32, device=dev),
    )
    # input sets: every layer's queries, indexer weights and SWA window, drawn
    # afresh per set (set 0 from the layer's own seeds); the timed steps cycle
    # through the sets, so consecutive steps gather different entries and read
    # different SWA rows instead of finding the previous step's in the caches
    def input_set(k):
        sd = lambda t, l: W.seed_for(seed, t, l, k)
        return dict(
            q=[W.bf16_normal((B, H, 512), sd(W.T_Q, l), device=dev) for l in range(L)],
            q_idx=[W.bf16_normal((B, 8, 128), sd(W.T_QIDX, l), device=dev) for l in range(L)],
            w=[W.uniform01((B, 8), sd(W.T_W, l), device=dev) for l in range(L)],
            swa=[csa2.Swa(W.swa_rows_e4m3(B * wl.swa, 512, sd(W.T_SWA, l), device=dev)
                          .reshape(B, wl.swa, 512), i32([wl.swa] * B), wl.swa) for l in range(L)])

    ctx["sets"] = [input_set(k) for k in range(N_INPUT_SETS)]
    use_set(ctx, 0)
    torch.cuda.synchronize()
    return ctx


def use_set(c, k):
    """Makes input set k the one the step reads (q, q_idx, w, swa per layer)."""
    for name in ("q", "q_idx", "w", "swa"):
        c[name] = c["sets"][k][name]


def _append(c):
    c["csa2"].csa2_cache_append(c["cache"], c["new_lat"], c["new_ik"], c["new_dst"])


def _scan_append(c, l):
    """The Full layer's append of the step's new entry (at n_vis - 1 of each
    sequence) and its scan, one launch."""
    c["csa2"].csa2_index_scan_append(c["cache"], c["new_lat"], c["new_ik"], c["q_idx"][l], c["w"][l],
                                     c["row_seq"], c["row_nvis"], c["T"], c["block_keys"])


def _layer_tail(c, l, mode, src):
    """Everything of layer l after the scan; returns the layer whose Top-512
    later Reuse layers attend over."""
    csa2, wl, T = c["csa2"], c["wl"], c["T"]
    cache, seqs, nvis = c["cache"], c["row_seq"], c["row_nvis"]
    if mode == "full":
        csa2.csa2_index_pool(cache, c["q_idx"][l], c["w"][l], seqs, nvis, T, c["block_keys"],
                             wl.k_blk, wl.k_pos, c["pool"], c["n_pool"], c["topk"][l],
                             c["n_topk"][l], c["ws_pool"])
        src = l
    elif mode == "reindex":
        csa2.csa2_index_reindex(cache, c["q_idx"][l], c["w"][l], seqs, nvis, T, c["pool"],
                                c["n_pool"], wl.k_blk, wl.k_pos, c["topk"][l], c["n_topk"][l],
                                c["ws_re"])
        src = l
    csa2.csa2_sparse_attn(cache, c["q"][l], seqs, c["topk"][src], c["n_topk"][src], SCALE,
                          c["o"], c["lse"], swa=c["swa"][l], workspace=c["ws_attn"])
    return src


def step(c, ev=None):
    """One decode step of the 20-layer stack, every kernel launched from
    Python.  ev: optional events to record (scan start/end, then one boundary
    after every layer)."""
    src = None
    for l, mode in enumerate(c["wl"].layers):
        if mode == "full":
            if ev is not None:
                ev["scan0"].record()
            _scan_append(c, l)
            if ev is not None:
                ev["scan1"].record()
        src = _layer_tail(c, l, mode, src)
        if ev is not None:
            ev["layer"][l].record()


def capture(c):
    """The step as two HIP graphs: the Full layer's scan with its append, and
    everything after it (the stack opens with its one Full layer)."""
    import torch

    layers = c["wl"].layers
    assert layers[0] == "full" and "full" not in layers[1:]

    def rest():
        src = None
        for l, mode in enumerate(layers):
            src = _layer_tail(c, l, mode, src)

    graphs = []
    for fn in (lambda: _scan_append(c, 0), rest):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def launches_per_layer(c):
    """Launches of each layer mode of the step, counted as the kernel nodes
    of one HIP graph per layer (the Full layer's with its scan-and-append);
    nodes of other kinds (copies, fills) are counted apart."""
    import ctypes

    import torch

    hip = ctypes.CDLL("libamdhip64.so.7")    # the runtime torch already loaded

    def count(fn):
        g = torch.cuda.CUDAGraph(keep_graph=True)
        with torch.cuda.graph(g):
            fn()
        h = ctypes.c_void_p(g.raw_cuda_graph())
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(h, None, ctypes.byref(n)) != 0:
            raise RuntimeError("hipGraphGetNodes failed")
        nodes = (ctypes.c_void_p * max(1, n.value))()
        if hip.hipGraphGetNodes(h, nodes, ctypes.byref(n)) != 0:
            raise RuntimeError("hipGraphGetNodes failed")
        kernels = 0
        for i in range(n.value):
            t = ctypes.c_int(-1)
            if hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) != 0:
                raise RuntimeError("hipGraphNodeGetType failed")
            kernels += t.value == 0              # hipGraphNodeTypeKernel
        del g
        return kernels, n.value - kernels

    layers = c["wl"].layers
    full = layers.index("full")
    out = {}
    for l, mode in enumerate(layers):
        if mode in out:
            continue
        if mode == "full":
            def fn(l=l):
                _scan_append(c, l)
                _layer_tail(c, l, "full", None)
        else:
            def fn(l=l, mode=mode):
                _layer_tail(c, l, mode, full)
        k, other = count(fn)
        out[mode] = {"kernels": k, "other_nodes": other}
    torch.cuda.synchronize()
    return out


def _outputs(c):
    """Copies of what a step writes: the selections of the Full and Reindex
    layers, the pool, and the last layer's attention output."""
    sel = [l for l, m in enumerate(c["wl"].layers) if m != "reuse"]
    return [t.clone() for t in [c["topk"][l] for l in sel] + [c["n_topk"][l] for l in sel]
            + [c["pool"], c["n_pool"], c["o"], c["lse"]]]


def run_gpu(c, steps, warmup, eager):
    """Times `steps` steps after `warmup` untimed ones, the steps cycling
    through the input sets.  Returns the wall time, the scan kernel's mean
    event time (ms), and the per-layer event times (ms) of a separate eager
    pass."""
    import torch

    n_sets = len(c["sets"])
    for i in range(warmup):
        use_set(c, i % n_sets)
        step(c)
    torch.cuda.synchronize()
    L = c["L"]
    # per-layer breakdown: eager launches with events after every layer (untimed)
    evs = [dict(scan0=torch.cuda.Event(enable_timing=True), scan1=torch.cuda.Event(enable_timing=True),
                start=torch.cuda.Event(enable_timing=True),
                layer=[torch.cuda.Event(enable_timing=True) for _ in range(L)]) for _ in range(3)]
    for j, e in enumerate(evs):
        use_set(c, j % n_sets)
        e["start"].record()
        step(c, e)
    torch.cuda.synchronize()
    per_layer = [0.0] * L
    for e in evs:
        prev = e["start"]
        for l in range(L):
            per_layer[l] += prev.elapsed_time(e["layer"][l]) / len(evs)
            prev = e["layer"][l]
    graphs = None
    if not eager:
        use_set(c, 0)
        step(c)
        torch.cuda.synchronize()
        ref = _outputs(c)
        graphs = []
        for k in range(n_sets):            # one set of graphs per input set
            use_set(c, k)
            graphs.append(capture(c))
        for g in graphs[0]:
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, _outputs(c)):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager step")
        for i in range(warmup):
            for g in graphs[i % n_sets]:
                g.replay()
    scan = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        if graphs is None:
            use_set(c, k % n_sets)
            step(c, dict(scan0=scan[k][0], scan1=scan[k][1], layer=[_NoEvent] * L))
        else:
            g = graphs[k % n_sets]
            scan[k][0].record()
            g[0].replay()
            scan[k][1].record()
            g[1].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    use_set(c, 0)
    scan_ms = sum(a.elapsed_time(b) for a, b in scan) / steps
    return wall, scan_ms, per_layer


class _NoEvent:
    @staticmethod
    def record():
        pass


_SPIN_PER_MS = None


def hold_stream(ms):
    """Keep the current stream busy for about `ms` milliseconds with torch's
    bounded spin kernel (its rate is measured once with events)."""
    import torch

    global _SPIN_PER_MS
    if _SPIN_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        torch.cuda.synchronize()
        _SPIN_PER_MS = (1 << 20) / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SPIN_PER_MS * ms))


def reuse_attention(steps, warmup):
    """The attention kernel where it carries enough bytes to be bandwidth-bound:
    one Reuse layer at batch 256, 64 heads, contexts U[64K, 256K] entries, an
    inherited uniform Top-512 per row and a 128-row FP8 SWA window, fused in
    one softmax; the launches cycle through four input sets.  Algorithmic
    bytes per query: 512 x 288 (gathered latents) + 128 x 512 (SWA) + 64 x
    1,024 (q) + 512 x 4 (ids) + 64 x 2,048 (o) + 64 x 4 (lse) = 411,904 B."""
    import torch

    import fp4_compressed_sparse_e2m1_amd as csa2
    import workloads as W

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
        del lat, dst
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    ntopk = i32([wl.k_pos] * B)
    seqs = i32(list(range(B)))
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = csa2.attn_workspace(B, H, wl.k_pos, wl.swa)

    # input sets (inherited Top-512, queries, SWA rows; set 0 from the
    # workload's own seeds): the launches cycle through them, so no launch
    # finds the previous one's gathers in the caches
    def input_set(k):
        topk = torch.stack([torch.from_numpy(W.topk_uniform(int(lens[s]), wl.k_pos,
                                                            W.seed_for(seed, W.T_TOPK, k, s)).astype("int32"))
                            for s in range(B)]).cuda()
        swa = csa2.Swa(W.swa_rows_e4m3(B * wl.swa, 512, W.seed_for(seed, W.T_SWA, k), device="cuda")
                       .reshape(B, wl.swa, 512), i32([wl.swa] * B), wl.swa)
        q = W.bf16_normal((B, H, 512), W.seed_for(seed, W.T_Q, k), device="cuda")
        return topk, swa, q

    sets = [input_set(k) for k in range(N_INPUT_SETS)]

    def run(k):
        topk, swa, q = sets[k % len(sets)]
        csa2.csa2_sparse_attn(cache, q, seqs, topk, ntopk, SCALE, o, lse, swa=swa, workspace=ws)

    for i in range(warmup):
        run(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    # each launch costs the host about as long as the kernel runs, so the
    # stream is held while the timed launches are queued: the events then
    # bracket back-to-back kernels instead of waits for the host
    hold_stream(0.2 * steps + 2.0)
    for k, (a, b) in enumerate(ev):
        a.record()
        run(k)
        b.record()
    torch.cuda.synchronize()
    us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
    per_query = 512 * 288 + wl.swa * 512 + H * 1024 + 512 * 4 + H * 2048 + H * 4
    achieved = per_query * B / (us * 1e-6) / 1e9
    del cache
    return {"workload": wl.name, "kernel": "attn_h64_kernel (csa2_sparse_attn, 64 heads, SWA fused)",
            "avg_launch_us": round(us, 2), "query_tokens_per_s": round(B / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic_bytes(ATTN64_COUNTERS),
                         "algorithmic_bytes_per_launch": per_query * B}}


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak


def _event_pairs(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def prefill_chunk(steps, warmup):
    """The encoder Full-mode prefill chunk: 4,096 new query tokens (t = 61,440
    .. 65,535) against a 65,536-token context stored at 2 tokens -> 1 entry
    (32,768 FP4 entries), each query scoring its causally visible entries
    (entry j visible to token t iff 2j + 1 <= t) and keeping a flat Top-512,
    then 16-head sparse attention over those entries with the last 128
    tokens' FP8 SWA rows in the same softmax.  The scoring and attention
    contractions are dense, so the roof is the matrix-core one: useful flops =
    2 x 8 x 128 per (query, visible entry) for the scores + 2 x 2 x 16 x 512
    per (query, attended key) for Q.K and P.V."""
    import numpy as np
    import torch

    import fp4_compressed_sparse_e2m1_amd as csa2
    import workloads as W

    wl = W.WORKLOADS[1]
    seed, H = wl.seed, wl.heads
    n_ent = wl.ctx // wl.entry_ratio
    t = np.arange(wl.ctx - wl.chunk, wl.ctx)
    n_vis = (t + 1) // 2
    R = len(t)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    cache = csa2.Cache(1, n_ent)
    lat = W.rms_rows(n_ent, 512, W.seed_for(seed, W.T_LATENT), device="cuda")
    ik = W.rms_rows(n_ent, 128, W.seed_for(seed, W.T_IKEY), device="cuda")
    csa2.csa2_quantize_fp4(lat, 16, cache.kv_codes, cache.kv_scales)
    csa2.csa2_quantize_fp4(ik, 32, cache.ik_codes, cache.ik_scales)
    del lat, ik
    q_idx = W.bf16_normal((R, 8, 128), W.seed_for(seed, W.T_QIDX), device="cuda")
    w = W.uniform01((R, 8), W.seed_for(seed, W.T_W), device="cuda")
    seqs, nvis = i32([0] * R), i32(n_vis)
    max_nvis = int(n_vis.max())
    topk = torch.empty((R, wl.k_pos), dtype=torch.int32, device="cuda")
    ntopk = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(csa2.CSA2_OP_INDEX_FULL, R, max_nvis, 0, wl.k_pos)
    swa_first = int(t[0]) - (wl.swa - 1)
    swa_kv = W.swa_rows_e4m3(int(t[-1]) - swa_first + 1, 512, W.seed_for(seed, W.T_SWA),
                             device="cuda").reshape(1, -1, 512)
    swa = csa2.Swa(swa_kv, i32(t - swa_first + 1), wl.swa)
    q = W.bf16_normal((R, H, 512), W.seed_for(seed, W.T_Q), device="cuda")
    o = torch.empty((R, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    wsa = csa2.attn_workspace(R, H, wl.k_pos, wl.swa)

    def index():
        csa2.csa2_index_full(cache, q_idx, w, seqs, nvis, max_nvis, 0, wl.k_pos, None, None, topk, ntopk, ws)

    def attend():
        csa2.csa2_sparse_attn(cache, q, seqs, topk, ntopk, SCALE, o, lse, swa=swa, workspace=wsa)

    for _ in range(warmup):
        index()
        attend()
    ev_i, ev_a = _event_pairs(steps), _event_pairs(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev_i[k][0].record()
        index()
        ev_i[k][1].record()
        ev_a[k][0].record()
        attend()
        ev_a[k][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    idx_us = 1e3 * sum(a.elapsed_time(b) for a, b in ev_i) / steps
    att_us = 1e3 * sum(a.elapsed_time(b) for a, b in ev_a) / steps
    keys = int(ntopk.sum().item()) + R * wl.swa
    score_flop = 2 * 8 * 128 * int(n_vis.sum())
    attn_flop = 2 * 2 * H * 512 * keys
    tf = lambda f, us: f / (us * 1e-6) / 1e12
    del cache
    return {"workload": wl.name, "query_tokens": R, "context_entries": n_ent,
            "query_tokens_per_s": round(R / wall, 1), "ms_per_chunk": round(wall * 1e3, 3),
            "index_us": round(idx_us, 1), "attention_us": round(att_us, 1),
            "roofline": {"bound": "mfma", "unit": "TFLOP/s", "peak": MFMA_F16_PEAK_TFLOPS,
                         "index": {"achieved": round(tf(score_flop, idx_us), 1),
                                   "frac": round(tf(score_flop, idx_us) / MFMA_F16_PEAK_TFLOPS, 4),
                                   "flop": score_flop},
                         "attention": {"achieved": round(tf(attn_flop, att_us), 1),
                                       "frac": round(tf(attn_flop, att_us) / MFMA_F16_PEAK_TFLOPS, 4),
                                       "flop": attn_flop}}}


def decode_b32(steps, warmup):
    """The 128K-context decode step at batch 32: append, a Full layer (scan of
    131,072 entries, 2,048 blocks -> 16,384-candidate pool -> Top-512,
    attention + SWA) and 18 Reindex layers (re-score the pool with their own
    indexer query, Top-512, attention + SWA)."""
    c = build(wid=2)
    wall, scan_ms, per_layer = run_gpu(c, steps, warmup, True)
    B, T, L = c["B"], c["T"], c["L"]
    scan_bytes = scan_bytes_per_launch(T, B)
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    modes = c["wl"].layers
    mode_us = {m: 1e3 * sum(t for t, mm in zip(per_layer, modes) if mm == m) /
               max(1, sum(1 for mm in modes if mm == m)) for m in ("full", "reindex")}
    out = {"workload": c["wl"].name, "batch": B, "context_entries": T, "layers": L,
           "query_tokens_per_s_per_layer": round(B * L / (wall / steps), 1),
           "ms_per_step": round(wall * 1e3 / steps, 4),
           "per_layer_us_eager": {k: round(v, 2) for k, v in mode_us.items()},
           "scan": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": scan_bytes,
                    "avg_launch_us": round(scan_ms * 1e3, 2)}}
    del c
    return out


def tiny_decode(steps, warmup):
    """The tiny decode workload: batch 1, 4,096 entries, one Full layer (append,
    scan, 64 of 512 blocks, Top-512, attention + SWA).  Latency-bound: its
    cache (1.46 MB) sits in the caches, so it is reported in microseconds."""
    c = build(wid=0)
    wall, scan_ms, per_layer = run_gpu(c, steps, warmup, True)
    out = {"workload": c["wl"].name, "batch": c["B"], "context_entries": c["T"],
           "us_per_step": round(wall * 1e6 / steps, 2),
           "query_tokens_per_s": round(c["B"] / (wall / steps), 1),
           "scan_us": round(scan_ms * 1e3, 2)}
    del c
    return out


def multi_query_scan(c, q_per_seq=4, steps=20, warmup=3):
    """The Full-layer scan of a multi-query decode step on the 1M-context cache:
    each of the 8 sequences checks q_per_seq queries at once (draft tokens,
    n_vis = T - q_per_seq + 1 .. T), so 8 x q_per_seq query rows, laid out
    sequence by sequence, share each indexer key read.  Algorithmic bytes:
    every visible key read once per sequence (68 B per entry); the 4-B block
    keys written per block of 8 and row are workspace traffic, not counted."""
    import torch

    import workloads as W

    csa2, T, B = c["csa2"], c["T"], c["B"]
    R = B * q_per_seq
    dev = "cuda"
    seqs = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(q_per_seq)
    nvis = (torch.arange(q_per_seq, dtype=torch.int32, device=dev) + (T - q_per_seq + 1)).repeat(B)
    q_idx = W.bf16_normal((R, 8, 128), W.seed_for(c["wl"].seed, W.T_QIDX, 99), device=dev)
    w = W.uniform01((R, 8), W.seed_for(c["wl"].seed, W.T_W, 99), device=dev)
    keys = csa2.block_keys_buffer(R, T)

    def run():
        csa2.csa2_index_scan(c["cache"], q_idx, w, seqs, nvis, T, keys)

    for _ in range(warmup):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / steps
    byt = IK_BYTES * T * B                         # key reads (68 B per visible entry)
    achieved = byt / (us * 1e-6) / 1e9
    return {"queries_per_sequence": q_per_seq, "rows": R, "avg_launch_us": round(us, 2),
            "query_tokens_per_s": round(R / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": byt}}


def path_flops_per_query(T, wl):
    """Useful flops of one decode query through this path's layer stack at T
    visible entries: the Full-layer scan (2 x 8 x 128 per entry), the pool
    re-score of the Full layer and of every Reindex layer (2 x 8 x 128 per
    candidate, at most 8 x k_blocks candidates), and every layer's attention
    (2 x 2 x heads x 512 per attended key: Top-K plus the SWA window)."""
    cand = min(8 * wl.k_blk, T)
    n_re = sum(1 for m in wl.layers if m == "reindex")
    keys = min(wl.k_pos, T) + min(wl.swa, T)
    return (2 * 8 * 128 * T + 2 * 8 * 128 * cand * (1 + n_re)
            + len(wl.layers) * 2 * 2 * wl.heads * 512 * keys)


def pages_figures(c, step_ms_1m=None, step_ms_4k=None, launches=None):
    """The pages' own figures (no hardware stated for any) beside what this
    library's layout and launch plan give, and the measured step-time ratio
    of the same 20-layer decode stack at 1M and at 4K context when given."""
    csa2, wl = c["csa2"], c["wl"]
    per_entry = c["cache"].nbytes // (c["B"] * c["T"])
    reuse = launches["reuse"]["kernels"] if launches else None
    return {
        "bytes_per_entry": {"csa2_amd": per_entry, "pages": 356},
        "bytes_per_token_at_2_5_entries": {"csa2_amd": per_entry * 2.5, "pages": 890},
        "kernels_per_reuse_layer_decode": {
            "csa2_amd": reuse,
            "pages": 11,
            "note": "ours (counted in the step's graph): sparse attention with the SWA branch "
                    "fused; up to 16 rows the split rows are merged inside the same kernel, from 17 "
                    "rows on by a second one; the pages count the whole fused layer"},
        "kernels_per_reuse_layer_prefill": {
            "csa2_amd": 1,
            "pages": 15,
            "note": "ours at the 4,096-query prefill chunk: one attention launch with the SWA branch fused"},
        "decode_flops_1m_over_4k": {
            "csa2_amd": round(path_flops_per_query(1 << 20, wl) / path_flops_per_query(4096, wl), 3),
            "pages": 1.25,
            "note": "ours: the CSA2 path alone (indexer scan, re-scores, attention of the 20-layer stack); "
                    "the pages: the whole model"},
        "decode_step_time_1m_over_4k": {
            "csa2_amd": round(step_ms_1m / step_ms_4k, 3) if step_ms_1m and step_ms_4k else None,
            "ms_at_4k": round(step_ms_4k, 4) if step_ms_4k else None,
            "note": "measured: the same 20-layer decode step (batch 8) at 4,096 and at 1,048,576 entries"},
    }


def copy_bandwidth():
    """A plain 1-GiB device-to-device copy on this GPU (read + write bytes / time)."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    del src, dst
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(c, rows):
    """The oracle, as it stands, on `rows` query rows of the same step (all 20
    layers, full 1M context), one host thread per row.  The oracle builds its
    own FP4 cache of those rows' sequences from the same fp32 generator before
    timing; the timed part is what the GPU step does: append, scan, pool,
    Top-512, 4 re-indexes and 20 attentions with SWA."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    wl, T, B = c["wl"], c["T"], c["B"]
    rows = max(1, min(rows, B))
    seed = wl.seed
    prep = []
    for s in range(rows):
        ik = W.rms_rows(T - 1, 128, W.seed_for(seed, W.T_IKEY, 0, s), device="cuda").cpu().numpy()
        ik = np.concatenate([ik, c["new_ik"][s:s + 1].cpu().numpy()])
        prep.append(ik)

    def quantize_seq(s):
        return oracle.quantize(prep[s], oracle.IK_GROUP)

    planes = oracle.parallel_map(quantize_seq, list(range(rows)), rows)
    del prep
    lat_rows = {}
    swa = [c["swa"][l].kv.cpu().numpy() for l in range(c["L"])]
    q = [W.bf16_bits(c["q"][l]) for l in range(c["L"])]
    qi = [W.bf16_bits(c["q_idx"][l]) for l in range(c["L"])]
    wv = [c["w"][l].cpu().numpy() for l in range(c["L"])]

    def full_step(s):
        ikc, iks = planes[s]
        sel = None
        out = []
        for l, mode in enumerate(wl.layers):
            if mode == "full":
                f = oracle.full_layer_select(qi[l][s], wv[l][s], ikc, iks, T, wl.k_blk, wl.k_pos)
                pool, sel = f["pool"], f["topk"]
            elif mode == "reindex":
                sel = oracle.reindex_select(qi[l][s], wv[l][s], ikc, iks, T, pool, wl.k_pos)["topk"]
            ids = sel[sel >= 0]
            kvc, kvs = lat_rows[s]
            kmap = {int(j): i for i, j in enumerate(lat_rows[(s, "ids")])}
            loc = np.array([kmap[int(j)] for j in ids], np.int32)
            out.append(oracle.attend_row(q[l][s], kvc, kvs, loc, swa[l][s], SCALE)["o"])
        return out

    # the main latents of every entry the oracle will gather (from the same
    # generator), quantised by the oracle itself before timing
    def gathered_ids(s):
        ikc, iks = planes[s]
        ids = set()
        f = oracle.full_layer_select(qi[0][s], wv[0][s], ikc, iks, T, wl.k_blk, wl.k_pos)
        ids.update(f["topk"][f["topk"] >= 0].tolist())
        for l, mode in enumerate(wl.layers):
            if mode == "reindex":
                r = oracle.reindex_select(qi[l][s], wv[l][s], ikc, iks, T, f["pool"], wl.k_pos)
                ids.update(r["topk"][r["topk"] >= 0].tolist())
        return np.array(sorted(ids), np.int64)

    all_ids = oracle.parallel_map(gathered_ids, list(range(rows)), rows)
    for s in range(rows):
        ids = all_ids[s]
        lat = W.rms_rows(T - 1, 512, W.seed_for(seed, W.T_LATENT, 0, s), device="cuda")
        lat = torch.cat([lat, c["new_lat"][s:s + 1]])
        lat_rows[s] = oracle.quantize(lat[torch.from_numpy(ids).cuda()].cpu().numpy(), oracle.KV_GROUP)
        lat_rows[(s, "ids")] = ids
        del lat
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    oracle.parallel_map(full_step, list(range(rows)), rows)
    dt = time.perf_counter() - t0
    # the same oracle on one row and one thread
    t0 = time.perf_counter()
    full_step(0)
    dt1 = time.perf_counter() - t0
    return {"value": rows * c["L"] / dt, "unit": "query-tokens/s per CSA2 layer", "cores": rows,
            "kind": "oracle",
            "value_1thread": c["L"] / dt1,
            "host_cores": host_cores(), "cpu_model": cpu_model(),
            "sample": f"{rows} of the {B} query rows of the 1M-context decode step, all {c['L']} layers "
                      f"(scan of {T} entries, pool, Top-512, 4 re-indexes, 20 attentions with SWA), "
                      f"one host thread per row; {dt:.1f} s wall; value_1thread: row 0 alone on one "
                      f"thread, {dt1:.1f} s"}


def host_cores():
    """Host CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(every step of the CSA2 path is independent per sequence, so N GPUs would each run "
              f"their own share of the batch).", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    import fp4_compressed_sparse_e2m1_amd as csa2
    csa2.load()
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.attention_only:
        print(json.dumps(reuse_attention(args.steps, args.warmup)))
        return
    if args.prefill_only:
        print(json.dumps(prefill_chunk(args.steps, args.warmup)))
        return
    t_build = time.perf_counter()
    c = build(args.ctx)
    t_build = time.perf_counter() - t_build
    wall, scan_ms, per_layer = run_gpu(c, args.steps, args.warmup, not args.graph)
    B, T, L = c["B"], c["T"], c["L"]
    ms_step = wall * 1e3 / args.steps
    value = B * L / (wall / args.steps)
    # algorithmic bytes of one scan launch: every entry's 68-B indexer key read
    # once (the 4-B block keys it writes per 8 entries are workspace traffic,
    # reported beside it, not counted)
    scan_bytes = scan_bytes_per_launch(T, B)
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    modes = c["wl"].layers
    mode_us = {m: 1e3 * sum(t for t, mm in zip(per_layer, modes) if mm == m) /
               max(1, sum(1 for mm in modes if mm == m)) for m in ("full", "reindex", "reuse")}
    line = {
        "metric": "decode query-tokens/s per CSA2 layer at 1M ctx; HBM GB/s % of peak",
        "value": round(value, 1),
        "unit": "query-tokens/s per CSA2 layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": c["wl"].name, "batch": B, "context_entries": T, "layers": L,
                   "layer_modes": {"full": 1, "reindex": 4, "reuse": 15}, "heads": c["H"],
                   "k_blocks": c["wl"].k_blk, "k_pos": c["wl"].k_pos, "swa": c["wl"].swa,
                   "parallelism": "single GPU",
                   "launch": "HIP graph replay (scan with append, rest)" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "kernel": "score_kernel<block max> (csa2_index_scan_append)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": scan_traffic_bytes(),
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "block_key_bytes_written": BLOCK_KEY_BYTES * ((T + 7) // 8) * B,
                     "avg_launch_us": round(scan_ms * 1e3, 2)},
        "per_layer_us_eager": {k: round(v, 2) for k, v in mode_us.items()},
        "full_layer_query_tokens_per_s": round(B / (mode_us["full"] * 1e-6), 1),
        "build_s": round(t_build, 1),
    }
    if not args.graph and not args.no_configs:
        # the same step replayed as two HIP graphs (checked bit for bit
        # against the eager step first): the launch cost is the GPU's, not the host's
        wall_g, _, _ = run_gpu(c, args.steps, args.warmup, False)
        line["graph_replay_ms_per_step"] = round(wall_g * 1e3 / args.steps, 4)
    line["multi_query_scan"] = multi_query_scan(c)
    ms_4k = None
    if not args.no_configs:             # the same stack at 4,096 entries, for the 4K -> 1M ratio
        c4k = build(4096)
        wall4k, _, _ = run_gpu(c4k, args.steps, args.warmup, True)
        del c4k
        ms_4k = wall4k * 1e3 / args.steps
    line["launches_per_layer"] = launches_per_layer(c)
    line["pages_figures"] = pages_figures(c, ms_step, ms_4k, line["launches_per_layer"])
    line["hbm_copy_GBs"] = copy_bandwidth()
    if not args.no_attention_roofline:
        line["attention_b256_h64"] = reuse_attention(20, 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, args.cpu_rows)
    if not args.no_configs:
        line["other_workloads"] = {"tiny_decode": tiny_decode(20, 3), "prefill_chunk": prefill_chunk(10, 2),
                                   "decode_b32_128k": decode_b32(10, 2)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
