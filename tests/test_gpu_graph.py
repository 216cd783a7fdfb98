"""Replays of the decode step captured as HIP graphs reproduce the eagerly
launched step bit for bit, replay after replay, with eager work and
synchronisations between the replays (the kernels are deterministic: fixed
reduction orders, no atomics on values)."""
import pytest
import torch

import bench


@pytest.mark.gpu
def test_graph_replays_match_eager_step():
    c = bench.build(ctx_override=65536)
    bench.step(c)
    torch.cuda.synchronize()
    ref = bench._outputs(c)
    graphs = bench.capture(c)
    for rep in range(3):
        for t in c["topk"] + c["n_topk"] + [c["pool"], c["n_pool"]]:
            t.fill_(-7)
        c["o"].fill_(float("nan"))
        c["lse"].fill_(float("nan"))
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        got = bench._outputs(c)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"
    # the eager step still agrees after the replays
    bench.step(c)
    torch.cuda.synchronize()
    for a, b in zip(ref, bench._outputs(c)):
        assert torch.equal(a, b)
