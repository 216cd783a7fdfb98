"""Host-side checks of bench.py that need no GPU: the one-GPU contract of its
command line, and the closed forms behind the figures it prints beside the
pages' own (bytes per entry and per token, decode flops from 4K to 1M)."""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_path_flops_closed_form():
    wl = W.WORKLOADS[3]          # 1 Full + 4 Reindex + 15 Reuse, 16 heads, 2,048 blocks, Top-512, SWA 128
    # 4,096 entries: the pool holds every entry (512 blocks < 2,048)
    scan, rescore, attn = 2048 * 4096, 2048 * 4096 * 5, 20 * 4 * 16 * 512 * (512 + 128)
    assert bench.path_flops_per_query(4096, wl) == scan + rescore + attn == 469_762_048
    # 1M entries: the pool is capped at 16,384 candidates, only the scan grows
    scan, rescore = 2048 * (1 << 20), 2048 * 16384 * 5
    assert bench.path_flops_per_query(1 << 20, wl) == scan + rescore + attn == 2_734_686_208


def test_pages_figures_from_the_cache_layout():
    import fp4_compressed_sparse_e2m1_amd as csa2

    class Planes:                # the four planes' bytes of an 8 x 1,000-entry cache
        nbytes = 8 * 1000 * (256 + 32 + 64 + 4)

    c = dict(csa2=csa2, wl=W.WORKLOADS[3], cache=Planes(), B=8, T=1000, H=16)
    launches = {"full": {"kernels": 7}, "reindex": {"kernels": 3}, "reuse": {"kernels": 1}}
    f = bench.pages_figures(c, launches=launches)
    assert f["bytes_per_entry"] == {"csa2_amd": 356, "pages": 356}
    assert f["bytes_per_token_at_2_5_entries"]["csa2_amd"] == 890
    assert f["kernels_per_reuse_layer_decode"]["csa2_amd"] == 1     # as counted in the step's graph
    assert bench.pages_figures(c)["kernels_per_reuse_layer_decode"]["csa2_amd"] is None
    assert abs(f["decode_flops_1m_over_4k"]["csa2_amd"] - 2_734_686_208 / 469_762_048) < 1e-3


def test_host_description():
    assert bench.host_cores() >= 1
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
