"""Seeded synthetic inputs and workload shapes for the CSA2 hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload shapes and the seeded random draws only -- none of the
method's arithmetic (no encoding, scoring, selection or attention).  Both the
HIP path and the oracle receive the tensors it produces.

The pages name no dataset for this path, so every input is synthetic, shaped
like the workloads the pages describe (P3 "레이어 40개 가운데 4개만 전역 캐시를
만듭니다": 512-channel main latent and 128-d indexer key per entry, 2,048 blocks
of 8, Top-512; P3 "전역 어텐션과 지역 어텐션": SWA window of 128; P3 "4비트로
적어도 되는 이유": cached values are normalised, so |x| <= sqrt(512)).

Value recipe:
  * main latent / indexer key / SWA rows: N(0,1) per element, then each row
    divided by its RMS (so |x_i| <= sqrt(dim)), fp32;
  * SWA rows are stored as OCP E4M3FN bytes (torch's float8_e4m3fn cast);
  * attention q and indexer q: N(0,1) rounded to bf16;
  * indexer head weights: U(0,1) fp32;
  * reuse-mode inherited Top-512: uniform without replacement over the
    visible entries, ascending;
  * reuse-mode context lengths: uniform integers in [64K, 256K].
Seeds: 0xC5A20000 + config id, mixed with a tensor id, a layer and a
sequence index through numpy's SeedSequence.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch

K = 1024
M = 1024 * 1024

# tensor ids for seed derivation
T_LATENT, T_IKEY, T_SWA, T_Q, T_QIDX, T_W, T_LEN, T_TOPK = range(8)


@dataclass
class Workload:
    cid: int
    name: str
    kind: str                 # "decode" | "prefill" | "reuse"
    batch: int                # query rows (decode/reuse) or sequences
    ctx: int                  # context tokens (max for reuse)
    entry_ratio: int          # tokens per stored entry (1 decoder, 2 encoder)
    heads: int                # attention heads sharing the 512-d latent
    k_blk: int                # blocks kept in the pool (0 = flat, no pool)
    k_pos: int                # Top-K positions
    swa: int                  # SWA window (tokens)
    layers: List[str] = field(default_factory=list)
    chunk: int = 0            # prefill: new query tokens
    ctx_min: int = 0          # reuse: minimum context

    @property
    def seed(self) -> int:
        return 0xC5A20000 + self.cid


WORKLOADS = {
    0: Workload(0, "tiny_full_decode_b1_4k", "decode", batch=1, ctx=4 * K, entry_ratio=1,
                heads=16, k_blk=64, k_pos=512, swa=128, layers=["full"]),
    1: Workload(1, "encoder_prefill_4k_chunk_64k_ctx", "prefill", batch=1, ctx=64 * K,
                entry_ratio=2, heads=16, k_blk=0, k_pos=512, swa=128, layers=["full"],
                chunk=4 * K),
    2: Workload(2, "decode_b32_128k_full_18reindex", "decode", batch=32, ctx=128 * K,
                entry_ratio=1, heads=16, k_blk=2048, k_pos=512, swa=128,
                layers=["full"] + ["reindex"] * 18),
    3: Workload(3, "decode_b8_1m_full_4reindex_15reuse", "decode", batch=8, ctx=1 * M,
                entry_ratio=1, heads=16, k_blk=2048, k_pos=512, swa=128,
                layers=["full"] + ["reindex"] * 4 + ["reuse"] * 15),
    4: Workload(4, "reuse_b256_64k_256k_h64", "reuse", batch=256, ctx=256 * K, entry_ratio=1,
                heads=64, k_blk=0, k_pos=512, swa=128, layers=["reuse"], ctx_min=64 * K),
}


def seed_for(base: int, tensor: int, layer: int = 0, seq: int = 0) -> int:
    ss = np.random.SeedSequence([base & 0xFFFFFFFF, tensor, layer, seq])
    return int(ss.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def rms_rows(n: int, dim: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 [n, dim]: N(0,1) rows divided by their RMS (|x_i| <= sqrt(dim))."""
    x = torch.randn(n, dim, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x * torch.rsqrt(x.square().mean(dim=1, keepdim=True))


def bf16_normal(shape, seed: int, device="cpu") -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, device), device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def uniform01(shape, seed: int, device="cpu") -> torch.Tensor:
    return torch.rand(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def swa_rows_e4m3(n: int, dim: int, seed: int, device="cpu") -> torch.Tensor:
    """uint8 [n, dim]: RMS-normalised N(0,1) rows cast to OCP E4M3FN bytes."""
    return rms_rows(n, dim, seed, device).to(torch.float8_e4m3fn).view(torch.uint8)


def lengths_uniform(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.Philox(seed))
    return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def topk_uniform(n_vis: int, k: int, seed: int) -> np.ndarray:
    """k distinct entry ids drawn uniformly from [0, n_vis), ascending, int32."""
    rng = np.random.Generator(np.random.Philox(seed))
    k = min(k, n_vis)
    return np.sort(rng.choice(n_vis, size=k, replace=False)).astype(np.int32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
