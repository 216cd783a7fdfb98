"""Pins for the oracle's sparse attention and SWA merge (CPU only).

  * brute-force dense attention: when the Top-K holds every visible entry, the
    sparse branch merged with the SWA branch must equal ordinary softmax
    attention over all keys, computed here with torch's fp64
    scaled_dot_product_attention (a library routine) on keys decoded
    independently of the oracle;
  * uniform keys give o = the key exactly;
  * the log-sum-exp merge of two disjoint key sets equals the joint softmax;
  * empty branches: no global keys -> SWA-only result, no SWA rows ->
    global-only result, nothing at all -> o = 0 and lse = -inf.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "ocp_e2m1_values.json")) as f:
    E2M1 = np.array(json.load(f)["magnitudes"])

SCALE = 1.0 / math.sqrt(512)


def decode_fp4(codes, scales, group=16):
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    s = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).double().numpy()
    return mag * np.repeat(s, group, axis=1)


def decode_e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).double().numpy()


def sdpa_fp64(q_bf16, keys):
    q = q_bf16.double()[None, :, None, :]                  # [1, H, 1, 512]
    k = torch.from_numpy(keys)[None, None].expand(1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, k, scale=SCALE)
    logits = (q @ k.transpose(-1, -2)) * SCALE
    return o[0, :, 0].numpy(), torch.logsumexp(logits, dim=-1)[0, :, 0].numpy()


@pytest.mark.parametrize("n_vis,n_swa,H", [(37, 20, 16), (300, 128, 16), (64, 0, 64), (5, 3, 16)])
def test_sparse_plus_swa_equals_dense_when_topk_covers_everything(n_vis, n_swa, H):
    lat = workloads.rms_rows(n_vis, 512, seed=n_vis).numpy()
    kvc, kvs = oracle.quantize(lat, 16)
    swa = workloads.swa_rows_e4m3(n_swa, 512, seed=n_swa + 1).numpy()
    q = workloads.bf16_normal((H, 512), seed=7)
    topk = np.full(512, -1, np.int32)
    topk[:n_vis] = np.arange(n_vis)
    r = oracle.attend_row(workloads.bf16_bits(q), kvc, kvs, topk, swa, SCALE)
    keys = np.concatenate([decode_fp4(kvc, kvs), decode_e4m3(swa).reshape(-1, 512)], axis=0)
    o_ref, lse_ref = sdpa_fp64(q, keys)
    np.testing.assert_allclose(r["o"], o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_ref, rtol=1e-12, atol=1e-12)
    og_ref, lseg_ref = sdpa_fp64(q, decode_fp4(kvc, kvs))
    np.testing.assert_allclose(r["o_g"], og_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse_g"], lseg_ref, rtol=1e-12, atol=1e-12)


def test_uniform_keys_give_the_key():
    lat = np.tile(workloads.rms_rows(1, 512, seed=3).numpy(), (50, 1))
    kvc, kvs = oracle.quantize(lat, 16)
    q = workloads.bf16_normal((16, 512), seed=4)
    r = oracle.attend_row(workloads.bf16_bits(q), kvc, kvs, np.arange(50, dtype=np.int32),
                          np.zeros((0, 512), np.uint8), SCALE)
    key = decode_fp4(kvc[:1], kvs[:1])[0]
    np.testing.assert_allclose(r["o"], np.tile(key, (16, 1)), rtol=0, atol=1e-13)
    # lse = logit + log(n) for n identical keys
    qd = q.double().numpy()
    np.testing.assert_allclose(r["lse"], SCALE * (qd @ key) + math.log(50), rtol=1e-12)


def test_lse_merge_of_disjoint_sets_equals_joint_softmax():
    rng = np.random.default_rng(0)
    keys = rng.standard_normal((200, 512))
    q = workloads.bf16_normal((16, 512), seed=9)
    qb = workloads.bf16_bits(q)
    perm = rng.permutation(200)
    a, b = keys[perm[:71]], keys[perm[71:]]
    o_a, l_a = oracle.attention(qb, a, SCALE)
    o_b, l_b = oracle.attention(qb, b, SCALE)
    o_m, l_m = oracle.lse_merge(o_a, l_a, o_b, l_b)
    o_j, l_j = oracle.attention(qb, keys, SCALE)
    np.testing.assert_allclose(o_m, o_j, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l_m, l_j, rtol=1e-12)


def test_empty_branches():
    lat = workloads.rms_rows(10, 512, seed=5).numpy()
    kvc, kvs = oracle.quantize(lat, 16)
    swa = workloads.swa_rows_e4m3(7, 512, seed=6).numpy()
    q = workloads.bf16_normal((16, 512), seed=8)
    qb = workloads.bf16_bits(q)
    none = np.full(512, -1, np.int32)
    r = oracle.attend_row(qb, kvc, kvs, none, swa, SCALE)             # no global keys
    assert np.all(np.isneginf(r["lse_g"])) and np.all(r["o_g"] == 0)
    o_s, l_s = sdpa_fp64(q, decode_e4m3(swa))
    np.testing.assert_allclose(r["o"], o_s, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"], l_s, rtol=1e-12)
    r2 = oracle.attend_row(qb, kvc, kvs, np.arange(10, dtype=np.int32),
                           np.zeros((0, 512), np.uint8), SCALE)       # no SWA rows
    np.testing.assert_array_equal(r2["o"], r2["o_g"])
    np.testing.assert_array_equal(r2["lse"], r2["lse_g"])
    r3 = oracle.attend_row(qb, kvc, kvs, none, np.zeros((0, 512), np.uint8), SCALE)
    assert np.all(np.isneginf(r3["lse"])) and np.all(r3["o"] == 0)


def test_single_key():
    lat = workloads.rms_rows(1, 512, seed=12).numpy()
    kvc, kvs = oracle.quantize(lat, 16)
    q = workloads.bf16_normal((16, 512), seed=13)
    r = oracle.attend_row(workloads.bf16_bits(q), kvc, kvs, np.array([0], np.int32),
                          np.zeros((0, 512), np.uint8), SCALE)
    key = decode_fp4(kvc, kvs)[0]
    np.testing.assert_allclose(r["o"], np.tile(key, (16, 1)), rtol=0, atol=0)
    np.testing.assert_allclose(r["lse"], SCALE * (q.double().numpy() @ key), rtol=1e-13)
