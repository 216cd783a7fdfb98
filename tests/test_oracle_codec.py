"""Pins for the oracle's FP4 E2M1 / E4M3 codec (CPU only).

The oracle is checked against things other than itself:
  * the E4M3FN decode against torch's float8_e4m3fn dtype (a library routine);
  * the E2M1 decode against the OCP MX value list (tests/golden);
  * encoding against an exact-rational brute force (nearest representable
    value, ties to the even code) on small random and constructed inputs;
  * the numbers the pages print: 256 + 32 = 288 B, 64 + 4 = 68 B, 356 B per
    entry, 890 B per token, 2,688 = 448 x 6, values bounded by about sqrt(512).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


PAGES = _gold("pages_numbers.json")
E2M1_MAGS = [Fraction(v).limit_denominator(4) for v in _gold("ocp_e2m1_values.json")["magnitudes"]]


def torch_e4m3(byte: int) -> float:
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


E4M3_POS = [Fraction(torch_e4m3(b)) for b in range(0x7F)]   # 0x00..0x7E, finite, >= 0


def nearest_even(value: Fraction, table):
    """Index of the entry of `table` nearest to `value`; ties go to the even index."""
    best, best_d = 0, abs(value - table[0])
    for i in range(1, len(table)):
        d = abs(value - table[i])
        if d < best_d or (d == best_d and i % 2 == 0 and best % 2 == 1):
            best, best_d = i, d
    return best


def brute_quantize(x: np.ndarray, group: int):
    """Exact-rational reading of the encoder: scale = nearest E4M3 to amax/6,
    magnitude = nearest E2M1 to |x|/scale (0 if the scale is 0), ties to the
    even code, sign bit = (x < 0), channel 2k in the low nibble."""
    n, dim = x.shape
    codes = np.zeros((n, dim // 2), np.uint8)
    scales = np.zeros((n, dim // group), np.uint8)
    for r in range(n):
        for g in range(dim // group):
            vals = [Fraction(float(v)) for v in x[r, g * group:(g + 1) * group]]
            amax = max(abs(v) for v in vals)
            sb = nearest_even(amax / 6, E4M3_POS)
            s = E4M3_POS[sb]
            scales[r, g] = sb
            for i, v in enumerate(vals):
                mag = 0 if s == 0 else nearest_even(abs(v) / s, E2M1_MAGS)
                code = (8 if v < 0 else 0) | mag
                ch = g * group + i
                codes[r, ch // 2] |= (code << 4) if ch % 2 else code
    return codes, scales


# ------------------------------------------------------------------ decode
def test_e4m3_decode_matches_torch_float8_for_all_bytes():
    for b in range(256):
        got = oracle.e4m3_value(b)
        ref = torch_e4m3(b)
        if math.isnan(ref):
            assert math.isnan(got), b
        else:
            assert got == ref, (b, got, ref)


def test_e2m1_decode_matches_ocp_table():
    for c in range(16):
        mag = float(E2M1_MAGS[c & 7])
        assert oracle.e2m1_value(c) == (-mag if c & 8 else mag)


def test_format_maxima_match_pages():
    # P3 '4비트로 적어도 되는 이유': the format reaches 2,688 = 448 x 6.
    assert oracle.e4m3_value(0x7E) == PAGES["scale_max"]["value"]
    assert oracle.e2m1_value(7) == PAGES["value_max"]["value"]
    codes = np.array([[0x77] * 8], np.uint8)                # code 7 in both nibbles
    scales = np.array([[0x7E]], np.uint8)
    xhat = oracle.dequantize(codes, scales, 16)
    assert xhat.max() == PAGES["fp4_range_max"]["value"]


# ------------------------------------------------------------------ encode
@pytest.mark.parametrize("dim,group", [(512, 16), (128, 32)])
def test_encode_matches_exact_rational_bruteforce_random(dim, group):
    x = workloads.rms_rows(6, dim, seed=11 + dim).numpy()
    x[1] *= 1e-3            # small groups -> small scales
    x[2] *= 3e-5            # subnormal E4M3 scales
    x[3, :group] = 0.0      # an all-zero group
    x[4] *= 50.0            # large values, scales in the tens
    codes, scales = oracle.quantize(x, group)
    bc, bs = brute_quantize(x, group)
    assert np.array_equal(scales, bs)
    assert np.array_equal(codes, bc)


def test_value_ties_round_to_even():
    # group with an element equal to 6*s fixes the scale at s exactly; the
    # other elements sit on every E2M1 midpoint.
    s = 0.5                                      # an E4M3 value (0x30)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0, 2, 2, 4, 4, 6, 6]               # ties go to the even code
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6 * s
    for i, t in enumerate(ties):
        x[0, 1 + i] = t * s
        x[0, 8 + i] = -t * s
    codes, scales = oracle.quantize(x, 16)
    assert oracle.e4m3_value(int(scales[0, 0])) == s
    nib = [(codes[0, c // 2] >> (4 * (c % 2))) & 15 for c in range(16)]
    assert nib[0] == 7
    assert nib[1:8] == expect
    assert nib[8:15] == [8 | e for e in expect]
    bc, bs = brute_quantize(x, 16)
    assert np.array_equal(codes, bc) and np.array_equal(scales, bs)


def test_scale_ties_round_to_even():
    # amax/6 exactly halfway between two E4M3 values -> the even code.
    pos = [float(v) for v in E4M3_POS]
    checked = 0
    for b in range(1, 0x7E):
        mid = (pos[b] + pos[b + 1]) / 2
        amax = np.float32(6 * mid)
        if float(amax) != 6 * mid:
            continue
        x = np.zeros((1, 16), np.float32)
        x[0, 3] = amax
        _, scales = oracle.quantize(x, 16)
        want = b if b % 2 == 0 else b + 1
        assert scales[0, 0] == want, (b, mid)
        checked += 1
    assert checked > 100


def test_sign_of_zero_and_tiny_negatives():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0                      # scale 1
    x[0, 1] = -0.0                     # -> 0x0
    x[0, 2] = -0.1                     # rounds to magnitude 0, keeps the sign -> 0x8
    x[0, 3] = 0.1                      # -> 0x0
    codes, _ = oracle.quantize(x, 16)
    nib = [(codes[0, c // 2] >> (4 * (c % 2))) & 15 for c in range(4)]
    assert nib == [7, 0, 8, 0]


def test_all_zero_group_and_scale_underflow():
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = -1e-5                  # amax/6 below half the smallest subnormal
    codes, scales = oracle.quantize(x, 16)
    assert list(scales[0]) == [0, 0]
    assert all(b == 0 for b in codes[0, :8])
    assert all(b == 0x88 for b in codes[0, 8:])


def test_roundtrip_and_error_bound():
    x = workloads.rms_rows(64, 512, seed=5).numpy()
    codes, scales = oracle.quantize(x, 16)
    xhat = oracle.dequantize(codes, scales, 16)
    s = np.repeat(np.array([[oracle.e4m3_value(int(b)) for b in row] for row in scales]), 16, axis=1)
    assert np.all(np.abs(x - xhat) <= s + 1e-12)
    # groups holding a +-6 code decode to amax = 6 s exactly and re-encode to
    # the same codes; a negative value that rounded to magnitude 0 (code 0x8)
    # decodes to -0.0, which re-encodes as 0x0, so zeros are compared unsigned.
    c2, s2 = oracle.quantize(xhat.astype(np.float32), 16)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(64, 32, 16)
    nib2 = np.stack([c2 & 15, c2 >> 4], axis=-1).reshape(64, 32, 16)
    has6 = (nib & 7).max(axis=2) == 7
    assert has6.mean() > 0.5
    assert np.array_equal(s2[has6], scales[has6])
    unsigned_zero = lambda n: np.where((n & 7) == 0, 0, n)
    assert np.array_equal(unsigned_zero(nib2)[has6], unsigned_zero(nib)[has6])


# ------------------------------------------------------------ page numbers
def test_entry_and_token_byte_accounting():
    x = workloads.rms_rows(1, 512, seed=1).numpy()
    k = workloads.rms_rows(1, 128, seed=2).numpy()
    kc, ks = oracle.quantize(x, oracle.KV_GROUP)
    ic, isc = oracle.quantize(k, oracle.IK_GROUP)
    assert kc.nbytes == PAGES["main_kv_value_bytes"]["value"]
    assert ks.nbytes == PAGES["main_kv_scale_bytes"]["value"]
    assert kc.nbytes + ks.nbytes == PAGES["main_kv_bytes"]["value"]
    assert ic.nbytes + isc.nbytes == PAGES["indexer_key_bytes"]["value"]
    entry = kc.nbytes + ks.nbytes + ic.nbytes + isc.nbytes
    assert entry == PAGES["entry_bytes"]["value"]
    # 3 encoder Full layers at 1 entry per 2 tokens + 1 decoder Full layer at 1 per token
    per_token = Fraction(PAGES["encoder_full_layers"]["value"], 2) + PAGES["decoder_full_layers"]["value"]
    assert per_token == Fraction(PAGES["entries_per_token"]["value"])
    assert per_token * entry == PAGES["bytes_per_token"]["value"]
    # every one of the 38 CSA2 layers storing its own cache: 18 encoder x 1/2 + 20 decoder x 1
    every = Fraction(PAGES["csa2_layers"]["value"] - 20, 2) + 20
    assert every == PAGES["entries_per_token_if_every_layer_stored"]["value"]
    assert round(float(every / per_token), 1) == PAGES["ratio_if_every_layer_stored"]["value"]
    # 3,514 / 890 is about 1/4; 389,120 / 890 rounds to 437
    assert round(PAGES["v1_bytes_per_token"]["value"] / PAGES["bytes_per_token"]["value"]) == \
        PAGES["v1_reduction"]["value"]
    assert abs(PAGES["v4_flash_bytes_per_token"]["value"] / PAGES["bytes_per_token"]["value"] - 4) < 0.1


def test_normalised_values_never_saturate():
    # P3 '4비트로 적어도 되는 이유': normalised cache values stay below about
    # sqrt(512) ~ 22.6, far inside the 2,688 range, so no global scale is needed.
    assert round(math.sqrt(512), 1) == PAGES["normalised_value_bound"]["value"]
    x = workloads.rms_rows(256, 512, seed=3).numpy()
    assert np.abs(x).max() <= math.sqrt(512) * (1 + 1e-6)
    _, scales = oracle.quantize(x, 16)
    smax = max(oracle.e4m3_value(int(b)) for b in np.unique(scales))
    assert smax <= 3.75
    # the one-hot extreme sqrt(512) * e_1: scale rounds to 3.75, |x|/s = 6.03 -> code 6.0 -> 22.5
    one_hot = np.zeros((1, 512), np.float32)
    one_hot[0, 0] = np.float32(math.sqrt(512))
    c, s = oracle.quantize(one_hot, 16)
    assert oracle.e4m3_value(int(s[0, 0])) == 3.75
    assert (c[0, 0] & 15) == 7
    assert oracle.dequantize(c, s, 16)[0, 0] == 22.5
    # the 128-d indexer key with one scale per 32 channels: bound sqrt(128)/6 -> 1.875
    k = workloads.rms_rows(256, 128, seed=4).numpy()
    _, ks = oracle.quantize(k, 32)
    assert max(oracle.e4m3_value(int(b)) for b in np.unique(ks)) <= 1.875
