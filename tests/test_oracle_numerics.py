"""Pins of the oracle's number formats against definitions, library routines and
brute force (CPU only)."""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import numerics as nx
from oracle import scalar

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_bf16_golden_points():
    for row in _rows("bf16_points.txt"):
        x = float.fromhex(row[0])
        assert int(oracle.bf16_round(np.array([x]))[0]) == int(row[1], 16), row


def test_bf16_matches_torch_on_fp32_inputs():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000).astype(np.float32) * np.float32(3.0),
                        (g.standard_normal(2000) * 1e-39).astype(np.float32),      # fp32 subnormals
                        np.array([1.00390625, 1.01171875, -2.5, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_direct_rounding_matches_exact_rationals():
    g = np.random.default_rng(2)
    # fp64 values with random low bits, including many just around bf16 midpoints
    base = g.standard_normal(3000)
    mid = (oracle.bf16_to_f64(oracle.bf16_round(base)) + np.ldexp(1.0, np.floor(np.log2(np.abs(base))).astype(int) - 8))
    x = np.concatenate([base, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    got = oracle.bf16_to_f64(oracle.bf16_round(x))
    for xi, gi in zip(x, got):
        assert scalar.bf16_of(float(xi)) == gi


def test_e2m1_table_golden_and_bitfields():
    for code, val in _rows("e2m1_values.txt"):
        v = float(val)
        assert nx.e2m1_value(int(code)) == v and np.signbit(nx.e2m1_value(int(code))) == np.signbit(v)
        assert scalar.e2m1(int(code)) == v


def test_e4m3_golden_points():
    for b, val in _rows("e4m3_points.txt"):
        got = float(nx.e4m3_value(int(b, 16)))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == np.signbit(float(val))


def test_e4m3_all_bytes_match_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = nx.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert all(scalar.e4m3(b) == got[b] for b in range(256) if ok[b])


def test_e4m3_rne_matches_torch_cast():
    g = np.random.default_rng(3)
    v = np.concatenate([np.abs(g.standard_normal(20000)) * 50, np.abs(g.standard_normal(2000)) * 0.01,
                        nx.E4M3_POS, (nx.E4M3_POS[:-1] + nx.E4M3_POS[1:]) / 2]).astype(np.float32)
    v = v[v <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = nx.e4m3_rne_scale(v.astype(np.float64), np.ones(len(v)))
    assert np.array_equal(got, ref)
    # saturation above the grid
    assert int(nx.e4m3_rne_scale(np.array([1e6]), np.array([1.0]))[0]) == 126


def test_product_of_element_and_scale_is_exact_in_bf16():
    # every E2M1 x E4M3 product has <= 6 significant bits and lies in [2^-10, 2688]
    p = nx.e2m1_value(np.arange(16))[:, None] * nx.e4m3_value(np.arange(127))[None, :]
    assert np.array_equal(oracle.bf16_to_f64(oracle.bf16_round(p)), p)
    nz = np.abs(p[p != 0])
    assert nz.min() == 2.0 ** -10 and nz.max() == 2688.0


def _brute_code(x: float, unit: float) -> int:
    best = None
    for c in range(16):
        v = Fraction(scalar.e2m1(c)) * Fraction(unit)
        dist = abs(Fraction(x) - v)
        key = (dist, c & 1, c)  # nearest; ties -> even magnitude code
        if c == 8:
            continue  # -0 is never produced
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_nvfp4_pack_codes_match_brute_force():
    g = np.random.default_rng(4)
    w = g.standard_normal((6, 64)) * 0.02
    w[0, :16] = 0.0                  # an all-zero block
    w[1, 3] = 0.5                    # a large outlier
    codes, scales, ts = oracle.nvfp4_pack(w)
    assert ts == np.float32(np.float32(np.abs(w).max()) / np.float32(2688.0))
    for n in range(w.shape[0]):
        for b in range(w.shape[1] // 16):
            blk = w[n, b * 16:(b + 1) * 16]
            # scale: nearest E4M3 to amax/(6 ts), ties to even byte
            target = Fraction(float(np.abs(blk).max())) / (6 * Fraction(float(ts)))
            e4 = [Fraction(scalar.e4m3(i)) for i in range(127)]
            si = min(range(127), key=lambda i: (abs(e4[i] - target), i & 1))
            assert scales[n, b] == si
            unit = float(e4[si]) * float(ts)
            for j in range(16):
                k = b * 16 + j
                byte = codes[n, k // 2]
                c = (byte >> 4) if (k & 1) else (byte & 15)
                want = 0 if unit == 0 else _brute_code(float(blk[j]), unit)
                assert c == want, (n, k, blk[j], unit)


def test_nvfp4_round_trip_on_grid_values():
    g = np.random.default_rng(5)
    N, K = 8, 64
    sc = g.integers(1, 127, size=(N, K // 16))
    c = g.integers(0, 16, size=(N, K))
    c[c == 8] = 0
    # force one |code| = 6 per block so the block amax pins its scale exactly
    c[:, ::16] = 7
    sc[0, 0] = 126                     # one block at the top scale pins ts = 1
    w = nx.e2m1_value(c) * np.repeat(nx.e4m3_value(sc), 16, axis=1)
    codes, scales, ts = oracle.nvfp4_pack(w)
    assert ts == np.float32(1.0)
    assert np.array_equal(oracle.nvfp4_decode(codes, scales, ts), w)


def test_nvfp4_decode_error_bound():
    g = np.random.default_rng(6)
    w = g.standard_normal((32, 256)) * 0.02
    codes, scales, ts = oracle.nvfp4_pack(w)
    dec = oracle.nvfp4_decode(codes, scales, ts)
    s = np.repeat(nx.e4m3_value(scales), 16, axis=1) * float(ts)
    # within half a grid step (the largest step, 2 units, between 4 and 6) of the block scale,
    # plus the scale's own rounding (the block max may saturate at 6 units)
    assert np.all(np.abs(dec - w) <= 1.0 * s + 1e-18)
    assert np.abs(dec - w).max() / np.abs(w).max() < 0.2


def test_fp4_act_quant_matches_scalar_oracle_on_fp64_values():
    g = np.random.default_rng(7)
    a = g.standard_normal((6, 64)) * 0.7
    a[2, :16] = 0
    a[3, 16:32] = 3000.0  # saturating block
    # a block whose scale is 1 (amax 6) and whose element sits above the 0 / 0.5 midpoint 0.25
    # by less than fp32 resolution: the decision is taken on the fp64 value, so it rounds up
    # to 0.5 (an fp32 copy of it would be the midpoint itself, a tie going to the even code 0)
    a[5, :16] = 0.0
    a[5, 0] = 6.0
    a[5, 1] = 0.25 * (1 + 2.0 ** -40)
    a[5, 2] = 0.25
    codes, scales = oracle.fp4_act_quant(a)
    dec = oracle.nvfp4_decode(codes, scales, 1.0)
    assert dec[5, 0] == 6.0 and dec[5, 1] == 0.5 and dec[5, 2] == 0.0
    for r in range(a.shape[0]):
        assert np.array_equal(dec[r], np.array(scalar.act_quant_dequant([float(x) for x in a[r]])))
    # the decision thresholds 6*mid(e4m3) and mid(e2m1)*s are exact fp32 numbers
    mids = (nx.E4M3_POS[:-1] + nx.E4M3_POS[1:]) / 2 * 6
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)
    m2 = ((nx.E2M1_GRID[:-1] + nx.E2M1_GRID[1:]) / 2)[:, None] * nx.E4M3_POS[None, :]
    assert np.array_equal(m2.astype(np.float32).astype(np.float64), m2)
