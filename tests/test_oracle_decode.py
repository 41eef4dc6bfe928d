"""Pins for the oracle's input decoders (CPU only).

Witnesses: torch's own format conversions (a library routine independent of
oracle.c) exhaustively over every code, and the format parameters printed in
Table 1 of "Accurate Models of AMD Matrix Cores" (tests/golden/table1_formats.txt).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table1_formats.txt")

TORCH_VIEW = {"bf16": (np.uint16, torch.int16, torch.bfloat16),
              "f16": (np.uint16, torch.int16, torch.float16),
              "e4m3": (np.uint8, torch.uint8, torch.float8_e4m3fn),
              "e5m2": (np.uint8, torch.uint8, torch.float8_e5m2)}


def all_codes(dt):
    npdt = TORCH_VIEW[dt][0]
    n = 1 << (8 * np.dtype(npdt).itemsize)
    return np.arange(n, dtype=np.int64).astype(npdt)


def torch_values(dt, codes):
    npdt, view, tdt = TORCH_VIEW[dt]
    t = torch.from_numpy(codes.view({np.uint16: np.int16, np.uint8: np.uint8}[npdt]))
    return t.view(tdt).to(torch.float64).numpy()


@pytest.mark.parametrize("dt", ["bf16", "f16", "e4m3", "e5m2"])
def test_decode_matches_torch_exhaustively(dt):
    codes = all_codes(dt)
    got = oracle.decode(dt, codes)
    want = torch_values(dt, codes)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w)
    assert np.array_equal(got[~nan_g], want[~nan_w])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan_g]), np.signbit(want[~nan_w]))


def test_decode_int8():
    codes = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(oracle.decode("i8", codes), np.arange(-128, 128, dtype=np.float64))


def read_table1():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, prec, minlog2, mx, approx = line.split()
            rows[name] = (int(prec), int(minlog2), float(mx), approx == "1")
    return rows


@pytest.mark.parametrize("dt", ["bf16", "f16", "e4m3", "e5m2"])
def test_decode_matches_table1(dt):
    prec, minlog2, mx, approx = read_table1()[dt]
    v = oracle.decode(dt, all_codes(dt))
    fin = v[np.isfinite(v)]
    # largest finite value
    if approx:
        assert abs(fin.max() - mx) / mx < 1e-3
    else:
        assert fin.max() == mx
    assert fin.min() == -fin.max()
    # smallest positive normal: the smallest positive value whose successor
    # is at the same spacing as its predecessor is not; equivalently the
    # values just above it are spaced by 2^(minlog2 - (prec - 1)).
    pos = np.unique(fin[fin > 0])
    spacing = np.diff(pos)
    sub_step = 2.0 ** (minlog2 - (prec - 1))
    # every positive value below 2^minlog2 is a multiple of the subnormal step
    below = pos[pos < 2.0 ** minlog2]
    assert np.all(np.mod(below, sub_step) == 0)
    assert 2.0 ** minlog2 in set(pos.tolist())
    # in [2^minlog2, 2^(minlog2+1)) the spacing is the same subnormal step,
    # and there are exactly 2^(prec-1) values (precision f incl. implicit bit)
    band = pos[(pos >= 2.0 ** minlog2) & (pos < 2.0 ** (minlog2 + 1))]
    assert band.size == 2 ** (prec - 1)
    assert np.all(np.diff(band) == sub_step)
    # precision: 1 + 2^(1-f) is representable, the spacing just above 1 is 2^(1-f)
    above_one = pos[pos > 1.0][0]
    assert above_one == 1.0 + 2.0 ** (1 - prec)
    assert spacing.min() > 0


def test_fp8_quantisation_targets():
    # 0.9 x the format maximum rounds (to nearest even) to these codes' values;
    # torch's conversion and the oracle's decoder must agree on them.
    for dt, mx, want in (("e4m3", 448.0, 416.0), ("e5m2", 57344.0, 49152.0)):
        t = torch.tensor([0.9 * mx], dtype=torch.float32).to(TORCH_VIEW[dt][2])
        code = t.view(torch.uint8).numpy()
        assert oracle.decode(dt, code)[0] == want
        assert math.isclose(want, 0.9 * mx, rel_tol=0.1)
