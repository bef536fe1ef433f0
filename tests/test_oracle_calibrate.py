"""Pins for the oracle's calibration and amax (CPU only).

The calibration guide prints scale = max(amax x 1.05 / 448, 1e-12).  What the
formula fixes beyond retyping it: (1) a tensor quantized with the scale
calibrated on itself never saturates, and its largest element lands exactly
on code 0x7D (416 = the E4M3 value nearest 448 / 1.05 = 426.67); dropping the
headroom would give 0x7E, a wrong maximum (e.g. 240) would saturate;
(2) the floor binds exactly below 1e-12 * 448 / 1.05; (3) the map is monotone
and scale-covariant by powers of two above the floor.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_constants_match_pages():
    assert GOLDEN["e4m3_max"]["value"] == 448
    assert GOLDEN["scale_headroom"]["value"] == 1.05
    assert GOLDEN["scale_floor"]["value"] == 1e-12


def test_floor_and_zero():
    s = oracle.calibrate([0.0, 1e-20, 4.0e-10])
    assert (s == np.float32(1e-12)).all()
    assert s[0].view(np.uint32) == 0x2B8CBCCC  # fp32(1e-12) = 9.999999960041972e-13
    thr = 1e-12 * 448.0 / 1.05  # 4.2667e-10
    lo, hi = oracle.calibrate([thr * 0.999, thr * 1.001])
    assert lo == np.float32(1e-12) and hi > np.float32(1e-12)


def test_self_calibrated_max_is_416_never_saturates():
    rng = np.random.default_rng(1)
    for e in rng.uniform(-12, 12, size=400):
        a = np.float32(2.0 ** e)
        bits = int(torch.tensor([a]).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        amax = float(torch.tensor([a]).to(torch.bfloat16).float().item())
        s = oracle.calibrate([amax])[0]
        code = oracle.e4m3_quantize(bits, float(s))
        assert code == 0x7D, (amax, s, hex(code))


def test_monotone_and_power_of_two_covariant():
    a = np.sort(np.random.default_rng(2).uniform(1e-3, 1e3, size=1000).astype(np.float32))
    s = oracle.calibrate(a)
    assert (np.diff(s) >= 0).all()
    s2 = oracle.calibrate(a * np.float32(4.0))
    assert np.array_equal(s2, s * np.float32(4.0))


def test_unity_point():
    # amax = 448 / 1.05 gives scale 1 (to fp32 rounding of the argument)
    s = oracle.calibrate([np.float32(448.0 / 1.05)])[0]
    assert abs(float(s) - 1.0) < 1e-7


@pytest.mark.parametrize("bad", [-1.0, float("nan"), float("inf"), -0.5e-30])
def test_rejects_bad_amax(bad):
    with pytest.raises(ValueError):
        oracle.calibrate([1.0, bad])


def test_nvfp4_global_scale_fits_e2m1_times_e4m3():
    # the largest element of a self-calibrated tensor must map to a block
    # scale <= 448 and an element code <= 6: amax / (6 * gscale) = 448 / 1.05
    a = np.float32(3.7)
    g = oracle.nvfp4_calibrate([a])[0]
    assert float(a) / (6.0 * float(g)) == pytest.approx(448.0 / 1.05, rel=1e-6)
    assert oracle.nvfp4_calibrate([0.0])[0] == np.float32(1e-12)


def test_amax_matches_numpy_and_propagates_nan():
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(37, 5, 64, generator=g) * 3).to(torch.bfloat16)
    want = float(x.float().abs().max())
    assert oracle.amax_bf16(x) == want
    x2 = x.clone()
    x2[3, 1, 7] = float("nan")
    assert math.isnan(oracle.amax_bf16(x2))
    x3 = x.clone()
    x3[0, 0, 0] = float("-inf")
    assert oracle.amax_bf16(x3) == float("inf")
    assert oracle.amax_bf16(torch.zeros(4, 8, dtype=torch.bfloat16)) == 0.0
