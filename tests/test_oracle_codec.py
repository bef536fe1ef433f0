"""Pins for the oracle's codecs (CPU only).

E4M3: the 256-code table is checked against torch's float8_e4m3fn decode (an
independent implementation of the OCP format the calibration guide names), the
maximum against the guide's printed 448, and the brute-force encoder against
torch's round-to-nearest-even cast on every bf16 bit pattern (clamped to +-448,
because torch's cast does not saturate) at several scales, plus every rounding
midpoint +-1 ulp.  E2M1: the value set of the OCP MX E2M1 element type and the
tie cases that follow from round-to-nearest-even.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_table_matches_independent_decode():
    ours = oracle.e4m3_table()
    ref = torch_e4m3_values()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert list(np.where(nan_ours)[0]) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    # signed zero kept in the table
    assert math.copysign(1.0, ours[0x80]) == -1.0 and ours[0x80] == 0.0


def test_e4m3_landmarks():
    t = oracle.e4m3_table()
    assert t[0x7E] == GOLDEN["e4m3_max"]["value"] == np.nanmax(t)
    assert t[0xFE] == -448.0
    assert t[0x38] == 1.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x7D] == 416.0
    finite = t[~np.isnan(t)]
    assert len(set(finite.tolist())) == 253  # +-0 collapse
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()       # codes 0..0x7E increasing
    assert list(t[0x78:0x7F]) == [256.0, 288.0, 320.0, 352.0, 384.0, 416.0, 448.0]


def _torch_encode_clamped(y: torch.Tensor) -> np.ndarray:
    return y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 0.0117, 1e-12, 3.3, 1.0e-3])
def test_e4m3_quantize_all_bf16_patterns(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32)
    s = np.float32(scale)
    y = x / torch.tensor(s)  # IEEE fp32 division
    ours = np.array([oracle.e4m3_quantize(int(b), float(s)) for b in bits], dtype=np.uint8)
    yn = y.numpy()
    finite = ~np.isnan(yn)
    ref = _torch_encode_clamped(y)
    assert np.array_equal(ours[finite], ref[finite])
    # NaN inputs: 0x7F with the NaN's sign
    nan_idx = np.where(~finite)[0]
    assert len(nan_idx) > 0
    sign = (bits[nan_idx] >> 15).astype(np.uint8)
    assert np.array_equal(ours[nan_idx], (0x7F | (sign << 7)).astype(np.uint8))


def test_e4m3_encode_rounding_midpoints():
    t = oracle.e4m3_table()
    pos = t[:0x7F]
    ys = []
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2.0)
        assert float(mid) == (a + b) / 2.0  # midpoints are exact in fp32
        for k in (-2, -1, 0, 1, 2):
            ys.append(np.nextafter(mid, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
                      if k else mid)
            if abs(k) == 2:
                ys[-1] = np.nextafter(ys[-1], np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
    ys = np.array(ys + [np.float32(448.0), np.float32(460.0), np.float32(464.0), np.float32(1e30)],
                  dtype=np.float32)
    ys = np.concatenate([ys, -ys])
    ours = np.array([oracle.e4m3_encode(float(y)) for y in ys], dtype=np.uint8)
    ref = _torch_encode_clamped(torch.from_numpy(ys))
    assert np.array_equal(ours, ref)


def test_e4m3_encode_special_values():
    enc = oracle.e4m3_encode
    assert enc(float("inf")) == 0x7E and enc(float("-inf")) == 0xFE  # saturating
    assert enc(465.0) == 0x7E and enc(-1e9) == 0xFE
    assert enc(float("nan")) == 0x7F
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00
    assert enc(-1e-4) == 0x80                                         # sign kept on underflow
    assert enc(2.0 ** -10) == 0x00                                    # tie -> even (0)
    assert enc(1.5 * 2.0 ** -9) == 0x02                               # tie -> even (2)
    assert enc(np.float32(1e-45)) == 0x00 and enc(-np.float32(1e-45)) == 0x80  # fp32 subnormal


def test_e2m1_values_and_ties():
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert vals[8:] == [-v for v in vals[:8]]
    enc = oracle.e2m1_encode
    # round-to-nearest-even on codes: ties go to the even code
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for y, want in ties.items():
        assert oracle.e2m1_value(enc(y)) == want
        assert oracle.e2m1_value(enc(-y)) == -want
    assert enc(6.5) == 0x7 and enc(float("inf")) == 0x7 and enc(-100.0) == 0xF
    assert enc(-0.0) == 0x8 and enc(-0.1) == 0x8
    # every representable value encodes to itself
    for c in range(16):
        assert enc(oracle.e2m1_value(c)) == c
    # nearest: a dense sweep never lands farther than half the local gap
    grid = np.array(vals[:8])
    for y in np.linspace(0, 6, 1201):
        got = oracle.e2m1_value(enc(float(y)))
        assert abs(got - y) <= np.min(np.abs(grid - y)) + 1e-12
