"""Pins for the oracle's storage formats: bf16 (RNE) and OCP e4m3fn (RNE, saturating)."""
import math

import numpy as np
import torch


def _ocp_e4m3(c):
    """OCP 8-bit FP spec, E4M3: bias 7, subnormals m*2^-9, S.1111.111 = NaN, no inf."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def test_bf16_decode_all_patterns(orc):
    h = np.arange(0, 65536, 7, dtype=np.uint16)
    lib = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for v, want in zip(h[:4000], lib[:4000]):
        got = orc.bf16_to_f64(int(v))
        assert (math.isnan(got) and math.isnan(want)) or got == want


def test_bf16_encode_matches_torch_rne(orc):
    x = torch.randn(20000, generator=torch.Generator().manual_seed(0), dtype=torch.float32) * 37.0
    want = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f64_to_bf16(float(v)) for v in x.tolist()], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_ties_and_direct_rounding(orc):
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even
    assert orc.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (up)
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie: no double rounding
    assert orc.f64_to_bf16(-2.5) == 0xC020
    assert orc.f64_to_bf16(1e39) == 0x7F80
    assert orc.f64_to_bf16(float("nan")) & 0x7F80 == 0x7F80


def test_e4m3_decode_all_codes(orc):
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got, want = orc.e4m3_to_f64(c), _ocp_e4m3(c)
        if math.isnan(want):
            assert math.isnan(got) and math.isnan(lib[c])
        else:
            assert got == want == lib[c]
    assert orc.e4m3_to_f64(0x7E) == 448.0 and orc.e4m3_to_f64(0x01) == 2.0 ** -9


def test_e4m3_roundtrip_codes(orc):
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert orc.f64_to_e4m3(orc.e4m3_to_f64(c)) == c


def test_e4m3_encode_matches_torch_in_range(orc):
    g = torch.Generator().manual_seed(1)
    x = torch.cat([torch.randn(4000, generator=g) * s for s in (0.003, 0.1, 1.0, 30.0, 150.0)])
    x = x[x.abs() < 440]
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.f64_to_e4m3(float(v)) for v in x.tolist()], np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_ties_saturation_and_bound(orc):
    assert orc.f64_to_e4m3(1.0625) == 0x38        # tie between 1.0 and 1.125 -> even (1.0)
    assert orc.f64_to_e4m3(1.1875) == 0x3A        # tie between 1.125 and 1.25 -> even (1.25)
    assert orc.f64_to_e4m3(460.0) == 0x7E         # rounds to 448
    assert orc.f64_to_e4m3(470.0) == 0x7E         # would round to 480: saturates
    assert orc.f64_to_e4m3(-1e9) == 0xFE
    assert orc.f64_to_e4m3(2.0 ** -10) == 0x00    # tie between 0 and 2^-9 -> even (0)
    assert orc.f64_to_e4m3(3 * 2.0 ** -10) == 0x02
    rs = np.random.default_rng(3)
    for v in rs.standard_normal(3000) * 50:
        if abs(v) > 448:
            continue
        d = orc.e4m3_to_f64(orc.f64_to_e4m3(float(v)))
        a = abs(v)
        ulp = 2.0 ** -9 if a < 2.0 ** -6 else 2.0 ** (math.floor(math.log2(a)) - 3)
        assert abs(d - v) <= ulp / 2 + 1e-300


def test_row_bytes(orc):
    assert orc.row_bytes(512, orc.BF16) == 1024
    assert orc.row_bytes(128, orc.BF16) == 256
    assert orc.row_bytes(512, orc.FP8) == 512 + 8 * 4
    assert orc.row_bytes(512, orc.F32) == 2048
