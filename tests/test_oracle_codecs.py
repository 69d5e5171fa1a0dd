"""Pins of the oracle's number codecs against library routines and the OCP MX
specification (bf16, FP8 E4M3FN, E8M0, MXFP8 block quantisation)."""
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_exhaustive_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_decode(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000).astype(np.float32),
        # exact ties: bf16 value + half an ulp (low 16 bits = 0x8000)
        (rng.integers(0, 2**31, 50000, dtype=np.uint32) & np.uint32(0x7F7F0000) | np.uint32(0x8000)).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.39e38, -3.4e38], dtype=np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = _torch_bf16_bits(x)
    got = orc.bf16_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_decode_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_golden_codes():
    for line in open(os.path.join(GOLDEN, "e4m3fn_codes.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = orc.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")
            if float(val) != 0.0 or not val.startswith("-"):
                assert orc.e4m3_encode(np.array([float(val)]))[0] == int(code, 16)


def test_e4m3_encode_all_bf16_in_range_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = orc.bf16_decode(bits)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    v = v[keep]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_encode(v)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    big = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e6, -1e6, -470.0])
    assert np.array_equal(orc.e4m3_encode(big), np.array([0x7E] * 6 + [0xFE, 0xFE], dtype=np.uint8))


def test_e4m3_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)


def test_e8m0_decode():
    s = np.array([0, 1, 126, 127, 128, 254, 255], dtype=np.uint8)
    d = orc.e8m0_decode(s)
    assert d[0] == 2.0 ** -127 and d[3] == 1.0 and d[4] == 2.0 and d[5] == 2.0 ** 127 and np.isnan(d[6])


def test_mx_quantize_properties_and_library_element_step():
    rng = np.random.default_rng(5)
    v = orc.bf16_round(rng.standard_normal((64, 256)) * 10.0 ** rng.integers(-6, 6, (64, 1)))
    v[3, 32:64] = 0.0                                 # an all-zero block
    codes, scales = orc.mx_quantize(v)
    assert codes.shape == v.shape and scales.shape == (64, 8)
    assert scales[3, 1] == 0 and not codes[3, 32:64].any()
    vb = v.reshape(64, 8, 32)
    amax = np.abs(vb).max(-1)
    nz = amax > 0
    s = scales.astype(np.int64) - 127
    # scale exponent = floor(log2 amax) - 8, read from the exponent bits
    assert np.array_equal(s[nz], (np.floor(np.log2(amax[nz])).astype(np.int64) - 8))
    # element step = torch's E4M3FN conversion of v / 2^s after clamping to +-448
    scaled = np.clip(vb / np.ldexp(1.0, s)[..., None], -448, 448)
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes.reshape(64, 8, 32)[nz], ref[nz])
    # error bound: half an E4M3 ulp (relative 2^-4), except saturated elements (< 12.5 %)
    dq = orc.mx_dequantize(codes, scales)
    err = np.abs(dq - v)
    assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, np.ldexp(1.0, np.repeat(s, 32, axis=1) - 10)) + np.abs(v) * 0.125 * (np.abs(v) * np.repeat(np.ldexp(1.0, -s), 32, axis=1) > 448))


def test_mx_quantize_lossless_for_representable_blocks():
    rng = np.random.default_rng(6)
    # values that are E4M3 codes times a power of two, max element sets the scale
    c = rng.integers(0, 256, (16, 64)).astype(np.uint8)
    c = np.where((c & 0x7F) == 0x7F, 0x38, c)
    vals = orc.e4m3_decode(c)
    vals[:, ::32] = 256.0                             # amax 256 -> shared exponent 0
    v = vals * 2.0 ** 3
    codes, scales = orc.mx_quantize(v)
    assert (scales == 130).all()
    assert np.array_equal(orc.mx_dequantize(codes, scales), v)


def test_bf16_round_delta_marks_only_midpoints():
    # a value exactly half-way between two bf16 neighbours, one a hair above it, and
    # values well inside a rounding interval
    lo = orc.bf16_decode(np.array([0x3F80], np.uint16))[0]          # 1.0
    step = 2.0 ** -7
    mids = np.array([lo + step / 2, lo + step / 2 * (1 + 1e-9), -(lo + step / 2)])
    inner = np.array([lo + step / 4, lo + 3 * step / 4, 3.0 + step / 8, -7.1])
    d_mid = orc.bf16_round_delta(mids)
    assert np.allclose(d_mid, step * np.array([1, 1, 1]))
    assert np.all(orc.bf16_round_delta(inner) == 0)
    # on random values only the few within 2^-14 (relative) of a midpoint are flagged:
    # about 2 * 2^-14 / 2^-7.5, i.e. 2 %
    v = np.random.default_rng(2).standard_normal(200000)
    assert np.count_nonzero(orc.bf16_round_delta(v)) < 0.03 * v.size


def test_mx_requant_delta_marks_only_ambiguous_decisions():
    rng = np.random.default_rng(8)
    # values sitting exactly between two E4M3 codes (after bf16 rounding) at scale 2^0
    c = np.array([0x40, 0x42, 0x50, 0x60], np.uint8)   # even mantissas: the tie rounds down to c
    lo, hi = orc.e4m3_decode(c), orc.e4m3_decode(c + 1)
    row = np.full(32, 1.0)
    row[0] = 256.0                                   # amax 256: shared exponent 0
    mid = (lo + hi) / 2                              # an E4M3 tie, itself a bf16 value
    ulp = 2.0 ** (np.floor(np.log2(mid)) - 7)
    row[1:5] = mid + ulp / 2                         # bf16 rounds it to mid (tie -> even code) or above
    row[5:9] = lo * (1 + 2.0 ** -12) + 0.0           # clearly inside a code interval
    base, delta = orc.mx_requant_delta(row[None])
    assert np.array_equal(base[0], orc.mx_fake_quant(orc.bf16_round(row))[None][0])
    assert np.all(delta[0, 1:5] > 0)                 # a tie can round either way
    assert np.all(delta[0, 5:9] == 0) and delta[0, 0] == 0
    # random data: most decisions are unambiguous, and every delta is one code step or a scale step
    v = rng.standard_normal((64, 256))
    base, delta = orc.mx_requant_delta(v)
    assert np.mean(delta > 0) < 0.01
    nz = delta > 0
    assert np.all(delta[nz] <= np.abs(base[nz]) * 0.25 + 2.0 ** -9 * 4)
