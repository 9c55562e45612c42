"""Pins for the oracle's number formats and the indexer-query quantization.

Each check ties the oracle to something outside itself: torch's own
float8_e4m3fn / bfloat16 conversions (library routines), closed-form values
of the OCP E4M3FN format, and exact properties of the power-of-two scale.
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def _torch_fp8_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_decode_matches_torch_on_every_finite_code():
    ref = _torch_fp8_values()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    got = O.fp8_e4m3fn_decode(codes)
    np.testing.assert_array_equal(got, ref[codes])
    # torch itself agrees the two excluded codes are NaN.
    assert np.isnan(ref[0x7F]) and np.isnan(ref[0xFF])


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6),
                                        (0x01, 2.0 ** -9), (0x38, 1.0), (0x00, 0.0),
                                        (0x07, 7 * 2.0 ** -9), (0x40, 2.0), (0x3C, 1.5)])
def test_fp8_decode_closed_forms(code, value):
    assert O.fp8_e4m3fn_decode(np.array([code], dtype=np.uint8))[0] == value


def test_fp8_nan_codes_rejected():
    for c in (0x7F, 0xFF):
        with pytest.raises(ValueError):
            O.fp8_e4m3fn_decode(np.array([1, c], dtype=np.uint8))


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(4096, generator=g) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_decode(bits), x.to(torch.float64).numpy())


def test_fp8_encode_rne_matches_torch_cast():
    g = torch.Generator().manual_seed(2)
    x = torch.cat([torch.randn(20000, generator=g) * 60, torch.randn(5000, generator=g) * 0.01])
    x = x.clamp(-448, 448).to(torch.float64)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.fp8_e4m3fn_encode_rne(x.numpy())
    # The sign of a value that rounds to zero may differ only in -0 vs +0 codes.
    np.testing.assert_array_equal(got, ref)


def test_fp8_encode_ties_go_to_even_mantissa():
    grid = O.fp8_e4m3fn_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2.0
    got = O.fp8_e4m3fn_encode_rne(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(got, expect.astype(np.uint8))
    # Exact grid points are fixed points; negatives mirror with the sign bit.
    np.testing.assert_array_equal(O.fp8_e4m3fn_encode_rne(grid), np.arange(127, dtype=np.uint8))
    np.testing.assert_array_equal(O.fp8_e4m3fn_encode_rne(-grid[1:]),
                                  (np.arange(1, 127) | 0x80).astype(np.uint8))
    # Half the smallest subnormal ties to zero; just above rounds up.
    assert O.fp8_e4m3fn_encode_rne(np.array([2.0 ** -10]))[0] == 0
    assert O.fp8_e4m3fn_encode_rne(np.array([2.0 ** -10 * 1.01]))[0] == 1


def _bf16_bits(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_quantize_q_against_torch_cast_and_scale_bounds():
    g = torch.Generator().manual_seed(3)
    q = torch.randn(5, 64, 128, generator=g) * torch.exp(torch.randn(5, 64, 1, generator=g) * 3)
    bits = _bf16_bits(q)
    codes, scale = O.quantize_q(bits)
    qf = O.bf16_decode(bits)
    amax = np.abs(qf).max(-1)
    # power of two, and the tightest one that keeps amax/scale <= 448
    m, e = np.frexp(scale)
    assert np.all(m == 0.5)
    assert np.all(amax / scale <= 448.0) and np.all(amax / scale > 224.0)
    ref = torch.from_numpy(qf / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)


def test_quantize_q_special_cases():
    q = np.zeros((1, 3, 128), dtype=np.float32)
    q[0, 1, 5] = 448.0          # amax exactly 448 -> scale 1, code 0x7E
    q[0, 2, 7] = -3.0           # amax 3 -> scale 2^-7 (3/2^-7 = 384 <= 448 < 768)
    codes, scale = O.quantize_q(_bf16_bits(q))
    assert scale[0, 0] == 1.0 and np.all(codes[0, 0] == 0)
    assert scale[0, 1] == 1.0 and codes[0, 1, 5] == 0x7E
    assert scale[0, 2] == 2.0 ** -7
    assert O.fp8_e4m3fn_decode(codes[0, 2, 7:8])[0] * scale[0, 2] == -3.0
