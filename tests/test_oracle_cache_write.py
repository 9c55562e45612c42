"""Pins for the oracle's cache write (quantization of new tokens into the
paged caches, with the rope part rotated).

They tie it to things outside itself: torch's float8_e4m3fn cast of the same
float32 quotients, the complex-multiplication form of a rotation in float64,
exact special angles, the format's bound on rounding error, and the block
table's placement rule.  Planted mistakes (in copies of the oracle's
arithmetic, on the CPU) must fail them.
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _tables(max_pos, seed=0, base=10000.0):
    j = np.arange(32, dtype=np.float64)
    theta = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-j / 32.0)[None, :]
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32), theta


def test_quantize_rows_matches_torch_fp8_cast_of_the_same_quotients():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((40, 576)) * rng.uniform(0.01, 50, (40, 1))).astype(np.float32)
    v[3] = 0.0                       # all-zero row: scale 1, codes 0
    v[4, 7] = -0.0
    codes, scale = O.quantize_rows_f32(v)
    t = torch.from_numpy(v)
    amax = t.abs().amax(1)
    ts = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    ref = (t / ts[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(scale, ts.numpy())
    np.testing.assert_array_equal(codes, ref)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)


def test_quantize_rows_error_bound_and_extreme_code():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 128)).astype(np.float32)
    codes, scale = O.quantize_rows_f32(v)
    dec = O.fp8_e4m3fn_decode(codes) * scale[:, None].astype(np.float64)
    # RNE to E4M3FN: at most half a unit of the 3-bit mantissa (2^-4 relative)
    # in the normal range, 2^-10 of the scale in the subnormal one.
    bound = np.maximum(np.abs(v) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(dec - v) <= bound)
    # the element of largest magnitude lands on +-448
    i = np.abs(v).argmax(1)
    top = codes[np.arange(64), i]
    assert np.all((top == 0x7E) | (top == 0xFE))


def test_rope_matches_complex_rotation_and_special_angles():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    bits = _bf16_bits(x)
    xb = O.bf16_decode(bits)
    cos, sin, theta = _tables(4096)
    pos = rng.integers(0, 4096, 50)
    y = O.rope_interleaved_f32(bits, cos, sin, pos).astype(np.float64)
    z = (xb[:, 0::2] + 1j * xb[:, 1::2]) * (cos[pos].astype(np.float64) + 1j * sin[pos].astype(np.float64))
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=0, atol=4e-7 * np.abs(xb).max())
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=0, atol=4e-7 * np.abs(xb).max())
    # pair norms are kept (up to the tables' and fp32 rounding)
    np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.abs(xb[:, 0::2] + 1j * xb[:, 1::2]),
                               rtol=2e-6, atol=1e-30)
    # exact special angles: 0 keeps the pair, a quarter turn maps (a, b) -> (-b, a)
    one, zero = np.ones((2, 32), np.float32), np.zeros((2, 32), np.float32)
    c = np.stack([one[0], zero[0]]); s = np.stack([zero[0], one[0]])
    y0 = O.rope_interleaved_f32(bits[:2], c, s, np.array([0, 1]))
    np.testing.assert_array_equal(y0[0], xb[0].astype(np.float32))
    np.testing.assert_array_equal(y0[1, 0::2], -xb[1, 1::2].astype(np.float32))
    np.testing.assert_array_equal(y0[1, 1::2], xb[1, 0::2].astype(np.float32))


def _mutant_rope(kind):
    def f(rope_bits, cos, sin, pos):
        x = O.bf16_decode(rope_bits).astype(np.float32)
        c = np.asarray(cos, np.float32)[pos]; s = np.asarray(sin, np.float32)[pos]
        x0, x1 = x[:, 0::2], x[:, 1::2]
        y = np.empty_like(x)
        if kind == "sign":          # rotation the other way
            y[:, 0::2] = x0 * c + x1 * s; y[:, 1::2] = x1 * c - x0 * s
        elif kind == "halves":      # pairs (j, j + 32) instead of (2j, 2j + 1)
            a, b = x[:, :32], x[:, 32:]
            y[:, :32] = a * c - b * s; y[:, 32:] = a * s + b * c
        elif kind == "swap":        # cosine and sine exchanged
            y[:, 0::2] = x0 * s - x1 * c; y[:, 1::2] = x0 * c + x1 * s
        return y
    return f


@pytest.mark.parametrize("kind", ["sign", "halves", "swap"])
def test_rope_pin_catches_planted_mistakes(kind):
    rng = np.random.default_rng(4)
    bits = _bf16_bits(rng.standard_normal((20, 64)))
    xb = O.bf16_decode(bits)
    cos, sin, _ = _tables(512)
    pos = rng.integers(1, 512, 20)
    y = _mutant_rope(kind)(bits, cos, sin, pos).astype(np.float64)
    z = (xb[:, 0::2] + 1j * xb[:, 1::2]) * (cos[pos] + 1j * sin[pos])
    assert not np.allclose(y[:, 0::2], z.real, rtol=0, atol=4e-7 * np.abs(xb).max())


def _pool(rng, n_pages=12, p=16):
    kv = rng.integers(0, 0x7F, (n_pages, p, O.KV_ROW_BYTES_W), dtype=np.uint8)
    kc = rng.integers(0, 0x7F, (n_pages, p, 128), dtype=np.uint8)
    ks = rng.uniform(0.1, 2, (n_pages, p)).astype(np.float32)
    return kv, kc, ks


def test_cache_write_places_rows_by_the_block_table_and_touches_nothing_else():
    rng = np.random.default_rng(5)
    p = 16
    kv, kc, ks = _pool(rng, p=p)
    page_table = np.array([[7, 2, 9, -1], [4, 11, -1, -1]], dtype=np.int32)
    tok_req = np.array([0, 1, 0, 1, 1, 0, 2, 0])
    tok_slot = np.array([5, 17, 40, 0, 40, 70, 3, -1])   # last four: past the span, no page, bad request, bad slot
    n = len(tok_req)
    lat = _bf16_bits(rng.standard_normal((n, 512)) * 3)
    rope = _bf16_bits(rng.standard_normal((n, 64)))
    idx = _bf16_bits(rng.standard_normal((n, 128)))
    cos, sin, _ = _tables(128)
    kv2, kc2, ks2, written = O.cache_write(lat, rope, idx, cos, sin, tok_req, tok_slot, page_table, p, kv, kc, ks)
    assert written.tolist() == [True, True, True, True, False, False, False, False]
    touched = set()
    for i in np.nonzero(written)[0]:
        b, t = tok_req[i], tok_slot[i]
        page, off = page_table[b, t // p], t % p
        touched.add((page, off))
        mla = np.concatenate([O.bf16_decode(lat[i:i + 1]).astype(np.float32),
                              O.rope_interleaved_f32(rope[i:i + 1], cos, sin, [t])], axis=1)
        codes, scale = O.quantize_rows_f32(mla)
        np.testing.assert_array_equal(kv2[page, off, :576], codes[0])
        assert kv2[page, off, 576:580].view(np.float32)[0] == scale[0]
        np.testing.assert_array_equal(kv2[page, off, 580:], kv[page, off, 580:])   # pad kept
        icodes, iscale = O.quantize_rows_f32(O.bf16_decode(idx[i:i + 1]).astype(np.float32))
        np.testing.assert_array_equal(kc2[page, off], icodes[0])
        assert ks2[page, off] == iscale[0]
    for page in range(kv.shape[0]):
        for off in range(p):
            if (page, off) not in touched:
                np.testing.assert_array_equal(kv2[page, off], kv[page, off])
                np.testing.assert_array_equal(kc2[page, off], kc[page, off])
                assert ks2[page, off] == ks[page, off]


def test_written_rows_decode_back_to_the_rotated_inputs():
    """The written MLA row, decoded, is the rotated input within the format's
    rounding bound; without tables the rope part is stored as given."""
    rng = np.random.default_rng(6)
    p = 16
    kv, kc, ks = _pool(rng, p=p)
    page_table = np.arange(12, dtype=np.int32).reshape(1, 12)
    n = 10
    tok_req = np.zeros(n, dtype=np.int64)
    tok_slot = rng.choice(12 * p, n, replace=False)
    lat = _bf16_bits(rng.standard_normal((n, 512)))
    rope = _bf16_bits(rng.standard_normal((n, 64)))
    idx = _bf16_bits(rng.standard_normal((n, 128)))
    for tables in (True, False):
        cos, sin, theta = _tables(12 * p) if tables else (None, None, None)
        kv2, _, _, written = O.cache_write(lat, rope, idx, cos, sin, tok_req, tok_slot, page_table, p, kv, kc, ks)
        assert written.all()
        for i in range(n):
            page, off = tok_slot[i] // p, tok_slot[i] % p
            sc = float(kv2[page, off, 576:580].view(np.float32)[0])
            dec = O.fp8_e4m3fn_decode(kv2[page, off, :576]) * sc
            xr = O.bf16_decode(rope[i])
            if tables:
                z = (xr[0::2] + 1j * xr[1::2]) * np.exp(1j * theta[tok_slot[i]])
                xr = np.empty(64); xr[0::2] = z.real; xr[1::2] = z.imag
            want = np.concatenate([O.bf16_decode(lat[i]), xr])
            bound = np.maximum(np.abs(want) * 2.0 ** -4, sc * 2.0 ** -10) + 1e-6 * np.abs(want).max()
            assert np.all(np.abs(dec - want) <= bound)
