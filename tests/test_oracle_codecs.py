"""Pins of the oracle's storage decoders and rounding helpers.

Each check compares against something other than the oracle's own formula:
an independent bit-level formula over every possible input, a library
conversion (torch / numpy), or exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs
import synth


def test_unpack_int4_exhaustive():
    """All 256 bytes: low nibble is element 0, high nibble element 1, two's complement."""
    b = np.arange(256, dtype=np.uint8).reshape(256, 1)
    q = codecs.unpack_int4(b)
    for v in range(256):
        lo, hi = v & 0xF, v >> 4
        assert q[v, 0] == ((lo ^ 8) - 8)
        assert q[v, 1] == ((hi ^ 8) - 8)


def test_pack_unpack_roundtrip_all_pairs():
    vals = np.arange(-8, 8)
    pairs = np.array([[a, b] for a in vals for b in vals], dtype=np.int8)
    packed = codecs.pack_int4(pairs)
    assert packed.shape == (256, 1)
    assert sorted(packed[:, 0].tolist()) == list(range(256))
    assert np.array_equal(codecs.unpack_int4(packed), pairs)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                       # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(codecs.bf16_to_f64(bits), ref)


def test_fp16_decode_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    assert np.array_equal(codecs.fp16_to_f64(bits), ref)


def test_rn_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(2)
    mant = rng.uniform(1.0, 2.0, size=50000)
    expo = rng.integers(-100, 100, size=50000)
    sign = rng.choice([-1.0, 1.0], size=50000)
    v32 = (sign * np.ldexp(mant, expo)).astype(np.float32)
    # constructed ties and near-ties at several binades
    ties = []
    for e in (-20, -1, 0, 3, 40):
        base = np.float32(2.0 ** e)
        for m in range(0, 256, 17):
            lo = np.float32(base * (1 + m / 128))
            ties.append(np.float32(lo + np.float32(base / 256)))       # exact midpoint
            ties.append(np.nextafter(ties[-1], np.float32(np.inf)))
            ties.append(np.nextafter(ties[-2], np.float32(-np.inf)))
    v32 = np.concatenate([v32, np.array(ties, dtype=np.float32), -np.array(ties, dtype=np.float32)])
    ref = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    got = codecs.rn_bf16(v32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_rn_bf16_subnormal_range_matches_torch():
    """Below 2**-126 bf16 has a fixed spacing of 2**-133 (subnormals), like fp32's
    own subnormal range; torch's float32 -> bfloat16 conversion is the reference."""
    rng = np.random.default_rng(6)
    k = rng.integers(1, 2 ** 23, size=20000)
    v32 = (np.ldexp(k.astype(np.float64), -149) * rng.choice([-1.0, 1.0], size=k.size)).astype(np.float32)
    ties = np.array([np.ldexp(2 * j + 1, -134) for j in range(0, 200, 7)], dtype=np.float32)  # midpoints
    near = np.array([np.float32(2.0 ** -126), np.nextafter(np.float32(2.0 ** -126), np.float32(0))],
                    dtype=np.float32)
    v32 = np.concatenate([v32, ties, -ties, near])
    ref = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(codecs.rn_bf16(v32.astype(np.float64)), ref)
    # float64 inputs below fp32's range round to zero or to the smallest step
    assert codecs.rn_bf16(np.array([2.0 ** -140]))[0] == 0.0
    assert codecs.rn_bf16(np.array([0.75 * 2.0 ** -133]))[0] == 2.0 ** -133


def test_rn_bf16_special_cases():
    one = 1.0
    assert codecs.rn_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0             # tie -> even
    assert codecs.rn_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    assert codecs.rn_bf16(np.array([-(one + 3 * 2.0 ** -8)]))[0] == -(one + 2.0 ** -6)
    assert codecs.rn_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == one + 2.0 ** -7
    assert codecs.rn_bf16(np.array([0.0]))[0] == 0.0
    with pytest.raises(ValueError):
        codecs.rn_bf16(np.array([np.nan]))


def test_rn_bf16_f64_inputs_against_rationals():
    """Single rounding from float64 (not via float32): compare with exact rationals."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal(400) * np.exp2(rng.integers(-30, 30, 400))
    got = codecs.rn_bf16(v)
    for x, g in zip(v.tolist(), got.tolist()):
        e = Fraction(x)
        # candidates: multiples of the bf16 spacing around x
        m, ex = np.frexp(abs(x))
        ulp = Fraction(2) ** (int(ex) - 8)
        k = (abs(e) / ulp).__floor__()
        cands = [k * ulp, (k + 1) * ulp]
        best = min(cands, key=lambda c: (abs(c - abs(e)), (c / ulp) % 2))
        assert Fraction(abs(g)) == best and (g >= 0) == (x >= 0)


def test_rn_f32_is_ieee():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(10000) * 1e3
    assert np.array_equal(codecs.rn_f32(v), v.astype(np.float32).astype(np.float64))


def test_dequant_hand_example():
    q = np.array([[1, -2, 3, -8, 7, 0, -1, 2]], dtype=np.int8)
    packed = codecs.pack_int4(q)
    s = np.array([[0.5, 0.25]], dtype=np.float16).view(np.uint16)
    got = codecs.dequant(packed, s, 8)
    assert np.array_equal(got, [[0.5, -1.0, 1.5, -4.0, 1.75, 0.0, -0.25, 0.5]])


def test_dequant_is_exact_product():
    rng = np.random.default_rng(5)
    q = rng.integers(-8, 8, size=(16, 64)).astype(np.int8)
    s = (rng.uniform(1e-4, 1.0, size=(16, 2))).astype(np.float16)
    got = codecs.dequant(codecs.pack_int4(q), s.view(np.uint16), 64)
    for n in range(16):
        for kk in range(64):
            assert Fraction(got[n, kk]) == Fraction(int(q[n, kk])) * Fraction(float(s[n, kk // 32]))


def test_silu_textbook():
    from scipy.special import expit
    v = np.linspace(-30, 30, 2001)
    assert codecs.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(codecs.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)
    assert codecs.silu(np.array([-800.0]))[0] == 0.0


def test_generator_quantiser_bounds_and_packing():
    """The input generator's int4 encoding decodes (with the oracle codec) to values
    within half a step of the drawn weights, with q in [-7, 7] and s = fp16(absmax/7)."""
    g = torch.Generator().manual_seed(7)
    w = torch.randn(37, 256, generator=g) * 0.02
    w[3, :32] = 0.0                                                     # an all-zero group
    packed, sbits = synth.quantize_int4_torch(w, 32)
    q = codecs.unpack_int4(packed.numpy())
    s = codecs.fp16_to_f64(sbits.numpy().view(np.uint16))
    wn = w.double().numpy()
    assert q.min() >= -7 and q.max() <= 7
    absmax = np.abs(wn.reshape(37, 8, 32)).max(-1)
    assert np.array_equal(s, (absmax.astype(np.float32) / np.float32(7)).astype(np.float16).astype(np.float64))
    assert s[3, 0] == 0.0 and np.all(q[3, :32] == 0)
    sr = np.repeat(s, 32, axis=1)
    assert np.all(np.abs(wn - q * sr) <= sr / 2 * (1 + 1e-6) + 1e-12)
