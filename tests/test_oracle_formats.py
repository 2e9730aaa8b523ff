"""Pins for the oracle's number formats: bf16 rounding and MXFP8 (E4M3 + E8M0).

The MXFP8 block format is the one the KOSMOS page describes in its MXFP8
training section (one power-of-two E8M0 scale per 32 consecutive elements,
quantized along the contraction) and that the OLMo-core Appendix A uses in
A.4/A.5.  Element codes are OCP E4M3FN; they are pinned against torch's
float8_e4m3fn cast, a library routine independent of the oracle's encoder.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _all_finite_bf16_values():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bits_to_f64(b)
    return v[np.isfinite(v)]


def test_round_bf16_matches_torch_cast_on_fp32_inputs():
    """torch rounds fp32 -> bf16 once, to nearest even."""
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000),
        rng.standard_normal(1000) * 1e-39,          # bf16 subnormal range
    ]).astype(np.float32)
    # exact midpoints between neighbouring bf16 values (ties to even)
    v = _all_finite_bf16_values()
    v = np.sort(v[(np.abs(v) > 0) & (np.abs(v) < 1e38)])
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), want)


def _exact_nearest_even_bf16(t: float) -> float:
    """Brute force with exact rationals: the two bf16 neighbours of t and the
    nearest, ties to the even significand."""
    from fractions import Fraction
    if t == 0:
        return t
    m, e = math.frexp(abs(t))
    e = max(e, -125)
    q = Fraction(2) ** (e - 8)
    n = Fraction(abs(t)) / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return math.copysign(float(lo * q), t)


def test_round_bf16_single_rounding_from_fp64():
    """fp64 inputs round once (not through fp32).  80.2500030 lies above the
    bf16 midpoint 80.25, so it must go up to 80.5."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        [80.2500030, -80.2500030, 80.25, 80.75, 1e-39, 3e-40]])
    want = np.array([_exact_nearest_even_bf16(float(t)) for t in x])
    assert np.array_equal(O.round_bf16(x), want)
    assert O.round_bf16(np.array([80.2500030]))[0] == 80.5


def test_round_bf16_fixed_points_and_bits():
    v = _all_finite_bf16_values()
    assert np.array_equal(O.round_bf16(v), v)
    assert np.array_equal(O.bits_to_f64(O.bf16_bits(v)), v)


def test_e4m3_encode_matches_torch_over_all_bf16_times_scales():
    """Element path of the quantizer: every finite bf16 value, scaled by the
    powers of two a block scale can apply, against clamp + float8_e4m3fn cast
    (the cast is round-to-nearest-even but does not saturate, hence the clamp)."""
    v = _all_finite_bf16_values()
    for sh in (-130, -20, -9, -8, -1, 0, 1, 8, 20, 127):
        y = np.ldexp(v, -sh)
        y = y[np.isfinite(y)]
        want = torch.from_numpy(np.clip(y, -448.0, 448.0)).to(torch.float8_e4m3fn) \
            .view(torch.uint8).numpy()
        got = O.e4m3_encode(y)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (sh, y[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("val,code", [
    (1.0, 0x38), (448.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E), (-448.0, 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -11, 0x01), (-0.0, 0x80),
    (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -6, 0x08), (7 * 2.0 ** -9, 0x07),
    (0.0155, 0x08), (240.0, 0x77), (256.0, 0x78)])
def test_e4m3_hand_values(val, code):
    # closed forms from the E4M3FN definition: bias 7, 3 mantissa bits,
    # subnormal step 2^-9, largest finite 1.75 * 2^8 = 448
    assert int(O.e4m3_encode(np.array([val]))[0]) == code


def test_e4m3_decode_encode_roundtrip_all_codes():
    codes = np.arange(256)
    vals = O.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(O.e4m3_encode(vals[ok]), codes[ok].astype(np.uint8))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and ok.sum() == 254
    # against torch's decoder
    tv = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(tv[ok], vals[ok])


def test_floor_log2_from_bits():
    rng = np.random.default_rng(2)
    a = np.concatenate([np.abs(rng.standard_normal(50000)) * 10.0 ** rng.integers(-37, 37, 50000),
                        np.abs(rng.standard_normal(2000)) * 1e-40, [2.0 ** -149, 1.0, 2.0, 3.999]])
    a = a.astype(np.float32)
    a = a[a > 0]
    want = np.array([math.frexp(float(t))[1] - 1 for t in a])
    assert np.array_equal(O.floor_log2_f32(a), want)


def test_quantize_block_rules():
    # amax 448 -> e = 0 (code 127) and 448 encodes as 0x7E
    blk = np.zeros(32)
    blk[3] = 448.0
    q, s = O.quantize_mxfp8(blk[None])
    assert s[0, 0] == 127 and q[0, 3] == 0x7E and np.all(np.delete(q[0], 3) == 0)
    # an all-zero block: code 0, elements keep their sign
    z = np.zeros(32)
    z[5] = -0.0
    q, s = O.quantize_mxfp8(z[None])
    assert s[0, 0] == 0 and q[0, 5] == 0x80 and q[0, 0] == 0
    # single 1.0: floor(log2 1) - 8 = -8 -> code 119, 1.0 * 2^8 = 256 -> 0x78
    one = np.zeros(32)
    one[0] = 1.0
    q, s = O.quantize_mxfp8(one[None])
    assert s[0, 0] == 119 and q[0, 0] == 0x78


def test_quantize_random_blocks_bounds():
    rng = np.random.default_rng(3)
    x = O.round_bf16(rng.standard_normal((64, 256)) * 10.0 ** rng.integers(-20, 20, (64, 1)))
    q, s = O.quantize_mxfp8(x)
    deq = O.dequantize_mxfp8(q, s)
    blk = x.reshape(64, 8, 32)
    amax = np.abs(blk).max(-1)
    e = s.astype(np.int64) - 127
    scaled = amax * np.ldexp(1.0, -e)
    assert np.all((scaled >= 256) & (scaled < 512))          # the floor rule
    # per element: error at most half a step of the value's own binade
    err = np.abs(deq - x).reshape(64, 8, 32)
    step = np.ldexp(1.0, np.maximum(np.frexp(np.abs(blk) * np.ldexp(1.0, -e)[..., None])[1] - 1, -6) - 3) \
        * np.ldexp(1.0, e)[..., None]
    sat = np.abs(blk) * np.ldexp(1.0, -e)[..., None] > 448
    assert np.all((err <= step / 2) | sat)


def test_eq87_with_unit_scales_is_the_plain_gemm():
    """eq. 87 (OLMo-core Appendix A, A.5) with every scale 2^0: the block-scaled
    product of E4M3-representable values equals the plain product."""
    rng = np.random.default_rng(4)
    codes_ok = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    def mat(m, k):
        v = O.e4m3_decode(rng.choice(codes_ok, size=(m, k)))
        v.reshape(m, k // 32, 32)[:, :, 0] = 256.0      # every block amax in [256,512)
        return v
    a, b = mat(16, 128), mat(8, 128)
    aq, as_ = O.quantize_mxfp8(a)
    bq, bs = O.quantize_mxfp8(b)
    assert np.all(as_ == 127) and np.all(bs == 127)
    assert np.array_equal(O.dequantize_mxfp8(aq, as_), a)
    assert np.array_equal(O.mxfp8_gemm(aq, as_, bq, bs), O.round_bf16(a @ b.T))


def test_mxfp8_gemm_vs_torch_dequant_matmul():
    rng = np.random.default_rng(5)
    a = O.round_bf16(rng.standard_normal((8, 64)))
    b = O.round_bf16(rng.standard_normal((4, 64)) * 0.01)
    aq, as_ = O.quantize_mxfp8(a)
    bq, bs = O.quantize_mxfp8(b)
    # independent dequantization through torch's float8 decoder
    def tdeq(q, s):
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64)
        sc = torch.pow(2.0, torch.from_numpy(s.astype(np.int64) - 127).to(torch.float64))
        return (v.reshape(q.shape[0], -1, 32) * sc[..., None]).reshape(q.shape)
    assert np.array_equal(O.dequantize_mxfp8(aq, as_), tdeq(aq, as_).numpy())
    ref = (tdeq(aq, as_) @ tdeq(bq, bs).T).numpy()
    # rounding to bf16 is pinned on its own above; torch's fp64->bf16 cast
    # rounds through fp32, so it is not used here
    assert np.allclose(O.mxfp8_gemm(aq, as_, bq, bs), ref, rtol=2.0 ** -8, atol=0)
