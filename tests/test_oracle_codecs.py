"""Pins of the oracle's storage codecs against independent library routines.

bf16 and fp16 decoding are checked on all 65536 codes (torch bfloat16, numpy
float16); E4M3 decoding on all 256 codes (torch float8_e4m3fn, an implementation
of the OCP 8-bit floating point E4M3 format).  The encoder is checked
  - exhaustively over equivalence classes of fp32 inputs: the rounding of x to
    E4M3 depends only on its sign, exponent, top mantissa bits and whether the
    rest is zero, exactly half or otherwise, so one representative of every
    class is compared with torch (which rounds to nearest, ties to even);
  - on a random sample of 2^22 fp32 bit patterns;
  - on hand-listed ties, subnormals, zero signs, saturation and NaN, where torch
    differs by design (it maps overflow to NaN; the reading here saturates).
int8 decoding is checked on all 256 codes (numpy int8) and the symmetric int8
encoder against numpy's rint (round half to even) and clip on ties, saturation,
NaN and random values.
"""
import numpy as np
import torch

import oracle


def test_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode(codes, "bf16")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_f16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = oracle.decode(codes, "f16")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode(codes, "fp8")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2  # S.1111.111 only
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.decode(codes, "fp8").astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_encode_equivalence_classes_vs_torch():
    reps = []
    for sign in (0, 1):
        for exp in range(0, 255):
            for top in range(32):  # mantissa bits 22..18: three kept bits, guard, one more
                for rest in (0, 1, 0x1FFFF, 0x20000, 0x20001, 0x3FFFF, 0x12345):
                    m = (top << 18) | (rest & 0x3FFFF)
                    reps.append((sign << 31) | (exp << 23) | m)
    bits = np.array(reps, np.uint32)
    x = bits.view(np.float32)
    inr = np.abs(x.astype(np.float64)) <= 464.0  # torch keeps these finite (464 ties to 448)
    got = oracle.e4m3_encode(x[inr])
    ref = _torch_e4m3(x[inr])
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[inr][i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_random_bit_patterns_vs_torch():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    with np.errstate(invalid="ignore"):
        inr = np.abs(x.astype(np.float64)) <= 464.0  # NaN compares False
    assert np.array_equal(oracle.e4m3_encode(x[inr]), _torch_e4m3(x[inr]))


def test_e4m3_encode_hand_cases():
    f = lambda v: int(oracle.e4m3_encode(np.array([v], np.float32))[0])
    assert f(0.0) == 0x00 and f(-0.0) == 0x80
    assert f(2.0 ** -9) == 0x01  # smallest subnormal
    assert f(2.0 ** -10) == 0x00  # tie between 0 and 2^-9: even code 0
    assert f(-(2.0 ** -10)) == 0x80
    assert f(3 * 2.0 ** -10) == 0x02  # tie between codes 1 and 2: even
    assert f(1.0) == 0x38 and f(1.0625) == 0x38 and f(1.1875) == 0x3A  # ties to even
    assert f(0.9375 + 2.0 ** -5) == 0x38  # tie across a binade boundary goes up to 1.0
    assert f(448.0) == 0x7E and f(449.0) == 0x7E and f(480.0) == 0x7E and f(1e30) == 0x7E
    assert f(float("inf")) == 0x7E and f(float("-inf")) == 0xFE and f(-1000.0) == 0xFE
    assert f(float("nan")) == 0x7F
    assert f(-float("nan")) == 0xFF


def test_int8_decode_all_codes():
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    assert np.array_equal(oracle.decode(codes, "int8"), codes.astype(np.float64))


def test_int8_encode_vs_numpy():
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 60,
        np.arange(-130.5, 131, 0.5, dtype=np.float32),            # every tie near the range
        np.array([0.0, -0.0, 126.49, 126.5, 127.5, -127.5, -128.0, 1e9, -1e9, np.inf,
                  -np.inf], np.float32)])
    want = np.clip(np.rint(x.astype(np.float64)), -127, 127).astype(np.int8)
    assert np.array_equal(oracle.int8_encode(x), want)
    assert oracle.int8_encode(np.array([np.nan], np.float32))[0] == 0
    assert list(oracle.int8_encode(np.array([0.5, 1.5, 2.5, -0.5, -2.5], np.float32))) == \
        [0, 2, 2, 0, -2]


def test_int8_encode_by_integer_arithmetic():
    """Every quarter step in [-140, 140] (exact in fp32): the nearest integer with
    ties to even, clamped to [-127, 127], computed with integers only (floor division
    and the remainder of 4 k by 4), so the pin shares no rounding routine with the
    encoder ([P1] §8.1: int8 codes with an fp32 scale; symmetric, no zero point)."""
    ks = np.arange(-560, 561, dtype=np.int64)          # x = k / 4
    x = (ks / 4).astype(np.float32)
    want = []
    for k in ks.tolist():
        q, r = divmod(k, 4)                             # k = 4 q + r, 0 <= r < 4
        if r > 2 or (r == 2 and q % 2 == 1):
            q += 1
        want.append(max(-127, min(127, q)))
    assert np.array_equal(oracle.int8_encode(x).astype(np.int64), np.array(want))


def test_int8_encode_vs_python_round():
    """Python's round() on a float is exact and breaks ties to even: an independent
    routine for random values across the clamp."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 80).astype(np.float32)
    want = [max(-127, min(127, round(float(v)))) for v in x]
    assert np.array_equal(oracle.int8_encode(x).astype(np.int64), np.array(want))
