"""Number formats used by the quantized MoE GEMM, decoded and encoded exactly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formats and the readings taken where the pages only name them:

* e4m3 - the pages say "fp8" / "e4m3" ("Tianxing/moe quantization",
  FP8_W8A8 Benchmark; "[PyTorch] Let GroupedLinear accept MXFP8 input and
  gradient", Description).  Reading: the OCP E4M3FN encoding - 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, no infinities, the single NaN
  pattern S.1111.111 per sign, largest finite value 448.  Encoding rounds to
  nearest with ties to even mantissa and saturates to +-448 (finite inputs
  never produce NaN).  Subnormals m * 2^-9 are kept.
* e8m0 - the MXFP8 shared scale: one unsigned byte b meaning 2^(b - 127);
  0xFF is NaN.
* bf16 - the top 16 bits of an IEEE float32; float32 -> bf16 rounds to nearest,
  ties to even.
* int8 - two's-complement signed byte, symmetric range [-127, 127] when
  produced by the quantizer.
"""

import numpy as np

E4M3_MAX = 448.0          # largest finite e4m3 value: 1.75 * 2^8
E4M3_MIN_NORMAL_EXP = -6  # exponent of the smallest normal value 2^-6
E4M3_SUB_QUANTUM = 2.0 ** -9  # spacing of the subnormals


# ----------------------------------------------------------------------------
# e4m3
# ----------------------------------------------------------------------------
def e4m3_decode(codes):
    """Exact value of each e4m3 byte as float64 (NaN for 0x7F / 0xFF).

    Normal codes (exponent field 1..15): (-1)^s * 2^(e-7) * (1 + m/8).
    Subnormal codes (exponent field 0): (-1)^s * 2^-6 * (m/8).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x):
    """Round each value to the nearest e4m3 code (ties to even), saturating.

    ``x`` is taken at its exact value (any float dtype; float32 inputs are
    widened exactly).  The grid spacing around |x| is 2^(floor(log2|x|) - 3)
    for normal magnitudes and 2^-9 below 2^-6; |x| / spacing is rounded half to
    even, which makes the mantissa LSB even on ties.  Magnitudes above 448
    (including infinity) give +-448.  NaN gives the NaN code with its sign.
    """
    v = np.asarray(x).astype(np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    isnan = np.isnan(a)
    a = np.where(isnan, 0.0, a)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    exp_unb = np.maximum(ex - 1, E4M3_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, exp_unb - 3)
    with np.errstate(over="ignore", invalid="ignore"):
        n = np.rint(a / quantum)              # exact division; half to even
        r = np.minimum(n * quantum, E4M3_MAX)
    r = np.where(np.isnan(r), E4M3_MAX, r)    # inf / inf guard
    # bits of the rounded magnitude r (an exact e4m3 value)
    _, rex = np.frexp(r)
    is_sub = r < 2.0 ** E4M3_MIN_NORMAL_EXP
    e_field = np.where(is_sub, 0, rex - 1 + 7)
    m_field = np.where(is_sub,
                       r / E4M3_SUB_QUANTUM,
                       np.ldexp(r, -(rex - 1) + 3) - 8)
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = np.where(isnan, 0x7F, code)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------
# e8m0
# ----------------------------------------------------------------------------
def e8m0_decode(b):
    """2^(b - 127) as float64; 0xFF is NaN."""
    bi = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(bi == 0xFF, np.nan, np.ldexp(1.0, bi - 127))


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------
def bf16_decode(bits):
    """Exact float64 value of each bf16 bit pattern (uint16)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(x32):
    """float32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN.

    The upper 16 bits are kept; the lower 16 bits decide: above half an ulp
    rounds up, below rounds down, exactly half rounds to the even upper half.
    """
    u = np.ascontiguousarray(np.asarray(x32, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    upper = u >> 16
    lower = u & 0xFFFF
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    r = upper + round_up.astype(np.uint64)
    f = np.asarray(x32, dtype=np.float32)
    r = np.where(np.isnan(f), (upper | 0x40), r)   # keep NaN a (quiet) NaN
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------
# float32 helpers (the precision in which the method takes its decisions)
# ----------------------------------------------------------------------------
def f32_exponent_field(x32):
    """Biased 8-bit exponent field of each float32 value."""
    u = np.ascontiguousarray(np.asarray(x32, dtype=np.float32)).view(np.uint32)
    return ((u >> 23) & 0xFF).astype(np.int64)
