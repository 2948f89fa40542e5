"""Pins of the oracle's quantizers.

* fp8 per tensor -> exact power-of-two scaling invariance, the amax element
                    landing on +-448, the scale equal to amax/448, the
                    round-trip of values that already sit on the scaled grid.
* int8 per channel -> brute force per element with Python's round-half-even
                    on exact fractions, the amax element on +-127, symmetry.
* MXFP8          -> the statement of "[PyTorch] Let GroupedLinear accept MXFP8
                    input and gradient" that quantizing the concatenated tensor
                    and quantizing each expert separately give the same data
                    (scales differ only by the per-expert padding to 128 rows),
                    its [64, 128] -> rowwise [128, 4] shape example, the
                    shared-exponent rule checked with math.frexp, and exact
                    power-of-two invariance.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return F.bf16_round(np.asarray(a, np.float32))


# ------------------------------------------------------------- fp8 ----
def test_fp8_per_tensor_scale_and_amax_code():
    rng = np.random.default_rng(0)
    x = _bf16(rng.standard_normal((33, 64)))
    q, s = O.quantize_act_fp8(x)
    xv = F.bf16_decode(x)
    amax = np.max(np.abs(xv))
    assert s == np.float32(amax / 448.0)          # one correctly rounded division
    i = np.unravel_index(np.argmax(np.abs(xv)), xv.shape)
    assert q[i] & 0x7F == 0x7E                    # the amax element maps to +-448
    assert np.all((q & 0x7F) <= 0x7E)             # never NaN
    # dequantized values are within half an e4m3 step (relative 2^-4) of x
    deq = F.e4m3_decode(q) * float(s)
    big = np.abs(xv) > 2.0 ** -6 * float(s)
    assert np.all(np.abs(deq - xv)[big] <= np.abs(xv)[big] * 2.0 ** -4 * (1 + 1e-6))


@pytest.mark.parametrize("p", [-7, -1, 3, 11])
def test_fp8_per_tensor_power_of_two_invariance(p):
    rng = np.random.default_rng(1)
    xf = rng.standard_normal((16, 32)).astype(np.float32)
    x = _bf16(xf)
    x2 = _bf16(F.bf16_decode(x) * 2.0 ** p)       # exact: a power-of-two scaling
    q1, s1 = O.quantize_act_fp8(x)
    q2, s2 = O.quantize_act_fp8(x2)
    np.testing.assert_array_equal(q1, q2)
    assert float(s2) == float(s1) * 2.0 ** p


def test_fp8_per_tensor_grid_values_round_trip():
    # x = code_value * s with s = 1 (amax = 448): quantization returns the codes
    codes = np.array([0x7E, 0x01, 0x30, 0x45, 0xB9, 0x80, 0x5A], np.uint8)
    x = _bf16(F.e4m3_decode(codes))
    q, s = O.quantize_act_fp8(x[None, :])
    assert s == 1.0
    np.testing.assert_array_equal(q[0], codes)


def test_fp8_zero_tensor():
    q, s = O.quantize_act_fp8(np.zeros((4, 16), np.uint16))
    assert s == 1.0 and np.all(q == 0)


def test_fp8_weight_scale_per_expert():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((3, 8, 32)) * np.array([1, 10, 0.01])[:, None, None]).astype(np.float32)
    q, s = O.quantize_weight_fp8(w)
    for e in range(3):
        assert s[e] == np.float32(np.max(np.abs(w[e])) / np.float32(448))
        assert np.max(q[e] & 0x7F) == 0x7E


# ------------------------------------------------------------- int8 ----
def _round_half_even(fr):
    f = math.floor(fr)
    d = fr - f
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def test_int8_per_channel_brute_force():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((2, 5, 24)) / 4).astype(np.float32)
    w[1, 3] = 0.0                                  # an all-zero channel
    q, s = O.quantize_weight_int8(w)
    for e in range(2):
        for n in range(5):
            row = w[e, n]
            amax = float(np.max(np.abs(row)))
            s_ref = np.float32(1.0) if amax == 0 else np.float32(Fraction(amax) / 127)
            assert s[e, n] == s_ref
            inv = np.float32(Fraction(1) / Fraction(float(s_ref)))
            for k in range(24):
                prod = np.float32(Fraction(float(row[k])) * Fraction(float(inv)))
                ref = max(-127, min(127, _round_half_even(Fraction(float(prod)))))
                assert int(q[e, n, k]) == ref
            if amax:
                assert int(np.max(np.abs(q[e, n].astype(int)))) == 127


def test_int8_symmetry():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((1, 4, 64)).astype(np.float32)
    q1, s1 = O.quantize_weight_int8(w)
    q2, s2 = O.quantize_weight_int8(-w)
    np.testing.assert_array_equal(q1, -q2)
    np.testing.assert_array_equal(s1, s2)


# ------------------------------------------------------------- MXFP8 ----
def test_mxfp8_page_example_shapes():
    g = json.load(open(os.path.join(GOLDEN, "mxfp8_padding_example.json")))
    rng = np.random.default_rng(5)
    E, m, K = g["experts"], g["rows_per_expert"], g["K"]
    x = _bf16(rng.standard_normal((E * m, K)))
    mo = np.arange(E + 1) * m
    q, sf = O.quantize_act_mxfp8(x, mo)
    assert list(q.shape) == g["concat_data_shape"]
    # per expert: data [64,128] and rowwise scales [128, 4]
    for e in range(E):
        qe, sfe = O.quantize_act_mxfp8(x[e * m:(e + 1) * m], [0, m])
        assert list(qe.shape) == g["per_expert_data_shape"]
        assert list(sfe.shape) == g["per_expert_rowwise_scale_shape"]
    # split + pad of the whole-tensor scales: every expert gets a 128-row block
    assert sf.shape == (E * g["per_expert_rowwise_scale_shape"][0], K // 32)


@pytest.mark.parametrize("seg", [(64, 64), (5, 130, 0, 77), (128,), (1, 1, 1)])
def test_mxfp8_whole_equals_per_expert(seg):
    """Quantizing the concatenated tensor, then splitting it, equals quantizing
    each expert's chunk on its own: identical data, identical scales once each
    expert's scale block is padded to 128 rows."""
    rng = np.random.default_rng(sum(seg))
    K = 96
    R = sum(seg)
    x = _bf16(rng.standard_normal((R, K)) * rng.uniform(0.01, 100, size=(R, 1)))
    mo = np.concatenate([[0], np.cumsum(seg)])
    q, sf = O.quantize_act_mxfp8(x, mo)
    po = O.mx_padded_offsets(mo)
    for e, n in enumerate(seg):
        qe, sfe = O.quantize_act_mxfp8(x[mo[e]:mo[e + 1]], [0, n])
        np.testing.assert_array_equal(q[mo[e]:mo[e + 1]], qe)
        np.testing.assert_array_equal(sf[po[e]:po[e + 1]], sfe)
        assert sfe.shape[0] == -(-n // 128) * 128
        assert np.all(sfe[n:] == 0)


def test_mxfp8_shared_exponent_rule():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((40, 64)) * np.exp(rng.uniform(-20, 20, size=(40, 1)))).astype(np.float32)
    q, b = O.quantize_mxfp8_rows(v)
    blk = v.reshape(40, 2, 32)
    for r in range(40):
        for j in range(2):
            amax = float(np.max(np.abs(blk[r, j])))
            _, ex = math.frexp(amax)                # amax = f * 2^ex, f in [0.5, 1)
            assert int(b[r, j]) == (ex - 1) - 8 + 127
            codes = q[r, 32 * j:32 * j + 32]
            # the block maximum lands in the top binade [256, 448] (codes 0x78..0x7E)
            assert 0x78 <= int(np.max(codes & 0x7F)) <= 0x7E
            # in scaled units y = x / 2^(b-127): unsaturated elements are within
            # half a step (relative 2^-4, absolute 2^-10 among subnormals);
            # elements beyond 448 are clamped to +-448
            y = blk[r, j].astype(np.float64) * 2.0 ** (127 - int(b[r, j]))
            deq = F.e4m3_decode(codes)
            sat = np.abs(y) > 448
            assert np.all(deq[sat] == np.sign(y[sat]) * 448)
            ok = np.abs(deq - y)[~sat] <= np.maximum(np.abs(y[~sat]) * 2.0 ** -4, 2.0 ** -10)
            assert np.all(ok)


@pytest.mark.parametrize("p", [-5, 4])
def test_mxfp8_power_of_two_invariance(p):
    rng = np.random.default_rng(7)
    v = rng.standard_normal((8, 64)).astype(np.float32)
    q1, b1 = O.quantize_mxfp8_rows(v)
    q2, b2 = O.quantize_mxfp8_rows((v * np.float32(2.0 ** p)).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(b2.astype(int), b1.astype(int) + p)


def test_mxfp8_zero_block_and_weights_layout():
    v = np.zeros((2, 64), np.float32)
    v[1, 40] = 3.0
    q, b = O.quantize_mxfp8_rows(v)
    assert b.tolist() == [[0, 0], [0, 128 - 8]]     # 3.0 has exponent field 128
    assert np.all(q[0] == 0) and np.all(q[1, :32] == 0)
    w = np.random.default_rng(8).standard_normal((2, 3, 64)).astype(np.float32)
    wq, wsf = O.quantize_weight_mxfp8(w)
    assert wq.shape == (2, 3, 64) and wsf.shape == (2, 3, 2)
    q2, b2 = O.quantize_mxfp8_rows(w[1])
    np.testing.assert_array_equal(wq[1], q2)
    np.testing.assert_array_equal(wsf[1], b2)


def test_int8_activation_rows_brute_force():
    """Per-token int8 of bf16 rows by exact arithmetic: the scale, every
    code, +-127 at the row's amax, a zero row."""
    rng = np.random.default_rng(5)
    x = F.bf16_round((rng.standard_normal((4, 40)) * np.array([[1.0], [1e-3], [50.0], [0.0]])).astype(np.float32))
    q, s = O.quantize_act_int8_rows(x)
    xv = F.bf16_decode(x)
    for t in range(4):
        amax = float(np.max(np.abs(xv[t])))
        s_ref = np.float32(1.0) if amax == 0 else np.float32(Fraction(amax) / 127)
        assert s[t] == s_ref
        inv = np.float32(Fraction(1) / Fraction(float(s_ref)))
        for k in range(40):
            prod = np.float32(Fraction(float(xv[t, k])) * Fraction(float(inv)))
            assert int(q[t, k]) == max(-127, min(127, _round_half_even(Fraction(float(prod)))))
        if amax:
            assert int(np.max(np.abs(q[t].astype(int)))) == 127
        else:
            assert not q[t].any()
    # the error bound of a round-to-nearest code: |q s - x| <= s / 2 (plus the
    # rounding of the product), and symmetry
    assert np.all(np.abs(q.astype(np.float64) * s[:, None] - xv) <= s[:, None] * (0.5 + 1e-6))
    q2, s2 = O.quantize_act_int8_rows(F.bf16_round(-xv.astype(np.float32)))
    np.testing.assert_array_equal(q2, -q)
    np.testing.assert_array_equal(s2, s)


def test_fp8_weight_rows_equal_per_tensor_rule_per_row():
    """Per-channel fp8 weights are the per-tensor rule applied to every row:
    the same codes and scales as the per-expert (per-tensor) quantizer run
    with one row per expert; a zero row gets scale 1 and zero codes, and each
    row's largest magnitude maps to +-448."""
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((2, 5, 48)) * np.array([1.0, 1e-3])[:, None, None]).astype(np.float32)
    w[1, 2] = 0.0
    q, s = O.quantize_weight_fp8_rows(w)
    q_t, s_t = O.quantize_weight_fp8(w.reshape(10, 1, 48))
    np.testing.assert_array_equal(q.reshape(10, 1, 48), q_t)
    np.testing.assert_array_equal(s.reshape(10), s_t)
    assert s[1, 2] == 1.0 and not q[1, 2].any()
    for e in range(2):
        for n in range(5):
            if (e, n) != (1, 2):
                k = int(np.argmax(np.abs(w[e, n])))
                assert abs(float(F.e4m3_decode(q[e, n, k]))) == 448.0


# ------------------------------------------------------------- int4 -----
def test_int4_per_channel_brute_force():
    """int4 weight-only codes and scales by exact rational arithmetic: the
    scale is amax/7 rounded once to float32, every code the float32 product
    w * fl32(1/s) rounded half to even and clamped to -7..7; each nonzero row
    reaches |q| = 7 at its largest element."""
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((2, 6, 40)) / 5).astype(np.float32)
    w[0, 2] = 0.0                                  # an all-zero channel
    w[1, 4, :8] = [0.5, -0.5, 1.5, 2.5, -3.5, 3.5, 0.25, 0.0]   # half-way codes at s = 0.5
    w[1, 4, 8:] = 0.0
    q, s = O.quantize_weight_int4(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    for e in range(2):
        for n in range(6):
            row = w[e, n]
            amax = float(np.max(np.abs(row)))
            s_ref = np.float32(1.0) if amax == 0 else np.float32(Fraction(amax) / 7)
            assert s[e, n] == s_ref
            inv = np.float32(Fraction(1) / Fraction(float(s_ref)))
            for k in range(40):
                prod = np.float32(Fraction(float(row[k])) * Fraction(float(inv)))
                ref = max(-7, min(7, _round_half_even(Fraction(float(prod)))))
                assert int(q[e, n, k]) == ref
            if amax:
                assert int(np.max(np.abs(q[e, n].astype(int)))) == 7
            else:
                assert not q[e, n].any()
    # the hand-made row: amax 3.5 -> s = 0.5, codes of w / 0.5 half to even
    assert s[1, 4] == np.float32(0.5)
    np.testing.assert_array_equal(q[1, 4, :8], [1, -1, 3, 5, -7, 7, 0, 0])


def test_int4_symmetry_and_error_bound():
    rng = np.random.default_rng(22)
    w = rng.standard_normal((2, 3, 64)).astype(np.float32)
    q1, s1 = O.quantize_weight_int4(w)
    q2, s2 = O.quantize_weight_int4(-w)
    np.testing.assert_array_equal(q1, -q2)
    np.testing.assert_array_equal(s1, s2)
    # every code is within half a step of w / s (no clamping below amax)
    err = np.abs(w.astype(np.float64) - q1 * s1[..., None].astype(np.float64))
    assert np.all(err <= 0.5 * s1[..., None] * (1 + 1e-6))


# ------------------------------------------------------ MXFP8 colwise ----
def test_mxfp8_colwise_page_shapes():
    """The worked example of the MXFP8 page: two [64, 128] experts have
    columnwise scales [4, 128] each (two 32-row blocks padded to four); the
    whole [128, 128] tensor has [4, 128], whose blocks are those of the
    experts (64 rows are whole blocks), and the codes agree."""
    g = json.load(open(os.path.join(GOLDEN, "mxfp8_padding_example.json")))
    rng = np.random.default_rng(31)
    E, m, K = g["experts"], g["rows_per_expert"], g["K"]
    x = _bf16(rng.standard_normal((E * m, K)))
    mo = np.arange(E + 1) * m
    qT, sfT = O.quantize_act_mxfp8_colwise(x, mo)
    rp = 128                                        # each expert padded to 128 rows
    assert qT.size == K * E * rp and sfT.size == K * E * rp // 32
    whole_q, whole_sf = O.quantize_act_mxfp8_colwise(x, [0, E * m])
    whole_sf = whole_sf.reshape(K, E * m // 32)
    assert list(whole_sf.T.shape) == g["concat_colwise_scale_shape"]
    whole_q = whole_q.reshape(K, E * m)
    for e in range(E):
        sfe = sfT[K * rp // 32 * e: K * rp // 32 * (e + 1)].reshape(K, rp // 32)
        assert list(sfe.T.shape) == g["per_expert_colwise_scale_shape"]
        np.testing.assert_array_equal(sfe[:, : m // 32], whole_sf[:, e * m // 32: (e + 1) * m // 32])
        assert not sfe[:, m // 32:].any()           # blocks of padding rows: scale byte 0
        qe = qT[K * rp * e: K * rp * (e + 1)].reshape(K, rp)
        np.testing.assert_array_equal(qe[:, :m], whole_q[:, e * m: (e + 1) * m])
        assert not qe[:, m:].any()


def test_mxfp8_colwise_is_rowwise_of_transpose():
    """One expert whose rows fill whole 128-row blocks: the columnwise codes
    and scales are the rowwise activation quantization of the transposed
    tensor (its single 128-multiple block needs no padding)."""
    rng = np.random.default_rng(32)
    R, C = 256, 96
    x = _bf16(rng.standard_normal((R, C)) * 3)
    qT, sfT = O.quantize_act_mxfp8_colwise(x, [0, R])
    qr, sfr = O.quantize_act_mxfp8(np.ascontiguousarray(x.T), [0, C])
    np.testing.assert_array_equal(qT.reshape(C, R), qr)
    np.testing.assert_array_equal(sfT.reshape(C, R // 32), sfr[:C])


def test_mxfp8_colwise_ragged_blocks():
    """Ragged experts: every scale byte is clamp(floor(log2 amax) + 127 - 8,
    0, 254) over the 32 rows of its block that belong to the expert (0 when
    they are all padding), and every code decodes to the value (saturated at
    448 times the block scale) within half an e4m3 step."""
    rng = np.random.default_rng(33)
    seg = [37, 0, 70, 5]
    C = 40
    x = (rng.standard_normal((sum(seg), C)) * np.exp(rng.standard_normal((sum(seg), 1)))).astype(np.float32)
    mo = np.concatenate([[0], np.cumsum(seg)])
    qT, sfT = O.quantize_mxfp8_colwise(x, mo)
    po = O.mx_colwise_offsets(mo)
    dec = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    for e in range(len(seg)):
        rp = int(po[e + 1] - po[e])
        qe = qT[C * po[e]: C * po[e + 1]].reshape(C, rp)
        be = sfT[C * po[e] // 32: C * po[e + 1] // 32].reshape(C, rp // 32)
        for c in range(C):
            for blk in range(rp // 32):
                r0 = mo[e] + 32 * blk
                vals = x[r0: min(r0 + 32, mo[e + 1]), c] if r0 < mo[e + 1] else np.zeros(0, np.float32)
                amax = float(np.max(np.abs(vals))) if vals.size else 0.0
                want = 0 if amax == 0 else max(0, min(254, math.frexp(amax)[1] - 1 + 127 - 8))
                assert int(be[c, blk]) == want
                codes = qe[c, 32 * blk: 32 * blk + 32]
                got = dec[codes].astype(np.float64) * 2.0 ** (int(be[c, blk]) - 127)
                ref = np.zeros(32)
                ref[: vals.size] = vals
                # the OCP rule lets amax * 2^(127-b) reach up to 512: values past
                # e4m3's 448 saturate
                top = 448.0 * 2.0 ** (int(be[c, blk]) - 127)
                ref = np.sign(ref) * np.minimum(np.abs(ref), top)
                step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))) - 3)
                step = np.maximum(step, 2.0 ** (int(be[c, blk]) - 127 - 9))   # e4m3 subnormal step
                assert np.all(np.abs(got - ref) <= 0.5 * step + 1e-300)
