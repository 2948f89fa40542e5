"""Pins of the oracle's fused activations ("[PyTorch] Let GroupedLinear accept
MXFP8 input and gradient", Description: SwiGLU / SReLU + MXFP8 quantization).

* SReLU: closed form (negatives -> 0, positives -> square) and exactness of
  the float32 result for bf16 inputs;
* SwiGLU: against scipy's logistic function (an independent routine), the
  identity silu(g) - silu(-g) = g, silu(0) = 0 and its limits;
* quantized forms: the MXFP8 and fp8 quantizers applied to the activation,
  and the concatenated-tensor quantization equal to the per-expert one with
  padded scale blocks (the page's statement for the fused act + quantize).
"""

import numpy as np
import pytest
from scipy.special import expit

from oracle import formats as F
from oracle import moe as O


def _bf16(rng, shape, scale=1.0):
    return F.bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def test_srelu_closed_form_and_exact():
    rng = np.random.default_rng(5)
    xb = _bf16(rng, (64, 96), 3.0)
    x = F.bf16_decode(xb)
    y = O.act_values(xb, O.ACT_SRELU)
    assert np.all(y[x <= 0] == 0)
    np.testing.assert_array_equal(y[x > 0], x[x > 0] ** 2)
    # the square of a bf16 value (8-bit significand) is exact in float32
    np.testing.assert_array_equal(y.astype(np.float32).astype(np.float64), y)


def test_swiglu_against_logistic_and_identities():
    rng = np.random.default_rng(6)
    xb = _bf16(rng, (32, 2 * 64), 4.0)
    x = F.bf16_decode(xb)
    g, u = x[:, :64], x[:, 64:]
    y = O.act_values(xb, O.ACT_SWIGLU)
    np.testing.assert_allclose(y, g * expit(g) * u, rtol=1e-13, atol=1e-300)
    # silu(g) - silu(-g) = g (sigmoid(g) + sigmoid(-g) = 1)
    gg = np.linspace(-20, 20, 401)
    row = np.concatenate([gg, np.ones_like(gg)])[None, :]
    rown = np.concatenate([-gg, np.ones_like(gg)])[None, :]
    np.testing.assert_allclose(O.swiglu(row) - O.swiglu(rown), gg[None, :], rtol=1e-12, atol=1e-12)
    assert O.swiglu(np.array([[0.0, 5.0]]))[0, 0] == 0.0
    big = O.swiglu(np.array([[60.0, -800.0, -2.0, 3.0]]))
    assert big[0, 0] == pytest.approx(-120.0, rel=1e-15)     # silu(60) = 60 in double: 60 * -2
    assert abs(big[0, 1]) < 1e-300                             # silu(-800) underflows to -0


@pytest.mark.parametrize("act", [O.ACT_SWIGLU, O.ACT_SRELU])
def test_act_quantizers_compose(act):
    rng = np.random.default_rng(7 + act)
    H = 64
    xb = _bf16(rng, (40, 2 * H if act == O.ACT_SWIGLU else H))
    y32 = O.act_values(xb, act).astype(np.float32)
    mo = np.array([0, 5, 5, 40])
    q, sf = O.act_quantize_mxfp8(xb, mo, act)
    q_ref, b_ref = O.quantize_mxfp8_rows(y32)
    np.testing.assert_array_equal(q, q_ref)
    po = O.mx_padded_offsets(mo)
    assert sf.shape == (int(po[-1]), H // 32)
    for e in range(3):
        n = mo[e + 1] - mo[e]
        np.testing.assert_array_equal(sf[po[e]:po[e] + n], b_ref[mo[e]:mo[e + 1]])
        assert np.all(sf[po[e] + n:po[e + 1]] == 0)
        # quantizing each expert's rows alone gives the same data and scales
        if n:
            qe, be = O.quantize_mxfp8_rows(y32[mo[e]:mo[e + 1]])
            np.testing.assert_array_equal(q[mo[e]:mo[e + 1]], qe)
            np.testing.assert_array_equal(sf[po[e]:po[e] + n], be)
    qf, s = O.act_quantize_fp8(xb, act)
    assert s == np.float32(np.max(np.abs(y32)) / np.float32(448.0))
    np.testing.assert_array_equal(qf, O.fp8_quantize_with_scale(y32, s))
