"""Pins of the oracle's grouped GEMM, epilogue and combine.

* brute force  -> pure-Python loops over tokens, experts and k with exact
                  rational arithmetic (fractions.Fraction) on tiny inputs,
                  for fp8 W8A8, int8 W8A16 and MXFP8; the oracle must equal
                  the exact result rounded to float32 (or bf16 for MXFP8).
* E=1, top_k=1 -> reduces to one dense product of the decoded operands times
                  the scales (no routing, no gather).
* exact integers -> small-integer bf16 activations, int8 weights, unit scales
                  and one expert give exact integer outputs.
* permutation  -> permuting the tokens permutes the per-slot results.
* combine      -> special cases with a known float32 sum.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as O


def _bf16(a):
    return F.bf16_round(np.asarray(a, np.float32))


def _fr(v):
    return Fraction(float(v))


def _tiny(rng, M, K, N, E):
    x = _bf16(rng.standard_normal((M, K)))
    w = (rng.standard_normal((E, N, K)) / np.sqrt(K)).astype(np.float32)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    return x, w, lg


def _exact_routed(decode_a, decode_w, scale, ids, wts, M, K, N, top_k):
    y = np.zeros((M * top_k, N), np.float32)
    for t in range(M):
        for j in range(top_k):
            e = int(ids[t, j])
            for n in range(N):
                acc = sum((decode_a(t, k) * decode_w(e, n, k) for k in range(K)), Fraction(0))
                y[t * top_k + j, n] = np.float32(float(acc * scale(e, n) * _fr(wts[t, j])))
    return y


def test_fp8_brute_force():
    rng = np.random.default_rng(10)
    M, K, N, E, top_k = 3, 32, 4, 4, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    ids, wts = O.route_topk(lg, top_k)
    aq, sa = O.quantize_act_fp8(x)
    wq, sw = O.quantize_weight_fp8(w)
    dec = {int(c): _fr(v) for c, v in zip(range(256), F.e4m3_decode(np.arange(256, dtype=np.uint8))) if np.isfinite(v)}
    ref = _exact_routed(lambda t, k: dec[int(aq[t, k])], lambda e, n, k: dec[int(wq[e, n, k])],
                        lambda e, n: _fr(sa) * _fr(sw[e]), ids, wts, M, K, N, top_k)
    got = O.grouped_gemm_fp8w8a8(aq, sa, wq, sw, ids, wts)
    np.testing.assert_array_equal(got, ref)


def test_int8_brute_force():
    rng = np.random.default_rng(11)
    M, K, N, E, top_k = 3, 32, 5, 4, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    ids, wts = O.route_topk(lg, top_k)
    wq, sw = O.quantize_weight_int8(w)
    xv = F.bf16_decode(x)
    ref = _exact_routed(lambda t, k: _fr(xv[t, k]), lambda e, n, k: Fraction(int(wq[e, n, k])),
                        lambda e, n: _fr(sw[e, n]), ids, wts, M, K, N, top_k)
    got = O.grouped_gemm_int8w8a16(x, wq, sw, ids, wts)
    np.testing.assert_array_equal(got, ref)


def test_mxfp8_brute_force():
    rng = np.random.default_rng(12)
    seg, K, N = (3, 0, 2), 64, 3
    R, E = sum(seg), len(seg)
    x = _bf16(rng.standard_normal((R, K)) * rng.uniform(0.1, 10, size=(R, 1)))
    w = rng.standard_normal((E, N, K)).astype(np.float32)
    mo = np.concatenate([[0], np.cumsum(seg)])
    aq, asf = O.quantize_act_mxfp8(x, mo)
    wq, wsf = O.quantize_weight_mxfp8(w)
    po = O.mx_padded_offsets(mo)
    dec = {c: _fr(v) for c, v in zip(range(256), F.e4m3_decode(np.arange(256, dtype=np.uint8))) if np.isfinite(v)}
    got = O.grouped_gemm_mxfp8(aq, asf, wq, wsf, mo)
    for e in range(E):
        for r in range(mo[e], mo[e + 1]):
            srow = asf[po[e] + r - mo[e]]
            for n in range(N):
                acc = Fraction(0)
                for kb in range(K // 32):
                    blk = sum((dec[int(aq[r, k])] * dec[int(wq[e, n, k])] for k in range(32 * kb, 32 * kb + 32)), Fraction(0))
                    acc += blk * Fraction(2) ** (int(srow[kb]) + int(wsf[e, n, kb]) - 254)
                ref = F.bf16_round(np.array([np.float32(float(acc))]))[0]
                assert got[r, n] == ref, (e, r, n)


def test_single_expert_reduces_to_dense_gemm():
    rng = np.random.default_rng(13)
    M, K, N = 20, 256, 48
    x, w, lg = _tiny(rng, M, K, N, 1)
    ids, wts = O.route_topk(lg, 1)
    assert np.all(wts == 1.0)
    aq, sa = O.quantize_act_fp8(x)
    wq, sw = O.quantize_weight_fp8(w)
    dense = (F.e4m3_decode(aq) @ F.e4m3_decode(wq[0]).T) * (float(sa) * float(sw[0]))
    np.testing.assert_array_equal(O.grouped_gemm_fp8w8a8(aq, sa, wq, sw, ids, wts), dense.astype(np.float32))
    wq8, sw8 = O.quantize_weight_int8(w)
    dense8 = (F.bf16_decode(x) @ wq8[0].astype(np.float64).T) * sw8[0][None, :].astype(np.float64)
    np.testing.assert_array_equal(O.grouped_gemm_int8w8a16(x, wq8, sw8, ids, wts), dense8.astype(np.float32))


def test_exact_integer_case():
    rng = np.random.default_rng(14)
    M, K, N = 6, 64, 8
    xi = rng.integers(-8, 9, size=(M, K))
    x = _bf16(xi)
    wq = rng.integers(-127, 128, size=(1, N, K)).astype(np.int8)
    ids = np.zeros((M, 1), np.int32)
    wts = np.ones((M, 1), np.float32)
    got = O.grouped_gemm_int8w8a16(x, wq, np.ones((1, N), np.float32), ids, wts)
    np.testing.assert_array_equal(got, (xi @ wq[0].astype(np.int64).T).astype(np.float32))


def test_token_permutation_equivariance():
    rng = np.random.default_rng(15)
    M, K, N, E, top_k = 24, 128, 16, 8, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    perm = rng.permutation(M)
    wq, sw = O.quantize_weight_fp8(w)
    aq, sa = O.quantize_act_fp8(x)
    ids, wts = O.route_topk(lg, top_k)
    y = O.grouped_gemm_fp8w8a8(aq, sa, wq, sw, ids, wts).reshape(M, top_k, N)
    aq2, sa2 = O.quantize_act_fp8(x[perm])
    ids2, wts2 = O.route_topk(lg[perm], top_k)
    y2 = O.grouped_gemm_fp8w8a8(aq2, sa2, wq, sw, ids2, wts2).reshape(M, top_k, N)
    np.testing.assert_array_equal(y2, y[perm])


def test_sampled_equals_full():
    rng = np.random.default_rng(16)
    M, K, N, E, top_k = 10, 128, 40, 4, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    ids, wts = O.route_topk(lg, top_k)
    wq, sw = O.quantize_weight_int8(w)
    full = O.grouped_gemm_int8w8a16(x, wq, sw, ids, wts)
    slots, cols = np.array([0, 7, 19, 3]), np.array([39, 0, 5])
    np.testing.assert_array_equal(O.grouped_gemm_int8w8a16(x, wq, sw, ids, wts, slots, cols),
                                  full[np.ix_(slots, cols)])


def test_combine_special_cases():
    rng = np.random.default_rng(17)
    y0 = rng.standard_normal((5, 8)).astype(np.float32)
    y = np.stack([y0, np.zeros_like(y0)], 1).reshape(10, 8)
    out32, out = O.combine(y, 2)
    np.testing.assert_array_equal(out32, y0)
    np.testing.assert_array_equal(out, F.bf16_round(y0))
    y = np.stack([y0, -y0], 1).reshape(10, 8)
    out32, _ = O.combine(y, 2)
    assert np.all(out32 == 0)
    # 1 + 2^-24 + 2^-24 in slot order: each add rounds back to 1 in float32
    y = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]], np.float32)
    out32, _ = O.combine(y, 3)
    assert out32[0, 0] == np.float32(1.0)
    y = np.array([[2.0 ** -24], [2.0 ** -24], [1.0]], np.float32)
    out32, _ = O.combine(y, 3)
    assert out32[0, 0] == np.float32(1.0) + np.float32(2.0 ** -23)


def test_slot_results_bf16_match_torch_rounding():
    """The per-slot bf16 storage step equals torch's float32 -> bfloat16
    conversion (round to nearest even), including ties, binade edges,
    subnormals and signed zero."""
    import torch
    rng = np.random.default_rng(23)
    y = rng.standard_normal((16, 64)).astype(np.float32) * np.float32(3.0)
    special = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.99999, 65504.0,
                        1e-40, -0.0, 2.0 ** -126, 3.0e38], np.float32)
    y.reshape(-1)[:special.size] = special
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.slot_results_bf16(y), ref)


# ------------------------------------------------- int8 W8A8 (dynamic) ----
def test_int8w8a8_brute_force():
    """Exact rational arithmetic on a tiny routed case: the integer dot
    product times the token scale, the channel scale and the router weight,
    rounded once to float32."""
    rng = np.random.default_rng(13)
    M, K, N, E, top_k = 3, 32, 5, 4, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    ids, wts = O.route_topk(lg, top_k)
    aq, sa = O.quantize_act_int8_rows(x)
    wq, sw = O.quantize_weight_int8(w)
    y = np.zeros((M * top_k, N), np.float32)
    for t in range(M):
        for j in range(top_k):
            e = int(ids[t, j])
            for n in range(N):
                dot = sum(int(aq[t, k]) * int(wq[e, n, k]) for k in range(K))
                y[t * top_k + j, n] = np.float32(float(Fraction(dot) * _fr(sa[t]) * _fr(sw[e, n])
                                                       * _fr(wts[t, j])))
    np.testing.assert_array_equal(O.grouped_gemm_int8w8a8(aq, sa, wq, sw, ids, wts), y)


def test_int8w8a8_integer_identity():
    """Unit scales and router weight 1: the result is the plain integer
    product of the codes (exact in float32 below 2^24)."""
    rng = np.random.default_rng(14)
    M, K, N = 5, 64, 7
    aq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (1, N, K)).astype(np.int8)
    ids = np.zeros((M, 1), np.int32)
    y = O.grouped_gemm_int8w8a8(aq, np.ones(M, np.float32), wq, np.ones((1, N), np.float32),
                                ids, np.ones((M, 1), np.float32))
    np.testing.assert_array_equal(y, (aq.astype(np.int64) @ wq[0].astype(np.int64).T).astype(np.float32))


def test_fp8w8a16_brute_force():
    """fp8 weight-only by exact rational arithmetic on a tiny routed case."""
    rng = np.random.default_rng(15)
    M, K, N, E, top_k = 3, 32, 5, 4, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    ids, wts = O.route_topk(lg, top_k)
    wq, sw = O.quantize_weight_fp8_rows(w)
    xv = F.bf16_decode(x)
    dec = {int(c): _fr(v) for c, v in zip(range(256), F.e4m3_decode(np.arange(256, dtype=np.uint8))) if np.isfinite(v)}
    ref = _exact_routed(lambda t, k: _fr(xv[t, k]), lambda e, n, k: dec[int(wq[e, n, k])],
                        lambda e, n: _fr(sw[e, n]), ids, wts, M, K, N, top_k)
    np.testing.assert_array_equal(O.grouped_gemm_fp8w8a16(x, wq, sw, ids, wts), ref)


def test_int4w16_brute_force():
    """int4 weight-only by exact rational arithmetic on a tiny routed case:
    bf16 activations times the integer codes, the channel scale and the
    router weight, rounded once to float32."""
    rng = np.random.default_rng(16)
    M, K, N, E, top_k = 3, 32, 5, 4, 2
    x, w, lg = _tiny(rng, M, K, N, E)
    ids, wts = O.route_topk(lg, top_k)
    wq, sw = O.quantize_weight_int4(w)
    assert wq.min() >= -7 and wq.max() <= 7
    xv = F.bf16_decode(x)
    ref = _exact_routed(lambda t, k: _fr(xv[t, k]), lambda e, n, k: Fraction(int(wq[e, n, k])),
                        lambda e, n: _fr(sw[e, n]), ids, wts, M, K, N, top_k)
    np.testing.assert_array_equal(O.grouped_gemm_int4w16(x, wq, sw, ids, wts), ref)


def test_int4w16_integer_identity():
    """Small-integer activations, unit scales, one expert and router weight 1:
    the plain integer product of the codes."""
    rng = np.random.default_rng(17)
    M, K, N = 4, 64, 6
    xi = rng.integers(-20, 21, (M, K))
    x = _bf16(xi.astype(np.float32))
    wq = rng.integers(-7, 8, (1, N, K)).astype(np.int8)
    ids = np.zeros((M, 1), np.int32)
    y = O.grouped_gemm_int4w16(x, wq, np.ones((1, N), np.float32), ids, np.ones((M, 1), np.float32))
    np.testing.assert_array_equal(y, (xi @ wq[0].astype(np.int64).T).astype(np.float32))


# ------------------------------------------------- MXFP8 gradients -----
def _int_rows(rng, R, C):
    """Small integers: every 32-block quantizes to MXFP8 without loss (|v| <= 7
    has at most three significant bits, scaled by a power of two)."""
    return rng.integers(-7, 8, (R, C)).astype(np.float32)


@pytest.mark.parametrize("seg", [(40, 0, 100), (128, 128), (1,)])
def test_mxfp8_dgrad_wgrad_closed_form(seg):
    """On losslessly quantized integers the gradients are the plain products:
    dx = dy W_e per row of expert e, dW_e = dy_e^T x_e, rounded to bf16."""
    rng = np.random.default_rng(41)
    E, N, K = len(seg), 128, 64
    R = sum(seg)
    mo = np.concatenate([[0], np.cumsum(seg)])
    x = _bf16(_int_rows(rng, R, K))
    dy = _bf16(_int_rows(rng, R, N))
    w = rng.integers(-7, 8, (E, N, K)).astype(np.float32)
    dy_q, dy_sf = O.quantize_act_mxfp8(dy, mo)
    wT_q, wT_sf = O.quantize_weight_mxfp8_colwise(w)
    dx = O.grouped_linear_dgrad_mxfp8(dy_q, dy_sf, wT_q, wT_sf, mo)
    dyv, xv = F.bf16_decode(dy).astype(np.float64), F.bf16_decode(x).astype(np.float64)
    ref = np.zeros((R, K))
    for e in range(E):
        ref[mo[e]:mo[e + 1]] = dyv[mo[e]:mo[e + 1]] @ w[e].astype(np.float64)
    np.testing.assert_array_equal(dx, F.bf16_round(ref.astype(np.float32)))
    dyT_q, dyT_sf = O.quantize_act_mxfp8_colwise(dy, mo)
    xT_q, xT_sf = O.quantize_act_mxfp8_colwise(x, mo)
    dw = O.grouped_linear_wgrad_mxfp8(dyT_q, dyT_sf, xT_q, xT_sf, mo, N, K)
    refw = np.stack([dyv[mo[e]:mo[e + 1]].T @ xv[mo[e]:mo[e + 1]] for e in range(E)])
    np.testing.assert_array_equal(dw, F.bf16_round(refw.astype(np.float32)))


def test_mxfp8_wgrad_brute_force():
    """Weight gradient by exact rational arithmetic on decoded codes: the sum
    over an expert's rows of 2^(b-127) e4m3 products, rounded once to float32."""
    rng = np.random.default_rng(42)
    seg = [45, 3]
    N, K = 4, 3
    R = sum(seg)
    mo = np.concatenate([[0], np.cumsum(seg)])
    dy = _bf16(rng.standard_normal((R, N)) * 2)
    x = _bf16(rng.standard_normal((R, K)))
    dyT_q, dyT_sf = O.quantize_act_mxfp8_colwise(dy, mo)
    xT_q, xT_sf = O.quantize_act_mxfp8_colwise(x, mo)
    got = O.grouped_linear_wgrad_mxfp8(dyT_q, dyT_sf, xT_q, xT_sf, mo, N, K, as_float32=True)
    dec = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    po = O.mx_colwise_offsets(mo)
    for e in range(len(seg)):
        rp = int(po[e + 1] - po[e])
        for n in range(N):
            for k in range(K):
                acc = Fraction(0)
                for j in range(rp):
                    qa = int(dyT_q[N * po[e] + n * rp + j])
                    qb = int(xT_q[K * po[e] + k * rp + j])
                    ba = int(dyT_sf[N * po[e] // 32 + n * (rp // 32) + j // 32])
                    bb = int(xT_sf[K * po[e] // 32 + k * (rp // 32) + j // 32])
                    acc += _fr(dec[qa]) * _fr(dec[qb]) * Fraction(2) ** (ba + bb - 254)
                assert got[e, n, k] == np.float32(float(acc))
