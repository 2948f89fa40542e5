"""Reference computation of the quantized MoE grouped GEMM, step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The problem is stated by the column heads of the benchmark tables on
"Tianxing/moe quantization" (FP8_W8A8 Benchmark, INT8_W8A16 Benchmark):
M tokens with K input features, E experts with N output features each, and
every token routed to top_k experts.  The computation follows the per-expert
decomposition of "Enabling MOE Quantization using linear decomposition"
(Summary): for each expert, gather the tokens routed to it and apply that
expert's quantized linear op to them; then weight each result by its router
weight and sum the top_k results of each token.

Flat slot numbering: the j-th expert choice of token t is slot i = t*top_k + j.
Per-slot results ``y`` have shape [M*top_k, N] in that order.

Readings taken where the pages are silent:

* routing selects the top_k experts by float32 logit, larger first, the lower
  expert index first on equal logits; router weights are the softmax over all
  E logits restricted to the chosen experts and renormalised to sum to one
  (the full softmax denominator cancels);
* block alignment keeps, inside each expert, the slots in ascending slot
  order; each expert's count is padded up to a multiple of block_m with the
  sentinel M*top_k; the block list names the expert of every block and -1
  after the last one;
* fp8 per-tensor scales are s = fl32(amax / 448), applied as
  fl32(x * fl32(1 / s)) before rounding to e4m3; an all-zero tensor has s = 1;
* int8 per-channel weights use s = fl32(amax_row / 127) and
  clamp(round_half_even(fl32(w * fl32(1 / s))), -127, 127);
* int4 weight-only weights take the same rule with 7 in place of 127 (codes
  -7..7, one scale per output channel);
* MXFP8 takes the OCP MX rule for the shared exponent of each block of 32
  values along K: 2^(floor(log2 amax) - 8), written as the e8m0 byte
  clamp(exponent_field(amax) - 8, 0, 254), with the elements x / 2^(b-127)
  rounded to e4m3 with saturation;
* the contraction itself is done in float64 (at these sizes it is exact or
  within a few float64 ulp), the epilogue multiplies by the scales and the
  router weight in float64 and rounds once to float32;
* the combine adds a token's top_k float32 results in slot order in float32
  and rounds the sum to bf16 (nearest, ties to even).
"""

import numpy as np

from .formats import (bf16_decode, bf16_round, e4m3_decode, e4m3_encode,
                      e8m0_decode, f32_exponent_field)

MX_BLOCK = 32        # values per shared e8m0 scale, along K
MX_ROW_PAD = 128     # each expert's rowwise scale block is padded to 128 rows
E4M3_EMAX = 8        # exponent of the largest e4m3 binade (448 = 1.75 * 2^8)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# routing (top-k) and block alignment
# ----------------------------------------------------------------------------
def route_topk(logits, top_k):
    """Top-k expert choice and renormalised router weights for each token.

    logits: float32 [M, E].  Returns (topk_ids int32 [M, top_k],
    topk_weights float32 [M, top_k]).  The choice is made on the float32
    logits (larger first, lower index first on ties), so it does not depend
    on how exp is evaluated.  Weights: p_e = exp(l_e - max_l) (float64); the
    chosen p's divided by their own sum, rounded to float32.
    """
    lg = _f32(logits)
    M, E = lg.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    idx = np.broadcast_to(np.arange(E), (M, E))
    order = np.lexsort((idx, -lg), axis=-1)          # primary: -logit; then index
    ids = order[:, :top_k].astype(np.int32)
    l64 = lg.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    pk = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = pk / pk.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


def align_max_padded(M, E, top_k, block_m):
    """Length of the sorted-slot buffer: M*top_k + E*(block_m-1), rounded up
    to a multiple of block_m (an upper bound on the padded length)."""
    n = M * top_k + E * (block_m - 1)
    return (n + block_m - 1) // block_m * block_m


def align_block_size(topk_ids, E, block_m):
    """Group the slots by expert and pad every group to a multiple of block_m.

    Returns (sorted_token_ids int32 [max_padded], expert_ids int32
    [max_padded // block_m], num_tokens_post_padded int).  Padding slots and
    the unused tail hold the sentinel M*top_k; blocks past the padded length
    hold expert -1.
    """
    ids = np.asarray(topk_ids)
    M, top_k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    sentinel = M * top_k
    max_padded = align_max_padded(M, E, top_k, block_m)
    sorted_ids = np.full(max_padded, sentinel, dtype=np.int32)
    expert_ids = np.full(max_padded // block_m, -1, dtype=np.int32)
    off = 0
    for e in range(E):
        members = np.nonzero(flat == e)[0]           # ascending slot order
        cnt = len(members)
        padded = (cnt + block_m - 1) // block_m * block_m
        sorted_ids[off:off + cnt] = members
        expert_ids[off // block_m:(off + padded) // block_m] = e
        off += padded
    return sorted_ids, expert_ids, off


# ----------------------------------------------------------------------------
# quantization
# ----------------------------------------------------------------------------
def fp8_tensor_scale(values):
    """Per-tensor e4m3 scale s = fl32(amax / 448); 1 for an all-zero tensor."""
    amax = np.float32(np.max(np.abs(_f32(values)))) if np.size(values) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(448.0))


def fp8_quantize_with_scale(values, s):
    """e4m3 codes of fl32(x * fl32(1 / s))."""
    inv = np.float32(np.float32(1.0) / np.float32(s))
    return e4m3_encode(_f32(values) * inv)


def quantize_act_fp8(x_bf16):
    """Dynamic per-tensor fp8 quantization of bf16 activations [M, K].

    Returns (a_q uint8 [M, K], a_scale float32)."""
    x = bf16_decode(x_bf16).astype(np.float32)
    s = fp8_tensor_scale(x)
    return fp8_quantize_with_scale(x, s), s


def quantize_weight_fp8(w):
    """Per-expert per-tensor fp8 weights: w float32 [E, N, K] ->
    (w_q uint8 [E, N, K], w_scale float32 [E])."""
    w = _f32(w)
    scales = np.array([fp8_tensor_scale(w[e]) for e in range(w.shape[0])], dtype=np.float32)
    q = np.stack([fp8_quantize_with_scale(w[e], scales[e]) for e in range(w.shape[0])])
    return q, scales


def quantize_weight_fp8_rows(w):
    """fp8 weight-only weights ("fp8wo" of "Enabling MOE Quantization using
    linear decomposition", Summary): one e4m3 scale per expert and output
    channel, the per-tensor rule applied to each row: s = fl32(amax_row /
    448) (1 for a zero row), q = e4m3(fl32(w * fl32(1 / s))).  w float32
    [E, N, K] -> (w_q uint8 [E, N, K], w_scale float32 [E, N])."""
    w = _f32(w)
    amax = np.max(np.abs(w), axis=-1)
    s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(448.0)).astype(np.float32))
    s = s.astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    return e4m3_encode(w * inv[..., None]), s


def int8_channel_scale(w_rows):
    """Per-row symmetric int8 scale fl32(amax_row / 127); 1 for a zero row."""
    amax = np.max(np.abs(_f32(w_rows)), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_weight_int8(w):
    """Per-output-channel symmetric int8 weights: w float32 [E, N, K] ->
    (w_q int8 [E, N, K], w_scale float32 [E, N])."""
    w = _f32(w)
    s = int8_channel_scale(w)
    inv = (np.float32(1.0) / s).astype(np.float32)
    q = np.rint(w * inv[..., None])                  # float32 product, half to even
    return np.clip(q, -127, 127).astype(np.int8), s


def quantize_weight_int4(w):
    """int4 weight-only weights ("int4wo" of "Enabling MOE Quantization using
    linear decomposition", Summary; the page gives no granularity): the int8
    per-output-channel rule with 7 in place of 127, s = fl32(amax_row / 7)
    (1 for a zero row), q = clamp(round_half_even(fl32(w * fl32(1 / s))),
    -7, 7).  w float32 [E, N, K] -> (w_q int8 [E, N, K] holding the codes,
    w_scale float32 [E, N])."""
    w = _f32(w)
    amax = np.max(np.abs(w), axis=-1)
    s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(7.0)).astype(np.float32))
    s = s.astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    q = np.rint(w * inv[..., None])                  # float32 product, half to even
    return np.clip(q, -7, 7).astype(np.int8), s


def quantize_act_int8_rows(x_bf16):
    """Dynamic per-token (per-row) symmetric int8 quantization of bf16
    activations [M, K] ("Enabling MOE Quantization using linear
    decomposition", Summary: the int8 dynamic-activation family, "int8dq"):
    the rule of the int8 weights applied to each activation row,
    s_t = fl32(amax_t / 127) (1 for a zero row),
    q = clamp(round_half_even(fl32(x * fl32(1 / s_t))), -127, 127).
    Returns (q int8 [M, K], s float32 [M])."""
    x = bf16_decode(x_bf16).astype(np.float32)
    s = int8_channel_scale(x)
    inv = (np.float32(1.0) / s).astype(np.float32)
    q = np.rint(x * inv[..., None])                  # float32 product, half to even
    return np.clip(q, -127, 127).astype(np.int8), s


def mx_scale_byte(amax32):
    """e8m0 byte of the shared scale 2^(floor(log2 amax) - 8) of each block:
    clamp(exponent_field(amax) - 8, 0, 254); an all-zero block gives 0."""
    return np.clip(f32_exponent_field(amax32) - E4M3_EMAX, 0, 254).astype(np.uint8)


def quantize_mxfp8_rows(values):
    """MXFP8 along the last axis: values float32 [R, K] (K % 32 == 0) ->
    (q uint8 [R, K], scale bytes uint8 [R, K/32]).

    Each element of a block is x * 2^(127 - b) (exact: a power-of-two scale)
    rounded to e4m3 with saturation."""
    v = _f32(values)
    R, K = v.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32 for MXFP8")
    blk = v.reshape(R, K // MX_BLOCK, MX_BLOCK)
    b = mx_scale_byte(np.max(np.abs(blk), axis=-1))
    scaled = blk.astype(np.float64) * np.ldexp(1.0, 127 - b.astype(np.int64))[..., None]
    return e4m3_encode(scaled).reshape(R, K), b


def mx_padded_offsets(m_offsets):
    """Start row of each expert's scale block when every block is padded to a
    multiple of 128 rows ("[PyTorch] Let GroupedLinear accept MXFP8 input and
    gradient", reply on the padding: each expert's rowwise scales are padded to
    128 rows).  Returns int64 [E+1]."""
    m = np.diff(np.asarray(m_offsets, dtype=np.int64))
    padded = (m + MX_ROW_PAD - 1) // MX_ROW_PAD * MX_ROW_PAD
    return np.concatenate([[0], np.cumsum(padded)])


def quantize_act_mxfp8(x_bf16, m_offsets):
    """MXFP8 quantization of expert-concatenated bf16 activations.

    x_bf16 uint16 [R, K]; m_offsets int [E+1] (rows of expert e are
    m_offsets[e] .. m_offsets[e+1]-1).  Returns (q uint8 [R, K],
    sf uint8 [sum_e roundup(m_e, 128), K/32]) where expert e's scale rows start
    at the padded offset and the pad rows are zero."""
    x = bf16_decode(x_bf16).astype(np.float32)
    q, b = quantize_mxfp8_rows(x)
    mo = np.asarray(m_offsets, dtype=np.int64)
    po = mx_padded_offsets(mo)
    sf = np.zeros((int(po[-1]), x.shape[1] // MX_BLOCK), dtype=np.uint8)
    for e in range(len(mo) - 1):
        n = mo[e + 1] - mo[e]
        sf[po[e]:po[e] + n] = b[mo[e]:mo[e + 1]]
    return q, sf


# ----------------------------------------------------------------------------
# fused activation + quantization (the step between the up and the down
# projection: "[PyTorch] Let GroupedLinear accept MXFP8 input and gradient",
# Description, SwiGLU / SReLU + MXFP8 quantization)
# ----------------------------------------------------------------------------
ACT_SWIGLU, ACT_SRELU = 0, 1


def swiglu(x):
    """SwiGLU of rows [R, 2H] in float64: silu(g) * u with the gate g the first
    half of the row, u the second, silu(g) = g / (1 + exp(-g))."""
    v = np.asarray(x, dtype=np.float64)
    h = v.shape[1] // 2
    g, u = v[:, :h], v[:, h:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def srelu(x):
    """Squared ReLU in float64: max(x, 0)^2."""
    r = np.maximum(np.asarray(x, dtype=np.float64), 0.0)
    return r * r


def act_values(x_bf16, act):
    """The activation of bf16 rows (uint16 bits) in float64."""
    x = bf16_decode(x_bf16)
    return swiglu(x) if act == ACT_SWIGLU else srelu(x)


def act_quantize_mxfp8(x_bf16, m_offsets, act):
    """Activation of expert-concatenated bf16 rows, rounded once to float32,
    then MXFP8 with per-expert padded scale blocks (as quantize_act_mxfp8).
    Exact for SReLU of bf16 inputs (the square of a bf16 value fits float32);
    for SwiGLU the float32 value of exp differs between implementations, so a
    comparison allows the codes of nearby values (act_code_bounds)."""
    y = act_values(x_bf16, act).astype(np.float32)
    q, b = quantize_mxfp8_rows(y)
    mo = np.asarray(m_offsets, dtype=np.int64)
    po = mx_padded_offsets(mo)
    sf = np.zeros((int(po[-1]), y.shape[1] // MX_BLOCK), dtype=np.uint8)
    for e in range(len(mo) - 1):
        n = mo[e + 1] - mo[e]
        sf[po[e]:po[e] + n] = b[mo[e]:mo[e + 1]]
    return q, sf


def act_quantize_fp8(x_bf16, act):
    """Activation rounded once to float32, then per-tensor fp8 (as
    quantize_act_fp8).  Returns (q uint8 [R, H], scale float32)."""
    y = act_values(x_bf16, act).astype(np.float32)
    s = fp8_tensor_scale(y)
    return fp8_quantize_with_scale(y, s), s


def quantize_weight_mxfp8(w):
    """MXFP8 weights: w float32 [E, N, K] -> (q uint8 [E, N, K],
    sf uint8 [E, N, K/32]), one scale per 32 values along K of each row."""
    w = _f32(w)
    E, N, K = w.shape
    q, b = quantize_mxfp8_rows(w.reshape(E * N, K))
    return q.reshape(E, N, K), b.reshape(E, N, K // MX_BLOCK)


def mx_colwise_offsets(m_offsets):
    """Start row of each expert's block in the columnwise layout: the expert's
    rows padded to a multiple of 128 (the padding of the rowwise scales, which
    also gives the [4, 128] columnwise scale shape of a [64, 128] expert in
    "[PyTorch] Let GroupedLinear accept MXFP8 input and gradient").  Returns
    int64 [E+1]; the padded totals are the same as ``mx_padded_offsets``."""
    return mx_padded_offsets(m_offsets)


def quantize_mxfp8_colwise(values, m_offsets):
    """Columnwise MXFP8 of expert-concatenated rows (the scaling factors along
    the rows that the gradient GEMMs contract over, "[PyTorch] Let
    GroupedLinear accept MXFP8 input and gradient": colwise scales, one per 32
    rows of a column).

    values float32-convertible [R, C]; for expert e (rows m_offsets[e] ..
    m_offsets[e+1]-1) the rows are padded with zeros to Rp_e = roundup(m_e,
    128) and every column is cut into blocks of 32 consecutive rows of the
    expert, each with one e8m0 scale by the rule of ``quantize_mxfp8_rows``.
    The result is stored transposed, expert by expert: expert e's codes are a
    [C, Rp_e] block (element (c, j) is the code of row m_offsets[e] + j,
    column c) and its scales a [C, Rp_e / 32] block.  Returns the flat
    concatenations (qT uint8 [C * sum Rp_e], sfT uint8 [C * sum Rp_e / 32])."""
    v = _f32(values)
    mo = np.asarray(m_offsets, dtype=np.int64)
    po = mx_colwise_offsets(mo)
    C = v.shape[1]
    qs, bs = [], []
    for e in range(len(mo) - 1):
        rp = int(po[e + 1] - po[e])
        seg = np.zeros((rp, C), np.float32)
        seg[: mo[e + 1] - mo[e]] = v[mo[e]:mo[e + 1]]
        q, b = quantize_mxfp8_rows(seg.T)                 # blocks along the rows
        qs.append(q.reshape(-1))
        bs.append(b.reshape(-1))
    if not qs:
        return np.zeros(0, np.uint8), np.zeros(0, np.uint8)
    return np.concatenate(qs), np.concatenate(bs)


def quantize_act_mxfp8_colwise(x_bf16, m_offsets):
    """Columnwise MXFP8 of bf16 rows (activations or output gradients), see
    ``quantize_mxfp8_colwise``."""
    return quantize_mxfp8_colwise(bf16_decode(x_bf16).astype(np.float32), m_offsets)


def quantize_weight_mxfp8_colwise(w):
    """MXFP8 weights quantized along N (the dimension the input gradient
    contracts over): w float32 [E, N, K] with N % 128 == 0 ->
    (qT uint8 [E, K, N], sfT uint8 [E, K, N / 32]), expert e's [K, N] block
    being the columnwise quantization of w[e]."""
    w = _f32(w)
    E, N, K = w.shape
    if N % MX_ROW_PAD:
        raise ValueError("N must be a multiple of 128")
    q, b = quantize_mxfp8_colwise(w.reshape(E * N, K), np.arange(E + 1) * N)
    return q.reshape(E, K, N), b.reshape(E, K, N // MX_BLOCK)


def grouped_linear_dgrad_mxfp8(dy_q, dy_sf, wT_q, wT_sf, m_offsets, rows=None, cols=None,
                               as_float32=False):
    """Input gradient of the MXFP8 grouped linear y = x W_e^T: for row r of
    expert e, dx[r, k] = sum_n dy[r, n] W_e[n, k], with the output gradient
    quantized rowwise (blocks along N, per-expert padded scales as for
    activations) and the weights columnwise (``quantize_weight_mxfp8_colwise``,
    blocks along N).  The same contraction as the forward grouped linear with
    W_e^T in place of the weights, so that routine is the step; output
    bf16 [rows, K]."""
    return grouped_gemm_mxfp8(dy_q, dy_sf, wT_q, wT_sf, m_offsets, rows, cols, as_float32)


def grouped_linear_wgrad_mxfp8(dyT_q, dyT_sf, xT_q, xT_sf, m_offsets, N, K, as_float32=False):
    """Weight gradient of the MXFP8 grouped linear: dW_e[n, k] = sum over the
    rows r of expert e of dy[r, n] x[r, k], both operands quantized columnwise
    (blocks of 32 rows, ``quantize_act_mxfp8_colwise`` layout).  Each expert's
    contraction runs over its padded rows (the padding is zero).  Returns
    bf16 [E, N, K] as uint16 (or float32 with as_float32)."""
    mo = np.asarray(m_offsets, dtype=np.int64)
    po = mx_colwise_offsets(mo)
    E = len(mo) - 1
    out = np.zeros((E, N, K), np.float64)
    for e in range(E):
        rp = int(po[e + 1] - po[e])
        if rp == 0:
            continue
        nb = rp // MX_BLOCK
        dy = _mx_decode_rows(np.asarray(dyT_q)[N * po[e]: N * po[e + 1]].reshape(N, rp),
                             np.asarray(dyT_sf)[N * po[e] // MX_BLOCK: N * po[e + 1] // MX_BLOCK].reshape(N, nb))
        xx = _mx_decode_rows(np.asarray(xT_q)[K * po[e]: K * po[e + 1]].reshape(K, rp),
                             np.asarray(xT_sf)[K * po[e] // MX_BLOCK: K * po[e + 1] // MX_BLOCK].reshape(K, nb))
        out[e] = dy @ xx.T
    out32 = out.astype(np.float32)
    return out32 if as_float32 else bf16_round(out32)


# ----------------------------------------------------------------------------
# grouped GEMM with the scale / router-weight epilogue
# ----------------------------------------------------------------------------
def _slots_by_expert(topk_ids, slots):
    flat = np.asarray(topk_ids).reshape(-1)
    sel = np.arange(flat.size) if slots is None else np.asarray(slots, dtype=np.int64)
    return sel, flat[sel]


def _grouped(decode_a, decode_w_rows, scale_of, topk_ids, topk_weights, N, slots, cols):
    """Shared per-expert loop: for every selected slot i (token t = i // top_k,
    expert e) and column n: y[i, n] = (A[t] . W[e, n]) * scale_of(e, n) * w[i],
    with the dot product in float64."""
    top_k = np.asarray(topk_ids).shape[1]
    sel, experts = _slots_by_expert(topk_ids, slots)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    wt = np.asarray(topk_weights, dtype=np.float32).reshape(-1).astype(np.float64)
    y = np.zeros((sel.size, cols.size), dtype=np.float64)
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        tokens = sel[rows] // top_k
        acc = decode_a(tokens) @ decode_w_rows(int(e), cols).T
        y[rows] = acc * scale_of(int(e), cols)[None, :] * wt[sel[rows]][:, None]
    return y.astype(np.float32)


def grouped_gemm_fp8w8a8(a_q, a_scale, w_q, w_scale, topk_ids, topk_weights,
                         slots=None, cols=None):
    """fp8 W8A8: e4m3 activations (one scale) x e4m3 weights (one scale per
    expert).  Returns float32 y for the selected slots x cols (all by default).
    ("Tianxing/moe quantization", FP8_W8A8 Benchmark.)"""
    a_q = np.asarray(a_q)
    w_q = np.asarray(w_q)
    ws = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    sa = float(np.float32(a_scale))
    return _grouped(lambda t: e4m3_decode(a_q[t]),
                    lambda e, c: e4m3_decode(w_q[e][c]),
                    lambda e, c: np.full(c.size, sa * ws[e]),
                    topk_ids, topk_weights, w_q.shape[1], slots, cols)


def grouped_gemm_int8w8a16(a_bf16, w_q, w_scale, topk_ids, topk_weights,
                           slots=None, cols=None):
    """int8 W8A16: bf16 activations x int8 weights with one scale per expert
    and output channel ("Tianxing/moe quantization", INT8_W8A16 Benchmark;
    "INT8 quantization support": int8 weights used with 16-bit activations)."""
    a = np.asarray(a_bf16)
    w_q = np.asarray(w_q)
    ws = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    return _grouped(lambda t: bf16_decode(a[t]),
                    lambda e, c: w_q[e][c].astype(np.float64),
                    lambda e, c: ws[e][c],
                    topk_ids, topk_weights, w_q.shape[1], slots, cols)


def grouped_gemm_int4w16(a_bf16, w_q, w_scale, topk_ids, topk_weights,
                         slots=None, cols=None):
    """int4 weight-only: bf16 activations x int4 codes (-7..7) with one scale
    per expert and output channel ("int4wo" of "Enabling MOE Quantization
    using linear decomposition", Summary); the codes are used as the exact
    integers they stand for."""
    a = np.asarray(a_bf16)
    w_q = np.asarray(w_q)
    ws = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    return _grouped(lambda t: bf16_decode(a[t]),
                    lambda e, c: w_q[e][c].astype(np.float64),
                    lambda e, c: ws[e][c],
                    topk_ids, topk_weights, w_q.shape[1], slots, cols)


def grouped_gemm_fp8w8a16(a_bf16, w_q, w_scale, topk_ids, topk_weights,
                          slots=None, cols=None):
    """fp8 weight-only: bf16 activations x e4m3 weights with one scale per
    expert and output channel ("fp8wo" of "Enabling MOE Quantization using
    linear decomposition", Summary); the weights are used at their exact
    decoded values."""
    a = np.asarray(a_bf16)
    w_q = np.asarray(w_q)
    ws = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    return _grouped(lambda t: bf16_decode(a[t]),
                    lambda e, c: e4m3_decode(w_q[e][c]),
                    lambda e, c: ws[e][c],
                    topk_ids, topk_weights, w_q.shape[1], slots, cols)


def grouped_gemm_int8w8a8(a_q, a_scale, w_q, w_scale, topk_ids, topk_weights,
                          slots=None, cols=None):
    """int8 W8A8 with dynamic per-token activation scales ("int8dq" of
    "Enabling MOE Quantization using linear decomposition", Summary): int8
    activation rows (scale a_scale[t] per token) x int8 weights (scale per
    expert and output channel).  For every selected slot i (token t = i //
    top_k, expert e) and column n: y[i, n] = (q_a[t] . q_w[e, n]) * a_scale[t]
    * w_scale[e, n] * w[i]; the integer dot product is exact in float64
    (|sum| < 2^53), the product of the factors is taken in float64 and
    rounded once to float32."""
    a_q = np.asarray(a_q)
    w_q = np.asarray(w_q)
    sa = np.asarray(a_scale, dtype=np.float32).astype(np.float64)
    ws = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    top_k = np.asarray(topk_ids).shape[1]
    sel, experts = _slots_by_expert(topk_ids, slots)
    cols = np.arange(w_q.shape[1]) if cols is None else np.asarray(cols, dtype=np.int64)
    wt = np.asarray(topk_weights, dtype=np.float32).reshape(-1).astype(np.float64)
    y = np.zeros((sel.size, cols.size), dtype=np.float64)
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        tokens = sel[rows] // top_k
        dot = a_q[tokens].astype(np.float64) @ w_q[int(e)][cols].astype(np.float64).T
        y[rows] = dot * sa[tokens][:, None] * ws[int(e)][cols][None, :] * wt[sel[rows]][:, None]
    return y.astype(np.float32)


def _mx_decode_rows(q_rows, sf_rows):
    """Decoded MXFP8 rows: e4m3 value * 2^(b - 127) for every block of 32."""
    R, K = q_rows.shape
    v = e4m3_decode(q_rows).reshape(R, K // MX_BLOCK, MX_BLOCK)
    return (v * e8m0_decode(sf_rows)[..., None]).reshape(R, K)


def grouped_gemm_mxfp8(a_q, a_sf, w_q, w_sf, m_offsets, rows=None, cols=None, as_float32=False):
    """MXFP8 grouped linear over expert-contiguous row segments ("[PyTorch] Let
    GroupedLinear accept MXFP8 input and gradient").

    a_q uint8 [R, K] with rowwise scales a_sf in per-expert blocks padded to
    128 rows (see ``quantize_act_mxfp8``); w_q uint8 [E, N, K] with w_sf
    [E, N, K/32].  acc[r, n] = sum over blocks of 2^(ba+bw-254) * sum(qa*qw),
    evaluated in float64; the output is bf16(fl32(acc)) as uint16
    [len(rows), len(cols)] (or fl32(acc) itself with as_float32)."""
    a_q = np.asarray(a_q)
    w_q = np.asarray(w_q)
    mo = np.asarray(m_offsets, dtype=np.int64)
    po = mx_padded_offsets(mo)
    R, K = a_q.shape
    N = w_q.shape[1]
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    expert = np.searchsorted(mo, rows, side="right") - 1
    out = np.zeros((rows.size, cols.size), dtype=np.float64)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        r = rows[sel]
        a = _mx_decode_rows(a_q[r], np.asarray(a_sf)[po[e] + (r - mo[e])])
        w = _mx_decode_rows(w_q[e][cols], np.asarray(w_sf)[e][cols])
        out[sel] = a @ w.T
    return out.astype(np.float32) if as_float32 else bf16_round(out.astype(np.float32))


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------
def slot_results_bf16(y):
    """The per-slot results as the hot path stores them between the grouped
    GEMM and the combine: bf16 bits (round to nearest even) of the float32
    values.  Two bytes per routed slot and output column is what the byte
    accounting behind the Bandwidth column of the FP8_W8A8 and INT8_W8A16
    benchmark tables ("Tianxing/moe quantization") charges for the output
    (M * top_k * N * 2).  y float32 [M*top_k, N] -> uint16 [M*top_k, N]."""
    return bf16_round(_f32(y))


def combine(y, top_k):
    """Per-token sum of the top_k slot results, in slot order, in float32, then
    rounded to bf16.  y float32 [M*top_k, N] -> (out32 float32 [M, N],
    out bf16 bits uint16 [M, N])."""
    y = _f32(y)
    M = y.shape[0] // top_k
    yy = y.reshape(M, top_k, -1)
    acc = yy[:, 0, :].copy()
    for j in range(1, top_k):
        acc = (acc + yy[:, j, :]).astype(np.float32)
    return acc, bf16_round(acc)


# ----------------------------------------------------------------------------
# accounting used by the measurements
# ----------------------------------------------------------------------------
def flops(M, K, N, top_k):
    """Useful flops of one grouped GEMM: 2 * M * top_k * K * N (the accounting
    behind the TFLOPS column of the "Tianxing/moe quantization" tables)."""
    return 2 * M * top_k * K * N
