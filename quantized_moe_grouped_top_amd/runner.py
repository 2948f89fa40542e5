"""Device buffers and call sequence of one quantized MoE layer.

Allocates the routing, quantization and output buffers with torch (device
memory only) and runs the hot path as a sequence of library calls on the
current stream:

    routed formats : moe_align_block_size -> [moe_quantize_act] ->
                     moe_grouped_gemm_{fp8w8a8,int8w8a8,int8w8a16,fp8w8a16,int4w4a16} ->
                     moe_combine
    MXFP8          : moe_quantize_act(MXFP8) -> moe_grouped_gemm_mxfp8
    MXFP8 backward : input gradient = the MXFP8 call with the output gradient
                     and MOE_Q_MXFP8_COLWISE weights; weight gradient =
                     moe_quantize_act_colwise (dy, x) -> moe_grouped_gemm_mxfp8_wgrad
    activation     : moe_act_quantize (SwiGLU / SReLU + MXFP8 or fp8)

Every step runs in the library's HIP kernels; nothing here computes.
"""

import torch

from . import (MOE_ACT_SRELU, MOE_ACT_SWIGLU, MOE_Q_FP8_PER_CHANNEL, MOE_Q_FP8_PER_TENSOR,
               MOE_Q_INT4_PER_CHANNEL, MOE_Q_INT8_PER_CHANNEL, MOE_Q_MXFP8, MOE_Q_MXFP8_COLWISE,
               MOE_W_FRAG,
               MOE_W_ROWMAJOR,
               MOE_W_TILED, moe_act_quantize, moe_align_block_size, moe_align_max_padded, moe_combine,
               moe_grouped_gemm_fp8w8a8, moe_grouped_gemm_fp8w8a16, moe_grouped_gemm_int4w4a16,
               moe_grouped_gemm_int8w8a8,
               moe_grouped_gemm_int8w8a16,
               moe_grouped_gemm_mxfp8, moe_grouped_gemm_mxfp8_wgrad, moe_quantize_act_colwise,
               moe_mx_scale_rows, moe_pack_weights, moe_packed_weight_bytes, moe_quantize_act,
               moe_quantize_weights, moe_quantize_workspace_bytes, moe_recommended_block_m)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def quantize_weights(w, fmt):
    """Offline weight quantization of float32 w [E, N, K] on its device.
    Returns (w_q, w_scale) for fp8/int8/fp8wo or (w_q, w_sf) for MXFP8."""
    E, N, K = w.shape
    dev = w.device
    if fmt == "fp8":
        q = _empty((E, N, K), torch.uint8, dev)
        s = _empty((E,), torch.float32, dev)
        ws = _empty((moe_quantize_workspace_bytes(MOE_Q_FP8_PER_TENSOR, E),), torch.uint8, dev)
        moe_quantize_weights(w, E, N, K, MOE_Q_FP8_PER_TENSOR, q, s, None, ws)
        return q, s
    if fmt == "int4wo":                  # packed codes [E, N, K/2]
        q = _empty((E, N, K // 2), torch.uint8, dev)
        s = _empty((E, N), torch.float32, dev)
        moe_quantize_weights(w, E, N, K, MOE_Q_INT4_PER_CHANNEL, q, s, None, None)
        return q, s
    if fmt == "fp8wo":
        q = _empty((E, N, K), torch.uint8, dev)
        s = _empty((E, N), torch.float32, dev)
        moe_quantize_weights(w, E, N, K, MOE_Q_FP8_PER_CHANNEL, q, s, None, None)
        return q, s
    if fmt in ("int8", "int8dq"):
        q = _empty((E, N, K), torch.int8, dev)
        s = _empty((E, N), torch.float32, dev)
        moe_quantize_weights(w, E, N, K, MOE_Q_INT8_PER_CHANNEL, q, s, None, None)
        return q, s
    if fmt == "mxfp8":
        q = _empty((E, N, K), torch.uint8, dev)
        sf = _empty((E, N, K // 32), torch.uint8, dev)
        moe_quantize_weights(w, E, N, K, MOE_Q_MXFP8, q, None, sf, None)
        return q, sf
    if fmt == "mxfp8_colwise":           # along N, transposed: [E, K, N]
        q = _empty((E, K, N), torch.uint8, dev)
        sf = _empty((E, K, N // 32), torch.uint8, dev)
        moe_quantize_weights(w, E, N, K, MOE_Q_MXFP8_COLWISE, q, None, sf, None)
        return q, sf
    raise ValueError(fmt)


def pack_weights(w_q, layout=MOE_W_TILED):
    """Packed copy (MOE_W_TILED or MOE_W_FRAG) of one-byte weights [E, N, K]
    on their device."""
    E, N, K = w_q.shape
    out = _empty((moe_packed_weight_bytes(E, N, K, layout),), torch.uint8, w_q.device)
    moe_pack_weights(w_q, E, N, K, layout, out)
    return out


class RoutedMoE:
    """fp8 W8A8, int8 W8A16 ("int8"), int8 W8A8 with per-token activation
    scales ("int8dq"), bf16 x fp8 weight-only ("fp8wo") or bf16 x int4
    weight-only ("int4wo", block_m 16) MoE layer of fixed (M, K, N, E, top_k)."""

    def __init__(self, fmt, M, K, N, E, top_k, device="cuda", block_m=None,
                 w_layout=MOE_W_ROWMAJOR):
        assert fmt in ("fp8", "int8", "int8dq", "fp8wo", "int4wo")
        self.w_layout = w_layout
        self.fmt, self.M, self.K, self.N, self.E, self.top_k = fmt, M, K, N, E, top_k
        self.block_m = block_m or moe_recommended_block_m(M, E, top_k)
        self.max_padded = moe_align_max_padded(M, E, top_k, self.block_m)
        dev = device
        S = M * top_k
        self.topk_ids = _empty((M, top_k), torch.int32, dev)
        self.topk_weights = _empty((M, top_k), torch.float32, dev)
        self.sorted_token_ids = _empty((self.max_padded,), torch.int32, dev)
        self.expert_ids = _empty((self.max_padded // self.block_m,), torch.int32, dev)
        self.num_tokens_post_padded = _empty((1,), torch.int32, dev)
        if fmt == "fp8":
            self.a_q = _empty((M, K), torch.uint8, dev)
            self.a_scale = _empty((1,), torch.float32, dev)
            self.ws = _empty((moe_quantize_workspace_bytes(MOE_Q_FP8_PER_TENSOR, 1),),
                             torch.uint8, dev)
        if fmt == "int8dq":
            self.a_q = _empty((M, K), torch.int8, dev)
            self.a_scale = _empty((max(M, 1),), torch.float32, dev)
        self.y = _empty((S, N), torch.int16, dev)      # bf16 bits, one row per slot
        self.out = _empty((M, N), torch.int16, dev)     # bf16 bits

    def route(self, logits):
        moe_align_block_size(logits, self.M, self.E, self.top_k, self.block_m, self.topk_ids,
                             self.topk_weights, self.sorted_token_ids, self.expert_ids,
                             self.num_tokens_post_padded)

    def quantize(self, x):
        if self.fmt == "fp8":
            moe_quantize_act(x, self.M, self.K, MOE_Q_FP8_PER_TENSOR, None, 1, self.a_q,
                             self.a_scale, None, self.ws)
        elif self.fmt == "int8dq":
            moe_quantize_act(x, self.M, self.K, MOE_Q_INT8_PER_CHANNEL, None, 1, self.a_q,
                             self.a_scale, None, None)

    def gemm(self, x, w_q, w_scale):
        if self.fmt == "fp8":
            moe_grouped_gemm_fp8w8a8(self.a_q, self.a_scale, w_q, w_scale, self.w_layout,
                                     self.sorted_token_ids,
                                     self.expert_ids, self.num_tokens_post_padded,
                                     self.topk_weights, self.M, self.K, self.N, self.E,
                                     self.top_k, self.block_m, self.y)
        elif self.fmt == "int8dq":
            moe_grouped_gemm_int8w8a8(self.a_q, self.a_scale, w_q, w_scale, self.w_layout,
                                      self.sorted_token_ids, self.expert_ids,
                                      self.num_tokens_post_padded, self.topk_weights, self.M,
                                      self.K, self.N, self.E, self.top_k, self.block_m, self.y)
        elif self.fmt == "int4wo":
            moe_grouped_gemm_int4w4a16(x, w_q, w_scale, self.w_layout, self.sorted_token_ids,
                                       self.expert_ids, self.num_tokens_post_padded,
                                       self.topk_weights, self.M, self.K, self.N, self.E,
                                       self.top_k, self.block_m, self.y)
        elif self.fmt == "fp8wo":
            moe_grouped_gemm_fp8w8a16(x, w_q, w_scale, self.w_layout, self.sorted_token_ids,
                                      self.expert_ids, self.num_tokens_post_padded,
                                      self.topk_weights, self.M, self.K, self.N, self.E,
                                      self.top_k, self.block_m, self.y)
        else:
            moe_grouped_gemm_int8w8a16(x, w_q, w_scale, self.w_layout, self.sorted_token_ids,
                                       self.expert_ids,
                                       self.num_tokens_post_padded, self.topk_weights, self.M,
                                       self.K, self.N, self.E, self.top_k, self.block_m, self.y)

    def combine(self):
        moe_combine(self.y, self.M, self.N, self.top_k, self.out)

    def forward(self, x, logits, w_q, w_scale):
        """One pass of the hot path; returns the bf16 output bits [M, N] (int16)."""
        self.route(logits)
        self.quantize(x)
        self.gemm(x, w_q, w_scale)
        self.combine()
        return self.out


class MxMoE:
    """MXFP8 grouped linear over expert-concatenated rows."""

    def __init__(self, rows, K, N, E, device="cuda"):
        self.rows, self.K, self.N, self.E = rows, K, N, E
        self.a_q = _empty((rows, K), torch.uint8, device)
        self.a_sf = _empty((moe_mx_scale_rows(rows, E), K // 32), torch.uint8, device)
        self.out = _empty((rows, N), torch.int16, device)

    def quantize(self, x, m_offsets):
        moe_quantize_act(x, self.rows, self.K, MOE_Q_MXFP8, m_offsets, self.E, self.a_q, None,
                         self.a_sf, None)

    def gemm(self, w_q, w_sf, m_offsets):
        moe_grouped_gemm_mxfp8(self.a_q, self.a_sf, w_q, w_sf, m_offsets, self.rows, self.K,
                               self.N, self.E, self.out)

    def forward(self, x, m_offsets, w_q, w_sf):
        self.quantize(x, m_offsets)
        self.gemm(w_q, w_sf, m_offsets)
        return self.out


class MxWgrad:
    """Weight gradient of the MXFP8 grouped linear: columnwise quantization
    of the output gradient dy [rows, N] and the input x [rows, K], then one
    grouped-GEMM launch over every expert into dw [E, N, K] (bf16 bits)."""

    def __init__(self, rows, K, N, E, m_splits, device="cuda"):
        self.rows, self.K, self.N, self.E = rows, K, N, E
        self.m_splits = [int(v) for v in m_splits]
        P = moe_mx_scale_rows(rows, E)
        self.dyT_q = _empty((N * P,), torch.uint8, device)
        self.dyT_sf = _empty((N * P // 32 + 1,), torch.uint8, device)
        self.xT_q = _empty((K * P,), torch.uint8, device)
        self.xT_sf = _empty((K * P // 32 + 1,), torch.uint8, device)
        self.dw = _empty((E, N, K), torch.int16, device)

    def quantize(self, dy, x, m_offsets):
        moe_quantize_act_colwise(dy, self.rows, self.N, m_offsets, self.E, self.dyT_q, self.dyT_sf)
        moe_quantize_act_colwise(x, self.rows, self.K, m_offsets, self.E, self.xT_q, self.xT_sf)

    def gemm(self):
        moe_grouped_gemm_mxfp8_wgrad(self.dyT_q, self.dyT_sf, self.xT_q, self.xT_sf, self.m_splits,
                                     self.E, self.N, self.K, self.dw)


class ActQuant:
    """Fused activation + quantization of expert-concatenated rows: x bf16
    [rows, 2H] (SwiGLU) or [rows, H] (SReLU) -> q [rows, H] e4m3 with MXFP8
    scale bytes (per-expert padded blocks) or one fp8 tensor scale."""

    def __init__(self, rows, H, E, act="swiglu", mode="mxfp8", device="cuda"):
        self.rows, self.H, self.E = rows, H, E
        self.act = {"swiglu": MOE_ACT_SWIGLU, "srelu": MOE_ACT_SRELU}[act]
        self.mode = {"mxfp8": MOE_Q_MXFP8, "fp8": MOE_Q_FP8_PER_TENSOR}[mode]
        self.q = _empty((rows, H), torch.uint8, device)
        self.scale = _empty((1,), torch.float32, device)
        self.sf = self.ws = None
        if self.mode == MOE_Q_MXFP8:
            self.sf = _empty((moe_mx_scale_rows(rows, E), H // 32), torch.uint8, device)
        else:
            self.ws = _empty((moe_quantize_workspace_bytes(MOE_Q_FP8_PER_TENSOR, 1),), torch.uint8,
                             device)

    def __call__(self, x, m_offsets=None):
        moe_act_quantize(x, self.rows, self.H, self.act, self.mode, m_offsets, self.E, self.q,
                         self.scale, self.sf, self.ws)
        return self.q
