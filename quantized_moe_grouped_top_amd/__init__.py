"""Python binding of libqmoe.so, the MI355X quantized MoE grouped GEMM library.

Argument marshalling only: every function below calls the C entry point of
the same name (declared in ``include/moe.h``) with the device pointers of the
torch tensors it is given and the current HIP stream, and raises ``MoeError``
on a non-zero status.  All computation happens in the HIP kernels of the
library; torch only provides device memory and streams.

The library is loaded on first use and must have been built
(``python -m quantized_moe_grouped_top_amd.build``); a missing library raises
``MoeLibraryMissing`` - there is no fallback path.
"""

import ctypes
import os

from . import synth  # noqa: F401  (seeded synthetic inputs; no method arithmetic)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP = 0, -1, -2, -3
MOE_Q_FP8_PER_TENSOR, MOE_Q_MXFP8, MOE_Q_INT8_PER_CHANNEL, MOE_Q_FP8_PER_CHANNEL = 0, 1, 2, 3
MOE_Q_INT4_PER_CHANNEL, MOE_Q_MXFP8_COLWISE = 4, 5
MOE_W_ROWMAJOR, MOE_W_TILED, MOE_W_FRAG = 0, 1, 2
MOE_ACT_SWIGLU, MOE_ACT_SRELU = 0, 1
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_SLOTS = 128, 8, 65536

EXPORTS = [
    "moe_last_error", "moe_last_hip_error", "moe_align_max_padded", "moe_recommended_block_m",
    "moe_quantize_workspace_bytes", "moe_packed_weight_bytes", "moe_mx_scale_rows",
    "moe_align_block_size", "moe_quantize_act", "moe_quantize_act_noalloc", "moe_act_quantize",
    "moe_quantize_weights",
    "moe_pack_weights",
    "moe_grouped_gemm_fp8w8a8",
    "moe_grouped_gemm_int8w8a8", "moe_grouped_gemm_fp8w8a16", "moe_grouped_gemm_int4w4a16",
    "moe_grouped_gemm_int8w8a16", "moe_grouped_gemm_mxfp8", "moe_combine",
    "moe_quantize_act_colwise", "moe_grouped_gemm_mxfp8_wgrad",
]


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class MoeLibraryMissing(ImportError):
    pass


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_last_hip_error": (_I, []),
    "moe_align_max_padded": (_I, [_I, _I, _I, _I]),
    "moe_recommended_block_m": (_I, [_I, _I, _I]),
    "moe_quantize_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "moe_packed_weight_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "moe_pack_weights": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "moe_mx_scale_rows": (_I, [_I, _I]),
    "moe_align_block_size": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_quantize_act": (_I, [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "moe_quantize_act_noalloc": (_I, [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P]),
    "moe_act_quantize": (_I, [_P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "moe_quantize_weights": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm_fp8w8a8": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_grouped_gemm_int8w8a8": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_grouped_gemm_int8w8a16": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_grouped_gemm_fp8w8a16": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_grouped_gemm_int4w4a16": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_quantize_act_colwise": (_I, [_P, _I, _I, _P, _I, _P, _P, _P]),
    "moe_grouped_gemm_mxfp8_wgrad": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_grouped_gemm_mxfp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_combine": (_I, [_P, _I, _I, _I, _P, _P]),
}


def lib():
    """The loaded ctypes library (loads it on first call)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m quantized_moe_grouped_top_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())
    return rc


def _size(rc):
    if rc < 0:
        raise MoeError(rc, lib().moe_last_error().decode())
    return rc


# ---- sizes ------------------------------------------------------------------
def moe_align_max_padded(M, E, top_k, block_m):
    return _size(lib().moe_align_max_padded(M, E, top_k, block_m))


def moe_recommended_block_m(M, E, top_k):
    return _size(lib().moe_recommended_block_m(M, E, top_k))


def moe_quantize_workspace_bytes(mode, tensors):
    return int(lib().moe_quantize_workspace_bytes(mode, tensors))


def moe_packed_weight_bytes(E, N, K, layout):
    return int(lib().moe_packed_weight_bytes(E, N, K, layout))


def moe_mx_scale_rows(rows, E):
    return _size(lib().moe_mx_scale_rows(rows, E))


# ---- hot path -----------------------------------------------------------------
def moe_align_block_size(logits, M, E, top_k, block_m, topk_ids, topk_weights,
                         sorted_token_ids, expert_ids, num_tokens_post_padded, stream=None):
    return _check(lib().moe_align_block_size(
        _ptr(logits), M, E, top_k, block_m, _ptr(topk_ids), _ptr(topk_weights),
        _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded), _stream(stream)))


def moe_quantize_act(x, rows, K, mode, m_offsets, E, q, scale, scale_e8m0, workspace,
                     stream=None):
    return _check(lib().moe_quantize_act(
        _ptr(x), rows, K, mode, _ptr(m_offsets), E, _ptr(q), _ptr(scale), _ptr(scale_e8m0),
        _ptr(workspace), _stream(stream)))


def moe_quantize_act_noalloc(x, rows, K, mode, m_offsets, E, q, scale, scale_e8m0, stream=None):
    return _check(lib().moe_quantize_act_noalloc(
        _ptr(x), rows, K, mode, _ptr(m_offsets), E, _ptr(q), _ptr(scale), _ptr(scale_e8m0),
        _stream(stream)))


def moe_act_quantize(x, rows, H, act, mode, m_offsets, E, q, scale, scale_e8m0, workspace,
                     stream=None):
    return _check(lib().moe_act_quantize(
        _ptr(x), rows, H, act, mode, _ptr(m_offsets), E, _ptr(q), _ptr(scale), _ptr(scale_e8m0),
        _ptr(workspace), _stream(stream)))


def moe_quantize_weights(w, E, N, K, mode, q, scale, scale_e8m0, workspace, stream=None):
    return _check(lib().moe_quantize_weights(
        _ptr(w), E, N, K, mode, _ptr(q), _ptr(scale), _ptr(scale_e8m0), _ptr(workspace),
        _stream(stream)))


def moe_pack_weights(w_q, E, N, K, layout, w_packed, stream=None):
    return _check(lib().moe_pack_weights(_ptr(w_q), E, N, K, layout, _ptr(w_packed),
                                         _stream(stream)))


def moe_grouped_gemm_fp8w8a8(a_q, a_scale, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, topk_weights, M, K, N, E, top_k, block_m,
                             y, stream=None):
    return _check(lib().moe_grouped_gemm_fp8w8a8(
        _ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), w_layout, _ptr(sorted_token_ids),
        _ptr(expert_ids), _ptr(num_tokens_post_padded), _ptr(topk_weights), M, K, N, E, top_k,
        block_m, _ptr(y), _stream(stream)))


def moe_grouped_gemm_int8w8a8(a_q, a_scale, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                              num_tokens_post_padded, topk_weights, M, K, N, E, top_k, block_m,
                              y, stream=None):
    return _check(lib().moe_grouped_gemm_int8w8a8(
        _ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), w_layout, _ptr(sorted_token_ids),
        _ptr(expert_ids), _ptr(num_tokens_post_padded), _ptr(topk_weights), M, K, N, E, top_k,
        block_m, _ptr(y), _stream(stream)))


def moe_grouped_gemm_int8w8a16(a, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                               num_tokens_post_padded, topk_weights, M, K, N, E, top_k, block_m,
                               y, stream=None):
    return _check(lib().moe_grouped_gemm_int8w8a16(
        _ptr(a), _ptr(w_q), _ptr(w_scale), w_layout, _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(topk_weights), M, K, N, E, top_k, block_m, _ptr(y),
        _stream(stream)))


def moe_grouped_gemm_fp8w8a16(a, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                              num_tokens_post_padded, topk_weights, M, K, N, E, top_k, block_m,
                              y, stream=None):
    return _check(lib().moe_grouped_gemm_fp8w8a16(
        _ptr(a), _ptr(w_q), _ptr(w_scale), w_layout, _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(topk_weights), M, K, N, E, top_k, block_m, _ptr(y),
        _stream(stream)))


def moe_grouped_gemm_int4w4a16(a, w_q, w_scale, w_layout, sorted_token_ids, expert_ids,
                               num_tokens_post_padded, topk_weights, M, K, N, E, top_k, block_m,
                               y, stream=None):
    return _check(lib().moe_grouped_gemm_int4w4a16(
        _ptr(a), _ptr(w_q), _ptr(w_scale), w_layout, _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(topk_weights), M, K, N, E, top_k, block_m, _ptr(y),
        _stream(stream)))


def moe_quantize_act_colwise(x, rows, C, m_offsets, E, qT, sfT, stream=None):
    return _check(lib().moe_quantize_act_colwise(_ptr(x), rows, C, _ptr(m_offsets), E, _ptr(qT),
                                                 _ptr(sfT), _stream(stream)))


def moe_grouped_gemm_mxfp8_wgrad(dyT_q, dyT_sf, xT_q, xT_sf, m_splits, E, N, K, dw, stream=None):
    """m_splits: rows per expert, a host sequence of E ints."""
    splits = (ctypes.c_int * E)(*[int(v) for v in m_splits])
    return _check(lib().moe_grouped_gemm_mxfp8_wgrad(
        _ptr(dyT_q), _ptr(dyT_sf), _ptr(xT_q), _ptr(xT_sf), ctypes.cast(splits, ctypes.c_void_p),
        E, N, K, _ptr(dw), _stream(stream)))


def moe_grouped_gemm_mxfp8(a_q, a_sf, w_q, w_sf, m_offsets, rows, K, N, E, out, stream=None):
    return _check(lib().moe_grouped_gemm_mxfp8(
        _ptr(a_q), _ptr(a_sf), _ptr(w_q), _ptr(w_sf), _ptr(m_offsets), rows, K, N, E, _ptr(out),
        _stream(stream)))


def moe_combine(y, M, N, top_k, out, stream=None):
    return _check(lib().moe_combine(_ptr(y), M, N, top_k, _ptr(out), _stream(stream)))
