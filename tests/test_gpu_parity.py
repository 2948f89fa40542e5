"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Bars:
* routing choices, the sorted-slot and block-expert buffers, the padded
  length, every quantized byte and every quantization scale: bit-exact;
* router weights: within 8 float32 units of the oracle's (the device exp
  differs from libm's), summing to one within 4 units;
* grouped GEMM outputs (per routed slot, stored as bf16): |gpu - ref| <=
  2e-2 * rms(ref) + half a bf16 unit of ref for every element, ref being the
  oracle's float32 result;
* bf16 layer outputs: see _parity.assert_bf16_out;
* the combine kernel on its own: bit-exact on seeded synthetic inputs.

Small cases are compared element by element; the workloads at their full
sizes (in the launch configuration the benchmark times) are compared on
sampled tokens, columns and rows, which the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import quantized_moe_grouped_top_amd as qm
from quantized_moe_grouped_top_amd import runner, synth
from oracle import formats as F
from oracle import moe as O

from _parity import (assert_bf16_out, assert_close_rms, bits16, oracle_weights_rows, pick,
                     unpack_int4)

pytestmark = pytest.mark.gpu
DEV = "cuda"
F32_EPS = float(np.finfo(np.float32).eps)


def _announce(what):
    print(f"\n[parity] {what}", flush=True)


# ----------------------------------------------------------------------------
# routed formats
# ----------------------------------------------------------------------------
def run_routed(wl, block_m=None, variant=0, full=True, n_tok=48, n_col=64, logits=None,
               layout=qm.MOE_W_ROWMAJOR):
    _announce(f"{wl.name} block_m={block_m} layout={layout} full={full}")
    M, K, N, E, top_k = wl.M, wl.K, wl.N, wl.E, wl.top_k
    case = synth.make_case(wl, variant, device=DEV)
    x, w = case["x"], case["w"]
    lg = case["logits"] if logits is None else logits.to(DEV)
    moe = runner.RoutedMoE(wl.fmt, M, K, N, E, top_k, block_m=block_m, w_layout=layout)
    w_q, w_scale = runner.quantize_weights(w, wl.fmt)
    w_gemm = runner.pack_weights(w_q, layout) if layout != qm.MOE_W_ROWMAJOR else w_q
    moe.y.fill_(0x7FC0)                      # bf16 NaN: unwritten slots show up
    moe.out.fill_(0x7FC0)
    moe.forward(x, lg, w_gemm, w_scale)
    torch.cuda.synchronize()

    rng = np.random.default_rng(synth.seed_of(wl.name, 99) % (1 << 32))
    lg_np = lg.cpu().numpy()
    x_np = bits16(x)

    # ---- routing and alignment: bit-exact -----------------------------------
    ids_ref, wts_ref = O.route_topk(lg_np, top_k)
    np.testing.assert_array_equal(moe.topk_ids.cpu().numpy(), ids_ref)
    wts = moe.topk_weights.cpu().numpy()
    np.testing.assert_allclose(wts, wts_ref, rtol=8 * F32_EPS, atol=1e-44)  # denormal weights
    assert np.max(np.abs(wts.astype(np.float64).sum(1) - 1.0)) <= 4 * F32_EPS
    s_ref, e_ref, n_ref = O.align_block_size(ids_ref, E, moe.block_m)
    assert int(moe.num_tokens_post_padded.item()) == n_ref
    np.testing.assert_array_equal(moe.sorted_token_ids.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(moe.expert_ids.cpu().numpy(), e_ref)

    # ---- which outputs the oracle computes ----------------------------------
    if full:
        toks, cols = np.arange(M), np.arange(N)
    else:
        toks = pick(M, n_tok, rng, must=(0, M - 1))
        # the first and last column, the middle, and both sides of the
        # 256-column tile edges at the start and the end
        cols = pick(N, n_col, rng, must=(0, N - 1, N // 2, 255, 256, N - 257, N - 256))
    slots = (toks[:, None] * top_k + np.arange(top_k)[None, :]).reshape(-1)

    # ---- weights: bit-exact quantization of the checked rows ----------------
    wq_rows, ws_ref = oracle_weights_rows(w, wl.fmt, cols)
    wq_dev = w_q.index_select(1, torch.as_tensor(cols, device=DEV)).cpu().numpy()
    if wl.fmt == "int4wo":
        wq_dev = unpack_int4(wq_dev)
    np.testing.assert_array_equal(wq_dev, wq_rows)
    if wl.fmt == "fp8":
        np.testing.assert_array_equal(w_scale.cpu().numpy(), ws_ref)
    else:
        np.testing.assert_array_equal(w_scale.cpu().numpy()[:, cols], ws_ref)
    # oracle weight tensors holding only the checked columns (other rows unused)
    wq_full = np.zeros((E, N, K), dtype=wq_rows.dtype)
    wq_full[:, cols] = wq_rows
    if wl.fmt == "fp8":
        ws_full = ws_ref
    else:
        ws_full = np.zeros((E, N), np.float32)
        ws_full[:, cols] = ws_ref

    # ---- activations and the GEMM --------------------------------------------
    if wl.fmt == "fp8":
        xv = F.bf16_decode(x_np).astype(np.float32)
        sa = O.fp8_tensor_scale(xv)
        assert moe.a_scale.item() == float(sa)
        aq_rows = O.fp8_quantize_with_scale(xv[toks], sa)
        np.testing.assert_array_equal(moe.a_q.cpu().numpy()[toks], aq_rows)
        aq_full = np.zeros((M, K), np.uint8)
        aq_full[toks] = aq_rows
        y_ref = O.grouped_gemm_fp8w8a8(aq_full, sa, wq_full, ws_full, ids_ref, wts_ref, slots, cols)
    elif wl.fmt == "int8dq":
        # per-token scales: the checked tokens' rows alone fix them
        aq_rows, sa_rows = O.quantize_act_int8_rows(x_np[toks])
        np.testing.assert_array_equal(moe.a_q.cpu().numpy()[toks], aq_rows)
        np.testing.assert_array_equal(moe.a_scale.cpu().numpy()[toks], sa_rows)
        aq_full = np.zeros((M, K), np.int8)
        aq_full[toks] = aq_rows
        sa_full = np.ones(M, np.float32)
        sa_full[toks] = sa_rows
        y_ref = O.grouped_gemm_int8w8a8(aq_full, sa_full, wq_full, ws_full, ids_ref, wts_ref, slots, cols)
    elif wl.fmt == "fp8wo":
        y_ref = O.grouped_gemm_fp8w8a16(x_np, wq_full, ws_full, ids_ref, wts_ref, slots, cols)
    elif wl.fmt == "int4wo":
        y_ref = O.grouped_gemm_int4w16(x_np, wq_full, ws_full, ids_ref, wts_ref, slots, cols)
    else:
        y_ref = O.grouped_gemm_int8w8a16(x_np, wq_full, ws_full, ids_ref, wts_ref, slots, cols)
    # the per-slot results are stored as bf16: the float32 tolerance plus half
    # a bf16 unit of the reference (the storage rounding itself)
    y_bits = bits16(moe.y)[np.ix_(slots, cols)]
    assert_bf16_out(y_bits, y_ref, O.slot_results_bf16(y_ref), f"{wl.name} y")

    # ---- combine ---------------------------------------------------------------
    # against the oracle's pipeline (its per-slot results rounded to bf16) ...
    out32_ref, out_ref = O.combine(F.bf16_decode(O.slot_results_bf16(y_ref)), top_k)
    out_gpu = bits16(moe.out)[np.ix_(toks, cols)]
    assert_bf16_out(out_gpu, out32_ref, out_ref, f"{wl.name} out")
    # ... and bit-exactly against the oracle's combine of the GPU's own slots
    np.testing.assert_array_equal(out_gpu, O.combine(F.bf16_decode(y_bits), top_k)[1])
    return moe


SMALL = [
    synth.WORKLOADS["fp8_m64_k128_n256"],
    synth.small("fp8", 37, 256, 200, 8, 2),
    synth.small("fp8", 300, 384, 320, 8, 2, bias_std=1.5),
    synth.small("int8", 50, 320, 136, 6, 3),
    synth.small("int8", 300, 256, 272, 8, 2, bias_std=1.5),
    synth.small("fp8", 1, 128, 64, 8, 2),
    synth.small("int8", 40, 128, 48, 1, 1),
    synth.small("fp8", 33, 256, 96, 4, 4),
    # >= 256 routed rows per expert: the four-wavefront persistent kernel
    synth.small("fp8", 400, 256, 320, 2, 2),
    synth.small("fp8", 800, 384, 136, 4, 2, bias_std=1.5),
    # int8 W8A8 with per-token activation scales
    synth.small("int8dq", 37, 256, 200, 8, 2),
    synth.small("int8dq", 300, 384, 320, 8, 2, bias_std=1.5),
    synth.small("int8dq", 400, 256, 136, 2, 2),
    # few rows per expert on average (32 rows per pass for bf16 activations)
    # with a biased router, so that some experts need several passes
    synth.small("int8", 60, 256, 136, 8, 2, bias_std=1.5),
    synth.small("fp8wo", 60, 256, 136, 8, 2, bias_std=1.5),
    # bf16 activations x fp8 weights with per-channel scales
    synth.small("fp8wo", 50, 320, 136, 6, 3),
    synth.small("fp8wo", 300, 256, 272, 8, 2, bias_std=1.5),
    synth.small("fp8wo", 40, 128, 48, 1, 1),
    # bf16 activations with >= 256 routed rows per expert: the tile kernel
    # (64-k stages; K = 320 ends on half a 128-byte weight block, K = 64 is one
    # stage per tile)
    synth.small("int8", 400, 256, 320, 2, 2),
    synth.small("int8", 500, 320, 200, 2, 2, bias_std=1.5),
    synth.small("fp8wo", 800, 384, 136, 4, 2, bias_std=1.5),
    synth.small("fp8wo", 400, 64, 264, 2, 2),
    # many experts, most with a few rows or none (the largest E and top_k the
    # library takes, and two in between)
    synth.small("fp8", 48, 256, 136, 128, 8),
    synth.small("int8", 100, 128, 200, 64, 6, bias_std=1.5),
    synth.small("int8dq", 300, 256, 72, 32, 4),
    synth.small("fp8wo", 48, 128, 264, 128, 8, bias_std=1.5),
]


# (block_m, weight layout): MOE_W_FRAG is for the streaming kernel only
KERNEL_LAYOUTS = [(16, qm.MOE_W_ROWMAJOR), (16, qm.MOE_W_TILED), (16, qm.MOE_W_FRAG),
                  (128, qm.MOE_W_ROWMAJOR), (128, qm.MOE_W_TILED)]
KL_IDS = ["16-rowmajor", "16-tiled", "16-frag", "128-rowmajor", "128-tiled"]


def bench_layout(wl):
    """The weight layout the benchmark uses for a workload's recommended block_m."""
    return (qm.MOE_W_FRAG if qm.moe_recommended_block_m(wl.M, wl.E, wl.top_k) == 16
            else qm.MOE_W_TILED)


@pytest.mark.parametrize("block_m,layout", KERNEL_LAYOUTS, ids=KL_IDS)
@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_routed_small(wl, block_m, layout):
    run_routed(wl, block_m=block_m, full=True, layout=layout)


# One k-stage per tile (K = 128 for one-byte activations, K = 64 for bf16)
# with several tiles per workgroup: the tile GEMM's copies then run whole
# tiles ahead of the tile being computed (its routing-info buffers must not
# be reused before that tile's epilogue).
ONE_STAGE = [synth.small("fp8", 4096, 128, 4096, 8, 2), synth.small("int8", 4096, 64, 4096, 8, 2),
             synth.small("fp8wo", 4096, 64, 2048, 8, 2, bias_std=1.5),
             synth.small("int8dq", 4096, 128, 2048, 8, 2)]


@pytest.mark.parametrize("layout", [qm.MOE_W_ROWMAJOR, qm.MOE_W_TILED], ids=["rowmajor", "tiled"])
@pytest.mark.parametrize("wl", ONE_STAGE, ids=[w.name for w in ONE_STAGE])
def test_routed_one_stage_tiles(wl, layout):
    run_routed(wl, block_m=128, full=False, n_tok=256, n_col=128, layout=layout)


# int4 weight-only: the streaming kernel only (block_m 16), plain or packed
INT4_SMALL = [
    synth.small("int4wo", 50, 384, 136, 6, 3),
    synth.small("int4wo", 300, 256, 272, 8, 2, bias_std=1.5),   # several passes per expert
    synth.small("int4wo", 40, 128, 48, 1, 1),
    synth.small("int4wo", 1, 128, 64, 8, 2),
    synth.small("int4wo", 60, 256, 136, 8, 2, bias_std=1.5),   # 32 rows per pass, several
    synth.small("int4wo", 100, 128, 200, 64, 6),                 # many experts
]


@pytest.mark.parametrize("layout", [qm.MOE_W_ROWMAJOR, qm.MOE_W_FRAG], ids=["rowmajor", "frag"])
@pytest.mark.parametrize("wl", INT4_SMALL, ids=[w.name for w in INT4_SMALL])
def test_routed_int4(wl, layout):
    run_routed(wl, block_m=16, full=True, layout=layout)


@pytest.mark.parametrize("block_m,layout", KERNEL_LAYOUTS, ids=KL_IDS)
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_routed_all_tokens_one_expert(fmt, block_m, layout):
    wl = synth.small(fmt, 150, 256, 80, 8, 2)
    lg = torch.randn(150, 8, generator=torch.Generator().manual_seed(5))
    lg[:, 3] += 100.0                        # every token picks expert 3 first
    run_routed(wl, block_m=block_m, full=True, logits=lg, layout=layout)


# the routing limits: the most experts and the largest top_k the library takes
LIMITS = [synth.small("fp8", 300, 128, 64, qm.MOE_MAX_EXPERTS, qm.MOE_MAX_TOPK),
          synth.small("int8", 70, 128, 64, qm.MOE_MAX_EXPERTS, qm.MOE_MAX_TOPK)]


@pytest.mark.parametrize("block_m", [16, 128])
@pytest.mark.parametrize("wl", LIMITS, ids=[w.name for w in LIMITS])
def test_routed_limits(wl, block_m):
    run_routed(wl, block_m=block_m, full=True, layout=qm.MOE_W_ROWMAJOR)


@pytest.mark.parametrize("block_m", [16, 128])
def test_routed_tied_logits(block_m):
    """All logits equal: the lower expert index wins every tie, router
    weights are 1/top_k."""
    wl = synth.small("fp8", 90, 128, 64, 8, 3)
    run_routed(wl, block_m=block_m, full=True, logits=torch.zeros(90, 8))


def _tied_logits(M, E, seed):
    """Small-integer logits (many exact ties, and ties that a larger value
    displaces down the top-k list), plus the rows [5, 3, 3, 4, ...] and
    [1, 1, 2, ...] that need a tied entry carried past a larger one."""
    g = torch.Generator().manual_seed(seed)
    lg = torch.randint(0, 4, (M, E), generator=g).to(torch.float32)
    lg[0, :] = 0.0
    lg[0, :4] = torch.tensor([5.0, 3.0, 3.0, 4.0])
    if M > 1:
        lg[1, :] = 0.0
        lg[1, :3] = torch.tensor([1.0, 1.0, 2.0])
    if M > 2:
        lg[2, :] = -1.0                      # one row of equal values
    return lg.contiguous()


# token counts on both sides of the split between the one-workgroup routing
# and the routing grid (above 1024 tokens)
TIE_CASES = [(M, E, k) for M in (300, 2500) for E in (8, 16, 128)
             for k in range(1, 9) if k <= E]


@pytest.mark.parametrize("block_m", [16, 128])
@pytest.mark.parametrize("M,E,top_k", TIE_CASES, ids=[f"m{M}_e{E}_k{k}" for M, E, k in TIE_CASES])
def test_route_tied_integer_logits(M, E, top_k, block_m):
    """Integer-valued router logits: the expert choice follows (value
    descending, expert ascending) bit-exactly, with the sorted slots, block
    labels and padded length bit-exact as well."""
    _announce(f"tied logits M={M} E={E} top_k={top_k} block_m={block_m}")
    lg = _tied_logits(M, E, synth.seed_of(f"ties {M} {E} {top_k}") % (1 << 31))
    moe = runner.RoutedMoE("fp8", M, 128, 64, E, top_k, block_m=block_m)
    moe.route(lg.to(DEV))
    torch.cuda.synchronize()
    ids_ref, w_ref = O.route_topk(lg.numpy(), top_k)
    np.testing.assert_array_equal(moe.topk_ids.cpu().numpy(), ids_ref)
    wts = moe.topk_weights.cpu().numpy()
    np.testing.assert_allclose(wts, w_ref, rtol=8 * F32_EPS, atol=1e-44)
    assert np.max(np.abs(wts.astype(np.float64).sum(1) - 1.0)) <= 4 * F32_EPS
    s_ref, e_ref, n_ref = O.align_block_size(ids_ref, E, block_m)
    assert int(moe.num_tokens_post_padded.item()) == n_ref
    np.testing.assert_array_equal(moe.sorted_token_ids.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(moe.expert_ids.cpu().numpy(), e_ref)


@pytest.mark.parametrize("block_m", [16, 128])
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_routed_integer_logits_end_to_end(fmt, block_m):
    """The whole layer with tied integer logits (top_k 3): routing, GEMM and
    combine against the oracle."""
    wl = synth.small(fmt, 200, 256, 96, 8, 3)
    run_routed(wl, block_m=block_m, full=True, logits=_tied_logits(200, 8, 77))


@pytest.mark.parametrize("block_m", [16, 128])
def test_align_most_slots(block_m):
    """The largest slot count (M * top_k = MOE_MAX_SLOTS): routing and block
    alignment bit-exact against the oracle."""
    _announce(f"align M*top_k = {qm.MOE_MAX_SLOTS} block_m={block_m}")
    E, top_k = 8, 2
    M = qm.MOE_MAX_SLOTS // top_k
    lg = synth.make_logits(M, E, synth.seed_of("most slots"), 0.5, DEV)
    moe = runner.RoutedMoE("fp8", M, 128, 64, E, top_k, block_m=block_m)
    moe.route(lg)
    torch.cuda.synchronize()
    ids_ref, _ = O.route_topk(lg.cpu().numpy(), top_k)
    np.testing.assert_array_equal(moe.topk_ids.cpu().numpy(), ids_ref)
    s_ref, e_ref, n_ref = O.align_block_size(ids_ref, E, block_m)
    assert int(moe.num_tokens_post_padded.item()) == n_ref
    np.testing.assert_array_equal(moe.sorted_token_ids.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(moe.expert_ids.cpu().numpy(), e_ref)


@pytest.mark.parametrize("M,E,top_k", [(1025, 8, 2), (3000, qm.MOE_MAX_EXPERTS, qm.MOE_MAX_TOPK),
                                         (5000, 4, 1), (2048, 16, 5)])
def test_route_many_tokens(M, E, top_k):
    """Above 1024 tokens the top-k choice runs on its own grid before the
    alignment: expert ids and block layout bit-exact, router weights within
    a few float32 units, for several top_k specialisations."""
    _announce(f"route M={M} E={E} top_k={top_k}")
    lg = synth.make_logits(M, E, synth.seed_of(f"route {M} {E} {top_k}"), 0.5, DEV)
    moe = runner.RoutedMoE("fp8", M, 128, 64, E, top_k, block_m=128)
    moe.route(lg)
    torch.cuda.synchronize()
    ids_ref, w_ref = O.route_topk(lg.cpu().numpy(), top_k)
    np.testing.assert_array_equal(moe.topk_ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(moe.topk_weights.cpu().numpy(), w_ref, rtol=1e-6, atol=1e-7)
    s_ref, e_ref, n_ref = O.align_block_size(ids_ref, E, 128)
    assert int(moe.num_tokens_post_padded.item()) == n_ref
    np.testing.assert_array_equal(moe.sorted_token_ids.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(moe.expert_ids.cpu().numpy(), e_ref)


def test_routed_empty_batch():
    _announce("M = 0")
    moe = runner.RoutedMoE("fp8", 0, 128, 64, 8, 2, block_m=16)
    lg = torch.empty(0, 8, device=DEV)
    moe.route(lg)
    torch.cuda.synchronize()
    assert int(moe.num_tokens_post_padded.item()) == 0
    assert torch.all(moe.sorted_token_ids == 0)          # the sentinel M*top_k = 0
    assert torch.all(moe.expert_ids == -1)
    w_q, w_s = runner.quantize_weights(torch.randn(8, 64, 128, device=DEV), "fp8")
    # a GEMM and a combine with M = 0 are no-ops
    qm.moe_grouped_gemm_fp8w8a8(moe.a_q, moe.a_scale, w_q, w_s, qm.MOE_W_ROWMAJOR,
                                moe.sorted_token_ids,
                                moe.expert_ids, moe.num_tokens_post_padded, moe.topk_weights, 0,
                                128, 64, 8, 2, 16, moe.y)
    qm.moe_combine(moe.y, 0, 64, 2, moe.out)
    torch.cuda.synchronize()


def test_routed_deterministic():
    wl = synth.small("fp8", 300, 384, 320, 8, 2, bias_std=1.5)
    case = synth.make_case(wl, 0, device=DEV)
    for bm in (16, 128):
        _announce(f"determinism block_m={bm}")
        moe = runner.RoutedMoE("fp8", wl.M, wl.K, wl.N, wl.E, wl.top_k, block_m=bm)
        w_q, w_s = runner.quantize_weights(case["w"], "fp8")
        moe.forward(case["x"], case["logits"], w_q, w_s)
        y1, o1 = moe.y.clone(), moe.out.clone()
        moe.y.fill_(0x7FC0)
        moe.forward(case["x"], case["logits"], w_q, w_s)
        torch.cuda.synchronize()
        assert torch.equal(y1, moe.y)
        assert torch.equal(o1, moe.out)


FULL = [synth.WORKLOADS[n] for n in [
    "int8dq_m64_k4096_n14336", "int8dq_bias_m4096_k4096_n14336",
    "int8w8a16_m64_k4096_n14336",
    "fp8wo_m64_k4096_n14336", "fp8wo_bias_m4096_k4096_n14336", "int4wo_m64_k4096_n14336",
    "fp8_bias_m128_k4096_n14336", "fp8_bias_m512_k4096_n14336",
    "fp8_bias_m1024_k4096_n14336", "fp8_bias_m4096_k4096_n14336",
    "mistral7b_up_fp8_m4096_k4096_n28672", "mistral7b_down_fp8_m4096_k14336_n4096",
    "mistral7b_up_int8_m4096_k4096_n28672", "mistral7b_down_int8_m4096_k14336_n4096",
]]


@pytest.mark.parametrize("wl", FULL, ids=[w.name for w in FULL])
def test_routed_full_size_sampled(wl):
    """The benchmark's launch configuration: recommended block_m, packed weights
    (128 tokens and 192 columns per case)."""
    run_routed(wl, block_m=None, full=False, n_tok=128, n_col=192, layout=bench_layout(wl))
    torch.cuda.empty_cache()


ROWMAJOR_FULL = [synth.WORKLOADS[n] for n in [
    "int8dq_m64_k4096_n14336", "int8dq_bias_m4096_k4096_n14336", "int8w8a16_m64_k4096_n14336",
    "fp8wo_m64_k4096_n14336", "int4wo_m64_k4096_n14336", "fp8_bias_m128_k4096_n14336",
    "fp8_bias_m4096_k4096_n14336",
    "mistral7b_down_int8_m4096_k14336_n4096",
]]


@pytest.mark.parametrize("wl", ROWMAJOR_FULL, ids=[w.name for w in ROWMAJOR_FULL])
def test_routed_full_size_sampled_rowmajor(wl):
    run_routed(wl, block_m=None, full=False, layout=qm.MOE_W_ROWMAJOR)
    torch.cuda.empty_cache()


def _pack_frag_reference(w, N, K):
    """The MOE_W_FRAG layout as its definition states it (numpy)."""
    E = w.shape[0]
    J, B = -(-N // 16), -(-K // 64)
    pad = np.zeros((E, J * 16, B * 64), np.uint8)
    pad[:, :N, :K] = w
    # [e, j, r, b, q, i] (n = 16j + r, k = 64b + 16q + i) -> [e, b, j, q, r, i]
    return pad.reshape(E, J, 16, B, 4, 16).transpose(0, 3, 1, 4, 2, 5).reshape(-1)


def _pack_reference(w, N, K):
    """The MOE_W_TILED layout as its definition states it (numpy)."""
    E = w.shape[0]
    T, S = -(-N // 64), -(-K // 128)
    pad = np.zeros((E, T * 64, S * 128), np.uint8)
    pad[:, :N, :K] = w
    blocks = pad.reshape(E, T, 64, S, 128).transpose(0, 1, 3, 2, 4)        # [E,T,S,64,128]
    r = np.arange(64)[:, None]
    pos = np.arange(8)[None, :]
    src = pos ^ ((r >> 1) & 7)                                             # chunk stored at pos
    chunks = blocks.reshape(E, T, S, 64, 8, 16)
    out = np.take_along_axis(chunks, np.broadcast_to(src[None, None, None, :, :, None], chunks.shape), axis=4)
    return out.reshape(-1)


@pytest.mark.parametrize("E,N,K", [(2, 64, 128), (3, 200, 320), (1, 17, 48), (8, 256, 4096)])
def test_pack_weights_layout(E, N, K):
    _announce(f"pack E={E} N={N} K={K}")
    g = torch.Generator(device=DEV).manual_seed(E * 1000 + N + K)
    w = torch.randint(0, 256, (E, N, K), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    p = runner.pack_weights(w, qm.MOE_W_TILED)
    f = runner.pack_weights(w, qm.MOE_W_FRAG)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(p.cpu().numpy(), _pack_reference(w.cpu().numpy(), N, K))
    np.testing.assert_array_equal(f.cpu().numpy(), _pack_frag_reference(w.cpu().numpy(), N, K))


# ----------------------------------------------------------------------------
# MXFP8
# ----------------------------------------------------------------------------
def run_mx(wl, full=True, n_row=64, n_col=64):
    _announce(f"{wl.name} full={full}")
    case = synth.make_case(wl, 0, device=DEV)
    x, w, mo = case["x"], case["w"], case["m_offsets"]
    R, K, N, E = wl.M, wl.K, wl.N, wl.E
    moe = runner.MxMoE(R, K, N, E)
    w_q, w_sf = runner.quantize_weights(w, "mxfp8")
    moe.a_sf.fill_(0xAB)
    moe.out.fill_(0x7FC0)
    moe.forward(x, mo, w_q, w_sf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(synth.seed_of(wl.name, 98) % (1 << 32))
    mo_np = mo.cpu().numpy().astype(np.int64)
    po = O.mx_padded_offsets(mo_np)
    x_np = bits16(x)
    rows = np.arange(R) if full else pick(R, n_row, rng, must=tuple(mo_np[:-1]) + (R - 1,))
    cols = np.arange(N) if full else pick(N, n_col, rng, must=(0, N - 1))

    # activations: bit-exact data and padded scales
    a_sf = moe.a_sf.cpu().numpy()
    if full:
        q_ref, sf_ref = O.quantize_act_mxfp8(x_np, mo_np)
        np.testing.assert_array_equal(moe.a_q.cpu().numpy(), q_ref)
        np.testing.assert_array_equal(a_sf[:po[-1]], sf_ref)
    q_rows, b_rows = O.quantize_mxfp8_rows(F.bf16_decode(x_np[rows]).astype(np.float32))
    np.testing.assert_array_equal(moe.a_q.cpu().numpy()[rows], q_rows)
    e_of = np.searchsorted(mo_np, rows, side="right") - 1
    np.testing.assert_array_equal(a_sf[po[e_of] + rows - mo_np[e_of]], b_rows)
    for e in range(E):                       # pad rows of every expert's block are zero
        assert np.all(a_sf[po[e] + (mo_np[e + 1] - mo_np[e]):po[e + 1]] == 0)

    # weights: bit-exact on the checked rows
    wq_rows, wsf_rows = oracle_weights_rows(w, "mxfp8", cols)
    ct = torch.as_tensor(cols, device=DEV)
    np.testing.assert_array_equal(w_q.index_select(1, ct).cpu().numpy(), wq_rows)
    np.testing.assert_array_equal(w_sf.index_select(1, ct).cpu().numpy(), wsf_rows)

    # GEMM output
    aq_full = np.zeros((R, K), np.uint8)
    aq_full[rows] = q_rows
    asf_full = np.zeros((int(po[-1]), K // 32), np.uint8)
    asf_full[po[e_of] + rows - mo_np[e_of]] = b_rows
    wq_full = np.zeros((E, N, K), np.uint8)
    wq_full[:, cols] = wq_rows
    wsf_full = np.zeros((E, N, K // 32), np.uint8)
    wsf_full[:, cols] = wsf_rows
    out_ref = O.grouped_gemm_mxfp8(aq_full, asf_full, wq_full, wsf_full, mo_np, rows, cols)
    out_gpu = bits16(moe.out)[np.ix_(rows, cols)]
    ref32 = F.bf16_decode(out_ref)
    assert_close_rms(F.bf16_decode(out_gpu), ref32, f"{wl.name} out")
    assert_bf16_out(out_gpu, ref32, out_ref, f"{wl.name} out")


MX_SMALL = [synth.small("mxfp8", 0, 256, 136, 0, 1, seg=(5, 130, 0, 77)),
            # many experts, several empty
            synth.small("mxfp8", 0, 128, 72, 0, 1,
                        seg=(0, 3, 129, 0, 0, 256, 1, 40, 0, 300, 7, 0, 0, 2, 128, 0)),
            synth.small("mxfp8", 0, 128, 64, 0, 1, seg=(128, 128)),
            synth.small("mxfp8", 0, 384, 16, 0, 1, seg=(1,))]


@pytest.mark.parametrize("wl", MX_SMALL, ids=[w.name for w in MX_SMALL])
def test_mxfp8_small(wl):
    run_mx(wl, full=True)


MX_FULL = [synth.WORKLOADS["mxfp8_8x4000_k4096_n4096"], synth.WORKLOADS["mxfp8_22b_8x4000_k6144_n32768"]]


@pytest.mark.parametrize("wl", MX_FULL, ids=[w.name for w in MX_FULL])
def test_mxfp8_full_size_sampled(wl):
    run_mx(wl, full=False)
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# fused activation + quantization (SwiGLU / SReLU -> MXFP8 or per-tensor fp8)
# ----------------------------------------------------------------------------
# SwiGLU is evaluated in float32 on the device with the device exp, so its
# float32 value may differ from the oracle's correctly rounded one by a few
# units: the check allows, per element, the codes of every value within a
# relative ACT_EPS of the exact activation (and per block or tensor the scales
# of the amax within ACT_EPS), and reports how many codes differ from the
# oracle's.  SReLU of bf16 inputs is exact in float32 and compared bit-exactly.
ACT_EPS = 2.0 ** -19
ACT_NAMES = {O.ACT_SWIGLU: "swiglu", O.ACT_SRELU: "srelu"}


def _act_run(x, rows, H, act, mode, mo=None, E=1):
    q = torch.full((rows, H), 0x5A, dtype=torch.uint8, device=DEV)
    s = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    sf = ws = None
    if mode == qm.MOE_Q_MXFP8:
        n_sf = qm.moe_mx_scale_rows(rows, E)
        sf = torch.full((max(n_sf, 1), H // 32), 0xA5, dtype=torch.uint8, device=DEV)
    else:
        ws = torch.empty(qm.moe_quantize_workspace_bytes(mode, 1), dtype=torch.uint8, device=DEV)
    qm.moe_act_quantize(x, rows, H, act, mode, mo, E, q, s, sf, ws)
    torch.cuda.synchronize()
    return q, s, sf


def _code_bounds(scaled64):
    """Decoded e4m3 values of the lowest and highest codes of the values within
    a relative ACT_EPS of scaled64 (the encoder is monotone)."""
    a = scaled64 * (1.0 - ACT_EPS)
    b = scaled64 * (1.0 + ACT_EPS)
    lo, hi = np.minimum(a, b), np.maximum(a, b)
    return F.e4m3_decode(F.e4m3_encode(lo)), F.e4m3_decode(F.e4m3_encode(hi))


def _check_codes(q, scaled64, what):
    got = F.e4m3_decode(q)
    lo, hi = _code_bounds(scaled64)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), f"{what}: {int(bad.sum())} codes outside the allowed range"


def _check_act_mx(x_bits, mo_np, act, q, sf, rows_sel, what):
    """MXFP8 of the activation on the rows rows_sel (all rows of a small
    case, sampled rows of a large one) and every pad row of the scales."""
    H = q.shape[1]
    po = O.mx_padded_offsets(mo_np)
    e_of = np.searchsorted(mo_np, rows_sel, side="right") - 1
    sf_rows = po[e_of] + rows_sel - mo_np[e_of]
    q_ref, sf_ref = O.act_quantize_mxfp8(x_bits[rows_sel], np.array([0, rows_sel.size]), act)
    sf_ref = sf_ref[:rows_sel.size]
    q_got, sf_got = q[rows_sel], sf[sf_rows]
    pad = np.zeros(sf.shape[0], bool)          # rows past po[-1] are not the kernel's
    pad[:po[-1]] = True
    for e in range(len(mo_np) - 1):
        pad[po[e]:po[e] + mo_np[e + 1] - mo_np[e]] = False
    assert not sf[pad].any(), f"{what}: nonzero scale bytes on pad rows"
    if act == O.ACT_SRELU:
        np.testing.assert_array_equal(sf_got, sf_ref, err_msg=f"{what} scales")
        np.testing.assert_array_equal(q_got, q_ref, err_msg=f"{what} codes")
        return
    y = O.act_values(x_bits[rows_sel], act)
    blk = y.reshape(rows_sel.size, H // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    b_lo = O.mx_scale_byte(np.float32(amax * (1 - ACT_EPS)))
    b_hi = O.mx_scale_byte(np.float32(amax * (1 + ACT_EPS)))
    assert np.all((sf_got >= b_lo) & (sf_got <= b_hi)), f"{what}: scale bytes out of range"
    scaled = blk * np.ldexp(1.0, 127 - sf_got.astype(np.int64))[..., None]
    _check_codes(q_got.reshape(blk.shape), scaled, what)
    print(f"  {what}: {np.mean(q_got != q_ref):.2e} of codes, {np.mean(sf_got != sf_ref):.2e} "
          f"of scale bytes differ from the oracle's", flush=True)


def _act_amax(x_bits, act, chunk=4096):
    """max |activation| over every row, in float64, a chunk of rows at a time."""
    return max((float(np.max(np.abs(O.act_values(x_bits[i:i + chunk], act))))
                for i in range(0, len(x_bits), chunk)), default=0.0)


def _check_act_fp8(x_bits, act, q, s, rows_sel, what):
    """Per-tensor fp8 of the activation: the scale from the amax over every row,
    the codes on rows_sel (every row of a small case)."""
    s_got = np.float32(s.item())
    if act == O.ACT_SRELU and rows_sel.size == len(x_bits):
        q_ref, s_ref = O.act_quantize_fp8(x_bits, act)
        assert s_got == s_ref, (what, s_got, s_ref)
        np.testing.assert_array_equal(q, q_ref, err_msg=f"{what} codes")
        return
    amax = _act_amax(x_bits, act)
    y = O.act_values(x_bits[rows_sel], act)
    if act == O.ACT_SRELU:                       # exact: the amax is a float32 value
        s_ref = O.fp8_tensor_scale(np.float32(amax))
        assert s_got == s_ref, (what, s_got, s_ref)
        np.testing.assert_array_equal(q[rows_sel], O.fp8_quantize_with_scale(y.astype(np.float32), s_ref),
                                      err_msg=f"{what} codes")
        return
    s_lo = O.fp8_tensor_scale(np.float32(amax * (1 - ACT_EPS)))
    s_hi = O.fp8_tensor_scale(np.float32(amax * (1 + ACT_EPS)))
    assert s_lo <= s_got <= s_hi, (what, s_got, s_lo, s_hi)
    inv = float(np.float32(np.float32(1.0) / s_got))
    _check_codes(q[rows_sel], y * inv, what)
    q_ref = O.fp8_quantize_with_scale(y.astype(np.float32), s_got)
    print(f"  {what}: {np.mean(q[rows_sel] != q_ref):.2e} of codes differ from the oracle's "
          f"(same scale)", flush=True)


ACT_MX_SMALL = [((5, 130, 0, 77), 256, 1.0), ((128,), 64, 30.0), ((1,), 2048, 3.0),
                ((0, 0, 3), 32, 1.0)]


@pytest.mark.parametrize("act", [O.ACT_SWIGLU, O.ACT_SRELU], ids=["swiglu", "srelu"])
@pytest.mark.parametrize("seg,H,std", ACT_MX_SMALL,
                         ids=[f"s{'-'.join(map(str, c[0]))}_h{c[1]}" for c in ACT_MX_SMALL])
def test_act_quantize_mxfp8_small(act, seg, H, std):
    what = f"act {ACT_NAMES[act]} mxfp8 seg={seg} H={H}"
    _announce(what)
    rows, E = sum(seg), len(seg)
    width = 2 * H if act == O.ACT_SWIGLU else H
    x = synth.make_act_input(rows, width, synth.seed_of(what), std)
    mo = synth.make_segments(seg)
    q, _, sf = _act_run(x.to(DEV), rows, H, act, qm.MOE_Q_MXFP8, mo.to(DEV), E)
    _check_act_mx(bits16(x), mo.numpy().astype(np.int64), act, q.cpu().numpy(),
                  sf.cpu().numpy(), np.arange(rows), what)


def test_act_quantize_srelu_tiny_and_huge_inputs():
    """SReLU of inputs whose squares are float32 subnormals or near the top of
    the range: the scale byte comes from the exponent field (0 for a
    subnormal amax) and the codes stay exact."""
    _announce("act srelu mxfp8 extreme magnitudes")
    H, rows = 64, 4
    v = np.array([1e-20, 3e-22, -1e-20, 2e-19, 1e18, -1e18, 1.5e19, 0.0], np.float32)
    x = torch.from_numpy(np.resize(v, rows * H).reshape(rows, H).copy()).to(torch.bfloat16)
    x[0, :32] = torch.tensor(3e-21)              # a block of subnormal squares only
    mo = synth.make_segments((rows,))
    q, _, sf = _act_run(x.to(DEV), rows, H, O.ACT_SRELU, qm.MOE_Q_MXFP8, mo.to(DEV), 1)
    _check_act_mx(bits16(x), mo.numpy().astype(np.int64), O.ACT_SRELU, q.cpu().numpy(),
                  sf.cpu().numpy(), np.arange(rows), "srelu extremes")


ACT_FP8_SMALL = [(333, 1024, 1.0), (7, 8, 30.0), (64, 128, 1e-3)]


@pytest.mark.parametrize("act", [O.ACT_SWIGLU, O.ACT_SRELU], ids=["swiglu", "srelu"])
@pytest.mark.parametrize("rows,H,std", ACT_FP8_SMALL, ids=[f"r{c[0]}_h{c[1]}" for c in ACT_FP8_SMALL])
def test_act_quantize_fp8_small(act, rows, H, std):
    what = f"act {ACT_NAMES[act]} fp8 rows={rows} H={H}"
    _announce(what)
    width = 2 * H if act == O.ACT_SWIGLU else H
    x = synth.make_act_input(rows, width, synth.seed_of(what), std)
    q, s, _ = _act_run(x.to(DEV), rows, H, act, qm.MOE_Q_FP8_PER_TENSOR)
    _check_act_fp8(bits16(x), act, q.cpu().numpy(), s, np.arange(rows), what)


def test_act_quantize_empty():
    _announce("act quantize, zero rows")
    x = torch.zeros(1, 64, dtype=torch.bfloat16, device=DEV)
    for mode in (qm.MOE_Q_MXFP8, qm.MOE_Q_FP8_PER_TENSOR):
        mo = torch.zeros(3, dtype=torch.int32, device=DEV)
        q, s, sf = _act_run(x, 0, 32, O.ACT_SWIGLU, mode, mo, 2)
        assert s.item() == -1.0                  # nothing written


@pytest.mark.parametrize("act", [O.ACT_SWIGLU, O.ACT_SRELU], ids=["swiglu", "srelu"])
@pytest.mark.parametrize("mode", [qm.MOE_Q_MXFP8, qm.MOE_Q_FP8_PER_TENSOR], ids=["mxfp8", "fp8"])
def test_act_quantize_full_size_sampled(act, mode):
    """The activation between the up (N = 2H = 4096) and the down projection
    of the 8 x 4000-row MXFP8 layer: 32000 rows, H = 2048; sampled rows (the
    per-tensor scale from the amax over every row)."""
    wl = synth.WORKLOADS["mxfp8_8x4000_k4096_n4096"]
    H = wl.N // 2 if act == O.ACT_SWIGLU else wl.N
    rows = wl.M
    what = f"act {ACT_NAMES[act]} {'mxfp8' if mode == qm.MOE_Q_MXFP8 else 'fp8'} {rows}x{H}"
    _announce(what)
    x = synth.make_act_input(rows, wl.N, synth.seed_of(what), 1.0)
    mo = synth.make_segments(wl.seg)
    q, s, sf = _act_run(x.to(DEV), rows, H, act, mode, mo.to(DEV), wl.E)
    rng = np.random.default_rng(7)
    mo_np = mo.numpy().astype(np.int64)
    rows_sel = pick(rows, 96, rng, must=[0, rows - 1, *mo_np[1:-1], *(mo_np[1:-1] - 1)])
    x_bits = bits16(x)
    if mode == qm.MOE_Q_MXFP8:
        _check_act_mx(x_bits, mo_np, act, q.cpu().numpy(), sf.cpu().numpy(), rows_sel, what)
    else:
        _check_act_fp8(x_bits, act, q.cpu().numpy(), s, rows_sel, what)
    del x, q, sf
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# a whole expert FFN: up projection -> fused SwiGLU + quantization -> down
# projection (the chaining of the up and down GEMMs through the activation)
# ----------------------------------------------------------------------------
def test_expert_ffn_mxfp8_chain():
    """MXFP8 (no router): x -> MXFP8 -> up GEMM [rows, 2H] bf16 -> SwiGLU +
    MXFP8 (per-expert padded scales) -> down GEMM [rows, N2] bf16.  Checked
    stage by stage through the chained buffers: the up projection against the
    oracle's, and the output against the oracle's activation + down
    projection of the device's own up-projection rows.  No end-to-end bar
    against the oracle's separate chain: a bf16 unit of difference in an
    intermediate value can move an e4m3 code or a block scale of the
    re-quantized activation, so the two chains may legitimately differ by
    more than the per-stage bound."""
    seg, K, H, N2 = (100, 37, 0, 200), 256, 128, 192
    what = f"ffn mxfp8 seg={seg} K={K} H={H} N2={N2}"
    _announce(what)
    rows, E = sum(seg), len(seg)
    s0 = synth.seed_of(what)
    x = synth.make_act_input(rows, K, s0)
    w1 = synth.make_weights(E, 2 * H, K, s0 + 1)
    w2 = synth.make_weights(E, N2, H, s0 + 2)
    mo = synth.make_segments(seg)
    # device chain
    up = runner.MxMoE(rows, K, 2 * H, E)
    w1q, w1s = runner.quantize_weights(w1.to(DEV), "mxfp8")
    w2q, w2s = runner.quantize_weights(w2.to(DEV), "mxfp8")
    mo_d = mo.to(DEV)
    y1 = up.forward(x.to(DEV), mo_d, w1q, w1s)
    act = runner.ActQuant(rows, H, E, "swiglu", "mxfp8")
    q2 = act(y1, mo_d)
    out = torch.empty(rows, N2, dtype=torch.int16, device=DEV)
    qm.moe_grouped_gemm_mxfp8(q2, act.sf, w2q, w2s, mo_d, rows, H, N2, E, out)
    torch.cuda.synchronize()
    # oracle, stage by stage
    mo_np = mo.numpy().astype(np.int64)
    aq, asf = O.quantize_act_mxfp8(bits16(x), mo_np)
    w1q_r, w1s_r = O.quantize_weight_mxfp8(w1.numpy())
    y1_32 = O.grouped_gemm_mxfp8(aq, asf, w1q_r, w1s_r, mo_np, as_float32=True)
    y1_ref = F.bf16_round(y1_32)
    y1_gpu = bits16(y1)
    assert_bf16_out(y1_gpu, y1_32, y1_ref, what + " up")
    w2q_r, w2s_r = O.quantize_weight_mxfp8(w2.numpy())
    q2_r, sf2_r = O.act_quantize_mxfp8(y1_gpu, mo_np, O.ACT_SWIGLU)
    q2_g = q2.cpu().numpy()
    sf2_g = act.sf.cpu().numpy()[:sf2_r.shape[0]]
    print(f"  {what}: activation codes differing {np.mean(q2_g != q2_r):.2e}, "
          f"scale bytes differing {np.mean(sf2_g != sf2_r):.2e}", flush=True)
    # the oracle's float32 result: the device's output is its bf16 rounding
    ref32 = O.grouped_gemm_mxfp8(q2_r, sf2_r, w2q_r, w2s_r, mo_np, as_float32=True)
    assert_bf16_out(bits16(out), ref32, F.bf16_round(ref32), what + " down")


def test_expert_ffn_fp8_routed_chain():
    """Routed fp8: route -> fp8 x -> up GEMM per slot (router weight 1) ->
    SwiGLU + fp8 per tensor over the slots -> down GEMM per slot (M' = M *
    top_k rows, top_k' = 1: a slot is its own row, the router weight applied
    here) -> combine.  Checked stage by stage as the MXFP8 chain."""
    M, K, H, N2, E, top_k = 96, 256, 128, 160, 4, 2
    what = f"ffn fp8 routed M={M} K={K} H={H} N2={N2} E={E}"
    _announce(what)
    s0 = synth.seed_of(what)
    x = synth.make_act_input(M, K, s0)
    lg = synth.make_logits(M, E, s0 + 3)
    w1 = synth.make_weights(E, 2 * H, K, s0 + 1)
    w2 = synth.make_weights(E, N2, H, s0 + 2)
    S = M * top_k
    moe = runner.RoutedMoE("fp8", M, K, 2 * H, E, top_k, block_m=16)
    w1q, w1s = runner.quantize_weights(w1.to(DEV), "fp8")
    w2q, w2s = runner.quantize_weights(w2.to(DEV), "fp8")
    moe.route(lg.to(DEV))
    moe.quantize(x.to(DEV))
    ones = torch.ones(M, top_k, dtype=torch.float32, device=DEV)
    qm.moe_grouped_gemm_fp8w8a8(moe.a_q, moe.a_scale, w1q, w1s, qm.MOE_W_ROWMAJOR,
                                moe.sorted_token_ids, moe.expert_ids, moe.num_tokens_post_padded,
                                ones, M, K, 2 * H, E, top_k, moe.block_m, moe.y)
    act = runner.ActQuant(S, H, 1, "swiglu", "fp8")
    q2 = act(moe.y)
    y2 = torch.empty(S, N2, dtype=torch.int16, device=DEV)
    qm.moe_grouped_gemm_fp8w8a8(q2, act.scale, w2q, w2s, qm.MOE_W_ROWMAJOR,
                                moe.sorted_token_ids, moe.expert_ids, moe.num_tokens_post_padded,
                                moe.topk_weights, S, H, N2, E, 1, moe.block_m, y2)
    out = torch.empty(M, N2, dtype=torch.int16, device=DEV)
    qm.moe_combine(y2, M, N2, top_k, out)
    torch.cuda.synchronize()
    # oracle, stage by stage (routing choices are bit-exact, so the oracle's
    # ids are the device's; its router weights are used on its side)
    ids, wts = O.route_topk(lg.numpy(), top_k)
    np.testing.assert_array_equal(moe.topk_ids.cpu().numpy(), ids)
    aq, sa = O.quantize_act_fp8(bits16(x))
    w1q_r, w1s_r = O.quantize_weight_fp8(w1.numpy())
    y1_32 = O.grouped_gemm_fp8w8a8(aq, sa, w1q_r, w1s_r, ids, np.ones_like(wts))
    y1_gpu = bits16(moe.y)
    assert_bf16_out(y1_gpu, y1_32, O.slot_results_bf16(y1_32), what + " up")
    q2_r, s2_r = O.act_quantize_fp8(y1_gpu, O.ACT_SWIGLU)
    w2q_r, w2s_r = O.quantize_weight_fp8(w2.numpy())
    y2_r = O.grouped_gemm_fp8w8a8(q2_r, s2_r, w2q_r, w2s_r, ids.reshape(-1, 1), wts.reshape(-1, 1))
    out32, out_ref = O.combine(F.bf16_decode(O.slot_results_bf16(y2_r)), top_k)
    assert_bf16_out(bits16(out), out32, out_ref, what + " down")


# ----------------------------------------------------------------------------
# codecs through the library
# ----------------------------------------------------------------------------
def _structured_values():
    hi = np.arange(1 << 17, dtype=np.uint64) << 15
    lows = np.array([0, 1, 0x3FFF, 0x4000, 0x4001, 0x7FFF], dtype=np.uint64)
    bits = (hi[:, None] | lows[None, :]).reshape(-1).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    rnd = np.random.default_rng(1).uniform(-448, 448, size=1 << 20).astype(np.float32)
    return np.concatenate([v, rnd, np.array([448.0], np.float32)])


def test_fp8_encoder_structured_values():
    """Weights whose largest magnitude is 448 have scale 1, so the fp8 weight
    quantizer returns e4m3(w) for every value: all rounding decisions of the
    device conversion against the oracle's encoder."""
    _announce("e4m3 encoder")
    v = _structured_values()
    K = 512
    n = -(-v.size // K) * K
    vals = np.zeros(n, np.float32)
    vals[:v.size] = v
    vals[-1] = 448.0
    w = torch.from_numpy(vals.reshape(1, n // K, K)).to(DEV)
    q, s = runner.quantize_weights(w, "fp8")
    torch.cuda.synchronize()
    assert s.item() == 1.0
    np.testing.assert_array_equal(q.cpu().numpy().reshape(-1), F.e4m3_encode(vals))


def test_int8_quantizer_full():
    _announce("int8 quantizer")
    w = torch.randn(3, 40, 256, device=DEV) * torch.tensor([1.0, 1e-3, 50.0], device=DEV)[:, None, None]
    w[1, 7] = 0.0
    q, s = runner.quantize_weights(w, "int8")
    torch.cuda.synchronize()
    q_ref, s_ref = O.quantize_weight_int8(w.cpu().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)


def test_fp8_activation_quantizer_full():
    _announce("fp8 activation quantizer")
    for M, K, scale in [(64, 128, 1.0), (333, 1024, 3e-3), (7, 8, 1e4)]:
        x = (torch.randn(M, K, device=DEV) * scale).to(torch.bfloat16)
        q = torch.empty(M, K, dtype=torch.uint8, device=DEV)
        s = torch.empty(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(qm.moe_quantize_workspace_bytes(qm.MOE_Q_FP8_PER_TENSOR, 1), dtype=torch.uint8, device=DEV)
        qm.moe_quantize_act(x, M, K, qm.MOE_Q_FP8_PER_TENSOR, None, 1, q, s, None, ws)
        torch.cuda.synchronize()
        q_ref, s_ref = O.quantize_act_fp8(bits16(x))
        assert s.item() == float(s_ref)
        np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def test_combine_bit_exact():
    _announce("combine")
    rng = np.random.default_rng(3)
    for M, N, top_k in [(64, 256, 2), (37, 104, 3), (5, 8, 1), (128, 4096, 8)]:
        y = rng.standard_normal((M * top_k, N)).astype(np.float32)
        # rounding ties and binade edges of bf16
        special = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.99999,
                            65504.0, 1e-40, -0.0, 2.0 ** -126] * 8, np.float32)
        n = min(special.size, y.size)
        y.reshape(-1)[:n] = special[:n]
        y_bits = F.bf16_round(y)                  # the per-slot results are bf16
        out = torch.empty(M, N, dtype=torch.int16, device=DEV)
        qm.moe_combine(torch.from_numpy(y_bits.view(np.int16)).to(DEV), M, N, top_k, out)
        torch.cuda.synchronize()
        _, ref = O.combine(F.bf16_decode(y_bits), top_k)
        np.testing.assert_array_equal(bits16(out), ref)
