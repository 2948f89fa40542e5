"""The allocation-free activation quantizer (moe_quantize_act_noalloc, its
partial maxima in the library's static device scratch) against the workspace
form (moe_quantize_act): codes and scale bit-exact, on two calls in a row,
the second smaller (the scratch keeps the first call's partials), and in a
HIP graph replayed several times."""

import numpy as np
import pytest
import torch

import quantized_moe_grouped_top_amd as qm
from quantized_moe_grouped_top_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _quantize_pair(x, rows, K):
    q_ws = torch.empty(rows, K, dtype=torch.uint8, device=DEV)
    s_ws = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(qm.moe_quantize_workspace_bytes(qm.MOE_Q_FP8_PER_TENSOR, 1),
                     dtype=torch.uint8, device=DEV)
    qm.moe_quantize_act(x, rows, K, qm.MOE_Q_FP8_PER_TENSOR, None, 1, q_ws, s_ws, None, ws)
    q_na = torch.full((rows, K), 0xAB, dtype=torch.uint8, device=DEV)
    s_na = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    qm.moe_quantize_act_noalloc(x, rows, K, qm.MOE_Q_FP8_PER_TENSOR, None, 1, q_na, s_na, None)
    torch.cuda.synchronize()
    return q_ws, s_ws, q_na, s_na


@pytest.mark.parametrize("first,second", [((4096, 4096), (64, 4096)), ((3000, 512), (7, 256))])
def test_noalloc_matches_workspace_form(first, second):
    print(f"\n[no-alloc] fp8 per tensor {first} then {second}", flush=True)
    for i, (rows, K) in enumerate((first, second)):
        # the first input's largest magnitude is far above the second's, so a
        # partial maximum left in the scratch would show in the second scale
        x = synth.make_act_input(rows, K, synth.seed_of(f"noalloc {rows} {K}"),
                                 std=4.0 if i == 0 else 0.25, device=DEV)
        q_ws, s_ws, q_na, s_na = _quantize_pair(x, rows, K)
        assert s_na.item() == s_ws.item()
        np.testing.assert_array_equal(q_na.cpu().numpy(), q_ws.cpu().numpy())


def test_noalloc_in_graph_replays():
    print("\n[no-alloc] graph capture, 4 replays", flush=True)
    rows, K = 1024, 2048
    x = synth.make_act_input(rows, K, synth.seed_of("noalloc graph"), device=DEV)
    q_ref, s_ref, _, _ = _quantize_pair(x, rows, K)        # also resolves the scratch address
    q = torch.zeros(rows, K, dtype=torch.uint8, device=DEV)
    s = torch.zeros(1, dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            qm.moe_quantize_act_noalloc(x, rows, K, qm.MOE_Q_FP8_PER_TENSOR, None, 1, q, s, None)
    for _ in range(4):
        q.fill_(0xAB)
        s.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert s.item() == s_ref.item()
        np.testing.assert_array_equal(q.cpu().numpy(), q_ref.cpu().numpy())
