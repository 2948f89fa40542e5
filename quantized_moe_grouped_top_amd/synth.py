"""Seeded synthetic inputs for the quantized MoE grouped GEMM workloads.

This module only draws random tensors with the shapes and value distributions
of the workloads; it holds none of the method's arithmetic (no routing, no
quantization, no contraction).  The tests feed the same tensors to the HIP
library and to the CPU oracle; ``bench.py`` uses it to build its inputs.

Workloads (shapes from the (M, K, N, E, top_k) columns of the FP8_W8A8 and
INT8_W8A16 tables on "Tianxing/moe quantization" and the (8*4000, 4096) MXFP8
input of "[PyTorch] Let GroupedLinear accept MXFP8 input and gradient"):

* activations x: bf16 [M, K], entries N(0, 1) rounded to bf16;
* expert weights W: float32 [E, N, K], entries N(0, 1/sqrt(K)) (std), to be
  quantized by the library (offline step) or by the oracle;
* router logits: float32 [M, E], entries N(0, 1), optionally plus a per-expert
  bias N(0, 0.5) that makes the expert loads unbalanced;
* MXFP8 grouped linear: rows concatenated by expert, equal segments;
* fused activation + quantization (the step between the up and the down
  projection): bf16 [rows, 2H] (SwiGLU) or [rows, H] (SReLU) entries N(0, 1),
  rows concatenated by expert as for the MXFP8 grouped linear.
"""

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str               # "fp8", "int8" (W8A16), "int8dq" (W8A8, per-token activation
                           # scales), "fp8wo" (bf16 x fp8 per-channel weights),
                           # "int4wo" (bf16 x int4 per-channel weights),
                           # "mxfp8", "mxfp8_dgrad", "mxfp8_wgrad" (its
                           # backward); "act_mxfp8", "act_fp8" (K = input
                           # width 2H or H, N = H)
    M: int                 # tokens (MXFP8: total rows)
    K: int
    N: int
    E: int = 8
    top_k: int = 2
    bias_std: float = 0.0  # std of the per-expert logit bias
    seg: tuple = field(default=())  # MXFP8 rows per expert
    act: str = ""          # fused activation workloads: "swiglu" or "srelu"

    @property
    def routed_rows(self):
        return self.M if self.fmt.startswith("mxfp8") else self.M * self.top_k

    @property
    def flops(self):
        return 2 * self.routed_rows * self.K * self.N


def _mx(name, rows_per_expert, E, K, N):
    return Workload(name, "mxfp8", rows_per_expert * E, K, N, E=E, top_k=1,
                    seg=tuple([rows_per_expert] * E))


def _act(act, mode, rows_per_expert, E, H):
    width = 2 * H if act == "swiglu" else H
    return Workload(f"{act}_{mode}_{E}x{rows_per_expert}_h{H}", f"act_{mode}", rows_per_expert * E,
                    width, H, E=E, top_k=1, seg=tuple([rows_per_expert] * E), act=act)


WORKLOADS = {w.name: w for w in [
    Workload("fp8_m64_k128_n256", "fp8", 64, 128, 256),
    Workload("int8w8a16_m64_k4096_n14336", "int8", 64, 4096, 14336),
    *[Workload(f"fp8_bias_m{m}_k4096_n14336", "fp8", m, 4096, 14336, bias_std=0.5)
      for m in (128, 512, 1024, 4096)],
    Workload("mistral7b_up_fp8_m4096_k4096_n28672", "fp8", 4096, 4096, 28672),
    Workload("mistral7b_down_fp8_m4096_k14336_n4096", "fp8", 4096, 14336, 4096),
    Workload("mistral7b_up_int8_m4096_k4096_n28672", "int8", 4096, 4096, 28672),
    Workload("mistral7b_down_int8_m4096_k14336_n4096", "int8", 4096, 14336, 4096),
    # int8 W8A8 with dynamic per-token activation scales, at the decode and
    # the M=4096 shapes of the INT8 / FP8 tables
    Workload("int8dq_m64_k4096_n14336", "int8dq", 64, 4096, 14336),
    Workload("int8dq_bias_m4096_k4096_n14336", "int8dq", 4096, 4096, 14336, bias_std=0.5),
    # bf16 activations x fp8 weights with per-channel scales, same shapes
    Workload("fp8wo_m64_k4096_n14336", "fp8wo", 64, 4096, 14336),
    Workload("fp8wo_bias_m4096_k4096_n14336", "fp8wo", 4096, 4096, 14336, bias_std=0.5),
    # bf16 activations x int4 weights with per-channel scales, decode shape
    Workload("int4wo_m64_k4096_n14336", "int4wo", 64, 4096, 14336),
    _mx("mxfp8_8x4000_k4096_n4096", 4000, 8, 4096, 4096),
    _mx("mxfp8_22b_8x4000_k6144_n32768", 4000, 8, 6144, 32768),
    # the backward of the (8*4000, 4096) grouped linear: input gradient
    # (dy [rows, N] x W) and weight gradient (dy^T x per expert), K = N = 4096
    Workload("mxfp8_dgrad_8x4000_k4096_n4096", "mxfp8_dgrad", 32000, 4096, 4096, E=8, top_k=1,
             seg=tuple([4000] * 8)),
    Workload("mxfp8_wgrad_8x4000_k4096_n4096", "mxfp8_wgrad", 32000, 4096, 4096, E=8, top_k=1,
             seg=tuple([4000] * 8)),
    # the (8*4000, 4096) activation input: SwiGLU halves it to H = 2048
    _act("swiglu", "mxfp8", 4000, 8, 2048),
    _act("srelu", "mxfp8", 4000, 8, 4096),
    _act("swiglu", "fp8", 4000, 8, 2048),
    _act("srelu", "fp8", 4000, 8, 4096),
]}


def seed_of(name, variant=0):
    """Stable 63-bit seed of a workload name and variant number."""
    h = 1469598103934665603
    for ch in f"{name}/{variant}".encode():
        h = ((h ^ ch) * 1099511628211) & ((1 << 63) - 1)
    return h


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_activations(M, K, seed, device="cpu"):
    """bf16 [M, K], N(0, 1)."""
    g = _gen(device, seed)
    return torch.randn(M, K, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_act_input(rows, width, seed, std=1.0, device="cpu"):
    """bf16 [rows, width], N(0, std^2): the input of the activation between
    the up and the down projection ([rows, 2H] for SwiGLU, [rows, H] else)."""
    g = _gen(device, seed)
    x = torch.randn(rows, width, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(torch.bfloat16)


def make_weights(E, N, K, seed, device="cpu"):
    """float32 [E, N, K], N(0, 1/sqrt(K)); drawn one expert at a time so the
    values do not depend on how much memory is free."""
    g = _gen(device, seed)
    w = torch.empty(E, N, K, device=device, dtype=torch.float32)
    for e in range(E):
        w[e].normal_(0.0, 1.0 / K ** 0.5, generator=g)
    return w


def make_logits(M, E, seed, bias_std=0.0, device="cpu"):
    """float32 [M, E], N(0, 1) plus (optionally) a per-expert N(0, bias_std)."""
    g = _gen(device, seed)
    lg = torch.randn(M, E, generator=g, device=device, dtype=torch.float32)
    if bias_std:
        lg = lg + bias_std * torch.randn(E, generator=g, device=device, dtype=torch.float32)
    return lg.contiguous()


def make_segments(seg, device="cpu"):
    """int32 [E+1] row offsets of expert-concatenated segments."""
    off = [0]
    for s in seg:
        off.append(off[-1] + int(s))
    return torch.tensor(off, dtype=torch.int32, device=device)


def make_case(wl, variant=0, device="cpu"):
    """All inputs of one workload: dict of x, w, logits (routed formats) or
    x, w, m_offsets (MXFP8)."""
    s = seed_of(wl.name, variant)
    if wl.fmt.startswith("act_"):
        return {"x": make_act_input(wl.M, wl.K, s + 1, 1.0, device),
                "m_offsets": make_segments(wl.seg, device)}
    case = {
        "x": make_activations(wl.M, wl.K, s + 1, device),
        "w": make_weights(wl.E, wl.N, wl.K, s + 2, device),
    }
    if wl.fmt.startswith("mxfp8"):
        case["m_offsets"] = make_segments(wl.seg, device)
        if wl.fmt != "mxfp8":            # backward: the output gradient [M, N]
            case["dy"] = make_act_input(wl.M, wl.N, s + 4, 0.5, device)
    else:
        case["logits"] = make_logits(wl.M, wl.E, s + 3, wl.bias_std, device)
    return case


def small(fmt, M, K, N, E, top_k, bias_std=0.0, seg=()):
    """An ad-hoc workload (parity cases at sizes the oracle finishes quickly)."""
    name = f"{fmt}_m{M}_k{K}_n{N}_e{E}_t{top_k}" + (f"_s{'-'.join(map(str, seg))}" if seg else "")
    if fmt == "mxfp8":
        return Workload(name, fmt, sum(seg), K, N, E=len(seg), top_k=1, seg=tuple(seg))
    return Workload(name, fmt, M, K, N, E=E, top_k=top_k, bias_std=bias_std)
