"""Oracle-side helpers of the GPU parity tests: CPU copies of device tensors and
the oracle's reference values for full or sampled comparisons.  Only the
oracle computes here.

Where the tests feed a device result into an oracle stage they say so: the
combine kernel is also checked bit-exactly against the oracle's combine of the
device's own per-slot results, and the expert-FFN chain tests check each
stage against the oracle applied to that stage's device input (the activation
quantization of the device's up-projection rows, the down projection of the
device's codes), so that each kernel is measured on its own error.  Every
other reference is computed by the oracle from the seeded inputs alone.
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import moe as O

REL_TOL = 2e-2          # max |gpu - ref| <= REL_TOL * rms(ref), per checked output


def bits16(t):
    """uint16 numpy copy of a bf16 / int16 device tensor."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def np32(t):
    return t.float().cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy()


def assert_close_rms(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values (unwritten outputs?)"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    print(f"  {what}: max|gpu-ref|/rms(ref) = {err / rms if rms else 0.0:.3e}", flush=True)
    assert err <= REL_TOL * rms, f"{what}: max|gpu-ref| = {err:.3e} > {REL_TOL} * rms {rms:.3e}"
    return err / rms if rms else 0.0


def _bf16_ordinal(bits):
    """Position of each bf16 value on the number line (adjacent values differ
    by one; +0 and -0 share a position)."""
    b = np.asarray(bits, np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_bf16_out(got_bits, ref32, ref_bits, what):
    """bf16 output check: every value within REL_TOL * rms(ref32) of the
    float32 reference plus half a bf16 unit of the reference (the output's
    own rounding, which alone exceeds REL_TOL * rms for values a few times
    the rms).  Printed beside it, not bounded: the literal figure max|gpu -
    ref32| / rms(ref32); max|gpu - ref_bf16| / rms(ref32) against the oracle's
    own bf16 value (both rounded: they differ by a whole bf16 unit where the
    two float32 results straddle a rounding boundary); and how many values
    differ from the oracle's bf16 value."""
    got = F.bf16_decode(got_bits)
    r32 = np.asarray(ref32, np.float64)
    rms = float(np.sqrt(np.mean(r32 * r32)))
    rb = F.bf16_decode(ref_bits)
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(r32))[1] - 9)
    bad = np.abs(got - r32) > REL_TOL * rms + half_ulp
    assert not bad.any(), f"{what}: {int(bad.sum())} bf16 outputs out of bounds"
    dist = np.abs(_bf16_ordinal(got_bits) - _bf16_ordinal(ref_bits))
    frac = float(np.mean(dist > 0)) if dist.size else 0.0
    literal = float(np.max(np.abs(got - r32))) / rms if rms and got.size else 0.0
    vs_bf16 = float(np.max(np.abs(got - rb))) / rms if rms and got.size else 0.0
    print(f"  {what}: max|gpu-ref32|/rms = {literal:.3e} (literal), "
          f"max|gpu-ref_bf16|/rms = {vs_bf16:.3e}; {frac:.2e} of bf16 outputs differ from the "
          f"oracle's (max {int(dist.max()) if dist.size else 0} units)", flush=True)
    return frac


def pick(n, k, rng, must=()):
    """k distinct indices in [0, n) including `must` (clipped to n)."""
    base = [m for m in must if 0 <= m < n]
    rest = np.setdiff1d(np.arange(n), base)
    k = min(n, k)
    extra = rng.choice(rest, size=max(0, k - len(base)), replace=False) if rest.size else []
    return np.sort(np.unique(np.concatenate([np.asarray(base, np.int64), np.asarray(extra, np.int64)])))


def oracle_weights_rows(w_dev, fmt, cols):
    """Oracle quantization of the weight rows `cols` of every expert.

    Returns (q [E, len(cols), K], scale) where scale is [E] (fp8, from the
    amax of the whole expert matrix), [E, len(cols)] (int8, fp8wo) or the e8m0 bytes
    [E, len(cols), K/32] (MXFP8)."""
    E = w_dev.shape[0]
    cols_t = torch.as_tensor(cols, device=w_dev.device)
    rows = w_dev.index_select(1, cols_t).cpu().numpy()
    if fmt == "fp8":
        s = np.array([O.fp8_tensor_scale(w_dev[e].cpu().numpy()) for e in range(E)], np.float32)
        q = np.stack([O.fp8_quantize_with_scale(rows[e], s[e]) for e in range(E)])
        return q, s
    if fmt in ("int8", "int8dq"):
        return O.quantize_weight_int8(rows)
    if fmt == "fp8wo":
        return O.quantize_weight_fp8_rows(rows)
    if fmt == "int4wo":
        return O.quantize_weight_int4(rows)
    q, b = O.quantize_weight_mxfp8(rows)
    return q, b


def unpack_int4(packed):
    """Codes of MOE_Q_INT4_PER_CHANNEL bytes [..., K/2] -> int8 [..., K], as
    the layout is defined: the 8 codes of k = 8c .. 8c+7 form little-endian
    dword c, code 8c + j stored as q + 8 in bits 4f .. 4f+3, f = (j >> 1) +
    4 (j & 1)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    words = packed.view("<u4").astype(np.int64)                     # [..., K/8]
    out = np.empty(words.shape + (8,), np.int8)
    for j in range(8):
        f = (j >> 1) + 4 * (j & 1)
        out[..., j] = ((words >> (4 * f)) & 0xF) - 8
    return out.reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
