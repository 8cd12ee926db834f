"""Glue between the synthetic inputs, the oracle and the comparisons.

Tolerances (from the workload definition): ids bit-exact, routing weights to
1e-6 relative, every BF16 output row within 2e-2 x the RMS of the oracle's
row (max |err| <= 2e-2 * rms).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

ROW_RTOL = 2e-2
WEIGHT_RTOL = 1e-6


def host(t: torch.Tensor) -> np.ndarray:
    """float64 host copy of a tensor of any dtype (bf16/f32 values exact)."""
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.detach().to(torch.float64).cpu().numpy()


def expert_fn(inp):
    """Lazily copies one expert's weights and scales to the host."""
    def get(e: int):
        return (inp.w13[e].cpu().numpy(), host(inp.w13_scale[e]),
                inp.w2[e].cpu().numpy(), host(inp.w2_scale[e]))
    return get


def oracle_layer(inp, **over):
    s = inp.shape
    kw = dict(top_k=s.top_k, routed_scale=s.routed_scale, limit=s.limit,
              ue8m0_act=s.ue8m0_act, inter=s.inter)
    kw.update(over)
    return oracle.moe_decode(host(inp.x), host(inp.logits), host(inp.bias), expert_fn(inp), **kw)


def oracle_layer_fp4(inp, local_begin=None, local_count=None):
    s = inp.shape
    def get(e: int):
        return (inp.w13[e].cpu().numpy(), inp.w13_scale[e].cpu().numpy(),
                inp.w2[e].cpu().numpy(), inp.w2_scale[e].cpu().numpy())
    lb = s.local_begin if local_begin is None else local_begin
    lc = s.local_experts if local_count is None else local_count
    return oracle.fp4.moe_decode_fp4(host(inp.x), host(inp.logits), host(inp.bias), get,
                                     top_k=s.top_k, routed_scale=s.routed_scale, limit=s.limit,
                                     local_begin=lb, local_count=lc, inter=s.inter)


def oracle_shared(inp, ue8m0_act: bool = True):
    s = inp.shape
    return oracle.shared_expert(host(inp.x), inp.sw13.cpu().numpy(), host(inp.sw13_scale),
                                inp.sw2.cpu().numpy(), host(inp.sw2_scale),
                                limit=s.shared_limit, ue8m0_act=ue8m0_act)


def row_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """max |got - ref| / rms(ref) per row (rows of all-zero ref compare to 0)."""
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    err = np.max(np.abs(got - ref), axis=1)
    out = np.where(rms > 0, err / np.where(rms > 0, rms, 1), np.where(err > 0, np.inf, 0.0))
    return out


def assert_rows_close(got, ref, rtol=ROW_RTOL, what="rows"):
    e = row_errors(got, ref)
    bad = np.nonzero(e > rtol)[0]
    assert bad.size == 0, f"{what}: {bad.size} rows over {rtol} x rms (worst {e.max():.3g} at row {int(e.argmax())})"
    return float(e.max()) if e.size else 0.0


def bf16_step(v):
    """Spacing of BF16 values at |v| (the smallest normal spacing below 2**-126)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0**-126))
    return np.ldexp(1.0, e - 8)


def check_combine(slots, weights, combined, max_differ=1e-3):
    """The GPU's combine against the oracle's combine of the GPU's own slot rows
    and weights: within one BF16 step everywhere and bit-exact on all but
    max_differ of the elements (an FP32 sum in another order may round to the
    neighbouring BF16 value). Rounding the weights, or applying them twice or
    not at all, fails."""
    got = host(combined)
    want = oracle.combine(host(slots), host(weights))
    diff = got != want
    step = bf16_step(np.maximum(np.abs(got), np.abs(want)))
    far = np.abs(got - want) > step
    assert not far.any(), f"combine: {far.sum()} elements beyond one BF16 step"
    assert diff.mean() <= max_differ, f"combine: {diff.mean():.3%} of elements differ"
