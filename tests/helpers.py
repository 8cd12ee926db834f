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


def assert_rows_close(got, ref, rtol=ROW_RTOL, what="rows", valid=None):
    """Every row within rtol x the RMS of the oracle's row (max |err|).

    valid(rows) -> bool [len(rows), cols], optional: which elements of those
    rows are the correct BF16 rounding of a valid FP32 result of the GPU's own
    inputs to the step (rounding_valid below). A BF16 output has two correct
    values when its exact value lies within the FP32 accumulation bound of the
    midpoint between two BF16 numbers (the summation order is not fixed by the
    pages); an element that is valid and one BF16 step from the oracle's is
    then no error. It is only consulted for rows over the bar."""
    got = np.asarray(got, np.float64).reshape(np.shape(ref)[0], -1)
    ref = np.asarray(ref, np.float64).reshape(np.shape(ref)[0], -1)
    e = row_errors(got, ref)
    bad = np.nonzero(e > rtol)[0]
    if bad.size and valid is not None:
        ok = valid(bad)
        step = bf16_step(np.maximum(np.abs(got[bad]), np.abs(ref[bad])))
        tie = ok & (np.abs(got[bad] - ref[bad]) <= step)
        g = np.where(tie, ref[bad], got[bad])
        e = e.copy()
        e[bad] = row_errors(g, ref[bad])
        bad = np.nonzero(e > rtol)[0]
    assert bad.size == 0, f"{what}: {bad.size} rows over {rtol} x rms (worst {e.max():.3g} at row {int(e.argmax())})"
    return float(e.max()) if e.size else 0.0


def rounding_valid(got_bf16, exact, bound):
    """got is bf16(v) for some v with |v - exact| <= bound (BF16 rounding of
    FP32 values is monotone, so the valid outputs are the interval between the
    roundings of exact - bound and exact + bound)."""
    lo = oracle.bf16_round(exact - bound)
    hi = oracle.bf16_round(exact + bound)
    return (got_bf16 >= lo) & (got_bf16 <= hi)


def bf16_step(v):
    """Spacing of BF16 values at |v| (the smallest normal spacing below 2**-126)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0**-126))
    return np.ldexp(1.0, e - 8)


FP32_U = 2.0**-24


def combine_bound(slots, weights):
    """Error bound of a k-term FP32 multiply-add chain: gamma_k * sum |w * slot|
    (gamma_k = k u / (1 - k u), u = 2**-24), per combined element."""
    w = np.asarray(weights, np.float64)
    M, k = w.shape
    rows = np.abs(np.asarray(slots, np.float64)).reshape(M, k, -1)
    gamma = k * FP32_U / (1 - k * FP32_U)
    return gamma * np.einsum("tk,tkh->th", np.abs(w), rows)


def check_combine(slots, weights, combined, max_differ=1e-3):
    """The GPU's combine against the oracle's combine of the GPU's own slot rows
    and weights: every element the BF16 rounding of a value within the FP32
    summation bound of the exact weighted sum (within one BF16 step of it
    beyond that bound), and bit-exact on all but max_differ of the elements.
    Rounding the weights, or applying them twice or not at all, fails."""
    got = host(combined)
    s, w = host(slots), host(weights)
    exact = np.einsum("tk,tkh->th", w, s.reshape(w.shape[0], w.shape[1], -1))
    want = oracle.combine(s, w)
    diff = got != want
    ok = rounding_valid(got, exact, combine_bound(s, w))
    assert ok.all(), f"combine: {np.count_nonzero(~ok)} elements not a rounding of the FP32 sum"
    assert diff.mean() <= max_differ, f"combine: {diff.mean():.3%} of elements differ"
