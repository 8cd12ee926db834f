"""Routing and the x quantisation inside the persistent GEMM1 launch
(MOE_LAUNCH_ROUTE_IN_GEMM1: at most 2 tokens and 64 routes) against the
five-launch form.

Every GEMM1 workgroup routes the tokens, groups their routes into jobs and
stages x as FP8 codes with the routing kernel's own functions, so the picks,
weights, buckets, codes and every sum must be bit-identical to the form with
a routing launch of its own, which test_gpu_parity.py holds to the oracle;
one case here also goes through the oracle directly ("mega_moe" page, module
docstring: routing redone per warp instead of a kernel boundary). Outputs
are pre-filled with a NaN pattern so that anything workgroup 0 fails to
write shows up.
"""

from __future__ import annotations

import pytest
import torch

import synth
from fp8_block_scaled_moe_amd import MoeDecode
from tests.test_gpu_parity import full_check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NAN_BF16 = -1  # 0xFFFF


def make(inp, mode, max_tokens=None, **kw):
    s = inp.shape
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=max_tokens or s.M,
                     logits_dtype=inp.logits.dtype, ue8m0_act=s.ue8m0_act, launch_mode=mode, **kw)


def run_filled(moe, inp, M):
    slots, ids, weights, combined = moe.outputs(M)
    for t in (slots, combined):
        t.view(torch.int16).fill_(NAN_BF16)
    ids.fill_(-7)
    weights.fill_(float("nan"))
    moe.run_into(inp.x[:M].contiguous(), inp.logits[:M].contiguous(), inp.bias, slots, ids, weights, combined)
    torch.cuda.synchronize()
    return slots, ids, weights, combined


def staged(moe, M):
    """Every stage a run leaves in the workspace of an FP8 handle without a
    shared expert, trimmed to M tokens."""
    R, H, I = M * moe.top_k, moe.hidden, moe.inter
    sizes = {"ctrl": (3, torch.int32), "x_q": (M * H, torch.uint8), "x_s": (M * H // 128, torch.float32),
             "part1": (R * 2 * I, torch.float32), "h_q": (R * I, torch.uint8),
             "h_s": (R * I // 128, torch.float32), "part2": (R * H, torch.float32)}
    out = {k: moe.stage(k, torch.empty(n, dtype=dt, device=DEV)) for k, (n, dt) in sizes.items()}
    U = int(out["ctrl"][1])
    for k in ("uexp", "uoff", "ucnt"):
        out[k] = moe.stage(k, torch.empty(max(U, 1), dtype=torch.int32, device=DEV))[:U]
    routes = int(out["ucnt"].sum()) if U else 0
    out["routes"] = moe.stage("routes", torch.empty(max(R, 1), dtype=torch.int32, device=DEV))[:routes]
    return out


def same(a, b, what):
    x = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
    y = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
    assert torch.equal(x, y), what


def compare(inp, Ms=(1, 2), **kw):
    """For each M, the fused form (one handle for all M) against the separate
    form: outputs and stages bit-identical, one launch fewer."""
    max_tokens = max(max(Ms), inp.shape.M)
    fused, sep = make(inp, "route_in_gemm1", max_tokens, **kw), make(inp, "separate", max_tokens, **kw)
    for M in Ms:
        fp, sp = fused.plan(M), sep.plan(M)
        assert sp["launches"] == 5 and fp["launches"] == (4 if M <= 2 else 5), (M, fp)
        assert fp["persist1"] > 0, fp
        a, b = run_filled(fused, inp, M), run_filled(sep, inp, M)
        for name, x, y in zip(("slots", "ids", "weights", "combined"), a, b):
            same(x, y, (M, name))
        sa, sb = staged(fused, M), staged(sep, M)
        for name in sa:
            same(sa[name], sb[name], (M, name))
    return fused, sep


def test_route_in_gemm1_dsv3():
    """DeepSeek-V3 shapes (256 experts, top-8) at 1 and 2 tokens, then 4 (a
    routing launch again, M > 2) and 1 on the same handle."""
    inp = synth.make_inputs(synth.CONFIGS["dsv3"], seed=3, device=DEV)
    compare(inp, Ms=(1, 2, 4, 1))


def test_route_in_gemm1_dsv3_against_the_oracle():
    """The fused form at one token through the oracle's full check: picks,
    weights, buckets, x staging bit-exact, GEMM sums within their bound, rows
    within the bar."""
    shape = synth.CONFIGS["dsv3"].with_(M=1)
    inp = synth.make_inputs(shape, seed=11, device=DEV)
    moe = make(inp, "route_in_gemm1")
    assert moe.plan(1)["launches"] == 4
    full_check(moe, inp)


@pytest.mark.parametrize("experts,top_k,hidden", [(1024, 32, 3072), (384, 6, 2048), (64, 8, 1024), (8, 3, 512)],
                         ids=["E1024_k32", "E384_k6", "E64_k8", "E8_k3"])
def test_route_in_gemm1_shapes(experts, top_k, hidden):
    """Experts per lane 16 (up to 1024 experts, 64 routes at 2 tokens) and 4,
    partly filled slots, and few experts."""
    shape = synth.CONFIGS["tiny"].with_(M=2, hidden=hidden, inter=512, experts=experts, top_k=top_k)
    compare(synth.make_inputs(shape, seed=60 + top_k, device=DEV))


def test_route_in_gemm1_bf16_logits_ue8m0_and_ties():
    """BF16 logits, power-of-two activation scales, and many equal keys (the
    lower expert wins a tie), including +-inf logits."""
    shape = synth.CONFIGS["tiny"].with_(M=2, hidden=1024, inter=512, experts=96, top_k=8, ue8m0_act=True)
    inp = synth.make_inputs(shape, seed=66, device=DEV)
    lg = inp.logits.float()
    lg[0, ::3] = 1.5
    lg[1, 10:40] = float("inf")
    lg[1, 50:60] = -float("inf")
    inp.logits = lg.to(torch.bfloat16)
    inp.bias.zero_()
    compare(inp)


def test_route_in_gemm1_local_share():
    """A local share (experts 9..11 of 16): routes of other experts take no
    part, a token may have no local pick, and with none at all no unit runs."""
    full = synth.CONFIGS["tiny"].with_(M=2, hidden=384 * 2, inter=256, experts=16, top_k=2)
    inp = synth.make_inputs(full, seed=45, device=DEV)
    for lb, lc, seed_bias in ((9, 3, None), (0, 2, 30.0)):
        sub = synth.MoeInputs(shape=full, seed=45, x=inp.x, logits=inp.logits, bias=inp.bias.clone(),
                              w13=inp.w13[lb:lb + lc].clone(), w13_scale=inp.w13_scale[lb:lb + lc].clone(),
                              w2=inp.w2[lb:lb + lc].clone(), w2_scale=inp.w2_scale[lb:lb + lc].clone())
        if seed_bias is not None:
            sub.bias[lc:] += seed_bias  # every pick lands outside the share
        fused, _ = compare(sub, experts=full.experts, local_begin=lb)
        if seed_bias is not None:
            assert int(staged(fused, 2)["ctrl"][2]) == 0  # no job


def test_route_in_gemm1_timing_slot():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=2, hidden=1024, inter=512, experts=32, top_k=4),
                            seed=67, device=DEV)
    moe = make(inp, "route_in_gemm1")
    moe.set_timing(True)
    run_filled(moe, inp, 2)
    ms = moe.last_timing()
    moe.set_timing(False)
    assert ms[0] == 0 and ms[1] > 0 and ms[2] > 0 and ms[3] > 0 and ms[4] > 0, ms


def test_auto_routes_in_gemm1_at_one_token():
    """MOE_LAUNCH_AUTO takes the routing prologue at one token (measured
    faster) and a routing launch from two tokens on; both bit-identical to
    the separate form."""
    inp = synth.make_inputs(synth.CONFIGS["dsv3"].with_(M=2), seed=5, device=DEV)
    auto, sep = make(inp, "auto"), make(inp, "separate")
    assert auto.plan(1)["launches"] == 4 and auto.plan(2)["launches"] == 5
    for M in (1, 2, 1):
        for name, x, y in zip(("slots", "ids", "weights", "combined"), run_filled(auto, inp, M),
                              run_filled(sep, inp, M)):
            same(x, y, (M, name))
