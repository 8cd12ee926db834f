"""The persistent form of the K-in-workgroup GEMMs (MOE_GEMM_AUTO, where it
applies) against one workgroup per unit (MOE_GEMM_MFMA by name).

Both forms cut the work into the same units (expert, 16-64 weight rows, all
of K) and add every unit's products, K parts and scale factors in the same
order; the persistent form only changes which workgroup takes a unit and
when its loads are requested. So every output and every staged value must be
bit-identical between the two, and the one-unit form is held to the oracle by
test_gpu_parity.py. Covered: K parts 1, 2 and 4 in either GEMM, several units
per workgroup (fewer workgroups than units), one routed expert, eight routes
on one expert, experts with more than 16 routes (several jobs), the full
DeepSeek-V3-shaped layer at 1 and 4 tokens, and calls of different token
counts on one handle. The persistent form is planned for at most 8 tokens, or
any number when K is at most 1024.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from fp8_block_scaled_moe_amd import MoeDecode
from tests.helpers import assert_rows_close, host, oracle_layer

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def make(inp, path, **kw):
    s = inp.shape
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=kw.pop("max_tokens", s.M),
                     logits_dtype=inp.logits.dtype, ue8m0_act=s.ue8m0_act, gemm_path=path, **kw)


def run(moe, inp, M):
    out = moe(inp.x[:M].contiguous(), inp.logits[:M].contiguous(), inp.bias)
    torch.cuda.synchronize()
    return out


def staged(moe, M):
    s = moe.top_k * M
    p1 = moe.stage("part1", torch.empty(s * 2 * moe.inter, dtype=torch.float32, device=DEV))
    p2 = moe.stage("part2", torch.empty(s * moe.hidden, dtype=torch.float32, device=DEV))
    return p1, p2


def compare(inp, M=None, want_persist=(True, True), **kw):
    """The persistent plan at M against the one-unit kernel with the same K
    parts (the persistent plan may take more of them)."""
    M = M or inp.shape.M
    pers = make(inp, "auto", **kw)
    plan = pers.plan(M)
    kw = dict(kw, splits1=plan["kparts1"], splits2=plan["kparts2"])
    one = make(inp, "mfma", **kw)
    assert (plan["persist1"] > 0, plan["persist2"] > 0) == tuple(want_persist), plan
    assert one.plan(M)["persist1"] == 0 and one.plan(M)["persist2"] == 0
    a, b = run(pers, inp, M), run(one, inp, M)
    for name, x, y in zip(("slots", "ids", "weights", "combined"), a, b):
        assert torch.equal(x, y), name
    for name, x, y in zip(("part1", "part2"), staged(pers, M), staged(one, M)):
        assert torch.equal(x, y), name
    return a, plan


@pytest.mark.parametrize("splits", [(0, 0), (1, 1), (2, 2), (4, 4)], ids=["auto", "kp1", "kp2", "kp4"])
def test_persistent_equals_one_unit(splits):
    shape = synth.CONFIGS["tiny"].with_(M=6, hidden=1024, inter=1024, experts=12, top_k=4)
    inp = synth.make_inputs(shape, seed=51, device=DEV)
    (slots, ids, weights, combined), plan = compare(inp, splits1=splits[0], splits2=splits[1])
    ref = oracle_layer(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_rows_close(host(slots), ref["slots"], what="slots")
    assert_rows_close(host(combined), ref["combined"], what="combined")


def test_persistent_single_expert_eight_routes():
    """Eight tokens all on expert 0 (the most routes the plan gives it)."""
    shape = synth.CONFIGS["tiny"].with_(M=8, hidden=512, inter=512, experts=8, top_k=1)
    inp = synth.make_inputs(shape, seed=52, device=DEV)
    inp.bias[0] += 50.0
    compare(inp)


def test_persistent_not_taken_past_eight_tokens():
    """Nine tokens and K = 2048: the one-unit kernel runs (and gives the same
    results)."""
    shape = synth.CONFIGS["tiny"].with_(M=9, hidden=2048, inter=2048, experts=8, top_k=2)
    inp = synth.make_inputs(shape, seed=53, device=DEV)
    compare(inp, want_persist=(False, False))


def test_persistent_short_k_many_tokens_and_jobs():
    """Past 8 tokens a GEMM with K <= 1024 still runs persistent. Forty
    tokens on the same two experts: each has 40 routes, three jobs of at most
    16 (one MFMA pass each), as the one-unit kernel's three passes."""
    shape = synth.CONFIGS["tiny"].with_(M=40, hidden=1024, inter=512, experts=32, top_k=4)
    inp = synth.make_inputs(shape, seed=56, device=DEV)
    inp.bias[:2] += 50.0
    (_, ids, _, _), plan = compare(inp, want_persist=(True, True))
    assert (ids[:, :2].sort(dim=1).values.cpu().numpy() == [0, 1]).all()


def test_persistent_local_share():
    """One GPU's share of the experts (local experts 10..19 of 32): the jobs
    hold local routes only; the other slots stay zero."""
    full = synth.CONFIGS["tiny"].with_(M=7, hidden=1024, inter=512, experts=32, top_k=4)
    inp = synth.make_inputs(full, seed=57, device=DEV)
    lb, lc = 10, 10
    w = [t[lb:lb + lc].clone() for t in (inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)]
    outs = []
    for path in ("auto", "mfma"):
        moe = MoeDecode(*w, top_k=full.top_k, limit=full.limit, routed_scale=full.routed_scale,
                        max_tokens=full.M, experts=full.experts, local_begin=lb, gemm_path=path,
                        splits1=1, splits2=1)
        plan = moe.plan(full.M)
        assert (plan["persist1"] > 0) == (path == "auto") and (plan["persist2"] > 0) == (path == "auto")
        outs.append(run(moe, inp, full.M))
    for name, x, y in zip(("slots", "ids", "weights", "combined"), *outs):
        assert torch.equal(x, y), name
    ids = outs[0][1].cpu().numpy().reshape(-1)
    local = (ids >= lb) & (ids < lb + lc)
    assert local.any() and (~local).any()
    assert not outs[0][0].float().cpu().numpy()[~local].any()
    ref = oracle_layer(inp)
    assert_rows_close(host(outs[0][0])[local], ref["slots"][local], what="slots")


def test_persistent_odd_steps_fall_back():
    """K / 128 = 3 blocks cannot give every wave an even number of steps."""
    shape = synth.CONFIGS["tiny"].with_(M=3, hidden=384, inter=256, experts=6, top_k=2)
    inp = synth.make_inputs(shape, seed=54, device=DEV)
    compare(inp, want_persist=(False, True))


def test_persistent_token_counts_on_one_handle():
    shape = synth.CONFIGS["tiny"].with_(M=9, hidden=2048, inter=1024, experts=32, top_k=6)
    inp = synth.make_inputs(shape, seed=55, device=DEV)
    pers, one = make(inp, "auto", splits1=2, splits2=1), make(inp, "mfma", splits1=2, splits2=1)
    for M in (9, 1, 4, 8, 9):
        for name, x, y in zip(("slots", "ids", "weights", "combined"), run(pers, inp, M), run(one, inp, M)):
            assert torch.equal(x, y), (M, name)


@pytest.fixture(scope="module")
def dsv3_m8():
    return synth.make_inputs(synth.CONFIGS["dsv3"].with_(M=8), seed=0, device=DEV)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_persistent_dsv3(dsv3_m8, M):
    """The DeepSeek-V3-shaped layer: thousands of units on the resident
    workgroups; GEMM1 in 4 K parts (16-row units)."""
    _, plan = compare(dsv3_m8, M=M)
    assert plan["persist1"] < plan["grid1"]  # several units per workgroup
    assert plan["kparts1"] == 4


# -- the SwiGLU inside the persistent GEMM1 launch (MOE_LAUNCH_SWIGLU_IN_GEMM1) --

def make_mode(inp, mode, **kw):
    return make(inp, "auto", launch_mode=mode, **kw)


def swiglu_pair(inp, M, **kw):
    """The same layer with the SwiGLU inside GEMM1 and as its own launch: every
    output and the staged FP8 hidden and its scales bit-identical."""
    fused, sep = make_mode(inp, "swiglu_in_gemm1", **kw), make_mode(inp, "separate", **kw)
    assert fused.plan(M)["launches"] == 4 and sep.plan(M)["launches"] == 5
    for moe in (fused, sep):
        assert moe.plan(M)["persist1"] > 0
    a, b = run(fused, inp, M), run(sep, inp, M)
    for name, x, y in zip(("slots", "ids", "weights", "combined"), a, b):
        assert torch.equal(x, y), name
    R, I = M * inp.shape.top_k, inp.shape.inter
    for st, n, dt in (("h_q", R * I, torch.uint8), ("h_s", R * (I // 128), torch.float32)):
        x = fused.stage(st, torch.empty(n, dtype=dt, device=DEV))
        y = sep.stage(st, torch.empty(n, dtype=dt, device=DEV))
        assert torch.equal(x, y), st
    return fused, sep


@pytest.mark.parametrize("splits1", [1, 2, 4], ids=["64rows", "32rows", "16rows"])
def test_swiglu_in_gemm1_equals_separate(splits1):
    shape = synth.CONFIGS["tiny"].with_(M=6, hidden=1024, inter=512, experts=12, top_k=4)
    inp = synth.make_inputs(shape, seed=58, device=DEV)
    fused, _ = swiglu_pair(inp, shape.M, splits1=splits1)
    assert fused.plan(shape.M)["kparts1"] == splits1
    slots, ids, _, combined = run(fused, inp, shape.M)
    ref = oracle_layer(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_rows_close(host(slots), ref["slots"], what="slots")
    assert_rows_close(host(combined), ref["combined"], what="combined")


def test_swiglu_in_gemm1_counters_reset_and_jobs():
    """Calls of 8, 1, 5 and 8 tokens on one handle (each block's count must
    be back at zero), experts with more than 16 routes (K <= 1024 keeps the
    GEMMs persistent past 8 tokens)."""
    shape = synth.CONFIGS["tiny"].with_(M=40, hidden=1024, inter=512, experts=32, top_k=4)
    inp = synth.make_inputs(shape, seed=59, device=DEV)
    inp.bias[:2] += 50.0
    fused, sep = make_mode(inp, "swiglu_in_gemm1"), make_mode(inp, "separate")
    for M in (8, 1, 40, 5, 40):
        for name, x, y in zip(("slots", "ids", "weights", "combined"), run(fused, inp, M), run(sep, inp, M)):
            assert torch.equal(x, y), (M, name)


def test_swiglu_in_gemm1_dsv3(dsv3_m8):
    for M in (1, 4, 8):
        swiglu_pair(dsv3_m8, M)
