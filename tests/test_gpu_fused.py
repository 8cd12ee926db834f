"""The combine inside the GEMM2 launch (MOE_LAUNCH_COMBINE_IN_GEMM2 on
MOE_GEMM_MFMA) against the same step run as a launch of its own.

Both forms take every arithmetic step in the same precision and order (the
slot is the GEMM output rounded once to BF16, the combine an FP32 sum in pick
order, the routing weights applied once: nvfp4-megamoe-kernel README, slot
representation), so every output must be bit-identical between them; the
separate form is itself held to the oracle by test_gpu_parity.py. Outputs
are pre-filled with a NaN pattern so that a slot or combined value the fused
launch fails to write shows up. The arrival counters must be back at zero
after each call: runs of different token counts (and so different K parts
and column tiles) follow each other on one handle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_block_scaled_moe_amd import MoeDecode
from tests.helpers import assert_rows_close, host, oracle_layer

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NAN_BF16 = -1  # 0xFFFF: a NaN in BF16, never written by either form


def make(inp, separate, max_tokens=None, shared=False, **kw):
    s = inp.shape
    extra = {}
    if shared:
        extra = dict(sw13=inp.sw13, sw13_scale=inp.sw13_scale, sw2=inp.sw2, sw2_scale=inp.sw2_scale,
                     shared_limit=s.shared_limit, shared_ue8m0_act=True)
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=max_tokens or s.M,
                     logits_dtype=inp.logits.dtype, ue8m0_act=s.ue8m0_act, gemm_path="mfma",
                     launch_mode="separate" if separate else "combine_in_gemm2", **extra, **kw)


def run_filled(moe, inp, M, shared=False):
    """Runs the first M tokens into outputs pre-filled with NaN bit patterns."""
    slots, ids, weights, combined = moe.outputs(M)
    for t in (slots, combined):
        t.view(torch.int16).fill_(NAN_BF16)
    so = None
    if shared:
        so = torch.empty((M, moe.hidden), dtype=torch.bfloat16, device=DEV)
        so.view(torch.int16).fill_(NAN_BF16)
    moe.run_into(inp.x[:M].contiguous(), inp.logits[:M].contiguous(), inp.bias, slots, ids, weights,
                 combined, shared_out=so)
    torch.cuda.synchronize()
    out = [slots, ids, weights, combined]
    return out + [so] if shared else out


def assert_same(a, b):
    names = ("slots", "ids", "weights", "combined", "shared_out")
    for n, x, y in zip(names, a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), n


def compare(inp, M=None, shared=False, **kw):
    M = M or inp.shape.M
    fused, sep = make(inp, False, shared=shared, **kw), make(inp, True, shared=shared, **kw)
    assert fused.plan(M)["launches"] == 4 and sep.plan(M)["launches"] == 5
    a, b = run_filled(fused, inp, M, shared), run_filled(sep, inp, M, shared)
    assert_same(a, b)
    return a


@pytest.mark.parametrize("splits2", [0, 1, 2, 4], ids=["auto", "64rows", "32rows", "16rows"])
def test_fused_equals_separate_small(splits2):
    """K parts of GEMM2 forced to 1, 2 and 4 (64, 32 and 16 columns per
    tile), several routes per expert, and the oracle's combined values."""
    shape = synth.CONFIGS["tiny"].with_(M=9, hidden=1024, inter=1024, experts=6, top_k=3)
    inp = synth.make_inputs(shape, seed=41, device=DEV)
    fused = make(inp, False, splits2=splits2)
    assert fused.plan(shape.M)["kparts2"] == (splits2 or fused.plan(shape.M)["kparts2"])
    slots, ids, weights, combined = compare(inp, splits2=splits2)
    ref = oracle_layer(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_rows_close(host(slots), ref["slots"], what="slots")
    assert_rows_close(host(combined), ref["combined"], what="combined")


def test_fused_tiny_one_token():
    compare(synth.make_inputs(synth.CONFIGS["tiny"], seed=0, device=DEV))


def test_fused_skewed_routing():
    """Every token on the same few experts: many arrivals per counter from
    one unit, tokens completed by different workgroups."""
    shape = synth.CONFIGS["tiny"].with_(M=40, hidden=512, inter=256, experts=32, top_k=4)
    inp = synth.make_inputs(shape, seed=42, device=DEV)
    inp.bias[:5] += 20.0  # experts 0..4 win every token's first four picks
    compare(inp)


def test_fused_wide_topk():
    """top_k = 32 (the largest): a tile's combine holds 32 x 64 slot values."""
    shape = synth.CONFIGS["tiny"].with_(M=3, hidden=512, inter=256, experts=40, top_k=32)
    compare(synth.make_inputs(shape, seed=43, device=DEV))


def test_fused_with_shared_expert():
    shape = synth.CONFIGS["tiny"].with_(M=5, hidden=512, inter=256, experts=12, top_k=3, shared_inter=384)
    inp = synth.make_inputs(shape, seed=44, device=DEV)
    compare(inp, shared=True)


def test_fused_local_experts_and_unrouted_tokens():
    """A local share no pick of some tokens falls on: their slot rows and
    combined row must still be written (as zeros) by the fused launch."""
    full = synth.CONFIGS["tiny"].with_(M=12, hidden=384, inter=256, experts=16, top_k=2)
    inp = synth.make_inputs(full, seed=45, device=DEV)
    lb, lc = 9, 3
    w = [t[lb:lb + lc].clone() for t in (inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)]
    outs = []
    for sep in (False, True):
        moe = MoeDecode(*w, top_k=full.top_k, limit=full.limit, routed_scale=full.routed_scale,
                        max_tokens=full.M, experts=full.experts, local_begin=lb,
                        launch_mode="separate" if sep else "combine_in_gemm2")
        outs.append(run_filled(moe, inp, full.M))
    assert_same(*outs)
    ids = outs[0][1].cpu().numpy()
    local = (ids >= lb) & (ids < lb + lc)
    none = ~local.any(axis=1)
    assert none.any() and local.any(), "the seed must give both kinds of token"
    combined = outs[0][3].view(torch.int16).cpu().numpy()
    assert not combined[none].any()
    ref = oracle_layer(inp)
    masked = np.where(local.reshape(-1)[:, None], ref["slots"], 0.0)
    assert_rows_close(host(outs[0][0]), masked, what="slots")
    assert_rows_close(host(outs[0][3]), oracle.combine(masked, ref["weights"]), what="combined")


def test_fused_counters_reset_between_calls():
    """Calls of 7, 2, 7 and 1 tokens on one handle, each bit-identical to the
    separate form. At this shape GEMM2 takes one K part (64 columns per tile)
    with 42 routes and two (32 columns) with 6 or 12, so the counters are
    indexed differently from one call to the next."""
    shape = synth.CONFIGS["tiny"].with_(M=7, hidden=7168, inter=3584, experts=48, top_k=6)
    inp = synth.make_inputs(shape, seed=46, device=DEV)
    fused, sep = make(inp, False), make(inp, True)
    parts = set()
    for M in (7, 2, 7, 1):
        parts.add(fused.plan(M)["kparts2"])
        assert_same(run_filled(fused, inp, M), run_filled(sep, inp, M))
    assert len(parts) > 1, "the sequence should change GEMM2's column tiles"


def test_fused_dsv3_m4():
    """The DeepSeek-V3-shaped layer at 4 tokens, as the benchmark runs it."""
    inp = synth.make_inputs(synth.CONFIGS["dsv3"], seed=0, device=DEV)
    compare(inp)
    compare(inp, M=1)
