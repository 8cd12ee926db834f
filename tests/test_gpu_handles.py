"""Separate handles are independent (include/moe_decode.h, thread safety):
each owns its workspace, so calls of different handles may be queued back to
back on one stream or run at once on several streams. Every output must be
bit-identical to the same handle's call run alone: the kernels take no
decision from another handle's state.
"""

from __future__ import annotations

import pytest
import torch

import synth
from fp8_block_scaled_moe_amd import MoeDecode

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

SHAPES = [
    # persistent GEMMs (few tokens)
    synth.CONFIGS["tiny"].with_(M=6, hidden=1024, inter=512, experts=16, top_k=4),
    # one workgroup per unit (more than 8 tokens, K > 1024)
    synth.CONFIGS["tiny"].with_(M=12, hidden=2048, inter=1536, experts=10, top_k=3),
    # the FP4 form on a local share
    synth.CONFIGS["fp4_share"].with_(M=5, hidden=512, inter=256, experts=24, top_k=3, local_begin=6,
                                     local_count=12),
]


def make(inp):
    s = inp.shape
    extra = dict(ue8m0_act=s.ue8m0_act)
    if s.weight_format == "fp4":
        extra = dict(weight_format="nvfp4", experts=s.experts, local_begin=s.local_begin)
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=s.M, logits_dtype=inp.logits.dtype, **extra)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.fixture(scope="module")
def cases():
    out = []
    for i, shape in enumerate(SHAPES):
        inp = synth.make_inputs(shape, seed=70 + i, device=DEV)
        moe = make(inp)
        ref = moe(inp.x, inp.logits, inp.bias)  # alone, then synchronised
        torch.cuda.synchronize()
        out.append((inp, moe, [t.clone() for t in ref]))
    return out


def check(got, ref):
    for name, a, b in zip(("slots", "ids", "weights", "combined"), got, ref):
        assert torch.equal(bits(a), bits(b)), name


def test_handles_back_to_back_on_one_stream(cases):
    outs = []
    for _ in range(3):
        for inp, moe, _ in cases:
            outs.append(moe(inp.x, inp.logits, inp.bias))
    torch.cuda.synchronize()
    for n, got in enumerate(outs):
        check(got, cases[n % len(cases)][2])


def test_handles_on_separate_streams(cases):
    streams = [torch.cuda.Stream() for _ in cases]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        for (inp, moe, _), s in zip(cases, streams):
            with torch.cuda.stream(s):
                outs.append(moe(inp.x, inp.logits, inp.bias, stream=s))
    torch.cuda.synchronize()
    for n, got in enumerate(outs):
        check(got, cases[n % len(cases)][2])


def test_timed_runs_change_nothing_and_time_each_kernel(cases):
    """Per-kernel timing (moe_decode_set_timing): outputs stay bit-identical,
    every launched kernel has a positive time, a slot whose work ran inside a
    GEMM launch reads 0, and the kernels' times add up to less than the
    layer's (the events take each dispatch's own timestamps)."""
    for inp, moe, ref in cases:
        layer = []
        for mode_timing in (False, True):
            moe.set_timing(mode_timing)
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                got = moe(inp.x, inp.logits, inp.bias)
                b.record()
                torch.cuda.synchronize()
                check(got, ref)
                if mode_timing:
                    ms = moe.last_timing()
                    assert all(t > 0 for t in (ms[0], ms[1], ms[3])), ms
                    assert all(t >= 0 for t in ms), ms
                    layer.append((sum(ms), a.elapsed_time(b)))
        moe.set_timing(False)
        # the events around the call add their own markers, so the layer's
        # span bounds the kernels' sum
        assert all(s < span for s, span in layer), layer


def test_timing_of_fused_launches():
    """With the SwiGLU inside GEMM1 and the combine inside GEMM2, their slots
    read 0 and the GEMM slots carry the time."""
    inp = synth.make_inputs(SHAPES[0], seed=77, device=DEV)
    for mode, zero in (("swiglu_in_gemm1", 2), ("combine_in_gemm2", 4)):
        s = inp.shape
        moe = MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                        routed_scale=s.routed_scale, max_tokens=s.M, logits_dtype=inp.logits.dtype,
                        ue8m0_act=s.ue8m0_act, launch_mode=mode)
        ref = [t.clone() for t in moe(inp.x, inp.logits, inp.bias)]
        moe.set_timing(True)
        got = moe(inp.x, inp.logits, inp.bias)
        torch.cuda.synchronize()
        ms = moe.last_timing()
        check(got, ref)
        assert ms[zero] == 0 and ms[1] > 0 and ms[3] > 0, (mode, ms)
        moe.close()
