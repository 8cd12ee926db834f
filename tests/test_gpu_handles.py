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
