"""One layer call captured into a HIP graph and replayed.

moe_decode_run allocates nothing, waits on nothing from the host, and its
kernels clear the counters they use, so a call can be recorded into a graph
on torch's capture stream. A replay reads the inputs at the addresses
captured, so each replay here first writes a new draw of x, logits and bias
into those buffers. The replay runs the same kernels in the same launch
shapes as an eager call of the same token count, so every output must be
bit-identical to an eager call on the same inputs. Eager calls on the same
handle run between the replays (they leave other routes and counters in the
workspace), and each graph is replayed several times.
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
REPLAYS = 4

DSV3_32 = synth.CONFIGS["dsv3"].with_(experts=32)  # DeepSeek-V3 expert shapes, fewer experts
CASES = {
    # K = 1024 for both GEMMs: persistent workgroups at any token count
    "small_m9": (synth.CONFIGS["tiny"].with_(M=9, hidden=1024, inter=1024, experts=6, top_k=3), {}),
    # 4 tokens: persistent GEMMs, jobs built by the routing kernel
    "dsv3_m4": (DSV3_32, {}),
    # 16 tokens at K = 7168: one workgroup per unit
    "dsv3_m16": (DSV3_32.with_(M=16), {}),
    "combine_in_gemm2": (DSV3_32, dict(launch_mode="combine_in_gemm2")),
    "swiglu_in_gemm1": (DSV3_32, dict(launch_mode="swiglu_in_gemm1")),
    # routing inside the GEMM1 launch: the default at one token, asked for at two
    "route_in_gemm1_m1": (DSV3_32.with_(M=1), {}),
    "route_in_gemm1_m2": (DSV3_32.with_(M=2), dict(launch_mode="route_in_gemm1")),
    "shared_expert": (synth.CONFIGS["tiny"].with_(M=5, hidden=512, inter=256, experts=12, top_k=3,
                                                  shared_inter=384), {}),
    "fp4_share": (synth.CONFIGS["fp4_share"].with_(M=5, hidden=512, inter=256, experts=24, top_k=3,
                                                   local_begin=6, local_count=12), {}),
}


def make(inp, **kw):
    s = inp.shape
    extra = {}
    if s.shared_inter:
        extra = dict(sw13=inp.sw13, sw13_scale=inp.sw13_scale, sw2=inp.sw2, sw2_scale=inp.sw2_scale,
                     shared_limit=s.shared_limit, shared_ue8m0_act=True)
    if s.weight_format == "fp4":
        extra = dict(weight_format="nvfp4", experts=s.experts, local_begin=s.local_begin)
    else:
        extra["ue8m0_act"] = s.ue8m0_act
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=s.M, logits_dtype=inp.logits.dtype,
                     **extra, **kw)


class Buffers:
    """Inputs and outputs at fixed addresses, as a captured graph needs."""

    def __init__(self, moe, inp):
        s = inp.shape
        self.x, self.logits, self.bias = inp.x.clone(), inp.logits.clone(), inp.bias.clone()
        self.out = list(moe.outputs(s.M))
        self.shared_out = None
        if s.shared_inter:
            self.shared_out = torch.empty((s.M, s.hidden), dtype=torch.bfloat16, device=DEV)

    def run(self, moe, stream=None):
        moe.run_into(self.x, self.logits, self.bias, *self.out, shared_out=self.shared_out, stream=stream)

    def outputs(self):
        return self.out + ([self.shared_out] if self.shared_out is not None else [])


def redraw(bufs, inp, gen):
    """A new input draw in place: rows of x permuted with random signs (the
    values stay those of the workload's recipe), fresh logits and bias."""
    M = inp.shape.M
    perm = torch.randperm(M, generator=gen, device=DEV)
    sign = torch.where(torch.rand(M, 1, generator=gen, device=DEV) < 0.5, -1.0, 1.0)
    bufs.x.copy_((inp.x[perm].float() * sign).to(torch.bfloat16))
    bufs.logits.copy_((torch.randn(bufs.logits.shape, generator=gen, device=DEV)
                       * inp.shape.logits_std).to(bufs.logits.dtype))
    bufs.bias.copy_(torch.randn(bufs.bias.shape, generator=gen, device=DEV) * inp.shape.bias_std)


def as_bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replay_equals_eager(case):
    shape, kw = CASES[case]
    inp = synth.make_inputs(shape, seed=61, device=DEV)
    moe = make(inp, **kw)
    static = Buffers(moe, inp)
    eager = Buffers(moe, inp)

    # first call outside the capture: kernels loaded, handle state settled
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        static.run(moe)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static.run(moe)

    gen = torch.Generator(device=DEV).manual_seed(62)
    routes = set()
    for _ in range(REPLAYS):
        redraw(static, inp, gen)
        for a, b in ((eager.x, static.x), (eager.logits, static.logits), (eager.bias, static.bias)):
            a.copy_(b)
        for t in static.outputs() + eager.outputs():
            as_bits(t).fill_(-1)  # a NaN pattern in BF16: an output left unwritten shows
        graph.replay()
        torch.cuda.synchronize()
        eager.run(moe)
        torch.cuda.synchronize()
        names = ("slots", "ids", "weights", "combined", "shared_out")
        for n, a, b in zip(names, static.outputs(), eager.outputs()):
            assert torch.equal(as_bits(a), as_bits(b)), f"{case}: {n} differs after a replay"
        routes.add(tuple(static.out[1].flatten().tolist()))
    assert len(routes) == REPLAYS, "each draw should route differently"

    if case == "small_m9":  # the replayed layer against the oracle as well
        probe = synth.MoeInputs(shape=shape, seed=61, x=static.x, logits=static.logits, bias=static.bias,
                                w13=inp.w13, w13_scale=inp.w13_scale, w2=inp.w2, w2_scale=inp.w2_scale)
        ref = oracle_layer(probe)
        slots, ids, weights, combined = static.out
        assert np.array_equal(ids.cpu().numpy(), ref["ids"])
        assert_rows_close(host(slots), ref["slots"], what="slots")
        assert_rows_close(host(combined), ref["combined"], what="combined")
