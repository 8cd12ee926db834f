"""The allocation-free entry point (moe_decode_run_noalloc) against the
handle's moe_decode_run: the same launches on a fixed per-GPU buffer, so the
outputs must be bit-identical, on two calls in a row (the second smaller),
and the oracle's bar holds for them. Size and configuration errors are
refused before anything is enqueued."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from fp8_block_scaled_moe_amd import MoeDecode, MoeDecodeError, _capi
from tests.helpers import WEIGHT_RTOL, assert_rows_close, host, oracle_layer

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def make(inp, M, **kw):
    s = inp.shape
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=M, logits_dtype=inp.logits.dtype,
                     ue8m0_act=s.ue8m0_act, **kw)


def both(moe, inp, M, shared=False):
    """(handle outputs, no-allocation outputs) for the first M tokens."""
    x, lg = inp.x[:M].contiguous(), inp.logits[:M].contiguous()
    sh = lambda: torch.full((M, moe.hidden), 3.0, dtype=torch.bfloat16, device=DEV) if shared else None
    a = list(moe.outputs(M)) + [sh()]
    b = [t.clone().fill_(7) for t in moe.outputs(M)] + [sh()]
    moe.run_into(x, lg, inp.bias, *a[:4], shared_out=a[4])
    moe.run_noalloc(x, lg, inp.bias, *b[:4], shared_out=b[4])
    torch.cuda.synchronize()
    return a, b


def assert_same(a, b):
    for u, v in zip(a, b):
        if u is not None:
            assert torch.equal(u, v)


@pytest.mark.parametrize("path", ["auto", "mfma_splitk"])
def test_noalloc_matches_handle_dsv3(path):
    """DeepSeek-V3 shapes: 8 tokens, then 3 on the same buffer, then 1 (with
    the automatic launch shape, routing inside the GEMM1 launch)."""
    inp = synth.make_inputs(synth.CONFIGS["dsv3"].with_(M=8), seed=40, device=DEV)
    moe = make(inp, 8, gemm_path=path)
    for M in (8, 3):
        a, b = both(moe, inp, M)
        assert_same(a, b)
    sub = synth.MoeInputs(shape=inp.shape.with_(M=3), seed=40, x=inp.x[:3], logits=inp.logits[:3],
                          bias=inp.bias, w13=inp.w13, w13_scale=inp.w13_scale, w2=inp.w2,
                          w2_scale=inp.w2_scale)
    ref = oracle_layer(sub)
    assert np.array_equal(b[1].cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(host(b[2]), ref["weights"], rtol=WEIGHT_RTOL, atol=0)
    assert_rows_close(host(b[3]), ref["combined"], what="combined")
    assert moe.plan(1)["launches"] == (4 if path == "auto" else 5)
    assert_same(*both(moe, inp, 1))


@pytest.mark.parametrize("mode", ["separate", "combine_in_gemm2", "swiglu_in_gemm1"])
def test_noalloc_launch_modes_and_shared(mode):
    """Every launch mode (the fused ones count arrivals in the buffer), with
    the shared expert (FP32 scales): 6 tokens, then 2."""
    shape = synth.CONFIGS["tiny"].with_(M=6, hidden=512, inter=256, experts=16, top_k=4, shared_inter=256)
    inp = synth.make_inputs(shape, seed=41, device=DEV)
    moe = make(inp, 6, launch_mode=mode, sw13=inp.sw13, sw13_scale=inp.sw13_scale, sw2=inp.sw2,
               sw2_scale=inp.sw2_scale, shared_limit=shape.shared_limit)
    for M in (6, 2, 6):
        a, b = both(moe, inp, M, shared=True)
        assert_same(a, b)


def test_noalloc_after_other_layouts():
    """Calls of different shapes in turn on one GPU: each clears what it needs."""
    small = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=5, experts=12, top_k=3), seed=42, device=DEV)
    wide = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=9, hidden=1024, inter=384, experts=40, top_k=6),
                             seed=43, device=DEV)
    m1, m2 = make(small, 5), make(wide, 9, launch_mode="combine_in_gemm2", gemm_path="mfma")
    for inp, moe, M in ((small, m1, 5), (wide, m2, 9), (small, m1, 4), (wide, m2, 2), (small, m1, 5)):
        a, b = both(moe, inp, M)
        assert_same(a, b)


def test_noalloc_refusals():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=2), seed=44, device=DEV)
    moe = make(inp, 2)
    out = moe.outputs(2)
    L = _capi.lib()
    cfg = moe.cfg
    ptrs = [t.data_ptr() for t in (inp.x, inp.logits, inp.bias)] + [t.data_ptr() for t in out]
    # M beyond the library's limit, a negative M, no config
    assert L.moe_decode_run_noalloc(cfg, 257, *ptrs, None, None) == _capi.ERR_TOO_MANY_TOKENS
    assert L.moe_decode_run_noalloc(cfg, -1, *ptrs, None, None) == _capi.ERR_INVALID_ARG
    assert L.moe_decode_run_noalloc(None, 1, *ptrs, None, None) == _capi.ERR_INVALID_ARG
    # a workspace larger than the buffer: 256 tokens at DeepSeek-V3 shapes (the
    # check comes before any pointer is used, so the tiny buffers are not read)
    big = _capi.MoeDecodeConfig.from_buffer_copy(cfg)
    big.hidden, big.inter, big.experts, big.top_k = 7168, 2048, 256, 8
    assert L.moe_decode_run_noalloc(big, 256, *ptrs, None, None) == _capi.ERR_SCRATCH_TOO_SMALL
    # FP4 weights and packed shared scales need handle-owned copies
    f = _capi.MoeDecodeConfig.from_buffer_copy(cfg)
    f.weight_format = 1
    f.hidden, f.inter = 256, 256
    assert L.moe_decode_run_noalloc(f, 1, *ptrs, None, None) == _capi.ERR_UNSUPPORTED
    # M = 0 is an empty call; the buffer still serves a real one afterwards
    assert L.moe_decode_run_noalloc(cfg, 0, *ptrs, None, None) == _capi.OK
    a, b = both(moe, inp, 2)
    assert_same(a, b)
