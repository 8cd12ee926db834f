"""GPU parity of the shared expert ("shared_expert" page) against the oracle.

The shared expert runs inside the routed launches (its GEMV units ahead of the
routed units, its SwiGLU waves after the routed ones, its output written by the
combine). Bars: its x_q / x_s bit-exact; gate_up sums within the FP32
accumulation bound; its FP8 hidden within one e4m3 step of the oracle's
requantisation of the GPU's own gate_up, on at most 1% of codes; shared_out
rows within 2e-2 x the oracle row's RMS. The routed outputs must not change by
a single bit when the shared expert runs beside them.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_block_scaled_moe_amd import MoeDecode, MoeDecodeError, _capi
from tests.helpers import (WEIGHT_RTOL, assert_rows_close, check_combine, host, oracle_layer,
                           oracle_shared)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = ["valu_splitk", "mfma_splitk", "mfma"]


def make(inp, shared=True, packed=False, shared_ue8m0=True, max_tokens=None, **kw):
    s = inp.shape
    extra = {}
    if shared:
        s13, s2 = inp.sw13_scale, inp.sw2_scale
        if packed:
            H, Is = s.hidden, s.shared_inter
            s13 = synth.pack_ue8m0(s13, 2 * Is, H)
            s2 = synth.pack_ue8m0(s2, H, Is)
        extra = dict(sw13=inp.sw13, sw13_scale=s13, sw2=inp.sw2, sw2_scale=s2,
                     shared_limit=s.shared_limit, shared_ue8m0_act=shared_ue8m0)
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=max_tokens or s.M,
                     logits_dtype=inp.logits.dtype, ue8m0_act=s.ue8m0_act, **extra, **kw)


def stage(moe, name, n, dtype):
    return moe.stage(name, torch.empty(n, dtype=dtype, device=DEV))


def run(moe, inp, M=None):
    M = M or inp.x.shape[0]
    out = moe(inp.x[:M].contiguous(), inp.logits[:M].contiguous(), inp.bias)
    torch.cuda.synchronize()
    return out


def gpu_gate_up(moe, M, Is):
    S = moe.plan(M)["shared_splits1"]
    p = stage(moe, "shared_part1", S * M * 2 * Is, torch.float32).view(S, M, 2 * Is)
    return host(p.sum(0))  # the kernel's fixed order: split 0, 1, ...


def check_shared_quant(moe, inp, ref, M):
    H = inp.shape.hidden
    xq = stage(moe, "shared_x_q", M * H, torch.uint8).cpu().numpy().reshape(M, H)
    xs = host(stage(moe, "shared_x_s", M * (H // 128), torch.float32)).reshape(M, -1)
    assert np.array_equal(xq, ref["x_q"][:M])
    assert np.array_equal(xs, ref["x_s"][:M])


def shared_hidden_from(gate_up, Is, limit, ue8m0):
    """The oracle's steps after gate_up ("shared_expert" page, _DownKernel),
    applied to a given FP32 gate_up."""
    gu = oracle.bf16_round(gate_up)
    gate = np.minimum(gu[:, :Is], limit)
    up = np.clip(gu[:, Is:], -limit, limit)
    act = oracle.bf16_round(oracle.silu_f32(gate) * up)
    return oracle.quantize_blocks(act, ue8m0=ue8m0, reciprocal=True)


def check_shared_hidden(moe, inp, M, gate_up, ue8m0=True):
    Is = inp.shape.shared_inter
    hq = stage(moe, "shared_h_q", M * Is, torch.uint8).cpu().numpy().reshape(M, Is)
    hs = host(stage(moe, "shared_h_s", M * (Is // 128), torch.float32)).reshape(M, -1)
    q, sc = shared_hidden_from(gate_up, Is, inp.shape.shared_limit, ue8m0)
    np.testing.assert_allclose(hs, sc, rtol=1e-5, atol=0)
    diff = hq != q
    assert diff.mean() <= 0.01, f"{diff.mean():.3%} of shared hidden codes differ"
    dq_ref = oracle.e4m3_decode(q)
    step = np.abs(oracle.e4m3_decode(q ^ 1) - dq_ref)
    assert np.all(np.abs(oracle.e4m3_decode(hq) - dq_ref)[diff] <= 2 * np.maximum(step, 2.0**-9)[diff])
    return hq, hs


def gate_up_bound(inp, ref, M):
    """FP32-accumulation bound of the gate_up sums: 2**-20 x sum |terms|."""
    a = oracle.block_scaled_gemm(inp.sw13.cpu().numpy() & 0x7F, host(inp.sw13_scale),
                                 ref["x_q"][:M] & 0x7F, ref["x_s"][:M])
    return a * 2.0**-20 + 1e-30


SMALL = synth.CONFIGS["tiny"].with_(name="shared_small", M=5, hidden=512, inter=256, experts=12,
                                    top_k=3, shared_inter=384)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("packed", [False, True], ids=["f32_scales", "ue8m0_packed"])
def test_shared_small(path, packed):
    inp = synth.make_inputs(SMALL, seed=21, device=DEV)
    moe = make(inp, packed=packed, gemm_path=path)
    M, Is = SMALL.M, SMALL.shared_inter
    slots, ids, weights, combined, shared_out = run(moe, inp)
    ref = oracle_shared(inp)
    check_shared_quant(moe, inp, ref, M)
    gu = gpu_gate_up(moe, M, Is)
    exact = oracle.block_scaled_gemm(inp.sw13.cpu().numpy(), host(inp.sw13_scale), ref["x_q"], ref["x_s"])
    bad = np.abs(gu - exact) > gate_up_bound(inp, ref, M)
    assert not bad.any(), f"gate_up: {bad.sum()} of {bad.size} sums outside the FP32 bound"
    check_shared_hidden(moe, inp, M, gu)
    assert_rows_close(host(shared_out), ref["out"], what="shared_out")
    # routed outputs: the oracle's, and bit-identical to a handle without the shared expert
    lref = oracle_layer(inp)
    assert np.array_equal(ids.cpu().numpy(), lref["ids"])
    np.testing.assert_allclose(host(weights), lref["weights"], rtol=WEIGHT_RTOL, atol=0)
    assert_rows_close(host(combined), lref["combined"], what="combined")
    plain = make(inp, shared=False, gemm_path=path)
    for a, b in zip(run(plain, inp), (slots, ids, weights, combined)):
        assert torch.equal(a, b)


def test_shared_own_quant_with_quantising_workgroups():
    """3 tokens of H = 7168 with the shared expert on its own scale rule
    (UE8M0, the routed x on plain FP32 scales): both quantisations of x are
    shared with a workgroup that only quantises, and both are bit-exact."""
    shape = SMALL.with_(M=3, hidden=7168, inter=256, experts=8, top_k=2, shared_inter=256)
    inp = synth.make_inputs(shape, seed=25, device=DEV)
    moe = make(inp)
    slots, ids, weights, combined, shared_out = run(moe, inp)
    ref = oracle_shared(inp)
    check_shared_quant(moe, inp, ref, shape.M)
    lref = oracle_layer(inp)
    xq = stage(moe, "x_q", shape.M * shape.hidden, torch.uint8).cpu().numpy().reshape(shape.M, -1)
    xs = host(stage(moe, "x_s", shape.M * (shape.hidden // 128), torch.float32)).reshape(shape.M, -1)
    assert np.array_equal(xq, lref["x_q"]) and np.array_equal(xs, lref["x_s"])
    assert np.array_equal(ids.cpu().numpy(), lref["ids"])
    assert_rows_close(host(combined), lref["combined"], what="combined")
    assert_rows_close(host(shared_out), ref["out"], what="shared_out")


@pytest.mark.parametrize("path", PATHS)
def test_shared_exact_pow2(path):
    """Integer weights and activations with power-of-two scales: every gate_up
    sum is exact in FP32, so the FP8 hidden and its scales agree bit for bit."""
    shape = SMALL.with_(weights="int", x_kind="int", pow2_scales=True)
    inp = synth.make_inputs(shape, seed=22, device=DEV)
    moe = make(inp, gemm_path=path)
    M, Is = shape.M, shape.shared_inter
    *_, shared_out = run(moe, inp)
    ref = oracle_shared(inp)
    check_shared_quant(moe, inp, ref, M)
    assert np.all(ref["x_s"] == 2.0**-6)
    exact = oracle.block_scaled_gemm(inp.sw13.cpu().numpy(), host(inp.sw13_scale), ref["x_q"], ref["x_s"])
    assert np.array_equal(gpu_gate_up(moe, M, Is), exact)
    hq = stage(moe, "shared_h_q", M * Is, torch.uint8).cpu().numpy().reshape(M, Is)
    hs = host(stage(moe, "shared_h_s", M * (Is // 128), torch.float32)).reshape(M, -1)
    assert np.array_equal(hq, ref["h_q"]) and np.array_equal(hs, ref["h_s"])
    assert_rows_close(host(shared_out), ref["out"], what="shared_out")


def test_shared_same_scale_rule_as_routed():
    """shared_ue8m0_act off, like the routed activations: the shared expert
    reads the routed x quantisation."""
    inp = synth.make_inputs(SMALL, seed=23, device=DEV)
    moe = make(inp, shared_ue8m0=False)
    M = SMALL.M
    *_, shared_out = run(moe, inp)
    ref = oracle_shared(inp, ue8m0_act=False)
    check_shared_quant(moe, inp, ref, M)
    gu = gpu_gate_up(moe, M, SMALL.shared_inter)
    check_shared_hidden(moe, inp, M, gu, ue8m0=False)
    assert_rows_close(host(shared_out), ref["out"], what="shared_out")


def test_shared_packed_equals_f32_and_token_counts():
    """Packed UE8M0 scales give the same bits as their FP32 form; one handle
    serves several token counts (the shared expert's routes follow M)."""
    inp = synth.make_inputs(SMALL.with_(M=7), seed=24, device=DEV)
    a = make(inp, packed=False, max_tokens=7)
    b = make(inp, packed=True, max_tokens=7)
    ref = oracle_shared(inp)
    for M in (7, 2, 1):
        ra, rb = run(a, inp, M), run(b, inp, M)
        for u, v in zip(ra, rb):
            assert torch.equal(u, v)
        assert_rows_close(host(ra[4]), ref["out"][:M], what=f"shared_out M={M}")


def test_shared_packed_scales_must_repeat_per_block():
    inp = synth.make_inputs(SMALL, seed=25, device=DEV)
    s = SMALL
    bad = synth.pack_ue8m0(inp.sw13_scale, 2 * s.shared_inter, s.hidden).clone()
    bad[5, 0] ^= 1  # row 5 of block 0 disagrees with row 0
    with pytest.raises(MoeDecodeError) as e:
        MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                  routed_scale=s.routed_scale, max_tokens=s.M, sw13=inp.sw13, sw13_scale=bad,
                  sw2=inp.sw2, sw2_scale=synth.pack_ue8m0(inp.sw2_scale, s.hidden, s.shared_inter))
    assert e.value.code == _capi.ERR_INVALID_ARG


def test_shared_skipped_without_output():
    """shared_out NULL: the handle runs the routed path alone, unchanged."""
    inp = synth.make_inputs(SMALL, seed=26, device=DEV)
    moe = make(inp)
    plain = make(inp, shared=False)
    outs = moe.outputs(SMALL.M)
    moe.run_into(inp.x, inp.logits, inp.bias, *outs)
    torch.cuda.synchronize()
    for a, b in zip(run(plain, inp), outs):
        assert torch.equal(a, b)


@pytest.mark.timeout(600)
def test_shared_dsv3_m32():
    """DeepSeek-V3 shapes at M = 32 with the shared expert (gate_up [4096, 7168],
    down [7168, 2048], UE8M0 scales): every shared_out row and every routed
    token (about 83 touched experts) against the oracle."""
    inp = synth.make_inputs(synth.CONFIGS["dsv3_m32_shared"], seed=0, device=DEV)
    moe = make(inp)
    M = inp.shape.M
    slots, ids, weights, combined, shared_out = run(moe, inp)
    ref = oracle_shared(inp)
    check_shared_quant(moe, inp, ref, M)
    check_shared_hidden(moe, inp, M, gpu_gate_up(moe, M, inp.shape.shared_inter))
    assert_rows_close(host(shared_out), ref["out"], what="shared_out")
    lref = oracle_layer(inp)   # the routed part: the shared expert is not in it
    assert np.array_equal(ids.cpu().numpy(), lref["ids"])
    np.testing.assert_allclose(host(weights), lref["weights"], rtol=WEIGHT_RTOL, atol=0)
    assert_rows_close(host(slots), lref["slots"], what="slots")
    assert_rows_close(host(combined), lref["combined"], what="combined")
    check_combine(slots, weights, combined)


def test_shared_ue8m0_every_byte():
    """Packed UE8M0 scales holding every exponent byte 0..255 (one per 128 x 128
    block of a [4096, 2048] gate_up): the FP32 scales create converts them to
    are the oracle's, bit for bit: byte << 23, so 0 is +0.0 and 255 is +inf
    ("shared_expert" page, block_scales). The handle is only created."""
    s = synth.CONFIGS["tiny"].with_(M=1, hidden=2048, shared_inter=2048)
    inp = synth.make_inputs(s, seed=27, device=DEV)
    H, Is = s.hidden, s.shared_inter
    nb = (2 * Is // 128) * (H // 128)
    assert nb == 512
    # block b carries exponent byte b % 256: the binary32 with bits byte << 23
    byte = torch.arange(nb, dtype=torch.int32, device=DEV) % 256
    bits = (byte << 23).view(2 * Is // 128, H // 128)
    packed13 = synth.pack_ue8m0(bits.view(torch.float32), 2 * Is, H)
    packed2 = synth.pack_ue8m0(inp.sw2_scale, H, Is)
    moe = MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                    routed_scale=s.routed_scale, max_tokens=1, sw13=inp.sw13,
                    sw13_scale=packed13.contiguous(), sw2=inp.sw2, sw2_scale=packed2)
    got = stage(moe, "shared_scale13", nb, torch.float32)
    torch.cuda.synchronize()
    want = oracle.unpack_ue8m0(packed13.cpu().numpy(), 2 * Is, H)
    g = got.cpu().numpy().astype(np.float64).reshape(want.shape)
    assert np.array_equal(g.view(np.int64), want.view(np.int64))
    flat = g.reshape(-1)
    assert flat[0] == 0.0 and np.isposinf(flat[255]) and flat[127] == 1.0
    got2 = stage(moe, "shared_scale2", (H // 128) * (Is // 128), torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(got2).reshape(H // 128, Is // 128), host(inp.sw2_scale))
    moe.close()
