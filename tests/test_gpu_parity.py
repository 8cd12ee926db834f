"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bars: ids bit-exact; weights within 1e-6 relative; x_q / x_s bit-exact (both
sides quantise with the same FP32 operations); GEMM1 sums within an
FP32-accumulation bound; h_q within one e4m3 step of the oracle's
requantisation of the GPU's own GEMM1 result, on at most 1% of codes; slot,
combined rows within 2e-2 x the oracle row's RMS.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_block_scaled_moe_amd import MoeDecode, MoeDecodeError, _capi, debug_codec
from tests.helpers import (WEIGHT_RTOL, assert_rows_close, expert_fn, host, oracle_layer)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = ["valu_splitk", "mfma_splitk", "mfma"]


def make(inp, M=None, **kw):
    s = inp.shape
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=kw.pop("max_tokens", M or s.M),
                     logits_dtype=inp.logits.dtype, ue8m0_act=s.ue8m0_act, **kw)


def stage(moe, name, n, dtype):
    return moe.stage(name, torch.empty(n, dtype=dtype, device=DEV))


def run(moe, inp):
    out = moe(inp.x, inp.logits, inp.bias)
    torch.cuda.synchronize()
    return out


def check_routing(ids, weights, ref):
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(host(weights), ref["weights"], rtol=WEIGHT_RTOL, atol=0)


def check_buckets(moe, ids):
    ids = ids.cpu().numpy().reshape(-1)
    R = ids.size
    ctrl = stage(moe, "ctrl", 2, torch.int32).cpu().numpy()
    uniq = np.unique(ids)
    assert ctrl[0] == 0 and ctrl[1] == uniq.size
    U = uniq.size
    assert np.array_equal(stage(moe, "uexp", U, torch.int32).cpu().numpy(), uniq)
    off = stage(moe, "uoff", U, torch.int32).cpu().numpy()
    cnt = stage(moe, "ucnt", U, torch.int32).cpu().numpy()
    routes = stage(moe, "routes", R, torch.int32).cpu().numpy()
    for u, e in enumerate(uniq):
        want = np.nonzero(ids == e)[0]
        assert cnt[u] == want.size
        assert np.array_equal(routes[off[u]:off[u] + cnt[u]], want)


def check_quant(moe, inp, ref):
    M, H = inp.x.shape
    xq = stage(moe, "x_q", M * H, torch.uint8).cpu().numpy().reshape(M, H)
    xs = host(stage(moe, "x_s", M * (H // 128), torch.float32)).reshape(M, -1)
    assert np.array_equal(xq, ref["x_q"])
    assert np.array_equal(xs, ref["x_s"])


def gpu_h1(moe, inp, M):
    s = inp.shape
    R, N = M * s.top_k, 2 * s.inter
    S = moe.plan(M)["splits1"]
    p = stage(moe, "part1", S * R * N, torch.float32).view(S, R, N)
    return host(p.sum(0))  # same fixed order as the kernel: split 0, 1, ...


# GEMM1 error bound relative to sum |terms|. Both inner products multiply
# exactly (e4m3 values are exact in F16) and add in FP32: the VALU path with
# v_dot2 pairs then per-lane and cross-lane adds, the MFMA path with the F16
# 16x16x32 instruction's FP32 sums; a few hundred roundings of 2**-24 at most,
# bounded here by 2**-20.
H1_BOUND = {"valu_splitk": 2.0**-20, "mfma_splitk": 2.0**-20, "mfma": 2.0**-20}


def h1_bound(inp, ref, path):
    ids = ref["ids"].reshape(-1)
    k = inp.shape.top_k
    get = expert_fn(inp)
    out = np.zeros_like(ref["h1"])
    for e in np.unique(ids):
        w13, s13, _, _ = get(int(e))
        rows = np.nonzero(ids == e)[0]
        out[rows] = oracle.block_scaled_gemm(w13 & 0x7F, s13, ref["x_q"][rows // k] & 0x7F,
                                             ref["x_s"][rows // k])
    return out * H1_BOUND[path] + 1e-30


def check_hidden(moe, inp, M, h1):
    s = inp.shape
    R, I = M * s.top_k, s.inter
    hq = stage(moe, "h_q", R * I, torch.uint8).cpu().numpy().reshape(R, I)
    hs = host(stage(moe, "h_s", R * (I // 128), torch.float32)).reshape(R, -1)
    act = oracle.swiglu(h1, I, s.limit)
    q, sc = oracle.requantize_hidden(act)
    np.testing.assert_allclose(hs, sc, rtol=1e-5, atol=0)
    dq_gpu = oracle.e4m3_decode(hq)
    dq_ref = oracle.e4m3_decode(q)
    diff = hq != q
    assert diff.mean() <= 0.01, f"{diff.mean():.3%} of hidden codes differ"
    # a differing code is a neighbour (one e4m3 step)
    step = np.abs(oracle.e4m3_decode(q ^ 1) - dq_ref)
    assert np.all(np.abs(dq_gpu - dq_ref)[diff] <= np.maximum(step, 2.0**-9)[diff] * 2 + 1e-12)


def full_check(moe, inp, stages=True):
    M = inp.x.shape[0]
    path = {v: k for k, v in _capi.GEMM_PATHS.items()}[moe.plan(M)["path"]]
    slots, ids, weights, combined = run(moe, inp)
    ref = oracle_layer(inp)
    check_routing(ids, weights, ref)
    if stages:
        check_buckets(moe, ids)
        check_quant(moe, inp, ref)
        h1 = gpu_h1(moe, inp, M)
        bound = h1_bound(inp, ref, path)
        bad = np.abs(h1 - ref["h1"]) > bound
        assert not bad.any(), f"GEMM1: {bad.sum()} of {bad.size} sums outside the FP32 bound"
        check_hidden(moe, inp, M, h1)
    e1 = assert_rows_close(host(slots), ref["slots"], what="slots")
    e2 = assert_rows_close(host(combined), ref["combined"], what="combined")
    return ref, (slots, ids, weights, combined), (e1, e2)


# ---------------------------------------------------------------------------


def test_device_codec():
    grid = oracle.E4M3_VALUES[[c for c in range(0x7F)]]
    mids = (grid[1:] + grid[:-1]) / 2
    f = np.float32
    vals = [grid, mids, np.nextafter(mids.astype(f), f(0)), np.nextafter(mids.astype(f), f(1000)),
            np.array([448, 460, 463.99, 464, 470, 480, 1e4, 3e38, 0, 2.0**-10, 2.0**-11, 1e-30])]
    bits = np.arange(0, 0x43F00000, 4099, dtype=np.uint32)  # every 4099th pattern up to 480
    vals.append(bits.view(np.float32))
    v = np.concatenate([np.asarray(a, dtype=np.float64) for a in vals]).astype(np.float32)
    v = np.concatenate([v, -v])
    q, dq = debug_codec(torch.from_numpy(v).to(DEV))
    want = oracle.e4m3_encode(v.astype(np.float64))
    got = q.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} encodings differ, first {v[bad[:5]]} -> {got[bad[:5]]} vs {want[bad[:5]]}"
    # the FP8 reader, every code through each byte position of a word
    q2, dq2 = debug_codec(torch.zeros(1024, dtype=torch.float32, device=DEV))
    ref = oracle.E4M3_VALUES[np.arange(1024) & 255]
    d = dq2.cpu().numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], ref[~nan])


@pytest.mark.parametrize("path", PATHS)
def test_tiny(path):
    inp = synth.make_inputs(synth.CONFIGS["tiny"], seed=0, device=DEV)
    moe = make(inp, gemm_path=path)
    assert moe.plan(1)["path"] == _capi.GEMM_PATHS[path]
    full_check(moe, inp)


SHAPES = [
    # (name, overrides)
    ("ragged", dict(M=5, hidden=384, inter=256, experts=10, top_k=3)),
    ("all_experts", dict(M=7, hidden=256, inter=128, experts=8, top_k=8)),
    ("minimal", dict(M=1, hidden=128, inter=128, experts=1, top_k=1)),
    ("e70_m33", dict(M=33, hidden=1024, inter=384, experts=70, top_k=6)),
    ("m65_two_words", dict(M=65, hidden=256, inter=128, experts=16, top_k=4)),
    ("bf16_logits", dict(M=6, hidden=512, inter=256, experts=40, top_k=5, logits_dtype="bf16")),
    ("ue8m0", dict(M=4, hidden=512, inter=256, experts=12, top_k=4, ue8m0_act=True)),
    ("wide_k", dict(M=3, hidden=2304, inter=640, experts=24, top_k=4)),
    # 3 x 56 blocks of x: more than the routing workgroup's quantising waves
    # take one each, so a workgroup that only quantises joins
    ("quant_wgs_m3", dict(M=3, hidden=7168, inter=256, experts=12, top_k=4)),
    # the largest hidden the GEMM workgroup's LDS takes (652 blocks per
    # token): the quantising-only workgroups stop at sixteen, so some groups
    # of eight lanes take two blocks
    ("max_hidden_m4", dict(M=4, hidden=83456, inter=128, experts=4, top_k=2)),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name,over", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(name, over, path):
    shape = synth.CONFIGS["tiny"].with_(name=name, **over)
    inp = synth.make_inputs(shape, seed=11, device=DEV)
    moe = make(inp, gemm_path=path)
    full_check(moe, inp)


# The largest sizes the library takes together: 256 tokens (four 64-bit token
# mask words per expert), top-32 and 512 experts (8,192 routes bucketed
# through LDS by the last of 64 routing workgroups); and 1024 experts with
# top-32.
LIMITS = [
    ("m256_e512_k32", dict(M=256, hidden=256, inter=128, experts=512, top_k=32)),
    ("m16_e1024_k32", dict(M=16, hidden=256, inter=256, experts=1024, top_k=32)),
]


@pytest.mark.parametrize("path", ["auto", "mfma_splitk"])
@pytest.mark.parametrize("name,over", LIMITS, ids=[s[0] for s in LIMITS])
def test_limits(name, over, path):
    shape = synth.CONFIGS["tiny"].with_(name=name, **over)
    inp = synth.make_inputs(shape, seed=17, device=DEV)
    moe = make(inp, gemm_path=path)
    slots, ids, weights, combined = run(moe, inp)
    ref = oracle_layer(inp)
    check_routing(ids, weights, ref)
    check_buckets(moe, ids)
    assert_rows_close(host(slots), ref["slots"], what="slots")
    assert_rows_close(host(combined), ref["combined"], what="combined")


@pytest.mark.parametrize("path", PATHS)
def test_skewed_routing_many_routes_per_expert(path):
    """Two experts taken by every token: 40 routes on one expert, more than one
    pass of either inner product."""
    shape = synth.CONFIGS["tiny"].with_(M=40, hidden=384, inter=256, experts=32, top_k=4)
    inp = synth.make_inputs(shape, seed=12, device=DEV)
    inp.bias[[5, 17]] += 10.0
    moe = make(inp, gemm_path=path)
    ref, (slots, ids, _, _), _ = full_check(moe, inp)
    assert np.all(np.sort(ids.cpu().numpy()[:, :2], axis=1) == [5, 17])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("splits", [(1, 1), (3, 2), (0, 0)])
def test_exact_pow2_case(path, splits):
    """Integer weights, pow2 scales, integer activations with a +-7 in every
    block: every GEMM1 sum is an exact multiple of a power of two below 2**24,
    so the GPU's FP32 result equals the oracle's exactly."""
    shape = synth.CONFIGS["tiny"].with_(M=6, hidden=768, inter=256, experts=12, top_k=3,
                                        weights="int", x_kind="int", pow2_scales=True)
    inp = synth.make_inputs(shape, seed=13, device=DEV)
    moe = make(inp, gemm_path=path, splits1=splits[0], splits2=splits[1])
    slots, ids, weights, combined = run(moe, inp)
    ref = oracle_layer(inp)
    check_routing(ids, weights, ref)
    check_quant(moe, inp, ref)
    assert np.all(ref["x_s"] == 2.0**-6)
    assert np.array_equal(gpu_h1(moe, inp, shape.M), ref["h1"])
    # with GEMM1 exact, the SwiGLU and the FP8 hidden agree bit for bit too
    R, I = shape.M * shape.top_k, shape.inter
    hq = stage(moe, "h_q", R * I, torch.uint8).cpu().numpy().reshape(R, I)
    hs = host(stage(moe, "h_s", R * (I // 128), torch.float32)).reshape(R, -1)
    assert np.array_equal(hq, ref["h_q"]) and np.array_equal(hs, ref["h_s"])
    assert_rows_close(host(slots), ref["slots"])


def test_zero_inputs():
    shape = synth.CONFIGS["tiny"].with_(M=3, x_kind="zero", experts=16, top_k=4)
    inp = synth.make_inputs(shape, seed=14, device=DEV)
    inp.logits.zero_()
    inp.bias.zero_()
    moe = make(inp)
    slots, ids, weights, combined = run(moe, inp)
    assert ids.cpu().numpy().tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(host(weights) == 2.5 / 4)
    assert not slots.float().abs().max().item() and not combined.float().abs().max().item()


@pytest.mark.parametrize("E,k", [(896, 16), (256, 8), (1024, 32)])
def test_routing_ties_and_infinities(E, k):
    """Logits from {-inf, -1, 0, 1, +inf} and biases from {0, 0.5}: most
    keys tie, across lanes and across the experts a lane holds, so the picks
    are decided by the lower-index rule throughout; +inf and -inf logits give
    scores of exactly 1 and 0."""
    shape = synth.CONFIGS["tiny"].with_(M=5, hidden=256, inter=128, experts=E, top_k=k)
    inp = synth.make_inputs(shape, seed=18, device=DEV)
    g = torch.Generator().manual_seed(19)
    vals = torch.tensor([-float("inf"), -1.0, 0.0, 1.0, float("inf")])
    inp.logits.copy_(vals[torch.randint(0, 5, (shape.M, E), generator=g)])
    inp.bias.copy_(torch.tensor([0.0, 0.5])[torch.randint(0, 2, (E,), generator=g)])
    slots, ids, weights, combined = run(make(inp), inp)
    ref = oracle_layer(inp)
    check_routing(ids, weights, ref)
    assert_rows_close(host(combined), ref["combined"], what="combined")


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_token_independent(path):
    shape = synth.CONFIGS["tiny"].with_(M=9, hidden=512, inter=256, experts=20, top_k=4)
    inp = synth.make_inputs(shape, seed=15, device=DEV)
    moe = make(inp, gemm_path=path)
    a = [t.clone() for t in run(moe, inp)]
    b = run(moe, inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # each token alone gives the same rows bit for bit
    k = shape.top_k
    for t in (0, 4, 8):
        out = moe(inp.x[t:t + 1].contiguous(), inp.logits[t:t + 1].contiguous(), inp.bias)
        torch.cuda.synchronize()
        assert torch.equal(out[0], a[0][t * k:(t + 1) * k])
        assert torch.equal(out[3][0], a[3][t])


def test_run_argument_errors():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=2), seed=16, device=DEV)
    moe = make(inp)
    slots, ids, weights, combined = moe.outputs(2)
    big = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=3), seed=16, device=DEV)
    with pytest.raises(MoeDecodeError) as e:
        moe.run_into(big.x, big.logits, big.bias, *moe.outputs(3))
    assert e.value.code == _capi.ERR_TOO_MANY_TOKENS
    with pytest.raises(MoeDecodeError) as e:
        moe.run_into(inp.x, inp.logits, inp.bias, slots, ids, weights, combined, shared_out=combined)
    assert e.value.code == _capi.ERR_INVALID_ARG
    # the handle still works, and M = 0 is an empty call
    moe.run_into(inp.x[:0], inp.logits[:0], inp.bias, slots, ids, weights, combined)
    out = moe(inp.x, inp.logits, inp.bias)
    torch.cuda.synchronize()
    ref = oracle_layer(inp)
    check_routing(out[1], out[2], ref)


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def dsv3():
    return synth.make_inputs(synth.CONFIGS["dsv3"], seed=0, device=DEV)


@pytest.mark.parametrize("path", PATHS)
def test_dsv3_m4(dsv3, path):
    moe = make(dsv3, gemm_path=path)
    full_check(moe, dsv3, stages=True)


def _sampled(inp, M_run, sample, path):
    """Runs M_run tokens on the GPU and checks the tokens in `sample` against
    the oracle computed for those tokens only."""
    moe = make(inp, gemm_path=path)
    slots, ids, weights, combined = run(moe, inp)
    sub = synth.MoeInputs(shape=inp.shape.with_(M=len(sample)), seed=inp.seed, x=inp.x[sample],
                          logits=inp.logits[sample], bias=inp.bias, w13=inp.w13,
                          w13_scale=inp.w13_scale, w2=inp.w2, w2_scale=inp.w2_scale)
    ref = oracle_layer(sub)
    k = inp.shape.top_k
    rows = np.concatenate([np.arange(t * k, (t + 1) * k) for t in sample])
    check_routing(ids[sample], weights[sample], ref)
    assert_rows_close(host(slots)[rows], ref["slots"], what="slots")
    assert_rows_close(host(combined)[sample], ref["combined"], what="combined")
    # every token's routing is checked in full (cheap)
    rid, rw, _ = oracle.route(host(inp.logits), host(inp.bias), k, inp.shape.routed_scale)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(host(weights), rw, rtol=WEIGHT_RTOL, atol=0)


@pytest.mark.parametrize("path", PATHS)
def test_dsv3_m32_sampled(path):
    inp = synth.make_inputs(synth.CONFIGS["dsv3"].with_(M=32), seed=1, device=DEV)
    _sampled(inp, 32, [0, 13, 31], path)


@pytest.mark.parametrize("path", PATHS)
def test_latent_m64_sampled(path):
    inp = synth.make_inputs(synth.CONFIGS["latent"], seed=0, device=DEV)
    _sampled(inp, 64, [0, 21, 63], path)

