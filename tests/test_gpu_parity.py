"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bars: ids bit-exact; weights within 1e-6 relative; x_q / x_s bit-exact (both
sides quantise with the same FP32 operations); GEMM1 sums within an
FP32-accumulation bound; h_q within one e4m3 step of the oracle's
requantisation of the GPU's own GEMM1 result, on at most 1% of codes; slot,
combined rows within 2e-2 x the oracle row's RMS; the combine, given the GPU's
own slots and weights, within one BF16 step of the oracle's combine and
bit-exact on at least 99.9% of elements (the weights applied once, in FP32,
in pick order: nvfp4-megamoe-kernel README, "slot representation" and bug 7).

"auto" is the plan the benchmark times (persistent GEMMs at up to 8 tokens,
GEMM1 in 4 K parts at DeepSeek-V3 shapes); it is checked stage by stage like
the named paths.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_block_scaled_moe_amd import MoeDecode, MoeDecodeError, _capi, debug_codec
from tests.helpers import (WEIGHT_RTOL, assert_rows_close, check_combine, combine_bound, expert_fn,
                           host, oracle_layer, rounding_valid)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = ["valu_splitk", "mfma_splitk", "mfma", "auto"]
PATH_USED = {"auto": "mfma"}  # the kernel family a path name resolves to


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


def h1_abs_terms(inp, ref):
    """sum |terms| of every GEMM1 output (cached in ref: it costs an oracle GEMM)."""
    if "h1_abs" not in ref:
        ids = ref["ids"].reshape(-1)
        k = inp.shape.top_k
        get = expert_fn(inp)
        out = np.zeros_like(ref["h1"])
        for e in np.unique(ids):
            w13, s13, _, _ = get(int(e))
            rows = np.nonzero(ids == e)[0]
            out[rows] = oracle.block_scaled_gemm(w13 & 0x7F, s13, ref["x_q"][rows // k] & 0x7F,
                                                 ref["x_s"][rows // k])
        ref["h1_abs"] = out
    return ref["h1_abs"]


def h1_bound(inp, ref, path):
    return h1_abs_terms(inp, ref) * H1_BOUND[path] + 1e-30


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


def full_check(moe, inp, stages=True, ref=None):
    M = inp.x.shape[0]
    path = {v: k for k, v in _capi.GEMM_PATHS.items()}[moe.plan(M)["path"]]
    slots, ids, weights, combined = run(moe, inp)
    if ref is None:
        ref = oracle_layer(inp)
    check_routing(ids, weights, ref)
    check_combine(slots, weights, combined)
    if stages:
        check_buckets(moe, ids)
        check_quant(moe, inp, ref)
        h1 = gpu_h1(moe, inp, M)
        bound = h1_bound(inp, ref, path)
        bad = np.abs(h1 - ref["h1"]) > bound
        assert not bad.any(), f"GEMM1: {bad.sum()} of {bad.size} sums outside the FP32 bound"
        check_hidden(moe, inp, M, h1)
    vs = slot_validity(moe, inp, M, ids, slots) if stages else None
    vc = combined_validity(slots, weights, combined)
    e1 = assert_rows_close(host(slots), ref["slots"], what="slots", valid=vs)
    e2 = assert_rows_close(host(combined), ref["combined"], what="combined", valid=vc)
    return ref, (slots, ids, weights, combined), (e1, e2)


def slot_validity(moe, inp, M, ids, slots):
    """valid(rows) for slot rows: each GPU BF16 value is the rounding of a value
    within the GEMM2 FP32 bound (2**-20 of sum |terms|) of the exact GEMM2 of
    the GPU's own FP8 hidden, whose codes check_hidden has validated."""
    s = inp.shape
    R, I = M * s.top_k, s.inter
    hq = stage(moe, "h_q", R * I, torch.uint8).cpu().numpy().reshape(R, I)
    hs = host(stage(moe, "h_s", R * (I // 128), torch.float32)).reshape(R, -1)
    g = host(slots)
    idl = ids.cpu().numpy().reshape(-1)
    get = expert_fn(inp)

    def valid(rows):
        out = []
        for r in rows:
            _, _, w2, s2 = get(int(idl[r]))
            y = oracle.block_scaled_gemm(w2, s2, hq[r:r + 1], hs[r:r + 1])[0]
            b = oracle.block_scaled_gemm(w2 & 0x7F, s2, hq[r:r + 1] & 0x7F, hs[r:r + 1])[0] * 2.0**-20
            out.append(rounding_valid(g[r], y, b))
        return np.array(out)
    return valid


def combined_validity(slots, weights, combined):
    """valid(rows) for combined rows: the rounding of the GPU's own slots and
    weights summed within the FP32 multiply-add bound."""
    g, sl, w = host(combined), host(slots), host(weights)
    exact = np.einsum("tk,tkh->th", w, sl.reshape(w.shape[0], w.shape[1], -1))
    bound = combine_bound(sl, w)
    return lambda rows: rounding_valid(g[rows], exact[rows], bound[rows])


# ---------------------------------------------------------------------------


def test_device_codec_exhaustive():
    """The device e4m3 encoder on every binary32 pattern of [0, 480] and its
    negation. The encoder's codes must rise by at most one step from each
    pattern to the next, from 0x00 to 0x7E; the oracle encoder (round to
    nearest even, saturating) is monotone, so agreement on both sides of each
    of the 126 steps, checked here, gives agreement on every pattern."""
    top = 0x43F00000 + 1                      # patterns 0 .. 480.0 inclusive
    chunk = 1 << 27
    prev_last = None
    steps = []
    for lo in range(0, top, chunk):
        n = min(chunk, top - lo)
        bits = torch.arange(lo, lo + n, dtype=torch.int32, device=DEV)
        q, _ = debug_codec(bits.view(torch.float32))
        qn, _ = debug_codec((bits | torch.tensor(-(1 << 31), dtype=torch.int32, device=DEV))
                            .view(torch.float32))
        assert torch.equal(qn, q | 0x80), f"negated patterns in [{lo:#x}, {lo + n:#x})"
        d = torch.diff(q.to(torch.int16))
        assert int(d.min()) >= 0 and int(d.max()) <= 1, f"codes not rising by single steps near {lo:#x}"
        if prev_last is not None:
            assert 0 <= int(q[0]) - prev_last <= 1
            if int(q[0]) != prev_last:
                steps.append(lo)
        steps += (lo + 1 + torch.nonzero(d).flatten()).tolist()
        if lo == 0:
            assert int(q[0]) == 0
        prev_last = int(q[-1])
        del bits, q, qn, d
    assert prev_last == 0x7E and len(steps) == 126
    pat = np.array(steps, dtype=np.uint32)
    both = np.concatenate([pat - 1, pat]).view(np.float32).astype(np.float64)
    want = oracle.e4m3_encode(both)
    assert np.array_equal(want[:126] + 1, want[126:]), "oracle steps differ from the device's"
    assert np.array_equal(want[126:], np.arange(1, 127)), "a device step lands on the wrong pattern"


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
    assert moe.plan(1)["path"] == _capi.GEMM_PATHS[PATH_USED.get(path, path)]
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
    with pytest.raises(ValueError):
        moe.run_into(inp.x, inp.logits, inp.bias, slots, ids, weights, combined, shared_out=combined)
    # the C ABI's own check of the same mistake
    rc = _capi.lib().moe_decode_run(moe._h, 2, inp.x.data_ptr(), inp.logits.data_ptr(),
                                    inp.bias.data_ptr(), slots.data_ptr(), ids.data_ptr(),
                                    weights.data_ptr(), combined.data_ptr(), combined.data_ptr(),
                                    None)
    assert rc == _capi.ERR_INVALID_ARG
    # the handle still works, and M = 0 is an empty call
    moe.run_into(inp.x[:0], inp.logits[:0], inp.bias, slots, ids, weights, combined)
    out = moe(inp.x, inp.logits, inp.bias)
    torch.cuda.synchronize()
    ref = oracle_layer(inp)
    check_routing(out[1], out[2], ref)


# ---------------------------------------------------------------------------
# Binding: every buffer's shape, dtype and device checked before a launch
# ---------------------------------------------------------------------------

def test_binding_rejects_mismatched_buffers():
    """The C ABI takes bare pointers and cannot see sizes, so the binding
    checks every buffer; each mistake raises ValueError, nothing is launched,
    and the outputs keep their sentinel values."""
    shape = synth.CONFIGS["tiny"].with_(M=3, experts=12, top_k=3)
    inp = synth.make_inputs(shape, seed=20, device=DEV)
    moe = make(inp)
    outs = moe.outputs(3)
    for t in outs:
        t.fill_(7)
    sentinel = [t.clone() for t in outs]
    torch.cuda.synchronize()
    H, E, k = shape.hidden, shape.experts, shape.top_k
    x, lg, b = inp.x, inp.logits, inp.bias
    bad_calls = {
        "x width": (x[:, :128].contiguous(), lg, b) + outs,
        "x dtype": (x.float(), lg, b) + outs,
        "logits width": (x, lg[:, :E - 1].contiguous(), b) + outs,
        "logits rows": (x, lg[:2].contiguous(), b) + outs,
        "logits dtype": (x, lg.to(torch.bfloat16), b) + outs,
        "bias length": (x, lg, b[:E - 1].clone()) + outs,
        "bias on host": (x, lg, b.cpu()) + outs,
        "slots rows": (x, lg, b, outs[0][:-1].clone()) + outs[1:],
        "slots dtype": (x, lg, b, outs[0].float()) + outs[1:],
        "ids shape": (x, lg, b, outs[0], outs[1].view(-1)) + outs[2:],
        "ids dtype": (x, lg, b, outs[0], outs[1].long()) + outs[2:],
        "weights shape": (x, lg, b, outs[0], outs[1], outs[2][:, :2].contiguous(), outs[3]),
        "combined width": (x, lg, b) + outs[:3] + (outs[3][:, :128].contiguous(),),
        "combined non-contiguous": (x, lg, b) + outs[:3] + (outs[3].t().contiguous().t(),),
    }
    for what, args in bad_calls.items():
        with pytest.raises(ValueError):
            moe.run_into(*args)
        if what.split()[0] in ("x", "logits", "bias"):   # the allocating call checks them too
            with pytest.raises(ValueError):
                moe(*args[:3])
    torch.cuda.synchronize()
    for t, want in zip(outs, sentinel):
        assert torch.equal(t, want), "a rejected call wrote an output"
    # weights and scales of the wrong shape are refused before create
    w2t = inp.w2.transpose(1, 2).contiguous()
    for args in ((inp.w13, inp.w13_scale, w2t, inp.w2_scale),
                 (inp.w13, inp.w13_scale[:, :1].contiguous(), inp.w2, inp.w2_scale),
                 (inp.w13, inp.w13_scale, inp.w2, inp.w2_scale[:-1].contiguous()),
                 (inp.w13[:, :-128].contiguous(), inp.w13_scale, inp.w2, inp.w2_scale)):
        with pytest.raises(ValueError):
            MoeDecode(*args, top_k=k, limit=7.0, routed_scale=2.5, max_tokens=3)
    # the handle is unharmed
    out = moe(x, lg, b)
    torch.cuda.synchronize()
    check_routing(out[1], out[2], oracle_layer(inp))


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def dsv3():
    return synth.make_inputs(synth.CONFIGS["dsv3"], seed=0, device=DEV)


@pytest.fixture(scope="module")
def dsv3_ref(dsv3):
    return oracle_layer(dsv3)


@pytest.mark.parametrize("path", PATHS)
def test_dsv3_m4(dsv3, dsv3_ref, path):
    moe = make(dsv3, gemm_path=path)
    if path == "auto":
        # the benchmark's plan: persistent GEMMs, GEMM1 in 4 K parts
        p = moe.plan(4)
        assert p["persist1"] > 0 and p["persist2"] > 0 and p["kparts1"] == 4
    full_check(moe, dsv3, stages=True, ref=dsv3_ref)


@pytest.fixture(scope="module")
def dsv3_m32():
    inp = synth.make_inputs(synth.CONFIGS["dsv3"].with_(M=32), seed=1, device=DEV)
    return inp, oracle_layer(inp)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", PATHS)
def test_dsv3_m32_all_tokens(dsv3_m32, path):
    """DeepSeek-V3 shapes at 32 tokens (about 83 touched experts): every
    token's slots and combined row against the oracle, stage by stage."""
    inp, ref = dsv3_m32
    full_check(make(inp, gemm_path=path), inp, stages=True, ref=ref)


@pytest.fixture(scope="module")
def latent_m64():
    inp = synth.make_inputs(synth.CONFIGS["latent"], seed=0, device=DEV)
    return inp, oracle_layer(inp)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", PATHS)
def test_latent_m64_all_tokens(latent_m64, path):
    """The latent shape (896 experts, top-16, BF16 logits) at 64 tokens, about
    613 touched experts: every token against the oracle, stage by stage."""
    inp, ref = latent_m64
    full_check(make(inp, gemm_path=path), inp, stages=True, ref=ref)
