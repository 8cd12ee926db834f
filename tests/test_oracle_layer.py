"""Pins for the oracle's SwiGLU, combine and the whole routed step, plus the
shared expert.

Pinned against: SwiGLU closed forms at hand-picked points (clamp semantics and
row order), combine closed forms, the all-zero warm-up case, exact linearity
(doubling a scale doubles the outputs bit for bit), locality, token
independence, and negative controls: the two bugs the nvfp4-megamoe-kernel
README lists (SiLU of a weighted sum, weights applied twice) must fail the
comparison tolerance.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import bf16_round, f32
from tests.helpers import assert_rows_close, expert_fn, host, oracle_layer, row_errors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_swiglu_golden_points():
    doc = json.load(open(os.path.join(GOLDEN, "swiglu_points.json")))
    pts = doc["points"]
    h1 = np.array([[p["up"], p["gate"]] for p in pts])     # I = 1: [up | gate]
    act = oracle.swiglu(h1, 1, doc["limit"])[:, 0]
    want = np.array([p["act"] for p in pts])
    np.testing.assert_allclose(act, want, rtol=doc["rel_tol"], atol=0)


def test_pins_catch_swapped_gate_up(monkeypatch):
    real = oracle.swiglu

    def swapped(h1, inter, limit):
        h1 = np.asarray(h1)
        return real(np.concatenate([h1[:, inter:], h1[:, :inter]], axis=1), inter, limit)

    monkeypatch.setattr(oracle, "swiglu", swapped)
    with pytest.raises(AssertionError):
        test_swiglu_golden_points()


def test_pins_catch_symmetric_gate_clamp(monkeypatch):
    real = oracle.swiglu

    def both_sides(h1, inter, limit):
        h1 = np.array(h1, dtype=np.float64)
        h1[:, inter:] = np.maximum(h1[:, inter:], -limit)
        return real(h1, inter, limit)

    monkeypatch.setattr(oracle, "swiglu", both_sides)
    with pytest.raises(AssertionError):
        test_swiglu_golden_points()


def test_combine_closed_form():
    slots = np.array([[1.0, -2.0, 0.5], [4.0, 8.0, -0.25],     # token 0
                      [3.0, 0.0, 1.0], [1.0, 1.0, 1.0]])      # token 1
    w = np.array([[0.25, 0.5], [1.5, -1.0]])
    got = oracle.combine(slots, w)
    assert np.array_equal(got, [[2.25, 3.5, 0.0], [3.5, -1.0, 0.5]])
    # BF16 rounding happens once, after the FP32 sum: 1 + 2**-8 + 2**-8 is
    # 1 + 2**-7 exactly, while rounding after each add would stay at 1.0
    s = np.array([[1.0], [2.0**-8], [2.0**-8]])
    assert oracle.combine(s, np.ones((1, 3)))[0, 0] == 1.0 + 2.0**-7


@pytest.fixture(scope="module")
def tiny():
    return synth.make_inputs(synth.CONFIGS["tiny"], seed=0, device="cpu")


def test_zero_warmup_case():
    """All-zero x, logits and bias (the pages' warm-up call): ids 0..k-1,
    weights scale/k, every slot and combined row exactly zero."""
    shape = synth.CONFIGS["tiny"].with_(M=3, x_kind="zero")
    inp = synth.make_inputs(shape, seed=1)
    inp.logits.zero_()
    inp.bias.zero_()
    r = oracle_layer(inp)
    assert r["ids"].tolist() == [[0, 1]] * 3
    assert np.all(r["weights"] == 1.25)
    assert np.all(r["slots"] == 0) and np.all(r["combined"] == 0)


def test_zero_x_gives_zero(tiny):
    shape = synth.CONFIGS["tiny"].with_(M=4, x_kind="zero")
    r = oracle_layer(synth.make_inputs(shape, seed=2))
    assert np.all(r["h1"] == 0) and np.all(r["slots"] == 0) and np.all(r["combined"] == 0)


def _wrapped(inp, e_change, fn):
    base = expert_fn(inp)

    def get(e):
        w13, s13, w2, s2 = base(e)
        if e == e_change:
            return fn(w13.copy(), s13.copy(), w2.copy(), s2.copy())
        return w13, s13, w2, s2
    return get


def _run(inp, expert, **kw):
    s = inp.shape
    args = dict(top_k=s.top_k, routed_scale=s.routed_scale, limit=s.limit, inter=s.inter)
    args.update(kw)
    return oracle.moe_decode(host(inp.x), host(inp.logits), host(inp.bias), expert, **args)


def test_doubling_w2_scale_doubles_that_expert_exactly():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=4), seed=3)
    r0 = oracle_layer(inp)
    e = int(r0["ids"][0, 0])
    r1 = _run(inp, _wrapped(inp, e, lambda a, b, c, d: (a, b, c, 2 * d)))
    rows = r0["ids"].reshape(-1) == e
    assert np.array_equal(r1["slots"][rows], 2 * r0["slots"][rows])
    assert np.array_equal(r1["slots"][~rows], r0["slots"][~rows])


def test_doubling_routed_scale_doubles_weights_and_combined():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=4), seed=4)
    r0 = oracle_layer(inp)
    r1 = oracle_layer(inp, routed_scale=2 * inp.shape.routed_scale)
    assert np.array_equal(r1["weights"], 2 * r0["weights"])
    assert np.array_equal(r1["slots"], r0["slots"])
    assert np.array_equal(r1["combined"], 2 * r0["combined"])


def test_doubling_up_scale_doubles_slots_when_unclamped():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=2), seed=5)
    inp.x = (inp.x.float() * 0.01).to(torch.bfloat16)   # |h1| << L: no clamp
    r0 = oracle_layer(inp)
    assert np.abs(r0["h1"]).max() * 2 < inp.shape.limit
    e = int(r0["ids"][0, 0])
    I = inp.shape.inter

    def dbl_up(w13, s13, w2, s2):
        s13[: I // 128] *= 2
        return w13, s13, w2, s2

    r1 = _run(inp, _wrapped(inp, e, dbl_up))
    rows = r0["ids"].reshape(-1) == e
    assert np.array_equal(r1["h_q"], r0["h_q"])
    assert np.array_equal(r1["slots"][rows], 2 * r0["slots"][rows])
    assert np.array_equal(r1["slots"][~rows], r0["slots"][~rows])


def test_locality_of_expert_weights():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=4), seed=6)
    r0 = oracle_layer(inp)
    e = int(r0["ids"][1, 1])

    def flip(w13, s13, w2, s2):
        return w13 ^ 0x80, s13, w2, s2       # negate every W13 weight of e

    r1 = _run(inp, _wrapped(inp, e, flip))
    rows = r0["ids"].reshape(-1) == e
    assert not np.array_equal(r1["slots"][rows], r0["slots"][rows])
    assert np.array_equal(r1["slots"][~rows], r0["slots"][~rows])
    toks = np.any(r0["ids"] == e, axis=1)
    assert np.array_equal(r1["combined"][~toks], r0["combined"][~toks])


def test_token_independence():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=5, experts=16, top_k=3), seed=7)
    r = oracle_layer(inp)
    k = inp.shape.top_k
    for t in range(5):
        one = oracle.moe_decode(host(inp.x)[t:t + 1], host(inp.logits)[t:t + 1], host(inp.bias),
                                expert_fn(inp), top_k=k, routed_scale=2.5, limit=7.0, inter=128)
        assert np.array_equal(one["ids"][0], r["ids"][t])
        assert np.array_equal(one["slots"], r["slots"][t * k:(t + 1) * k])
        assert np.array_equal(one["combined"][0], r["combined"][t])


def _negative_controls(inp, r):
    """Outputs of the two wrong pipelines the nvfp4-megamoe-kernel README
    lists: SiLU after mixing the experts' GEMM1 outputs with the routing
    weights, and routing weights applied twice."""
    k, I, L = inp.shape.top_k, inp.shape.inter, inp.shape.limit
    ids, w = r["ids"], r["weights"]
    M = ids.shape[0]
    get = expert_fn(inp)
    # (1) silu(sum_j w_j gate_j) * (sum_j w_j up_j), then each expert's W2,
    #     summed without weights
    h1 = r["h1"].reshape(M, k, 2 * I)
    mixed = np.einsum("tk,tkn->tn", w, h1)
    act = oracle.swiglu(mixed, I, L)
    hq, hs = oracle.requantize_hidden(act)
    out1 = np.zeros((M, inp.shape.hidden))
    for t in range(M):
        for j in range(k):
            _, _, w2, s2 = get(int(ids[t, j]))
            out1[t] += oracle.block_scaled_gemm(w2, s2, hq[t:t + 1], hs[t:t + 1])[0]
    # (2) w^2 weighting
    out2 = bf16_round(np.einsum("tk,tkh->th", w * w, r["slots"].reshape(M, k, -1)))
    return bf16_round(out1), out2


def test_negative_controls_fail_tolerance():
    inp = synth.make_inputs(synth.CONFIGS["tiny"].with_(M=8), seed=8)
    r = oracle_layer(inp)
    assert_rows_close(r["combined"], r["combined"])
    bad1, bad2 = _negative_controls(inp, r)
    assert np.all(row_errors(bad1, r["combined"]) > 2e-2)
    assert np.all(row_errors(bad2, r["combined"]) > 2e-2)


# --------------------------------------------------------------------------
# Shared expert
# --------------------------------------------------------------------------

def test_unpack_ue8m0_hand_example():
    word = 127 | (128 << 8) | (126 << 16) | (129 << 24)
    packed = np.full((128, 1), word - (1 << 32), np.int64)   # as int32
    s = oracle.unpack_ue8m0(packed, 128, 512)
    assert s.tolist() == [[1.0, 2.0, 0.5, 4.0]]
    bad = packed.copy()
    bad[5, 0] = 127
    with pytest.raises(ValueError):
        oracle.unpack_ue8m0(bad, 128, 512)


def test_unpack_ue8m0_inverts_packing():
    rng = np.random.default_rng(9)
    s = np.exp2(rng.integers(-6, 6, size=(3, 7))).astype(np.float32)
    packed = synth.pack_ue8m0(torch.from_numpy(s), 384, 896).numpy()
    assert packed.shape == (384, 2)
    assert np.array_equal(oracle.unpack_ue8m0(packed, 384, 896), s)


def _shared_inputs(seed, **kw):
    shape = synth.CONFIGS["tiny"].with_(M=3, shared_inter=128, **kw)
    return synth.make_inputs(shape, seed=seed)


def test_shared_zero_x():
    inp = _shared_inputs(10, x_kind="zero")
    r = oracle.shared_expert(host(inp.x), inp.sw13.numpy(), host(inp.sw13_scale), inp.sw2.numpy(),
                             host(inp.sw2_scale), limit=7.0)
    assert np.all(r["gate_up"] == 0) and np.all(r["out"] == 0)


def test_shared_gate_up_exact_integer_case():
    inp = _shared_inputs(11, x_kind="int", weights="int", pow2_scales=True)
    x = host(inp.x)
    r = oracle.shared_expert(x, inp.sw13.numpy(), host(inp.sw13_scale), inp.sw2.numpy(),
                             host(inp.sw2_scale), limit=7.0)
    # x_s = 2**-6 exactly, so gate_up = BF16(sum_b S[n/128, b] * sum W x) exactly
    W = oracle.e4m3_decode(inp.sw13.numpy())
    S = np.repeat(host(inp.sw13_scale), 128, axis=0)
    nb = W.shape[1] // 128
    inner = np.einsum("nbk,tbk->tnb", W.reshape(-1, nb, 128), x.reshape(-1, nb, 128))
    want = bf16_round(np.einsum("tnb,nb->tn", inner, S))
    assert np.array_equal(r["gate_up"], want)


def test_shared_gate_rows_first():
    """Gate rows come first on the shared expert ("shared_expert" page,
    _DownKernel reads gate at row offset 0 and up at offset inter): a gate
    driven strongly negative silences the output, an up driven negative
    does not."""
    inp = _shared_inputs(12)
    Is = 128
    x = host(inp.x)
    w13 = inp.sw13.numpy().copy()
    s13 = host(inp.sw13_scale)
    base = oracle.shared_expert(x, w13, s13, inp.sw2.numpy(), host(inp.sw2_scale), limit=7.0)
    # pin gate ~ -large: make the gate rows a copy of -(x sign pattern)
    sign = np.where(x[0] >= 0, 1.0, -1.0)
    rowbits = oracle.e4m3_encode(-4.0 * sign)
    w13g = w13.copy()
    w13g[:Is] = rowbits
    r = oracle.shared_expert(x[:1], w13g, s13, inp.sw2.numpy(), host(inp.sw2_scale), limit=7.0)
    assert np.all(r["gate_up"][0, :Is] < -50)
    assert np.max(np.abs(r["act"])) < 1e-6
    assert np.max(np.abs(base["act"][:1])) > 1e-2


def test_combine_check_catches_rounded_or_repeated_weights():
    """The GPU tests' combine check (the oracle's combine of the GPU's own slots
    and weights, one BF16 step, >= 99.9% bit-exact) fails a combine that rounds
    the weights to BF16 or applies them twice, and passes the FP32 sum in
    pick order rounded once."""
    from tests.helpers import check_combine
    rng = np.random.default_rng(31)
    M, k, H = 16, 8, 1024
    slots = torch.from_numpy(bf16_round(rng.standard_normal((M * k, H)))).to(torch.bfloat16)
    w = torch.from_numpy(f32(rng.uniform(0.05, 0.6, (M, k)))).float()
    rows = slots.float().view(M, k, H)
    acc = torch.zeros(M, H)
    for j in range(k):                      # FP32 multiply-add in pick order
        acc = acc + w[:, j:j + 1] * rows[:, j]
    check_combine(slots, w, acc.to(torch.bfloat16))
    wb = w.to(torch.bfloat16).float()
    with pytest.raises(AssertionError):
        check_combine(slots, w, torch.einsum("tk,tkh->th", wb, rows).to(torch.bfloat16))
    with pytest.raises(AssertionError):
        check_combine(slots, w, torch.einsum("tk,tkh->th", w * w, rows).to(torch.bfloat16))
