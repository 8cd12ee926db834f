"""Pins of the FP4 oracle (oracle/fp4.py) against what the nvfp4-megamoe-kernel
README and the E2M1 definition fix: the code table, nearest-even encoding
with saturation, the block_max / 6 staging, exact block sums when every
scale is 1 (the README's constant-scale diagnostic), single-scale probes
(a scale touches only its own row and group), brute force on tiny inputs,
local-slot filtering and the slot invariants (SiLU per slot, weights once).
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from oracle import fp4
from oracle.codecs import e4m3_decode, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.json")
ONE = int(e4m3_encode(np.array([1.0]))[0])  # e4m3 byte of 1.0


@pytest.fixture(scope="module")
def gold():
    with open(GOLDEN) as f:
        return json.load(f)


def test_e2m1_table(gold):
    for c, v in gold["codes"].items():
        got = fp4.e2m1_decode(int(c))
        assert got == v and np.signbit(got) == np.signbit(v)


def test_e2m1_round_trip_every_code():
    codes = np.arange(16)
    assert np.array_equal(fp4.e2m1_encode(fp4.e2m1_decode(codes)), codes)


def test_e2m1_ties_and_saturation(gold):
    for v, c in gold["nearest_ties_to_even"] + gold["saturating"]:
        assert int(fp4.e2m1_encode(v)) == c, v


def test_e2m1_nearest_everywhere():
    """Off the midpoints the code is the plain nearest value."""
    rng = np.random.default_rng(0)
    v = rng.uniform(-8, 8, 20000)
    got = fp4.e2m1_decode(fp4.e2m1_encode(v))
    err = np.abs(got - np.clip(v, -6, 6))
    best = np.min(np.abs(np.clip(v, -6, 6)[:, None] - fp4.E2M1_VALUES[None, :]), axis=1)
    assert np.all(err == best)


def test_packing_nibble_order(gold):
    ex = gold["packing_example"]
    assert fp4.pack_e2m1(np.array(ex["codes"], np.uint8)).tolist() == ex["bytes"]
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    assert np.array_equal(fp4.unpack_e2m1(fp4.pack_e2m1(c)), c)


def test_staging_exact_grid_values():
    """Blocks whose values are E2M1 grid points times 2^k with a +-6 * 2^k
    present: scale = 2^k exactly (a power of two is exact in e4m3) and every
    code is recovered."""
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, size=(4, 64)).astype(np.uint8)
    codes[:, ::16] = 7  # a 6 in every block
    k = rng.integers(-5, 4, size=(4, 4))
    v = fp4.e2m1_decode(codes).reshape(4, 4, 16) * np.exp2(k)[..., None]
    q, s = fp4.quantize_fp4_blocks(v.reshape(4, 64))
    assert np.array_equal(e4m3_decode(s), np.exp2(k))
    assert np.array_equal(fp4.e2m1_decode(q), fp4.e2m1_decode(codes))  # (-0 and +0 compare equal)


def test_staging_scale_is_block_max_over_6():
    """The stored scale is block_max / 6, not block_max (the README's bug 2B),
    and negatives survive (bug 2A: no clamp at zero)."""
    v = np.zeros((1, 16))
    v[0, 3] = -9.0
    v[0, 5] = 1.5
    q, s = fp4.quantize_fp4_blocks(v)
    assert e4m3_decode(s)[0, 0] == 1.5
    assert fp4.e2m1_decode(q[0, 3]) == -6.0 and fp4.e2m1_decode(q[0, 5]) == 1.0


def test_staging_zero_block():
    q, s = fp4.quantize_fp4_blocks(np.zeros((2, 32)))
    assert not q.any() and not s.any()


def test_gemm_constant_scales_is_plain_dot():
    """Every scale 1.0 (the README's constant-scale diagnostic): the GEMM is
    the plain dot product of the decoded codes."""
    rng = np.random.default_rng(3)
    W = rng.integers(0, 16, size=(5, 48)).astype(np.uint8)
    A = rng.integers(0, 16, size=(3, 48)).astype(np.uint8)
    ones_w = np.full((5, 3), ONE, np.uint8)
    ones_a = np.full((3, 3), ONE, np.uint8)
    got = fp4.fp4_block_gemm(W, ones_w, A, ones_a)
    assert np.array_equal(got, fp4.e2m1_decode(A) @ fp4.e2m1_decode(W).T)


def test_gemm_brute_force_and_scale_probes():
    rng = np.random.default_rng(4)
    N, R, K = 4, 3, 48
    W = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    A = rng.integers(0, 16, size=(R, K)).astype(np.uint8)
    sw = rng.integers(0x20, 0x50, size=(N, K // 16)).astype(np.uint8)
    sa = rng.integers(0x20, 0x50, size=(R, K // 16)).astype(np.uint8)
    got = fp4.fp4_block_gemm(W, sw, A, sa)
    for r in range(R):
        for n in range(N):
            acc = 0.0
            for i in range(K):
                g = i // 16
                acc += (fp4.e2m1_decode(W[n, i]) * e4m3_decode(sw[n, g]) *
                        fp4.e2m1_decode(A[r, i]) * e4m3_decode(sa[r, g]))
            assert got[r, n] == pytest.approx(acc, rel=1e-15, abs=1e-300)
    # a weight scale touches only its row; an activation scale only its token
    sw2 = sw.copy()
    sw2[2, 1] = 0x60
    d = fp4.fp4_block_gemm(W, sw2, A, sa) != got
    assert not d[:, [0, 1, 3]].any()
    sa2 = sa.copy()
    sa2[1, 2] = 0x61
    d = fp4.fp4_block_gemm(W, sw, A, sa2) != got
    assert not d[[0, 2]].any()


def _fp4_layer_inputs(seed, E=12, local=(4, 5), M=5, H=64, I=32, k=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, H))
    logits = rng.standard_normal((M, E)) * 2
    bias = rng.standard_normal(E) * 0.1
    lb, lc = local
    w13 = rng.integers(0, 256, size=(lc, 2 * I, H // 2)).astype(np.uint8)
    s13 = rng.integers(0x28, 0x38, size=(lc, 2 * I, H // 16)).astype(np.uint8)
    w2 = rng.integers(0, 256, size=(lc, H, I // 2)).astype(np.uint8)
    s2 = rng.integers(0x28, 0x38, size=(lc, H, I // 16)).astype(np.uint8)
    expert = lambda e: (w13[e], s13[e], w2[e], s2[e])  # noqa: E731
    kw = dict(top_k=k, routed_scale=2.5, limit=7.0, local_begin=lb, local_count=lc, inter=I)
    return x, logits, bias, expert, kw


def test_layer_local_slots_only():
    x, logits, bias, expert, kw = _fp4_layer_inputs(5)
    r = fp4.moe_decode_fp4(x, logits, bias, expert, **kw)
    ids = r["ids"].reshape(-1)
    lb, lc = kw["local_begin"], kw["local_count"]
    local = (ids >= lb) & (ids < lb + lc)
    assert np.array_equal(r["local"], local) and local.any() and (~local).any()
    assert not r["slots"][~local].any()
    # combined = sum over local slots of weight x slot, rounded once
    w = r["weights"].reshape(-1)
    M, k = r["ids"].shape
    want = oracle.bf16_round(np.einsum("tk,tkh->th", (w * local).reshape(M, k),
                                       r["slots"].reshape(M, k, -1)))
    assert np.array_equal(r["combined"], want)


def test_layer_matches_stepwise_definition():
    """Every local slot recomputed from the definitions by hand."""
    x, logits, bias, expert, kw = _fp4_layer_inputs(6)
    r = fp4.moe_decode_fp4(x, logits, bias, expert, **kw)
    I, L, k = kw["inter"], kw["limit"], kw["top_k"]
    xq, xs = fp4.quantize_fp4_blocks(oracle.f32(x))
    for s in np.nonzero(r["local"])[0]:
        e = int(r["ids"].reshape(-1)[s]) - kw["local_begin"]
        w13, s13, w2, s2 = expert(e)
        t = s // k
        h = oracle.bf16_round(fp4.fp4_block_gemm(fp4.unpack_e2m1(w13), s13, xq[t:t + 1], xs[t:t + 1]))[0]
        gate, up = np.minimum(h[:I], L), np.clip(h[I:], -L, L)   # gate rows first
        a = oracle.bf16_round(oracle.silu_f32(gate) * up)
        q, sc = fp4.quantize_fp4_blocks(a[None])
        y = oracle.bf16_round(fp4.fp4_block_gemm(fp4.unpack_e2m1(w2), s2, q, sc))[0]
        assert np.array_equal(r["slots"][s], y)


def test_layer_negative_controls():
    """SiLU of the weight-summed paths and weights applied on both GEMMs (the
    README's bugs 6 and 7) give visibly different outputs."""
    x, logits, bias, expert, kw = _fp4_layer_inputs(7, local=(0, 12))
    r = fp4.moe_decode_fp4(x, logits, bias, expert, **kw)
    M, k = r["ids"].shape
    w = r["weights"]
    rows = r["slots"].reshape(M, k, -1)
    squared = oracle.bf16_round(np.einsum("tk,tkh->th", w * w, rows))
    rms = np.sqrt(np.mean(r["combined"] ** 2, axis=1))
    assert np.all(np.max(np.abs(squared - r["combined"]), axis=1) > 2e-2 * rms)
    I, L = kw["inter"], kw["limit"]
    h1 = r["h1"].reshape(M, k, -1)
    summed = np.einsum("tk,tkn->tn", w, h1)
    act_sum = oracle.silu_f32(np.minimum(summed[:, :I], L)) * np.clip(summed[:, I:], -L, L)
    act_slot = np.einsum("tk,tki->ti", w, r["act"].reshape(M, k, -1))
    assert np.max(np.abs(act_sum - act_slot)) > 1e-2 * np.max(np.abs(act_slot))


# ---------------------------------------------------------------------------
# Mutations planted in the oracle: each must make one of the pins above fail.
# ---------------------------------------------------------------------------

def _ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), fp4.E2M1_MAX)
    dist = np.abs(a[..., None] - fp4.E2M1_MAGNITUDES)
    pick = len(fp4.E2M1_MAGNITUDES) - 1 - np.argmin(dist[..., ::-1], axis=-1)  # ties upward
    return (pick | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def _high_nibble_first(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 1::2] & 0xF) | ((c[..., 0::2] & 0xF) << 4)


_orig_gemm = fp4.fp4_block_gemm


def _scales_reversed(W, sw, A, sa):
    return _orig_gemm(W, sw[:, ::-1], A, sa)


@pytest.mark.parametrize("attr,mutant,pin", [
    ("e2m1_encode", _ties_away, "ties"),
    ("pack_e2m1", _high_nibble_first, "packing"),
    ("E2M1_MAX", 1.0, "scale"),
    ("fp4_block_gemm", _scales_reversed, "gemm"),
])
def test_planted_mistakes_fail_a_pin(monkeypatch, gold, attr, mutant, pin):
    monkeypatch.setattr(fp4, attr, mutant)
    run = {"ties": lambda: test_e2m1_ties_and_saturation(gold),
           "packing": lambda: test_packing_nibble_order(gold),
           "scale": test_staging_scale_is_block_max_over_6,
           "gemm": test_gemm_brute_force_and_scale_probes}[pin]
    with pytest.raises(AssertionError):
        run()
