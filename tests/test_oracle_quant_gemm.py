"""Pins for the oracle's FP8 block quantiser and block-scaled GEMM.

Pinned against: exact integer cases (scales exactly 2**-6, pow2 weight scales,
integer weights -> exact integer matmul), the all-ones-scale case reducing to a
plain float64 matmul (library routine), single-scale probes (only the affected
rows move, by exactly that block's contribution), the rounding-error bound of
e4m3, and the UE8M0 power-of-two property.
"""

import numpy as np
import pytest

import oracle
from oracle import block_scaled_gemm, e4m3_decode, e4m3_encode, f32, quantize_blocks


def _int_x(rng, R, K):
    v = rng.integers(-7, 8, size=(R, K // 128, 128))
    v[..., 0] = np.where(rng.integers(0, 2, size=(R, K // 128)) == 0, -7, 7)
    return rng.permuted(v, axis=2).reshape(R, K).astype(np.float64)


def test_quant_exact_integer_case():
    rng = np.random.default_rng(0)
    x = _int_x(rng, 3, 512)
    for recip in (True, False):
        q, s = quantize_blocks(x, ue8m0=False, reciprocal=recip)
        assert np.all(s == 2.0**-6)
        assert np.array_equal(e4m3_decode(q), 64 * x)


def test_quant_zero_rows():
    q, s = quantize_blocks(np.zeros((2, 256)), ue8m0=False, reciprocal=True)
    assert np.all(q == 0)
    assert np.all(s == f32(f32(1e-10) / 448.0))
    # with UE8M0 the scale is floored at 1e-10 before rounding up to a power of
    # two: 1e-10 lies in [2**-34, 2**-33), so the scale is 2**-33
    q, s = quantize_blocks(np.zeros((1, 128)), ue8m0=True, reciprocal=True)
    assert np.all(q == 0)
    assert s[0, 0] == 2.0**-33
    # a block with amax just under 448e-10 is floored too; one well above is not
    x = np.zeros((2, 128))
    x[0, 3] = 1e-9
    x[1, 3] = 1e-3
    q, s = quantize_blocks(x, ue8m0=True, reciprocal=True)
    assert s[0, 0] == 2.0**-33
    assert s[1, 0] == 2.0**-18   # 1e-3 / 448 = 2.23e-6 in [2**-19, 2**-18)


def test_quant_error_bound_and_amax():
    rng = np.random.default_rng(1)
    x = f32(rng.standard_normal((8, 1024)) * np.exp2(rng.integers(-8, 8, size=(8, 1))))
    for ue8m0 in (False, True):
        for recip in (False, True):
            q, s = quantize_blocks(x, ue8m0=ue8m0, reciprocal=recip)
            d = e4m3_decode(q).reshape(8, 8, 128) * s[..., None]
            xb = x.reshape(8, 8, 128)
            # half an e4m3 ulp: 2**-4 relative for normals, 2**-10 * s absolute below
            err = np.abs(d - xb)
            bound = np.maximum(np.abs(xb) * 2.0**-4, s[..., None] * 2.0**-10) * (1 + 1e-6)
            assert np.all(err <= bound)
            # the block maximum maps to (close to) 448 without ue8m0
            if not ue8m0:
                top = np.max(np.abs(e4m3_decode(q).reshape(8, 8, 128)), axis=2)
                assert np.all(top == 448.0)
            else:
                m, _ = np.frexp(s)
                assert np.all(m == 0.5)
                assert np.all(s >= np.abs(xb).max(axis=2) / 448.0)


def test_ue8m0_round_up():
    s = np.array([1.0, 1.5, 0.75, 2.0**-20, 3.0 * 2.0**-30])
    assert np.array_equal(oracle.ue8m0_round_up(s), [1.0, 2.0, 1.0, 2.0**-20, 2.0**-28])


def _pow2(rng, shape):
    return np.exp2(rng.integers(-2, 3, size=shape)).astype(np.float64)


def test_gemm_exact_integer_case():
    rng = np.random.default_rng(2)
    N, K, R = 256, 384, 3
    W = rng.integers(-4, 5, size=(N, K))
    S = _pow2(rng, (N // 128, K // 128))
    x = _int_x(rng, R, K)
    xq, xs = quantize_blocks(x, ue8m0=False, reciprocal=True)
    y = block_scaled_gemm(e4m3_encode(W), S, xq, xs)
    # exact: sum over blocks of S * (1/64) * sum W * 64 x, in integers
    Wb = W.reshape(N, K // 128, 128).astype(np.int64)
    xb = x.reshape(R, K // 128, 128).astype(np.int64)
    inner = np.einsum("nbk,rbk->rnb", Wb, xb)  # integer
    Sf = np.repeat(S, 128, axis=0)
    exact = np.einsum("rnb,nb->rn", inner.astype(np.float64), Sf)  # pow2 * int: exact
    assert np.array_equal(y, exact)
    assert np.array_equal(f32(y), y)


def test_gemm_unit_scales_is_plain_matmul():
    rng = np.random.default_rng(3)
    N, K, R = 256, 512, 4
    wq = e4m3_encode(f32(rng.standard_normal((N, K))))
    aq = e4m3_encode(f32(rng.standard_normal((R, K))))
    y = block_scaled_gemm(wq, np.ones((2, 4)), aq, np.ones((R, 4)))
    ref = e4m3_decode(aq) @ e4m3_decode(wq).T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-9)


def test_gemm_single_scale_probe():
    """Changing one weight scale S[nb, kb] moves only rows of block nb, each by
    exactly that block's contribution (after the nvfp4-megamoe-kernel README's
    single-element scale probes)."""
    rng = np.random.default_rng(4)
    N, K, R = 384, 640, 2
    wq = e4m3_encode(f32(rng.standard_normal((N, K))))
    aq = e4m3_encode(f32(rng.standard_normal((R, K))))
    S = rng.uniform(0.25, 4, size=(N // 128, K // 128))
    A = rng.uniform(0.25, 4, size=(R, K // 128))
    y0 = block_scaled_gemm(wq, S, aq, A)
    for nb, kb in [(0, 0), (1, 3), (2, 4), (0, 4)]:
        S1 = S.copy()
        S1[nb, kb] *= 3.0
        y1 = block_scaled_gemm(wq, S1, aq, A)
        rows = np.arange(N) // 128 == nb
        assert np.array_equal(y1[:, ~rows], y0[:, ~rows])
        blk = slice(kb * 128, kb * 128 + 128)
        contrib = e4m3_decode(aq[:, blk]) @ e4m3_decode(wq[rows, blk]).T  # [R, 128]
        want = y0[:, rows] + 2.0 * S[nb, kb] * A[:, kb:kb + 1] * contrib
        np.testing.assert_allclose(y1[:, rows], want, rtol=1e-12, atol=1e-12)
    # activation scale probe: only block kb of every row moves
    A1 = A.copy()
    A1[1, 2] *= 0.5
    y2 = block_scaled_gemm(wq, S, aq, A1)
    assert np.array_equal(y2[0], y0[0])
    blk = slice(256, 384)
    contrib = e4m3_decode(aq[1, blk]) @ e4m3_decode(wq[:, blk]).T  # [N]
    want = y0[1] - 0.5 * A[1, 2] * np.repeat(S[:, 2], 128) * contrib
    np.testing.assert_allclose(y2[1], want, rtol=1e-12, atol=1e-12)


def test_pins_catch_transposed_scale(monkeypatch):
    """Indexing the weight scale as [kb, nb] instead of [nb, kb] fails a pin."""
    real = oracle.moe.block_scaled_gemm

    def wrong(wq, ws, aq, as_):
        ws = np.asarray(ws)
        nb, kb = ws.shape
        flipped = ws.T.reshape(-1)[: nb * kb].reshape(nb, kb) if nb != kb else ws.T
        return real(wq, flipped, aq, as_)

    monkeypatch.setitem(globals(), "block_scaled_gemm", wrong)
    with pytest.raises(AssertionError):
        test_gemm_single_scale_probe()
