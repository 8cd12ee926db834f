"""GPU parity of the boundary steps (include/moe_boundary.h) against the oracle
(oracle/boundary.py): the MXFP8 quantisation of the latent ("kimi_k3 ...
ep.comm" page, EpDispatch) bit-exact, codes and scale bytes; the reduce and
RMSNorm of the combine (EpCombine, rms_rstd) within one BF16 step of the
oracle's exact-arithmetic values per element (the device takes the sums,
the mean and the root in FP32), and bit-exact on most elements.

Inputs: seeded BF16 rows of the page's latent width (3584) and token count
per rank (5), partials from 16 ranks; edge widths (32 or 8, and the longest
row the calls take), zero blocks, blocks whose max falls in the saturation
band, rows spanning many binades, an empty call."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from fp8_block_scaled_moe_amd import mxfp8_quantize, reduce_rmsnorm
from oracle import boundary
from oracle.codecs import bf16_round

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LATENT = 3584  # the page's latent width


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in BF16 steps between BF16-valued arrays (same sign or zero)."""
    ia = torch.from_numpy(a.astype(np.float32)).view(torch.int32).numpy() >> 16
    ib = torch.from_numpy(b.astype(np.float32)).view(torch.int32).numpy() >> 16
    return np.abs(ia.astype(np.int64) - ib.astype(np.int64))


def latent_rows(T, D, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    if spread:  # rows and blocks spanning many binades
        x *= 2.0 ** rng.integers(-30, 30, size=(T, 1))
        x *= 2.0 ** rng.integers(-6, 6, size=(T, D // 32, 1)).repeat(32, axis=2).reshape(T, D)
    return bf16_round(x)


def check_mxfp8(x: np.ndarray):
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(DEV)
    q, sf = mxfp8_quantize(xt)
    torch.cuda.synchronize()
    wq, wsf = boundary.mxfp8_quantize(x)
    got_q, got_sf = q.cpu().numpy(), sf.cpu().numpy()
    assert np.array_equal(got_sf, wsf), f"{np.sum(got_sf != wsf)} scale bytes differ"
    bad = np.nonzero(got_q != wq)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][:3]}, {bad[1][:3]}"


@pytest.mark.parametrize("T,D,seed", [(5, LATENT, 1), (3, 32, 2), (2, 16384, 3), (7, 4096 + 96, 4)])
def test_mxfp8_matches_oracle(T, D, seed):
    check_mxfp8(latent_rows(T, D, seed))


def test_mxfp8_special_blocks():
    """Zero blocks, maxima in the saturation band [448, 512) after scaling,
    subnormal BF16 values, exact powers of two."""
    x = latent_rows(4, 256, 5, spread=False)
    x[0, :32] = 0.0
    x[0, 32:64] *= 0.0
    x[1, 64] = 496.0
    x[1, 96] = 255.0
    x[2, :32] = bf16_round(np.full(32, 1e-39))   # subnormal in BF16
    x[2, 40] = 2.0**-133                           # the smallest BF16 subnormal
    x[3, :] = 2.0 ** (np.arange(256) % 254 - 126.0)   # 2^-126 .. 2^127, all finite in BF16
    x[3] = bf16_round(np.where(np.arange(256) % 2, -x[3], x[3]))
    check_mxfp8(x)


def test_mxfp8_empty():
    q, sf = mxfp8_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert q.shape == (0, 64) and sf.shape == (0, 2)


def check_rmsnorm(T, N, D, seed, eps=1e-5, spread=True):
    rng = np.random.default_rng(seed)
    p = bf16_round(rng.standard_normal((T, N, D)) * (2.0 ** rng.integers(-8, 8, size=(T, N, 1)) if spread else 1.0))
    g = bf16_round(rng.uniform(0.5, 1.5, size=D))
    pt = torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).to(DEV)
    gt = torch.from_numpy(g.astype(np.float32)).to(torch.bfloat16).to(DEV)
    latent, out = reduce_rmsnorm(pt, gt, eps)
    torch.cuda.synchronize()
    want_lat, want_out = boundary.reduce_rmsnorm(p, g, eps)
    gl, go = bf16_host(latent), bf16_host(out)
    dl, do = bf16_ulps(gl, want_lat), bf16_ulps(go, want_out)
    assert dl.max() <= 1 and do.max() <= 1, (dl.max(), do.max())
    assert np.mean(dl == 0) >= 0.99 and np.mean(do == 0) >= 0.98
    return gl, go


@pytest.mark.parametrize("T,N,D,seed", [(5, 16, LATENT, 11), (5, 1, LATENT, 12), (1, 3, 8, 13),
                                        (2, 64, 16384, 14), (9, 2, 2048 + 8, 15)])
def test_reduce_rmsnorm_matches_oracle(T, N, D, seed):
    check_rmsnorm(T, N, D, seed)


def test_reduce_rmsnorm_single_rank_is_norm_of_input():
    """N = 1: the latent is the input row itself."""
    rng = np.random.default_rng(16)
    p = bf16_round(rng.standard_normal((3, 1, LATENT)))
    pt = torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).to(DEV)
    gt = torch.ones(LATENT, dtype=torch.bfloat16, device=DEV)
    latent, out = reduce_rmsnorm(pt, gt, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(latent), p[:, 0])
    assert bf16_ulps(bf16_host(out), boundary.rms_norm(p[:, 0], np.ones(LATENT), 0.0)).max() <= 1


def test_reduce_rmsnorm_zero_rows_and_no_latent():
    pt = torch.zeros((2, 4, 256), dtype=torch.bfloat16, device=DEV)
    gt = torch.ones(256, dtype=torch.bfloat16, device=DEV)
    latent, out = reduce_rmsnorm(pt, gt, 1e-5, want_latent=False)
    torch.cuda.synchronize()
    assert latent is None and not out.float().abs().max().item()
