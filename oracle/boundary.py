"""The boundary steps either side of the routed path in the expert-parallel
pipeline, in their one-GPU form, in float64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"kimi_k3 ... ep.comm" page:
  * EpDispatch: each token's BF16 latent is quantised to MXFP8 (E8M0 scale
    per 32 values, e4m3 elements) before it is sent to the experts' ranks;
    the scales are stored one byte per 32-block in plain block
    order.
  * EpCombine: a token's per-rank BF16 partials are summed in FP32 in rank
    order and rounded once to BF16 (the routed latent), then normalised:
    an FP32 sum of squares, rstd = rsqrt(total / D + eps) with the division
    correctly rounded (rms_rstd), and each output x * rstd * w rounded once
    to BF16.

The page calls the scale helpers (mx_exponent, mx_rescale) without showing
them. Reading taken: the OCP Microscaling (MX) v1.0 definition for an e4m3
element format, whose largest power of two is 2^8: the shared exponent of a
block is floor(log2(max |v|)) - 8, kept within E8M0's [-127, 127]; the
scale byte is that exponent + 127; each element is e4m3(v * 2^-exponent),
round to nearest even, saturating at +-448 (a block max in [448, 512) maps
above 448 and saturates). An all-zero block gets exponent -127 (byte 0)
and zero elements.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .codecs import bf16_round, e4m3_encode, f32

MX_BLOCK = 32
E4M3_EMAX = 8          # floor(log2(448)): the largest power of two of the e4m3 grid
E8M0_BIAS = 127


def e8m0_decode(codes) -> np.ndarray:
    """Value of each E8M0 byte: 2^(b - 127), NaN for 0xFF."""
    b = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(b == 0xFF, np.nan, np.exp2(b - float(E8M0_BIAS)))


def mxfp8_quantize(x) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 of rows x [T, D] (BF16 values), D a multiple of 32.

    Returns the e4m3 codes [T, D] (uint8) and the E8M0 scale bytes
    [T, D / 32] (uint8), block b of row t covering columns 32b .. 32b + 31."""
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    if D % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blocks = x.reshape(T, D // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        # floor(log2(amax)) exactly: frexp gives amax = f * 2^ex with f in [0.5, 1)
        _, ex = np.frexp(amax)
    shared = np.where(amax > 0, ex.astype(np.int64) - 1 - E4M3_EMAX, -E8M0_BIAS)
    shared = np.clip(shared, -E8M0_BIAS, E8M0_BIAS)
    scaled = f32(blocks * np.exp2(-shared.astype(np.float64))[..., None])
    codes = e4m3_encode(scaled).astype(np.uint8)
    return codes.reshape(T, D), (shared + E8M0_BIAS).astype(np.uint8)


def reduce_latent(partials) -> np.ndarray:
    """The routed latent of each token from its per-rank BF16 partials
    [T, N, D]: their sum in rank order rounded once to BF16 (EpCombine).
    The sum is taken exactly (float64; at most a few hundred terms of BF16
    values), so the only rounding is the final one."""
    p = np.asarray(partials, dtype=np.float64)
    return bf16_round(p.sum(axis=1))


def rms_norm(latent, gamma, eps: float) -> np.ndarray:
    """vLLM's RMSNorm of BF16 rows latent [T, D] with BF16 gains gamma [D]
    (EpCombine, rms_rstd): rstd = 1 / sqrt(sum(x^2) / D + eps), and each
    output BF16(x * rstd * gamma). The sum of squares, the mean and the
    reciprocal square root are exact here (float64); the GPU takes them in
    FP32, within a few FP32 roundings."""
    x = np.asarray(latent, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    D = x.shape[-1]
    total = (x * x).sum(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(total / D + float(f32(eps)))
    return bf16_round(x * rstd * g)


def reduce_rmsnorm(partials, gamma, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Both combine-side steps: (routed latent, its RMSNorm), each BF16."""
    latent = reduce_latent(partials)
    return latent, rms_norm(latent, gamma, eps)
