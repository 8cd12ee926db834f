"""The FP4 form of the routed-expert step, in float64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The nvfp4-megamoe-kernel README ("Data Formats", "Bugs Found & Fixed") runs
the same slot pipeline with NVFP4 operands on one rank's share of experts:
packed E2M1 weights with one UE4M3 scale per 16 values along K, activations
staged from BF16 to E2M1 with a per-16 scale of block_max / 6, SiLU times up
per slot, and the routing weights applied once, in the final scatter over
the slots whose expert is local. Where the README leaves a step open, the
reading taken is stated on the function (and listed in the design notes).

E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; magnitudes
0, 0.5, 1, 1.5, 2, 3, 4, 6. UE4M3 scales are e4m3 bytes with the sign clear.
"""

from __future__ import annotations

from typing import Callable, Dict, Tuple

import numpy as np

from .codecs import bf16_round, e4m3_decode, e4m3_encode, f32
from .moe import combine, route, silu_f32

GROUP = 16
E2M1_MAX = 6.0
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# code c: magnitude of c & 7, negative when bit 3 is set
E2M1_VALUES = np.concatenate([E2M1_MAGNITUDES, -E2M1_MAGNITUDES])


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_VALUES[np.asarray(codes, dtype=np.int64) & 0xF]


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code, ties to the even code (mantissa bit clear),
    saturating at +-6; the sign of -0.0 is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    dist = np.abs(a[..., None] - E2M1_MAGNITUDES)            # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    # among the nearest magnitudes prefer an even code; exactly one is even
    # at every tie because neighbouring codes alternate parity
    even = tied & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tied, axis=-1))
    return (pick | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def pack_e2m1(codes) -> np.ndarray:
    """Two codes per byte along the last axis: element 2i in the low nibble,
    element 2i+1 in the high nibble (reading: the README gives the packing as
    two values per byte without the order; low-first is the order of the
    OCP FP4 pair types)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_fp4_blocks(v) -> Tuple[np.ndarray, np.ndarray]:
    """Per 16 consecutive values of each row ("Bugs Found & Fixed", bug 2:
    stage_activation): scale = block_max / 6 stored as UE4M3, codes the
    nearest E2M1 of v / scale, signed.

    Readings: block_max = max |v|; the quotient block_max / 6 is taken in
    FP32 and then rounded to e4m3 (nearest, ties to even, saturating at
    448); each value is divided by the decoded stored scale in FP32 and
    rounded to E2M1 (nearest, ties to even, saturating at 6); a block whose
    stored scale is 0 gets all-zero codes.

    Returns codes [R, K] (unpacked, uint8) and scale bytes [R, K/16]."""
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    if K % GROUP:
        raise ValueError("row length must be a multiple of 16")
    b = v.reshape(R, K // GROUP, GROUP)
    amax = np.abs(b).max(axis=2)
    s_code = e4m3_encode(f32(amax / E2M1_MAX))
    s = e4m3_decode(s_code)
    safe = np.where(s > 0, s, 1.0)
    q = e2m1_encode(f32(b / safe[..., None]))
    q = np.where((s > 0)[..., None], q, 0).astype(np.uint8)
    return q.reshape(R, K), s_code


def fp4_block_gemm(w_codes, w_scale, a_codes, a_scale) -> np.ndarray:
    """y[r, n] = sum_g dec(Sw[n, g]) * dec(Sa[r, g]) *
    sum_{i in group g} e2m1(W[n, i]) * e2m1(A[r, i]), unrounded float64
    (every product and every 16-term sum is exact in float64).

    w_codes [N, K] and a_codes [R, K] unpacked E2M1 codes; w_scale [N, K/16]
    and a_scale [R, K/16] e4m3 bytes."""
    W = e2m1_decode(w_codes)
    A = e2m1_decode(a_codes)
    N, K = W.shape
    R = A.shape[0]
    G = K // GROUP
    inner = np.einsum("ngi,rgi->rng", W.reshape(N, G, GROUP), A.reshape(R, G, GROUP))
    sw = e4m3_decode(w_scale)                      # [N, G]
    sa = e4m3_decode(a_scale)                      # [R, G]
    return np.einsum("rng,ng,rg->rn", inner, sw, sa)


ExpertFn4 = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]


def moe_decode_fp4(x, logits, bias, expert: ExpertFn4, *, top_k: int, routed_scale: float,
                   limit: float, local_begin: int, local_count: int, inter: int) -> Dict:
    """One rank's share of the FP4 routed step (README: slot representation,
    "Data Formats", bugs 2, 6 and 7).

    Routing over all experts as in the FP8 form; a slot (token, pick) is
    local when its expert lies in [local_begin, local_begin + local_count).
    For a local slot: x staged to FP4; L1 = BF16(FP32(GEMM)) with gate rows
    first then up rows (the README's [gate; up] concatenation); gate =
    min(gate, L), up = clamp(up, -L, L) (reading: the clamped SwiGLU of the
    FP8 form, with the limit a parameter); act = BF16(silu(gate) * up) in FP32
    steps; act staged to FP4; L2 = BF16(FP32(GEMM)). Non-local slot rows are
    zero; combined applies the routing weights once, so only local slots
    contribute.

    expert(e_local) returns (W13 packed [2I, H/2], S13 [2I, H/16], W2 packed
    [H, I/2], S2 [H, I/16])."""
    x = np.asarray(x, dtype=np.float64)
    M, H = x.shape
    ids, weights, _ = route(logits, bias, top_k, routed_scale)
    x_q, x_s = quantize_fp4_blocks(f32(x))
    R = M * top_k
    local = (ids.reshape(-1) >= local_begin) & (ids.reshape(-1) < local_begin + local_count)
    h1 = np.zeros((R, 2 * inter))
    act = np.zeros((R, inter))
    h_q = np.zeros((R, inter), dtype=np.uint8)
    h_s = np.zeros((R, inter // GROUP), dtype=np.uint8)
    slots = np.zeros((R, H))
    for e in np.unique(ids.reshape(-1)[local]):
        w13, s13, w2, s2 = expert(int(e) - local_begin)
        rows = np.nonzero(ids.reshape(-1) == e)[0]
        t = rows // top_k
        g1 = bf16_round(fp4_block_gemm(unpack_e2m1(w13), s13, x_q[t], x_s[t]))
        h1[rows] = g1
        gate = np.minimum(g1[:, :inter], limit)
        up = np.clip(g1[:, inter:], -limit, limit)
        a = bf16_round(silu_f32(gate) * up)
        act[rows] = a
        q, s = quantize_fp4_blocks(a)
        h_q[rows] = q
        h_s[rows] = s
        slots[rows] = bf16_round(fp4_block_gemm(unpack_e2m1(w2), s2, q, s))
    combined = combine(slots, weights)
    return dict(ids=ids, weights=weights, x_q=x_q, x_s=x_s, local=local, h1=h1, act=act,
                h_q=h_q, h_s=h_s, slots=slots, combined=combined)
