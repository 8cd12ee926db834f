"""The routed-expert step, step by step, in float64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each function states the passage it follows. Rounding points are the pages':
binary32 where the pages compute in FP32 (scores, keys, the routing
normaliser, scales, the quantiser's products and quotients, the GEMM results
and the activation), BF16 where they store BF16. Sums inside a GEMM are taken
in float64; with FP8 x FP8 products every 128-element block sum is exact in
float64, so only the final binary32 rounding is taken.

Where an operation maps a float64 value that is an exact function of binary32
operands to binary32 (one add, multiply or divide of two binary32 values),
computing in float64 and rounding once gives the correctly rounded binary32
result, because 53 >= 2 * 24 + 2 (double rounding is innocuous at that width).
"""

from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np

from .codecs import FP8_MAX, E4M3_VALUES, bf16_round, e4m3_encode, f32

TILE = 128
AMAX_FLOOR = float(np.float32(1e-10))


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

def sigmoid_f32(z: np.ndarray) -> np.ndarray:
    """binary32 rounding of 1 / (1 + exp(-z)) evaluated in float64.

    The "mega_moe" page (top_k_pick docstring) computes the sigmoid with an
    approximate exp and divide, a few units in the last place off; the reading
    taken here is the correctly rounded FP32 sigmoid, which the GPU side also
    computes."""
    with np.errstate(over="ignore"):
        return f32(1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64))))


def route(logits, bias, top_k: int, routed_scale: float):
    """Biased sigmoid top-k ("mega_moe" page, top_k_pick and _ordered).

    For each token: s_e = sigmoid(z_e) in FP32; key_e = FP32(s_e + bias_e);
    the top_k experts by key, highest first, equal keys going to the lower
    expert index; weights are the picked *unbiased* scores divided by their
    FP32 sum (accumulated in pick order) and multiplied by routed_scale, each
    step rounded to FP32.

    Returns ids [M, k] int32 (pick order), weights [M, k] float64 (binary32
    values) and the scores s [M, E]."""
    z = f32(logits)
    M, E = z.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    s = sigmoid_f32(z)
    key = f32(s + f32(bias)[None, :])
    ids = np.empty((M, top_k), np.int32)
    weights = np.empty((M, top_k), np.float64)
    scale = f32(routed_scale)
    for t in range(M):
        # lexsort: last key is primary -> key descending, then index ascending.
        order = np.lexsort((np.arange(E), -key[t]))
        picked = order[:top_k]
        total = 0.0
        for e in picked:
            total = float(f32(total + s[t, e]))
        ids[t] = picked
        weights[t] = f32(f32(s[t, picked] / total) * scale)
    return ids, weights, s


# --------------------------------------------------------------------------
# Quantisation
# --------------------------------------------------------------------------

def ue8m0_round_up(s: np.ndarray) -> np.ndarray:
    """Smallest power of two >= s (for positive binary32 s): the exponent is
    kept when the mantissa is zero and incremented otherwise ("mega_moe" page,
    epilogue, the ue8m0 branch; "shared_expert" page, _group_scale)."""
    m, e = np.frexp(np.asarray(s, dtype=np.float64))  # s = m * 2**e
    return np.where(m == 0.5, s, np.ldexp(1.0, e))


def quantize_blocks(v, ue8m0: bool, reciprocal: bool):
    """FP8 per 128-element block of each row of v (binary32 values).

    amax = max(1e-10, max |v|); s = FP32(amax / 448); with ue8m0, s is floored
    at 1e-10 and then rounded up to a power of two; then either q = e4m3(FP32(v * FP32(1 / s)))
    (reciprocal=True: the activation quantiser of the "mega_moe" epilogue and
    of "shared_expert" _GateUpKernel/_DownKernel, via _group_scale) or
    q = e4m3(FP32(v / s)) (reciprocal=False: "mega_moe" hidden_block).

    Returns codes [R, K] uint8 and scales [R, K/128] (binary32 values)."""
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    if K % TILE:
        raise ValueError("row length must be a multiple of 128")
    b = v.reshape(R, K // TILE, TILE)
    amax = np.maximum(np.abs(b).max(axis=2), AMAX_FLOOR)
    s = f32(amax / FP8_MAX)
    if ue8m0:
        s = ue8m0_round_up(np.maximum(s, AMAX_FLOOR))
    if reciprocal:
        scaled = f32(b * f32(1.0 / s)[..., None])
    else:
        scaled = f32(b / s[..., None])
    return e4m3_encode(scaled).reshape(R, K), s


def requantize_hidden(act):
    """FP8 hidden of the routed path: per 128, s = FP32(max(amax, 1e-10) / 448),
    never UE8M0, q = e4m3(act / s) ("mega_moe" page, hidden_block)."""
    return quantize_blocks(act, ue8m0=False, reciprocal=False)


# --------------------------------------------------------------------------
# Block-scaled GEMM
# --------------------------------------------------------------------------

def block_scaled_gemm(wcodes, wscale, acodes, ascale) -> np.ndarray:
    """y[r, n] = sum_b wscale[n/128, b] * ascale[r, b] *
    sum_{i in block b} dec(W[n, i]) * dec(A[r, i]), unrounded float64.

    The scale-once-per-K-block structure is the one the "mega_moe" page's
    module docstring describes (each K block's unscaled partial, scaled and
    summed in the epilogue; the GEMM1 and GEMM2 scale-sums in `epilogue`).

    wcodes [N, K] uint8 e4m3; wscale [N/128, K/128]; acodes [R, K] uint8;
    ascale [R, K/128]."""
    wcodes = np.asarray(wcodes)
    acodes = np.asarray(acodes)
    N, K = wcodes.shape
    R = acodes.shape[0]
    nb = K // TILE
    W = E4M3_VALUES[wcodes].reshape(N, nb, TILE).transpose(1, 0, 2)   # [nb, N, 128]
    A = E4M3_VALUES[acodes].reshape(R, nb, TILE).transpose(1, 2, 0)   # [nb, 128, R]
    inner = np.matmul(W, A)                                          # [nb, N, R], exact
    ws = np.repeat(np.asarray(wscale, dtype=np.float64), TILE, axis=0)  # [N, nb]
    a_s = np.asarray(ascale, dtype=np.float64)                       # [R, nb]
    return np.einsum("nb,rb,bnr->rn", ws, a_s, inner)


# --------------------------------------------------------------------------
# Clamped SwiGLU
# --------------------------------------------------------------------------

def silu_f32(gate) -> np.ndarray:
    """gate / (1 + exp(-gate)) as the pages evaluate it in FP32: each of the
    exp, the add and the divide rounded to binary32 in that order (the exp
    correctly rounded, the reading taken for the pages' FP32 exp)."""
    gate = np.asarray(gate, dtype=np.float64)
    with np.errstate(over="ignore"):
        e = f32(np.exp(-gate))
    return f32(gate / f32(1.0 + e))


def swiglu(h1, inter: int, limit: float) -> np.ndarray:
    """Routed clamped SwiGLU ("mega_moe" page, hidden_block; the GEMM1 row
    order "up rows, then gate rows" of the module docstring).

    up = clamp(h1[:, :I], -L, L); gate = min(h1[:, I:], L) (the gate is not
    clamped from below); act = (gate / (1 + exp(-gate))) * up with every
    operation rounded to FP32 in the page's order. The FP8 hidden codes are
    decided from act, so the rounding points are kept exactly."""
    h1 = np.asarray(h1, dtype=np.float64)
    up = np.clip(h1[:, :inter], -limit, limit)
    gate = np.minimum(h1[:, inter:], limit)
    return f32(silu_f32(gate) * up)


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------

def combine(slots, weights) -> np.ndarray:
    """combined[t] = BF16(FP32(sum_j w[t, j] * slot[t*k + j])): the routing
    weights applied exactly once, at the end, to the unweighted BF16 slot rows
    (nvfp4-megamoe-kernel README, "slot representation" and bug 7; the FP32
    sum rounded once is the "kimi_k3 ... ep.comm" page's combine)."""
    slots = np.asarray(slots, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    M, k = w.shape
    rows = slots.reshape(M, k, -1)
    return bf16_round(np.einsum("tk,tkh->th", w, rows))


# --------------------------------------------------------------------------
# The whole routed step
# --------------------------------------------------------------------------

ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]


def moe_decode(x, logits, bias, expert: ExpertFn, *, top_k: int, routed_scale: float,
               limit: float, ue8m0_act: bool = False, inter: Optional[int] = None) -> Dict:
    """Routing -> activation quant -> GEMM1 -> clamped SwiGLU -> FP8 hidden ->
    GEMM2 -> unweighted BF16 slots -> weighted combine.

    The order of steps is the "mega_moe" page's (module docstring and the
    kernel's epilogue), the slot semantics the nvfp4-megamoe-kernel README's.

    x: [M, H] BF16 values (float64); logits [M, E]; bias [E];
    expert(e) -> (w13 [2I, H] uint8, w13_scale [2I/128, H/128],
                  w2 [H, I] uint8, w2_scale [H/128, I/128]).
    Only the experts the routing touches are requested.

    Returns a dict of every stage: ids, weights, x_q, x_s, h1 [M*k, 2I]
    (binary32), act, h_q, h_s, slots [M*k, H] (BF16 values), combined [M, H]."""
    x = np.asarray(x, dtype=np.float64)
    M, H = x.shape
    ids, weights, scores = route(logits, bias, top_k, routed_scale)
    x_q, x_s = quantize_blocks(x, ue8m0=ue8m0_act, reciprocal=True)
    R = M * top_k
    cache = {}
    for e in np.unique(ids):
        cache[int(e)] = expert(int(e))
    if inter is None:
        inter = cache[int(ids[0, 0])][0].shape[0] // 2
    h1 = np.zeros((R, 2 * inter))
    for e, (w13, s13, _, _) in cache.items():
        rows = np.nonzero(ids.reshape(-1) == e)[0]
        toks = rows // top_k
        h1[rows] = f32(block_scaled_gemm(w13, s13, x_q[toks], x_s[toks]))
    act = swiglu(h1, inter, limit)
    h_q, h_s = requantize_hidden(act)
    slots = np.zeros((R, H))
    for e, (_, _, w2, s2) in cache.items():
        rows = np.nonzero(ids.reshape(-1) == e)[0]
        slots[rows] = bf16_round(block_scaled_gemm(w2, s2, h_q[rows], h_s[rows]))
    combined = combine(slots, weights)
    return dict(ids=ids, weights=weights, scores=scores, x_q=x_q, x_s=x_s, h1=h1, act=act,
                h_q=h_q, h_s=h_s, slots=slots, combined=combined)


# --------------------------------------------------------------------------
# Shared expert
# --------------------------------------------------------------------------

def unpack_ue8m0(packed, n: int, k: int) -> np.ndarray:
    """FP32 [n/128, k/128] block scales from packed UE8M0 words.

    Layout ("shared_expert" page, block_scales docstring): an int32 word per
    row and per four K blocks of 128; the exponent byte of K block b sits in
    bits 8*(b%4)..8*(b%4)+7 of word b//4. The scale of a (128-row, K) block is
    the binary32 whose bit pattern is that byte shifted into the exponent field
    (byte << 23), so byte 0 gives +0.0, 127 gives 1.0 and 255 gives +inf. The
    page takes the byte of the block's first row and requires the other 127
    rows to repeat it; a block where they differ is rejected (ValueError)."""
    words = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    nblocks = k // TILE
    out = np.empty((n // TILE, nblocks), np.float64)
    for b in range(nblocks):
        byte = (words[:, b // 4] >> (8 * (b % 4))) & 0xFF       # one per row
        by_block = byte.reshape(n // TILE, TILE)
        if np.any(by_block != by_block[:, :1]):
            raise ValueError(f"UE8M0 exponent byte not uniform over a 128-row block (K block {b})")
        bits = (by_block[:, 0] << 23).astype(np.uint32)
        out[:, b] = bits.view(np.float32)
    return out


def shared_expert(x, sw13, sw13_scale, sw2, sw2_scale, *, limit: float,
                  ue8m0_act: bool = True) -> Dict:
    """Dense shared expert ("shared_expert" page: module docstring,
    _GateUpKernel, _DownKernel, _group_scale).

    x quantised per 128 with the stock rule (UE8M0 scales when ue8m0_act,
    multiplying by the reciprocal, which is an exact power of two then);
    gate_up = BF16(FP32(GEMV)) with gate rows first; gate = min(gate, L),
    up = clamp(up, -L, L); silu = gate / (1 + exp(-gate)) in FP32 steps
    (_DownKernel: IEEE divide, accurate exp); act = BF16(silu * up); act
    quantised like x; out = BF16(FP32(GEMV))."""
    x = np.asarray(x, dtype=np.float64)
    x_q, x_s = quantize_blocks(x, ue8m0=ue8m0_act, reciprocal=True)
    gu = bf16_round(block_scaled_gemm(sw13, sw13_scale, x_q, x_s))
    Is = gu.shape[1] // 2
    gate = np.minimum(gu[:, :Is], limit)
    up = np.clip(gu[:, Is:], -limit, limit)
    act = bf16_round(silu_f32(gate) * up)
    h_q, h_s = quantize_blocks(act, ue8m0=ue8m0_act, reciprocal=True)
    out = bf16_round(block_scaled_gemm(sw2, sw2_scale, h_q, h_s))
    return dict(x_q=x_q, x_s=x_s, gate_up=gu, act=act, h_q=h_q, h_s=h_s, out=out)
