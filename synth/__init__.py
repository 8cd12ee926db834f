"""Seeded synthetic inputs for the routed-expert FP8 MoE decode step.

This module only draws numbers. It holds none of the method's arithmetic
(no routing, no quantisation rule, no GEMM): both the CPU oracle and the HIP
library consume exactly the tensors it returns, so a mismatch between them can
never come from input generation.

Shapes and value distributions follow the workloads the pages describe:
routed experts of a few decode tokens with DeepSeek-style block-128 FP32 weight
scales (vLLM `mega_moe` page, module docstring), the same at a larger token
count with the shared expert beside it (vLLM `shared_expert` page, module
docstring), and the latent MoE with 896 experts and top-16 routing at latent
width 3584 (vLLM `kimi_k3 ... ep.comm` page, module docstring).

Draw order (host, numpy PCG64 seeded with `seed`): logits, bias, x, then all
FP32 block scales (the FP4 share draws its scales on the device with its
weights; see `_make_inputs_fp4`). Weights are drawn expert by expert with
`torch.Generator(device).manual_seed(seed * 1000 + e)` as `randn / scale`
and cast to OCP e4m3 with torch's own cast (ties to even); a weight that
would overflow the cast is impossible at these scales (|randn| would need to
exceed 112). BF16 activations are torch casts of FP32 draws.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

TILE = 128
GROUP4 = 16  # FP4 values per UE4M3 scale


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """One routed-expert decode workload.

    `scale_lo`/`scale_hi` bound the U(lo, hi) FP32 block scales; when
    `pow2_scales` is set the scales are instead 2**U{-2..2}. `weights` is
    "normal" (randn / scale, e4m3) or "int" (integers in [-4, 4], exact in
    e4m3), and `x_kind` is "normal" (N(0,1) BF16) or "int" (integers in
    [-7, 7] with a +-7 in every 128-block, so every activation scale is
    exactly 7/448 = 2**-6).
    """

    name: str
    M: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    scale_lo: float = 0.25
    scale_hi: float = 4.0
    logits_std: float = 2.0
    logits_dtype: str = "f32"  # "f32" or "bf16"
    bias_std: float = 0.1
    routed_scale: float = 2.5
    limit: float = 7.0
    pow2_scales: bool = False
    weights: str = "normal"
    x_kind: str = "normal"
    ue8m0_act: bool = False
    # Shared expert (dense FP8 gate_up [2*Is, H] gate rows first, down [H, Is]
    # with power-of-two block scales); 0 means absent.
    shared_inter: int = 0
    shared_limit: float = 7.0
    # "fp8": e4m3 weights, FP32 128x128 scales. "fp4": packed E2M1 weights
    # with a UE4M3 byte per 16 values along K (gate rows first), for the
    # local experts [local_begin, local_begin + local_count) of `experts`.
    weight_format: str = "fp8"
    local_begin: int = 0
    local_count: int = 0
    # FP4 weight scale bytes: "mid" draws UE4M3 codes 0x30..0x3F (0.5 ..
    # 1.875), "full" every finite code 0x00..0x7E (zero, the subnormals
    # 2^-9 .. 7 * 2^-9 and the normals up to 448)
    scale_codes: str = "mid"

    def with_(self, **kw) -> "MoeShape":
        return dataclasses.replace(self, **kw)

    @property
    def routes(self) -> int:
        return self.M * self.top_k

    def expert_bytes(self) -> int:
        """Weight bytes plus scale bytes of one routed expert."""
        H, I = self.hidden, self.inter
        if self.weight_format == "fp4":
            return (2 * I * H + H * I) // 2 + (2 * I * H + H * I) // GROUP4
        w = 2 * I * H + H * I
        s = (2 * I // TILE) * (H // TILE) * 4 + (H // TILE) * (I // TILE) * 4
        return w + s

    @property
    def local_experts(self) -> int:
        return self.local_count or self.experts

    def shared_bytes(self) -> int:
        if not self.shared_inter:
            return 0
        H, Is = self.hidden, self.shared_inter
        return 2 * Is * H + H * Is + ((2 * Is // TILE) * (H // TILE) + (H // TILE) * (Is // TILE)) * 4


# The workloads. "tiny" is the small parity case; "dsv3" is the
# DeepSeek-V3-shaped decode (H=7168, I=2048, 256 experts, top-8) at M=4;
# "dsv3_m32_shared" adds the dense shared expert at M=32; "latent" is the
# 896-expert top-16 latent MoE at M=64 with BF16 logits.
CONFIGS = {
    "tiny": MoeShape(
        name="tiny", M=1, hidden=256, inter=128, experts=8, top_k=2,
        scale_lo=0.5, scale_hi=2.0, logits_std=1.0,
    ),
    "dsv3": MoeShape(name="dsv3", M=4, hidden=7168, inter=2048, experts=256, top_k=8),
    "dsv3_m32_shared": MoeShape(
        name="dsv3_m32_shared", M=32, hidden=7168, inter=2048, experts=256, top_k=8,
        shared_inter=2048,
    ),
    "latent": MoeShape(
        name="latent", M=64, hidden=3584, inter=1024, experts=896, top_k=16,
        logits_dtype="bf16", routed_scale=1.0, limit=10.0,
    ),
    # One GPU's share of the FP4 variant: 48 local experts of 384, top-6,
    # 16 tokens (nvfp4-megamoe-kernel README: 8 ranks x 48 experts, top-6,
    # L1 6144 x 7168 and L2 7168 x 3072 per expert).
    "fp4_share": MoeShape(
        name="fp4_share", M=16, hidden=7168, inter=3072, experts=384, top_k=6,
        weight_format="fp4", local_begin=0, local_count=48,
    ),
}


@dataclasses.dataclass
class MoeInputs:
    """Tensors of one workload. Device tensors live on `device`.

    x [M,H] bf16; logits [M,E] f32 or bf16; bias [E] f32;
    w13 [E,2I,H] uint8 (e4m3 bits; rows 0..I-1 up, I..2I-1 gate);
    w13_scale [E,2I/128,H/128] f32; w2 [E,H,I] uint8; w2_scale [E,H/128,I/128] f32.
    Shared expert (optional): sw13 [2Is,H] uint8 (gate rows first),
    sw13_scale [2Is/128,H/128] f32 (powers of two), sw2 [H,Is] uint8,
    sw2_scale [H/128,Is/128] f32.
    """

    shape: MoeShape
    seed: int
    x: torch.Tensor
    logits: torch.Tensor
    bias: torch.Tensor
    w13: torch.Tensor
    w13_scale: torch.Tensor
    w2: torch.Tensor
    w2_scale: torch.Tensor
    sw13: Optional[torch.Tensor] = None
    sw13_scale: Optional[torch.Tensor] = None
    sw2: Optional[torch.Tensor] = None
    sw2_scale: Optional[torch.Tensor] = None


def _scales(rng: np.random.Generator, shape: MoeShape, size) -> np.ndarray:
    if shape.pow2_scales:
        return np.exp2(rng.integers(-2, 3, size=size)).astype(np.float32)
    return rng.uniform(shape.scale_lo, shape.scale_hi, size=size).astype(np.float32)


def _x_values(rng: np.random.Generator, shape: MoeShape) -> np.ndarray:
    M, H = shape.M, shape.hidden
    if shape.x_kind == "normal":
        return rng.standard_normal((M, H)).astype(np.float32)
    if shape.x_kind == "int":
        v = rng.integers(-7, 8, size=(M, H // TILE, TILE))
        pos = rng.integers(0, TILE, size=(M, H // TILE))
        sign = np.where(rng.integers(0, 2, size=(M, H // TILE)) == 0, -7, 7)
        np.put_along_axis(v, pos[..., None], sign[..., None], axis=2)
        return v.reshape(M, H).astype(np.float32)
    if shape.x_kind == "zero":
        return np.zeros((M, H), np.float32)
    raise ValueError(shape.x_kind)


def _expert_weights(gen: torch.Generator, rows: int, cols: int, scale: torch.Tensor,
                    kind: str, device) -> torch.Tensor:
    """One expert's [rows, cols] e4m3 bits from its [rows/128, cols/128] scales."""
    if kind == "normal":
        w = torch.randn((rows, cols), generator=gen, device=device, dtype=torch.float32)
        full = scale.repeat_interleave(TILE, 0).repeat_interleave(TILE, 1)
        w = w / full
    elif kind == "int":
        w = torch.randint(-4, 5, (rows, cols), generator=gen, device=device).to(torch.float32)
    else:
        raise ValueError(kind)
    return w.to(torch.float8_e4m3fn).view(torch.uint8)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _x_values_fp4(rng: np.random.Generator, shape: MoeShape) -> np.ndarray:
    """x_kind "int" for the FP4 form: E2M1 grid values with a +-6 in every
    16-block, so every staged scale is exactly 1 and every code exact."""
    M, H = shape.M, shape.hidden
    v = E2M1_GRID[rng.integers(0, 8, size=(M, H // GROUP4, GROUP4))]
    v *= np.where(rng.integers(0, 2, size=v.shape) == 0, -1.0, 1.0)
    pos = rng.integers(0, GROUP4, size=(M, H // GROUP4))
    sign = np.where(rng.integers(0, 2, size=(M, H // GROUP4)) == 0, -6.0, 6.0)
    np.put_along_axis(v, pos[..., None], sign[..., None], axis=2)
    return v.reshape(M, H).astype(np.float32)


def _make_inputs_fp4(shape: MoeShape, seed: int, device) -> MoeInputs:
    """FP4 workload: packed weights are uniform random bytes (each nibble an
    E2M1 code, low nibble first), scale bytes uniform over the UE4M3 codes
    0x30..0x3F (0.5 .. 1.875), over 0x00..0x7E with scale_codes="full", or
    over {0x30, 0x38, 0x40} (0.5, 1, 2) with `pow2_scales`; local expert e
    draws from
    torch.Generator(device).manual_seed(seed * 1000 + e)."""
    rng = np.random.default_rng(seed)
    M, H, I, E = shape.M, shape.hidden, shape.inter, shape.experts
    assert H % TILE == 0 and I % TILE == 0
    logits = (rng.standard_normal((M, E)) * shape.logits_std).astype(np.float32)
    bias = (rng.standard_normal(E) * shape.bias_std).astype(np.float32)
    xv = _x_values_fp4(rng, shape) if shape.x_kind == "int" else _x_values(rng, shape)
    dev = torch.device(device)
    lt = torch.from_numpy(logits)
    if shape.logits_dtype == "bf16":
        lt = lt.to(torch.bfloat16)
    El = shape.local_experts
    w13 = torch.empty((El, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    s13 = torch.empty((El, 2 * I, H // GROUP4), dtype=torch.uint8, device=dev)
    w2 = torch.empty((El, H, I // 2), dtype=torch.uint8, device=dev)
    s2 = torch.empty((El, H, I // GROUP4), dtype=torch.uint8, device=dev)
    pow2 = torch.tensor([0x30, 0x38, 0x40], dtype=torch.uint8, device=dev)

    def scales(gen, shape_):
        if shape.pow2_scales:
            return pow2[torch.randint(0, 3, shape_, generator=gen, device=dev)]
        lo, hi = (0x00, 0x7F) if shape.scale_codes == "full" else (0x30, 0x40)
        return torch.randint(lo, hi, shape_, generator=gen, device=dev).to(torch.uint8)

    for e in range(El):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed * 1000 + e)
        w13[e] = torch.randint(0, 256, (2 * I, H // 2), generator=gen, device=dev).to(torch.uint8)
        s13[e] = scales(gen, (2 * I, H // GROUP4))
        w2[e] = torch.randint(0, 256, (H, I // 2), generator=gen, device=dev).to(torch.uint8)
        s2[e] = scales(gen, (H, I // GROUP4))
    return MoeInputs(shape=shape, seed=seed, x=torch.from_numpy(xv).to(torch.bfloat16).to(dev),
                     logits=lt.to(dev), bias=torch.from_numpy(bias).to(dev),
                     w13=w13, w13_scale=s13, w2=w2, w2_scale=s2)


def make_inputs(shape: MoeShape, seed: int = 0, device="cpu") -> MoeInputs:
    """Draws one workload; see the module docstring for the recipe."""
    if shape.weight_format == "fp4":
        return _make_inputs_fp4(shape, seed, device)
    rng = np.random.default_rng(seed)
    M, H, I, E = shape.M, shape.hidden, shape.inter, shape.experts
    assert H % TILE == 0 and I % TILE == 0
    logits = (rng.standard_normal((M, E)) * shape.logits_std).astype(np.float32)
    bias = (rng.standard_normal(E) * shape.bias_std).astype(np.float32)
    xv = _x_values(rng, shape)
    s13 = _scales(rng, shape, (E, 2 * I // TILE, H // TILE))
    s2 = _scales(rng, shape, (E, H // TILE, I // TILE))

    dev = torch.device(device)
    lt = torch.from_numpy(logits)
    if shape.logits_dtype == "bf16":
        lt = lt.to(torch.bfloat16)
    x = torch.from_numpy(xv).to(torch.bfloat16).to(dev)
    w13_scale = torch.from_numpy(s13).to(dev)
    w2_scale = torch.from_numpy(s2).to(dev)
    w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=dev)
    w2 = torch.empty((E, H, I), dtype=torch.uint8, device=dev)
    for e in range(E):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed * 1000 + e)
        w13[e] = _expert_weights(gen, 2 * I, H, w13_scale[e], shape.weights, dev)
        w2[e] = _expert_weights(gen, H, I, w2_scale[e], shape.weights, dev)

    inp = MoeInputs(
        shape=shape, seed=seed, x=x, logits=lt.to(dev),
        bias=torch.from_numpy(bias).to(dev),
        w13=w13, w13_scale=w13_scale, w2=w2, w2_scale=w2_scale,
    )
    if shape.shared_inter:
        Is = shape.shared_inter
        assert Is % TILE == 0
        srng = np.random.default_rng(seed + 7919)
        ss13 = np.exp2(srng.integers(-2, 3, size=(2 * Is // TILE, H // TILE))).astype(np.float32)
        ss2 = np.exp2(srng.integers(-2, 3, size=(H // TILE, Is // TILE))).astype(np.float32)
        inp.sw13_scale = torch.from_numpy(ss13).to(dev)
        inp.sw2_scale = torch.from_numpy(ss2).to(dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed * 1000 + 999_983)
        inp.sw13 = _expert_weights(gen, 2 * Is, H, inp.sw13_scale, shape.weights, dev)
        inp.sw2 = _expert_weights(gen, H, Is, inp.sw2_scale, shape.weights, dev)
    return inp


def pack_ue8m0(scales: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """FP32 power-of-two block scales [n/128, k/128] in DeepGEMM's packed UE8M0
    form: int32 [n, ceil(k/128/4)], byte g % 4 of word g // 4 holding the biased
    exponent of K group g, every row of a 128-row block repeating its scale
    (vLLM `shared_expert` page, `block_scales`). A layout transform for inputs
    only; it computes nothing of the method."""
    groups = k // TILE
    exps = (scales.contiguous().view(torch.int32) >> 23) & 0xFF  # [n/128, groups]
    rows = exps.repeat_interleave(TILE, 0)  # [n, groups]
    words = (groups + 3) // 4
    out = torch.zeros((n, words), dtype=torch.int64, device=scales.device)
    for g in range(groups):
        out[:, g // 4] |= rows[:, g].to(torch.int64) << (8 * (g % 4))
    # reinterpret the low 32 bits as int32 (two's complement)
    out = torch.where(out >= 2**31, out - 2**32, out)
    return out.to(torch.int32)
