"""Parity against the oracle on seeded random configurations: shapes
(multiples of 128), expert counts, top-k, token counts, a local share of the
experts, BF16 logits, power-of-two activation scales, every FP8 GEMM path and
launch mode. Each draw is small enough for the oracle; the draws are fixed by
the seed, so a failure names a reproducible case.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_block_scaled_moe_amd import MoeDecode
from tests.helpers import WEIGHT_RTOL, assert_rows_close, host, oracle_layer

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = ["auto", "mfma", "mfma_splitk", "valu_splitk"]
MODES = ["auto", "combine_in_gemm2", "swiglu_in_gemm1"]


def draw(i):
    rng = np.random.default_rng(1000 + i)
    E = int(rng.choice([2, 7, 16, 33, 64, 100, 257]))
    k = int(rng.integers(1, min(E, 12) + 1))
    shape = synth.CONFIGS["tiny"].with_(
        name=f"random{i}", M=int(rng.choice([1, 2, 3, 5, 8, 9, 17, 40])),
        hidden=128 * int(rng.integers(1, 17)), inter=128 * int(rng.integers(1, 9)), experts=E, top_k=k,
        logits_dtype=str(rng.choice(["f32", "bf16"])), ue8m0_act=bool(rng.integers(0, 2)))
    local = rng.integers(0, 3) == 0  # a third of the draws keep a share of the experts
    lb = int(rng.integers(0, E)) if local else 0
    lc = int(rng.integers(1, E - lb + 1)) if local else E
    return shape, lb, lc, PATHS[i % len(PATHS)], MODES[(i // len(PATHS)) % len(MODES)]


@pytest.mark.parametrize("i", range(16))
def test_random_configuration(i):
    shape, lb, lc, path, mode = draw(i)
    inp = synth.make_inputs(shape, seed=2000 + i, device=DEV)
    # copies: the C ABI takes 16-byte aligned buffers, and a slice of the
    # scales need not start on one
    w = [t[lb:lb + lc].clone() for t in (inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)]
    moe = MoeDecode(*w, top_k=shape.top_k, limit=shape.limit, routed_scale=shape.routed_scale,
                    max_tokens=shape.M, logits_dtype=inp.logits.dtype, ue8m0_act=shape.ue8m0_act,
                    experts=shape.experts, local_begin=lb, gemm_path=path, launch_mode=mode)
    slots, ids, weights, combined = moe(inp.x, inp.logits, inp.bias)
    torch.cuda.synchronize()
    ref = oracle_layer(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"]), f"{shape} lb={lb} lc={lc} {path} {mode}"
    np.testing.assert_allclose(host(weights), ref["weights"], rtol=WEIGHT_RTOL, atol=0)
    rids = ref["ids"].reshape(-1)
    local = (rids >= lb) & (rids < lb + lc)
    want = np.where(local[:, None], ref["slots"], 0.0)
    assert_rows_close(host(slots), want, what=f"slots ({path}, {mode})")
    assert_rows_close(host(combined), oracle.combine(want, ref["weights"]), what=f"combined ({path}, {mode})")


def draw_fp4(i):
    rng = np.random.default_rng(3000 + i)
    E = int(rng.choice([4, 9, 24, 64, 384]))
    k = int(rng.integers(1, min(E, 8) + 1))
    lb = int(rng.integers(0, E))
    lc = int(rng.integers(1, E - lb + 1))
    shape = synth.CONFIGS["fp4_share"].with_(
        name=f"random_fp4_{i}", M=int(rng.choice([1, 2, 5, 8, 16, 33])),
        hidden=256 * int(rng.integers(1, 9)), inter=256 * int(rng.integers(1, 5)), experts=E, top_k=k,
        local_begin=lb, local_count=lc, logits_dtype=str(rng.choice(["f32", "bf16"])))
    return shape


@pytest.mark.parametrize("i", range(8))
def test_random_fp4_configuration(i):
    from tests.helpers import oracle_layer_fp4
    shape = draw_fp4(i)
    inp = synth.make_inputs(shape, seed=4000 + i, device=DEV)
    moe = MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=shape.top_k, limit=shape.limit,
                    routed_scale=shape.routed_scale, max_tokens=shape.M, logits_dtype=inp.logits.dtype,
                    weight_format="nvfp4", experts=shape.experts, local_begin=shape.local_begin)
    slots, ids, weights, combined = moe(inp.x, inp.logits, inp.bias)
    torch.cuda.synchronize()
    ref = oracle_layer_fp4(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"]), f"{shape}"
    np.testing.assert_allclose(host(weights), ref["weights"], rtol=WEIGHT_RTOL, atol=0)
    local = ref["local"]
    got = host(slots)
    assert not got[~local].any(), "slots of non-local experts must be zero"
    if local.any():
        assert_rows_close(got[local], ref["slots"][local], what="slots")
    assert_rows_close(host(combined), ref["combined"], what="combined")
