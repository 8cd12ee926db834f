"""GPU parity of the FP4 form (nvfp4-megamoe-kernel README) and of local
experts, through the C ABI, against the oracle.

Bars: the device E2M1 encoder and FP4 reader bit-exact against the oracle's
codecs; ids bit-exact; weights within 1e-6 relative; the x staging (packed
codes and UE4M3 scales) bit-exact; GEMM1 within the FP32 accumulation bound of
the exact sum; the staged hidden within one E2M1 step of the oracle's staging
of the GPU's own GEMM1 output, on at most 1% of codes; slot and combined rows
within 2e-2 x the oracle row's RMS; slots of non-local experts exactly zero.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_block_scaled_moe_amd import MoeDecode, debug_codec_fp4
from oracle import fp4
from tests.helpers import (WEIGHT_RTOL, assert_rows_close, host, oracle_layer, oracle_layer_fp4)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def make_fp4(inp, **kw):
    s = inp.shape
    return MoeDecode(inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, top_k=s.top_k, limit=s.limit,
                     routed_scale=s.routed_scale, max_tokens=kw.pop("max_tokens", s.M),
                     logits_dtype=inp.logits.dtype, weight_format="nvfp4", experts=s.experts,
                     local_begin=s.local_begin, **kw)


def stage(moe, name, n, dtype):
    return moe.stage(name, torch.empty(n, dtype=dtype, device=DEV))


def run(moe, inp):
    out = moe(inp.x, inp.logits, inp.bias)
    torch.cuda.synchronize()
    return out


def test_device_e2m1_codec():
    grid = fp4.E2M1_MAGNITUDES
    mids = (grid[1:] + grid[:-1]) / 2
    f = np.float32
    vals = [grid, mids, np.nextafter(mids.astype(f), f(0)), np.nextafter(mids.astype(f), f(100)),
            np.array([6.5, 7.0, 1e4, 3e38, 0.0, 1e-30, 2.0**-10])]
    bits = np.arange(0, 0x40F00000, 7919, dtype=np.uint32)  # every 7919th pattern up to 7.5
    vals.append(bits.view(np.float32))
    v = np.concatenate([np.asarray(a, dtype=np.float64) for a in vals]).astype(np.float32)
    v = np.concatenate([v, -v])
    q, _ = debug_codec_fp4(torch.from_numpy(v).to(DEV))
    want = fp4.e2m1_encode(v.astype(np.float64))
    got = q.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} encodings differ, first {v[bad[:5]]} -> {got[bad[:5]]} vs {want[bad[:5]]}"
    # the reader: every code through every nibble position of a word
    _, dq = debug_codec_fp4(torch.zeros(128, dtype=torch.float32, device=DEV))
    assert np.array_equal(dq.cpu().numpy(), fp4.E2M1_VALUES[np.arange(128) & 15].astype(np.float32))


TINY = synth.CONFIGS["fp4_share"].with_(name="fp4_tiny", M=5, hidden=512, inter=256, experts=24,
                                        top_k=3, local_begin=6, local_count=12)


def check_fp4_layer(moe, inp, stages=True):
    s = inp.shape
    M, H, I, k = s.M, s.hidden, s.inter, s.top_k
    slots, ids, weights, combined = run(moe, inp)
    ref = oracle_layer_fp4(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(host(weights), ref["weights"], rtol=WEIGHT_RTOL, atol=0)
    local = ref["local"]
    if stages:
        xq = stage(moe, "x_q", M * H // 2, torch.uint8).cpu().numpy().reshape(M, H // 2)
        xs = stage(moe, "x_s", M * H // 16, torch.uint8).cpu().numpy().reshape(M, H // 16)
        assert np.array_equal(xq, fp4.pack_e2m1(ref["x_q"])) and np.array_equal(xs, ref["x_s"])
        # GEMM1 (FP32, before the BF16 rounding) against the exact sum
        R = M * k
        h1 = host(stage(moe, "part1", R * 2 * I, torch.float32)).reshape(R, 2 * I)
        rows = np.nonzero(local)[0]
        for r in rows:
            e = int(ref["ids"].reshape(-1)[r]) - s.local_begin
            t = r // k
            w13 = fp4.unpack_e2m1(inp.w13[e].cpu().numpy())
            s13 = inp.w13_scale[e].cpu().numpy()
            exact = fp4.fp4_block_gemm(w13, s13, ref["x_q"][t:t + 1], ref["x_s"][t:t + 1])[0]
            bound = fp4.fp4_block_gemm(w13 & 7, s13, ref["x_q"][t:t + 1] & 7, ref["x_s"][t:t + 1])[0]
            assert np.all(np.abs(h1[r] - exact) <= bound * 2.0**-20 + 1e-30), f"GEMM1 slot {r}"
        # the staged hidden from the GPU's own GEMM1 output, by the oracle's steps
        g1 = oracle.bf16_round(h1[rows])
        gate, up = np.minimum(g1[:, :I], s.limit), np.clip(g1[:, I:], -s.limit, s.limit)
        act = oracle.bf16_round(oracle.silu_f32(gate) * up)
        q, sc = fp4.quantize_fp4_blocks(act)
        hq = stage(moe, "h_q", R * I // 2, torch.uint8).cpu().numpy().reshape(R, I // 2)[rows]
        hs = stage(moe, "h_s", R * I // 16, torch.uint8).cpu().numpy().reshape(R, I // 16)[rows]
        assert np.mean(hs != sc) <= 0.01
        diff = fp4.unpack_e2m1(hq) != q
        assert diff.mean() <= 0.01, f"{diff.mean():.3%} of hidden codes differ"
    got = host(slots)
    assert not got[~local].any(), "slots of non-local experts must be zero"
    if local.any():
        assert_rows_close(got[local], ref["slots"][local], what="slots")
    assert_rows_close(host(combined), ref["combined"], what="combined")
    return ref, (slots, ids, weights, combined)


TINY_X_FACTORS = [1.0, 0.1, 0.03, 0.01, 0.004, 0.001]


def test_fp4_full_scale_code_range():
    """Weight scale bytes over every finite UE4M3 code (zero, subnormals
    0x01..0x07, normals up to 0x7E = 448), and tokens whose activations are
    small enough that their staged scales are subnormal or zero: the staging
    bit-exact, GEMM1 within the FP32 bound, the rows within the bar
    (nvfp4-megamoe-kernel README, "Data Formats": the scale is an e4m3 byte
    read as its value)."""
    shape = TINY.with_(M=6, hidden=768, inter=512, scale_codes="full")
    inp = synth.make_inputs(shape, seed=37, device=DEV)
    w = inp.w13_scale.cpu().numpy()
    assert w.min() == 0 and w.max() == 0x7E and np.isin(np.arange(1, 8), w).all()
    # tokens scaled down: their staged scales block_max / 6 fall from normal
    # codes into the subnormal ones (below 2^-6) and, in the smallest, to zero
    f = torch.tensor(TINY_X_FACTORS, device=DEV)[:, None]
    inp.x = (inp.x.float() * f).to(torch.bfloat16)
    moe = make_fp4(inp)
    ref, _ = check_fp4_layer(moe, inp)
    xs = ref["x_s"]
    assert ((xs >= 1) & (xs <= 7)).any(), "no subnormal activation scales staged"
    assert (xs >= 8).any() and (xs == 0).any()


def test_fp4_tiny():
    inp = synth.make_inputs(TINY, seed=31, device=DEV)
    moe = make_fp4(inp)
    assert moe.plan(TINY.M)["path"] == 4
    check_fp4_layer(moe, inp)


JOB_ROUTES = 4  # routes of one job: one pass over an expert's weights (an MFMA block's columns)


def check_jobs(moe, shape, ids):
    """The job table against the buckets and the routing ids: each touched
    local expert's routes (ascending) cut into jobs of at most JOB_ROUTES, experts
    ascending; every local route mapped to the job holding it."""
    M, k = shape.M, shape.top_k
    R = M * k
    ctrl = stage(moe, "ctrl", 3, torch.int32).cpu().numpy()
    U, J = int(ctrl[1]), int(ctrl[2])
    e_loc = ids.reshape(-1).astype(np.int64) - shape.local_begin
    local = (e_loc >= 0) & (e_loc < shape.local_experts)
    experts = np.unique(e_loc[local])
    assert U == experts.size
    want, want_rjob = [], np.full(R, -1)
    first = 0
    for e in experts:
        routes = np.nonzero(e_loc == e)[0]
        for p in range(0, routes.size, JOB_ROUTES):
            part = routes[p:p + JOB_ROUTES]
            want_rjob[part] = len(want)
            want.append((e, first + p, part.size, 0))
        first += routes.size
    assert J == len(want)
    jobs = stage(moe, "jobs", 4 * J, torch.int32).cpu().numpy().reshape(J, 4)
    assert np.array_equal(jobs, np.array(want, dtype=np.int32).reshape(J, 4))
    rjob = stage(moe, "route_jobs", R, torch.int32).cpu().numpy()
    assert np.array_equal(rjob[local], want_rjob[local])
    routes = stage(moe, "routes", R, torch.int32).cpu().numpy()
    assert np.array_equal(routes[:local.sum()], np.concatenate([np.nonzero(e_loc == e)[0] for e in experts]))


def test_fp4_jobs_one_wave():
    """At most 64 routes, so one wave groups them (ballot ranking): several
    jobs per expert, and routes outside the local range left out."""
    shape = TINY.with_(M=32, hidden=512, inter=256, experts=10, top_k=2, local_begin=3, local_count=5)
    inp = synth.make_inputs(shape, seed=35, device=DEV)
    inp.bias[[3, 5]] += 10.0  # experts 3 and 5 take every token: 32 routes, 8 jobs each
    moe = make_fp4(inp)
    ref, _ = check_fp4_layer(moe, inp)
    check_jobs(moe, shape, ref["ids"])


def test_fp4_quantising_workgroups():
    """3 tokens of H = 7168: the x staging is shared with a workgroup that
    only quantises; the staged codes and scales bit-exact."""
    shape = TINY.with_(M=3, hidden=7168, inter=256, experts=8, top_k=3, local_begin=0, local_count=8)
    inp = synth.make_inputs(shape, seed=36, device=DEV)
    check_fp4_layer(make_fp4(inp), inp)


def test_fp4_jobs_and_slots():
    """Many routes per expert (several jobs, so several passes over its
    weights) and a local range covering all experts; the job table bit-exact."""
    shape = TINY.with_(M=24, hidden=1024, inter=512, experts=10, top_k=4, local_begin=0, local_count=10)
    inp = synth.make_inputs(shape, seed=32, device=DEV)
    inp.bias[[2, 7]] += 10.0  # two experts take every token: 24 routes each
    moe = make_fp4(inp)
    ref, _ = check_fp4_layer(moe, inp)
    assert np.all(np.sort(ref["ids"][:, :2], axis=1) == [2, 7])
    check_jobs(moe, shape, ref["ids"])


def test_fp4_many_jobs():
    """Many jobs (256 tokens, top-32 of 512 experts: about 2,100 jobs of up
    to four routes, more than the resident workgroups), so every workgroup
    takes at most one job's items; the grid holds at least one workgroup per
    job."""
    shape = TINY.with_(M=256, hidden=512, inter=256, experts=512, top_k=32, local_begin=0, local_count=512)
    inp = synth.make_inputs(shape, seed=36, device=DEV)
    moe = make_fp4(inp)
    plan = moe.plan(shape.M)
    ref, _ = check_fp4_layer(moe, inp, stages=False)
    check_jobs(moe, shape, ref["ids"])
    J = int(stage(moe, "ctrl", 3, torch.int32).cpu().numpy()[2])
    assert J > 1536 and plan["grid1"] >= J and plan["grid2"] >= J


def test_fp4_long_k_many_jobs():
    """GEMM1 of K = 4096 (three items in flight, three waves per SIMD, 768
    resident workgroups) with more jobs than resident workgroups: token t's
    logits favour experts 16t .. 16t + 15 of 1,024 (bias zero, so the
    sigmoid decides), so each expert takes one route and there are 1,024
    jobs."""
    shape = TINY.with_(M=64, hidden=4096, inter=256, experts=1024, top_k=16, local_begin=0,
                       local_count=1024)
    inp = synth.make_inputs(shape, seed=38, device=DEV)
    favour = (torch.arange(shape.M, device=DEV)[:, None] * 16 + torch.arange(16, device=DEV)) % shape.experts
    inp.logits.scatter_add_(1, favour, torch.full((shape.M, 16), 20.0, device=DEV, dtype=inp.logits.dtype))
    inp.bias.zero_()
    moe = make_fp4(inp)
    plan = moe.plan(shape.M)
    ref, _ = check_fp4_layer(moe, inp, stages=False)
    check_jobs(moe, shape, ref["ids"])
    J = int(stage(moe, "ctrl", 3, torch.int32).cpu().numpy()[2])
    assert J == 1024 and plan["grid1"] >= J and plan["grid2"] >= J


def test_fp4_long_k_gemm2():
    """GEMM2 of K = 4096 (three items in flight) with its slot bookkeeping,
    stages checked."""
    shape = TINY.with_(M=3, hidden=512, inter=4096, experts=8, top_k=3, local_begin=0, local_count=8)
    inp = synth.make_inputs(shape, seed=39, device=DEV)
    check_fp4_layer(make_fp4(inp), inp)


def test_fp4_exact_grid_case():
    """x on the E2M1 grid with a +-6 in every 16-block (every staged scale
    exactly 1) and power-of-two weight scales: every GEMM1 sum is exact in
    FP32, so the staged hidden agrees bit for bit."""
    shape = TINY.with_(x_kind="int", pow2_scales=True)
    inp = synth.make_inputs(shape, seed=33, device=DEV)
    moe = make_fp4(inp)
    slots, ids, weights, combined = run(moe, inp)
    ref = oracle_layer_fp4(inp)
    assert np.all(oracle.e4m3_decode(ref["x_s"]) == 1.0)
    M, I, k = shape.M, shape.inter, shape.top_k
    R = M * k
    h1 = host(stage(moe, "part1", R * 2 * I, torch.float32)).reshape(R, 2 * I)
    local = ref["local"]
    assert np.array_equal(oracle.bf16_round(h1[local]), ref["h1"][local])
    hq = stage(moe, "h_q", R * I // 2, torch.uint8).cpu().numpy().reshape(R, I // 2)
    hs = stage(moe, "h_s", R * I // 16, torch.uint8).cpu().numpy().reshape(R, I // 16)
    assert np.array_equal(fp4.unpack_e2m1(hq[local]), ref["h_q"][local])
    assert np.array_equal(hs[local], ref["h_s"][local])
    assert_rows_close(host(slots)[local], ref["slots"][local], what="slots")


def test_fp4_no_local_routes():
    """A local range no token routes to: every slot and every combined row is
    zero."""
    shape = TINY.with_(local_begin=20, local_count=4)
    inp = synth.make_inputs(shape, seed=34, device=DEV)
    inp.bias[20:] -= 50.0
    moe = make_fp4(inp)
    slots, ids, weights, combined = run(moe, inp)
    assert (ids.cpu().numpy() < 20).all()
    assert stage(moe, "ctrl", 3, torch.int32).cpu().numpy()[2] == 0  # no jobs
    assert not slots.float().abs().max().item() and not combined.float().abs().max().item()


def test_fp4_share_full():
    """One GPU's share of the FP4 variant at full size: 48 local experts of
    384, top-6, 16 tokens, H = 7168, I = 3072."""
    inp = synth.make_inputs(synth.CONFIGS["fp4_share"], seed=0, device=DEV)
    moe = make_fp4(inp)
    ref, _ = check_fp4_layer(moe, inp, stages=False)
    assert ref["local"].sum() >= 4


def test_fp8_local_experts():
    """The FP8 form on a local share: weights of experts [lb, lb + lc) only;
    local slots as the oracle's, the others zero, combined over local slots."""
    full = synth.CONFIGS["tiny"].with_(M=6, hidden=384, inter=256, experts=16, top_k=4)
    inp = synth.make_inputs(full, seed=35, device=DEV)
    lb, lc = 5, 7
    # clone: a slice along the expert dimension is contiguous but not 16-byte aligned
    moe = MoeDecode(inp.w13[lb:lb + lc].clone(), inp.w13_scale[lb:lb + lc].clone(),
                    inp.w2[lb:lb + lc].clone(), inp.w2_scale[lb:lb + lc].clone(),
                    top_k=full.top_k, limit=full.limit, routed_scale=full.routed_scale,
                    max_tokens=full.M, experts=full.experts, local_begin=lb)
    slots, ids, weights, combined = run(moe, inp)
    ref = oracle_layer(inp)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    ids_f = ref["ids"].reshape(-1)
    local = (ids_f >= lb) & (ids_f < lb + lc)
    assert local.any() and (~local).any()
    got = host(slots)
    assert not got[~local].any()
    assert_rows_close(got[local], ref["slots"][local], what="slots")
    masked = np.where(local[:, None], ref["slots"], 0.0)
    want = oracle.combine(masked, ref["weights"])
    assert_rows_close(host(combined), want, what="combined")
