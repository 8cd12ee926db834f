"""Host checks of the Python binding: every buffer's shape, dtype, device and
layout is checked before the C ABI (which sees bare pointers) is called.
These run on the CPU: the checks raise before any library call."""

import pytest
import torch

from fp8_block_scaled_moe_amd import MoeDecode

H, I, E, K = 256, 128, 8, 2


def weights(fp4=False):
    if fp4:
        return (torch.zeros(E, 2 * I, H // 2, dtype=torch.uint8), torch.zeros(E, 2 * I, H // 16, dtype=torch.uint8),
                torch.zeros(E, H, I // 2, dtype=torch.uint8), torch.zeros(E, H, I // 16, dtype=torch.uint8))
    return (torch.zeros(E, 2 * I, H, dtype=torch.uint8), torch.ones(E, 2 * I // 128, H // 128),
            torch.zeros(E, H, I, dtype=torch.uint8), torch.ones(E, H // 128, I // 128))


def bad_weight_sets():
    w13, s13, w2, s2 = weights()
    yield "w2 transposed", (w13, s13, w2.transpose(1, 2).contiguous(), s2), {}
    yield "w2 fewer experts", (w13, s13, w2[:-1].contiguous(), s2), {}
    yield "w13_scale short", (w13, s13[:, :1].contiguous(), w2, s2), {}
    yield "w2_scale per row", (w13, s13, w2, torch.ones(E, H, I // 128)), {}
    yield "w13_scale dtype", (w13, s13.double(), w2, s2), {}
    yield "w13 2-D", (w13[0], s13, w2, s2), {}
    yield "w13 odd rows", (w13[:, :-1].contiguous(), s13, w2, s2), {}
    yield "local range past experts", (w13, s13, w2, s2), dict(experts=E + 2, local_begin=3)
    f13, fs13, f2, fs2 = weights(fp4=True)
    yield "fp4 scale per 32", (f13, fs13[:, :, ::2].contiguous(), f2, fs2), dict(weight_format="nvfp4")
    yield "fp4 w2 unpacked", (f13, fs13, torch.zeros(E, H, I, dtype=torch.uint8), fs2), dict(weight_format="nvfp4")
    yield "fp8 layout given as nvfp4", weights(), dict(weight_format="nvfp4")


@pytest.mark.parametrize("what,args,kw", list(bad_weight_sets()), ids=[b[0] for b in bad_weight_sets()])
def test_weights_of_the_wrong_shape_are_refused(what, args, kw):
    with pytest.raises(ValueError):
        MoeDecode(*args, top_k=K, limit=7.0, routed_scale=2.5, max_tokens=4, **kw)


def fake_handle(shared=False):
    """A binding object with the attributes check_run_args reads (no library)."""
    m = object.__new__(MoeDecode)
    m.device, m.hidden, m.top_k, m.experts = torch.device("cpu"), H, K, E
    m.logits_dtype, m.shared_inter = torch.float32, 128 if shared else 0
    return m


def run_args(M=3):
    return [torch.zeros(M, H, dtype=torch.bfloat16), torch.zeros(M, E), torch.zeros(E),
            torch.zeros(M * K, H, dtype=torch.bfloat16), torch.zeros(M, K, dtype=torch.int32),
            torch.zeros(M, K), torch.zeros(M, H, dtype=torch.bfloat16)]


def test_good_run_arguments_pass():
    m = fake_handle()
    assert m.check_run_args(*run_args()) == 3
    # outputs (and logits) with room for more rows are accepted
    big = run_args(5)
    args = run_args()
    args[1], args[3:] = big[1], big[3:]
    assert m.check_run_args(*args) == 3
    assert fake_handle(shared=True).check_run_args(*run_args(), torch.zeros(3, H, dtype=torch.bfloat16)) == 3


BAD_RUN = {
    "x width": (0, lambda a: a[0][:, :128].contiguous()),
    "x dtype": (0, lambda a: a[0].float()),
    "logits width": (1, lambda a: a[1][:, :E - 1].contiguous()),
    "logits rows": (1, lambda a: a[1][:2].contiguous()),
    "logits dtype": (1, lambda a: a[1].to(torch.bfloat16)),
    "bias length": (2, lambda a: a[2][:E - 1].clone()),
    "slots rows": (3, lambda a: a[3][:-1].clone()),
    "slots width": (3, lambda a: torch.zeros(3 * K, H + 128, dtype=torch.bfloat16)),
    "ids flat": (4, lambda a: a[4].view(-1)),
    "ids dtype": (4, lambda a: a[4].long()),
    "weights k": (5, lambda a: a[5][:, :1].contiguous()),
    "combined rows": (6, lambda a: a[6][:2].clone()),
    "combined transposed": (6, lambda a: a[6].t().contiguous().t()),
    "combined misaligned": (6, lambda a: torch.zeros(3 * H + 4, dtype=torch.bfloat16)[4:].view(3, H)),
}


@pytest.mark.parametrize("what", sorted(BAD_RUN))
def test_bad_run_arguments_are_refused(what):
    i, f = BAD_RUN[what]
    args = run_args()
    args[i] = f(args)
    with pytest.raises(ValueError):
        fake_handle().check_run_args(*args)


def test_shared_out_needs_a_shared_expert_and_its_shape():
    with pytest.raises(ValueError):
        fake_handle().check_run_args(*run_args(), torch.zeros(3, H, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fake_handle(shared=True).check_run_args(*run_args(), torch.zeros(3, H - 128, dtype=torch.bfloat16))
