"""attn_bwd_noalloc through the C ABI: the dense backward with the library's static
scratch must give the gradients of attn_bwd with a workspace (bitwise: the same kernels
run on the same data), on two calls in a row, the second with a smaller input.  (The
rejection of params that need more scratch than the static array is a CPU test in
test_abi.py.)"""
import pytest
import torch

import workloads
from parity import check_close

DEV = "cuda:0"


def rnd(shape, seed):
    return workloads.random_tensor(shape, seed, dtype=torch.bfloat16)


def run_case(gpu, B, S, Hq, Hkv, D, Dv, seed, **kw):
    q, k, v, do = (rnd((B, S, Hq, D), seed), rnd((B, S, Hkv, D), seed + 1), rnd((B, S, Hkv, Dv), seed + 2),
                   rnd((B, S, Hq, Dv), seed + 3))
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, m, l = gpu.attn_fwd(qd, kd, vd, **kw)
    ref = gpu.attn_bwd(qd, kd, vd, o, dod, m, l, **kw)
    out = (torch.full_like(qd, float("nan")), torch.full_like(kd, float("nan")), torch.full_like(vd, float("nan")))
    gpu.attn_bwd_noalloc(qd, kd, vd, o, dod, m, l, out=out, **kw)
    torch.cuda.synchronize()
    for nm, a, b in zip(("dq", "dk", "dv"), out, ref):
        check_close(nm, a, b.double().cpu(), "bf16")
        assert torch.equal(a, b), f"{nm}: not bitwise equal to attn_bwd"


@pytest.mark.gpu
def test_noalloc_matches_attn_bwd_twice(gpu):
    # first call: causal GQA-4 with the group's heads split over dk/dv workgroups (fp32
    # partials in the scratch); second, smaller: a window on a different shape
    run_case(gpu, 2, 640, 8, 2, 128, 128, 11, causal=True)
    run_case(gpu, 1, 200, 4, 4, 64, 64, 21, causal=True, window=(30, 0))
