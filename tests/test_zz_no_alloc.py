"""The allocation-free causal call (lin_attn_causal_chunked_noalloc) through
the C ABI: its outputs and final states equal those of
lin_attn_causal_chunked with a caller workspace on the same inputs -- it
runs the same kernels on the same plan, so they agree bit for bit, which is
within the bf16 / fp32 parity bars -- on two calls in a row sharing the
static scratch, the second on a smaller input, and from a carried-in state.
"""
import numpy as np
import pytest
import torch

from tests.parity import Case, TOL, assert_parity, host

pytestmark = pytest.mark.gpu


def _both(gpu_lib, c, kind, **kw):
    ref = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, **c.gkw(**kw))
    got = gpu_lib.lin_attn_causal_chunked_noalloc(c.q, c.k, c.v, kind, **c.gkw(**kw))
    torch.cuda.synchronize()
    return ref, got


def _check(ref, got, tol, what):
    for name, a, b in zip(("out", "S", "z"), ref, got):
        assert torch.equal(a, b), f"{what}: {name} differs from lin_attn_causal_chunked"
        assert_parity(b, host(a), tol, f"{what}: {name}")


def test_noalloc_equals_workspace_call_twice_then_smaller(gpu_lib):
    scale = 64 ** -0.25
    big = Case(3101, 1, 8, 4096, "favor", torch.bfloat16, r=256)
    ref, got = _both(gpu_lib, big, "favor", scale=scale)
    _check(ref, got, TOL[torch.bfloat16], "first call, H=8 N=4096")
    small = Case(3102, 2, 3, 700, "favor", torch.bfloat16, r=256)
    ref, got = _both(gpu_lib, small, "favor", scale=scale)
    _check(ref, got, TOL[torch.bfloat16], "second call, B=2 H=3 N=700")


def test_noalloc_vector_path_and_carried_state(gpu_lib):
    c = Case(3103, 1, 4, 1000, "elu1", torch.float32)
    S0 = torch.from_numpy(np.random.default_rng(5).random((1, 4, 64, 64), dtype=np.float32)).cuda()
    z0 = torch.from_numpy(np.random.default_rng(6).random((1, 4, 64), dtype=np.float32) + 1).cuda()
    ref = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "elu1", S=S0.clone(), z=z0.clone(),
                                          state_in=True)
    got = gpu_lib.lin_attn_causal_chunked_noalloc(c.q, c.k, c.v, "elu1", S=S0.clone(),
                                                  z=z0.clone(), state_in=True)
    torch.cuda.synchronize()
    _check(ref, got, TOL[torch.float32], "ELU+1 fp32 from a carried state")
    c2 = Case(3104, 1, 1, 33, "elu1", torch.float32)
    ref, got = _both(gpu_lib, c2, "elu1")
    _check(ref, got, TOL[torch.float32], "ELU+1 fp32, N=33")


def test_noalloc_refuses_more_than_its_scratch(gpu_lib):
    c = Case(3105, 4, 256, 40, "favor", torch.bfloat16, r=256)
    with pytest.raises(gpu_lib.LinAttnError):
        gpu_lib.lin_attn_causal_chunked_noalloc(c.q, c.k, c.v, "favor", **c.gkw())
