"""GPU parity: every entry point of the C ABI (through the binding) against the
fp64 oracle on the same seeded inputs.  Small cases span several segments,
chunks and a ragged tail; the workload cases run at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from kernelized_linear_attention_amd import inputs, workloads
from tests.parity import TOL, DT, Case, assert_parity, dev, host, oracle_prefix_state

pytestmark = pytest.mark.gpu

# (kind, dtype, r, nu, sum_norm, scale)
MAPS = [
    ("identity", torch.float32, 64, 1, False, 0.5),
    ("elu1", torch.float32, 64, 1, False, 1.0),
    ("elu1", torch.bfloat16, 64, 1, True, 1.0),
    ("favor", torch.float32, 128, 1, False, 64 ** -0.25),
    ("favor", torch.bfloat16, 256, 1, False, 64 ** -0.25),
    ("favor", torch.bfloat16, 128, 1, True, 64 ** -0.25),
    ("dpfp", torch.float32, 256, 2, True, 1.0),
    ("dpfp", torch.bfloat16, 128, 1, False, 1.0),
]
MAP_IDS = [f"{k}-{str(dt)[6:]}-r{r}{'-sn' if sn else ''}" for k, dt, r, _, sn, _ in MAPS]


def _norm_ok(kind, norm):
    # the identity map has no sign guarantee: its denominator may cross zero
    return not (kind == "identity" and norm == "attn")


@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", MAPS, ids=MAP_IDS)
def test_featuremap(gpu_lib, kind, dtype, r, nu, sum_norm, scale):
    c = Case(101, 2, 3, 67, kind, dtype, r=r, nu=nu)
    got = gpu_lib.lin_attn_featuremap(c.q, kind, **c.gkw(sum_norm=sum_norm, scale=scale))
    ref = oracle.featuremap(c.qh, kind, **c.okw(sum_norm=sum_norm, scale=scale))
    # the map itself is computed in float32 from exact inputs
    assert_parity(got, ref, 1e-4, f"featuremap {kind}")


@pytest.mark.parametrize("norm", ["attn", "none"])
@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", MAPS, ids=MAP_IDS)
def test_bidir(gpu_lib, kind, dtype, r, nu, sum_norm, scale, norm):
    if not _norm_ok(kind, norm):
        pytest.skip("identity map with attention normalisation has no positive denominator")
    c = Case(102, 2, 2, 300, kind, dtype, r=r, nu=nu)
    B, H = 2, 2
    S = torch.empty((B, H, r, 64), device="cuda")
    z = torch.empty((B, H, r), device="cuda")
    kw = dict(sum_norm=sum_norm, scale=scale, norm=norm)
    out = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, kind, S_out=S, z_out=z, **c.gkw(**kw))
    ro, rS, rz = oracle.bidir(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
    tol = TOL[dtype]
    assert_parity(out, ro, tol, "bidir out")
    assert_parity(S, rS, tol, "bidir S")
    assert_parity(z, rz, tol, "bidir z")


@pytest.mark.parametrize("norm", ["attn", "none"])
@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", MAPS, ids=MAP_IDS)
def test_causal(gpu_lib, kind, dtype, r, nu, sum_norm, scale, norm):
    if not _norm_ok(kind, norm):
        pytest.skip("identity map with attention normalisation has no positive denominator")
    c = Case(103, 2, 2, 300, kind, dtype, r=r, nu=nu)
    kw = dict(sum_norm=sum_norm, scale=scale, norm=norm)
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
    tol = TOL[dtype]
    assert_parity(out, ro, tol, "causal out")
    assert_parity(S, rS, tol, "causal S")
    assert_parity(z, rz, tol, "causal z")


@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", MAPS, ids=MAP_IDS)
def test_causal_from_carried_state(gpu_lib, kind, dtype, r, nu, sum_norm, scale):
    """state_in = 1: continue from a state (the oracle's prefix state)."""
    norm = "none" if kind == "identity" else "attn"
    pre = Case(104, 1, 3, 40, kind, dtype, r=r, nu=nu, rep=1)
    c = Case(104, 1, 3, 150, kind, dtype, r=r, nu=nu, rep=2)
    if kind == "favor":
        pre.omega, pre.omega_h = c.omega, c.omega_h
    kw = dict(sum_norm=sum_norm, scale=scale, norm=norm)
    S0, z0 = oracle_prefix_state(pre.qh, pre.kh, pre.vh, kind, **pre.okw(**kw))
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, S=S, z=z, state_in=True,
                                                **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, S0=S0, z0=z0, **c.okw(**kw))
    tol = TOL[dtype]
    assert_parity(out, ro, tol, "carried out")
    assert_parity(S, rS, tol, "carried S")
    assert_parity(z, rz, tol, "carried z")


# ---------------------------------------------------------------------------
# Wide feature maps (r = 384 = d log2 d, 480, 512): forward and decode only.
# The vector kernels keep S in LDS and shorten the chunk as r grows (16 tokens
# up to r = 384, 4 up to 512), so N = 300 spans many chunks and a ragged tail.
# ---------------------------------------------------------------------------
WIDE_MAPS = [
    ("favor", torch.float32, 384, 1, False, 64 ** -0.25),
    ("favor", torch.bfloat16, 384, 1, True, 64 ** -0.25),
    ("favor", torch.bfloat16, 512, 1, False, 64 ** -0.25),
    ("favor", torch.float32, 480, 1, False, 64 ** -0.25),
    ("dpfp", torch.float32, 384, 3, True, 1.0),
    ("dpfp", torch.bfloat16, 512, 4, False, 1.0),
    ("dpfp", torch.float32, 512, 4, True, 1.0),
]
WIDE_IDS = [f"{k}-{str(dt)[6:]}-r{r}{'-sn' if sn else ''}" for k, dt, r, _, sn, _ in WIDE_MAPS]


@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", WIDE_MAPS, ids=WIDE_IDS)
def test_wide_featuremap(gpu_lib, kind, dtype, r, nu, sum_norm, scale):
    c = Case(111, 2, 3, 67, kind, dtype, r=r, nu=nu)
    got = gpu_lib.lin_attn_featuremap(c.q, kind, **c.gkw(sum_norm=sum_norm, scale=scale))
    ref = oracle.featuremap(c.qh, kind, **c.okw(sum_norm=sum_norm, scale=scale))
    assert_parity(got, ref, 1e-4, f"featuremap {kind} r={r}")


@pytest.mark.parametrize("norm", ["attn", "none"])
@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", WIDE_MAPS, ids=WIDE_IDS)
def test_wide_bidir_and_causal(gpu_lib, kind, dtype, r, nu, sum_norm, scale, norm):
    c = Case(112, 2, 2, 300, kind, dtype, r=r, nu=nu)
    kw = dict(sum_norm=sum_norm, scale=scale, norm=norm)
    tol = TOL[dtype]
    S = torch.empty((2, 2, r, 64), device="cuda")
    z = torch.empty((2, 2, r), device="cuda")
    out = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, kind, S_out=S, z_out=z, **c.gkw(**kw))
    ro, rS, rz = oracle.bidir(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
    assert_parity(out, ro, tol, "bidir out")
    assert_parity(S, rS, tol, "bidir S")
    assert_parity(z, rz, tol, "bidir z")
    for n_seg in (0, 3):
        out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, n_seg=n_seg,
                                                    **c.gkw(**kw))
        ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
        assert_parity(out, ro, tol, f"causal out n_seg={n_seg}")
        assert_parity(S, rS, tol, f"causal S n_seg={n_seg}")
        assert_parity(z, rz, tol, f"causal z n_seg={n_seg}")


@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", WIDE_MAPS, ids=WIDE_IDS)
def test_wide_causal_from_carried_state_and_decode(gpu_lib, kind, dtype, r, nu, sum_norm, scale):
    """A prefill from a carried state, then one decode step from its final
    state, both against the oracle (r = 480 takes the 512-thread decode)."""
    pre = Case(113, 2, 3, 40, kind, dtype, r=r, nu=nu, rep=1)
    c = Case(113, 2, 3, 150, kind, dtype, r=r, nu=nu, rep=2)
    if kind == "favor":
        pre.omega, pre.omega_h = c.omega, c.omega_h
    kw = dict(sum_norm=sum_norm, scale=scale, norm="attn")
    tol = TOL[dtype]
    S0, z0 = oracle_prefix_state(pre.qh, pre.kh, pre.vh, kind, **pre.okw(**kw))
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, S=torch.from_numpy(S0).cuda(),
                                                z=torch.from_numpy(z0).cuda(), state_in=True,
                                                **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, S0=S0, z0=z0, **c.okw(**kw))
    assert_parity(out, ro, tol, "carried out")
    assert_parity(S, rS, tol, "carried S")
    S1, z1 = rS.astype(np.float32), rz.astype(np.float32)
    tok = Case(113, 2, 3, 1, kind, dtype, r=r, nu=nu, rep=3)
    q, k, v = (t[:, :, 0].contiguous() for t in (tok.q, tok.k, tok.v))
    Sd, zd = torch.from_numpy(S1).cuda(), torch.from_numpy(z1).cuda()
    od = gpu_lib.lin_attn_decode_step(q, k, v, Sd, zd, kind, omega=c.omega, nu=nu, **kw)
    rd, rSd, rzd = oracle.decode(host(q), host(k), host(v), S1, z1, kind, omega=c.omega_h, nu=nu,
                                 **kw)
    assert_parity(od, rd, tol, "decode out")
    assert_parity(Sd, rSd, tol, "decode S")
    assert_parity(zd, rzd, tol, "decode z")


# feature widths that are not multiples of 64 take the 512-thread decode kernel
DECODE_MAPS = MAPS + [
    ("favor", torch.float32, 96, 1, False, 64 ** -0.25),
    ("favor", torch.bfloat16, 32, 1, True, 64 ** -0.25),
    ("favor", torch.bfloat16, 224, 1, False, 64 ** -0.25),
]
DECODE_IDS = [f"{k}-{str(dt)[6:]}-r{r}{'-sn' if sn else ''}" for k, dt, r, _, sn, _ in DECODE_MAPS]


@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", DECODE_MAPS, ids=DECODE_IDS)
def test_decode_step(gpu_lib, kind, dtype, r, nu, sum_norm, scale):
    norm = "none" if kind == "identity" else "attn"
    B, H = 5, 3
    pre = Case(105, B, H, 20, kind, dtype, r=r, nu=nu, rep=1)
    kw = dict(sum_norm=sum_norm, scale=scale, norm=norm)
    S0, z0 = oracle_prefix_state(pre.qh, pre.kh, pre.vh, kind, **pre.okw(**kw))
    tok = Case(105, B, H, 1, kind, dtype, r=r, nu=nu, rep=2)
    q, k, v = (t[:, :, 0].contiguous() for t in (tok.q, tok.k, tok.v))
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    out = gpu_lib.lin_attn_decode_step(q, k, v, S, z, kind, omega=pre.omega, nu=nu, **kw)
    ro, rS, rz = oracle.decode(host(q), host(k), host(v), S0, z0, kind, omega=pre.omega_h, nu=nu,
                               **kw)
    tol = TOL[dtype]
    assert_parity(out, ro, tol, "decode out")
    assert_parity(S, rS, tol, "decode S")
    assert_parity(z, rz, tol, "decode z")


# ---------------------------------------------------------------------------
# Invariances of the scan and edge cases
# ---------------------------------------------------------------------------

def test_segment_count_does_not_change_results(gpu_lib):
    """Segment counts change only the rounding (the carry is an exact
    re-association); chunk 0 selects the 32-token block that chunk 32 names,
    so the two give identical bits; 64 and 128 are refused, not ignored."""
    c = Case(106, 1, 2, 1000, "favor", torch.bfloat16, r=256)
    kw = c.gkw(scale=64 ** -0.25)
    ref, rS, _ = oracle.causal(c.qh, c.kh, c.vh, "favor", **c.okw(scale=64 ** -0.25))
    for n_seg in (1, 3, 16):
        out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", n_seg=n_seg, **kw)
        assert_parity(out, ref, 2e-2, f"n_seg={n_seg}")
        assert_parity(S, rS, 2e-2, f"S n_seg={n_seg}")
        o32, S32, z32 = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", n_seg=n_seg,
                                                        chunk=32, **kw)
        assert torch.equal(out, o32) and torch.equal(S, S32) and torch.equal(z, z32)
    for chunk in (64, 128):
        with pytest.raises(gpu_lib.LinAttnError) as err:
            gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", chunk=chunk, **kw)
        assert err.value.code == -2


@pytest.mark.parametrize("n_seg", [9, 20, 79])
def test_many_segments_split_the_scan_into_ranges(gpu_lib, n_seg):
    """The segment scan splits each element's segments into 1, 2 or 4 ranges
    by their count (here 18, 40 and 158 half segments on the matrix-core
    route, the last with ranges longer than the register batch): prefill,
    final state and the causal backward (suffix scan over 79 segments) against
    the oracle, and bitwise repeatability."""
    c = Case(131, 1, 2, 5000, "favor", torch.bfloat16, r=256)
    kw = c.gkw(scale=64 ** -0.25)
    ref, rS, rz = oracle.causal(c.qh, c.kh, c.vh, "favor", **c.okw(scale=64 ** -0.25))
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", n_seg=n_seg, **kw)
    out2, S2, z2 = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", n_seg=n_seg, **kw)
    assert torch.equal(out, out2) and torch.equal(S, S2) and torch.equal(z, z2)
    assert_parity(out, ref, 2e-2, f"out n_seg={n_seg}")
    assert_parity(S, rS, 2e-2, f"S n_seg={n_seg}")
    assert_parity(z, rz, 2e-2, f"z n_seg={n_seg}")
    if n_seg == 79:
        do = dev(inputs.normal((1, 2, 5000, 64), 131, inputs.T_DOUT), torch.bfloat16)
        got = gpu_lib.lin_attn_causal_backward(c.q, c.k, c.v, do, "favor", n_seg=n_seg, **kw)
        gref = oracle.causal_backward(c.qh, c.kh, c.vh, host(do), "favor",
                                      **c.okw(scale=64 ** -0.25))
        _assert_grads(got, gref, 2e-2, f"causal backward n_seg={n_seg}")


def test_bitwise_deterministic(gpu_lib):
    c = Case(107, 1, 8, 2000, "favor", torch.bfloat16, r=256)
    kw = c.gkw(scale=64 ** -0.25)
    o1, S1, z1 = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", **kw)
    for _ in range(3):
        o2, S2, z2 = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", **kw)
        assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(z1, z2)
    b1 = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, "favor", **kw)
    b2 = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, "favor", **kw)
    assert torch.equal(b1, b2)


def test_split_call_equals_one_call(gpu_lib):
    """Carrying (S, z) across calls (Kernel Zoo sec. 9.3) matches one call."""
    c = Case(108, 2, 2, 700, "elu1", torch.float32, r=64)
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "elu1")
    m = 333
    o1, S1, z1 = gpu_lib.lin_attn_causal_chunked(c.q[:, :, :m].contiguous(),
                                                 c.k[:, :, :m].contiguous(),
                                                 c.v[:, :, :m].contiguous(), "elu1")
    o2, S2, z2 = gpu_lib.lin_attn_causal_chunked(c.q[:, :, m:].contiguous(),
                                                 c.k[:, :, m:].contiguous(),
                                                 c.v[:, :, m:].contiguous(), "elu1",
                                                 S=S1, z=z1, state_in=True)
    assert_parity(torch.cat([o1, o2], dim=2), host(out), 1e-5, "split out")
    assert_parity(S2, host(S), 1e-5, "split S")


def test_decode_equals_next_causal_row(gpu_lib):
    c = Case(109, 3, 2, 65, "favor", torch.float32, r=256)
    kw = c.gkw(scale=64 ** -0.25)
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", **kw)
    _, S64, z64 = gpu_lib.lin_attn_causal_chunked(c.q[:, :, :64].contiguous(),
                                                  c.k[:, :, :64].contiguous(),
                                                  c.v[:, :, :64].contiguous(), "favor", **kw)
    o = gpu_lib.lin_attn_decode_step(c.q[:, :, 64].contiguous(), c.k[:, :, 64].contiguous(),
                                     c.v[:, :, 64].contiguous(), S64, z64, "favor", **kw)
    assert_parity(o, host(out[:, :, 64]), 1e-5, "decode row")
    assert_parity(S64, host(S), 1e-5, "decode state")


@pytest.mark.parametrize("N", [0, 1, 63, 64, 65])
def test_short_and_empty_sequences(gpu_lib, N):
    c = Case(110, 1, 2, max(N, 1), "favor", torch.bfloat16, r=256)
    q, k, v = (t[:, :, :N].contiguous() for t in (c.q, c.k, c.v))
    S = torch.full((1, 2, 256, 64), 7.0, device="cuda")
    z = torch.full((1, 2, 256), 7.0, device="cuda")
    out, S, z = gpu_lib.lin_attn_causal_chunked(q, k, v, "favor", S=S, z=z, **c.gkw(scale=0.35))
    ro, rS, rz = oracle.causal(host(q), host(k), host(v), "favor", **c.okw(scale=0.35))
    if N == 0:
        assert out.numel() == 0
        assert torch.count_nonzero(S) == 0 and torch.count_nonzero(z) == 0
        return
    assert_parity(out, ro, 2e-2, "short out")
    assert_parity(S, rS, 2e-2, "short S")
    b = gpu_lib.lin_attn_bidir(q, k, v, "favor", **c.gkw(scale=0.35))
    rb, _, _ = oracle.bidir(host(q), host(k), host(v), "favor", **c.okw(scale=0.35))
    assert_parity(b, rb, 2e-2, "short bidir")


def test_zero_features_hit_the_eps_clamp(gpu_lib):
    """DPFP of non-negative keys is mostly zero (Kernel Zoo sec. 6.6): the
    denominators are 0 and the clamp gives exact zeros, never NaN."""
    B, H, N = 1, 1, 70
    x = np.zeros((B, H, N, 64), np.float32)
    x[..., 0] = 1.0  # kt = (1, 0, ...): every DPFP product is zero
    q = dev(x, torch.float32)
    v = dev(inputs.normal((B, H, N, 64), 111, inputs.T_V), torch.float32)
    out, S, z = gpu_lib.lin_attn_causal_chunked(q, q, v, "dpfp", nu=1)
    assert torch.count_nonzero(out) == 0 and torch.count_nonzero(S) == 0
    out2 = gpu_lib.lin_attn_causal_chunked(q, q, v, "dpfp", nu=1, sum_norm=True)[0]
    assert torch.count_nonzero(out2) == 0 and bool(torch.isfinite(out2).all())


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def _wl_case(w, rep=0):
    return Case(w.wid, w.B, w.H, w.N, w.kind, DT[w.dtype], r=w.r, nu=w.nu, d=w.d, dv=w.dv,
                rep=rep)


def _wl_kw(w):
    return dict(sum_norm=w.sum_norm, norm=w.norm, scale=workloads.scale_of(w), eps=w.eps)


def test_workload_elu1_small(gpu_lib):
    w = workloads.ELU_SMALL
    c = _wl_case(w)
    kw = _wl_kw(w)
    b = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, w.kind, **c.gkw(**kw))
    assert_parity(b, oracle.bidir(c.qh, c.kh, c.vh, w.kind, **c.okw(**kw))[0], 1e-4, "C1 bidir")
    o, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, w.kind, **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, w.kind, **c.okw(**kw))
    assert_parity(o, ro, 1e-4, "C1 causal")
    assert_parity(S, rS, 1e-4, "C1 S")


def test_workload_favor_bidir(gpu_lib):
    w = workloads.FAVOR_BIDIR
    c = _wl_case(w)
    kw = _wl_kw(w)
    S = torch.empty((w.B, w.H, w.r, w.dv), device="cuda")
    z = torch.empty((w.B, w.H, w.r), device="cuda")
    b = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, w.kind, S_out=S, z_out=z, **c.gkw(**kw))
    ro, rS, rz = oracle.bidir(c.qh, c.kh, c.vh, w.kind, **c.okw(**kw))
    assert_parity(b, ro, 2e-2, "C2 out")
    assert_parity(S, rS, 2e-2, "C2 S")
    assert_parity(z, rz, 2e-2, "C2 z")


def test_workload_favor_causal_prefill(gpu_lib):
    w = workloads.FAVOR_CAUSAL
    c = _wl_case(w)
    kw = _wl_kw(w)
    o, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, w.kind, chunk=32, **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, w.kind, **c.okw(**kw))
    assert_parity(o, ro, 2e-2, "C3 out")
    assert_parity(S, rS, 2e-2, "C3 S")
    assert_parity(z, rz, 2e-2, "C3 z")


def test_workload_dpfp_causal(gpu_lib):
    w = workloads.DPFP_CAUSAL
    c = _wl_case(w)
    for norm in ("none", "attn"):
        kw = dict(_wl_kw(w), norm=norm)
        o, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, w.kind, **c.gkw(**kw))
        ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, w.kind, **c.okw(**kw))
        assert_parity(o, ro, 1e-4, f"C4 out {norm}")
        assert_parity(S, rS, 1e-4, "C4 S")
        assert_parity(z, rz, 1e-4, "C4 z")


def test_workload_favor_decode_layers(gpu_lib):
    """Decode through the layers back to back, each with its own omega and
    state; the state comes from the oracle's causal prefill of a prefix."""
    w = workloads.FAVOR_DECODE
    kw = _wl_kw(w)
    for layer in range(w.layers):
        pre = Case(w.wid, w.B, w.H, w.prefix, w.kind, DT[w.dtype], r=w.r, rep=100 + layer)
        S0, z0 = oracle_prefix_state(pre.qh, pre.kh, pre.vh, w.kind, **pre.okw(**kw))
        tok = Case(w.wid, w.B, w.H, 1, w.kind, DT[w.dtype], r=w.r, rep=200 + layer)
        q, k, v = (t[:, :, 0].contiguous() for t in (tok.q, tok.k, tok.v))
        S = torch.from_numpy(S0).cuda()
        z = torch.from_numpy(z0).cuda()
        out = gpu_lib.lin_attn_decode_step(q, k, v, S, z, w.kind, omega=pre.omega, **kw)
        ro, rS, rz = oracle.decode(host(q), host(k), host(v), S0, z0, w.kind,
                                   omega=pre.omega_h, **kw)
        assert_parity(out, ro, 2e-2, f"C5 layer {layer} out")
        assert_parity(S, rS, 2e-2, f"C5 layer {layer} S")
        assert_parity(z, rz, 2e-2, f"C5 layer {layer} z")


# ---------------------------------------------------------------- packed sequences
VARLEN_LENS = [70, 0, 1, 33, 150, 64]   # empty, one-token, ragged and multi-segment sequences


def _packed(wid, lens, kind, dtype, r, nu, H=2, rep=0):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    c = Case(wid, 1, H, int(cu[-1]), kind, dtype, r=r, nu=nu, rep=rep)
    q, k, v = c.q[0], c.k[0], c.v[0]                       # [H, total, d]
    return c, q, k, v, cu, torch.from_numpy(cu).to("cuda")


@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", MAPS, ids=MAP_IDS)
def test_causal_varlen(gpu_lib, kind, dtype, r, nu, sum_norm, scale):
    norm = "none" if kind == "identity" else "attn"
    c, q, k, v, cu, cu_d = _packed(105, VARLEN_LENS, kind, dtype, r, nu)
    kw = dict(sum_norm=sum_norm, scale=scale, norm=norm)
    out, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, cu_d, kind, **c.gkw(**kw))
    ro, rS, rz = oracle.causal_varlen(c.qh[0], c.kh[0], c.vh[0], cu, kind, **c.okw(**kw))
    tol = TOL[dtype]
    assert_parity(out, ro, tol, "varlen out", lead_dims=1)
    assert_parity(S, rS, tol, "varlen S")
    assert_parity(z, rz, tol, "varlen z")


@pytest.mark.parametrize("kind,dtype,r", [("favor", torch.bfloat16, 256), ("elu1", torch.float32, 64)])
def test_causal_varlen_from_carried_states(gpu_lib, kind, dtype, r):
    """Each sequence continues from its own state (carry across calls)."""
    c, q, k, v, cu, cu_d = _packed(106, [40, 0, 97], kind, dtype, r, 1)
    g = np.random.default_rng(107)
    S0 = np.abs(g.standard_normal((3, 2, r, 64))).astype(np.float32)
    z0 = np.abs(g.standard_normal((3, 2, r))).astype(np.float32) + 1.0
    S = torch.from_numpy(S0).to("cuda")
    z = torch.from_numpy(z0).to("cuda")
    scale = 64 ** -0.25 if kind == "favor" else 1.0
    out, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, cu_d, kind, S=S, z=z, state_in=True,
                                               **c.gkw(scale=scale))
    ro, rS, rz = oracle.causal_varlen(c.qh[0], c.kh[0], c.vh[0], cu, kind, S0=S0, z0=z0,
                                      **c.okw(scale=scale))
    tol = TOL[dtype]
    assert_parity(out, ro, tol, "varlen carried out", lead_dims=1)
    assert_parity(S, rS, tol, "varlen carried S")
    assert_parity(z, rz, tol, "varlen carried z")


def test_causal_varlen_one_sequence_matches_chunked(gpu_lib):
    c, q, k, v, cu, cu_d = _packed(108, [1000], "favor", torch.bfloat16, 256, 1, H=3)
    kw = c.gkw(scale=64 ** -0.25)
    out, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, cu_d, "favor", **kw)
    o2, S2, z2 = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", **kw)
    assert_parity(out, host(o2[0]), 2e-2, "varlen vs chunked out", lead_dims=1)
    assert_parity(S[0], host(S2[0]), 1e-5, "varlen vs chunked S", lead_dims=1)


def test_causal_varlen_many_sequences_at_scale(gpu_lib):
    """16 ragged sequences (~16k tokens), 8 heads: the matrix-core path with
    several segments per sequence and partial segments at every boundary."""
    g = np.random.default_rng(109)
    lens = g.integers(1, 2048, size=16)
    lens[3] = 0
    c, q, k, v, cu, cu_d = _packed(109, list(lens), "favor", torch.bfloat16, 256, 1, H=8)
    kw = dict(scale=64 ** -0.25)
    out, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, cu_d, "favor", **c.gkw(**kw))
    ro, rS, rz = oracle.causal_varlen(c.qh[0], c.kh[0], c.vh[0], cu, "favor", **c.okw(**kw))
    assert_parity(out, ro, 2e-2, "varlen at scale out", lead_dims=1)
    assert_parity(S, rS, 2e-2, "varlen at scale S")
    assert_parity(z, rz, 2e-2, "varlen at scale z")


def test_workload_favor_causal_packed(gpu_lib):
    """The benchmark's packed workload at full size: 32 documents of mixed
    length over 65,536 tokens, 8 heads."""
    w = workloads.FAVOR_VARLEN
    lens = inputs.packed_lengths(w.B, w.N, w.wid)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = (dev(inputs.normal((w.H, w.N, w.d), w.wid, t, 0), DT[w.dtype])
               for t in (inputs.T_Q, inputs.T_K, inputs.T_V))
    om = dev(inputs.orf_omega(w.r, w.d, w.wid), DT[w.dtype])
    kw = dict(scale=workloads.scale_of(w), eps=w.eps)
    o, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, torch.from_numpy(cu).to("cuda"), w.kind,
                                             omega=om, **kw)
    ro, rS, rz = oracle.causal_varlen(host(q), host(k), host(v), cu, w.kind, omega=host(om), **kw)
    assert_parity(o, ro, 2e-2, "packed out", lead_dims=1)
    assert_parity(S, rS, 2e-2, "packed S")
    assert_parity(z, rz, 2e-2, "packed z")


# ---------------------------------------------------------------- on-device ORF
def _orf_case(n_mat, r, d, wid, with_lengths=True):
    draws = [inputs.orf_draws(r, d, wid, rep) for rep in range(n_mat)]
    gauss = np.stack([g for g, _ in draws])
    lens = np.stack([l for _, l in draws]) if with_lengths else None
    ref = np.stack([oracle.orf(gauss[m], r, None if lens is None else lens[m]) for m in range(n_mat)])
    g_d = torch.from_numpy(gauss).to("cuda")
    l_d = None if lens is None else torch.from_numpy(lens).to("cuda")
    return g_d, l_d, ref


@pytest.mark.parametrize("n_mat,r,d,lengths", [(3, 256, 64, True), (2, 100, 48, True),
                                               (1, 64, 64, False), (4, 33, 7, True)])
def test_orf_omega_float32(gpu_lib, n_mat, r, d, lengths):
    g, l, ref = _orf_case(n_mat, r, d, 110, lengths)
    om = gpu_lib.lin_attn_orf_omega(g, l, r=r, dtype=torch.float32)
    got = host(om)
    want = ref.astype(np.float32).astype(np.float64)
    # float64 arithmetic on both sides, rounded once to float32: equal up to
    # a rounding-boundary ulp
    assert np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30)) <= 2.0 ** -22
    # rows orthogonal within each block
    for m in range(n_mat):
        for b in range(0, r, d):
            blk = got[m, b:b + d]
            gram = blk @ blk.T
            off = gram - np.diag(np.diag(gram))
            assert np.max(np.abs(off)) < 1e-5 * np.max(np.diag(gram))


def test_orf_omega_bfloat16(gpu_lib):
    g, l, ref = _orf_case(12, 256, 64, 111)
    om = gpu_lib.lin_attn_orf_omega(g, l, dtype=torch.bfloat16)
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    got = om.cpu()
    # the same rounding (float64 -> float32 -> bfloat16, nearest-even) on both
    # sides: bit-equal except at a rounding boundary, where one ulp apart
    bits_got = got.view(torch.int16).to(torch.int32)
    bits_want = want.view(torch.int16).to(torch.int32)
    diff = (bits_got - bits_want).abs()
    assert int(diff.max()) <= 1
    assert int((diff > 0).sum()) <= got.numel() // 1000


def test_orf_omega_drives_favor_like_the_host_sampler(gpu_lib):
    """Attention with the device-built omega matches the oracle run with the
    oracle-built omega (bfloat16 inputs, r = 256: the matrix-core path)."""
    g, l, ref = _orf_case(1, 256, 64, 112)
    om = gpu_lib.lin_attn_orf_omega(g[0], l[0], dtype=torch.bfloat16)
    c = Case(112, 1, 2, 300, "favor", torch.bfloat16, r=256)
    kw = dict(scale=64 ** -0.25)
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, "favor", omega=om, **kw)
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, "favor", omega=host(om), **kw)
    assert_parity(out, ro, 2e-2, "orf causal out")
    np.testing.assert_allclose(host(om), ref[0], rtol=2 ** -8, atol=1e-6)


# ---------------------------------------------------------------- backward pass
def _bwd(gpu_lib, oracle_too, form, c, do, kind, **kw):
    fn = gpu_lib.lin_attn_bidir_backward if form == "bidir" else gpu_lib.lin_attn_causal_backward
    got = fn(c.q, c.k, c.v, do, kind, **c.gkw(**kw))
    if not oracle_too:
        return got, None
    ofn = oracle.bidir_backward if form == "bidir" else oracle.causal_backward
    return got, ofn(c.qh, c.kh, c.vh, host(do), kind, **c.okw(**kw))


def _assert_grads(got, ref, tol, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert g.dtype == got[0].dtype
        assert_parity(g, r, tol, f"{what} {name}")


@pytest.mark.parametrize("form", ["bidir", "causal"])
@pytest.mark.parametrize("norm", ["attn", "none"])
@pytest.mark.parametrize("kind,dtype,r,nu,sum_norm,scale", MAPS, ids=MAP_IDS)
def test_backward(gpu_lib, form, kind, dtype, r, nu, sum_norm, scale, norm):
    """dq, dk, dv over several segments, chunks and a ragged tail (300
    tokens: segments of 64, chunks of 16, a last segment of 44)."""
    if not _norm_ok(kind, norm):
        pytest.skip("identity map with attention normalisation has no positive denominator")
    B, H, N = 2, 2, 300
    c = Case(120, B, H, N, kind, dtype, r=r, nu=nu)
    do = dev(inputs.normal((B, H, N, 64), 120, inputs.T_DOUT), dtype)
    got, ref = _bwd(gpu_lib, True, form, c, do, kind, sum_norm=sum_norm, scale=scale, norm=norm)
    _assert_grads(got, ref, TOL[dtype], f"{form} backward")


@pytest.mark.parametrize("form", ["bidir", "causal"])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 64, 65])
def test_backward_short_sequences(gpu_lib, form, N):
    c = Case(121, 1, 3, N, "favor", torch.float32, r=96)
    do = dev(inputs.normal((1, 3, N, 64), 121, inputs.T_DOUT), torch.float32)
    got, ref = _bwd(gpu_lib, True, form, c, do, "favor", scale=0.4)
    if N == 1:
        # one token: out = v whatever q and k are, so dv = dout and dq = dk = 0
        # exactly; only rounding is left in them
        assert_parity(got[2], host(do), 1e-6, "N=1 dv")
        for g in got[:2]:
            assert float(g.abs().max()) <= 1e-5 * float(do.abs().max())
        return
    _assert_grads(got, ref, 1e-4, f"{form} N={N}")


@pytest.mark.parametrize("form", ["bidir", "causal"])
def test_backward_segment_count_changes_rounding_only(gpu_lib, form):
    c = Case(122, 1, 2, 1000, "elu1", torch.float32, r=64)
    do = dev(inputs.normal((1, 2, 1000, 64), 122, inputs.T_DOUT), torch.float32)
    ofn = oracle.bidir_backward if form == "bidir" else oracle.causal_backward
    ref = ofn(c.qh, c.kh, c.vh, host(do), "elu1", **c.okw())
    fn = gpu_lib.lin_attn_bidir_backward if form == "bidir" else gpu_lib.lin_attn_causal_backward
    first = None
    for n_seg in (1, 3, 16):
        got = fn(c.q, c.k, c.v, do, "elu1", n_seg=n_seg, **c.gkw())
        _assert_grads(got, ref, 1e-4, f"{form} n_seg={n_seg}")
        again = fn(c.q, c.k, c.v, do, "elu1", n_seg=n_seg, **c.gkw())
        assert all(torch.equal(a, b) for a, b in zip(got, again)), "not bitwise reproducible"


def test_backward_zero_features_stay_finite(gpu_lib):
    """DPFP of vectors with one positive component has no nonzero feature
    (Kernel Zoo sec. 6.6): every denominator is clamped and every gradient
    is exactly zero, never NaN, with and without sum normalisation."""
    B, H, N = 1, 1, 70
    x = np.zeros((B, H, N, 64), np.float32)
    x[..., 0] = 1.0
    q = dev(x, torch.float32)
    v = dev(inputs.normal((B, H, N, 64), 123, inputs.T_V), torch.float32)
    do = dev(inputs.normal((B, H, N, 64), 123, inputs.T_DOUT), torch.float32)
    for sn in (False, True):
        for fn in (gpu_lib.lin_attn_bidir_backward, gpu_lib.lin_attn_causal_backward):
            for g in fn(q, q, v, do, "dpfp", nu=1, sum_norm=sn):
                assert bool(torch.isfinite(g).all()) and torch.count_nonzero(g) == 0


def test_causal_backward_of_last_row_equals_bidirectional(gpu_lib):
    """A loss on the last row alone: both forms give the same gradients
    (that query sees every key in both)."""
    B, H, N = 1, 2, 777
    c = Case(124, B, H, N, "favor", torch.float32, r=256)
    do_np = np.zeros((B, H, N, 64), np.float32)
    do_np[:, :, -1] = inputs.normal((B, H, 64), 124, inputs.T_DOUT)
    do = dev(do_np, torch.float32)
    kw = c.gkw(scale=64 ** -0.25)
    a = gpu_lib.lin_attn_causal_backward(c.q, c.k, c.v, do, "favor", **kw)
    b = gpu_lib.lin_attn_bidir_backward(c.q, c.k, c.v, do, "favor", **kw)
    for x, y in zip(a, b):
        assert_parity(x, host(y), 1e-4, "last-row gradients")  # two summation orders


def test_workload_favor_bidir_backward(gpu_lib):
    w = workloads.FAVOR_BIDIR
    c = _wl_case(w)
    do = dev(inputs.normal((w.B, w.H, w.N, w.dv), w.wid, inputs.T_DOUT), DT[w.dtype])
    got, ref = _bwd(gpu_lib, True, "bidir", c, do, w.kind, **_wl_kw(w))
    _assert_grads(got, ref, 2e-2, "bidir workload backward")


def test_workload_favor_causal_backward(gpu_lib):
    w = workloads.FAVOR_CAUSAL
    c = _wl_case(w)
    do = dev(inputs.normal((w.B, w.H, w.N, w.dv), w.wid, inputs.T_DOUT), DT[w.dtype])
    got, ref = _bwd(gpu_lib, True, "causal", c, do, w.kind, **_wl_kw(w))
    _assert_grads(got, ref, 2e-2, "causal prefill backward")


# ---------------------------------------------------------------- fused input projection
# (kind, r, nu, sum_norm, scale, norm): bfloat16 tokens and weights only
PROJ_MAPS = [
    ("favor", 256, 1, False, 64 ** -0.25, "attn"),
    ("favor", 96, 1, False, 64 ** -0.25, "none"),
    ("elu1", 64, 1, True, 1.0, "attn"),
    ("dpfp", 256, 2, True, 1.0, "none"),
    ("identity", 64, 1, False, 0.5, "none"),
]
PROJ_IDS = [f"{k}-r{r}{'-sn' if sn else ''}-{nm}" for k, r, _, sn, _, nm in PROJ_MAPS]


class ProjCase:
    """Seeded tokens x [B, N, dm] and weights W_q, W_k, W_v [H*64, dm] on the
    device (bf16), their exact values for the oracle, and omega."""

    def __init__(self, wid, B, H, N, dm, kind, r, rep=0):
        self.H = H
        self.x = dev(inputs.normal((B, N, dm), wid, inputs.T_X, rep), torch.bfloat16)
        self.w = [dev(w, torch.bfloat16) for w in inputs.projection_weights(H, 64, dm, wid, rep)]
        self.xh = host(self.x)
        self.wh = [host(w) for w in self.w]
        self.omega = self.omega_h = None
        if kind == "favor":
            self.omega = dev(inputs.orf_omega(r, 64, wid, rep), torch.bfloat16)
            self.omega_h = host(self.omega)


@pytest.mark.parametrize("kind,r,nu,sum_norm,scale,norm", PROJ_MAPS, ids=PROJ_IDS)
@pytest.mark.parametrize("B,H,N,dm", [(2, 2, 300, 128), (1, 8, 200, 512)])
def test_causal_proj(gpu_lib, kind, r, nu, sum_norm, scale, norm, B, H, N, dm):
    c = ProjCase(130, B, H, N, dm, kind, r)
    kw = dict(nu=nu, sum_norm=sum_norm, scale=scale, norm=norm)
    out, S, z = gpu_lib.lin_attn_causal_proj(c.x, *c.w, H, kind, omega=c.omega, **kw)
    ro, rS, rz = oracle.causal_proj(c.xh, *c.wh, H, kind, omega=c.omega_h, **kw)
    assert_parity(out, ro, 2e-2, "causal_proj out")
    assert_parity(S, rS, 2e-2, "causal_proj S")
    assert_parity(z, rz, 2e-2, "causal_proj z")


@pytest.mark.parametrize("kind,r,nu,sum_norm,scale,norm", PROJ_MAPS, ids=PROJ_IDS)
def test_bidir_proj(gpu_lib, kind, r, nu, sum_norm, scale, norm):
    B, H, N, dm = 2, 2, 300, 128
    c = ProjCase(131, B, H, N, dm, kind, r)
    kw = dict(nu=nu, sum_norm=sum_norm, scale=scale, norm=norm)
    r_ = oracle.feature_dim(kind, 64, nu, c.omega_h)
    S = torch.empty((B, H, r_, 64), device="cuda")
    z = torch.empty((B, H, r_), device="cuda")
    out = gpu_lib.lin_attn_bidir_proj(c.x, *c.w, H, kind, omega=c.omega, S_out=S, z_out=z, **kw)
    ro, rS, rz = oracle.bidir_proj(c.xh, *c.wh, H, kind, omega=c.omega_h, **kw)
    assert_parity(out, ro, 2e-2, "bidir_proj out")
    assert_parity(S, rS, 2e-2, "bidir_proj S")
    assert_parity(z, rz, 2e-2, "bidir_proj z")


def test_causal_proj_carried_state_and_short_inputs(gpu_lib):
    """A split call carrying (S, z) equals one call; N in {1, 31, 33}."""
    H, dm = 2, 64
    c = ProjCase(132, 1, H, 400, dm, "favor", 128)
    kw = dict(omega=c.omega, scale=64 ** -0.25)
    out, S, z = gpu_lib.lin_attn_causal_proj(c.x, *c.w, H, "favor", **kw)
    m = 157
    o1, S1, z1 = gpu_lib.lin_attn_causal_proj(c.x[:, :m].contiguous(), *c.w, H, "favor", **kw)
    o2, _, _ = gpu_lib.lin_attn_causal_proj(c.x[:, m:].contiguous(), *c.w, H, "favor", S=S1,
                                            z=z1, state_in=True, **kw)
    assert_parity(torch.cat([o1, o2], dim=2), host(out), 1e-2, "split out")
    assert_parity(S1, host(S), 1e-2, "split S")  # S1 was updated in place by the second call
    for n in (1, 31, 33):
        o, Sn, _ = gpu_lib.lin_attn_causal_proj(c.x[:, :n].contiguous(), *c.w, H, "favor", **kw)
        ro, rS, _ = oracle.causal_proj(c.xh[:, :n], *c.wh, H, "favor", omega=c.omega_h,
                                       scale=64 ** -0.25)
        assert_parity(o, ro, 2e-2, f"N={n} out")
        assert_parity(Sn, rS, 2e-2, f"N={n} S")


def test_workload_favor_causal_prefill_from_tokens(gpu_lib):
    """The causal prefill workload (B=1, H=8, N=65536, r=256) from tokens of
    the pages' model width d_model = 512."""
    w = workloads.FAVOR_CAUSAL
    c = ProjCase(w.wid, w.B, w.H, w.N, 512, w.kind, w.r)
    kw = _wl_kw(w)
    out, S, z = gpu_lib.lin_attn_causal_proj(c.x, *c.w, w.H, w.kind, omega=c.omega, **kw)
    ro, rS, rz = oracle.causal_proj(c.xh, *c.wh, w.H, w.kind, omega=c.omega_h, **kw)
    assert_parity(out, ro, 2e-2, "prefill from tokens out")
    assert_parity(S, rS, 2e-2, "prefill from tokens S")
    assert_parity(z, rz, 2e-2, "prefill from tokens z")


@pytest.mark.parametrize("B,H,N,dm", [(2, 3, 300, 48), (1, 8, 200, 512), (3, 1, 1, 16),
                                      (1, 2, 128, 128)])
def test_qkv_project(gpu_lib, B, H, N, dm):
    """One GEMM for all three projections, head-major outputs: ragged token
    count, an odd number of heads (half-empty column tile), K not a multiple
    of the 32-wide step.  Rounding to bf16 bounds the error by 2^-9
    relative."""
    c = ProjCase(133, B, H, N, dm, "elu1", 64)
    q, k, v = gpu_lib.lin_attn_qkv_project(c.x, *c.w, H)
    for name, got, w in zip("qkv", (q, k, v), c.wh):
        ref = oracle.project(c.xh, w, H)
        assert_parity(got, ref, 4e-3, f"projection {name}")


def test_workload_favor_causal_prefill_from_projected_tokens(gpu_lib):
    """The unfused route from tokens: the projection GEMM, then the
    matrix-core prefill, at the prefill workload with d_model = 512."""
    w = workloads.FAVOR_CAUSAL
    c = ProjCase(w.wid, w.B, w.H, w.N, 512, w.kind, w.r)
    kw = _wl_kw(w)
    q, k, v = gpu_lib.lin_attn_qkv_project(c.x, *c.w, w.H)
    out, S, z = gpu_lib.lin_attn_causal_chunked(q, k, v, w.kind, omega=c.omega, chunk=32, **kw)
    ro, rS, rz = oracle.causal_proj(c.xh, *c.wh, w.H, w.kind, omega=c.omega_h, **kw)
    assert_parity(out, ro, 2e-2, "projected route out")
    assert_parity(S, rS, 2e-2, "projected route S")
    assert_parity(z, rz, 2e-2, "projected route z")


@pytest.mark.parametrize("N,n_seg", [(1, 0), (31, 0), (33, 1), (300, 0), (300, 5), (1000, 3)])
@pytest.mark.parametrize("norm", ["attn", "none"])
def test_bidir_backward_matrix_core_route(gpu_lib, N, n_seg, norm):
    """bf16 FAVOR+ with r = 256 runs the bidirectional backward on the matrix
    cores: ragged chunks (each wave owns 32-token chunks), segment counts,
    both readouts, and bitwise repeatability."""
    B, H = 2, 2
    c = Case(125, B, H, N, "favor", torch.bfloat16, r=256)
    do = dev(inputs.normal((B, H, N, 64), 125, inputs.T_DOUT), torch.bfloat16)
    kw = dict(scale=64 ** -0.25, norm=norm)
    got = gpu_lib.lin_attn_bidir_backward(c.q, c.k, c.v, do, "favor", n_seg=n_seg, **c.gkw(**kw))
    again = gpu_lib.lin_attn_bidir_backward(c.q, c.k, c.v, do, "favor", n_seg=n_seg,
                                            **c.gkw(**kw))
    assert all(torch.equal(a, b) for a, b in zip(got, again)), "not bitwise reproducible"
    if N == 1 and norm == "attn":
        # one token: dv = dout, dq = dk = 0 up to rounding (out = v)
        assert_parity(got[2], host(do), 1e-2, "N=1 dv")
        for g in got[:2]:
            assert float(g.abs().max()) <= 1e-2 * float(do.abs().max())
        return
    ref = oracle.bidir_backward(c.qh, c.kh, c.vh, host(do), "favor", **c.okw(**kw))
    _assert_grads(got, ref, 2e-2, f"bidir backward N={N} n_seg={n_seg} {norm}")


@pytest.mark.parametrize("num_seqs", [1000, 1100])
def test_causal_varlen_thousand_documents(gpu_lib, num_seqs):
    """Many short documents (empty ones included), on both sides of the
    1024-document limit of the per-head scan (above it the per-document scan
    runs)."""
    g = np.random.default_rng(126 + num_seqs)
    lens = g.integers(0, 40, size=num_seqs)
    lens[::97] = 0
    c, q, k, v, cu, cu_d = _packed(126, list(lens), "elu1", torch.float32, 64, 1, H=2)
    S0 = inputs.normal((num_seqs, 2, 64, 64), 126, inputs.T_PREFIX).astype(np.float32) * 0.1
    z0 = np.abs(inputs.normal((num_seqs, 2, 64), 126, inputs.T_PREFIX, 1)).astype(np.float32)
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    out, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, cu_d, "elu1", S=S, z=z, state_in=True,
                                               **c.gkw())
    ro, rS, rz = oracle.causal_varlen(c.qh[0], c.kh[0], c.vh[0], cu, "elu1", S0=S0, z0=z0,
                                      **c.okw())
    assert_parity(out, ro, 1e-4, "many documents out", lead_dims=1)
    assert_parity(S, rS, 1e-4, "many documents S")
    assert_parity(z, rz, 1e-4, "many documents z")


def test_causal_varlen_scan_range_counts(gpu_lib):
    """Packed documents from carried states at segment counts whose part
    totals put the per-head scan at 1, 2, 4, 8 and 16 ranges: documents
    spanning range boundaries, empty documents, one output set for every
    count against one oracle run."""
    g = np.random.default_rng(150)
    lens = g.integers(0, 1500, size=24)
    lens[[2, 9]] = 0
    c, q, k, v, cu, cu_d = _packed(150, list(lens), "favor", torch.bfloat16, 256, 1, H=2)
    ns, H, total = len(lens), 2, int(cu[-1])
    S0 = np.abs(inputs.normal((ns, H, 256, 64), 150, inputs.T_PREFIX)).astype(np.float32) * 0.1
    z0 = np.abs(inputs.normal((ns, H, 256), 150, inputs.T_PREFIX, 1)).astype(np.float32) + 1.0
    kw = dict(scale=64 ** -0.25)
    ro, rS, rz = oracle.causal_varlen(c.qh[0], c.kh[0], c.vh[0], cu, "favor", S0=S0, z0=z0,
                                      **c.okw(**kw))
    units = -(-total // 64)
    seen = set()
    for n_seg in (1, 12, 80, 150, 300):
        per = -(-units // min(n_seg, units))
        parts = -(-units // per) + ns  # the automatic plan's segments plus one partial per document
        seen.add(next(p for p in (1, 2, 4, 8, 16) if parts <= 32 * p or p == 16))
        S = torch.from_numpy(S0.copy()).cuda()
        z = torch.from_numpy(z0.copy()).cuda()
        out, S, z = gpu_lib.lin_attn_causal_varlen(q, k, v, cu_d, "favor", S=S, z=z, state_in=True,
                                                   n_seg=n_seg, **c.gkw(**kw))
        tag = f"varlen n_seg={n_seg} parts={parts}"
        assert_parity(out, ro, 2e-2, f"{tag} out", lead_dims=1)
        assert_parity(S, rS, 2e-2, f"{tag} S")
        assert_parity(z, rz, 2e-2, f"{tag} z")
    assert seen == {1, 2, 4, 8, 16}, seen


@pytest.mark.parametrize("N,n_seg", [(1, 0), (31, 0), (33, 1), (100, 2), (300, 0), (1000, 3)])
@pytest.mark.parametrize("norm", ["attn", "none"])
def test_causal_backward_matrix_core_route(gpu_lib, N, n_seg, norm):
    """bf16 FAVOR+ with r = 256 runs the causal backward on the matrix cores:
    ragged chunks, several segments (carried prefix and suffix states), both
    readouts, bitwise repeatability."""
    B, H = 2, 2
    c = Case(127, B, H, N, "favor", torch.bfloat16, r=256)
    do = dev(inputs.normal((B, H, N, 64), 127, inputs.T_DOUT), torch.bfloat16)
    kw = dict(scale=64 ** -0.25, norm=norm)
    got = gpu_lib.lin_attn_causal_backward(c.q, c.k, c.v, do, "favor", n_seg=n_seg, **c.gkw(**kw))
    again = gpu_lib.lin_attn_causal_backward(c.q, c.k, c.v, do, "favor", n_seg=n_seg,
                                             **c.gkw(**kw))
    assert all(torch.equal(a, b) for a, b in zip(got, again)), "not bitwise reproducible"
    if N == 1 and norm == "attn":
        assert_parity(got[2], host(do), 1e-2, "N=1 dv")
        for g in got[:2]:
            assert float(g.abs().max()) <= 1e-2 * float(do.abs().max())
        return
    ref = oracle.causal_backward(c.qh, c.kh, c.vh, host(do), "favor", **c.okw(**kw))
    _assert_grads(got, ref, 2e-2, f"causal backward N={N} n_seg={n_seg} {norm}")


F32MM_MAPS = [("identity", 64, 1), ("elu1", 64, 1), ("dpfp", 128, 1), ("dpfp", 256, 2)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,r,nu", F32MM_MAPS, ids=[f"{k}-r{r}" for k, r, _ in F32MM_MAPS])
def test_f32_matrix_core_route(gpu_lib, kind, r, nu, dtype):
    """Identity, ELU+1 and DPFP run the increments, the chunked scan and the
    bidirectional readout on the float32 matrix cores: one token, a chunk
    less one, several chunks with a ragged tail, segment counts 1, 3, 5 and
    automatic, both readouts, sum normalisation on and off, bitwise
    repeatability, then a carried-in state."""
    dt = DT[dtype]
    tol = TOL[dt]
    for i, (N, n_seg) in enumerate([(1, 0), (31, 0), (33, 1), (100, 3), (517, 0), (2000, 5)]):
        sum_norm = kind != "identity" and i % 2 == 1
        norm = "none" if kind == "identity" or i % 3 == 0 else "attn"
        c = Case(140 + i, 2, 3, N, kind, dt, r=r, nu=nu)
        kw = dict(sum_norm=sum_norm, norm=norm)
        tag = f"{kind} r={r} {dtype} N={N} n_seg={n_seg} sum_norm={sum_norm} {norm}"
        out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, n_seg=n_seg,
                                                    **c.gkw(**kw))
        o2, S2, z2 = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, n_seg=n_seg,
                                                     **c.gkw(**kw))
        assert torch.equal(out, o2) and torch.equal(S, S2) and torch.equal(z, z2), tag
        ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
        assert_parity(out, ro, tol, f"{tag} causal out")
        assert_parity(S, rS, tol, f"{tag} causal S")
        assert_parity(z, rz, tol, f"{tag} causal z")
        bo = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, kind, n_seg=n_seg, **c.gkw(**kw))
        rb, _, _ = oracle.bidir(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
        assert_parity(bo, rb, tol, f"{tag} bidir out")
    norm = "none" if kind == "identity" else "attn"
    kw = dict(sum_norm=kind == "dpfp", norm=norm)
    pre = Case(150, 1, 2, 45, kind, dt, r=r, nu=nu, rep=1)
    c = Case(150, 1, 2, 130, kind, dt, r=r, nu=nu, rep=2)
    S0, z0 = oracle_prefix_state(pre.qh, pre.kh, pre.vh, kind, **pre.okw(**kw))
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, S=torch.from_numpy(S0).cuda(),
                                                z=torch.from_numpy(z0).cuda(), state_in=True,
                                                n_seg=2, **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, S0=S0, z0=z0, **c.okw(**kw))
    assert_parity(out, ro, tol, f"{kind} carried out")
    assert_parity(S, rS, tol, f"{kind} carried S")
    assert_parity(z, rz, tol, f"{kind} carried z")


# ---------------------------------------------------------------------------
# Randomized configurations: a fixed-seed draw of shapes, maps, dtypes, segment
# counts and readouts through every forward form, decode and both backwards
# ---------------------------------------------------------------------------

def _random_configs(n, seed=20261202):
    import random
    rng = random.Random(seed)
    maps = [("favor", 256), ("favor", 128), ("favor", 96), ("favor", 32), ("elu1", 64),
            ("dpfp", 128), ("dpfp", 256)]
    out = []
    for _ in range(n):
        kind, r = rng.choice(maps)
        out.append(dict(kind=kind, r=r, nu=r // 128 if kind == "dpfp" else 1,
                        dtype=rng.choice(["bf16", "f32"]), B=rng.randint(1, 3),
                        H=rng.randint(1, 3),
                        N=rng.choice([1, 7, 31, 32, 33, 95, 200, 513, 1500, 3000]),
                        n_seg=rng.choice([0, 0, 1, 2, 5, 13, 40]),
                        sum_norm=kind != "favor" and rng.random() < 0.3,
                        norm=rng.choice(["attn", "attn", "none"])))
    return out


RANDOM_CONFIGS = _random_configs(40)


@pytest.mark.parametrize("i", range(len(RANDOM_CONFIGS)))
def test_random_configuration(gpu_lib, i):
    cfg = RANDOM_CONFIGS[i]
    kind, r, nu, N = cfg["kind"], cfg["r"], cfg["nu"], cfg["N"]
    dtype = DT[cfg["dtype"]]
    c = Case(3000 + i, cfg["B"], cfg["H"], N, kind, dtype, r=r, nu=nu)
    kw = dict(scale=64 ** -0.25 if kind == "favor" else 1.0, norm=cfg["norm"],
              sum_norm=cfg["sum_norm"])
    tol = TOL[dtype]
    out, S, z = gpu_lib.lin_attn_causal_chunked(c.q, c.k, c.v, kind, n_seg=cfg["n_seg"],
                                                **c.gkw(**kw))
    ro, rS, rz = oracle.causal(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
    assert_parity(out, ro, tol, f"{cfg} causal out")
    assert_parity(S, rS, tol, f"{cfg} causal S")
    assert_parity(z, rz, tol, f"{cfg} causal z")
    bo = gpu_lib.lin_attn_bidir(c.q, c.k, c.v, kind, n_seg=cfg["n_seg"], **c.gkw(**kw))
    rb, _, _ = oracle.bidir(c.qh, c.kh, c.vh, kind, **c.okw(**kw))
    assert_parity(bo, rb, tol, f"{cfg} bidir out")
    q1, k1, v1 = (t[:, :, 0].contiguous() for t in (c.q, c.k, c.v))
    S2, z2 = S.clone(), z.clone()
    o1 = gpu_lib.lin_attn_decode_step(q1, k1, v1, S2, z2, kind, omega=c.omega, nu=nu, **kw)
    rd, rS2, rz2 = oracle.decode(host(q1), host(k1), host(v1), host(S), host(z), kind,
                                 omega=c.omega_h, nu=nu, **kw)
    assert_parity(o1, rd, tol, f"{cfg} decode out")
    assert_parity(S2, rS2, tol, f"{cfg} decode S")
    if 1 < N <= 1500:
        do = dev(inputs.normal((cfg["B"], cfg["H"], N, 64), 3000 + i, inputs.T_DOUT), dtype)
        for form, fn, ofn in (("causal", gpu_lib.lin_attn_causal_backward, oracle.causal_backward),
                              ("bidir", gpu_lib.lin_attn_bidir_backward, oracle.bidir_backward)):
            got = fn(c.q, c.k, c.v, do, kind, n_seg=cfg["n_seg"], **c.gkw(**kw))
            ref = ofn(c.qh, c.kh, c.vh, host(do), kind, **c.okw(**kw))
            _assert_grads(got, ref, tol, f"{cfg} {form} backward")
