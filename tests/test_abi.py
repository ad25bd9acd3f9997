"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, agrees with the header on constants and struct layout, and rejects
bad arguments before enqueueing anything.  No call here reaches a kernel
launch: each one fails validation (or is an empty no-op) first.
"""
import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "lin_attn.h")

binding = pytest.importorskip("kernelized_linear_attention_amd.binding")
lib = binding.raw()
P = binding.LinAttnParams

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def header_text():
    with open(HEADER) as f:
        return f.read()


def header_defines():
    out = {}
    for m in re.finditer(r"#define\s+(LIN_ATTN_\w+)\s+\(?(-?\d+)\)?", header_text()):
        out[m.group(1)] = int(m.group(2))
    return out


def test_every_declared_symbol_is_exported():
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*|int32_t)\s+(lin_attn_\w+)\s*\(",
                              header_text(), flags=re.M))
    assert declared == set(binding.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(lin_attn_\w+)", nm))
    assert declared <= exported
    for name in declared:
        assert hasattr(lib, name)


def test_constants_match_header():
    d = header_defines()
    assert d["LIN_ATTN_ABI_VERSION"] == binding.lin_attn_abi_version() == binding.ABI_VERSION
    assert {k: d["LIN_ATTN_PHI_" + k.upper().replace("ELU1", "ELU1")] for k in binding.PHI} == \
        binding.PHI
    assert d["LIN_ATTN_NORM_ATTN"] == binding.NORM["attn"]
    assert d["LIN_ATTN_NORM_NONE"] == binding.NORM["none"]
    assert d["LIN_ATTN_F32"] == 0 and d["LIN_ATTN_BF16"] == 1
    assert d["LIN_ATTN_OP_BIDIR"] == binding.OP_BIDIR
    assert d["LIN_ATTN_OP_CAUSAL"] == binding.OP_CAUSAL
    assert d["LIN_ATTN_OP_CAUSAL_VARLEN"] == binding.OP_CAUSAL_VARLEN
    assert d["LIN_ATTN_OP_BIDIR_BACKWARD"] == binding.OP_BIDIR_BACKWARD
    assert d["LIN_ATTN_OP_CAUSAL_BACKWARD"] == binding.OP_CAUSAL_BACKWARD
    assert d["LIN_ATTN_OP_CAUSAL_PROJ"] == binding.OP_CAUSAL_PROJ
    assert d["LIN_ATTN_OP_BIDIR_PROJ"] == binding.OP_BIDIR_PROJ
    assert (d["LIN_ATTN_OK"], d["LIN_ATTN_ERR_INVALID"], d["LIN_ATTN_ERR_UNSUPPORTED"],
            d["LIN_ATTN_ERR_WORKSPACE"], d["LIN_ATTN_ERR_HIP"]) == (0, -1, -2, -3, -4)


def test_params_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    fields = [f for f, _ in P._fields_]
    body = "".join(f'printf("%zu ", offsetof(lin_attn_params, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "lin_attn.h"\n'
                   f'int main(void){{ {body} printf("%zu\\n", sizeof(lin_attn_params)); return 0; }}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    assert got[:-1] == [getattr(P, f).offset for f in fields]
    assert got[-1] == ctypes.sizeof(P)


def test_strerror_covers_every_code():
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert binding.lin_attn_strerror(code) != "unknown error code"
    assert binding.lin_attn_strerror(7) == "unknown error code"


def params(kind="favor", r=256, **kw):
    base = dict(nu=1, sum_norm=0, norm=0, dtype=1, scale=0.35, eps=1e-6, n_seg=0, reserved=0)
    base.update(kw)
    return P(binding.PHI[kind], r, base["nu"], base["sum_norm"], base["norm"], base["dtype"],
             base["scale"], base["eps"], base["n_seg"], base["reserved"])


def bidir(p, B=1, H=2, N=100, d=64, dv=64, ptr=FAKE, omega=FAKE, ws=FAKE, ws_bytes=1 << 40,
          S_out=None, z_out=None):
    pp = None if p is None else ctypes.byref(p)
    return lib.lin_attn_bidir(pp, ptr, ptr, ptr, B, H, N, d, dv, omega, ptr, S_out, z_out, ws,
                              ws_bytes, None)


def causal(p, B=1, H=2, N=100, d=64, dv=64, ptr=FAKE, omega=FAKE, chunk=0, state_in=0, ws=FAKE,
           ws_bytes=1 << 40, S=FAKE, z=FAKE):
    return lib.lin_attn_causal_chunked(ctypes.byref(p), ptr, ptr, ptr, B, H, N, d, dv, omega, chunk,
                                       S, z, state_in, ptr, ws, ws_bytes, None)


def varlen(p, num_seqs=2, H=2, total=100, d=64, dv=64, ptr=FAKE, cu=FAKE, omega=FAKE, state_in=0,
           ws=FAKE, ws_bytes=1 << 40, S=FAKE, z=FAKE):
    return lib.lin_attn_causal_varlen(ctypes.byref(p), ptr, ptr, ptr, cu, num_seqs, H, total, d, dv,
                                      omega, S, z, state_in, ptr, ws, ws_bytes, None)


def decode(p, B=4, H=2, d=64, dv=64, ptr=FAKE, omega=FAKE):
    return lib.lin_attn_decode_step(ctypes.byref(p), ptr, ptr, ptr, B, H, d, dv, omega, ptr, ptr,
                                    ptr, None)


def featuremap(p, B=1, H=1, N=10, d=64, ptr=FAKE, omega=FAKE):
    return lib.lin_attn_featuremap(ctypes.byref(p), ptr, B, H, N, d, omega, ptr, None)


@pytest.mark.parametrize("bad", [
    dict(phi=7), dict(norm=3), dict(dtype=5), dict(sum_norm=2), dict(reserved=1), dict(eps=0.0),
    dict(eps=-1e-6), dict(eps=float("nan")), dict(scale=float("inf")), dict(n_seg=-1),
])
def test_bad_parameters_are_invalid(bad):
    p = params()
    for k, v in bad.items():
        setattr(p, k, v)
    for call in (bidir, causal, decode, featuremap):
        assert call(p) == INVALID


def test_feature_width_must_match_the_map():
    assert bidir(params("elu1", r=32)) == INVALID        # r must equal d
    assert bidir(params("identity", r=128)) == INVALID
    assert bidir(params("dpfp", r=256, nu=0)) == INVALID  # 1 <= nu <= 2d - 1
    assert bidir(params("dpfp", r=256, nu=128)) == INVALID
    assert bidir(params("dpfp", r=128, nu=2)) == INVALID  # r = 2 d nu
    assert bidir(params("favor", r=256), omega=None) == INVALID
    assert bidir(params("favor", r=0)) == INVALID


def test_pointers_sizes_and_enums():
    p = params()
    assert bidir(None) == INVALID
    assert bidir(p, ptr=None) == INVALID
    assert bidir(p, ptr=FAKE + 4) == INVALID             # 16-byte alignment
    assert bidir(p, N=-1) == INVALID
    assert bidir(p, B=-2) == INVALID
    assert causal(p, chunk=16) == INVALID
    assert causal(p, chunk=-32) == INVALID
    assert causal(p, state_in=2) == INVALID
    assert causal(p, S=None) == INVALID
    assert decode(p, ptr=None) == INVALID
    assert featuremap(p, ptr=None) == INVALID


def test_outside_gpu_coverage_is_unsupported():
    assert bidir(params("elu1", r=32), d=32, dv=64) == UNSUPPORTED
    assert bidir(params(), dv=32) == UNSUPPORTED
    assert bidir(params("favor", r=544)) == UNSUPPORTED   # r <= 512 on the forward kernels
    assert bidir(params("favor", r=48)) == UNSUPPORTED    # a multiple of 32
    assert causal(params("dpfp", r=640, nu=5)) == UNSUPPORTED
    assert decode(params("favor", r=272)) == UNSUPPORTED
    assert decode(params("favor", r=576)) == UNSUPPORTED
    # 64- and 128-token intra-chunk blocks are valid but run by no kernel
    assert causal(params(), chunk=64) == UNSUPPORTED
    assert causal(params(), chunk=128) == UNSUPPORTED
    assert causal(params("elu1", r=64, dtype=0), chunk=128) == UNSUPPORTED
    # past r = 256 the vector kernels run 16- or 4-token blocks: only chunk 0
    assert causal(params("favor", r=384), chunk=32) == UNSUPPORTED
    assert causal(params("dpfp", r=512, nu=4, dtype=0), chunk=32) == UNSUPPORTED
    # accepted by validation (without a GPU the launch itself then fails)
    assert causal(params("favor", r=384), chunk=0) not in (INVALID, UNSUPPORTED)
    assert causal(params("favor", r=256), chunk=32) not in (INVALID, UNSUPPORTED)


def test_chunk_sizes_the_causal_workspace_only():
    p = params()
    args = (p, 1, 8, 4096, 64, 64)
    need = binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, *args, 0)
    assert need > 0
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, *args, 32) == need
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, *args, 64) == 0
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, *args, 16) == 0
    assert binding.lin_attn_workspace_bytes(binding.OP_BIDIR, *args, 64) == \
        binding.lin_attn_workspace_bytes(binding.OP_BIDIR, *args, 0)
    wide = (params("favor", r=384), 1, 8, 4096, 64, 64)
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, *wide, 0) > 0
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, *wide, 32) == 0


def causal_noalloc(p, B=1, H=2, N=100, d=64, dv=64, ptr=FAKE, omega=FAKE, chunk=0, state_in=0,
                   S=FAKE, z=FAKE):
    return lib.lin_attn_causal_chunked_noalloc(ctypes.byref(p), ptr, ptr, ptr, B, H, N, d, dv, omega,
                                               chunk, S, z, state_in, ptr, None)


def test_noalloc_arguments():
    """The allocation-free causal call validates like lin_attn_causal_chunked
    and refuses problems whose workspace exceeds its static scratch."""
    p = params()
    assert causal_noalloc(p, ptr=None) == INVALID
    assert causal_noalloc(p, chunk=16) == INVALID
    assert causal_noalloc(p, state_in=2) == INVALID
    assert causal_noalloc(p, S=None) == INVALID
    assert causal_noalloc(p, chunk=64) == UNSUPPORTED
    assert causal_noalloc(params("favor", r=544)) == UNSUPPORTED
    assert causal_noalloc(p, H=0) == OK
    # one (S | z) block of 66,560 bytes per head at least: 1024 heads need 68 MB
    big = binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, p, 4, 256, 100, 64, 64, 0)
    assert big > binding.NOALLOC_SCRATCH_BYTES
    assert causal_noalloc(p, B=4, H=256) == WORKSPACE
    assert header_defines_size("LIN_ATTN_NOALLOC_SCRATCH_BYTES") == binding.NOALLOC_SCRATCH_BYTES


def header_defines_size(name):
    m = re.search(r"#define\s+" + name + r"\s+\(\(size_t\)(\d+) << (\d+)\)", header_text())
    return int(m.group(1)) << int(m.group(2))


def test_sizes_past_the_grid_limits_are_unsupported():
    """Flattened grids stay within 32 bits: more than 2^24 heads in a batch,
    a B*H product past 2^31 or more than 2^40 tokens is refused before any
    launch (and B*H = 2^24 exactly is still accepted)."""
    p = params()
    assert causal(p, B=1 << 13, H=1 << 12) == UNSUPPORTED        # 2^25 heads
    assert causal(p, B=1 << 31, H=2) == UNSUPPORTED              # product past 2^31
    assert bidir(p, B=1, H=1, N=(1 << 40) + 1) == UNSUPPORTED
    assert decode(p, B=1 << 20, H=1 << 5) == UNSUPPORTED
    assert varlen(p, num_seqs=1 << 20, H=1 << 5) == UNSUPPORTED
    # the limit itself is inside the coverage: only the workspace is short
    assert causal(p, B=1 << 12, H=1 << 12, ws_bytes=0) == WORKSPACE


def test_small_workspace_is_rejected():
    p = params()
    need = binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, p, 1, 2, 100, 64, 64)
    assert need > 0
    assert causal(p, ws_bytes=need - 4) == WORKSPACE
    assert causal(p, ws=None, ws_bytes=0) == WORKSPACE
    need_b = binding.lin_attn_workspace_bytes(binding.OP_BIDIR, p, 1, 2, 100, 64, 64)
    assert bidir(p, ws_bytes=need_b - 4) == WORKSPACE


def test_empty_inputs_are_noops():
    p = params()
    assert bidir(p, B=0) == OK
    assert bidir(p, N=0, S_out=None, z_out=None) == OK
    assert causal(p, H=0) == OK
    assert causal(p, N=0, state_in=1) == OK   # the state after no token is the input state
    assert decode(p, B=0) == OK
    assert featuremap(p, N=0) == OK


def test_workspace_size_formula():
    """One (S | z) block of r*dv + r floats per head and sequence segment;
    bidirectional adds one per head for the full summary.  Both kernel
    families aim at two workgroups per CU: at B=1, H=8, N=65536 that is 64
    segments of 1024 tokens per head (FAVOR+ with bfloat16 inputs and r = 256
    on the matrix-core kernels, float32 on the vector kernels)."""
    p = params()
    E = 256 * 64 + 256
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, p, 1, 8, 65536, 64, 64) == \
        8 * 64 * E * 4
    assert binding.lin_attn_workspace_bytes(binding.OP_BIDIR, p, 1, 8, 65536, 64, 64) == \
        (8 * 64 + 8) * E * 4
    pf = params(dtype=0)
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, pf, 1, 8, 65536, 64, 64) == \
        8 * 64 * E * 4
    p1 = params(n_seg=1)
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, p1, 2, 3, 1000, 64, 64) == 6 * 1 * E * 4
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL, p, 2, 3, 0, 64, 64) == 0
    assert binding.lin_attn_workspace_bytes(9, p, 2, 3, 10, 64, 64) == 0


def test_varlen_arguments():
    p = params()
    assert varlen(p, num_seqs=-1) == INVALID
    assert varlen(p, total=-1) == INVALID
    assert varlen(p, num_seqs=0, total=10) == INVALID   # tokens of no sequence
    assert varlen(p, cu=None) == INVALID
    assert varlen(p, cu=FAKE + 2) == INVALID            # int32 array: 4-byte alignment
    assert varlen(p, state_in=2) == INVALID
    assert varlen(p, S=None) == INVALID
    assert varlen(p, ptr=None) == INVALID
    assert varlen(params("favor", r=544)) == UNSUPPORTED
    need = binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_VARLEN, p, 2, 2, 100, 64, 64)
    assert need > 0
    assert varlen(p, ws_bytes=need - 8) == WORKSPACE
    assert varlen(p, ws=None, ws_bytes=0) == WORKSPACE
    assert varlen(p, num_seqs=0, total=0) == OK
    assert varlen(p, H=0) == OK


def test_varlen_workspace_formula():
    """Increments of every part of every head -- the segments of the uniform
    plan over all tokens plus one partial segment per sequence, one part
    each -- then the segment table (two int64 per part, after 256-byte
    alignment), the first part of every sequence and the dispatch order (one
    int64 per segment)."""
    p = params()
    E = 256 * 64 + 256
    # H = 8, total = 65536: 64 segments of 1024 tokens per head, + 4 sequences
    parts = 64 + 4
    inc = 8 * parts * E * 4
    assert inc % 256 == 0
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_VARLEN, p, 4, 8, 65536, 64, 64) == \
        inc + parts * 16 + 5 * 8 + parts * 8
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_VARLEN, p, 4, 8, 0, 64, 64) == 0


def test_orf_arguments():
    orf = lib.lin_attn_orf_omega
    assert orf(None, None, 1, 256, 64, 1, FAKE, None) == INVALID
    assert orf(FAKE, None, 1, 256, 64, 1, None, None) == INVALID
    assert orf(FAKE + 4, None, 1, 256, 64, 1, FAKE, None) == INVALID
    assert orf(FAKE, FAKE + 8, 1, 256, 64, 1, FAKE, None) == INVALID
    assert orf(FAKE, None, -1, 256, 64, 1, FAKE, None) == INVALID
    assert orf(FAKE, None, 1, -2, 64, 1, FAKE, None) == INVALID
    assert orf(FAKE, None, 1, 256, 0, 1, FAKE, None) == INVALID
    assert orf(FAKE, None, 1, 256, 64, 2, FAKE, None) == INVALID
    assert orf(FAKE, None, 1, 256, 65, 1, FAKE, None) == UNSUPPORTED
    assert orf(FAKE, None, 0, 256, 64, 1, FAKE, None) == OK
    assert orf(FAKE, None, 1, 0, 64, 1, FAKE, None) == OK


def backward(p, fn="lin_attn_causal_backward", B=1, H=2, N=100, d=64, dv=64, ptr=FAKE,
             dout=FAKE, grads=FAKE, omega=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return getattr(lib, fn)(ctypes.byref(p), ptr, ptr, ptr, dout, B, H, N, d, dv, omega, grads,
                            grads, grads, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["lin_attn_bidir_backward", "lin_attn_causal_backward"])
def test_backward_arguments(fn):
    p = params()
    assert backward(p, fn, B=-1) == INVALID
    assert backward(p, fn, N=-1) == INVALID
    assert backward(p, fn, ptr=None) == INVALID
    assert backward(p, fn, dout=None) == INVALID
    assert backward(p, fn, dout=FAKE + 2) == INVALID
    assert backward(p, fn, grads=None) == INVALID
    assert backward(p, fn, omega=None) == INVALID
    assert backward(p, fn, ws=FAKE + 4) == INVALID
    assert backward(params(eps=0.0), fn) == INVALID
    assert backward(params("favor", r=512), fn) == UNSUPPORTED   # r <= 256 for the backward
    assert backward(params("dpfp", r=384, nu=3), fn) == UNSUPPORTED
    op_ = binding.OP_BIDIR_BACKWARD if "bidir" in fn else binding.OP_CAUSAL_BACKWARD
    assert binding.lin_attn_workspace_bytes(op_, params("favor", r=384), 1, 2, 100, 64, 64) == 0
    assert backward(p, fn, d=32) == UNSUPPORTED
    op = binding.OP_BIDIR_BACKWARD if "bidir" in fn else binding.OP_CAUSAL_BACKWARD
    need = binding.lin_attn_workspace_bytes(op, p, 1, 2, 100, 64, 64)
    assert need > 0
    assert backward(p, fn, ws_bytes=need - 4) == WORKSPACE
    assert backward(p, fn, ws=None, ws_bytes=0) == WORKSPACE
    assert backward(p, fn, N=0, ptr=None, dout=None, grads=None) == OK
    assert backward(p, fn, H=0) == OK


def test_backward_workspace_formula():
    """Forward and backward increments of every segment (the vector kernels'
    plan: two workgroups per CU, 64 segments of 1024 tokens per head at H = 8,
    N = 65536), then the two full summaries per head (bidirectional only),
    then the dnum (bf16) and dden of every token (the vector route's causal
    pass uses two floats per token of that space: 1 / max(den, eps) and the
    denominator's gradient), then r * 64 floats for omega^T (used in bfloat16
    by FAVOR+)."""
    p = params()
    E = 256 * 64 + 256
    inc = 2 * 8 * 64 * E * 4
    om_t = 256 * 64 * 4
    # bidirectional: + dnum (bf16) and dden per token for the matrix-core route
    tokens = 8 * 65536 * (32 + 1) * 4
    assert binding.lin_attn_workspace_bytes(binding.OP_BIDIR_BACKWARD, p, 1, 8, 65536, 64, 64) == \
        inc + 2 * 8 * E * 4 + tokens + om_t
    # the causal matrix-core route (these parameters: bf16 FAVOR+, r = 256)
    # plans one segment per CU: 32 segments of 2048 tokens per head at H = 8
    inc32 = 2 * 8 * 32 * E * 4
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_BACKWARD, p, 1, 8, 65536, 64, 64) == \
        inc32 + tokens + om_t
    # ... and the vector route (float32 inputs) two per CU, as above
    p32 = params(dtype=0)
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_BACKWARD, p32, 1, 8, 65536, 64, 64) == \
        inc + tokens + om_t
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_BACKWARD, p, 1, 8, 0, 64, 64) == 0


def causal_proj(p, B=1, H=2, N=100, dm=512, d=64, dv=64, x=FAKE, w=FAKE, omega=FAKE, state_in=0,
                out=FAKE, ws=FAKE, ws_bytes=1 << 40, S=FAKE, z=FAKE):
    return lib.lin_attn_causal_proj(ctypes.byref(p), x, w, w, w, B, H, N, dm, d, dv, omega, S, z,
                                    state_in, out, ws, ws_bytes, None)


def bidir_proj(p, B=1, H=2, N=100, dm=512, d=64, dv=64, x=FAKE, w=FAKE, omega=FAKE, out=FAKE,
               ws=FAKE, ws_bytes=1 << 40):
    return lib.lin_attn_bidir_proj(ctypes.byref(p), x, w, w, w, B, H, N, dm, d, dv, omega, out,
                                   None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("call", [causal_proj, bidir_proj])
def test_projected_call_arguments(call):
    p = params()
    assert call(p, dm=0) == INVALID
    assert call(p, dm=-16) == INVALID
    assert call(p, x=None) == INVALID
    assert call(p, x=FAKE + 8) == INVALID
    assert call(p, w=None) == INVALID
    assert call(p, out=None) == INVALID
    assert call(p, omega=None) == INVALID
    assert call(p, N=-1) == INVALID
    assert call(p, dm=520) == UNSUPPORTED               # not a multiple of 16
    assert call(params(dtype=0)) == UNSUPPORTED          # bfloat16 tokens and weights only
    assert call(p, d=32) == UNSUPPORTED
    assert call(params("favor", r=384)) == UNSUPPORTED   # r <= 256 for the projected calls
    op = binding.OP_CAUSAL_PROJ if call is causal_proj else binding.OP_BIDIR_PROJ
    need = binding.lin_attn_workspace_bytes(op, p, 1, 2, 100, 64, 64)
    assert need > 0
    assert call(p, ws_bytes=need - 4) == WORKSPACE
    assert call(p, B=0) == OK
    if call is causal_proj:
        assert call(p, state_in=3) == INVALID
        assert call(p, S=None) == INVALID


def test_projected_workspace_formula():
    """Matrix-core configuration (bf16 FAVOR+, r = 256): q, k, v in bfloat16
    (3 B H N d, 256-byte aligned) then the matrix-core workspace (64 segments
    per head at H = 8, N = 65536; one (S | z) block per segment, plus the
    summary per head when bidirectional).  Other maps: the vector kernels'
    plan alone, which at this shape is also 64 segments per head."""
    p = params()
    E = 256 * 64 + 256
    qkv = 3 * 8 * 65536 * 64 * 2
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_PROJ, p, 1, 8, 65536, 64, 64) == \
        qkv + 8 * 64 * E * 4
    assert binding.lin_attn_workspace_bytes(binding.OP_BIDIR_PROJ, p, 1, 8, 65536, 64, 64) == \
        qkv + (8 * 64 + 8) * E * 4
    pe = params("elu1", r=64)
    E64 = 64 * 64 + 64
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_PROJ, pe, 1, 8, 65536, 64, 64) == \
        8 * 64 * E64 * 4
    # an odd token count: q, k, v padded to a 256-byte boundary
    odd = 3 * 1 * 3 * 64 * 2
    assert binding.lin_attn_workspace_bytes(binding.OP_CAUSAL_PROJ, params(n_seg=1), 1, 1, 3, 64, 64) \
        == (odd + 255) // 256 * 256 + E * 4


def test_qkv_project_arguments():
    f = lib.lin_attn_qkv_project

    def call(x=FAKE, w=FAKE, B=1, N=100, dm=512, H=8, d=64, out=FAKE):
        return f(x, w, w, w, B, N, dm, H, d, out, out, out, None)

    assert call(x=None) == INVALID
    assert call(w=FAKE + 4) == INVALID
    assert call(out=None) == INVALID
    assert call(B=-1) == INVALID
    assert call(dm=0) == INVALID
    assert call(d=32) == UNSUPPORTED
    assert call(dm=520) == UNSUPPORTED
    assert call(N=0, x=None, w=None, out=None) == OK
    assert call(H=0) == OK
