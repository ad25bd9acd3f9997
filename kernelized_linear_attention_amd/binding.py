"""Python binding of liblinattn.so: the entry points of include/lin_attn.h under
the same names, taking torch tensors that live on the GPU.

This module only marshals arguments: it checks devices, dtypes and
contiguity, allocates outputs and workspaces with torch (device memory is
torch's), passes raw pointers and the current HIP stream, and raises on a
nonzero return code.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  Importing it fails when the library has
not been built (``python kernelized_linear_attention_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: the library binds to the HIP runtime torch already loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
# LINATTN_LIBRARY names another build of the same library (the host-side
# sanitizer build of tests/sanitizers.py); there is no other choice of code.
LIB_PATH = os.environ.get("LINATTN_LIBRARY") or os.path.join(_HERE, "liblinattn.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python kernelized_linear_attention_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

PHI = {"identity": 0, "elu1": 1, "favor": 2, "dpfp": 3}
NORM = {"attn": 0, "none": 1}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
OP_BIDIR = 1
OP_CAUSAL = 2
OP_CAUSAL_VARLEN = 3
OP_BIDIR_BACKWARD = 4
OP_CAUSAL_BACKWARD = 5
OP_CAUSAL_PROJ = 6
OP_BIDIR_PROJ = 7
ABI_VERSION = 1
NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol include/lin_attn.h declares.
EXPORTS = ("lin_attn_featuremap", "lin_attn_bidir", "lin_attn_causal_chunked",
           "lin_attn_causal_chunked_noalloc",
           "lin_attn_causal_varlen", "lin_attn_orf_omega", "lin_attn_bidir_backward",
           "lin_attn_causal_backward", "lin_attn_causal_proj", "lin_attn_bidir_proj",
           "lin_attn_qkv_project",
           "lin_attn_decode_step", "lin_attn_workspace_bytes", "lin_attn_strerror",
           "lin_attn_abi_version")


class LinAttnParams(ctypes.Structure):
    _fields_ = [("phi", ctypes.c_int32), ("r", ctypes.c_int32), ("nu", ctypes.c_int32),
                ("sum_norm", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("eps", ctypes.c_float),
                ("n_seg", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_PP = ctypes.POINTER(LinAttnParams)
_lib.lin_attn_featuremap.argtypes = [_PP, _P, _I64, _I64, _I64, _I64, _P, _P, _P]
_lib.lin_attn_featuremap.restype = ctypes.c_int
_lib.lin_attn_bidir.argtypes = [_PP, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                                _P, ctypes.c_size_t, _P]
_lib.lin_attn_bidir.restype = ctypes.c_int
_lib.lin_attn_causal_chunked.argtypes = [_PP, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _I32,
                                         _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]
_lib.lin_attn_causal_chunked.restype = ctypes.c_int
_lib.lin_attn_causal_chunked_noalloc.argtypes = [_PP, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P,
                                                 _I32, _P, _P, _I32, _P, _P]
_lib.lin_attn_causal_chunked_noalloc.restype = ctypes.c_int
_lib.lin_attn_causal_varlen.argtypes = [_PP, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P,
                                        _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]
_lib.lin_attn_causal_varlen.restype = ctypes.c_int
_lib.lin_attn_orf_omega.argtypes = [_P, _P, _I64, _I64, _I64, _I32, _P, _P]
_lib.lin_attn_orf_omega.restype = ctypes.c_int
for _fn in (_lib.lin_attn_bidir_backward, _lib.lin_attn_causal_backward):
    _fn.argtypes = [_PP, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P,
                    ctypes.c_size_t, _P]
    _fn.restype = ctypes.c_int
_lib.lin_attn_causal_proj.argtypes = [_PP, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                                      _P, _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]
_lib.lin_attn_causal_proj.restype = ctypes.c_int
_lib.lin_attn_bidir_proj.argtypes = [_PP, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P,
                                     _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.lin_attn_bidir_proj.restype = ctypes.c_int
_lib.lin_attn_qkv_project.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                                      _P]
_lib.lin_attn_qkv_project.restype = ctypes.c_int
_lib.lin_attn_decode_step.argtypes = [_PP, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]
_lib.lin_attn_decode_step.restype = ctypes.c_int
_lib.lin_attn_workspace_bytes.argtypes = [_I32, _PP, _I64, _I64, _I64, _I64, _I64, _I32]
_lib.lin_attn_workspace_bytes.restype = ctypes.c_size_t
_lib.lin_attn_strerror.argtypes = [_I32]
_lib.lin_attn_strerror.restype = ctypes.c_char_p
_lib.lin_attn_abi_version.argtypes = []
_lib.lin_attn_abi_version.restype = _I32


class LinAttnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code}: {lin_attn_strerror(code)}")
        self.code = code


def lin_attn_strerror(code: int) -> str:
    return _lib.lin_attn_strerror(int(code)).decode()


def lin_attn_abi_version() -> int:
    return int(_lib.lin_attn_abi_version())


def feature_width(kind: str, d: int, nu: int = 1, omega=None) -> int:
    if kind in ("identity", "elu1"):
        return d
    if kind == "dpfp":
        return 2 * d * nu
    if kind == "favor":
        if omega is None:
            raise ValueError("FAVOR+ needs omega")
        return int(omega.shape[0])
    raise ValueError(f"unknown feature map {kind!r}")


def make_params(kind: str, r: int, *, nu: int = 1, sum_norm: bool = False, norm: str = "attn",
                dtype=torch.bfloat16, scale: float = 1.0, eps: float = 1e-6,
                n_seg: int = 0) -> LinAttnParams:
    return LinAttnParams(PHI[kind], int(r), int(nu), int(bool(sum_norm)), NORM[norm],
                         DTYPE[dtype], float(scale), float(eps), int(n_seg), 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev, stream):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise LinAttnError(fn, rc)


def _dev_tensor(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return t


def lin_attn_workspace_bytes(op: int, params: LinAttnParams, B: int, H: int, N: int, d: int,
                             dv: int, chunk: int = 0) -> int:
    return int(_lib.lin_attn_workspace_bytes(op, ctypes.byref(params), B, H, N, d, dv, chunk))


def _omega(kind, omega, dtype):
    if kind != "favor":
        return None
    return _dev_tensor("omega", omega, dtype)


def lin_attn_featuremap(x, kind, *, omega=None, nu=1, sum_norm=False, scale=1.0, eps=1e-6,
                        out=None, stream=None):
    """phi(scale * x) for x [B, H, N, d]; returns float32 [B, H, N, r]."""
    _dev_tensor("x", x)
    B, H, N, d = x.shape
    om = _omega(kind, omega, x.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, dtype=x.dtype, scale=scale, eps=eps)
    if out is None:
        out = torch.empty((B, H, N, r), dtype=torch.float32, device=x.device)
    _dev_tensor("out", out, torch.float32)
    rc = _lib.lin_attn_featuremap(ctypes.byref(p), _ptr(x), B, H, N, d, _ptr(om), _ptr(out),
                                  _stream(x.device, stream))
    _check("lin_attn_featuremap", rc)
    return out


def _workspace(op, p, B, H, N, d, dv, chunk, device, workspace):
    need = lin_attn_workspace_bytes(op, p, B, H, N, d, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _dev_tensor("workspace", workspace)
    return workspace, workspace.numel() * workspace.element_size()


def lin_attn_bidir(q, k, v, kind, *, omega=None, nu=1, sum_norm=False, norm="attn", scale=1.0,
                   eps=1e-6, n_seg=0, out=None, S_out=None, z_out=None, workspace=None,
                   stream=None):
    """Bidirectional reassociated attention.  q, k [B, H, N, d], v [B, H, N, dv].
    Returns out (and fills S_out [B, H, r, dv], z_out [B, H, r] when given)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, q.dtype)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    om = _omega(kind, omega, q.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=q.dtype, scale=scale,
                    eps=eps, n_seg=n_seg)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    _dev_tensor("out", out, q.dtype)
    for n, t in (("S_out", S_out), ("z_out", z_out)):
        if t is not None:
            _dev_tensor(n, t, torch.float32)
    ws, ws_bytes = _workspace(OP_BIDIR, p, B, H, N, d, dv, 0, q.device, workspace)
    rc = _lib.lin_attn_bidir(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), B, H, N, d, dv, _ptr(om),
                             _ptr(out), _ptr(S_out), _ptr(z_out), _ptr(ws), ws_bytes,
                             _stream(q.device, stream))
    _check("lin_attn_bidir", rc)
    return out


def lin_attn_causal_chunked(q, k, v, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
                            scale=1.0, eps=1e-6, n_seg=0, chunk=0, S=None, z=None,
                            state_in=False, out=None, workspace=None, stream=None):
    """Causal prefill.  Returns (out, S, z); S, z are updated in place when
    given (and read first when state_in)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, q.dtype)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    om = _omega(kind, omega, q.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=q.dtype, scale=scale,
                    eps=eps, n_seg=n_seg)
    if S is None:
        if state_in:
            raise ValueError("state_in needs S and z")
        S = torch.empty((B, H, r, dv), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, r), dtype=torch.float32, device=q.device)
    _dev_tensor("S", S, torch.float32)
    _dev_tensor("z", z, torch.float32)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    _dev_tensor("out", out, q.dtype)
    ws, ws_bytes = _workspace(OP_CAUSAL, p, B, H, N, d, dv, chunk, q.device, workspace)
    rc = _lib.lin_attn_causal_chunked(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), B, H, N, d, dv,
                                      _ptr(om), int(chunk), _ptr(S), _ptr(z), int(bool(state_in)),
                                      _ptr(out), _ptr(ws), ws_bytes, _stream(q.device, stream))
    _check("lin_attn_causal_chunked", rc)
    return out, S, z


def lin_attn_causal_chunked_noalloc(q, k, v, kind, *, omega=None, nu=1, sum_norm=False,
                                    norm="attn", scale=1.0, eps=1e-6, n_seg=0, chunk=0, S=None,
                                    z=None, state_in=False, out=None, stream=None):
    """lin_attn_causal_chunked with the library's static per-GPU scratch as the
    workspace (the library allocates nothing for the call).  Returns (out, S,
    z) like lin_attn_causal_chunked; outputs are allocated here only when not
    given."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, q.dtype)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    om = _omega(kind, omega, q.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=q.dtype, scale=scale,
                    eps=eps, n_seg=n_seg)
    if S is None:
        if state_in:
            raise ValueError("state_in needs S and z")
        S = torch.empty((B, H, r, dv), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, r), dtype=torch.float32, device=q.device)
    _dev_tensor("S", S, torch.float32)
    _dev_tensor("z", z, torch.float32)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    _dev_tensor("out", out, q.dtype)
    rc = _lib.lin_attn_causal_chunked_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), B, H, N,
                                              d, dv, _ptr(om), int(chunk), _ptr(S), _ptr(z),
                                              int(bool(state_in)), _ptr(out),
                                              _stream(q.device, stream))
    _check("lin_attn_causal_chunked_noalloc", rc)
    return out, S, z


def lin_attn_causal_varlen(q, k, v, cu_seqlens, kind, *, omega=None, nu=1, sum_norm=False,
                           norm="attn", scale=1.0, eps=1e-6, n_seg=0, S=None, z=None,
                           state_in=False, out=None, workspace=None, stream=None):
    """Causal prefill of packed sequences.  q, k [H, total, d], v [H, total, dv];
    cu_seqlens int32 [num_seqs + 1] on the device.  Returns (out, S, z) with
    S [num_seqs, H, r, dv], z [num_seqs, H, r] (updated in place when given,
    read first when state_in)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, q.dtype)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32)
    H, total, d = q.shape
    dv = v.shape[-1]
    num_seqs = cu_seqlens.numel() - 1
    om = _omega(kind, omega, q.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=q.dtype, scale=scale,
                    eps=eps, n_seg=n_seg)
    if S is None:
        if state_in:
            raise ValueError("state_in needs S and z")
        S = torch.empty((num_seqs, H, r, dv), dtype=torch.float32, device=q.device)
        z = torch.empty((num_seqs, H, r), dtype=torch.float32, device=q.device)
    _dev_tensor("S", S, torch.float32)
    _dev_tensor("z", z, torch.float32)
    if out is None:
        out = torch.empty((H, total, dv), dtype=q.dtype, device=q.device)
    _dev_tensor("out", out, q.dtype)
    ws, ws_bytes = _workspace(OP_CAUSAL_VARLEN, p, num_seqs, H, total, d, dv, 0, q.device,
                              workspace)
    rc = _lib.lin_attn_causal_varlen(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                     num_seqs, H, total, d, dv, _ptr(om), _ptr(S), _ptr(z),
                                     int(bool(state_in)), _ptr(out), _ptr(ws), ws_bytes,
                                     _stream(q.device, stream))
    _check("lin_attn_causal_varlen", rc)
    return out, S, z


def lin_attn_orf_omega(gauss, len_gauss=None, *, r=None, dtype=torch.bfloat16, out=None,
                       stream=None):
    """Orthogonal random features from Gaussian draws on the device: gauss
    float32 [n_mat, nblk, d, d] (or [nblk, d, d]), len_gauss float32
    [n_mat, nblk*d, d] or None (rows scaled to sqrt(d)).  Returns omega
    [n_mat, r, d] (or [r, d]) in dtype; r defaults to nblk * d."""
    _dev_tensor("gauss", gauss, torch.float32)
    single = gauss.dim() == 3
    g = gauss.unsqueeze(0) if single else gauss
    n_mat, nblk, d, _ = g.shape
    r = nblk * d if r is None else int(r)
    if len_gauss is not None:
        _dev_tensor("len_gauss", len_gauss, torch.float32)
    if out is None:
        out = torch.empty((n_mat, r, d), dtype=dtype, device=gauss.device)
    _dev_tensor("out", out, dtype)
    rc = _lib.lin_attn_orf_omega(_ptr(g), _ptr(len_gauss), n_mat, r, d, DTYPE[dtype], _ptr(out),
                                 _stream(gauss.device, stream))
    _check("lin_attn_orf_omega", rc)
    return out[0] if single else out


def lin_attn_decode_step(q, k, v, S, z, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
                         scale=1.0, eps=1e-6, out=None, stream=None):
    """One decode step for q, k [B, H, d], v [B, H, dv]; S, z updated in place.
    Returns out [B, H, dv]."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, q.dtype)
    B, H, d = q.shape
    dv = v.shape[-1]
    om = _omega(kind, omega, q.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=q.dtype, scale=scale,
                    eps=eps)
    _dev_tensor("S", S, torch.float32)
    _dev_tensor("z", z, torch.float32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _dev_tensor("out", out, q.dtype)
    rc = _lib.lin_attn_decode_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), B, H, d, dv,
                                   _ptr(om), _ptr(S), _ptr(z), _ptr(out),
                                   _stream(q.device, stream))
    _check("lin_attn_decode_step", rc)
    return out


def _proj_args(x, w_q, w_k, w_v, heads, kind, omega, nu):
    _dev_tensor("x", x, torch.bfloat16)
    for n, t in (("w_q", w_q), ("w_k", w_k), ("w_v", w_v)):
        _dev_tensor(n, t, torch.bfloat16)
    B, N, dm = x.shape
    d = w_q.shape[0] // heads
    dv = w_v.shape[0] // heads
    om = _omega(kind, omega, torch.bfloat16)
    return B, N, dm, d, dv, om, feature_width(kind, d, nu, om)


def lin_attn_causal_proj(x, w_q, w_k, w_v, heads, kind, *, omega=None, nu=1, sum_norm=False,
                         norm="attn", scale=1.0, eps=1e-6, n_seg=0, S=None, z=None,
                         state_in=False, out=None, workspace=None, stream=None):
    """Causal prefill from tokens x [B, N, d_model] (bf16) with the q/k/v
    projection w_* [heads * 64, d_model] fused into the kernels.  Returns
    (out [B, heads, N, 64], S, z)."""
    B, N, dm, d, dv, om, r = _proj_args(x, w_q, w_k, w_v, heads, kind, omega, nu)
    H = heads
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=torch.bfloat16,
                    scale=scale, eps=eps, n_seg=n_seg)
    if S is None:
        if state_in:
            raise ValueError("state_in needs S and z")
        S = torch.empty((B, H, r, dv), dtype=torch.float32, device=x.device)
        z = torch.empty((B, H, r), dtype=torch.float32, device=x.device)
    _dev_tensor("S", S, torch.float32)
    _dev_tensor("z", z, torch.float32)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=torch.bfloat16, device=x.device)
    _dev_tensor("out", out, torch.bfloat16)
    ws, ws_bytes = _workspace(OP_CAUSAL_PROJ, p, B, H, N, d, dv, 0, x.device, workspace)
    rc = _lib.lin_attn_causal_proj(ctypes.byref(p), _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), B, H,
                                   N, dm, d, dv, _ptr(om), _ptr(S), _ptr(z), int(bool(state_in)),
                                   _ptr(out), _ptr(ws), ws_bytes, _stream(x.device, stream))
    _check("lin_attn_causal_proj", rc)
    return out, S, z


def lin_attn_bidir_proj(x, w_q, w_k, w_v, heads, kind, *, omega=None, nu=1, sum_norm=False,
                        norm="attn", scale=1.0, eps=1e-6, n_seg=0, out=None, S_out=None,
                        z_out=None, workspace=None, stream=None):
    """Bidirectional attention from tokens x [B, N, d_model] (bf16) with the
    q/k/v projection fused into the kernels.  Returns out [B, heads, N, 64]."""
    B, N, dm, d, dv, om, r = _proj_args(x, w_q, w_k, w_v, heads, kind, omega, nu)
    H = heads
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=torch.bfloat16,
                    scale=scale, eps=eps, n_seg=n_seg)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=torch.bfloat16, device=x.device)
    _dev_tensor("out", out, torch.bfloat16)
    for n, t in (("S_out", S_out), ("z_out", z_out)):
        if t is not None:
            _dev_tensor(n, t, torch.float32)
    ws, ws_bytes = _workspace(OP_BIDIR_PROJ, p, B, H, N, d, dv, 0, x.device, workspace)
    rc = _lib.lin_attn_bidir_proj(ctypes.byref(p), _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), B, H,
                                  N, dm, d, dv, _ptr(om), _ptr(out), _ptr(S_out), _ptr(z_out),
                                  _ptr(ws), ws_bytes, _stream(x.device, stream))
    _check("lin_attn_bidir_proj", rc)
    return out


def lin_attn_qkv_project(x, w_q, w_k, w_v, heads, *, q=None, k=None, v=None, stream=None):
    """q, k, v [B, heads, N, 64] (bf16, head-major) projected from tokens
    x [B, N, d_model] by w_* [heads * 64, d_model]."""
    _dev_tensor("x", x, torch.bfloat16)
    for n, t in (("w_q", w_q), ("w_k", w_k), ("w_v", w_v)):
        _dev_tensor(n, t, torch.bfloat16)
    B, N, dm = x.shape
    d = w_q.shape[0] // heads
    outs = []
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            t = torch.empty((B, heads, N, d), dtype=torch.bfloat16, device=x.device)
        outs.append(_dev_tensor(n, t, torch.bfloat16))
    rc = _lib.lin_attn_qkv_project(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), B, N, dm, heads, d,
                                   _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                   _stream(x.device, stream))
    _check("lin_attn_qkv_project", rc)
    return tuple(outs)


def _backward(name, op, q, k, v, dout, kind, omega, nu, sum_norm, norm, scale, eps, n_seg,
              workspace, stream):
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _dev_tensor(n, t, q.dtype)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    om = _omega(kind, omega, q.dtype)
    r = feature_width(kind, d, nu, om)
    p = make_params(kind, r, nu=nu, sum_norm=sum_norm, norm=norm, dtype=q.dtype, scale=scale,
                    eps=eps, n_seg=n_seg)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    ws, ws_bytes = _workspace(op, p, B, H, N, d, dv, 0, q.device, workspace)
    rc = getattr(_lib, name)(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d,
                             dv, _ptr(om), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(ws), ws_bytes,
                             _stream(q.device, stream))
    _check(name, rc)
    return dq, dk, dvv


def lin_attn_bidir_backward(q, k, v, dout, kind, *, omega=None, nu=1, sum_norm=False,
                            norm="attn", scale=1.0, eps=1e-6, n_seg=0, workspace=None,
                            stream=None):
    """Gradients (dq, dk, dv) of sum(lin_attn_bidir(q, k, v) * dout), each of
    the input dtype and shape."""
    return _backward("lin_attn_bidir_backward", OP_BIDIR_BACKWARD, q, k, v, dout, kind, omega, nu,
                     sum_norm, norm, scale, eps, n_seg, workspace, stream)


def lin_attn_causal_backward(q, k, v, dout, kind, *, omega=None, nu=1, sum_norm=False,
                             norm="attn", scale=1.0, eps=1e-6, n_seg=0, workspace=None,
                             stream=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for the causal recurrence from
    zero state (lin_attn_causal_chunked with state_in = 0)."""
    return _backward("lin_attn_causal_backward", OP_CAUSAL_BACKWARD, q, k, v, dout, kind, omega,
                     nu, sum_norm, norm, scale, eps, n_seg, workspace, stream)


def raw():
    """The ctypes handle of the library (for tests of the C ABI itself)."""
    return _lib
