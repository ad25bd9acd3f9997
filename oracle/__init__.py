"""fp64 CPU oracle for kernelized linear attention (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library under ``kernelized_linear_attention_amd`` and never imports it.

Every function takes numpy arrays (any float dtype; they are converted to
float64 once, on entry) and returns float64 arrays.  Feature-map kinds are
named by string: ``"identity"``, ``"elu1"``, ``"favor"``, ``"dpfp"``; readout
modes by ``"attn"`` (num / max(den, eps)) or ``"none"`` (num only).

Definitions followed (see the header of oracle.c for the passages):
  * feature maps: Kernel Zoo sec. 1.3 (identity), the running example
    (ELU+1), sec. 4.2 / 5.4 (FAVOR+), sec. 6.3 (DPFP), sec. 7.2 (sum norm);
  * bidirectional form: "Reassociate a feature-map kernel..." first paragraph,
    Performer page sec. 2 step 5;
  * causal recurrence and decode: Kernel Zoo sec. 1.2-1.3 and 5.4;
  * packed sequences: the causal recurrence per sequence, the state reset at
    each boundary ("Reassociate a feature-map kernel..." par. 4);
  * explicit N x N form: the interactive chapter's "rescan every key";
  * orthogonal random features: Performer page sec. 2 step 4, Kernel Zoo
    sec. 5.1-5.3 (Gram-Schmidt of Gaussian rows, chi or sqrt(d) lengths);
  * input projection: q, k, v = W_q x, W_k x, W_v x per token (Kernel Zoo
    sec. 1.2 step 1), a float64 matmul ahead of the calls above;
  * backward pass: the chain rule through the readout, the summaries and
    the feature map ("Reassociate a feature-map kernel..." par. 6 asks for
    gradient error to be evaluated).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LINATTN_ORACLE_LIB names another build of oracle.c (the sanitizer build of
# tests/sanitizers.py)
_LIB_PATH = os.environ.get("LINATTN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_KINDS = {"identity": 0, "elu1": 1, "favor": 2, "dpfp": 3}
_NORMS = {"attn": 0, "none": 1}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # compiling the checker is not using it
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    D = ctypes.c_double
    lib.orc_feature_dim.argtypes = [I, I, L, L]
    lib.orc_feature_dim.restype = I
    lib.orc_threads.argtypes = []
    lib.orc_threads.restype = I
    lib.orc_featuremap.argtypes = [I, I, I, I, D, D, P, L, L, L, P, P]
    lib.orc_featuremap.restype = I
    lib.orc_bidir.argtypes = [I, I, I, I, I, D, D, P, P, P, L, L, L, L, P, P, P, P]
    lib.orc_bidir.restype = I
    lib.orc_causal.argtypes = [I, I, I, I, I, D, D, P, P, P, L, L, L, L, P, I, P, P, P]
    lib.orc_causal.restype = I
    lib.orc_decode.argtypes = [I, I, I, I, I, D, D, P, P, P, L, L, L, P, P, P, P]
    lib.orc_decode.restype = I
    lib.orc_explicit.argtypes = [I, I, I, I, I, D, D, I, P, P, P, L, L, L, L, P, I, P, P, P]
    lib.orc_explicit.restype = I
    lib.orc_orf.argtypes = [P, P, L, L, P]
    lib.orc_orf.restype = I
    for name in ("orc_bidir_backward", "orc_causal_backward"):
        fn = getattr(lib, name)
        fn.argtypes = [I, I, I, I, I, D, D, P, P, P, P, L, L, L, L, P, P, P, P]
        fn.restype = I
    _lib = lib
    return lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS, else all cores)."""
    return int(_load().orc_threads())


def feature_dim(kind: str, d: int, nu: int = 1, omega=None) -> int:
    r_omega = 0 if omega is None else int(np.shape(omega)[0])
    return int(_load().orc_feature_dim(_KINDS[kind], nu, d, r_omega))


def _split(x):
    """[..., N, d] -> (lead shape, BH, N, d)."""
    x = _f64(x)
    lead = x.shape[:-2]
    N, d = x.shape[-2], x.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    return x, lead, BH, N, d


def _cfg(kind, d, nu, omega):
    r = feature_dim(kind, d, nu, omega)
    if r <= 0:
        raise ValueError(f"bad feature map configuration kind={kind} d={d} nu={nu}")
    return _KINDS[kind], r


def featuremap(x, kind, *, omega=None, nu=1, sum_norm=False, scale=1.0, eps=1e-6):
    """phi applied to every row of x [..., N, d] -> [..., N, r]."""
    x, lead, BH, N, d = _split(x)
    om = _f64(omega)
    k, r = _cfg(kind, d, nu, om)
    out = np.zeros(lead + (N, r), dtype=np.float64)
    rc = _load().orc_featuremap(k, r, nu, int(bool(sum_norm)), float(scale), float(eps),
                                _ptr(x), BH, N, d, _ptr(om), _ptr(out))
    if rc:
        raise ValueError("oracle featuremap: invalid argument")
    return out


def bidir(q, k, v, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
          scale=1.0, eps=1e-6):
    """Bidirectional reassociated attention.  Returns (out, S, z)."""
    q, lead, BH, N, d = _split(q)
    k = _f64(k)
    v = _f64(v)
    dv = v.shape[-1]
    om = _f64(omega)
    kk, r = _cfg(kind, d, nu, om)
    out = np.zeros(lead + (N, dv))
    S = np.zeros(lead + (r, dv))
    z = np.zeros(lead + (r,))
    rc = _load().orc_bidir(kk, r, nu, int(bool(sum_norm)), _NORMS[norm], float(scale), float(eps),
                           _ptr(q), _ptr(k), _ptr(v), BH, N, d, dv, _ptr(om),
                           _ptr(out), _ptr(S), _ptr(z))
    if rc:
        raise ValueError("oracle bidir: invalid argument")
    return out, S, z


def causal(q, k, v, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
           scale=1.0, eps=1e-6, S0=None, z0=None):
    """Causal recurrence from zero state, or from (S0, z0) when given.
    Returns (out, S_final, z_final)."""
    q, lead, BH, N, d = _split(q)
    k = _f64(k)
    v = _f64(v)
    dv = v.shape[-1]
    om = _f64(omega)
    kk, r = _cfg(kind, d, nu, om)
    state_in = S0 is not None
    if state_in != (z0 is not None):
        raise ValueError("give both S0 and z0, or neither")
    S = np.array(_f64(S0), copy=True) if state_in else np.zeros(lead + (r, dv))
    z = np.array(_f64(z0), copy=True) if state_in else np.zeros(lead + (r,))
    out = np.zeros(lead + (N, dv))
    rc = _load().orc_causal(kk, r, nu, int(bool(sum_norm)), _NORMS[norm], float(scale), float(eps),
                            _ptr(q), _ptr(k), _ptr(v), BH, N, d, dv, _ptr(om),
                            int(state_in), _ptr(S), _ptr(z), _ptr(out))
    if rc:
        raise ValueError("oracle causal: invalid argument")
    return out, S, z


def causal_varlen(q, k, v, cu_seqlens, kind, *, omega=None, nu=1, sum_norm=False,
                  norm="attn", scale=1.0, eps=1e-6, S0=None, z0=None):
    """Causal recurrence over sequences packed along the token axis: q, k
    [H, total, d], v [H, total, dv], cu_seqlens [num_seqs + 1].  Sequence i
    (tokens cu_seqlens[i] .. cu_seqlens[i+1] - 1 of every head) runs the
    recurrence of causal() from zero, or from (S0[i], z0[i]), and nothing
    carries from one sequence to the next (packing resets the state at the
    boundary, "Reassociate a feature-map kernel..." par. 4).
    Returns out [H, total, dv], S [num_seqs, H, r, dv], z [num_seqs, H, r]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(x) for x in cu_seqlens]
    n = len(cu) - 1
    H, total, d = q.shape
    dv = v.shape[-1]
    r = feature_dim(kind, d, nu, omega)
    if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to total")
    if (S0 is None) != (z0 is None):
        raise ValueError("give both S0 and z0, or neither")
    out = np.zeros((H, total, dv))
    S = np.zeros((n, H, r, dv))
    z = np.zeros((n, H, r))
    for i in range(n):
        a, b = cu[i], cu[i + 1]
        kw = {} if S0 is None else dict(S0=_f64(S0)[i], z0=_f64(z0)[i])
        o, S[i], z[i] = causal(q[:, a:b], k[:, a:b], v[:, a:b], kind, omega=omega, nu=nu,
                               sum_norm=sum_norm, norm=norm, scale=scale, eps=eps, **kw)
        out[:, a:b] = o
    return out, S, z


def decode(q, k, v, S, z, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
           scale=1.0, eps=1e-6):
    """One decode step for q, k, v [..., d]; returns (out [..., dv], S', z')."""
    q = _f64(q)
    lead = q.shape[:-1]
    d = q.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    k = _f64(k)
    v = _f64(v)
    dv = v.shape[-1]
    om = _f64(omega)
    kk, r = _cfg(kind, d, nu, om)
    S = np.array(_f64(S), copy=True)
    z = np.array(_f64(z), copy=True)
    out = np.zeros(lead + (dv,))
    rc = _load().orc_decode(kk, r, nu, int(bool(sum_norm)), _NORMS[norm], float(scale), float(eps),
                            _ptr(q), _ptr(k), _ptr(v), BH, d, dv, _ptr(om),
                            _ptr(S), _ptr(z), _ptr(out))
    if rc:
        raise ValueError("oracle decode: invalid argument")
    return out, S, z


def explicit(q, k, v, kind, *, causal_mask, omega=None, nu=1, sum_norm=False,
             norm="attn", scale=1.0, eps=1e-6, S0=None, z0=None):
    """Explicit N x N form (small N only).  Returns out."""
    q, lead, BH, N, d = _split(q)
    k = _f64(k)
    v = _f64(v)
    dv = v.shape[-1]
    om = _f64(omega)
    kk, r = _cfg(kind, d, nu, om)
    state_in = S0 is not None
    S0 = _f64(S0)
    z0 = _f64(z0)
    out = np.zeros(lead + (N, dv))
    rc = _load().orc_explicit(kk, r, nu, int(bool(sum_norm)), _NORMS[norm], float(scale),
                              float(eps), int(bool(causal_mask)), _ptr(q), _ptr(k), _ptr(v),
                              BH, N, d, dv, _ptr(om), int(state_in), _ptr(S0),
                              _ptr(z0), _ptr(out))
    if rc:
        raise ValueError("oracle explicit: invalid argument")
    return out


def orf(gauss, r, len_gauss=None):
    """Orthogonal random features [r, d] from the Gaussian draws gauss
    [ceil(r/d), d, d] (Gram-Schmidt on each block's rows, in order) and
    len_gauss [ceil(r/d)*d, d] (each row scaled to the norm of its row of
    len_gauss; sqrt(d) when None)."""
    g = _f64(gauss)
    d = g.shape[-1]
    lg = _f64(len_gauss)
    out = np.zeros((r, d))
    if _load().orc_orf(_ptr(g), _ptr(lg), r, d, _ptr(out)):
        raise ValueError("oracle orf: invalid argument")
    return out


def _backward(fname, q, k, v, dout, kind, omega, nu, sum_norm, norm, scale, eps):
    q, lead, BH, N, d = _split(q)
    k = _f64(k)
    v = _f64(v)
    dout = _f64(dout)
    dv = v.shape[-1]
    om = _f64(omega)
    kk, r = _cfg(kind, d, nu, om)
    dq = np.zeros(lead + (N, d))
    dk = np.zeros(lead + (N, d))
    dvv = np.zeros(lead + (N, dv))
    rc = getattr(_load(), fname)(kk, r, nu, int(bool(sum_norm)), _NORMS[norm], float(scale),
                                 float(eps), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), BH, N, d, dv,
                                 _ptr(om), _ptr(dq), _ptr(dk), _ptr(dvv))
    if rc:
        raise ValueError(f"oracle {fname}: invalid argument")
    return dq, dk, dvv


def bidir_backward(q, k, v, dout, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
                   scale=1.0, eps=1e-6):
    """Gradients (dq, dk, dv) of sum(out * dout) for the bidirectional form."""
    return _backward("orc_bidir_backward", q, k, v, dout, kind, omega, nu, sum_norm, norm,
                     scale, eps)


def causal_backward(q, k, v, dout, kind, *, omega=None, nu=1, sum_norm=False, norm="attn",
                    scale=1.0, eps=1e-6):
    """Gradients (dq, dk, dv) of sum(out * dout) for the causal recurrence
    from zero state."""
    return _backward("orc_causal_backward", q, k, v, dout, kind, omega, nu, sum_norm, norm,
                     scale, eps)


def project(x, w, heads):
    """Per-token projection W x (Kernel Zoo sec. 1.2 step 1) of x [B, N, dm]
    by w [heads * d, dm] (output row h*d + i is feature i of head h):
    returns [B, heads, N, d] in float64."""
    x = _f64(x)
    w = _f64(w)
    B, N, _ = x.shape
    d = w.shape[0] // heads
    y = np.matmul(x, w.T)                                  # [B, N, heads * d]
    return np.ascontiguousarray(y.reshape(B, N, heads, d).transpose(0, 2, 1, 3))


def causal_proj(x, w_q, w_k, w_v, heads, kind, **kw):
    """The causal recurrence on q, k, v projected from x."""
    return causal(project(x, w_q, heads), project(x, w_k, heads), project(x, w_v, heads), kind,
                  **kw)


def bidir_proj(x, w_q, w_k, w_v, heads, kind, **kw):
    """The bidirectional form on q, k, v projected from x."""
    return bidir(project(x, w_q, heads), project(x, w_k, heads), project(x, w_v, heads), kind,
                 **kw)
