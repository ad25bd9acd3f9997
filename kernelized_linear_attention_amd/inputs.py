"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws random numbers.
Both the HIP path and the fp64 oracle receive exactly the arrays produced
here (cast to the compute dtype by the caller), so neither side re-draws.

Seeding: every tensor comes from numpy's PCG64 seeded by
``SeedSequence([workload_id, tensor_id, rep])``; tensor ids are fixed below.

The random-feature matrix omega is the one random draw the method itself
makes.  It is drawn here and handed to both sides as an input:

* ``orf_omega`` -- orthogonal random features as the Performer page (sec. 2,
  step 4) describes them: rows of independent random orthogonal d x d blocks,
  each row rescaled to a Gaussian-distributed length, i.e. the length of an
  independent N(0, I_d) vector (chi distribution with d degrees of freedom).
  The Kernel Zoo (sec. 5.1, 5.3) builds the orthogonal directions by
  Gram-Schmidt; ``orthonormal_rows`` is that Gram-Schmidt, computed through a
  QR factorisation whose signs are fixed so that it returns the same vectors.
* ``iid_omega`` -- independent N(0, I_d) rows (Kernel Zoo sec. 4.2).
"""
from __future__ import annotations

import numpy as np

T_Q, T_K, T_V, T_OMEGA, T_PREFIX, T_LENGTHS, T_DOUT = 0, 1, 2, 3, 4, 5, 6
T_X, T_WQ, T_WK, T_WV = 7, 8, 9, 10


def rng(workload: int, tensor: int, rep: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, tensor, rep])))


def normal(shape, workload: int, tensor: int, rep: int = 0) -> np.ndarray:
    """i.i.d. N(0, 1) float32 array of the given shape."""
    return rng(workload, tensor, rep).standard_normal(size=tuple(shape), dtype=np.float32)


def orthonormal_rows(m: np.ndarray) -> np.ndarray:
    """Gram-Schmidt on the rows of m (rows in order), in float64.

    Uses the QR factorisation of m^T: Gram-Schmidt on the columns of m^T is
    Q with each column's sign chosen so that diag(R) > 0.
    """
    m = np.asarray(m, dtype=np.float64)
    q, r = np.linalg.qr(m.T)
    signs = np.sign(np.diag(r))
    signs[signs == 0] = 1.0
    return np.ascontiguousarray((q * signs).T)


def orf_draws(r: int, d: int, workload: int, rep: int = 0):
    """The Gaussian draws behind orf_omega, in the same order: per block of d
    rows, a d x d matrix for the directions, then a d x d matrix whose row
    norms are the lengths.  Returns (gauss [nblk, d, d], len_gauss
    [nblk * d, d]) as float32 -- the inputs of an on-device ORF build."""
    g = rng(workload, T_OMEGA, rep)
    nblk = (r + d - 1) // d
    gauss = np.empty((nblk, d, d), dtype=np.float64)
    lens = np.empty((nblk * d, d), dtype=np.float64)
    for b in range(nblk):
        gauss[b] = g.standard_normal((d, d))
        lens[b * d:(b + 1) * d] = g.standard_normal((d, d))
    return gauss.astype(np.float32), lens.astype(np.float32)


def orf_omega(r: int, d: int, workload: int, rep: int = 0) -> np.ndarray:
    """[r, d] float64: ceil(r/d) independent orthogonal blocks, rows scaled to
    chi(d)-distributed lengths; the last block is truncated when d does not
    divide r."""
    g = rng(workload, T_OMEGA, rep)
    blocks = []
    for _ in range((r + d - 1) // d):
        directions = orthonormal_rows(g.standard_normal((d, d)))
        lengths = np.linalg.norm(g.standard_normal((d, d)), axis=1)
        blocks.append(directions * lengths[:, None])
    return np.ascontiguousarray(np.concatenate(blocks, axis=0)[:r])


def iid_omega(r: int, d: int, workload: int, rep: int = 0) -> np.ndarray:
    """[r, d] float64 with i.i.d. N(0, 1) entries."""
    return rng(workload, T_OMEGA, rep).standard_normal((r, d))


def packed_lengths(num_seqs: int, total: int, workload: int, rep: int = 0,
                   lo: int = 256, hi: int = 8192) -> np.ndarray:
    """Lengths of num_seqs packed sequences that sum to total: log-uniform
    draws in [lo, hi] (a mix of short and long documents), scaled to the
    total and rounded, the rounding remainder added to the last one."""
    g = rng(workload, T_LENGTHS, rep)
    w = np.exp(g.uniform(np.log(lo), np.log(hi), size=num_seqs))
    lens = np.floor(w / w.sum() * total).astype(np.int64)
    lens[-1] += total - lens.sum()
    return lens


def projection_weights(heads: int, d: int, d_model: int, workload: int, rep: int = 0):
    """W_q, W_k, W_v [heads * d, d_model]: i.i.d. N(0, 1/d_model) float32, so
    that W x has unit-variance entries for x ~ N(0, I)."""
    std = np.float32(1.0 / np.sqrt(d_model))
    return tuple(normal((heads * d, d_model), workload, t, rep) * std
                 for t in (T_WQ, T_WK, T_WV))
