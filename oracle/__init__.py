"""Oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 CPU statement of two-sided (Kronecker-factored) GPTQ
rounding, written from the pages about arXiv 2608.06291 (BaKron, also
published as FastKron).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library (``two_sided_gptq_amd``) and imports nothing from it.

Sources (page, then section):
  * pith.science review of 2608.06291 -- "What carries the argument"
    (Proposition 3.1: the vectorised GPTQ step is an outer product
    L^B_i . delta . (L^A_j)^T in matrix space; lower triangularity confines it
    to the bottom-right; anti-diagonals are independent), "Core claim"
    (Theorem 3.2: naive, anti-diagonal, recursive and BaKron agree),
    "Circularity Check" (Algorithm 2 = GPTQ on vec(W) with Hessian A (x) B),
    "If this is right" (bound ||B^{1/2}(V-W)A^{1/2}||_F^2 <= tr(A) tr(B) / 4),
    "Load-bearing premise" (one-sided GPTQ is the case E[xx^T] (x) I),
    "Assumptions" (Cholesky of a Kronecker product is the Kronecker product
    of the Cholesky factors; loss ||vec(W)-vec(V)||_H^2 with H = A (x) B).
  * mlsanity.com index of 2608.06291 -- abstract (two-sided GPTQ/LDLQ,
    modular in the base quantizer and in the Hessian estimator).

Every function states the passage it follows.  Parity status of each one is
listed in ``PINS`` (all pinned by tests in ``tests/test_oracle.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SYM, ASYM, UNIT = 0, 1, 2

PINS = {
    "qparams": "hand-worked fixture tests/golden/qparams.txt",
    "naive": "brute force vs vec_gptq; B=I vs gptq_rows (bitwise); completion; "
             "unit-grid bound; RTN for diagonal factors; hand-worked 2x2 fixture",
    "antidiag": "equals naive (Theorem 3.2)",
    "recursive": "equals naive (Theorem 3.2)",
    "gptq_rows": "hand-worked 1x3 fixture; equals naive at B=I",
    "vec_gptq": "reduces to RTN for diagonal A, B; hand-worked 2x2 fixture",
    "hessian": "closed form for orthogonal columns",
    "factor": "L L^T H = I, lower, positive diagonal; closed form for diagonal H",
    "loss": "equals ||E||_F^2 (completion + L^T A L = I) and a closed form",
}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no FMA contraction) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
               _SRC, "-lm", "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        lib.orc_qparams.argtypes = [P, I64, I64, I, I, P, P]
        lib.orc_qparams.restype = I
        lib.orc_qparams_mse.argtypes = [P, I64, I64, I, I, I, I, P, P, P, P, P, P]
        lib.orc_qparams_mse.restype = I
        lib.orc_naive.argtypes = [I64, I64, P, P, P, P, P, I, I, I, I, P, D, P, P, P, P, P]
        lib.orc_naive.restype = I
        lib.orc_antidiag.argtypes = [I64, I64, P, P, P, P, P, I, I, I, P, P, P, P]
        lib.orc_antidiag.restype = I
        lib.orc_recursive.argtypes = [I64, I64, P, P, P, P, P, I, I, I, P, P, P, P]
        lib.orc_recursive.restype = I
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def qrange(kind: int, bits: int) -> tuple[int, int]:
    """Code range of the base quantizer.  Symmetric b-bit: [-2^(b-1), 2^(b-1)-1];
    asymmetric b-bit: [0, 2^b - 1]; unit grid: the int8 range."""
    if kind == SYM:
        return -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    if kind == ASYM:
        return 0, (1 << bits) - 1
    if kind == UNIT:
        return -128, 127
    raise ValueError(kind)


def qparams(W: np.ndarray, kind: int, bits: int):
    """Per-row scale (and integer zero point) from the original fp32 weights,
    in fp32 semantics.  Symmetric: s = max|W_i| / (2^(b-1) - 1); asymmetric:
    s = (max W_i - min W_i) / (2^b - 1), z = clamp(rint(-min W_i / s), 0, 2^b-1);
    s = 0 becomes 1.  (Review page, free parameters: a per-row scale.)"""
    W = np.ascontiguousarray(W, dtype=np.float32)
    m, n = W.shape
    s = np.empty(m, np.float32)
    z = np.empty(m, np.float32)
    rc = _load().orc_qparams(_p(W), m, n, kind, bits, _p(s), _p(z))
    if rc:
        raise ValueError(f"orc_qparams rc={rc}")
    return s, z


MSE_GRID, MSE_MAXK = 100, 50


def qparams_mse(W: np.ndarray, kind: int, bits: int, grid: int = MSE_GRID, maxk: int = MSE_MAXK,
                cands: bool = False):
    """Per-row parameters with the scale shrink chosen by an MSE search (review
    page, free parameters: shrink up to a factor 2, MSE search).  Candidates
    p_k = (grid - k) / grid, k = 0..maxk, applied to the row's range; the
    first candidate with the least sum of squared errors (w - v)^2 wins.
    Returns (scales, zeros, kbest, errs); with cands=True also (cand_s, cand_z):
    errs, cand_s, cand_z[i, k] are candidate k's error, scale and zero point."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    m, n = W.shape
    s = np.empty(m, np.float32)
    z = np.empty(m, np.float32)
    kb = np.empty(m, np.int32)
    errs = np.empty((m, maxk + 1), np.float64)
    cs = np.empty((m, maxk + 1), np.float32)
    cz = np.empty((m, maxk + 1), np.float32)
    rc = _load().orc_qparams_mse(_p(W), m, n, kind, bits, grid, maxk, _p(s), _p(z), _p(kb), _p(errs),
                                 _p(cs), _p(cz))
    if rc:
        raise ValueError(f"orc_qparams_mse rc={rc}")
    return (s, z, kb, errs, cs, cz) if cands else (s, z, kb, errs)


def _prep(W, LA, LB, scales, zeros):
    W = np.ascontiguousarray(W, dtype=np.float64)
    LA = np.ascontiguousarray(LA, dtype=np.float64)
    LB = np.ascontiguousarray(LB, dtype=np.float64)
    s = np.ascontiguousarray(scales, dtype=np.float64)
    z = np.ascontiguousarray(zeros, dtype=np.float64)
    m, n = W.shape
    assert LA.shape == (n, n) and LB.shape == (m, m) and s.shape == (m,) and z.shape == (m,)
    return W, LA, LB, s, z, m, n


def naive(W, LA, LB, scales, zeros, kind, bits, order=0, ref_codes=None, window=1e-4):
    """BaKron-naive (raster order, full rank-1 updates; Proposition 3.1).

    Returns dict(codes, V, E, U, ties, mismatches) where U = P / s is the
    pre-rounding value in code units.  With ``ref_codes`` the oracle adopts the
    reference code at boundary ties (see oracle.c)."""
    W, LA, LB, s, z, m, n = _prep(W, LA, LB, scales, zeros)
    qmin, qmax = qrange(kind, bits)
    codes = np.zeros((m, n), np.int32)
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    U = np.zeros((m, n))
    counts = np.zeros(2, np.int64)
    ref = None
    if ref_codes is not None:
        ref = np.ascontiguousarray(ref_codes, dtype=np.int8)
        assert ref.shape == (m, n)
    rc = _load().orc_naive(m, n, _p(W), _p(LA), _p(LB), _p(s), _p(z), kind, qmin, qmax,
                           order, _p(ref) if ref is not None else None, window,
                           _p(codes), _p(V), _p(E), _p(U), _p(counts))
    if rc:
        raise MemoryError("orc_naive")
    return dict(codes=codes, V=V, E=E, U=U, ties=int(counts[0]), mismatches=int(counts[1]))


def antidiag(W, LA, LB, scales, zeros, kind, bits):
    """BaKron-antidiagonal: whole anti-diagonal rounded, then its updates."""
    W, LA, LB, s, z, m, n = _prep(W, LA, LB, scales, zeros)
    qmin, qmax = qrange(kind, bits)
    codes = np.zeros((m, n), np.int32)
    V, E, U = np.zeros((m, n)), np.zeros((m, n)), np.zeros((m, n))
    _load().orc_antidiag(m, n, _p(W), _p(LA), _p(LB), _p(s), _p(z), kind, qmin, qmax,
                         _p(codes), _p(V), _p(E), _p(U))
    return dict(codes=codes, V=V, E=E, U=U)


def recursive(W, LA, LB, scales, zeros, kind, bits):
    """BaKron (Algorithm 6, plain reading) at single-diagonal granularity."""
    W, LA, LB, s, z, m, n = _prep(W, LA, LB, scales, zeros)
    qmin, qmax = qrange(kind, bits)
    codes = np.zeros((m, n), np.int32)
    V, E, U = np.zeros((m, n)), np.zeros((m, n)), np.zeros((m, n))
    _load().orc_recursive(m, n, _p(W), _p(LA), _p(LB), _p(s), _p(z), kind, qmin, qmax,
                          _p(codes), _p(V), _p(E), _p(U))
    return dict(codes=codes, V=V, E=E, U=U)


def _round_np(P, s, z, qmin, qmax):
    """Base quantizer on numpy vectors: c = clamp(rint(P/s) + z), v = s (c - z)."""
    c = np.clip(np.rint(P / s) + z, qmin, qmax)
    return c, s * (c - z)


def gptq_rows(W, LA, scales, zeros, kind, bits, ref_codes=None, window=1e-4):
    """Ordinary one-sided GPTQ (every row independent), Hessian A on the input
    side: for each column j, round, err = (w_j - q_j) / LA[j,j], and feed the
    error forward along the row through column j of LA.  (Load-bearing premise:
    GPTQ is the case E[xx^T] (x) I, i.e. B = I.)

    With ``ref_codes`` the boundary ties are settled as in ``naive``: an entry
    whose pre-rounding value u = P / s lies within ``window`` code units of an
    interior rounding boundary takes the reference code if that is one of the
    two adjacent codes (counted in ``ties``); a tie whose reference is neither
    neighbour, and any other disagreement, is counted in ``mismatches`` and the
    oracle keeps its own code."""
    Wk = np.array(W, dtype=np.float64)
    LA = np.asarray(LA, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    z = np.asarray(zeros, dtype=np.float64)
    qmin, qmax = qrange(kind, bits)
    m, n = Wk.shape
    ref = None if ref_codes is None else np.asarray(ref_codes).astype(np.int64)
    codes = np.zeros((m, n), np.int32)
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    ties = mismatches = 0
    for j in range(n):
        P = Wk[:, j].copy()
        c, v = _round_np(P, s, z, qmin, qmax)
        if ref is not None:
            u = P / s
            fl = np.floor(u)
            lower = fl + z
            tie = ((lower >= qmin) & (lower + 1 <= qmax) & (np.abs((u - fl) - 0.5) < window))
            r = ref[:, j]
            adopt = tie & ((r == lower) | (r == lower + 1))
            ties += int(np.sum(adopt))
            mismatches += int(np.sum(tie & ~adopt)) + int(np.sum(~tie & (r != c)))
            c = np.where(adopt, r, c)
            v = s * (c - z)
        err = (P - v) / LA[j, j]
        codes[:, j] = c
        V[:, j] = v
        E[:, j] = err
        Wk[:, j:] -= np.outer(err, LA[j:, j])
    return dict(codes=codes, V=V, E=E, ties=ties, mismatches=mismatches)


def vec_gptq(W, A, B, scales, zeros, kind, bits):
    """Algorithm 2 by brute force: GPTQ on vec(W) (column-major, q = i + m j)
    with Hessian H = A (x) B, using the Cholesky factor of H^{-1} formed
    directly (no Kronecker structure used).  Review page, Circularity Check."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    H = np.kron(np.asarray(A, np.float64), np.asarray(B, np.float64))
    Lc = np.linalg.cholesky(np.linalg.inv(H))
    w = W.reshape(-1, order="F").copy()
    s = np.asarray(scales, np.float64)
    z = np.asarray(zeros, np.float64)
    qmin, qmax = qrange(kind, bits)
    codes = np.zeros(m * n, np.int32)
    V = np.zeros(m * n)
    for q in range(m * n):
        i = q % m
        c, v = _round_np(np.array([w[q]]), s[i], z[i], qmin, qmax)
        err = (w[q] - v[0]) / Lc[q, q]
        codes[q] = int(c[0])
        V[q] = v[0]
        w[q:] -= err * Lc[q:, q]
    return dict(codes=codes.reshape((m, n), order="F"), V=V.reshape((m, n), order="F"))


def hessian(X, damp_rel):
    """Input- or output-side factor from samples: G = X^T X / N, then
    H = G + damp_rel * mean(diag G) * I (Gram regularisation by a multiple of the
    mean diagonal; review page, free parameters).  fp64."""
    X = np.asarray(X, dtype=np.float64)
    N = X.shape[0]
    G = X.T @ X / N
    return G + damp_rel * np.mean(np.diag(G)) * np.eye(G.shape[0])


def hessian_entries(X, rows, cols, damp_rel):
    """Selected entries of ``hessian(X, damp_rel)``, each computed on its own
    (for sizes where the full product is too slow on the host)."""
    X = np.asarray(X)
    N = X.shape[0]
    diag_mean = np.mean(np.einsum("ij,ij->j", X, X, dtype=np.float64)) / N
    out = np.empty(len(rows))
    for t, (a, b) in enumerate(zip(rows, cols)):
        g = float(np.dot(X[:, a].astype(np.float64), X[:, b].astype(np.float64))) / N
        out[t] = g + (damp_rel * diag_mean if a == b else 0.0)
    return out


def factor(H):
    """Lower Cholesky factor of H^{-1}: L L^T = H^{-1} (review page, "What
    carries the argument": L^A, L^B are the lower-triangular Cholesky factors of
    A^{-1}, B^{-1}).  The definition, written out in fp64."""
    return np.linalg.cholesky(np.linalg.inv(np.asarray(H, dtype=np.float64)))


def loss(A, B, W, V):
    """Proxy loss ||B^{1/2}(V-W)A^{1/2}||_F^2 = tr((V-W)^T B (V-W) A) in fp64
    (review page, "If this is right"; equals ||vec(W)-vec(V)||^2_{A (x) B} with
    column-major vec, Assumptions)."""
    D = np.asarray(V, np.float64) - np.asarray(W, np.float64)
    return float(np.sum(D * (np.asarray(B, np.float64) @ D @ np.asarray(A, np.float64))))


def sharp_bound(LA, LB):
    """(1/4) sum_ij 1/(LB_ii^2 LA_jj^2): the unit-grid error bound before the
    final step 1/LA_jj^2 <= A_jj (which gives the pages' tr(A) tr(B) / 4)."""
    a = np.diag(np.asarray(LA, np.float64)) ** -2
    b = np.diag(np.asarray(LB, np.float64)) ** -2
    return 0.25 * float(np.sum(b) * np.sum(a))


def trace_bound(A, B):
    """The pages' bound tr(A) tr(B) / 4 (review page, "If this is right")."""
    return 0.25 * float(np.trace(A)) * float(np.trace(B))


def completion_residual(W, V, E, LA, LB, rows=None):
    """R = (W - V) - LB E LA^T on the given rows (all rows if None), fp64.
    The rounding run ends with W - V = LB E LA^T (every entry's update sums to
    that product), so R is zero up to rounding."""
    W = np.asarray(W, np.float64)
    V = np.asarray(V, np.float64)
    E = np.asarray(E, np.float64)
    LA = np.asarray(LA, np.float64)
    LB = np.asarray(LB, np.float64)
    if rows is None:
        rows = np.arange(W.shape[0])
    rows = np.asarray(rows)
    prod = (LB[rows, :] @ E) @ LA.T
    return (W[rows] - V[rows]) - prod


def rounding_consistency(codes, V, E, LA_diag, LB_diag, scales, zeros, kind, bits, window=1e-4):
    """Re-derive each entry's pre-rounding value P = V + LB_ii LA_jj E_ij (from
    e = (P - v) / (LB_ii LA_jj)) and check that the base quantizer maps it to the
    stored code; entries within
    ``window`` code units of an interior boundary may take either neighbour.
    Returns (n_bad, n_ties)."""
    V = np.asarray(V, np.float64)
    E = np.asarray(E, np.float64)
    s = np.asarray(scales, np.float64)[:, None]
    z = np.asarray(zeros, np.float64)[:, None]
    d = np.asarray(LB_diag, np.float64)[:, None] * np.asarray(LA_diag, np.float64)[None, :]
    P = V + d * E
    qmin, qmax = qrange(kind, bits)
    u = P / s
    c, _ = _round_np(P, s, z, qmin, qmax)
    fl = np.floor(u)
    lower = fl + z
    tie = (np.abs((u - fl) - 0.5) < window) & (lower >= qmin) & (lower + 1 <= qmax)
    codes = np.asarray(codes)
    ok = (codes == c) | (tie & ((codes == lower) | (codes == lower + 1)))
    return int(np.sum(~ok)), int(np.sum(tie))
