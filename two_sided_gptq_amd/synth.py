"""Seeded synthetic inputs for the two-sided rounding solver.

This module only draws random numbers (numpy PCG64) and arranges them into
the shapes of the workloads; it holds none of the solver's arithmetic (no
Gram matrix, no damping, no factorisation, no rounding).  Both the HIP path
and the fp64 oracle take their inputs from here.

Workloads (m outputs x n inputs).  The pages quantise layers of Llama-3 and
Qwen3 (pith.science review, Referee Report) at the 4096 x 4096 benchmark size
("If this is right") and time a 14336 x 4096 matrix (major comment 2); none of
those weights or calibration sets is available, so Gaussian / heavy-tailed
stand-ins of the same shapes are drawn here:

  c1  64 x 64      W ~ N(0, 0.02^2); X 512 x 64 and Y 256 x 64 i.i.d. N(0,1); INT4 sym
  c2a 1024 x 1024  W ~ N(0, 0.02^2); X 4096 x 1024 N(0,1) with 8 random input
                   channels scaled x20; Y 2048 x 1024 N(0,1); INT4 sym
  c2b as c2a with B = I (one-sided GPTQ)
  c3  4096 x 4096  W ~ N(0, 0.02^2); X 8192 x 4096 with 32 outlier channels x20;
                   Y = Z diag(k^-1/2) Q^T, Z 4096 x 4096 N(0,1), Q Haar-orthogonal
                   (output covariance eigenvalues decaying as 1/k); INT4 sym
  c4  11008 x 4096 W Student-t(5) scaled to std 0.02; X as c3; Y as c3 with
                   Z 16384 x 11008 and Q 11008 x 11008; INT3 sym
  c5  4096 x 14336 W ~ N(0, 0.02^2) rounded to bf16 and widened back to fp32;
                   X 16384 x 14336, column j scaled by exp(g_j), g_j ~ N(0,1)
                   (log-normal channel scales); Y 8192 x 4096 N(0,1); INT2 asym
All use damping 0.01 x mean diagonal.  Seeds: 20260000 + 100*config + role,
role 0 W, 1 X, 2 Y or Z, 3 outlier choice, 4 eigenbasis, 5 t / log-scale draws.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SYM, ASYM, UNIT = 0, 1, 2
DAMP = 0.01


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    m: int
    n: int
    qkind: int
    qbits: int
    n_x: int
    n_y: int            # 0 means B = I
    outliers: int = 0
    eig_decay: bool = False
    w_dist: str = "normal"   # normal | student_t | normal_bf16
    x_dist: str = "normal"   # normal | lognormal_cols

    @property
    def b_identity(self) -> bool:
        return self.n_y == 0


WORKLOADS = {
    "c1": Workload("c1", 1, 64, 64, SYM, 4, 512, 256),
    "c2a": Workload("c2a", 2, 1024, 1024, SYM, 4, 4096, 2048, outliers=8),
    "c2b": Workload("c2b", 2, 1024, 1024, SYM, 4, 4096, 0, outliers=8),
    "c3": Workload("c3", 3, 4096, 4096, SYM, 4, 8192, 4096, outliers=32, eig_decay=True),
    "c4": Workload("c4", 4, 11008, 4096, SYM, 3, 8192, 16384, outliers=32, eig_decay=True,
                   w_dist="student_t"),
    "c5": Workload("c5", 5, 4096, 14336, ASYM, 2, 16384, 8192, w_dist="normal_bf16",
                   x_dist="lognormal_cols"),
}


def seed(index: int, role: int) -> int:
    return 20260000 + 100 * index + role


def rng(index: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed(index, role)))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even) and widen back."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(np.float32)


def weights(w: Workload) -> np.ndarray:
    g = rng(w.index, 0)
    if w.w_dist == "student_t":
        nu = 5.0
        t = rng(w.index, 5).standard_t(nu, size=(w.m, w.n)).astype(np.float32)
        return (t * np.float32(0.02 / np.sqrt(nu / (nu - 2.0)))).astype(np.float32)
    W = g.standard_normal((w.m, w.n), dtype=np.float32) * np.float32(0.02)
    if w.w_dist == "normal_bf16":
        W = round_to_bf16(W)
    return W


def input_samples(w: Workload) -> np.ndarray:
    """Activation samples X (n_x x n) for the input-side factor A."""
    X = rng(w.index, 1).standard_normal((w.n_x, w.n), dtype=np.float32)
    if w.outliers:
        cols = rng(w.index, 3).choice(w.n, size=w.outliers, replace=False)
        X[:, cols] *= np.float32(20.0)
    if w.x_dist == "lognormal_cols":
        g = rng(w.index, 5).standard_normal(w.n).astype(np.float32)
        X *= np.exp(g)[None, :].astype(np.float32)
    return X


def haar_orthogonal(m: int, g: np.random.Generator) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian, signs fixed by
    the diagonal of R."""
    G = g.standard_normal((m, m), dtype=np.float32)
    Q, R = np.linalg.qr(G)
    return (Q * np.sign(np.diag(R))[None, :]).astype(np.float32)


def output_samples(w: Workload) -> np.ndarray | None:
    """Output-side samples Y (n_y x m) for the factor B, or None for B = I."""
    if w.b_identity:
        return None
    Z = rng(w.index, 2).standard_normal((w.n_y, w.m), dtype=np.float32)
    if not w.eig_decay:
        return Z
    k = np.arange(1, w.m + 1, dtype=np.float32)
    Q = haar_orthogonal(w.m, rng(w.index, 4))
    return ((Z * (k ** -0.5)[None, :]) @ Q.T).astype(np.float32)


def custom(m: int, n: int, seed_value: int, n_x: int | None = None, n_y: int | None = None,
           w_std: float = 0.02, outliers: int = 0):
    """Small Gaussian problem of any shape (for odd-shape and edge cases).
    Returns (W, X, Y); Y is None when n_y == 0."""
    g = np.random.Generator(np.random.PCG64(seed_value))
    n_x = n_x if n_x is not None else max(2 * n, 8)
    n_y = n_y if n_y is not None else max(2 * m, 8)
    W = g.standard_normal((m, n), dtype=np.float32) * np.float32(w_std)
    X = g.standard_normal((n_x, n), dtype=np.float32)
    if outliers:
        X[:, g.choice(n, size=outliers, replace=False)] *= np.float32(20.0)
    Y = g.standard_normal((n_y, m), dtype=np.float32) if n_y else None
    return W, X, Y
