"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a hand-worked
fixture, a brute-force computation by a different route, a closed form, an
invariant, or a special case that reduces to a textbook routine.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import ASYM, SYM, UNIT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = np.array([float(v) for v in vals])
    m, n = int(d["m"][0]), int(d["n"][0])
    return d, m, n


def _spd(k, rng, n_samples=None, damp=0.01):
    """Random SPD matrix from Gaussian samples plus damping (inputs only)."""
    n_samples = n_samples or 2 * k + 3
    X = rng.standard_normal((n_samples, k))
    G = X.T @ X / n_samples
    return G + damp * np.mean(np.diag(G)) * np.eye(k)


def _problem(m, n, seed, w_std=0.02, kind=SYM, bits=4, b_identity=False):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((m, n)) * w_std).astype(np.float32)
    A = _spd(n, rng)
    B = np.eye(m) if b_identity else _spd(m, rng)
    LA = oracle.factor(A)
    LB = oracle.factor(B)
    s, z = oracle.qparams(W, kind, bits)
    return W, A, B, LA, LB, s, z


# ---------------------------------------------------------------- fixtures

def test_golden_2x2_unit_grid():
    d, m, n = _read_fixture("naive_2x2_unit.txt")
    W = d["W"].reshape(m, n)
    LA = d["LA"].reshape(n, n)
    LB = d["LB"].reshape(m, m)
    s, z = np.ones(m), np.zeros(m)
    for fn in (lambda: oracle.naive(W, LA, LB, s, z, UNIT, 8),
               lambda: oracle.naive(W, LA, LB, s, z, UNIT, 8, order=1),
               lambda: oracle.antidiag(W, LA, LB, s, z, UNIT, 8),
               lambda: oracle.recursive(W, LA, LB, s, z, UNIT, 8)):
        r = fn()
        np.testing.assert_array_equal(r["codes"].ravel(), d["codes"])
        np.testing.assert_array_equal(r["V"].ravel(), d["V"])
        np.testing.assert_array_equal(r["E"].ravel(), d["E"])
        np.testing.assert_array_equal(r["U"].ravel(), d["U"])
    # the brute-force vectorised route on A (x) B with A = (LA LA^T)^-1, B = (LB LB^T)^-1
    A = np.linalg.inv(LA @ LA.T)
    B = np.linalg.inv(LB @ LB.T)
    rv = oracle.vec_gptq(W, A, B, s, z, UNIT, 8)
    np.testing.assert_array_equal(rv["codes"].ravel(), d["codes"])
    np.testing.assert_allclose(rv["V"].ravel(), d["V"], atol=1e-12)


def test_golden_1x3_sym4():
    d, m, n = _read_fixture("gptq_1x3_sym4.txt")
    W = d["W"].reshape(m, n).astype(np.float32)
    LA = d["LA"].reshape(n, n)
    LB = d["LB"].reshape(m, m)
    s, z = oracle.qparams(W, SYM, 4)
    np.testing.assert_array_equal(s, d["scales"].astype(np.float32))
    r = oracle.naive(W, LA, LB, s, z, SYM, 4)
    np.testing.assert_array_equal(r["codes"].ravel(), d["codes"])
    np.testing.assert_array_equal(r["V"].ravel(), d["V"])
    np.testing.assert_array_equal(r["E"].ravel(), d["E"])
    np.testing.assert_array_equal(r["U"].ravel(), d["U"])
    g = oracle.gptq_rows(W, LA, s, z, SYM, 4)
    np.testing.assert_array_equal(g["codes"].ravel(), d["codes"])
    np.testing.assert_array_equal(g["V"].ravel(), d["V"])


def test_golden_qparams():
    kinds = {"sym": SYM, "asym": ASYM}
    with open(os.path.join(GOLDEN, "qparams.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, vals, sbits, zero = [p.strip() for p in line.split("|")]
            kname, bits = head.split()
            W = np.array([[float(v) for v in vals.split()]], dtype=np.float32)
            s, z = oracle.qparams(W, kinds[kname], int(bits))
            assert s.view(np.uint32)[0] == int(sbits, 16), (line, hex(s.view(np.uint32)[0]))
            assert z[0] == float(zero)


# ---------------------------------------------- brute force on A (x) B

@pytest.mark.parametrize("m,n", [(1, 1), (1, 7), (9, 1), (2, 3), (5, 4), (8, 8),
                                 (16, 3), (3, 16), (12, 15), (16, 16)])
@pytest.mark.parametrize("kind,bits", [(SYM, 4), (ASYM, 2), (UNIT, 8)])
def test_naive_equals_vectorised_gptq(m, n, kind, bits):
    """Algorithm 2 (GPTQ on vec(W) with H = A (x) B, Cholesky of H^-1 taken
    directly) and the matrix-space naive solver give the same codes
    (Proposition 3.1 + Cholesky of a Kronecker product)."""
    w_std = 3.0 if kind == UNIT else 0.02
    W, A, B, LA, LB, s, z = _problem(m, n, 1000 * m + n + 7 * kind, w_std=w_std, kind=kind, bits=bits)
    rv = oracle.vec_gptq(W, A, B, s, z, kind, bits)
    r = oracle.naive(W, LA, LB, s, z, kind, bits, ref_codes=rv["codes"], window=1e-9)
    assert r["mismatches"] == 0
    assert r["ties"] == 0
    np.testing.assert_array_equal(r["codes"], rv["codes"])
    np.testing.assert_allclose(r["V"], rv["V"], rtol=0, atol=1e-12)


def test_brute_force_catches_transposed_factor():
    """Planted mistake: feeding LB^T instead of LB must change the result
    (the brute force distinguishes the two sides)."""
    W, A, B, LA, LB, s, z = _problem(10, 9, 5, w_std=3.0, kind=UNIT, bits=8)
    rv = oracle.vec_gptq(W, A, B, s, z, UNIT, 8)
    r = oracle.naive(W, LA, np.ascontiguousarray(LB.T), s, z, UNIT, 8)
    assert not np.array_equal(r["codes"], rv["codes"])


# ---------------------------------------------------- B = I is row GPTQ

@pytest.mark.parametrize("m,n,kind,bits", [(7, 33, SYM, 4), (16, 64, SYM, 3), (5, 40, ASYM, 2),
                                           (1, 100, SYM, 4), (24, 24, UNIT, 8)])
def test_b_identity_is_rowwise_gptq_bitwise(m, n, kind, bits):
    w_std = 3.0 if kind == UNIT else 0.02
    W, A, B, LA, LB, s, z = _problem(m, n, 31 * m + n, w_std=w_std, kind=kind, bits=bits,
                                     b_identity=True)
    assert np.array_equal(LB, np.eye(m))
    r = oracle.naive(W, LA, LB, s, z, kind, bits)
    g = oracle.gptq_rows(W, LA, s, z, kind, bits)
    assert np.array_equal(r["codes"], g["codes"])
    assert np.array_equal(r["V"], g["V"])
    assert np.array_equal(r["E"], g["E"])


@pytest.mark.parametrize("kind,bits", [(SYM, 4), (ASYM, 2)])
def test_b_identity_tie_adoption_matches_naive(kind, bits):
    """Row GPTQ with tie adoption settles ties as the naive solver does at
    B = I: with a wide window (many entries count as ties) and reference codes
    that pick the other neighbour at every second tie, plus one reference code
    that is no neighbour, both reach the same codes, values and counts."""
    m, n = 12, 40
    W, A, B, LA, LB, s, z = _problem(m, n, 907 + bits, kind=kind, bits=bits, b_identity=True)
    window = 0.2
    own = oracle.naive(W, LA, LB, s, z, kind, bits)
    u = own["U"]
    fl = np.floor(u)
    qmin, qmax = oracle.qrange(kind, bits)
    tie = (np.abs(u - fl - 0.5) < window) & (fl + z[:, None] >= qmin) & (fl + z[:, None] + 1 <= qmax)
    assert np.sum(tie) > 20
    ref = own["codes"].copy()
    idx = np.argwhere(tie)[::2]
    for i, j in idx:
        lo = int(fl[i, j] + z[i])
        ref[i, j] = lo if ref[i, j] == lo + 1 else lo + 1
    ref[3, 7] = qmax if own["codes"][3, 7] < qmax - 2 else qmin
    ref = ref.astype(np.int8)
    r = oracle.naive(W, LA, LB, s, z, kind, bits, ref_codes=ref, window=window)
    g = oracle.gptq_rows(W, LA, s, z, kind, bits, ref_codes=ref, window=window)
    assert r["ties"] > 10 and r["mismatches"] >= 1
    assert (g["ties"], g["mismatches"]) == (r["ties"], r["mismatches"])
    assert np.array_equal(g["codes"], r["codes"])
    assert np.array_equal(g["V"], r["V"]) and np.array_equal(g["E"], r["E"])
    assert not np.array_equal(r["codes"], own["codes"])


def test_a_identity_is_columnwise_gptq():
    """A = I: the problem is GPTQ down each column under B (the transposed
    problem), here on the unit grid so the per-row scale does not matter."""
    m, n = 20, 11
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((m, n)) * 3.0).astype(np.float32)
    LB = oracle.factor(_spd(m, rng))
    LA = np.eye(n)
    r = oracle.naive(W, LA, LB, np.ones(m), np.zeros(m), UNIT, 8)
    g = oracle.gptq_rows(W.T, LB, np.ones(n), np.zeros(n), UNIT, 8)
    np.testing.assert_array_equal(r["codes"], g["codes"].T)
    np.testing.assert_allclose(r["E"], g["E"].T, rtol=0, atol=1e-12)


def test_diagonal_factors_give_round_to_nearest():
    """Diagonal A and B: every update lands outside the entry's own row and
    column with a zero factor, so V = Q(W) (plain round-to-nearest)."""
    m, n = 13, 17
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32)
    LA = np.diag(rng.uniform(0.5, 2.0, n))
    LB = np.diag(rng.uniform(0.5, 2.0, m))
    s, z = oracle.qparams(W, SYM, 4)
    r = oracle.naive(W, LA, LB, s, z, SYM, 4)
    rtn = np.clip(np.rint(W.astype(np.float64) / s[:, None].astype(np.float64)), -8, 7)
    np.testing.assert_array_equal(r["codes"], rtn)


# -------------------------------------------- invariants and the bound

@pytest.mark.parametrize("m,n,kind,bits", [(23, 31, SYM, 4), (40, 17, SYM, 3), (30, 30, ASYM, 2),
                                           (1, 50, SYM, 4), (50, 1, SYM, 4)])
def test_completion_identity(m, n, kind, bits):
    """W - V = LB E LA^T after the run (the rank-1 updates sum to it)."""
    W, A, B, LA, LB, s, z = _problem(m, n, 77 + m * n, kind=kind, bits=bits)
    r = oracle.naive(W, LA, LB, s, z, kind, bits)
    R = oracle.completion_residual(W, r["V"], r["E"], LA, LB)
    scale = np.max(np.abs(W)) + np.max(np.abs(r["V"]))
    assert np.max(np.abs(R)) <= 1e-12 * scale


@pytest.mark.parametrize("seed", range(12))
def test_unit_grid_bound(seed):
    """||B^1/2 (V-W) A^1/2||_F^2 <= (1/4) sum 1/(LB_ii^2 LA_jj^2) <= tr(A) tr(B)/4
    on the unclamped unit grid (review page, "If this is right"); the loss also
    equals ||E||_F^2."""
    rng = np.random.default_rng(seed)
    m, n = int(rng.integers(1, 25)), int(rng.integers(1, 25))
    W = (rng.standard_normal((m, n)) * 3.0).astype(np.float32)
    A = _spd(n, rng, n_samples=n + 2, damp=0.05)
    B = _spd(m, rng, n_samples=m + 2, damp=0.05)
    LA, LB = oracle.factor(A), oracle.factor(B)
    r = oracle.naive(W, LA, LB, np.ones(m), np.zeros(m), UNIT, 8)
    assert np.max(np.abs(r["codes"])) < 100
    L = oracle.loss(A, B, W, r["V"])
    sharp = oracle.sharp_bound(LA, LB)
    tb = oracle.trace_bound(A, B)
    assert L <= sharp * (1 + 1e-12)
    assert sharp <= tb * (1 + 1e-12)
    np.testing.assert_allclose(L, np.sum(r["E"] ** 2), rtol=1e-9)


def test_loss_closed_form_identity_hessian():
    """A = I, B = I: the loss is ||V - W||_F^2."""
    rng = np.random.default_rng(5)
    W = rng.standard_normal((6, 9))
    V = np.rint(W)
    assert oracle.loss(np.eye(9), np.eye(6), W, V) == pytest.approx(np.sum((V - W) ** 2), rel=1e-15)


# ----------------------------------------------------- order independence

@pytest.mark.parametrize("m,n,kind,bits", [(9, 14, SYM, 4), (21, 6, ASYM, 2), (16, 16, SYM, 3),
                                           (31, 29, UNIT, 8)])
def test_variants_agree(m, n, kind, bits):
    """Theorem 3.2: naive (row or column raster), anti-diagonal and the
    recursive Algorithm-6 reading give the same codes."""
    w_std = 3.0 if kind == UNIT else 0.02
    W, A, B, LA, LB, s, z = _problem(m, n, 5 * m + 3 * n, w_std=w_std, kind=kind, bits=bits)
    base = oracle.naive(W, LA, LB, s, z, kind, bits)
    for other in (oracle.naive(W, LA, LB, s, z, kind, bits, order=1),
                  oracle.antidiag(W, LA, LB, s, z, kind, bits),
                  oracle.recursive(W, LA, LB, s, z, kind, bits)):
        np.testing.assert_array_equal(other["codes"], base["codes"])
        np.testing.assert_allclose(other["E"], base["E"], rtol=0, atol=1e-12 * np.max(np.abs(base["E"])))
        np.testing.assert_allclose(other["U"], base["U"], rtol=0, atol=1e-9)


# ------------------------------------------------------ tie adoption

def test_replay_adopts_a_boundary_tie_and_counts_mismatches():
    W = np.array([[0.2, 2.50005]], dtype=np.float32)
    LA, LB = np.eye(2), np.eye(1)
    s, z = np.ones(1), np.zeros(1)
    own = oracle.naive(W, LA, LB, s, z, UNIT, 8)
    assert own["codes"].tolist() == [[0, 3]]
    r = oracle.naive(W, LA, LB, s, z, UNIT, 8, ref_codes=np.array([[0, 2]]), window=1e-4)
    assert r["codes"].tolist() == [[0, 2]] and r["ties"] == 1 and r["mismatches"] == 0
    r = oracle.naive(W, LA, LB, s, z, UNIT, 8, ref_codes=np.array([[1, 3]]), window=1e-4)
    assert r["codes"].tolist() == [[0, 3]] and r["ties"] == 1 and r["mismatches"] == 1


# ----------------------------------------------- hessian, factor checkers

def test_hessian_closed_form():
    X = np.array([[3.0, 0.0], [0.0, 2.0], [0.0, 0.0], [0.0, 0.0]], dtype=np.float32)
    H = oracle.hessian(X, 0.5)
    # G = diag(9/4, 4/4); mean diag = 1.625; damping 0.8125
    np.testing.assert_allclose(H, np.diag([2.25 + 0.8125, 1.0 + 0.8125]), rtol=1e-15)
    e = oracle.hessian_entries(X, [0, 1, 0], [0, 1, 1], 0.5)
    np.testing.assert_allclose(e, [3.0625, 1.8125, 0.0], rtol=1e-15)


def test_factor_properties():
    rng = np.random.default_rng(9)
    H = _spd(37, rng)
    L = oracle.factor(H)
    assert np.allclose(L, np.tril(L))
    assert np.all(np.diag(L) > 0)
    np.testing.assert_allclose(L @ L.T @ H, np.eye(37), atol=1e-9)
    D = np.diag([4.0, 0.25, 9.0])
    np.testing.assert_allclose(oracle.factor(D), np.diag([0.5, 2.0, 1.0 / 3.0]), rtol=1e-15)


def test_checkers_detect_planted_mistakes():
    W, A, B, LA, LB, s, z = _problem(12, 10, 2024)
    r = oracle.naive(W, LA, LB, s, z, SYM, 4)
    assert oracle.rounding_consistency(r["codes"], r["V"], r["E"], np.diag(LA), np.diag(LB),
                                       s, z, SYM, 4)[0] == 0
    E2 = r["E"].copy()
    E2[3, 4] += 1e-3
    R = oracle.completion_residual(W, r["V"], E2, LA, LB)
    assert np.max(np.abs(R)) > 1e-6
    c2 = r["codes"].copy()
    c2[5, 5] += 1 if c2[5, 5] < 7 else -1
    assert oracle.rounding_consistency(c2, r["V"], r["E"], np.diag(LA), np.diag(LB),
                                       s, z, SYM, 4)[0] >= 1


# --------------------------------------------------------------------------
# per-row scale shrink by MSE search (review page, free parameters: shrink up
# to a factor 2, MSE search); pins independent of the search itself
# --------------------------------------------------------------------------
def test_mse_shrink_closed_form_sym():
    # one entry 1.0 and 63 entries 0.1, INT4 symmetric (qmax 7): on the grid of
    # p (scale p/7) every 0.1 rounds to code 1 and 1.0 clamps to code 7, so the
    # error is f(p) = 63 (p/7 - 0.1)^2 + (1 - p)^2, minimal at p = 0.8313; the
    # grid's best candidate is p = 0.83 (k = 17)
    W = np.array([[1.0] + [0.1] * 63], np.float32)
    s, z, kb, errs = oracle.qparams_mse(W, oracle.SYM, 4)
    assert kb[0] == 17 and z[0] == 0
    assert s[0] == np.float32(np.float32(0.83) / np.float32(7))
    for k in range(51):
        p = (100 - k) / 100
        f = 63 * (p / 7 - 0.1) ** 2 + (1 - p) ** 2
        assert abs(errs[0, k] - f) < 1e-6, k
    assert errs[0, 17] < errs[0, 16] - 1e-4 and errs[0, 17] < errs[0, 18] - 1e-4


def test_mse_shrink_closed_form_asym_boundary():
    # entries 0.0, 1.0 and 63 x 0.1, INT2 asymmetric (qmax 3, zero point 0):
    # for p > 0.6 the 0.1s round to code 0 (error 63 * 0.01 + (1 - p)^2), for
    # p < 0.6 to code 1 (error 63 (p/3 - 0.1)^2 + (1 - p)^2, decreasing down to
    # p = 0.3875): the search ends at its last candidate p = 1/2 with error 0.53
    W = np.array([[0.0, 1.0] + [0.1] * 63], np.float32)
    s, z, kb, errs = oracle.qparams_mse(W, oracle.ASYM, 2)
    assert kb[0] == 50 and z[0] == 0
    assert abs(errs[0, 50] - (63 * (0.5 / 3 - 0.1) ** 2 + 0.25)) < 1e-6
    for k in range(0, 40):       # p > 0.6
        p = (100 - k) / 100
        assert abs(errs[0, k] - (0.63 + (1 - p) ** 2)) < 1e-6, k


def test_mse_shrink_properties():
    g = np.random.default_rng(11)
    W = (g.standard_t(4, size=(40, 300)) * 0.02).astype(np.float32)
    W[3] = 0.0                                   # all candidates tie: keep p = 1
    for kind, bits in [(oracle.SYM, 4), (oracle.SYM, 3), (oracle.ASYM, 4), (oracle.ASYM, 2)]:
        s, z, kb, errs = oracle.qparams_mse(W, kind, bits)
        s0, z0 = oracle.qparams(W, kind, bits)
        # never worse than the plain grid, and the first minimum is taken
        assert np.all(errs[np.arange(40), kb] <= errs[:, 0])
        for i in range(40):
            assert kb[i] == int(np.argmin(errs[i]))
        # candidate 0 is the plain quantizer
        plain = kb == 0
        assert np.array_equal(s[plain], s0[plain]) and np.array_equal(z[plain], z0[plain])
        assert kb[3] == 0 and s[3] == 1.0
        # heavy tails make shrinking pay on most rows
        assert np.mean(kb > 0) > 0.5
        # exact under scaling by a power of two
        s2, z2, kb2, _ = oracle.qparams_mse(W * np.float32(8), kind, bits)
        nz = np.arange(40) != 3                  # the zero row keeps scale 1
        assert np.array_equal(kb2, kb) and np.array_equal(z2, z)
        assert np.array_equal(s2[nz], s[nz] * np.float32(8))
