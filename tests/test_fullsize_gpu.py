"""Full-size solves of the 4096 x 4096 (INT4 sym), 11008 x 4096 (INT3 sym) and
4096 x 14336 (INT2 asym) workloads through the C ABI, in the launch
configuration the benchmark times (cached graph replay, automatic product
order), with the factors made by the library's own hessian and factor calls.

These sizes are beyond the naive oracle, so the oracle's invariants decide.
Every schedule ends in the same state (the pages' Theorem 3.2), and
completion together with rounding consistency determines E uniquely
(induction over the product order), so the checks below, run on EVERY entry,
verify the whole output up to floating-point tolerance:
  definition   each entry's pre-rounding value recomputed in fp64 from the
               GPU's own errors by the order-free form
                 P~ = W - LB E LA^T + LB_ii LA_jj E_ij
               rounds to the GPU's code (boundary ties excepted), and differs
               from the value the GPU rounded, V + LB_ii LA_jj E_ij, by less
               than the tie window in code units (the drift);
  completion   |W - V - LB E LA^T| <= 1e-4 (|LB| |E| |LA|^T) entrywise (a bound
               derived from fp32 accumulation);
  rounding     every code is the base quantizer of V + LB_ii LA_jj E_ij;
  loss         tr((V-W)^T B (V-W) A), with A and B the oracle's fp64 Gram
               matrices of the same samples, equals sum e^2 within a tolerance
               derived from how far the pipeline's fp32 factors are from exact
               for those matrices (||L^T H L - I||_2) and from the completion
               residual, and within 1e-3 relative;
  factors      the library's factors at these sizes satisfy L^T H L = I to
               1e-3 in the 2-norm for the fp32 matrix H they were computed
               from (the library's fp32 Gram product, whose own rounding moves
               the ill-conditioned output-side factors further from the fp64
               Gram matrices: that part enters the loss tolerance);
  replay       a second call into the same buffers (a cached-graph replay)
               reproduces the first bitwise.
"""
import time

import numpy as np
import pytest

import oracle
from two_sided_gptq_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WINDOW = 1e-4
ROW_BLOCK = 1024


@pytest.fixture(scope="module")
def bk():
    from two_sided_gptq_amd import bakron
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    bakron.load()
    return bakron


def _spectral_norm(matvec, d):
    """Largest |eigenvalue| of a symmetric operator (Lanczos, scipy)."""
    from scipy.sparse.linalg import LinearOperator, eigsh
    op = LinearOperator((d, d), matvec=matvec, dtype=np.float64)
    vals = eigsh(op, k=1, which="LM", tol=1e-4, return_eigenvectors=False,
                 v0=np.ones(d) / np.sqrt(d))
    return float(abs(vals[0]))


def _factor_defect(L, H):
    """||L^T H L - I||_2 for the fp32 factor L of the fp64 matrix H."""
    L64 = L.astype(np.float64)
    return _spectral_norm(lambda x: L64.T @ (H @ (L64 @ x)) - x, H.shape[0])


@pytest.fixture(scope="module")
def solved(bk):
    """One full-size solve per workload (cached): host copies of the inputs and
    outputs, the GPU's factors, and the oracle's fp64 Gram matrices."""
    cache = {}

    def get(name):
        if name in cache:
            return cache[name]
        w = synth.WORKLOADS[name]
        print(f"[fullsize] {name} {w.m}x{w.n} kind={w.qkind} bits={w.qbits}", flush=True)
        t0 = time.time()
        W = synth.weights(w)
        Xh = synth.input_samples(w)
        Yh = synth.output_samples(w)
        HA = bk.hessian(torch.from_numpy(Xh).cuda(), synth.DAMP)
        HB = bk.hessian(torch.from_numpy(Yh).cuda(), synth.DAMP)
        LA, LB = bk.factor(HA), bk.factor(HB)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        Wd = torch.from_numpy(W).cuda()
        ws = torch.empty(bk.quantize_workspace_size(w.m, w.n, w.qkind, w.qbits), dtype=torch.uint8,
                         device="cuda")
        out = bk.quantize(Wd, LA, LB, kind=w.qkind, bits=w.qbits, want_E=True, want_sum=True,
                          dev_status=status, workspace=ws)
        torch.cuda.synchronize()
        first = {k: v.clone() for k, v in out.items() if v is not None}
        # the same buffers again: the cached graph is replayed
        bk.quantize(Wd, LA, LB, kind=w.qkind, bits=w.qbits, want_E=True, want_sum=True,
                    dev_status=status, workspace=ws, out=out)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        replay_equal = all(torch.equal(v, out[k]) for k, v in first.items())
        h = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
        h["zeros"] = h["zeros"] if "zeros" in h else np.zeros(w.m, np.float32)
        h.update(W=W, LA=LA.cpu().numpy(), LB=LB.cpu().numpy(), HA=HA.cpu().numpy(),
                 HB=HB.cpu().numpy(), replay_equal=replay_equal, w=w)
        del Wd, ws, out, first, LA, LB, HA, HB
        torch.cuda.empty_cache()
        print(f"[fullsize] {name}: GPU part {time.time() - t0:.1f} s", flush=True)
        t0 = time.time()
        h["A"] = oracle.hessian(Xh, synth.DAMP)
        del Xh
        h["B"] = oracle.hessian(Yh, synth.DAMP)
        del Yh
        print(f"[fullsize] {name}: oracle Gram matrices {time.time() - t0:.1f} s", flush=True)
        cache[name] = h
        return h

    return get


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_fullsize_every_entry(solved, name):
    h = solved(name)
    w = h["w"]
    W, V, E, codes = h["W"], h["V"], h["E"], h["codes"]
    s, z = h["scales"], h["zeros"]
    LAh, LBh = h["LA"], h["LB"]
    assert h["replay_equal"], "graph replay differs"
    qmin, qmax = oracle.qrange(w.qkind, w.qbits)
    assert codes.min() >= qmin and codes.max() <= qmax
    assert np.array_equal(z, np.round(z))
    # the scales are the oracle's (fp32 semantics, bitwise)
    so, zo = oracle.qparams(W, w.qkind, w.qbits)
    assert np.array_equal(s.view(np.uint32), np.asarray(so, np.float32).view(np.uint32))
    if w.qkind == synth.ASYM:
        assert np.array_equal(z, zo)
    # rounding consistency on the values the GPU rounded
    dA, dB = np.diag(LAh), np.diag(LBh)
    bad, ties = oracle.rounding_consistency(codes, V, E, dA, dB, s, z, w.qkind, w.qbits, WINDOW)
    print(f"[fullsize] {name}: rounding bad={bad} ties={ties}", flush=True)
    assert bad == 0

    # completion and the definition, every row, in fp64 row blocks
    t0 = time.time()
    LA64 = LAh.astype(np.float64)
    absLAt = np.abs(LA64).T.copy()
    LAt = LA64.T.copy()
    E64 = E.astype(np.float64)
    absE = np.abs(E64)
    m = w.m
    worst_ratio = drift = 0.0
    bad_def = ties_def = 0
    for r0 in range(0, m, ROW_BLOCK):
        r1 = min(m, r0 + ROW_BLOCK)
        LBb = LBh[r0:r1, :r1].astype(np.float64)  # LB is lower triangular
        prod = (LBb @ E64[:r1]) @ LAt
        bound = (np.abs(LBb) @ absE[:r1]) @ absLAt
        R = (W[r0:r1].astype(np.float64) - V[r0:r1]) - prod
        worst_ratio = max(worst_ratio, float(np.max(np.abs(R) / (bound + 1e-30))))
        # P~ - (V + d E) = R, so the drift in code units is |R| / s
        drift = max(drift, float(np.max(np.abs(R) / s[r0:r1, None])))
        b, t = oracle.rounding_consistency(codes[r0:r1], W[r0:r1].astype(np.float64) - prod,
                                           E[r0:r1], dA, dB[r0:r1], s[r0:r1], z[r0:r1],
                                           w.qkind, w.qbits, WINDOW)
        bad_def += b
        ties_def += t
    print(f"[fullsize] {name}: every row ({time.time() - t0:.1f} s): max |R|/bound {worst_ratio:.3e}, "
          f"drift {drift:.3e} code units, definition bad={bad_def} ties={ties_def}", flush=True)
    assert worst_ratio <= 1e-4
    assert drift < WINDOW
    assert bad_def == 0

    e2 = float(np.sum(E64 ** 2))
    assert abs(float(h["sum_e2"][0]) - e2) <= 1e-9 * e2


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_fullsize_loss_and_factors(solved, name):
    """Direct proxy loss against sum e^2, and the factors' defect."""
    h = solved(name)
    A, B, LAh, LBh = h["A"], h["B"], h["LA"], h["LB"]
    t0 = time.time()
    facA = _factor_defect(LAh, h["HA"].astype(np.float64))
    facB = _factor_defect(LBh, h["HB"].astype(np.float64))
    rhoA = _factor_defect(LAh, A)
    rhoB = _factor_defect(LBh, B)
    normA = _spectral_norm(lambda x: A @ x, A.shape[0])
    normB = _spectral_norm(lambda x: B @ x, B.shape[0])
    print(f"[fullsize] {name}: factor of its own input: ||LA^T HA LA - I|| {facA:.3e}, "
          f"||LB^T HB LB - I|| {facB:.3e}; against the fp64 Gram matrices: {rhoA:.3e}, {rhoB:.3e} "
          f"({time.time() - t0:.1f} s)", flush=True)
    # rounding the exact factor to fp32 alone leaves about 2^-24 sqrt(cond H)
    # (about 3e-5 for the 11008 x 11008 output side, cond ~ 3e5)
    assert facA < 1e-3 and facB < 1e-3

    t0 = time.time()
    W, V, E = h["W"], h["V"], h["E"]
    D = V.astype(np.float64) - W.astype(np.float64)
    loss = float(np.sum(D * ((B @ D) @ A)))
    e2 = float(np.sum(E.astype(np.float64) ** 2))
    # completion residual R = W - V - LB E LA^T in the A (x) B norm
    LA64 = LAh.astype(np.float64)
    Rn = 0.0
    for r0 in range(0, W.shape[0], ROW_BLOCK):
        r1 = min(W.shape[0], r0 + ROW_BLOCK)
        prod = (LBh[r0:r1, :r1].astype(np.float64) @ E[:r1].astype(np.float64)) @ LA64.T
        Rn += float(np.sum((-D[r0:r1] - prod) ** 2))
    r = np.sqrt(normA * normB * Rn)
    # |<E, GB E GA> - ||E||^2| <= ||E||^2 (rA + rB + rA rB), G = L^T H L, with a
    # factor 2 on the Lanczos estimates; then the residual by the triangle inequality
    tol = 2.0 * e2 * (rhoA + rhoB + rhoA * rhoB) + 2.0 * np.sqrt(e2) * r + r * r
    rel = abs(loss - e2) / e2
    print(f"[fullsize] {name}: loss {loss:.6e}, sum e^2 {e2:.6e}, rel diff {rel:.3e}, "
          f"tolerance {tol / e2:.3e} relative ({time.time() - t0:.1f} s)", flush=True)
    assert abs(loss - e2) <= tol
    assert rel <= 1e-3
