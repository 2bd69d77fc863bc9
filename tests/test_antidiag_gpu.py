"""BaKron-antidiagonal on the GPU (bakron_quantize_antidiag): the same output as
the raster-order naive solver up to fp32 rounding order (pith.science review of
arXiv 2608.06291, "Core claim", Theorem 3.2), checked against the oracle with
tie adoption, and the same codes as the BaKron solver except at ties."""
import numpy as np
import pytest

import oracle
from two_sided_gptq_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WINDOW = 1e-4
LOSS_RTOL = 1e-3


@pytest.fixture(scope="module")
def bk():
    from two_sided_gptq_amd import bakron
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    bakron.load()
    return bakron


def _factors(X, Y, m):
    A = oracle.hessian(X, synth.DAMP)
    B = oracle.hessian(Y, synth.DAMP)
    return A, B, oracle.factor(A).astype(np.float32), oracle.factor(B).astype(np.float32)


@pytest.mark.parametrize("m,n,kind,bits", [(130, 150, synth.SYM, 4), (192, 256, synth.ASYM, 3),
                                           (64, 200, synth.SYM, 2), (150, 70, synth.UNIT, 8)])
def test_antidiag_parity(bk, m, n, kind, bits):
    print(f"[antidiag] {m}x{n} kind {kind} bits {bits}", flush=True)
    w_std = 3.0 if kind == synth.UNIT else 0.02
    W, X, Y = synth.custom(m, n, 8100 + m + n + kind, w_std=w_std, outliers=3)
    A, B, LA, LB = _factors(X, Y, m)
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    Wd, LAd, LBd = (torch.from_numpy(a).to(dev) for a in (W, LA, LB))
    out = bk.quantize_antidiag(Wd, LAd, LBd, kind=kind, bits=bits, want_E=True, dev_status=status)
    ref = bk.quantize(Wd, LAd, LBd, kind=kind, bits=bits, want_E=True)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    res = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
    s, z = oracle.qparams(W, kind, bits)
    assert np.array_equal(res["scales"].view(np.uint32), s.view(np.uint32))
    r = oracle.naive(W, LA, LB, s, z, kind, bits, ref_codes=res["codes"], window=WINDOW)
    assert r["mismatches"] == 0, f"{r['mismatches']} mismatches, {r['ties']} ties"
    assert np.array_equal(r["codes"], res["codes"].astype(np.int32))
    np.testing.assert_allclose(res["V"], r["V"], rtol=2 ** -23, atol=0)
    lg, lo = oracle.loss(A, B, W, res["V"]), oracle.loss(A, B, W, r["V"])
    assert abs(lg - lo) <= LOSS_RTOL * abs(lo) + 1e-12 * oracle.loss(A, B, W, np.zeros_like(W))
    # the BaKron solver's codes agree except at ties (both pass the same oracle)
    c2 = ref["codes"].cpu().numpy()
    r2 = oracle.naive(W, LA, LB, s, z, kind, bits, ref_codes=c2, window=WINDOW)
    assert r2["mismatches"] == 0
    assert np.count_nonzero(c2 != res["codes"]) <= r["ties"] + r2["ties"]
