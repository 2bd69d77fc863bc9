"""The hybrid schedule (BAKRON_FLAG_SPLIT_COLS / _ROWS): one row or column split
at the top level (BaKron-recursive's split, pith.science review of arXiv
2608.06291, "Circularity Check": the recurrence of Appendix C), the recursion
over anti-diagonals inside each part.  All four variants give the same result
(Theorem 3.2, "Core claim"), so the split solve is held to the same oracle
parity as the plain one: the naive fp64 solver, codes equal except at adopted
ties.
"""
import numpy as np
import pytest

import oracle
from two_sided_gptq_amd import synth

from test_quantize_gpu import _check_parity, _factors, _mse_params

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bk():
    from two_sided_gptq_amd import bakron
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    bakron.load()
    return bakron


def _gpu_split(bk, W, LA, LB, kind, bits, order, split, graph=True, mse=False):
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = bk.quantize(torch.from_numpy(W).to(dev), torch.from_numpy(LA).to(dev),
                      torch.from_numpy(LB).to(dev), kind=kind, bits=bits, order=order,
                      want_V=True, want_E=True, want_sum=True, dev_status=status, split=split,
                      graph=graph, mse=mse)
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    res["status"] = int(status.item())
    return res


@pytest.mark.parametrize("m,n", [(300, 260), (257, 200), (64, 128), (130, 70), (200, 333)])
@pytest.mark.parametrize("split", ["cols", "rows"])
def test_split_parity_shapes(bk, m, n, split):
    print(f"[split] {m}x{n} {split}", flush=True)
    W, X, Y = synth.custom(m, n, 9000 + 3 * m + n)
    A, B, LA, LB = _factors(X, Y, m)
    for order in (1, 2):
        res = _gpu_split(bk, W, LA, LB, synth.SYM, 4, order, split)
        _check_parity(W, A, B, LA, LB, synth.SYM, 4, res, f"{m}x{n} {split} order {order}")


@pytest.mark.parametrize("kind,bits", [(synth.ASYM, 2), (synth.SYM, 3)])
def test_split_parity_quantizers(bk, kind, bits):
    m, n = 190, 230
    W, X, Y = synth.custom(m, n, 9500 + 10 * kind + bits, outliers=4)
    A, B, LA, LB = _factors(X, Y, m)
    for split in ("cols", "rows"):
        res = _gpu_split(bk, W, LA, LB, kind, bits, 0, split)
        _check_parity(W, A, B, LA, LB, kind, bits, res, f"kind {kind} bits {bits} {split}")


def test_split_with_mse_scale_search(bk):
    # the scale search runs once on the whole W, before the parts; the split
    # solve then matches the naive oracle on those parameters
    m, n = 200, 300
    W, X, Y = synth.custom(m, n, 9700, outliers=6)
    A, B, LA, LB = _factors(X, Y, m)
    for split in ("cols", "rows"):
        print(f"[split] mse {split}", flush=True)
        res = _gpu_split(bk, W, LA, LB, synth.ASYM, 4, 0, split, mse=True)
        zeros = res["zeros"] if res["zeros"] is not None else np.zeros(m, np.float32)
        s, z, kb, ndiff = _mse_params(W, synth.ASYM, 4, res["scales"], zeros)
        assert ndiff <= 2
        _check_parity(W, A, B, LA, LB, synth.ASYM, 4, res, f"mse {split}", sz=(s, z))


@pytest.mark.parametrize("split", ["cols", "rows"])
def test_split_parity_workload(bk, split):
    # the 1024 x 1024 workload with B from output samples
    print(f"[split] c2a {split}", flush=True)
    w = synth.WORKLOADS["c2a"]
    W = synth.weights(w)
    A, B, LA, LB = _factors(synth.input_samples(w), synth.output_samples(w), w.m)
    res = _gpu_split(bk, W, LA, LB, w.qkind, w.qbits, 0, split)
    info = _check_parity(W, A, B, LA, LB, w.qkind, w.qbits, res, f"c2a {split}")
    print(split, info)


def test_split_graph_matches_eager(bk):
    # parts wide enough to defer work to the side stream: graph replay and the
    # eager two-stream launch agree bit for bit, for both splits
    m, n = 2048, 1024
    assert bk.schedule_info(m, n // 2, 0)["side_launches"] > 0
    W, X, Y = synth.custom(m, n, 9900)
    A, B, LA, LB = _factors(X, Y, m)
    for split in ("cols", "rows"):
        print(f"[split] modes {split}", flush=True)
        a = _gpu_split(bk, W, LA, LB, synth.SYM, 4, 0, split, graph=True)
        b = _gpu_split(bk, W, LA, LB, synth.SYM, 4, 0, split, graph=False)
        c = _gpu_split(bk, W, LA, LB, synth.SYM, 4, 0, split, graph=True)
        for k in ("codes", "scales", "V", "E", "sum_e2"):
            assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), (split, k)
        assert a["status"] == 0


@pytest.mark.parametrize("split", ["cols", "rows"])
def test_split_full_size_invariants(bk, split):
    # 4096 x 4096: every entry rounds its own pre-rounding value (up to the tie
    # window) and W - V = LB E LA^T on sampled rows, as for the plain schedule
    print(f"[split] c3 {split}", flush=True)
    w = synth.WORKLOADS["c3"]
    W = synth.weights(w)
    LAd = bk.factor(bk.hessian(torch.from_numpy(synth.input_samples(w)).cuda(), synth.DAMP))
    LBd = bk.factor(bk.hessian(torch.from_numpy(synth.output_samples(w)).cuda(), synth.DAMP))
    LA, LB = LAd.cpu().numpy(), LBd.cpu().numpy()
    res = _gpu_split(bk, W, LA, LB, w.qkind, w.qbits, 0, split)
    assert res["status"] == 0
    s = res["scales"]
    bad, _ = oracle.rounding_consistency(res["codes"], res["V"], res["E"], np.diag(LA), np.diag(LB),
                                         s, np.zeros_like(s), w.qkind, w.qbits)
    assert bad == 0
    rows = np.array([0, 63, 64, 2047, 2048, 3000, 4095])
    R = oracle.completion_residual(W, res["V"], res["E"], LA, LB, rows=rows)
    bound = (np.abs(LB[rows, :].astype(np.float64)) @ np.abs(res["E"].astype(np.float64))) @ \
        np.abs(LA.astype(np.float64)).T
    assert np.max(np.abs(R) / (bound + 1e-30)) <= 1e-4
    assert abs(float(res["sum_e2"][0]) - float(np.sum(res["E"].astype(np.float64) ** 2))) <= \
        1e-9 * float(res["sum_e2"][0])
