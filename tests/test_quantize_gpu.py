"""Parity of the HIP solver (through the C ABI) with the fp64 oracle.

Protocol: the oracle replays BaKron-naive on the same fp32 inputs the GPU
consumed; where the oracle's pre-rounding value lies within 1e-4 code units
of an interior rounding boundary it adopts the GPU's code if that is one of
the two adjacent codes (such entries are counted as ties).  Everything else
must match exactly: zero mismatches, identical codes, scales bit for bit.
The proxy loss ||B^1/2 (V-W) A^1/2||_F^2 must agree within 1e-3 relative, and
the drift of the pre-rounding values must stay below the tie window.
LA and LB come from the oracle's fp64 factorisation, rounded to fp32, so no
input of the oracle is produced by the HIP path.
"""
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


def _factors(X, Y, m, damp=synth.DAMP):
    A = oracle.hessian(X, damp)
    B = np.eye(m) if Y is None else oracle.hessian(Y, damp)
    LA = oracle.factor(A).astype(np.float32)
    LB = np.eye(m, dtype=np.float32) if Y is None else oracle.factor(B).astype(np.float32)
    return A, B, LA, LB


def _gpu(bk, W, LA, LB, kind, bits, order=0, mse=False):
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = bk.quantize(torch.from_numpy(W).to(dev), torch.from_numpy(LA).to(dev),
                      torch.from_numpy(LB).to(dev), kind=kind, bits=bits, order=order,
                      want_V=True, want_E=True, want_sum=True, dev_status=status, mse=mse)
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    res["status"] = int(status.item())
    return res


def _check_parity(W, A, B, LA, LB, kind, bits, res, label="", sz=None):
    m, n = W.shape
    s, z = oracle.qparams(W, kind, bits) if sz is None else sz
    assert np.array_equal(res["scales"].view(np.uint32), s.view(np.uint32)), label
    zeros = res["zeros"] if res["zeros"] is not None else np.zeros(m, np.float32)
    assert np.array_equal(zeros, z), label
    assert res["status"] == 0, label
    r = oracle.naive(W, LA, LB, s, z, kind, bits, ref_codes=res["codes"], window=WINDOW)
    assert r["mismatches"] == 0, f"{label}: {r['mismatches']} mismatches, {r['ties']} ties"
    assert np.array_equal(r["codes"], res["codes"].astype(np.int32)), label
    # dequantised values: v = s (c - z) in fp32
    np.testing.assert_allclose(res["V"], r["V"], rtol=2 ** -23, atol=0, err_msg=label)
    # drift of the pre-rounding value in code units
    d = LB.astype(np.float64).diagonal()[:, None] * LA.astype(np.float64).diagonal()[None, :]
    u_gpu = (res["V"].astype(np.float64) + d * res["E"].astype(np.float64)) / s[:, None]
    drift = float(np.max(np.abs(u_gpu - r["U"])))
    assert drift < WINDOW, f"{label}: drift {drift}"
    lg = oracle.loss(A, B, W, res["V"])
    lo = oracle.loss(A, B, W, r["V"])
    # relative bar, with an absolute floor at fp64 noise of the loss of V = 0
    floor = 1e-12 * oracle.loss(A, B, W, np.zeros_like(W))
    assert abs(lg - lo) <= LOSS_RTOL * abs(lo) + floor, f"{label}: loss {lg} vs {lo}"
    e2 = float(np.sum(res["E"].astype(np.float64) ** 2))
    assert abs(float(res["sum_e2"][0]) - e2) <= 1e-9 * e2 + 1e-300, label
    return dict(ties=r["ties"], drift=drift, loss_gpu=lg, loss_oracle=lo)


@pytest.mark.parametrize("name", ["c1", "c2a", "c2b"])
def test_workload_parity(bk, name):
    w = synth.WORKLOADS[name]
    W = synth.weights(w)
    X = synth.input_samples(w)
    Y = synth.output_samples(w)
    A, B, LA, LB = _factors(X, Y, w.m)
    res = _gpu(bk, W, LA, LB, w.qkind, w.qbits)
    info = _check_parity(W, A, B, LA, LB, w.qkind, w.qbits, res, name)
    print(name, info)
    if w.b_identity:
        # B = I: ordinary row-wise GPTQ (review page, "Load-bearing premise"),
        # under the same tie-adoption rule: no code may differ except by an
        # adopted boundary tie
        s, z = oracle.qparams(W, w.qkind, w.qbits)
        g = oracle.gptq_rows(W, LA, s, z, w.qkind, w.qbits, ref_codes=res["codes"], window=WINDOW)
        print(name, "row GPTQ: ties", g["ties"], "mismatches", g["mismatches"])
        assert g["mismatches"] == 0, name
        assert np.array_equal(g["codes"], res["codes"].astype(np.int32)), name


@pytest.mark.parametrize("m,n", [(1, 1), (1, 300), (300, 1), (65, 127), (200, 70), (64, 4096),
                                 (128, 64), (129, 193)])
def test_odd_shapes(bk, m, n):
    W, X, Y = synth.custom(m, n, 4000 + 7 * m + n)
    A, B, LA, LB = _factors(X, Y, m)
    for order in (1, 2):
        res = _gpu(bk, W, LA, LB, synth.SYM, 4, order)
        _check_parity(W, A, B, LA, LB, synth.SYM, 4, res, f"{m}x{n} order {order}")


@pytest.mark.parametrize("kind,bits", [(synth.SYM, 2), (synth.SYM, 3), (synth.SYM, 8),
                                       (synth.ASYM, 2), (synth.ASYM, 3), (synth.ASYM, 4),
                                       (synth.UNIT, 8)])
def test_quantizers(bk, kind, bits):
    m, n = 130, 150
    w_std = 3.0 if kind == synth.UNIT else 0.02
    W, X, Y = synth.custom(m, n, 5000 + 10 * kind + bits, w_std=w_std, outliers=4)
    A, B, LA, LB = _factors(X, Y, m)
    res = _gpu(bk, W, LA, LB, kind, bits)
    _check_parity(W, A, B, LA, LB, kind, bits, res, f"kind {kind} bits {bits}")


def test_deterministic_and_order_free(bk):
    W, X, Y = synth.custom(320, 256, 77)
    A, B, LA, LB = _factors(X, Y, 320)
    r1 = _gpu(bk, W, LA, LB, synth.SYM, 4, 1)
    r2 = _gpu(bk, W, LA, LB, synth.SYM, 4, 1)
    for k in ("codes", "V", "E", "scales", "sum_e2"):
        assert np.array_equal(r1[k], r2[k]), k
    r3 = _gpu(bk, W, LA, LB, synth.SYM, 4, 2)
    # the other product order reaches the same codes (Theorem 3.2) up to ties
    diff = np.sum(r1["codes"] != r3["codes"])
    assert diff <= 0.01 * W.size


def test_nonfinite_flag(bk):
    W, X, Y = synth.custom(64, 96, 9)
    W[3, 5] = np.nan
    A, B, LA, LB = _factors(X, Y, 64)
    res = _gpu(bk, W, LA, LB, synth.SYM, 4)
    assert res["status"] & bk.DEV_NONFINITE


def test_graph_replay_matches_eager(bk):
    """The cached graph of a solve reads the buffers' current contents: replays
    with new data in the same buffers match eager launches bit for bit, with
    eager work and synchronisations between the replays."""
    m, n = 192, 256
    W1, X, Y = synth.custom(m, n, 901)
    W2, _, _ = synth.custom(m, n, 902)
    A, B, LA, LB = _factors(X, Y, m)
    dev = torch.device("cuda:0")
    Wd = torch.from_numpy(W1).to(dev)
    LAd, LBd = torch.from_numpy(LA).to(dev), torch.from_numpy(LB).to(dev)
    ws = torch.empty(bk.quantize_workspace_size(m, n, 0, 4), dtype=torch.uint8, device=dev)
    out = dict(codes=torch.empty((m, n), dtype=torch.int8, device=dev),
               scales=torch.empty(m, device=dev), zeros=None,
               V=torch.empty((m, n), device=dev), E=torch.empty((m, n), device=dev),
               sum_e2=torch.empty(1, dtype=torch.float64, device=dev))

    def run(W_host, graph):
        Wd.copy_(torch.from_numpy(W_host))
        bk.quantize(Wd, LAd, LBd, workspace=ws, out=out, graph=graph)
        torch.cuda.synchronize()
        return {k: v.cpu().numpy().copy() for k, v in out.items() if v is not None}

    ref1, ref2 = run(W1, False), run(W2, False)
    for rep in range(3):
        for W_host, ref in ((W1, ref1), (W2, ref2)):
            got = run(W_host, True)
            for k in ref:
                assert np.array_equal(got[k], ref[k]), (rep, k)
            # eager work between replays
            run(W_host, False)


@pytest.mark.parametrize("m,n,order", [(1024, 1024, 1), (1536, 1024, 2), (1024, 3008, 0)])
def test_two_stream_modes_agree(bk, m, n, order):
    """At sizes where wide recursion nodes defer part of their band products to
    the side stream, the graph capture, the eager two-stream launch, the
    timing pass (the same plan in order on one stream) and a replay of the
    cached graph (same buffers, so the second graph call is a cache hit) give
    the same results bit for bit, and agree with the oracle's invariants on
    every row."""
    print(f"[modes] {m}x{n} order {order}", flush=True)
    assert bk.schedule_info(m, n, order)["side_launches"] > 0
    W, X, Y = synth.custom(m, n, 7000 + m + n)
    A, B, LA, LB = _factors(X, Y, m)
    dev = torch.device("cuda:0")
    Wd, LAd, LBd = (torch.from_numpy(a).to(dev) for a in (W, LA, LB))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(bk.quantize_workspace_size(m, n, 0, 4), dtype=torch.uint8, device=dev)
    out = dict(codes=torch.empty((m, n), dtype=torch.int8, device=dev),
               scales=torch.empty(m, device=dev), zeros=None,
               V=torch.empty((m, n), device=dev), E=torch.empty((m, n), device=dev),
               sum_e2=torch.empty(1, dtype=torch.float64, device=dev))
    runs = []
    for mode in ("graph", "eager", "timing", "graph"):
        for v in out.values():
            if v is not None:
                v.fill_(0)  # a replay must rewrite every output
        bk.quantize(Wd, LAd, LBd, kind=0, bits=4, order=order, dev_status=status, workspace=ws,
                    out=out, graph=(mode == "graph"), timing=(mode == "timing"))
        torch.cuda.synchronize()
        runs.append({k: v.cpu().numpy().copy() for k, v in out.items() if v is not None})
    assert int(status.item()) == 0
    for r in runs[1:]:
        for k in runs[0]:
            assert np.array_equal(r[k], runs[0][k]), k
    res = runs[0]
    s = res["scales"]
    bad, _ = oracle.rounding_consistency(res["codes"], res["V"], res["E"], np.diag(LA), np.diag(LB),
                                         s, np.zeros_like(s), 0, 4)
    assert bad == 0
    R = oracle.completion_residual(W, res["V"], res["E"], LA, LB)
    bound = (np.abs(LB.astype(np.float64)) @ np.abs(res["E"].astype(np.float64))) @ \
        np.abs(LA.astype(np.float64)).T
    assert np.max(np.abs(R) / (bound + 1e-30)) <= 1e-4


@pytest.mark.parametrize("m,n,order,split", [(1024, 1024, 1, None), (1536, 1024, 2, None),
                                             (200, 333, 0, None), (520, 780, 0, "rows")])
def test_workspace_never_read_before_written(bk, m, n, order, split):
    """A solve reads no workspace byte that it has not written first (the
    tile counters it clears itself): with every workspace byte set to 0xFF (a
    NaN in every float, -1 in every counter) the outputs equal, bit for bit,
    those of a zeroed workspace, and no non-finite value is flagged.  Graph and
    eager launches, with side launches at the two larger shapes."""
    print(f"[poison] {m}x{n} order {order} split {split}", flush=True)
    W, X, Y = synth.custom(m, n, 8100 + m + n)
    A, B, LA, LB = _factors(X, Y, m)
    dev = torch.device("cuda:0")
    Wd, LAd, LBd = (torch.from_numpy(a).to(dev) for a in (W, LA, LB))
    size = bk.quantize_workspace_size(m, n, 0, 4)
    runs = []
    for fill, graph in ((0, True), (255, True), (255, False)):
        ws = torch.full((size,), fill, dtype=torch.uint8, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        out = bk.quantize(Wd, LAd, LBd, kind=0, bits=4, order=order, want_E=True, want_sum=True,
                          dev_status=status, workspace=ws, graph=graph, split=split)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, (fill, graph)
        runs.append({k: v.cpu().numpy().copy() for k, v in out.items() if v is not None})
        del ws
    for r in runs[1:]:
        for k in runs[0]:
            assert np.array_equal(r[k].view(np.uint8), runs[0][k].view(np.uint8)), k


def _mse_params(W, kind, bits, got_s, got_z):
    """The oracle's MSE-searched parameters, with the GPU's choice accepted on a
    row where it differs only if it is a candidate whose error equals the least
    one up to the order of the fp64 sum (the two sides sum in different orders;
    the first-minimum rule then decides between near-equal candidates)."""
    s, z, kb, errs, cs, cz = oracle.qparams_mse(W, kind, bits, cands=True)
    diff = np.nonzero((got_s.view(np.uint32) != s.view(np.uint32)) | (got_z != z))[0]
    for i in diff:
        ks = np.nonzero((cs[i].view(np.uint32) == got_s[i].view(np.uint32)) & (cz[i] == got_z[i]))[0]
        assert len(ks), f"row {i}: scale {got_s[i]} is no candidate"
        assert errs[i, ks[0]] <= errs[i].min() * (1 + 1e-12), f"row {i}: not a least-error candidate"
    return got_s.copy(), got_z.copy(), kb, len(diff)


@pytest.mark.parametrize("kind,bits", [(synth.SYM, 4), (synth.SYM, 3), (synth.ASYM, 4), (synth.ASYM, 2)])
def test_mse_scale_search(bk, kind, bits):
    """Per-row scale shrink by MSE search (BAKRON_FLAG_MSE_SCALE): the GPU's
    parameters are the oracle's, and the solve with them matches the naive
    oracle run on the same parameters."""
    m, n = 200, 300
    print(f"[mse] kind {kind} bits {bits}", flush=True)
    W, X, Y = synth.custom(m, n, 6100 + 10 * kind + bits, outliers=6)
    A, B, LA, LB = _factors(X, Y, m)
    res = _gpu(bk, W, LA, LB, kind, bits, mse=True)
    zeros = res["zeros"] if res["zeros"] is not None else np.zeros(m, np.float32)
    s, z, kb, ndiff = _mse_params(W, kind, bits, res["scales"], zeros)
    assert ndiff <= 2
    assert np.mean(kb > 0) > 0.3          # the search does shrink
    _check_parity(W, A, B, LA, LB, kind, bits, res, f"mse kind {kind} bits {bits}", sz=(s, z))


def test_mse_scale_search_full_size(bk):
    """The search on the 4096 x 4096 workload's weights, in the launch
    configuration the benchmark uses (graph replay); the unit grid ignores it."""
    w = synth.WORKLOADS["c3"]
    W = synth.weights(w)
    dev = torch.device("cuda:0")
    eye = torch.eye(w.n, device=dev)
    out = bk.quantize(torch.from_numpy(W).to(dev), eye, eye, kind=w.qkind, bits=w.qbits, mse=True)
    torch.cuda.synchronize()
    got = out["scales"].cpu().numpy()
    s, z, kb, ndiff = _mse_params(W, w.qkind, w.qbits, got, np.zeros(w.m, np.float32))
    assert ndiff <= 4
    plain, _ = oracle.qparams(W, w.qkind, w.qbits)
    assert np.all(got <= plain)
    out = bk.quantize(torch.from_numpy(W[:64, :64].copy()).to(dev), eye[:64, :64].contiguous(),
                      eye[:64, :64].contiguous(), kind=synth.UNIT, bits=8, mse=True)
    torch.cuda.synchronize()
    assert np.all(out["scales"].cpu().numpy() == 1.0)
