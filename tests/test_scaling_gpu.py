"""The pages' complexity check (pith.science review, "What would settle it"):
time the solver on weight matrices of doubling size.  Total work growing as
m^2 n^2 would make every doubling of a square matrix cost 16 times as much;
the method's mn(m + n) work costs at most 8 times as much, and less while the
solve's m + n - 1 sequential tile diagonals set the time.  The inputs are
seeded Gaussian weights and the library's own factors of Gaussian samples
(2n of them), at 512^2, 1024^2, 2048^2 and 4096^2, INT4 symmetric; each time
is the mean of five cached-graph solves after two warm-up calls, between HIP
events on the solve's stream."""
import math

import pytest

from two_sided_gptq_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SIZES = (512, 1024, 2048, 4096)


@pytest.fixture(scope="module")
def bk():
    from two_sided_gptq_amd import bakron
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    bakron.load()
    return bakron


def _solve_ms(bk, n, reps=5):
    W, X, Y = synth.custom(n, n, 6100 + n)
    dev = torch.device("cuda:0")
    LA = bk.factor(bk.hessian(torch.from_numpy(X).to(dev), synth.DAMP))
    LB = bk.factor(bk.hessian(torch.from_numpy(Y).to(dev), synth.DAMP))
    Wd = torch.from_numpy(W).to(dev)
    ws = torch.empty(bk.quantize_workspace_size(n, n, synth.SYM, 4), dtype=torch.uint8, device=dev)
    out = dict(codes=torch.empty((n, n), dtype=torch.int8, device=dev),
               scales=torch.empty(n, device=dev), zeros=None,
               V=torch.empty((n, n), device=dev), E=None,
               sum_e2=torch.empty(1, dtype=torch.float64, device=dev))
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        bk.quantize(Wd, LA, LB, kind=synth.SYM, bits=4, dev_status=status, workspace=ws, out=out)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return e0.elapsed_time(e1) / reps


def test_doubling_sizes(bk):
    t = {n: _solve_ms(bk, n) for n in SIZES}
    for a, b in zip(SIZES, SIZES[1:]):
        # the work count itself: mn(m+n) grows exactly 8x per doubling
        fa, fb = bk.schedule_info(a, a)["F"], bk.schedule_info(b, b)["F"]
        ratio = t[b] / t[a]
        print(f"[scaling] {a}^2 -> {b}^2: {t[a]:.3f} -> {t[b]:.3f} ms, x{ratio:.2f} "
              f"(work x{fb / fa:.2f}; m^2 n^2 would be x16)")
        assert fb / fa == pytest.approx(8.0, rel=1e-12)
        assert ratio < 10.0
    slope = math.log2(t[SIZES[-1]] / t[SIZES[0]]) / (len(SIZES) - 1)
    print(f"[scaling] growth exponent per doubling of n: {slope:.2f} (cubic work: 3, m^2 n^2: 4)")
    assert slope < 3.2
