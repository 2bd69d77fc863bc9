"""bakron_quantize_noalloc, the entry point that allocates nothing, against
bakron_quantize on the same inputs, through the C ABI.

Two calls in a row, the second with a smaller input: the second runs on a
scratch array that still holds the first call's contents.  Each result must
equal the workspace entry point's bit for bit (the same kernels run the same
plan, and the plan's results do not depend on the streams it runs on), which
is stricter than the oracle parity bar that entry point is held to.  The first
size has band products deferred to the side stream, which the allocation-free
call runs in order on the caller's stream.
"""
import numpy as np
import pytest

import oracle
from two_sided_gptq_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bk():
    from two_sided_gptq_amd import bakron
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    bakron.load()
    return bakron


def _factor32(S):
    return oracle.factor(oracle.hessian(S, synth.DAMP)).astype(np.float32)


def test_noalloc_matches_workspace_entry_point(bk):
    dev = torch.device("cuda:0")
    cases = [(1024, 1024, synth.SYM, 4, 3101), (320, 200, synth.ASYM, 2, 3102)]
    assert bk.schedule_info(1024, 1024)["side_launches"] > 0
    for m, n, kind, bits, seed in cases:
        print(f"[noalloc] {m}x{n} kind {kind} bits {bits}", flush=True)
        W, X, Y = synth.custom(m, n, seed, outliers=4)
        Wd = torch.from_numpy(W).to(dev)
        LA = torch.from_numpy(_factor32(X)).to(dev)
        LB = torch.from_numpy(_factor32(Y)).to(dev)
        st_ref = torch.zeros(1, dtype=torch.int32, device=dev)
        st_got = torch.zeros(1, dtype=torch.int32, device=dev)
        ref = bk.quantize(Wd, LA, LB, kind=kind, bits=bits, want_E=True, want_sum=True,
                          dev_status=st_ref)
        got = bk.quantize_noalloc(Wd, LA, LB, kind=kind, bits=bits, want_E=True, want_sum=True,
                                  dev_status=st_got)
        torch.cuda.synchronize()
        assert int(st_ref.item()) == 0 and int(st_got.item()) == 0
        for k, v in ref.items():
            if v is None:
                assert got[k] is None, k
                continue
            assert torch.equal(v, got[k]), (m, n, k)
        # and the codes are the base quantizer of the pre-rounding values
        c, V, E, s = (got[k].cpu().numpy() for k in ("codes", "V", "E", "scales"))
        z = got["zeros"].cpu().numpy() if got["zeros"] is not None else np.zeros_like(s)
        bad, _ = oracle.rounding_consistency(c, V, E, np.diag(LA.cpu().numpy()),
                                             np.diag(LB.cpu().numpy()), s, z, kind, bits)
        assert bad == 0
