"""CPU-side checks of the C ABI: the library loads, exports every function
declared in include/bakron.h, validates arguments before touching a device,
and its static schedule has the shape the method prescribes."""
import ctypes
import os
import re

import pytest

from two_sided_gptq_amd import bakron

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "bakron.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"\b(bakron_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bakron.LIB_PATH):
        from two_sided_gptq_amd import build
        build.build()
    return bakron.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(bakron.EXPORTS)


def test_missing_library_raises():
    saved = bakron._lib
    bakron._lib = None
    try:
        with pytest.raises(bakron.BakronError):
            bakron.load("/nonexistent/libbakron.so")
    finally:
        bakron._lib = saved


def test_workspace_sizes(lib):
    assert lib.bakron_quantize_workspace_size(64, 64, 0, 4) > 0
    assert lib.bakron_quantize_workspace_size(0, 64, 0, 4) == 0
    assert lib.bakron_quantize_workspace_size(64, 64, 0, 5) == 0      # 5-bit symmetric unsupported
    assert lib.bakron_quantize_workspace_size(64, 64, 1, 8) == 0      # 8-bit asym does not fit int8
    assert lib.bakron_quantize_workspace_size(64, 64, 7, 4) == 0
    big = lib.bakron_quantize_workspace_size(4096, 14336, 1, 2)
    # three mp x np fp32 buffers + padded LA, LB
    assert big >= 4 * (3 * 4096 * 14336 + 14336 ** 2 + 4096 ** 2)
    assert lib.bakron_factor_workspace_size(100) >= 2 * 128 * 128 * 8


def test_argument_errors_without_device(lib):
    P = ctypes.c_void_p
    fake = P(4096)
    rc = lib.bakron_quantize(None, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None, None, None,
                             0, fake, 1 << 20, None)
    assert rc == 1 and b"non-NULL" in lib.bakron_last_error()
    rc = lib.bakron_quantize(fake, 0, 4, fake, fake, 0, 4, fake, fake, None, None, None, None, None,
                             0, fake, 1 << 20, None)
    assert rc == 1
    rc = lib.bakron_quantize(fake, 4, 4, fake, fake, 0, 6, fake, fake, None, None, None, None, None,
                             0, fake, 1 << 20, None)
    assert rc == 1
    rc = lib.bakron_quantize(fake, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None, None, None,
                             0x80, fake, 1 << 20, None)
    assert rc == 1
    # the two split flags exclude each other, and a split is not phase-timed
    for flags in (0x20 | 0x40, 0x20 | 0x4, 0x40 | 0x4):
        rc = lib.bakron_quantize(fake, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None, None,
                                 None, flags, fake, 1 << 20, None)
        assert rc == 1 and b"SPLIT" in lib.bakron_last_error(), flags
    rc = lib.bakron_quantize(fake, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None, None, None,
                             0, fake, 16, None)
    assert rc == 2 and b"workspace" in lib.bakron_last_error()
    rc = lib.bakron_quantize(fake, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None, None, None,
                             0, P(4096 + 8), 1 << 30, None)
    assert rc == 2  # misaligned workspace
    assert lib.bakron_quantize_antidiag(None, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None,
                                        None, fake, 1 << 20, None) == 1
    assert lib.bakron_quantize_antidiag(fake, 4, 4, fake, fake, 0, 4, fake, fake, None, None, None,
                                        None, fake, 8, None) == 2
    assert lib.bakron_quantize_antidiag_workspace_size(4, 4, 0, 5) == 0
    assert lib.bakron_hessian(None, 4, 4, 0.01, fake, None, 0, None) == 1
    assert lib.bakron_hessian(fake, 4, 4, -1.0, fake, None, 0, None) == 1
    assert lib.bakron_factor(fake, 0, fake, None, fake, 1 << 20, None) == 1
    assert lib.bakron_factor(fake, 8, fake, None, fake, 8, None) == 2
    assert lib.bakron_status_string(2) == b"workspace too small"
    buf = (ctypes.c_double * 6)()
    assert lib.bakron_last_phase_ms(buf) == 1


def _brute_alg_flops(m, n):
    """Band MACs of the recursion at single anti-diagonal granularity, by
    enumeration: node [k, k+l) split at h = l // 2; T[i, jj] = sum over the
    S-sources (i, j), j <= jj, for every band entry some target row consumes;
    U[i2, jj] on R sums T over the rows i <= i2 that hold a source."""
    macs = 0

    def rec(k, l):
        nonlocal macs
        if l <= 1:
            return
        h = l // 2
        rec(k, h)
        for i in range(m):
            src = [j for j in range(n) if k <= i + j < k + h]
            if not src:
                continue
            for jj in range(n):
                if not (k <= i + jj < k + l):
                    continue
                if not any(k + h <= i2 + jj < k + l for i2 in range(i, m)):
                    continue
                macs += sum(1 for j in src if j <= jj)
        for i2 in range(m):
            for jj in range(n):
                if k + h <= i2 + jj < k + l:
                    macs += sum(1 for i in range(i2 + 1)
                                if any(k <= i + j < k + h and j <= jj for j in range(n)))
        rec(k + h, l - h)

    rec(0, m + n - 1)
    return 2 * macs


@pytest.mark.parametrize("m,n", [(3, 4), (4, 3), (8, 13), (16, 16), (5, 40)])
def test_algorithmic_flops_match_enumeration(lib, m, n):
    assert bakron.schedule_info(m, n)["alg_band_flops"] == _brute_alg_flops(m, n)


def _tile_recursion(D):
    """Band nodes (K, L, H) with a launch of their own (L >= 3) and the leaves
    that pull a two-diagonal node's update, of the recursion over D tile
    anti-diagonals (split at floor(L / 2))."""
    band, pulls = [], []

    def rec(K, L):
        if L == 1:
            return
        if L == 2:
            pulls.append(K + 1)
            return
        H = L // 2
        rec(K, H)
        band.append((K, L, H))
        rec(K + H, L - H)

    rec(0, D)
    return band, pulls


def test_schedule_shape(lib):
    # 4096 x 4096 in 64-tiles: 127 tile anti-diagonals, each swept in 127 steps;
    # O(m + n) sequential steps; product-order choice per shape.
    s = bakron.schedule_info(4096, 4096)
    band, pulls = _tile_recursion(127)
    assert s["leaf_launches"] == 127 and s["leaf_steps"] == 127 * 127
    assert len(band) + len(pulls) == 126          # every node of the recursion
    # two products per node; a node deferring part of its work adds two more
    assert s["band_launches"] == 2 * len(band) + s["side_launches"]
    assert s["side_launches"] == 2 * sum(1 for (K, L, H) in band if L - H >= 16)
    assert s["pull_leaves"] == len(pulls)
    tiles = lambda K: [(I, K - I) for I in range(max(0, K - 63), min(63, K) + 1)]
    prods = sum((2 if I >= 1 else 0) + (2 if J >= 1 else 0) for K in pulls for I, J in tiles(K))
    assert s["pull_flops"] == prods * 2 * 64 ** 3
    assert s["F"] == 4096 * 4096 * 8192
    assert abs(s["alg_band_flops"] / 2.369e11 - 1) < 1e-3
    # the band launches and the leaf pulls together never execute fewer flops
    # than the algorithmic count; the useful part excludes triangle zeros only
    for (m, n) in [(1024, 1024), (11008, 4096), (4096, 14336)]:
        for order in (1, 2):
            si = bakron.schedule_info(m, n, order)
            assert si["exec_band_flops"] + si["pull_flops"] >= si["alg_band_flops"] * 0.999
            assert 0.9 * si["exec_band_flops"] < si["useful_band_flops"] <= si["exec_band_flops"]
    assert bakron.schedule_info(11008, 4096)["order"] == 1
    assert bakron.schedule_info(4096, 14336)["order"] == 2
    # a single tile has no band update
    s = bakron.schedule_info(64, 64)
    assert s["leaf_launches"] == 1 and s["band_launches"] == 0
    # linear growth of the sequential step count (doubling sizes)
    steps = [bakron.schedule_info(k, k)["leaf_steps"] for k in (1024, 2048, 4096, 8192)]
    for a, b in zip(steps, steps[1:]):
        assert 1.9 < b / a < 2.1


def test_noalloc_argument_errors_without_device(lib):
    """The allocation-free entry point validates before touching a device: too
    large a shape for its fixed scratch is BAKRON_ERR_WORKSPACE, timing and
    unknown flags are invalid arguments."""
    fake = ctypes.c_void_p(4096)
    args = lambda m, n, flags: (fake, m, n, fake, fake, 0, 4, fake, fake, None, None, None, None,
                                None, flags, None)
    assert bakron.NOALLOC_SCRATCH_BYTES == 256 << 20
    assert lib.bakron_quantize_workspace_size(2048, 2048, 0, 4) <= bakron.NOALLOC_SCRATCH_BYTES
    assert lib.bakron_quantize_workspace_size(4096, 4096, 0, 4) > bakron.NOALLOC_SCRATCH_BYTES
    rc = lib.bakron_quantize_noalloc(*args(4096, 4096, 0))
    assert rc == 2 and b"bakron_quantize_noalloc has" in lib.bakron_last_error()
    rc = lib.bakron_quantize_noalloc(*args(64, 64, 0x4))
    assert rc == 1 and b"PHASE_TIMING" in lib.bakron_last_error()
    rc = lib.bakron_quantize_noalloc(*args(64, 64, 0x80))
    assert rc == 1
    rc = lib.bakron_quantize_noalloc(None, 64, 64, fake, fake, 0, 4, fake, fake, None, None, None,
                                     None, None, 0, None)
    assert rc == 1 and b"non-NULL" in lib.bakron_last_error()
