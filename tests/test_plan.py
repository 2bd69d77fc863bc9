"""The two-stream schedule of a solve (bakron_schedule_plan) is race-free and
respects every data dependency, checked on the CPU against a model of what
each step reads and writes.

Model.  Steps run on two streams: leaves and critical band products on the
main stream, deferred band products on the side stream.  Happens-before (HB)
is stream order plus the plan's record -> wait edges (a wait orders everything
recorded before it).  Each step touches 64 x 64 tiles:
  leaf K      reads W and writes E on the tiles of diagonal K; a pushing leaf
              writes the two-diagonal buffers Cd(I+1, J), Cr(I, J+1); a
              pulling leaf reads Cd, Cr of its own tiles;
  band mode 0 T(J', I) = sum_J LA(J', J) E(I, J)^T       (writes T, reads E)
       mode 1 W(I', J') -= sum_I LB(I', I) T(J', I)^T     (reads T, updates W)
       mode 2 S(I', J) = sum_I LB(I', I) E(I, J)           (writes S, reads E)
       mode 3 W(I', J') -= sum_J S(I', J) LA(J', J)^T      (reads S, updates W)
with the staircase k range of each output tile (Algorithm 6's band update:
pith.science review of arXiv 2608.06291, Algorithm 6), T / S in the node's T
buffer (plan field 7).  Checked: every two steps that touch a tile, one of them
writing it, are HB-ordered, writers of E and T before their readers, every W
update of a tile before the leaf that reads it; the plan's band products cover
exactly the tiles of the recursion nodes they come from.
"""
import pytest

from two_sided_gptq_amd import bakron

LEAF, BAND, RECORD, WAIT = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(bakron.LIB_PATH):
        from two_sided_gptq_amd import build
        build.build()
    return bakron.load()


def tile_range(op, M, N):
    """(ci, cj, klo, khi) of every output tile of a band step (band_tile)."""
    K, H, mode = op["K"], op["H"], op["mode"]
    for row in range(op["rlo"], op["rlo"] + op["rows"]):
        for o in range(op["olo"], op["olo"] + op["cols"]):
            if mode == 0:
                I, Jp = row, K - row + o
                if not 0 <= Jp < N:
                    continue
                ci, cj, lo, hi = Jp, I, max(0, K - I), min(Jp, K + H - 1 - I)
            elif mode == 1:
                Ip, Jp = row, K + H + o - row
                if not 0 <= Jp < N:
                    continue
                ci, cj, lo, hi = Ip, Jp, max(0, K - Jp), min(Ip, K + H - 1)
            elif mode == 2:
                J, Ip = row, K - row + o
                if not 0 <= Ip < M:
                    continue
                ci, cj, lo, hi = Ip, J, max(0, K - J), min(Ip, K + H - 1 - J)
            else:
                Ip, Jp = row, K + H + o - row
                if not 0 <= Jp < N:
                    continue
                ci, cj, lo, hi = Ip, Jp, max(0, K - Ip), min(Jp, K + H - 1)
            if lo <= hi:
                yield ci, cj, lo, hi


def accesses(op, M, N):
    """(reads, writes) of one compute step as sets of tile keys."""
    rd, wr = set(), set()
    if op["kind"] == LEAF:
        K = op["K"]
        for I in range(max(0, K - N + 1), min(M - 1, K) + 1):
            J = K - I
            rd.add(("W", I, J))
            wr.add(("E", I, J))
            if op["flags"] == 1:
                rd.update({("Cd", I, J), ("Cr", I, J)})
            if op["flags"] == 2:
                if I + 1 < M:
                    wr.add(("Cd", I + 1, J))
                if J + 1 < N:
                    wr.add(("Cr", I, J + 1))
        return rd, wr
    d, mode = op["depth"], op["mode"]
    for ci, cj, lo, hi in tile_range(op, M, N):
        if mode == 0:      # T(ci = J', cj = I) from E(I, J), J in lo..hi
            wr.add(("T", d, ci, cj))
            rd.update(("E", cj, J) for J in range(lo, hi + 1))
        elif mode == 2:    # S(ci = I', cj = J) from E(I, J), I in lo..hi
            wr.add(("T", d, ci, cj))
            rd.update(("E", I, cj) for I in range(lo, hi + 1))
        elif mode == 1:    # W(ci, cj) -= ... T(J' = cj, I), I in lo..hi
            rd.add(("W", ci, cj))
            wr.add(("W", ci, cj))
            rd.update(("T", d, cj, I) for I in range(lo, hi + 1))
        else:              # W(ci, cj) -= ... S(I' = ci, J), J in lo..hi
            rd.add(("W", ci, cj))
            wr.add(("W", ci, cj))
            rd.update(("T", d, ci, J) for J in range(lo, hi + 1))
    return rd, wr


def happens_before(plan):
    """Compute steps (index list) and, per step, the bit set of its HB ancestors."""
    steps, anc = [], []
    frontier = {0: set(), 1: set()}   # steps whose completion a stream has seen
    ev = {}
    for op in plan:
        if op["kind"] == RECORD:
            ev[op["ev"]] = set(frontier[op["side"]])
            continue
        if op["kind"] == WAIT:
            frontier[op["side"]] |= ev[op["ev"]]
            continue
        if op["kind"] == BAND and op["rows"] < 0:
            continue          # no tile: nothing is launched
        s = 1 if (op["kind"] == BAND and op["side"] == 1) else 0
        k = len(steps)
        bits = 0
        for p in frontier[s]:
            bits |= anc[p] | (1 << p)
        steps.append(op)
        anc.append(bits)
        frontier[s] = {k}
    return steps, anc


def check_plan(m, n, order, mutate=None):
    si = bakron.schedule_info(m, n, order)
    order = int(si["order"])
    plan = bakron.schedule_plan(m, n, order)
    if mutate is not None:
        plan = mutate(plan)
    M, N = (m + 63) // 64, (n + 63) // 64
    steps, anc = happens_before(plan)
    hb = lambda a, b: (anc[b] >> a) & 1 == 1
    touch = {}
    for k, op in enumerate(steps):
        rd, wr = accesses(op, M, N)
        for key in rd:
            touch.setdefault(key, []).append((k, 0))
        for key in wr:
            touch.setdefault(key, []).append((k, 1))
    for key, acc in touch.items():
        writers = {k for k, w in acc if w}
        users = {k for k, _ in acc}
        for w in writers:
            for u in users:
                assert u == w or hb(w, u) or hb(u, w), (m, n, key, steps[w], steps[u])
        if key[0] == "E":              # the single producer comes first
            assert len(writers) == 1, key
            w = next(iter(writers))
            assert all(u == w or hb(w, u) for u in users), (m, n, key)
        if key[0] == "T":              # T buffers are reused by later nodes: each
            node = lambda k: (steps[k]["K"], steps[k]["L"])   # reader sees its own
            for u in users - writers:                         # node's product, and
                own = [w for w in writers if node(w) == node(u)]   # no other write
                assert len(own) == 1, (m, n, key)             # lies in between
                p = own[0]
                assert hb(p, u), (m, n, key)
                assert all(w == p or hb(u, w) or hb(w, p) for w in writers), (m, n, key)
        if key[0] == "W":              # every update before the leaf that reads the tile
            leaf = [k for k in users if steps[k]["kind"] == LEAF]
            assert len(leaf) == 1, key
            assert all(hb(w, leaf[0]) for w in writers), (m, n, key)
    # the deferred and critical pieces of a node cover exactly its tiles
    cover = {}
    for op in steps:
        if op["kind"] == BAND:
            key = (op["K"], op["L"], op["prod"])
            for t in tile_range(op, M, N):
                assert (key, t) not in cover, (m, n, key, t)
                cover[(key, t)] = 1
    whole = {}
    for op in steps:
        if op["kind"] == BAND:
            K, L, H, mode = op["K"], op["L"], op["H"], op["mode"]
            full = dict(op)
            if op["prod"] == 0:   # rows of the first product: the node's source rows
                X = N if mode == 0 else M
                rlo = max(0, K - X + 1)
                rhi = min((M if mode == 0 else N) - 1, K + H - 1)
                full.update(olo=0, cols=L)
            else:                 # rows of the second product: the target rows
                rlo = max(0, K + H - N + 1)
                rhi = min(M - 1, K + L - 1)
                full.update(olo=0, cols=L - H)
            full.update(rlo=rlo, rows=rhi - rlo + 1)
            whole[(K, L, op["prod"])] = full
    expect = {(k, t) for k, full in whole.items() for t in tile_range(full, M, N)}
    assert set(cover) == expect, (m, n)
    # some work is deferred once the recursion is wide enough
    n_side = sum(1 for op in steps if op["kind"] == BAND and op["side"] == 1)
    if mutate is None:
        assert n_side == si["side_launches"]
    return n_side


@pytest.mark.parametrize("m,n", [(64, 64), (192, 256), (1024, 1024), (1000, 3000), (4096, 4096),
                                 (2048, 512)])
@pytest.mark.parametrize("order", [1, 2])
def test_plan_race_free_and_ordered(lib, m, n, order):
    n_side = check_plan(m, n, order)
    if (m + 63) // 64 + (n + 63) // 64 - 1 >= 63:
        assert n_side > 0


def test_plan_full_size(lib):
    # the three full workloads with the order the solver picks
    for m, n in [(11008, 4096), (4096, 14336)]:
        assert check_plan(m, n, 0) > 0


PREP_TILES = 16   # tile rows / columns the critical stream sets up itself


@pytest.mark.parametrize("m,n", [(1024, 1024), (4096, 4096), (11008, 4096), (4096, 14336),
                                 (1000, 3000)])
def test_setup_join_covers_every_early_step(lib, m, n):
    """With a side stream the solve's set-up is split: the critical stream
    prepares tile rows and columns 0 .. PREP_TILES-1 (W and its row parameters,
    the factor copies, the leaf tables) and joins the side stream's part before
    the first critical step that is a leaf of diagonal >= PREP_TILES-1 or a band
    product of a node reaching diagonal PREP_TILES.  Every critical step before
    that point touches only tiles and factor blocks below PREP_TILES."""
    M, N = (m + 63) // 64, (n + 63) // 64
    if M + N - 1 <= 2 * PREP_TILES:
        pytest.skip("set-up not split")
    order = int(bakron.schedule_info(m, n, 0)["order"])
    early = 0
    for op in bakron.schedule_plan(m, n, order):
        if op["kind"] == LEAF:
            if op["K"] >= PREP_TILES - 1:
                break
            assert op["K"] + 1 < PREP_TILES   # a pushing leaf reads blocks one past K
        elif op["kind"] == BAND and op["side"] == 0 and op["rows"] > 0:
            if op["K"] + op["L"] > PREP_TILES:
                break
            for ci, cj, lo, hi in tile_range(op, M, N):
                assert max(ci, cj, hi) < PREP_TILES, (m, n, op)
        else:
            continue
        early += 1
    assert early > 0


def test_plan_flops_split(lib):
    # deferring moves work between streams but executes the same tiles
    for m, n in [(4096, 4096), (11008, 4096)]:
        si = bakron.schedule_info(m, n)
        assert 0 < si["side_useful_flops"] < si["useful_band_flops"]
        assert si["side_launches"] < si["band_launches"]


def _drop(pred):
    """A plan mutation that removes the first step matching pred."""
    def mutate(plan):
        k = next(i for i, op in enumerate(plan) if pred(plan, i))
        return plan[:k] + plan[k + 1:]
    return mutate


def test_plan_check_catches_missing_sync(lib):
    # each kind of event edge is needed: the model rejects the plan without the
    # side stream's wait before a deferred product (its fork), or without the
    # critical stream's wait for it (its join)
    fork = _drop(lambda pl, i: pl[i]["kind"] == WAIT and pl[i]["side"] == 1)
    join = _drop(lambda pl, i: pl[i]["kind"] == WAIT and pl[i]["side"] == 0)
    for mutate in (fork, join):
        with pytest.raises(AssertionError):
            check_plan(4096, 4096, 1, mutate)


def test_plan_check_catches_shared_t_buffer(lib):
    # a deferred product keeps its node's T buffer while later nodes run: the
    # model rejects a plan in which every node uses the same T buffer
    def one_buffer(plan):
        return [dict(op, depth=0) if op["kind"] == BAND else op for op in plan]
    with pytest.raises(AssertionError):
        check_plan(4096, 4096, 1, one_buffer)
    with pytest.raises(AssertionError):
        check_plan(4096, 4096, 2, one_buffer)
