"""Pins for the schedule model: hand-derived fixtures, the partition
property over many sizes, special cases that reduce to textbook orders, the
work-stealing invariants under random interleavings, and planted mistakes."""
import itertools
import random

import pytest

from oracle import sched_model as sm


def _prog_table(rows):
    out = {}
    for r in rows:
        p, _, rest = r.partition(":")
        out[int(p)] = [int(v) for v in rest.split()]
    return out


@pytest.mark.parametrize("name,kind,T,G", [
    ("sched_blocked_T10_G4.txt", "blocked", 10, 4),
    ("sched_blocked_T3_G8.txt", "blocked", 3, 8),
    ("sched_interleaved_T10_G4.txt", "interleaved", 10, 4),
])
def test_static_golden(golden, name, kind, T, G):
    want = _prog_table(golden(name))
    f = sm.blocked_vpids if kind == "blocked" else sm.interleaved_vpids
    for p in range(G):
        assert f(p, T, G) == want[p]


def test_plain_decode_golden(golden):
    for r in golden("decode_plain_m5_n2.txt"):
        v, m, n = map(int, r.split())
        assert sm.plain_decode(v, 5) == (m, n)


def test_grouped_decode_golden(golden):
    for r in golden("decode_grouped_m10_n3_g4.txt"):
        v, m, n = map(int, r.split())
        assert sm.grouped_decode(v, 10, 3, 4) == (m, n)


def test_ws_golden(golden):
    rows = [tuple(map(int, r.split())) for r in golden("ws_T10_X4_G8.txt")]
    assert sm.ws_ranges(10, 4) == [(s, e) for _, s, e, _ in rows]
    assert sm.ws_final_counters(10, 8, 4) == [c for *_, c in rows]
    seqs, cnt = sm.ws_simulate(5, 2, 8, 4, gs=8, seed=1)
    assert cnt == [c for *_, c in rows]


SIZES = [(1, 1), (1, 7), (7, 1), (3, 5), (16, 16), (13, 23), (10, 30), (32, 4), (17, 17)]


@pytest.mark.parametrize("kind", sm.STATIC_KINDS)
@pytest.mark.parametrize("G", [1, 7, 8, 256])
def test_static_partition(kind, G):
    for (pm, pn), gs in itertools.product(SIZES, [1, 3, 8, 16]):
        sm.check_partition(sm.static_schedule(kind, pm, pn, G, gs), pm, pn)


def test_grouped_special_cases():
    for pm, pn in SIZES:
        for v in range(pm * pn):
            # group_size 1: row-major (pid_n fastest)
            assert sm.grouped_decode(v, pm, pn, 1) == (v // pn, v % pn)
            # group_size >= num_pid_m: the plain decode
            assert sm.grouped_decode(v, pm, pn, pm) == sm.plain_decode(v, pm)
            assert sm.grouped_decode(v, pm, pn, pm + 5) == sm.plain_decode(v, pm)


def test_blocked_fewer_tiles_than_programs():
    s = sm.static_schedule("blocked", 4, 4, 256)
    assert [len(x) for x in s[:16]] == [1] * 16 and all(len(x) == 0 for x in s[16:])
    s = sm.static_schedule("blocked", 20, 20, 256)          # T = 400: bs = 2
    assert all(len(x) == 2 for x in s[:200]) and all(len(x) == 0 for x in s[200:])


@pytest.mark.parametrize("pm,pn,G,X,chunk", [
    (5, 2, 8, 4, 1), (32, 32, 256, 8, 1), (20, 20, 256, 8, 1), (19, 32, 256, 8, 1),
    (12, 28, 256, 8, 1), (2, 2, 256, 8, 1), (1, 1, 8, 8, 1), (9, 7, 11, 8, 1),
    (256, 8, 256, 8, 8), (33, 5, 16, 8, 4),
])
def test_ws_simulated_invariants(pm, pn, G, X, chunk):
    T = pm * pn
    for seed in range(3):
        seqs, cnt = sm.ws_simulate(pm, pn, G, X, gs=8, chunk=chunk, seed=seed)
        sm.check_partition(seqs, pm, pn)
        visits, owner, order = [0] * T, [-1] * T, [-1] * T
        for p, seq in enumerate(seqs):
            for i, (v, _, _) in enumerate(seq):
                visits[v] += 1
                owner[v] = p
                order[v] = i
        sm.check_ws_execution(visits, owner, order, cnt, T, G, X, chunk)


def test_ws_rebalances_straggler():
    # program 0 is 10x slower: its XCD peers take over its share
    G, X = 16, 8
    speeds = [10.0] + [1.0] * (G - 1)
    seqs, _ = sm.ws_simulate(8, 8, G, X, speeds=speeds)
    assert len(seqs[0]) < len(seqs[8])
    sm.check_partition(seqs, 8, 8)


def test_ws_rejects_grid_below_xcds():
    with pytest.raises(ValueError):
        sm.ws_simulate(4, 4, 7, 8)


def _witness(seqs, T):
    visits, owner, order = [0] * T, [-1] * T, [-1] * T
    for p, seq in enumerate(seqs):
        for i, (v, _, _) in enumerate(seq):
            visits[v] += 1
            owner[v] = p
            order[v] = i
    return visits, owner, order


def test_checkers_catch_planted_mistakes():
    seqs = sm.static_schedule("interleaved", 4, 4, 3)
    bad = [list(s) for s in seqs]
    bad[0].append(bad[1][0])                                # a tile twice
    with pytest.raises(AssertionError):
        sm.check_partition(bad, 4, 4)
    bad = [list(s) for s in seqs]
    bad[2].pop()                                            # a tile dropped
    with pytest.raises(AssertionError):
        sm.check_partition(bad, 4, 4)
    seqs, cnt = sm.ws_simulate(4, 4, 8, 4, seed=2)
    T = 16
    v, o, r = _witness(seqs, T)
    with pytest.raises(AssertionError):                      # wrong final counter
        sm.check_ws_execution(v, o, r, [c + 1 for c in cnt], T, 8, 4)
    o2 = list(o)
    o2[0] = (o2[0] + 1) % 8                                 # owner on another XCD
    with pytest.raises(AssertionError):
        sm.check_ws_execution(v, o2, r, cnt, T, 8, 4)
    v2 = list(v)
    v2[5] = 2
    with pytest.raises(AssertionError):
        sm.check_ws_execution(v2, o, r, cnt, T, 8, 4)


@pytest.mark.parametrize("name,T,nk,G,partials", [
    ("sk_T5_nk4_G3.txt", 5, 4, 3, {3: [(0, 0, 2), (1, 2, 4)], 4: [(1, 0, 1), (2, 1, 4)]}),
    ("sk_T2_nk3_G4.txt", 2, 3, 4, {0: [(0, 0, 1), (1, 1, 3)], 1: [(2, 0, 1), (3, 1, 3)]}),
])
def test_streamk_golden(golden, name, T, nk, G, partials):
    rows = [tuple(map(int, r.split())) for r in golden(name)]
    want = {}
    for p, v, kb, ke in rows:
        want.setdefault(p, []).append((v, kb, ke))
    got = sm.streamk_schedule(T, nk, G)
    assert {p: s for p, s in enumerate(got)} == want
    assert sm.streamk_partials(T, nk, G) == partials


@pytest.mark.parametrize("T,nk,G", [(10, 4, 4), (16, 3, 4), (1, 7, 8), (7, 1, 8), (608, 128, 256),
                                    (400, 64, 256), (448, 64, 512), (1024, 128, 256), (3, 5, 256),
                                    (300, 2, 7)])
def test_streamk_cover_and_balance(T, nk, G):
    sched = sm.streamk_schedule(T, nk, G)
    sm.check_streamk_cover(sched, T, nk)
    dp = sm.streamk_dp_tiles(T, G)
    # data-parallel part: stride by grid, whole tiles
    for p, segs in enumerate(sched):
        whole = [v for v, kb, ke in segs if v < dp]
        assert whole == list(range(p, dp, G))
    # stream-K part: per-program slab counts differ by at most one
    sk = [sum(ke - kb for v, kb, ke in segs if v >= dp) for segs in sched]
    assert max(sk) - min(sk) <= 1 and sum(sk) == (T - dp) * nk
    # every full wave is data-parallel: fewer than G tiles are left to split,
    # so no run is longer than one tile and none touches more than two tiles
    assert dp % G == 0 and 0 <= T - dp < G
    assert max(sk) <= nk
    assert all(len([s for s in segs if s[0] >= dp]) <= 2 for segs in sched)
    # G divides T: nothing is split
    if T % G == 0:
        assert dp == T and not sm.streamk_partials(T, nk, G)
    # a program has at most two partial segments: the first and the last of its run
    for segs in sched:
        run = [s for s in segs if s[0] >= dp]
        part = [i for i, (v, kb, ke) in enumerate(run) if kb != 0 or ke != nk]
        assert all(i in (0, len(run) - 1) for i in part)


def test_streamk_checker_catches_planted_mistakes():
    sched = [list(s) for s in sm.streamk_schedule(5, 4, 3)]
    sched[2][1] = (4, 0, 4)                                 # slab 0 of tile 4 twice
    with pytest.raises(AssertionError):
        sm.check_streamk_cover(sched, 5, 4)
    sched = [list(s) for s in sm.streamk_schedule(5, 4, 3)]
    sched[2].pop()                                          # slabs 1..3 of tile 4 dropped
    with pytest.raises(AssertionError):
        sm.check_streamk_cover(sched, 5, 4)
    # a run boundary off by one slab breaks the cover
    sched = [list(s) for s in sm.streamk_schedule(5, 4, 3)]
    sched[0][1] = (3, 0, 3)
    with pytest.raises(AssertionError):
        sm.check_streamk_cover(sched, 5, 4)


# ---- work stealing across XCDs ----

def test_wsx_golden(golden):
    rows = [r.split() for r in golden("wsx_T6_X2_G3.txt")]
    want = {}
    for r in rows:
        if r[0] == "counters":
            counters = list(map(int, r[1:]))
            continue
        p, v, m, n = map(int, r)
        want.setdefault(p, []).append((v, m, n))
    seqs, cnt = sm.wsx_simulate(3, 2, 3, 2, homes=[0, 0, 1], speeds=[1, 1, 4])
    assert {p: s for p, s in enumerate(seqs)} == want
    assert cnt == counters
    assert sm.wsx_counter_bounds(6, 3, 2, [0, 0, 1]) == [(5, 6), (4, 6)]


def _wsx_arrays(seqs, T):
    visits, owner, order = [0] * T, [-1] * T, [-1] * T
    for p, seq in enumerate(seqs):
        for i, (v, _, _) in enumerate(seq):
            visits[v] += 1
            owner[v] = p
            order[v] = i
    return visits, owner, order


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(4, 4, 8, 4, 1), (5, 7, 3, 8, 1), (16, 16, 256, 8, 1),
                                             (13, 23, 64, 8, 2), (1, 1, 8, 8, 1), (32, 4, 12, 8, 4)])
def test_wsx_simulated_invariants(pm, pn, G, X, chunk):
    T = pm * pn
    rng = random.Random(G * 31 + X)
    # homes: round-robin, all programs on one XCD, and random placements
    for homes in ([p % X for p in range(G)], [0] * G, [rng.randrange(X) for _ in range(G)]):
        for seed in range(3):
            seqs, cnt = sm.wsx_simulate(pm, pn, G, X, homes, chunk=chunk, seed=seed)
            sm.check_partition(seqs, pm, pn)
            visits, owner, order = _wsx_arrays(seqs, T)
            sm.check_wsx_execution(visits, owner, order, cnt, homes, T, G, X, chunk)


def test_wsx_steals_from_a_slow_xcd():
    # programs on XCD 0 are ten times slower: the others take most of its range
    G, X = 16, 4
    homes = [p % X for p in range(G)]
    speeds = [10.0 if homes[p] == 0 else 1.0 for p in range(G)]
    seqs, _ = sm.wsx_simulate(16, 16, G, X, homes, speeds=speeds)
    s0, e0 = sm.ws_ranges(256, X)[0]
    stolen = sum(1 for p, seq in enumerate(seqs) if homes[p] != 0 for v, _, _ in seq if s0 <= v < e0)
    assert stolen > (e0 - s0) // 2
    # without stealing, XCD 0's programs compute all of it
    seqs_ws, _ = sm.ws_simulate(16, 16, G, X, speeds=speeds)
    assert all(p % X == 0 for p, seq in enumerate(seqs_ws) for v, _, _ in seq if s0 <= v < e0)


def test_wsx_checker_catches_planted_mistakes():
    pm, pn, G, X = 4, 4, 6, 4
    T = pm * pn
    homes = [0, 0, 1, 1, 2, 2]
    seqs, cnt = sm.wsx_simulate(pm, pn, G, X, homes, seed=5)
    v, o, r = _wsx_arrays(seqs, T)
    sm.check_wsx_execution(v, o, r, cnt, homes, T, G, X)
    lo = [b[0] for b in sm.wsx_counter_bounds(T, G, X, homes)]
    hi = [b[1] for b in sm.wsx_counter_bounds(T, G, X, homes)]
    with pytest.raises(AssertionError):                    # a missing failing claim at home
        sm.check_wsx_execution(v, o, r, [lo[0] - 1] + list(cnt[1:]), homes, T, G, X)
    with pytest.raises(AssertionError):                    # two failing claims by one program
        sm.check_wsx_execution(v, o, r, [hi[0] + 1] + list(cnt[1:]), homes, T, G, X)
    with pytest.raises(AssertionError):                    # a tile computed twice
        v2 = list(v)
        v2[3] = 2
        sm.check_wsx_execution(v2, o, r, cnt, homes, T, G, X)
    # a program whose tiles are not in cyclic counter order from its home
    p = max(range(G), key=lambda q: len({sm.ws_owner(t, T, X) for t, _, _ in seqs[q]}))
    assert len({sm.ws_owner(t, T, X) for t, _, _ in seqs[p]}) > 1
    with pytest.raises(AssertionError):
        sm.check_wsx_execution(v, o, r, cnt, [(h + 1) % X if q == p else h
                                              for q, h in enumerate(homes)], T, G, X)


# ---- paired claims ----

def test_ws_pairs_golden(golden):
    rows = [r.split() for r in golden("ws_pairs_T10_X2_G4.txt")]
    want = {}
    for r in rows:
        if r[0] == "counters":
            counters = list(map(int, r[1:]))
            continue
        p, v, m, n = map(int, r)
        want.setdefault(p, []).append((v, m, n))
    seqs, cnt = sm.ws_simulate(5, 2, 4, 2, chunk=sm.PAIRS, speeds=[1, 1, 1, 1])
    assert {p: s for p, s in enumerate(seqs)} == want
    assert cnt == counters


def test_pair_claim_map():
    # P = ceil(256 / 8) = 32 programs per counter
    assert sm.pair_span(128, 256, 8) == 128        # four rounds: all pairs
    assert sm.pair_span(76, 256, 8) == 64          # three rounds: one round of pairs
    assert sm.pair_span(50, 256, 8) == 50          # two rounds: all pairs
    assert sm.pair_span(32, 256, 8) == 0           # one round: singles
    assert sm.pair_span(33, 256, 8) == 32
    assert sm.pair_claims(76, 256, 8) == 32 + 12
    assert [sm.pair_claim(k, 76, 256, 8) for k in (0, 31, 32, 43, 44)] == \
        [(0, 2), (62, 64), (64, 65), (75, 76), None]
    # every tile of a range exactly once, in order
    for n in range(0, 140):
        tiles = [t for k in range(sm.pair_claims(n, 256, 8))
                 for t in range(*sm.pair_claim(k, n, 256, 8))]
        assert tiles == list(range(n))
        assert sm.pair_claim(sm.pair_claims(n, 256, 8), n, 256, 8) is None


@pytest.mark.parametrize("pm,pn,G,X", [(4, 4, 8, 4), (16, 16, 256, 8), (20, 20, 256, 8),
                                       (19, 32, 256, 8), (12, 28, 256, 8), (5, 7, 9, 8)])
def test_pairs_simulated_invariants(pm, pn, G, X):
    T = pm * pn
    for seed in range(3):
        seqs, cnt = sm.ws_simulate(pm, pn, G, X, chunk=sm.PAIRS, seed=seed)
        sm.check_partition(seqs, pm, pn)
        v, o, r = _wsx_arrays(seqs, T)
        sm.check_ws_execution(v, o, r, cnt, T, G, X, sm.PAIRS)
        homes = [random.Random(seed).randrange(X) for _ in range(G)]
        seqs, cnt = sm.wsx_simulate(pm, pn, G, X, homes, chunk=sm.PAIRS, seed=seed)
        sm.check_partition(seqs, pm, pn)
        v, o, r = _wsx_arrays(seqs, T)
        sm.check_wsx_execution(v, o, r, cnt, homes, T, G, X, sm.PAIRS)


def test_pairs_keep_the_makespan_of_single_claims():
    # equal speeds: no program computes more tiles than under single claims,
    # and for 1.3-2.4 rounds per XCD most tiles come in consecutive pairs
    for pm, pn in [(20, 20), (19, 32), (12, 28), (32, 32)]:
        G, X = 256, 8
        one, _ = sm.ws_simulate(pm, pn, G, X, chunk=1, speeds=[1] * G)
        two, _ = sm.ws_simulate(pm, pn, G, X, chunk=sm.PAIRS, speeds=[1] * G)
        assert max(map(len, two)) == max(map(len, one)), (pm, pn)
        paired = sum(1 for s in two for a, b in zip(s, s[1:]) if b[0] == a[0] + 1)
        assert paired >= (pm * pn) // 4, (pm, pn, paired)
    # fixed pairs lose a round where a range is just over two rounds
    fixed, _ = sm.ws_simulate(19, 32, 256, 8, chunk=2, speeds=[1] * 256)
    one, _ = sm.ws_simulate(19, 32, 256, 8, chunk=1, speeds=[1] * 256)
    assert max(map(len, fixed)) > max(map(len, one))


def test_pairs_checker_catches_planted_mistakes():
    pm, pn, G, X = 5, 2, 4, 2
    T = pm * pn
    seqs, cnt = sm.ws_simulate(pm, pn, G, X, chunk=sm.PAIRS, speeds=[1] * G)
    v, o, r = _wsx_arrays(seqs, T)
    sm.check_ws_execution(v, o, r, cnt, T, G, X, sm.PAIRS)
    with pytest.raises(AssertionError):                     # one failing claim too many
        sm.check_ws_execution(v, o, r, [cnt[0] + 1, cnt[1]], T, G, X, sm.PAIRS)
    with pytest.raises(AssertionError):                     # a program's failing claim missing
        sm.check_ws_execution(v, o, r, [cnt[0] - 1, cnt[1]], T, G, X, sm.PAIRS)
    with pytest.raises(AssertionError):                     # a pair split across programs
        o2 = list(o)
        o2[1] = 2
        sm.check_ws_execution(v, o2, r, cnt, T, G, X, sm.PAIRS)


# ---- several problems in one launch ----

def test_multi_blocked_golden(golden):
    want = {}
    for r in golden("multi_blocked_2problems_G4.txt"):
        p, v, g, m, n = map(int, r.split())
        want.setdefault(p, []).append((v, g, m, n))
    got = sm.multi_static_schedule("blocked", [(3, 2), (2, 2)], 4)
    assert {p: s for p, s in enumerate(got)} == want


def test_multi_decode_reduces_to_single_problem():
    # one problem: the shared space is the problem's own
    for kind in sm.STATIC_KINDS:
        for v in range(13 * 7):
            assert sm.multi_decode(kind, v, [(13, 7)], 4) == (0,) + sm.decode(kind, v, 13, 7, 4)
    # an empty problem takes no ids
    assert sm.multi_offsets([(2, 3), (0, 5), (1, 1)]) == [0, 6, 6, 7]
    assert sm.multi_decode("blocked", 6, [(2, 3), (0, 5), (1, 1)]) == (2, 0, 0)


@pytest.mark.parametrize("kind", sm.STATIC_KINDS)
@pytest.mark.parametrize("G", [1, 7, 256])
def test_multi_partition(kind, G):
    for grids in ([(3, 2), (2, 2)], [(1, 1)] * 5, [(17, 9), (0, 3), (4, 40), (33, 1)]):
        sm.check_multi_partition(sm.multi_static_schedule(kind, grids, G, 3), grids)


def test_multi_checker_catches_planted_mistakes():
    grids = [(3, 2), (2, 2)]
    seqs = [list(s) for s in sm.multi_static_schedule("interleaved", grids, 3)]
    seqs[0][0] = (0, 1, 0, 0)                 # problem 0's first tile decoded in problem 1
    with pytest.raises(AssertionError):
        sm.check_multi_partition(seqs, grids)
    seqs = [list(s) for s in sm.multi_static_schedule("interleaved", grids, 3)]
    seqs[2].pop()                              # a tile dropped
    with pytest.raises(AssertionError):
        sm.check_multi_partition(seqs, grids)


# Balanced default grid, values worked by hand from its definition (256 CUs,
# 8 XCDs, one program per CU at 256x256 tiles, two at 128x128):
#   T = 400: ranges of 50 tiles, 32 programs per XCD take 2 rounds; 25 per XCD
#   also take 2 (50 / 25), 24 would take 3, so 200 programs.
#   T = 608: ranges of 76, 3 rounds at 32; 26 per XCD take 3 (76 / 26 < 3),
#   25 take 4, so 208.  T = 336: ranges of 42, 2 rounds; 21 per XCD, 168.
#   T = 1024: ranges of 128, 4 rounds, 32 per XCD, 256 (unchanged).
#   T = 16: ranges of 2, 1 round, 2 per XCD, 16.  T = 1: one range of 1
#   tile (the others empty), 1 per XCD, 8.  T = 448 at 512 programs: ranges
#   of 56, 1 round at 64 per XCD, 56 per XCD, 448.  T = 1025: ranges of 128
#   or 129, 5 rounds at 32 per XCD; 26 per XCD also take 5 (129 / 26 < 5),
#   25 take 6, so 208.  T = 257: ranges of 32 or 33, 2 rounds; 17 per XCD, 136.
@pytest.mark.parametrize("T,G,want", [(400, 256, 200), (608, 256, 208), (336, 256, 168),
                                      (1024, 256, 256), (16, 256, 16), (1, 256, 8),
                                      (448, 512, 448), (0, 256, 256), (112, 256, 112),
                                      (1025, 256, 208), (257, 256, 136)])
def test_balanced_grid_hand_values(T, G, want):
    assert sm.balanced_grid(T, G, 8) == want


@pytest.mark.parametrize("G,X", [(256, 8), (512, 8), (64, 4), (24, 8)])
def test_balanced_grid_properties(G, X):
    """No scheduler takes more rounds under the balanced grid than work
    stealing under G (static walks counted from the model's own schedules),
    one multiple of X fewer would take more, and it never exceeds G."""
    for T in list(range(1, 400)) + [400, 608, 336, 1024, 1500, 2048]:
        g = sm.balanced_grid(T, G, X)
        assert g % X == 0 and X <= g <= G, (T, g)
        want = sm.ws_rounds(T, G, X)
        assert sm.ws_rounds(T, g, X) <= want
        if g > X:
            assert sm.ws_rounds(T, g - X, X) > want, (T, g)
        if T <= 400:
            pm = T  # one row of tiles per column: the static walks over T tiles
            for kind in ("blocked", "interleaved"):
                seqs = sm.static_schedule(kind, pm, 1, g)
                assert max(len(s) for s in seqs) <= want, (kind, T, g)


def test_balanced_grid_planted_mistake():
    """A grid one multiple of X too small (a plausible off-by-one in the
    rounding) takes an extra round on a wave-quantised shape."""
    T, G, X = 608, 256, 8
    assert sm.ws_rounds(T, sm.balanced_grid(T, G, X) - X, X) == sm.ws_rounds(T, G, X) + 1


def test_claim_counts_hand_worked():
    """One counter (X = 1), T = 4, G = 2, single claims: program 0 takes tiles
    0 and 2, program 1 tiles 1 and 3, then each makes its failing claim:
    three claims each, and the counter ends at 6."""
    owner = [0, 1, 0, 1]
    sm.check_claim_counts([[3], [3]], owner, [6], [0, 0], 4, 2, 1)
    with pytest.raises(AssertionError):             # a claim left out of the count
        sm.check_claim_counts([[3], [2]], owner, [6], [0, 0], 4, 2, 1)
    with pytest.raises(AssertionError):             # two failing claims by program 1
        sm.check_claim_counts([[2], [4]], owner, [6], [0, 0], 4, 2, 1)
    # chunk 2: program 0 takes [0, 2), program 1 [2, 4): two claims each, counter 8
    sm.check_claim_counts([[2], [2]], [0, 0, 1, 1], [8], [0, 0], 4, 2, 1, chunk=2)
    # pairs with P = 2 programs: L = 2 * min(2, 2 * (2 // 2)) = 4, claims 0 and 1
    # are the pairs (0, 1) and (2, 3); with one each, the counter ends at 4
    sm.check_claim_counts([[2], [2]], [1, 1, 0, 0], [4], [0, 0], 4, 2, 1, chunk=sm.PAIRS)


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(5, 2, 8, 4, 1), (19, 32, 256, 8, 1), (9, 7, 11, 8, 1),
                                             (33, 5, 16, 8, 4), (20, 20, 256, 8, "pairs"),
                                             (13, 11, 24, 8, "pairs")])
def test_ws_claim_counts_of_simulated_runs(pm, pn, G, X, chunk):
    chunk = sm.PAIRS if chunk == "pairs" else chunk
    T = pm * pn
    for seed in range(3):
        claims = []
        seqs, cnt = sm.ws_simulate(pm, pn, G, X, chunk=chunk, seed=seed, claims_out=claims)
        v, o, r = _witness(seqs, T)
        sm.check_ws_execution(v, o, r, cnt, T, G, X, chunk, claims=claims)
        assert all(claims[p][c] == 0 for p in range(G) for c in range(X) if c != p % X)


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(4, 4, 8, 4, 1), (5, 7, 3, 8, 1), (16, 16, 256, 8, 1),
                                             (13, 23, 64, 8, 2), (32, 4, 12, 8, 4), (13, 11, 24, 8, "pairs")])
def test_wsx_claim_counts_of_simulated_runs(pm, pn, G, X, chunk):
    chunk = sm.PAIRS if chunk == "pairs" else chunk
    T = pm * pn
    rng = random.Random(G * 17 + X)
    for homes in ([p % X for p in range(G)], [0] * G, [rng.randrange(X) for _ in range(G)]):
        for seed in range(3):
            claims = []
            seqs, cnt = sm.wsx_simulate(pm, pn, G, X, homes, chunk=chunk, seed=seed, claims_out=claims)
            v, o, r = _wsx_arrays(seqs, T)
            sm.check_wsx_execution(v, o, r, cnt, homes, T, G, X, chunk, claims=claims)


def test_claim_count_checker_catches_planted_mistakes():
    pm, pn, G, X = 6, 6, 8, 4
    T = pm * pn
    homes = [0, 0, 0, 1, 1, 2, 3, 3]
    claims = []
    seqs, cnt = sm.wsx_simulate(pm, pn, G, X, homes, seed=3, claims_out=claims)
    v, o, r = _wsx_arrays(seqs, T)
    sm.check_claim_counts(claims, o, cnt, homes, T, G, X, across=True)
    # an extra failing claim on a home counter, the counter raised to match
    bad = [list(row) for row in claims]
    bad[0][0] += 1
    with pytest.raises(AssertionError):
        sm.check_claim_counts(bad, o, [cnt[0] + 1] + list(cnt[1:]), homes, T, G, X, across=True)
    # a claim booked on the wrong counter
    bad = [list(row) for row in claims]
    bad[3][1] -= 1
    bad[3][2] += 1
    with pytest.raises(AssertionError):
        sm.check_claim_counts(bad, o, cnt, homes, T, G, X, across=True)
    # a program that never failed at home (its failing claim unrecorded)
    bad = [list(row) for row in claims]
    bad[5][2] -= 1
    with pytest.raises(AssertionError):
        sm.check_claim_counts(bad, o, [cnt[0], cnt[1], cnt[2] - 1, cnt[3]], homes, T, G, X, across=True)
    # per-XCD work stealing allows no claim away from home
    ws_claims = []
    seqs, cnt = sm.ws_simulate(pm, pn, G, X, seed=1, claims_out=ws_claims)
    v, o, r = _witness(seqs, T)
    bad = [list(row) for row in ws_claims]
    bad[1][2] += 1
    with pytest.raises(AssertionError):
        sm.check_claim_counts(bad, o, [cnt[0], cnt[1], cnt[2] + 1, cnt[3]], [p % X for p in range(G)],
                              T, G, X)
