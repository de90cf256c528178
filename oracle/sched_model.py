"""Model of the four tile schedulers: which workgroup (program) computes which
output tile, and in which order.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Notation: T tiles, G programs (the persistent grid), X XCDs, tile grid
num_pid_m x num_pid_n.  A virtual tile id v in [0, T) is decoded into
(pid_m, pid_n).

Sources:
* Blocked ranges, stride-by-grid and the plain decode: "Implement persistent
  kernels" (Helion PR #238), example output, PERSISTENT BLOCKED KERNEL and
  PERSISTENT INTERLEAVED KERNEL.  A program p with block size cdiv(T, G)
  takes [p*bs, min(p*bs + bs, T)); interleaved takes p, p+G, p+2G, ...;
  decode puts dimension 0 fastest: pid_m = v mod num_pid_m.
* Grouped decode: the same page, PERSISTENT BLOCKED WITH L2 GROUPING (group
  of 8 rows of tiles there; group_size here), with the last group shortened
  by the min().
* Grouped scheduler = stride-by-grid over the grouped order, the persistent
  loop plus swizzle of "[Feature] Introduce tile scheduler" (TileLang PR
  #2441), scheduler with swizzle_size / group_size.
* Work stealing: "Work Stealing Scheduler Kernel" (tritonBLAS PR #65),
  overview and review of the kernel: one int32 counter per XCD, program p
  uses counter p mod X, counters zeroed before each launch, programs claim
  their XCD's tiles until none are left.  Reading taken where the page is
  silent: XCD x owns the contiguous range [floor(x*T/X), floor((x+1)*T/X))
  of the grouped order; a claim is fetch_add(counter, chunk) and a program
  stops at its first claim that starts at or beyond the range's length.
* Work stealing across XCDs (reading taken where the pages stop: they keep
  one counter per XCD and never cross XCDs).  Same ranges and counters; a
  program's home counter is the XCD it runs on (any map of programs to
  counters is allowed, so completion never depends on placement).  A
  program claims from its home counter until a claim fails; it then looks
  at the counters it has not passed yet, in cyclic order x + 1, x + 2, ...,
  skips those already past their range, and claims from the first that is
  not; it stops when none is left.  So it makes exactly one failing claim on
  its home counter and at most one on any other.
* Several problems in one launch: "Implement persistent kernels" (Helion PR
  #238), example output, PERSISTENT BLOCKED / INTERLEAVED WITH FOR EACH
  PROGRAM ID (Multi-loop): the tiles of two problems share one virtual id
  space, the first problem's ids first; an id past the first problem's tile
  count is reduced by that count and decoded in the second.  Generalised
  here to several problems by prefix sums of their tile counts; any
  scheduler walks the shared space, and the id within a problem is decoded
  as that scheduler decodes a single problem.
* Paired claims (an option of both work-stealing kinds, not on the pages,
  which claim one tile at a time).  The counter then counts claims, and
  claim k of a range of n tiles takes tiles 2k, 2k+1 while k < L/2 and the
  single tile L + (k - L/2) after that, with P = ceil(G / X) programs per
  counter and L = 2 * min(floor(n / 2), P * floor(ceil(n / P) / 2)): pairs
  for as many whole rounds of two as the range holds, so with equal speeds
  no program computes more tiles than with single claims.
* Stream-K (the comparator "Work Stealing Scheduler Kernel", tritonBLAS PR
  #65, benchmarks work stealing against; the page names it only).  Reading
  taken: a data-parallel + stream-K hybrid in the spirit of the published
  Stream-K method, with only the partial wave split.  With T tiles of nk
  K-slabs on G programs, the first floor(T/G)*G tiles (all of them when G
  divides T, none when T < G) are taken stride-by-grid, whole, and the
  slabs of the remaining T mod G tiles, in order, are split into G
  contiguous runs of floor(p*W/G) .. floor((p+1)*W/G) (W = their slab
  count), so every run is shorter than one tile.  A tile whose slabs fall
  into several runs is summed from the runs' partial results in slab order.
"""
from __future__ import annotations

import random
from typing import Dict, List, Sequence, Tuple

BLOCKED = "blocked"
INTERLEAVED = "interleaved"
GROUPED = "grouped"
WORK_STEALING = "work_stealing"
BLOCKED_GROUPED = "blocked_grouped"
STREAM_K = "stream_k"
WORK_STEALING_XCC = "work_stealing_xcc"
STATIC_KINDS = (BLOCKED, INTERLEAVED, GROUPED, BLOCKED_GROUPED)


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def plain_decode(v: int, num_pid_m: int) -> Tuple[int, int]:
    return v % num_pid_m, v // num_pid_m


def grouped_decode(v: int, num_pid_m: int, num_pid_n: int, gs: int) -> Tuple[int, int]:
    num_pid_in_group = gs * num_pid_n
    group_id = v // num_pid_in_group
    first_pid_m = group_id * gs
    group_size_m = min(num_pid_m - first_pid_m, gs)
    pid_m = first_pid_m + (v % num_pid_in_group) % group_size_m
    pid_n = (v % num_pid_in_group) // group_size_m
    return pid_m, pid_n


def blocked_vpids(p: int, T: int, G: int) -> List[int]:
    bs = cdiv(T, G)
    start = p * bs
    end = min(start + bs, T)
    return list(range(start, end))


def interleaved_vpids(p: int, T: int, G: int) -> List[int]:
    return list(range(p, T, G))


def decode(kind: str, v: int, num_pid_m: int, num_pid_n: int, gs: int) -> Tuple[int, int]:
    if kind in (BLOCKED, INTERLEAVED):
        return plain_decode(v, num_pid_m)
    return grouped_decode(v, num_pid_m, num_pid_n, gs)


def static_schedule(kind: str, num_pid_m: int, num_pid_n: int, G: int,
                    gs: int = 8) -> List[List[Tuple[int, int, int]]]:
    """Per program p, the ordered list of (v, pid_m, pid_n) it computes."""
    T = num_pid_m * num_pid_n
    out = []
    for p in range(G):
        if kind in (BLOCKED, BLOCKED_GROUPED):
            vs = blocked_vpids(p, T, G)
        elif kind in (INTERLEAVED, GROUPED):
            vs = interleaved_vpids(p, T, G)
        else:
            raise ValueError(kind)
        out.append([(v,) + decode(kind, v, num_pid_m, num_pid_n, gs) for v in vs])
    return out


def multi_offsets(grids: Sequence[Tuple[int, int]]) -> List[int]:
    """Prefix sums of the problems' tile counts: problem g owns virtual ids
    [offsets[g], offsets[g + 1])."""
    out = [0]
    for pm, pn in grids:
        out.append(out[-1] + pm * pn)
    return out


def multi_decode(kind: str, v: int, grids: Sequence[Tuple[int, int]], gs: int = 8) -> Tuple[int, int, int]:
    """Virtual id v of the shared space -> (problem, pid_m, pid_n)."""
    off = multi_offsets(grids)
    g = 0
    while v >= off[g + 1]:           # the ids of the problems before g are skipped
        g += 1
    pm, pn = grids[g]
    return (g,) + decode(kind, v - off[g], pm, pn, gs)


def multi_static_schedule(kind: str, grids: Sequence[Tuple[int, int]], G: int,
                          gs: int = 8) -> List[List[Tuple[int, int, int, int]]]:
    """Per program p, the ordered (v, problem, pid_m, pid_n) it computes."""
    T = multi_offsets(grids)[-1]
    out = []
    for p in range(G):
        if kind in (BLOCKED, BLOCKED_GROUPED):
            vs = blocked_vpids(p, T, G)
        elif kind in (INTERLEAVED, GROUPED):
            vs = interleaved_vpids(p, T, G)
        else:
            raise ValueError(kind)
        out.append([(v,) + multi_decode(kind, v, grids, gs) for v in vs])
    return out


def check_multi_partition(seqs, grids: Sequence[Tuple[int, int]]) -> None:
    """Every tile of every problem computed exactly once."""
    seen = {}
    for p, seq in enumerate(seqs):
        for v, g, pm, pn in seq:
            if not (0 <= g < len(grids)) or not (0 <= pm < grids[g][0] and 0 <= pn < grids[g][1]):
                raise AssertionError(f"program {p}: tile {(g, pm, pn)} outside its problem")
            if (g, pm, pn) in seen:
                raise AssertionError(f"tile {(g, pm, pn)} computed by {seen[(g, pm, pn)]} and {p}")
            seen[(g, pm, pn)] = p
    want = sum(pm * pn for pm, pn in grids)
    if len(seen) != want:
        raise AssertionError(f"{want - len(seen)} tiles never computed")


def ws_ranges(T: int, X: int) -> List[Tuple[int, int]]:
    return [((x * T) // X, ((x + 1) * T) // X) for x in range(X)]


def ws_programs_per_xcd(G: int, X: int) -> List[int]:
    return [sum(1 for p in range(G) if p % X == x) for x in range(X)]


def ws_rounds(T: int, G: int, X: int) -> int:
    """Rounds of tiles the busiest program of per-XCD work stealing takes at
    equal tile times: the most, over the XCDs, of ceil(range length /
    programs on that counter) (counter p mod X)."""
    return max(cdiv(e - b, w) if w else (0 if e == b else 10**9)
               for (b, e), w in zip(ws_ranges(T, X), ws_programs_per_xcd(G, X)))


def balanced_grid(T: int, G: int, X: int) -> int:
    """Default grid of the data-parallel GEMM schedulers, by its definition:
    the smallest multiple of X, at most G, under which per-XCD work stealing
    takes no more rounds than under G programs (searched one multiple at a
    time).  G when T < 1, G < X or G is not a multiple of X."""
    if T < 1 or G < X or G % X:
        return G
    want = ws_rounds(T, G, X)
    for g in range(X, G + 1, X):
        if ws_rounds(T, g, X) <= want:
            return g
    return G


def ws_final_counters(T: int, G: int, X: int, chunk=1) -> List[int]:
    """Counter values after a complete launch: every successful claim and
    exactly one failing claim per program each added ``chunk`` (under
    PAIRS the counter counts claims)."""
    out = []
    for (s, e), w in zip(ws_ranges(T, X), ws_programs_per_xcd(G, X)):
        n = e - s
        out.append(pair_claims(n, G, X) + w if chunk == PAIRS else chunk * (cdiv(n, chunk) + w))
    return out


PAIRS = "pairs"


def pair_span(n: int, G: int, X: int) -> int:
    """Paired claims: the first L tiles of a range of n go out in pairs."""
    P = cdiv(G, X)
    return 2 * min(n // 2, P * (cdiv(n, P) // 2))


def pair_claims(n: int, G: int, X: int) -> int:
    """Paired claims: successful claims a range of n tiles hands out."""
    L = pair_span(n, G, X)
    return L // 2 + (n - L)


def pair_claim(k: int, n: int, G: int, X: int):
    """Paired claims: tiles [first, end) of claim k (counted from 0) of a
    range of n tiles, relative to the range's start, or None past the end."""
    L = pair_span(n, G, X)
    if k < L // 2:
        return 2 * k, 2 * k + 2
    t = L + (k - L // 2)
    return (t, t + 1) if t < n else None


def _take(chunk, cnt, x, n, G, X):
    """One claim on counter x: the tiles it gets, relative to the range's
    start, as (first, end), or None when the range is exhausted."""
    if chunk == PAIRS:
        k = cnt[x]
        cnt[x] += 1
        return pair_claim(k, n, G, X)
    i = cnt[x]
    cnt[x] += chunk
    return (i, min(i + chunk, n)) if i < n else None


def ws_simulate(num_pid_m: int, num_pid_n: int, G: int, X: int, gs: int = 8,
                chunk=1, seed: int = 0, speeds: Sequence[float] = None, claims_out=None):
    """One possible work-stealing execution.

    Programs run concurrently; the interleaving is drawn at random (or, with
    ``speeds``, the program with the earliest finish time claims next).
    ``chunk`` is the tiles per claim, or PAIRS.  ``claims_out``, a list,
    receives per program the claims it made on each counter ([G][X]).
    Returns (per-program list of (v, pid_m, pid_n), final counters)."""
    T = num_pid_m * num_pid_n
    if G < X:
        raise ValueError("work stealing needs at least one program per XCD")
    ranges = ws_ranges(T, X)
    cnt = [0] * X
    made = [[0] * X for _ in range(G)]
    seqs: List[List[Tuple[int, int, int]]] = [[] for _ in range(G)]
    active = list(range(G))
    clock = [0.0] * G
    r = random.Random(seed)
    while active:
        if speeds is None:
            p = r.choice(active)
        else:
            p = min(active, key=lambda q: (clock[q], q))
        x = p % X
        s, e = ranges[x]
        made[p][x] += 1
        got = _take(chunk, cnt, x, e - s, G, X)
        if got is None:
            active.remove(p)
            continue
        for v in range(s + got[0], s + got[1]):
            seqs[p].append((v,) + grouped_decode(v, num_pid_m, num_pid_n, gs))
        if speeds is not None:
            clock[p] += speeds[p] * (got[1] - got[0])
    if claims_out is not None:
        claims_out[:] = made
    return seqs, cnt


def ws_owner(v: int, T: int, X: int) -> int:
    """Counter (XCD range) that holds tile id v."""
    for x, (s, e) in enumerate(ws_ranges(T, X)):
        if s <= v < e:
            return x
    raise ValueError(f"tile {v} outside [0, {T})")


def wsx_counter_bounds(T: int, G: int, X: int, homes: Sequence[int],
                       chunk=1) -> List[Tuple[int, int]]:
    """Bounds on the counters after a complete launch of work stealing across
    XCDs: every successful claim and each program's failing claim on its
    home counter (lower), plus at most one failing claim per program on
    every other counter (upper); each claim adds ``chunk`` (under PAIRS the
    counter counts claims)."""
    out = []
    for x, (s, e) in enumerate(ws_ranges(T, X)):
        n = e - s
        at_home = sum(1 for h in homes if h % X == x)
        if chunk == PAIRS:
            out.append((pair_claims(n, G, X) + at_home, pair_claims(n, G, X) + G))
        else:
            claims = cdiv(n, chunk)
            out.append((chunk * (claims + at_home), chunk * (claims + G)))
    return out


def wsx_simulate(num_pid_m: int, num_pid_n: int, G: int, X: int, homes: Sequence[int],
                 gs: int = 8, chunk=1, seed: int = 0, speeds: Sequence[float] = None,
                 claims_out=None):
    """One possible execution of work stealing across XCDs.  ``homes[p]`` is
    the counter program p starts on.  The interleaving is random, or with
    ``speeds`` the program with the earliest clock (then the lowest id)
    claims next; a failing claim takes no time.  ``claims_out``, a list,
    receives per program the claims it made on each counter ([G][X]).
    Returns (per-program list of (v, pid_m, pid_n), final counters)."""
    T = num_pid_m * num_pid_n
    ranges = ws_ranges(T, X)
    cnt = [0] * X
    made = [[0] * X for _ in range(G)]
    seqs: List[List[Tuple[int, int, int]]] = [[] for _ in range(G)]
    cur = [homes[p] % X for p in range(G)]
    passed = [0] * G
    active = list(range(G))
    clock = [0.0] * G
    r = random.Random(seed)
    while active:
        if speeds is None:
            p = r.choice(active)
        else:
            p = min(active, key=lambda q: (clock[q], q))
        x = cur[p]
        s, e = ranges[x]
        made[p][x] += 1
        got = _take(chunk, cnt, x, e - s, G, X)
        if got is None:
            passed[p] += 1
            nxt = None
            for j in range(X - passed[p]):          # counters not passed yet, in order
                c = (x + 1 + j) % X
                cs, ce = ranges[c]
                left = pair_claims(ce - cs, G, X) if chunk == PAIRS else ce - cs
                if cnt[c] < left:
                    nxt = (j, c)
                    break
            if nxt is None:
                active.remove(p)
            else:
                passed[p] += nxt[0]
                cur[p] = nxt[1]
            continue
        for v in range(s + got[0], s + got[1]):
            seqs[p].append((v,) + grouped_decode(v, num_pid_m, num_pid_n, gs))
        if speeds is not None:
            clock[p] += speeds[p] * (got[1] - got[0])
    if claims_out is not None:
        claims_out[:] = made
    return seqs, cnt


def claim_of(i: int, n: int, G: int, X: int, chunk=1) -> int:
    """The claim (counted from 0) that hands out tile i (relative to the
    start) of a counter range of n tiles: claims of ``chunk`` consecutive
    tiles, or under PAIRS the pair / single-tile claims of pair_claim."""
    if chunk == PAIRS:
        L = pair_span(n, G, X)
        return i // 2 if i < L else L // 2 + (i - L)
    return i // chunk


def check_claim_counts(claims: Sequence[Sequence[int]], owner: Sequence[int],
                       counters: Sequence[int], homes: Sequence[int], T: int, G: int, X: int,
                       chunk=1, across: bool = False) -> None:
    """Claim accounting of a complete work-stealing launch.  claims[p][c] is
    the number of claims (counter increments) program p made on counter c;
    owner[v] the program that computed tile v; homes[p] the counter program p
    started on.  Every claim adds one step (``chunk`` tiles, one under PAIRS)
    to its counter, so each final counter is the step times the claims made
    on it.  The claims of p on c that handed out no tile are its failing
    claims there: exactly one on its home counter (claims go on there until
    one fails), and on any other counter none (per-XCD work stealing) or at
    most one (across XCDs: each counter not yet passed is claimed from at
    most once more after it was seen not exhausted)."""
    step = 1 if chunk == PAIRS else chunk
    got: List[List[set]] = [[set() for _ in range(X)] for _ in range(G)]
    for x, (s, e) in enumerate(ws_ranges(T, X)):
        for v in range(s, e):
            got[owner[v]][x].add(claim_of(v - s, e - s, G, X, chunk))
    for c in range(X):
        made = sum(claims[p][c] for p in range(G))
        if counters[c] != step * made:
            raise AssertionError(f"counter {c} ended at {counters[c]}, the claims on it add {step * made}")
    for p in range(G):
        for c in range(X):
            fails = claims[p][c] - len(got[p][c])
            if c == homes[p] % X:
                if fails != 1:
                    raise AssertionError(f"program {p}: {fails} failing claims on its home counter {c}")
            elif fails < 0 or fails > (1 if across else 0):
                raise AssertionError(f"program {p}: {fails} failing claims on counter {c} (home {homes[p] % X})")


def check_wsx_execution(visits: Sequence[int], owner: Sequence[int], local_order: Sequence[int],
                        counters: Sequence[int], homes: Sequence[int], T: int, G: int, X: int,
                        chunk=1, claims=None) -> None:
    """Invariants of every correct launch of work stealing across XCDs.
    visits / owner / local_order are indexed by tile id; homes[p] is the
    counter program p started on; claims[p][c], if given, the claims p made
    on counter c (check_claim_counts, which fixes each final counter
    exactly)."""
    for v in range(T):
        if visits[v] != 1:
            raise AssertionError(f"tile {v} visited {visits[v]} times")
        if not (0 <= owner[v] < G):
            raise AssertionError(f"tile {v} computed by program {owner[v]}")
    by_prog: Dict[int, List[Tuple[int, int]]] = {}
    for v in range(T):
        by_prog.setdefault(owner[v], []).append((local_order[v], v))
    for p, lst in by_prog.items():
        lst.sort()
        orders = [o for o, _ in lst]
        if orders != list(range(len(lst))):
            raise AssertionError(f"program {p}: local order {orders} not 0..n-1")
        # counters are visited in the cyclic order from home, and the tiles
        # taken from one counter rise
        key = [((ws_owner(v, T, X) - homes[p]) % X, v) for _, v in lst]
        if any(b <= a for a, b in zip(key, key[1:])):
            raise AssertionError(f"program {p} (home {homes[p]}): tiles out of claim order "
                                 f"{[v for _, v in lst]}")
    for x, (lo, hi) in enumerate(wsx_counter_bounds(T, G, X, homes, chunk)):
        if not (lo <= counters[x] <= hi):
            raise AssertionError(f"counter {x} ended at {counters[x]}, outside [{lo}, {hi}]")
    if claims is not None:
        check_claim_counts(claims, owner, counters, homes, T, G, X, chunk, across=True)


def check_partition(seqs: Sequence[Sequence[Tuple[int, int, int]]],
                    num_pid_m: int, num_pid_n: int) -> None:
    """Every tile id in [0, T) and every (pid_m, pid_n) appears exactly once."""
    T = num_pid_m * num_pid_n
    seen_v: Dict[int, int] = {}
    seen_mn: Dict[Tuple[int, int], int] = {}
    for p, seq in enumerate(seqs):
        for v, pm, pn in seq:
            if not (0 <= v < T):
                raise AssertionError(f"program {p}: tile id {v} outside [0, {T})")
            if not (0 <= pm < num_pid_m and 0 <= pn < num_pid_n):
                raise AssertionError(f"program {p}: tile ({pm},{pn}) outside the grid")
            if v in seen_v:
                raise AssertionError(f"tile id {v} computed by {seen_v[v]} and {p}")
            if (pm, pn) in seen_mn:
                raise AssertionError(f"tile {(pm, pn)} computed twice")
            seen_v[v] = p
            seen_mn[(pm, pn)] = p
    if len(seen_v) != T or len(seen_mn) != T:
        raise AssertionError(f"{T - len(seen_mn)} tiles never computed")


def check_ws_execution(visits: Sequence[int], owner: Sequence[int],
                       local_order: Sequence[int], counters: Sequence[int],
                       T: int, G: int, X: int, chunk=1, claims=None) -> None:
    """Invariants every correct work-stealing launch satisfies (the exact
    assignment depends on timing).  Arrays are indexed by tile id v:
    visits[v] = times computed, owner[v] = program, local_order[v] = its
    position in that program's sequence; claims[p][c], if given, the claims
    program p made on counter c (check_claim_counts)."""
    ranges = ws_ranges(T, X)
    for v in range(T):
        if visits[v] != 1:
            raise AssertionError(f"tile {v} visited {visits[v]} times")
    for x, (s, e) in enumerate(ranges):
        for v in range(s, e):
            if owner[v] % X != x or not (0 <= owner[v] < G):
                raise AssertionError(f"tile {v} of XCD {x} computed by program {owner[v]}")
    # claims of one program come from one counter, so its tiles rise with its order
    by_prog: Dict[int, List[Tuple[int, int]]] = {}
    for v in range(T):
        by_prog.setdefault(owner[v], []).append((local_order[v], v))
    for p, lst in by_prog.items():
        lst.sort()
        orders = [o for o, _ in lst]
        if orders != list(range(len(lst))):
            raise AssertionError(f"program {p}: local order {orders} not 0..n-1")
        vs = [v for _, v in lst]
        if any(b <= a for a, b in zip(vs, vs[1:])):
            raise AssertionError(f"program {p}: tiles not increasing {vs}")
    want = ws_final_counters(T, G, X, chunk)
    if list(counters[:X]) != want:
        raise AssertionError(f"final counters {list(counters[:X])} != {want}")
    if claims is not None:
        check_claim_counts(claims, owner, counters, [p % X for p in range(G)], T, G, X, chunk)


def streamk_dp_tiles(T: int, G: int) -> int:
    """Tiles taken whole (data-parallel) before the stream-K part: every
    full wave of G tiles."""
    return (T // G) * G


def streamk_schedule(T: int, nk: int, G: int) -> List[List[Tuple[int, int, int]]]:
    """Per program, its segments (tile id, first slab, end slab) in order."""
    dp = streamk_dp_tiles(T, G)
    W = (T - dp) * nk
    out: List[List[Tuple[int, int, int]]] = []
    for p in range(G):
        segs = [(v, 0, nk) for v in range(p, dp, G)]
        i, end = dp * nk + (p * W) // G, dp * nk + ((p + 1) * W) // G
        while i < end:
            v, kb = divmod(i, nk)
            ke = min(nk, kb + end - i)
            segs.append((v, kb, ke))
            i += ke - kb
        out.append(segs)
    return out


def streamk_partials(T: int, nk: int, G: int) -> Dict[int, List[Tuple[int, int, int]]]:
    """Tiles split over several programs: tile -> [(program, first slab, end
    slab)] in slab order (the order the partial results are summed in)."""
    parts: Dict[int, List[Tuple[int, int, int]]] = {}
    for p, segs in enumerate(streamk_schedule(T, nk, G)):
        for v, kb, ke in segs:
            if kb != 0 or ke != nk:
                parts.setdefault(v, []).append((p, kb, ke))
    for v in parts:
        parts[v].sort(key=lambda t: t[1])
    return parts


def check_streamk_cover(sched: Sequence[Sequence[Tuple[int, int, int]]], T: int, nk: int) -> None:
    """Every (tile, slab) pair is computed exactly once."""
    seen: Dict[Tuple[int, int], int] = {}
    for p, segs in enumerate(sched):
        for v, kb, ke in segs:
            if not (0 <= v < T and 0 <= kb < ke <= nk):
                raise AssertionError(f"program {p}: bad segment {(v, kb, ke)}")
            for k in range(kb, ke):
                if (v, k) in seen:
                    raise AssertionError(f"tile {v} slab {k} computed by {seen[(v, k)]} and {p}")
                seen[(v, k)] = p
    if len(seen) != T * nk:
        raise AssertionError(f"{T * nk - len(seen)} (tile, slab) pairs never computed")
