"""The library's scheduler header, built for the host with g++, against the
oracle's schedule model: static walks tile for tile, and the work-stealing
claim loops (per-XCD, and across XCDs from arbitrary home counters) on real
threads with std::atomic counters against the model's invariants, and the
stream-K walker segment for segment."""
import itertools
import os
import subprocess

import pytest

from oracle import sched_model as sm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KINDS = {"blocked": 0, "interleaved": 1, "grouped": 2, "blocked_grouped": 4}


SRC = os.path.join(ROOT, "tests", "host", "sched_host.cpp")
# Sanitizer builds of the host harness (g++, CPU code only): ThreadSanitizer
# for the claim loops on real threads, AddressSanitizer + UndefinedBehavior-
# Sanitizer for every mode; any report aborts the run.
SANITIZERS = {"thread": ["-fsanitize=thread"],
              "address,undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]}
SAN_ENV = {"TSAN_OPTIONS": "halt_on_error=1:exitcode=66", "ASAN_OPTIONS": "detect_leaks=1:exitcode=66",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _build(tmp_path_factory, name, flags):
    exe = str(tmp_path_factory.mktemp("sched") / name)
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Werror", "-pthread", *flags, SRC, "-o", exe],
                   check=True)
    return exe


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    return _build(tmp_path_factory, "sched_host", [])


@pytest.fixture(scope="module", params=sorted(SANITIZERS))
def sanitized(request, tmp_path_factory):
    return request.param, _build(tmp_path_factory, "sched_host_" + request.param.replace(",", "_"),
                                 SANITIZERS[request.param])


def _run_sanitized(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True,
                       env={**os.environ, **SAN_ENV})
    assert r.returncode == 0 and "Sanitizer" not in r.stderr, (args, r.returncode, r.stderr[-3000:])
    return r.stdout.strip().splitlines()


def _static(exe, kind, pm, pn, G, gs):
    out = subprocess.run([exe, "static", str(KINDS[kind]), str(pm), str(pn), str(G), str(gs)],
                         check=True, capture_output=True, text=True).stdout
    seqs = []
    for line in out.strip().splitlines():
        _, _, rest = line.partition(":")
        seqs.append([tuple(map(int, t.split(","))) for t in rest.split()])
    return seqs


@pytest.mark.parametrize("kind", list(KINDS))
def test_static_walk_matches_model(harness, kind):
    for (pm, pn), G, gs in itertools.product([(1, 1), (5, 2), (13, 23), (32, 32), (20, 20), (19, 32)],
                                             [1, 7, 8, 256], [1, 3, 8, 16]):
        got = _static(harness, kind, pm, pn, G, gs)
        assert got == sm.static_schedule(kind, pm, pn, G, gs), (kind, pm, pn, G, gs)


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(5, 2, 8, 4, 1), (32, 32, 256, 8, 1),
                                             (19, 32, 256, 8, 1), (33, 7, 64, 8, 4),
                                             (1, 1, 16, 8, 1), (19, 32, 256, 8, -1),
                                             (20, 20, 256, 8, -1), (5, 2, 4, 2, -1)])
def test_ws_threads_satisfy_model_invariants(harness, pm, pn, G, X, chunk):
    out = subprocess.run([harness, "ws", str(pm), str(pn), str(G), str(X), "8", str(chunk)],
                         check=True, capture_output=True, text=True).stdout.strip().splitlines()
    _check_ws(out, pm, pn, G, X, chunk)


def _claims(out, G, X):
    """The harness's last line: the claims each thread made on each counter."""
    assert out[-1].startswith("claims:")
    made = list(map(int, out[-1].split(":")[1].split()))
    assert len(made) == G * X
    return [made[p * X:(p + 1) * X] for p in range(G)]


def _check_ws(out, pm, pn, G, X, chunk):
    homes = list(map(int, out[0].split(":")[1].split()))
    assert homes == [p % X for p in range(G)]
    counters = list(map(int, out[1].split(":")[1].split()))
    T = pm * pn
    rows = [tuple(map(int, l.split())) for l in out[2:-1]]
    assert len(rows) == T
    visits = [r[1] for r in rows]
    owner = [r[2] for r in rows]
    order = [r[3] for r in rows]
    sm.check_ws_execution(visits, owner, order, counters, T, G, X, sm.PAIRS if chunk < 0 else chunk,
                          claims=_claims(out, G, X))


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(5, 2, 8, 4, 1), (32, 32, 256, 8, 1), (19, 32, 256, 8, 1),
                                             (33, 7, 64, 8, 4), (1, 1, 16, 8, 1), (3, 1, 5, 8, 1),
                                             (13, 11, 3, 8, 2), (19, 32, 256, 8, -1), (13, 11, 3, 8, -1)])
@pytest.mark.parametrize("home_mode", [0, 1, 2])
def test_wsx_threads_satisfy_model_invariants(harness, pm, pn, G, X, chunk, home_mode):
    out = subprocess.run([harness, "wsx", str(pm), str(pn), str(G), str(X), str(chunk), str(home_mode)],
                         check=True, capture_output=True, text=True).stdout.strip().splitlines()
    _check_wsx(out, pm, pn, G, X, chunk)


def _check_wsx(out, pm, pn, G, X, chunk):
    homes = list(map(int, out[0].split(":")[1].split()))
    counters = list(map(int, out[1].split(":")[1].split()))
    T = pm * pn
    rows = [tuple(map(int, l.split())) for l in out[2:-1]]
    assert len(rows) == T and len(homes) == G
    sm.check_wsx_execution([r[1] for r in rows], [r[2] for r in rows], [r[3] for r in rows],
                           counters, homes, T, G, X, sm.PAIRS if chunk < 0 else chunk,
                           claims=_claims(out, G, X))


@pytest.mark.parametrize("T,nk,G", [(10, 4, 4), (16, 3, 4), (1, 7, 8), (7, 1, 8), (608, 128, 256),
                                    (400, 64, 256), (448, 64, 512), (3, 5, 256), (300, 2, 7),
                                    (1024, 128, 256)])
def test_streamk_walk_matches_model(harness, T, nk, G):
    out = subprocess.run([harness, "sk", str(T), str(nk), str(G)], check=True, capture_output=True,
                         text=True).stdout.strip().splitlines()
    segs = [l for l in out if not l.startswith("split")]
    got = []
    slots = {}
    for p, line in enumerate(segs):
        _, _, rest = line.partition(":")
        lst = [tuple(map(int, t.split(","))) for t in rest.split()]
        got.append([(v, kb, ke) for v, kb, ke, _ in lst])
        for v, kb, ke, slot in lst:
            assert (slot >= 0) == (kb != 0 or ke != nk)
            if slot >= 0:
                slots[(p, v)] = slot
    assert got == sm.streamk_schedule(T, nk, G)
    # the split tiles and, for each, its contributors in slab order with the
    # slot each one wrote its partial sum to
    want = {v: [(q, slots[(q, v)]) for q, _, _ in parts]
            for v, parts in sm.streamk_partials(T, nk, G).items()}
    split = {}
    for line in (l for l in out if l.startswith("split")):
        head, _, rest = line.partition(":")
        split[int(head.split()[1])] = [tuple(map(int, t.split(","))) for t in rest.split()]
    assert split == want


def test_pair_claim_map_matches_model(harness):
    out = subprocess.run([harness, "pairs", "256", "8"], check=True, capture_output=True,
                         text=True).stdout.strip().splitlines()
    for line in out:
        n, L, claims, *tiles = map(int, line.split())
        assert L == sm.pair_span(n, 256, 8) and claims == sm.pair_claims(n, 256, 8), n
        want = [t for k in range(claims) for t in sm.pair_claim(k, n, 256, 8)]
        assert tiles == want, n


@pytest.mark.parametrize("G,X", [(256, 8), (512, 8), (64, 4), (13, 8), (8, 8), (7, 8), (32, 1)])
def test_balanced_grid_matches_model(harness, G, X):
    """The library's default GEMM grid equals the oracle's search over
    multiples of X for every tile count up to 3000."""
    out = subprocess.run([harness, "grid", "3000", str(G), str(X)], check=True, capture_output=True,
                         text=True).stdout.strip().splitlines()
    assert len(out) == 3001
    for line in out:
        T, g = map(int, line.split())
        assert g == sm.balanced_grid(T, G, X), (T, G, X, g)


@pytest.mark.parametrize("G,X", [(256, 8), (224, 8), (8, 8), (64, 4), (250, 8), (7, 8), (96, 1), (1, 1)])
def test_program_order(harness, G, X):
    """XCD-major program numbering: a bijection of the grid; with X > 1
    dividing G, the workgroups the hardware places on XCD x (ids = x mod X,
    round robin) play exactly programs [x*G/X, (x+1)*G/X), in workgroup
    order; otherwise, and with the option off, workgroup i plays program i."""
    for xm in (0, 1):
        out = subprocess.run([harness, "order", str(G), str(X), str(xm)], check=True, capture_output=True,
                             text=True).stdout.strip().splitlines()
        prog = [int(line.split()[1]) for line in out]
        assert [int(line.split()[0]) for line in out] == list(range(G))
        assert sorted(prog) == list(range(G))
        if xm and X > 1 and G % X == 0:
            per = G // X
            for x in range(X):
                assert [prog[hw] for hw in range(x, G, X)] == list(range(x * per, (x + 1) * per)), (G, X, x)
        else:
            assert prog == list(range(G))


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(32, 32, 256, 8, 1), (19, 32, 256, 8, -1), (33, 7, 64, 8, 4),
                                             (13, 11, 3, 8, 2)])
def test_claim_loops_under_sanitizers(sanitized, pm, pn, G, X, chunk):
    """The kernels' claim and sweep code on real threads, built with
    ThreadSanitizer and with AddressSanitizer + UndefinedBehaviorSanitizer:
    no report, and the executions still satisfy the model's invariants."""
    _, exe = sanitized
    if G >= X:  # per-XCD work stealing needs a program on every counter
        _check_ws(_run_sanitized(exe, "ws", pm, pn, G, X, 8, chunk), pm, pn, G, X, chunk)
    for home_mode in (0, 1, 2):
        _check_wsx(_run_sanitized(exe, "wsx", pm, pn, G, X, chunk, home_mode), pm, pn, G, X, chunk)


def test_other_modes_under_sanitizers(sanitized):
    name, exe = sanitized
    if name == "thread":
        pytest.skip("single-threaded modes: covered by the address / undefined build")
    for kind in KINDS.values():
        _run_sanitized(exe, "static", kind, 19, 32, 256, 8)
    assert len(_run_sanitized(exe, "pairs", 256, 8)) == 140
    assert len(_run_sanitized(exe, "grid", 3000, 256, 8)) == 3001
    assert len(_run_sanitized(exe, "order", 224, 8, 1)) == 224
    for T, nk, G in [(608, 128, 256), (3, 5, 256), (300, 2, 7)]:
        _run_sanitized(exe, "sk", T, nk, G)


def test_oracle_gemm_under_sanitizers(tmp_path):
    """The oracle's C GEMM built with AddressSanitizer + UndefinedBehavior-
    Sanitizer (and OpenMP), run on small and edge shapes against a plain loop."""
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "tests", "host", "oracle_sanitize.c"), "-o", exe, "-lm"], check=True)
    out = _run_sanitized(exe)
    assert out == ["mismatches: 0"]


def _check_wsr(out, pm, pn, G, X, chunk):
    """Self-resetting per-XCD work stealing: the reset value of each counter is
    the oracle's final counter value minus one step, every counter ends at
    zero, and the execution satisfies the model's invariants."""
    T = pm * pn
    c = sm.PAIRS if chunk < 0 else chunk
    step = 1 if chunk < 0 else chunk
    reset_at = list(map(int, out[0].split(":")[1].split()))
    final = sm.ws_final_counters(T, G, X, c)
    assert reset_at == [f - step for f in final], (reset_at, final)
    counters = list(map(int, out[2].split(":")[1].split()))
    assert counters == [0] * X
    rows = [tuple(map(int, l.split())) for l in out[3:-1]]
    sm.check_ws_execution([r[1] for r in rows], [r[2] for r in rows], [r[3] for r in rows],
                          final, T, G, X, c, claims=_claims(out, G, X))


@pytest.mark.parametrize("pm,pn,G,X,chunk", [(5, 2, 8, 4, 1), (32, 32, 256, 8, 1), (19, 32, 256, 8, 1),
                                             (33, 7, 64, 8, 4), (1, 1, 16, 8, 1), (19, 32, 256, 8, -1),
                                             (20, 20, 256, 8, -1), (5, 2, 4, 2, -1), (20, 20, 200, 8, 1),
                                             (7, 9, 13, 8, 1), (16, 25, 200, 8, 3)])
def test_ws_self_reset_leaves_counters_zero(harness, pm, pn, G, X, chunk):
    out = subprocess.run([harness, "wsr", str(pm), str(pn), str(G), str(X), str(chunk)],
                         check=True, capture_output=True, text=True).stdout.strip().splitlines()
    _check_wsr(out, pm, pn, G, X, chunk)


def test_ws_self_reset_under_sanitizers(sanitized):
    _, exe = sanitized
    for pm, pn, G, X, chunk in [(32, 32, 256, 8, 1), (19, 32, 256, 8, -1), (7, 9, 13, 8, 1)]:
        _check_wsr(_run_sanitized(exe, "wsr", pm, pn, G, X, chunk), pm, pn, G, X, chunk)
