"""The clamped sequence layout of the prefill kernels (gdn_seqmap.h), on the
CPU: the same header the kernels include is compiled into a host probe and
fed well-formed and malformed device offsets.  Whatever the offsets hold,
every range lies inside [0, T], the ranges are disjoint and ordered, and the
chunk slots they need fit the workspace's T / C + N; well-formed offsets pass
through unchanged.  No GPU is used."""
import os
import random
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE_SRC = os.path.join(ROOT, "tests", "seqmap_probe.hip")
INT32_MIN, INT32_MAX = -2 ** 31, 2 ** 31 - 1


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("seqmap") / "seqmap_probe")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950",
                           "-O1", "-std=c++17", PROBE_SRC, "-o", exe],
                          stderr=subprocess.DEVNULL)
    return exe


def run(exe, cases):
    lines = []
    for N, T, seq_len, cu, C in cases:
        lines.append("%d %d %d %d %d" % (N, T, seq_len, 0 if cu is None else 1, C))
        if cu is not None:
            lines.append(" ".join(str(v) for v in cu))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", text=True,
                         capture_output=True, check=True).stdout.splitlines()
    res = []
    for (N, T, seq_len, cu, C), line in zip(cases, out):
        v = [int(t) for t in line.split()]
        beg, end = v[0:2 * N:2], v[1:2 * N:2]
        prefix = v[2 * N:3 * N + 1]
        lb, le = v[3 * N + 1::2], v[3 * N + 2::2]
        res.append((beg, end, prefix, lb, le))
    return res


def reference(N, T, seq_len, cu, C):
    """The clamp rule written out: beg_n = clamp(cu[n], end_{n-1}, T),
    end_n = clamp(cu[n+1], beg_n, T)."""
    beg, end, prefix = [], [], [0]
    prev = 0
    for n in range(N):
        b = cu[n] if cu is not None else n * seq_len
        e = cu[n + 1] if cu is not None else b + seq_len
        b = min(max(b, prev), T)
        e = min(max(e, b), T)
        beg.append(b)
        end.append(e)
        prefix.append(prefix[-1] + (e - b + C - 1) // C)
        prev = e
    return beg, end, prefix


def check(case, got):
    N, T, seq_len, cu, C = case
    beg, end, prefix, lb, le = got
    assert (beg, end, prefix) == reference(N, T, seq_len, cu, C), case
    prev = 0
    for b, e in zip(beg, end):
        assert prev <= b <= e <= T
        prev = e
    assert prefix[0] == 0 and prefix[-1] <= T // C + N
    for b, e in zip(lb, le):
        assert 0 <= b <= e <= T


def test_well_formed_offsets_pass_through(probe):
    rng = random.Random(1)
    cases = []
    for _ in range(200):
        N = rng.randint(1, 12)
        lens = [rng.choice([0, 1, 63, 64, 65, rng.randint(0, 3000)]) for _ in range(N)]
        cu = [0]
        for l in lens:
            cu.append(cu[-1] + l)
        cases.append((N, cu[-1], 0, cu, 64))
    cases.append((8, 131048, 0, [0, 1024, 3072, 7168, 15360, 31744, 64512,
                                 130048, 131048], 64))
    cases.append((4, 400, 100, None, 64))        # even split, no offsets
    for case, got in zip(cases, run(probe, cases)):
        check(case, got)
        beg, end, _, lb, le = got
        if case[3] is not None:
            assert beg == case[3][:-1] and end == case[3][1:]
            assert lb == case[3][:-1] and le == case[3][1:]


def test_malformed_offsets_stay_in_bounds(probe):
    rng = random.Random(2)
    special = [INT32_MIN, -1, 0, 1, 63, 64, 65, INT32_MAX]
    cases = []
    for _ in range(400):
        N = rng.randint(1, 10)
        T = rng.choice([0, 1, 64, 100, 4096, 70000])
        cu = [rng.choice(special + [rng.randint(-5000, 80000)]) for _ in range(N + 1)]
        cases.append((N, T, 0, cu, 64))
    # decreasing, overlapping, and all-huge offsets
    cases.append((3, 200, 0, [0, 150, 50, 200], 64))
    cases.append((3, 200, 0, [300, 300, 300, 300], 64))
    cases.append((2, 200, 0, [INT32_MAX, INT32_MIN, INT32_MAX], 64))
    for case, got in zip(cases, run(probe, cases)):
        check(case, got)
