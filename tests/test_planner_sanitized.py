"""The planner's C ABI under the address and undefined-behaviour sanitizers.

`planner_abi_driver.cpp` is built here with g++ together with the library's
host planner source. It makes every planner call with output buffers of
exactly the capacity a case gives. The cases are random and edge-case inputs:
two-call sizing, capacities too small by one, zero-length batches, null
arrays, lengths near INT32_MAX, token totals that overflow int32, and DCP
alignments that are not multiples of world * interleave. Every line the driver
prints is checked against the oracle planner, or against the documented error
code for inputs the ABI rejects. A sanitizer report makes the driver exit
non-zero, which fails the test.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
import oracle.dcp as OD
from tests.conftest import ROOT

OK, INVALID, CAPACITY = 0, 1, 2
I32_MAX = 2**31 - 1
CSRC = os.path.join(ROOT, "mla_chunked_context_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("planner_asan") / "planner_abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "planner_abi_driver.cpp"), os.path.join(CSRC, "planner.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    out = res.stdout.strip().splitlines()
    assert len(out) == len(lines)
    return out


# ---------------------------------------------------------------- expectations

def _expected_plan(ctx, q, budget, cap, align, world, il):
    """Oracle plan as the driver prints it, or None when the ABI must reject."""
    if any(c < 0 for c in ctx) or any(x < 0 for x in q) or sum(q) > I32_MAX or budget > I32_MAX:
        return None
    m = cap if cap > 0 else None
    try:
        if world == 0:
            plans = O.plan_mla_context_chunks(ctx, budget, m, align)
        else:
            if world < 1 or il < 1:
                return None
            plans = OD.plan_dcp_context_chunks(ctx, budget, align, world, il, m)
    except ValueError:
        return None
    qsl = np.concatenate([[0], np.cumsum(np.asarray(q, dtype=np.int64))]).astype(int).tolist()
    chunks, entries, local = [], [], []
    for pl in plans:
        rs, re_ = pl.request_start, pl.request_end
        if world == 0:
            rows = sum(pl.seq_lens)
        else:
            ls, lens, cu = OD.dcp_local_entries(pl, world, il)
            rows = world * int(cu[-1])
            local += [x for pair in zip(ls, lens) for x in pair]
        chunks.append([rs, re_, qsl[rs], qsl[re_], len(entries) // 2, len(pl.seq_lens), rows, max(pl.seq_lens),
                       max(q[rs:re_]), int(pl.starts[0] > 0)])
        entries += [x for pair in zip(pl.starts, pl.seq_lens) for x in pair]
    return chunks, entries, local


def _check_plan_line(line, case):
    ctx, q, budget, cap, align, world, il, ccap, ecap = case
    parts = line.split("|")
    head = parts[0].split()
    assert head[0] == "P"
    s1, nc1, ne1, s2, nc2, ne2 = map(int, head[1:7])
    exp = _expected_plan(ctx, q, budget, cap, align, world, il)
    if exp is None:
        assert (s1, nc1, ne1, s2, nc2, ne2) == (INVALID, -1, -1, INVALID, -1, -1), (line, case)
        assert head[7] == "-"
        return
    chunks, entries, local = exp
    nc, ne = len(chunks), len(entries) // 2
    assert (s1, nc1, ne1) == (OK if nc == 0 and ne == 0 else CAPACITY, nc, ne), (line, case)
    assert (s2, nc2, ne2) == (OK if nc <= ccap and ne <= ecap else CAPACITY, nc, ne), (line, case)
    assert int(head[7]) == OK
    got_chunks = [list(map(int, c.split())) for c in parts[1].split(";") if c.strip()]
    assert got_chunks == chunks, (case, got_chunks, chunks)
    assert list(map(int, parts[2].split())) == entries
    if world != 0:
        assert list(map(int, parts[3].split())) == local


def _check_tokens_line(line, ctx, q, ecap):
    head, tail = line.split("|")
    _, s, prefix, count = head.split()
    s, prefix, count = int(s), int(prefix), int(count)
    if any(c < 0 for c in ctx) or any(x < 0 for x in q) or sum(q) > I32_MAX:
        assert (s, prefix, count) == (INVALID, -1, -1)
        return
    qsl = np.concatenate([[0], np.cumsum(np.asarray(q, dtype=np.int64))]).astype(int).tolist()
    with_ctx = [r for r, c in enumerate(ctx) if c > 0]
    exp_prefix = qsl[with_ctx[-1] + 1] if with_ctx else 0
    empties = [(qsl[r], qsl[r + 1]) for r, c in enumerate(ctx) if c == 0]
    assert (s, prefix, count) == (OK if len(empties) <= ecap else CAPACITY, exp_prefix, len(empties))
    got = list(map(int, tail.split()))
    assert got == [x for e in empties[:ecap] for x in e]


def _check_windows_line(line, ctx, budget, align):
    _, s, w, it = line.split()
    s, w, it = int(s), int(w), int(it)
    if any(c < 0 for c in ctx) or budget < 1 or align < 1:
        assert (s, w, it) == (INVALID, -1, -1)
        return
    try:
        exp_w = O.uniform_window_size(ctx, budget, align)
    except ValueError:
        assert s == INVALID
        return
    exp_it = math.ceil(max(ctx) / exp_w) if exp_w else 0
    assert (s, w, it) == (OK, exp_w, exp_it)


# ---------------------------------------------------------------- case generation

def _plan_cases(rng):
    cases = []
    worlds = [(0, 1), (0, 1), (1, 1), (2, 1), (4, 1), (2, 4), (8, 2), (3, 1)]
    for i in range(700):
        world, il = worlds[int(rng.integers(0, len(worlds)))]
        step = world * il if world else 1
        align = step * int(rng.choice([1, 2, 16])) if rng.random() < 0.9 else int(rng.choice([1, 3, 7, 0, -4]))
        n = int(rng.integers(0, 10))
        ctx = [0 if rng.random() < 0.25 else int(rng.integers(1, 3000)) for _ in range(n)]
        q = [int(rng.integers(0, 40)) for _ in range(n)]
        budget = int(rng.integers(1, 4000)) if rng.random() < 0.9 else int(rng.choice([0, -1, 2**31]))
        cap = 0 if rng.random() < 0.6 else int(rng.integers(-5, 2000))
        if rng.random() < 0.05 and n:
            ctx[int(rng.integers(0, n))] = -1
        if rng.random() < 0.05 and n:
            q[int(rng.integers(0, n))] = -3
        exp = _expected_plan(ctx, q, budget, cap, align, world, il)
        need_c, need_e = (len(exp[0]), len(exp[1]) // 2) if exp else (3, 3)
        # capacities: exact, one short, generous or zero
        ccap = max(0, need_c + int(rng.choice([0, -1, 2, -need_c])))
        ecap = max(0, need_e + int(rng.choice([0, -1, 3, -need_e])))
        cases.append((ctx, q, budget, cap, align, world, il, ccap, ecap))
    # lengths near the int32 limit; budgets keep the chunk count small, and a
    # 2^20 alignment keeps the oracle's candidate scan short
    big = [I32_MAX, I32_MAX - 1, 2**30 + 7, 2**31 - 64]
    for c0 in big:
        for budget in (2**30, I32_MAX, 2**29 + 2**20):
            for world, il in ((0, 1), (2, 1), (4, 2)):
                align = 2**20
                ctx, q = [c0, 5, c0 // 3], [1, 2, 3]
                exp = _expected_plan(ctx, q, budget, 0, align, world, il)
                need_c, need_e = (len(exp[0]), len(exp[1]) // 2) if exp else (0, 0)
                cases.append((ctx, q, budget, 0, align, world, il, need_c, max(0, need_e - 1)))
    # token totals past int32
    cases.append(([10, 10], [I32_MAX, 1], 64, 0, 16, 0, 1, 4, 4))
    cases.append(([10, 10], [2**30, 2**30], 64, 0, 16, 2, 1, 4, 4))
    cases.append(([], [], 64, 0, 16, 0, 1, 0, 0))
    cases.append(([0, 0, 0], [1, 2, 3], 64, 0, 16, 4, 1, 0, 0))
    return cases


def test_planner_abi_under_sanitizers(driver):
    rng = np.random.default_rng(2024)
    plan_cases = _plan_cases(rng)
    token_cases, window_cases = [], []
    for _ in range(300):
        n = int(rng.integers(0, 12))
        ctx = [0 if rng.random() < 0.4 else int(rng.integers(1, 100)) for _ in range(n)]
        q = [int(rng.integers(0, 50)) for _ in range(n)]
        if rng.random() < 0.05 and n:
            q[0] = -1
        n_empty = sum(c == 0 for c in ctx)
        token_cases.append((ctx, q, max(0, n_empty + int(rng.choice([0, -1, 2, -n_empty])))))
        budget = int(rng.integers(-2, 5000))
        align = int(rng.choice([0, 1, 16, 64]))
        window_cases.append((ctx, budget, align))
    token_cases.append(([0, 5], [I32_MAX, 1], 2))
    window_cases.append(([I32_MAX, 1, 0], I32_MAX, 64))
    window_cases.append(([I32_MAX], 64, 64))

    lines = []
    for ctx, q, budget, cap, align, world, il, ccap, ecap in plan_cases:
        lines.append(" ".join(map(str, ["P", len(ctx), budget, cap, align, world, il, ccap, ecap] + ctx + q)))
    for ctx, q, ecap in token_cases:
        lines.append(" ".join(map(str, ["T", len(ctx), ecap] + ctx + q)))
    for ctx, budget, align in window_cases:
        lines.append(" ".join(map(str, ["U", len(ctx), budget, align] + ctx)))
    lines += ["N 0", "N 3", "N -1"]

    out = _run(driver, lines)
    k = 0
    for case in plan_cases:
        _check_plan_line(out[k], case)
        k += 1
    for ctx, q, ecap in token_cases:
        _check_tokens_line(out[k], ctx, q, ecap)
        k += 1
    for ctx, budget, align in window_cases:
        _check_windows_line(out[k], ctx, budget, align)
        k += 1
    assert out[k:] == ["N 0 0 0 0", "N 1 1 1 1", "N 1 1 1 1"]
