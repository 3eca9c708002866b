"""Pins for the Python prefix-tree model: hand-worked golden tables, brute-force
prefix counts, the L_p + N*L_s memory formula of the prefix-aware KV cache
(explainer 0h-n0.github.io/posts/paper-2402-15220, "Prefix-Aware KV Cache"),
and structural invariants of the DFS table."""

import itertools

import numpy as np
import pytest

from oracle.tree_model import PrefixTreeModel, TreeError
from tests.golden_cases import load_cases
from workloads import make_config


def run_case_on_model(case):
    m = PrefixTreeModel(case.chunk, case.capacity, case.share)
    for op in case.ops:
        if op.kind == "table":
            rows, order = m.table()
            assert rows == op.rows, (case.name, rows)
            assert order == op.order, (case.name, order)
            if op.unique is not None:
                assert m.unique_tokens() == op.unique
            continue
        before = m.table()
        try:
            if op.kind == "insert":
                got = str(m.insert(op.seq, op.tokens))
            elif op.kind == "append":
                m.append(op.seq, op.tokens)
                got = None
            else:
                m.remove(op.seq)
                got = None
        except TreeError as e:
            got = e.code
            assert m.table() == before, "a failed call must not change the tree"
        assert got == op.expect, (case.name, op, got)


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c.name)
def test_golden_cases(case):
    run_case_on_model(case)


def check_invariants(m, live_tokens):
    rows, order = m.table()
    n = len(order)
    assert sorted(order) == sorted(live_tokens)
    # ranges: children nest inside parents, siblings in order, disjoint
    for r, (nid, prow, start, ntok, b, e, slot) in enumerate(rows):
        assert 0 <= b < e <= n
        assert 1 <= ntok <= m.chunk
        if prow >= 0:
            pb, pe = rows[prow][4], rows[prow][5]
            assert pb <= b and e <= pe
            assert start == rows[prow][2] + rows[prow][3]
        else:
            assert start == 0
    refs = m.refcounts()
    for nid, prow, start, ntok, b, e, slot in rows:
        assert refs[nid] == e - b
    # slots unique and disjoint from the free list
    slots = [r[6] for r in rows]
    assert len(set(slots)) == len(slots)
    assert len(slots) + m.free_slots() == m.capacity
    # every sequence's path reproduces its tokens exactly
    for s, toks in live_tokens.items():
        path = m.seq_path(s)
        assert [p[1] for p in path] == list(itertools.accumulate([0] + [p[2] for p in path[:-1]]))
        assert sum(p[2] for p in path) == len(toks)
    # attended tokens: sum over chunks of n_tokens * range
    assert sum(r[3] * (r[5] - r[4]) for r in rows) == sum(len(t) for t in live_tokens.values())
    # each sequence's path rows are exactly the rows whose range contains its DFS position
    for pos, s in enumerate(order):
        contained = [r for r in rows if r[4] <= pos < r[5]]
        assert sorted((r[6], r[2], r[3]) for r in contained) == sorted(m.seq_path(s))


def distinct_prefixes(seqs):
    return len({tuple(t[: j + 1]) for t in seqs for j in range(len(t))})


@pytest.mark.parametrize("chunk", [1, 2, 3, 4])
@pytest.mark.parametrize("vocab", [2, 3])
def test_unique_tokens_equal_distinct_prefixes(chunk, vocab):
    rng = np.random.default_rng(chunk * 10 + vocab)
    for trial in range(30):
        n = int(rng.integers(1, 9))
        seqs = [list(rng.integers(0, vocab, size=int(rng.integers(1, 13)))) for _ in range(n)]
        m = PrefixTreeModel(chunk, 1000)
        live = {}
        for i, t in enumerate(seqs):
            m.insert(i, t)
            live[i] = t
        assert m.unique_tokens() == distinct_prefixes(seqs)
        check_invariants(m, live)


def test_random_insert_append_remove_keeps_paths_exact():
    rng = np.random.default_rng(42)
    for trial in range(40):
        chunk = int(rng.integers(2, 5))
        m = PrefixTreeModel(chunk, 10_000)
        live = {}
        next_id = 0
        appended = False
        for step in range(60):
            r = rng.random()
            if r < 0.45 or not live:
                t = list(rng.integers(0, 3, size=int(rng.integers(1, 13))))
                matched = m.insert(next_id, t)
                # the matched count is the longest common prefix with any live
                # sequence; once appends (never deduplicated) exist, sibling
                # chunks may share a first token and matching follows the
                # first of them, so it can only be shorter.
                best = max((len(list(itertools.takewhile(lambda ab: ab[0] == ab[1], zip(t, u))))
                            for u in live.values()), default=0)
                assert matched == best if not appended else matched <= best
                live[next_id] = t
                next_id += 1
            elif r < 0.75:
                s = int(rng.choice(list(live)))
                t = list(rng.integers(0, 3, size=int(rng.integers(1, 6))))
                m.append(s, t)
                live[s] = live[s] + t
                appended = True
            else:
                s = int(rng.choice(list(live)))
                m.remove(s)
                del live[s]
            check_invariants(m, live)
        for s in list(live):
            m.remove(s)
        assert m.table() == ([], [])
        assert m.free_slots() == m.capacity


def _model_for(wl, capacity=10**6):
    m = PrefixTreeModel(wl.chunk, capacity)
    for i in range(wl.n_seq):
        m.insert(i, wl.seq_tokens(i))
    return m


@pytest.mark.parametrize("k,expected", [(1, 256 + 4 * 32), (2, 1024 + 32 * 512), (3, 4096 + 32 * 512),
                                        (4, 32 * 2048)])
def test_unique_tokens_formula_on_workloads(k, expected):
    wl = make_config(k, heads=1)
    m = _model_for(wl)
    assert m.unique_tokens() == expected == wl.unique_tokens()
    rows, order = m.table()
    assert order == list(range(wl.n_seq))
    shared = [r for r in rows if r[5] - r[4] >= 2]
    private = [r for r in rows if r[5] - r[4] == 1]
    n_shared, n_private = {1: (4, 4), 2: (16, 256), 3: (64, 256), 4: (0, 1024)}[k]
    assert (len(shared), len(private)) == (n_shared, n_private)
    check_invariants(m, {i: list(wl.seq_tokens(i)) for i in range(wl.n_seq)})


def test_multi_branch_workload_tree():
    wl = make_config(5, heads=1)
    m = _model_for(wl)
    suffix = wl.lengths() - 2048
    assert m.unique_tokens() == 5 * 1024 + int(suffix.sum())
    rows, order = m.table()
    assert order == list(range(128))
    root = [r for r in rows if r[5] - r[4] == 128]
    branch = [r for r in rows if r[5] - r[4] == 32]
    private = [r for r in rows if r[5] - r[4] == 1]
    assert len(root) == 16 and len(branch) == 64
    assert len(private) == int(sum((s + 63) // 64 for s in suffix))
    for b in range(4):
        rs = [r for r in branch if r[4] == 32 * b]
        assert len(rs) == 16 and all(r[5] == 32 * b + 32 for r in rs)
