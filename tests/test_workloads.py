"""The seeded generators: determinism, shapes, and the structure each workload claims."""

import numpy as np

from workloads import from_token_lists, make_config, make_prefix_suffix


def test_deterministic_and_shaped():
    a, b = make_config(1), make_config(1)
    assert np.array_equal(a.q, b.q)
    assert a.q.shape == (4, 8, 128) and a.q.dtype == np.float16
    for sa, sb in zip(a.segments, b.segments):
        assert np.array_equal(sa.k, sb.k) and np.array_equal(sa.v, sb.v)
    assert [a.seq_len(i) for i in range(4)] == [288] * 4
    k, v = a.seq_kv(2)
    assert k.shape == (288, 8, 128)
    assert np.array_equal(k[:256], a.segments[0].k)


def test_token_ids_unique_per_segment():
    wl = make_config(2, heads=1)
    seen = set()
    for s in wl.segments:
        t = set(s.tokens.tolist())
        assert len(t) == s.length and not (t & seen)
        seen |= t


def test_multi_branch_lengths():
    wl = make_config(5, heads=1)
    L = wl.lengths()
    assert wl.n_seq == 128
    assert ((L >= 2048 + 64) & (L <= 2048 + 1024)).all()
    assert [p[1] for p in wl.paths] == [1 + 33 * (i // 32) for i in range(128)]


def test_token_list_workload_shares_rows_for_shared_prefixes():
    wl = from_token_lists([[1, 2, 3], [1, 2, 4], [5]], heads=2, seed=3, head_dim=8)
    k0, v0 = wl.seq_kv(0)
    k1, v1 = wl.seq_kv(1)
    assert np.array_equal(k0[:2], k1[:2]) and not np.array_equal(k0[2], k1[2])
    assert np.array_equal(v0[:2], v1[:2])


def test_prefix_suffix_workload():
    wl = make_prefix_suffix(1766, [512] * 4, heads=2, seed=5)
    again = make_prefix_suffix(1766, [512] * 4, heads=2, seed=5)
    assert np.array_equal(wl.q, again.q)
    assert [wl.seq_len(i) for i in range(4)] == [2278] * 4
    assert wl.unique_tokens() == 1766 + 4 * 512
    k0, _ = wl.seq_kv(0)
    k3, _ = wl.seq_kv(3)
    assert np.array_equal(k0[:1766], k3[:1766]) and not np.array_equal(k0[1766:], k3[1766:])
    flat = make_prefix_suffix(0, [3, 70], heads=1, seed=5)
    assert flat.paths == [[0], [1]] and flat.unique_tokens() == 73
