"""Pins for the fp64 attention oracle, each against something other than itself:
closed forms and special cases of softmax(q K^T / sqrt(d)) V, a pure-Python
brute force, a library routine (torch SDPA on CPU in float64), and the exact
log-sum-exp re-association that the two-phase partition relies on."""

import math

import numpy as np
import pytest

from oracle import attention as A

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def brute_force(q, keys, values, scale):
    """Single head, pure Python, sum_j e^{x_j} v_j / sum_j e^{x_j} without
    any max subtraction (tiny inputs only)."""
    xs = [sum(a * b for a, b in zip(q, kj)) * scale for kj in keys]
    ws = [math.exp(x) for x in xs]
    z = sum(ws)
    return [sum(w * vj[c] for w, vj in zip(ws, values)) / z for c in range(len(values[0]))]


def rnd(rng, *shape):
    return rng.standard_normal(shape).astype(np.float16)


@pytest.mark.parametrize("d", [1, 2, 3])
@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_brute_force_tiny(d, L):
    rng = np.random.default_rng(7 * d + L)
    for trial in range(20):
        H = 2
        q = rnd(rng, H, d)
        k = rnd(rng, L, H, d)
        v = rnd(rng, L, H, d)
        scale = 1.0 / math.sqrt(d)
        got = A.attend_sequence(q, k, v)
        for h in range(H):
            ref = brute_force([float(x) for x in q[h]],
                              [[float(x) for x in k[j, h]] for j in range(L)],
                              [[float(x) for x in v[j, h]] for j in range(L)], scale)
            np.testing.assert_allclose(got[h], ref, rtol=1e-12, atol=1e-14)


def test_single_token_is_value_exactly():
    rng = np.random.default_rng(1)
    q, k, v = rnd(rng, 4, 128), rnd(rng, 1, 4, 128), rnd(rng, 1, 4, 128)
    out = A.attend_sequence(q, k, v)
    assert np.array_equal(out, v[0].astype(np.float64))


def test_identical_keys_or_zero_query_give_mean_value():
    rng = np.random.default_rng(2)
    L, H, d = 37, 3, 128
    v = rnd(rng, L, H, d)
    k_same = np.broadcast_to(rnd(rng, 1, H, d), (L, H, d))
    mean = v.astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(A.attend_sequence(rnd(rng, H, d), k_same, v), mean, rtol=0, atol=1e-12)
    np.testing.assert_allclose(A.attend_sequence(np.zeros((H, d), np.float16), rnd(rng, L, H, d), v),
                               mean, rtol=0, atol=1e-12)


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(3)
    L, H, d = 50, 2, 128
    c = rnd(rng, H, d)
    v = np.broadcast_to(c, (L, H, d))
    out = A.attend_sequence(rnd(rng, H, d), rnd(rng, L, H, d), v)
    np.testing.assert_allclose(out, c.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_score_gap_ln3_gives_three_quarters():
    # d = 1, scale 1: scores ln3 and 0 -> weights 3/4 and 1/4.
    q = np.array([[1.0]])
    k = np.array([[[math.log(3.0)]], [[0.0]]])
    v = np.array([[[8.0]], [[-4.0]]])
    out = A.attend_sequence(q, k, v, scale=1.0)
    assert abs(out[0, 0] - (0.75 * 8.0 + 0.25 * -4.0)) < 1e-14


def test_heads_are_independent_and_not_transposed():
    rng = np.random.default_rng(4)
    L, H, d = 9, 5, 16
    q, k, v = rnd(rng, H, d), rnd(rng, L, H, d), rnd(rng, L, H, d)
    full = A.attend_sequence(q, k, v)
    for h in range(H):
        one = A.attend_sequence(q[h:h + 1], k[:, h:h + 1], v[:, h:h + 1])
        np.testing.assert_array_equal(full[h], one[0])


def test_matches_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    for L in (1, 63, 64, 65, 300):
        H, d = 4, 128
        q, k, v = rnd(rng, H, d), rnd(rng, L, H, d), rnd(rng, L, H, d)
        tq = torch.from_numpy(q.astype(np.float64))[:, None, :]       # [H,1,d]
        tk = torch.from_numpy(k.astype(np.float64)).transpose(0, 1).contiguous()  # [H,L,d]
        tv = torch.from_numpy(v.astype(np.float64)).transpose(0, 1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0, :].numpy()
        np.testing.assert_allclose(A.attend_sequence(q, k, v), ref, rtol=1e-12, atol=1e-13)


def test_key_order_does_not_matter():
    rng = np.random.default_rng(6)
    L, H, d = 200, 3, 128
    q, k, v = rnd(rng, H, d), rnd(rng, L, H, d), rnd(rng, L, H, d)
    perm = rng.permutation(L)
    np.testing.assert_allclose(A.attend_sequence(q, k, v), A.attend_sequence(q, k[perm], v[perm]),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_partition_then_lse_merge_equals_whole(seed):
    rng = np.random.default_rng(100 + seed)
    L, H, d = int(rng.integers(2, 700)), 4, 128
    q, k, v = rnd(rng, H, d), rnd(rng, L, H, d), rnd(rng, L, H, d)
    whole = A.attend_sequence(q, k, v)
    n_cut = int(rng.integers(1, min(L, 9)))
    cuts = np.sort(rng.choice(np.arange(1, L), size=n_cut, replace=False))
    bounds = [0, *cuts.tolist(), L]
    parts = [A.partial(q, k[a:b], v[a:b]) for a, b in zip(bounds, bounds[1:])]
    merged = A.finalize(A.merge_all(parts))
    np.testing.assert_allclose(merged, whole, rtol=1e-12, atol=1e-14)
    # reversed order: the merge is commutative/associative
    merged_rev = A.finalize(A.merge_all(parts[::-1]))
    np.testing.assert_allclose(merged_rev, whole, rtol=1e-12, atol=1e-14)
    # tree-shaped association
    mid = len(parts) // 2 or 1
    left = A.merge_all(parts[:mid])
    right = A.merge_all(parts[mid:]) if parts[mid:] else A.partial(q, k[:0], v[:0])
    np.testing.assert_allclose(A.finalize(A.merge(left, right)), whole, rtol=1e-12, atol=1e-14)


def test_explainer_two_part_form_equals_whole():
    rng = np.random.default_rng(8)
    H, d = 8, 128
    for lp, ls in ((256, 32), (1024, 512), (1, 1), (64, 0)):
        q = rnd(rng, H, d)
        kp, vp = rnd(rng, lp, H, d), rnd(rng, lp, H, d)
        ks, vs = rnd(rng, ls, H, d), rnd(rng, ls, H, d)
        whole = A.attend_sequence(q, np.concatenate([kp, ks]), np.concatenate([vp, vs]))
        if ls == 0:
            got = A.finalize(A.merge(A.partial(q, kp, vp), A.partial(q, ks, vs)))
        else:
            got = A.two_phase(q, kp, vp, ks, vs)
        np.testing.assert_allclose(got, whole, rtol=1e-12, atol=1e-14)


def test_empty_partial_is_identity():
    rng = np.random.default_rng(9)
    H, d = 2, 128
    q, k, v = rnd(rng, H, d), rnd(rng, 10, H, d), rnd(rng, 10, H, d)
    p = A.partial(q, k, v)
    e = A.partial(q, k[:0], v[:0])
    for got in (A.merge(p, e), A.merge(e, p)):
        np.testing.assert_array_equal(got[0], p[0])
        np.testing.assert_array_equal(got[1], p[1])
        np.testing.assert_array_equal(got[2], p[2])


def test_tolerance_detects_a_dropped_or_doubled_chunk():
    """The abs 2e-3 / rel 1e-2 bar is tight enough that a kernel which drops or
    double-counts one 64-token chunk, or uses the wrong scale, fails it."""
    rng = np.random.default_rng(10)
    L, H, d = 1536, 32, 128
    q, k, v = rnd(rng, H, d), rnd(rng, L, H, d), rnd(rng, L, H, d)
    ref = A.attend_sequence(q, k, v)
    dropped = A.attend_sequence(q, np.concatenate([k[:640], k[704:]]), np.concatenate([v[:640], v[704:]]))
    doubled = A.attend_sequence(q, np.concatenate([k, k[:64]]), np.concatenate([v, v[:64]]))
    wrong_scale = A.attend_sequence(q, k, v, scale=1.0 / 128)
    for bad in (dropped, doubled, wrong_scale):
        rep = A.allclose_report(bad, ref)
        assert not rep["ok"] and rep["n_bad"] > 500
    # fp16 rounding of the exact result stays well inside the bar
    rep = A.allclose_report(ref.astype(np.float16), ref)
    assert rep["ok"] and rep["max_abs"] < 2.5e-4


# --- the batch-level entry points the GPU parity tests compare against --------

def _sdpa_rows(torch, q, seq_kv):
    """Per-sequence torch SDPA in float64 (a library routine, no tree, no
    chunks): row i of q over the i-th (K, V)."""
    out = []
    for i, (k, v) in enumerate(seq_kv):
        tq = torch.from_numpy(np.asarray(q[i], np.float64))[:, None, :]
        tk = torch.from_numpy(np.asarray(k, np.float64)).transpose(0, 1).contiguous()
        tv = torch.from_numpy(np.asarray(v, np.float64)).transpose(0, 1).contiguous()
        out.append(torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0, :].numpy())
    return np.stack(out)


def _ragged_shared_workload():
    """Sequences that share a 150-token prefix, then split into two branches
    (one cut inside a 64-token chunk), with private tails of 1..300 tokens, a
    sequence that ends inside the tree and an exact duplicate."""
    from workloads import from_token_lists
    rng = np.random.default_rng(31)
    pre = [int(x) for x in rng.integers(0, 40, size=150)]
    seqs = []
    for i in range(9):
        branch = [700 + (i % 2)] + [int(x) for x in rng.integers(0, 40, size=20 + 17 * (i % 2))]
        tail = [900 + i] + [int(x) for x in rng.integers(0, 40, size=int(rng.integers(0, 300)))]
        seqs.append(pre + branch + tail)
    seqs.append(pre[:97])       # ends inside the shared prefix
    seqs.append(list(seqs[3]))  # duplicate of a live sequence
    return from_token_lists(seqs, heads=3, seed=32)


def test_decode_workload_equals_per_sequence_sdpa():
    torch = pytest.importorskip("torch")
    wl = _ragged_shared_workload()
    kv = [wl.seq_kv(i) for i in range(wl.n_seq)]
    ref = _sdpa_rows(torch, wl.q, kv)
    np.testing.assert_allclose(A.decode_workload(wl), ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A.decode_step(wl.q, kv), ref, rtol=1e-12, atol=1e-13)
    # the duplicate attends the same keys with its own query
    assert not np.array_equal(A.decode_workload(wl, [3]), A.decode_workload(wl, [10]))


def test_decode_workload_row_subset_is_those_rows_in_that_order():
    """The row-subset path, as the large GPU tests use it: shuffled rows with a
    repeat come back in the order asked, each equal to its own sequence's
    attention by SDPA."""
    torch = pytest.importorskip("torch")
    wl = _ragged_shared_workload()
    rows = [7, 0, 10, 3, 3, 9]
    got = A.decode_workload(wl, rows)
    assert got.shape == (len(rows), wl.heads, wl.head_dim)
    ref = _sdpa_rows(torch, wl.q[rows], [wl.seq_kv(i) for i in rows])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(got, A.decode_workload(wl)[rows])
    assert A.decode_workload(wl, []).shape == (0, wl.heads, wl.head_dim)


def test_decode_step_brute_force_tiny_batch():
    """Three sequences of 1..4 tokens at d = 2, against the pure-Python sum
    without max subtraction; rows must not be mixed up."""
    rng = np.random.default_rng(33)
    H, d = 2, 2
    lens = (1, 4, 3)
    q = rnd(rng, len(lens), H, d)
    kv = [(rnd(rng, L, H, d), rnd(rng, L, H, d)) for L in lens]
    got = A.decode_step(q, kv)
    for i, (k, v) in enumerate(kv):
        for h in range(H):
            ref = brute_force([float(x) for x in q[i, h]], [[float(x) for x in k[j, h]] for j in range(lens[i])],
                              [[float(x) for x in v[j, h]] for j in range(lens[i])], 1.0 / math.sqrt(d))
            np.testing.assert_allclose(got[i, h], ref, rtol=1e-12, atol=1e-14)
    assert A.decode_step(q[:0], []).shape == (0, H, d)


def test_decode_workload_on_the_multi_branch_shape():
    """The multi-branch workload's paths (root, branch, suffix) at one head:
    sequence i's keys are its three segments in order; a sample of rows from
    every branch equals SDPA over that concatenation built here."""
    torch = pytest.importorskip("torch")
    from workloads import make_config
    wl = make_config(5, heads=1)
    rows = [0, 31, 32, 95, 127]
    kv = []
    for i in rows:
        b = i // 32
        segs = [wl.segments[0], wl.segments[1 + b * 33], wl.segments[2 + b * 33 + (i % 32)]]
        assert [s.length for s in segs][:2] == [1024, 1024]
        kv.append((np.concatenate([s.k for s in segs]), np.concatenate([s.v for s in segs])))
    np.testing.assert_allclose(A.decode_workload(wl, rows), _sdpa_rows(torch, wl.q[rows], kv),
                               rtol=1e-12, atol=1e-13)


# --- the parity bar ------------------------------------------------------------

def _edge(ref, bar, beyond):
    """The float64 value nearest ref + bar whose distance from ref is <= bar
    (beyond=False), or the next one up, whose distance is > bar."""
    g = ref + bar
    while abs(g - ref) > bar:
        g = np.nextafter(g, -np.inf)
    if beyond:
        while abs(g - ref) <= bar:
            g = np.nextafter(g, np.inf)
    return g


@pytest.mark.parametrize("ref", [0.0, 1.0, 100.0, -100.0, 0.37])
def test_parity_bar_boundary_is_atol_plus_rtol_times_ref(ref):
    """|got - ref| <= 2e-3 + 1e-2 * |ref| passes at the bar and fails one
    float64 step beyond it, on either side of ref."""
    bar = 2e-3 + 1e-2 * abs(ref)
    for sign in (1.0, -1.0):
        at = ref + sign * (_edge(ref, bar, False) - ref)
        past = ref + sign * (_edge(ref, bar, True) - ref)
        assert A.allclose_report(np.array([at]), np.array([ref]))["ok"]
        rep = A.allclose_report(np.array([past]), np.array([ref]))
        assert not rep["ok"] and rep["n_bad"] == 1


def test_parity_bar_is_not_swapped_or_relative_to_got():
    # at |ref| = 100 the bar is 1.002: an error of 0.5 passes (swapped, 0.21, would fail)
    assert A.allclose_report(np.array([100.5]), np.array([100.0]))["ok"]
    # at ref = 0 the bar is 2e-3: an error of 5e-3 fails (swapped, 1e-2, would pass)
    assert not A.allclose_report(np.array([5e-3]), np.array([0.0]))["ok"]
    # the relative part scales with |ref|, not |got|: 1.001 off -100 passes
    # (bar 1.002) though 1e-2 * |got| would give 0.992
    assert A.allclose_report(np.array([-98.999]), np.array([-100.0]))["ok"]
    # and an error the size of |got|'s bar but above |ref|'s fails
    assert not A.allclose_report(np.array([1.5]), np.array([1.0]))["ok"]


def test_parity_bar_rejects_non_finite_and_counts_elements():
    ref = np.zeros((2, 3))
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[1, 2] = bad
        assert not A.allclose_report(got, ref)["ok"]
    got = ref.copy()
    got[0, :] = 0.01
    rep = A.allclose_report(got, ref)
    assert not rep["ok"] and rep["n_bad"] == 3 and rep["max_abs"] == pytest.approx(0.01, rel=1e-15)
    # rel-L2 = ||got - ref|| / ||ref||: errors (3, 4) on a reference of norm 10
    ref2 = np.array([6.0, 8.0])
    rep = A.allclose_report(ref2 + np.array([3.0, 4.0]), ref2)
    assert rep["rel_l2"] == pytest.approx(0.5, rel=1e-15)
    assert A.allclose_report(ref2, ref2) == {"ok": True, "n_bad": 0, "max_abs": 0.0, "rel_l2": 0.0}
