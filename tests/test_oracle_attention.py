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
