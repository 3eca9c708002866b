"""Failure handling of the device path, forced from the host: the
CA_OPT_FAIL_DEVICE_OPS knob makes the context's next device operations fail
with CA_E_HIP before anything is enqueued, so every kernel that does run
exits normally.  A failed step leaves the context usable (the table is
uploaded again, one-launch counters restart); a failed insert puts the tree
back; a decode step whose launch fails stores its tokens with a write launch;
appends whose writes cannot be enqueued make the context refuse further work.
"""

import sys

import numpy as np
import pytest

from oracle import attention as A
from workloads import make_config, make_prefix_suffix

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ctx(wl, capacity=None):
    import torch
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slots_needed
    ca = ChunkAttention(wl.heads, capacity or slots_needed(wl) + 8, device="cuda:0")
    load_workload(ca, wl, device="cuda:0")
    torch.cuda.synchronize()
    return ca


def _step(ca, q_np):
    import torch
    out = ca.attend(torch.from_numpy(np.ascontiguousarray(q_np)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _parity(got, ref, label):
    rep = A.allclose_report(got, ref, ATOL, RTOL)
    _say(f"{label}: max_abs={rep['max_abs']:.3e} bad={rep['n_bad']}")
    assert rep["ok"], (label, rep)


@pytest.mark.parametrize("fused", [0, 1])
def test_failed_step_leaves_the_context_usable(fused):
    """A step whose launch fails returns CA_E_HIP; the next steps give the same
    bits as before the failure (in the one-launch step the arrival epoch did
    not advance for the launch that never ran)."""
    _say(f"failed step, fused={fused}")
    from decode_attention_prefix_tree_amd import CaError, _capi
    wl = make_config(1)
    ca = _ctx(wl)
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, fused)
    ref = _step(ca, wl.q)
    _parity(ref, A.decode_workload(wl), "before")
    for _ in range(2):
        ca.set_option(_capi.CA_OPT_FAIL_DEVICE_OPS, 1)
        with pytest.raises(CaError) as ei:
            _step(ca, wl.q)
        assert ei.value.name == "hip"
        for _ in range(3):
            assert np.array_equal(_step(ca, wl.q).view(np.uint16), ref.view(np.uint16))


def test_failed_insert_changes_nothing():
    """An insert that would split a shared chunk and take new slots fails at its
    copy: table, sequence list and stats are those from before; the same
    insert then succeeds and the step matches the oracle."""
    _say("failed insert")
    import torch
    from decode_attention_prefix_tree_amd import CaError, _capi
    wl = make_prefix_suffix(200, [30, 90, 5], heads=4, seed=301)
    ca = _ctx(wl, capacity=40)
    rows0, order0 = ca.export_table()
    st0 = ca.stats()
    tokens = np.concatenate([wl.seq_tokens(0)[:150], np.arange(7000, 7100, dtype=np.int32)])
    rng = np.random.default_rng(302)
    k = np.concatenate([wl.seq_kv(0)[0][:150],
                        rng.standard_normal((100, 4, 128), dtype=np.float32).astype(np.float16)])
    v = np.concatenate([wl.seq_kv(0)[1][:150],
                        rng.standard_normal((100, 4, 128), dtype=np.float32).astype(np.float16)])
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    ca.set_option(_capi.CA_OPT_FAIL_DEVICE_OPS, 1)
    with pytest.raises(CaError) as ei:
        ca.insert(9, tokens, kt, vt)
    assert ei.value.name == "hip"
    rows1, order1 = ca.export_table()
    assert np.array_equal(rows0, rows1) and order0 == order1
    st1 = ca.stats()
    for key in ("live_sequences", "chunks", "free_slots", "unique_tokens", "attended_tokens", "shared_chunks"):
        assert st1[key] == st0[key], key
    assert ca.insert(9, tokens, kt, vt) == 150
    assert ca.stats()["chunks"] > st0["chunks"]
    q = rng.standard_normal((4, 4, 128), dtype=np.float32).astype(np.float16)
    kv = [wl.seq_kv(i) for i in range(3)] + [(k, v)]
    _parity(_step(ca, q), A.decode_step(q, kv), "after the insert")


@pytest.mark.parametrize("succeed_first", [0, 1])
def test_failed_insert_into_decoded_chunks(succeed_first):
    """An insert that shares a decoded sequence's row-major chunks (so they
    are first rewritten as tiles, in a launch of their own), splits one and
    adds new chunks fails at a copy.  When the conversion launch itself fails
    (succeed_first 0) nothing changes; when it went out and the copies failed
    (succeed_first 1), the table and sequences are still those from before and
    only the converted chunks' layout changed.  Either way the steps then
    match the oracle, and the same insert then succeeds."""
    _say(f"failed insert into decoded chunks, {succeed_first} operation(s) first")
    import torch
    from decode_attention_prefix_tree_amd import CaError, ChunkAttention, _capi
    rng = np.random.default_rng(310 + succeed_first)
    H = 2
    ca = ChunkAttention(H, 64, device="cuda:0")

    def rnd(n):
        return rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)

    toks = [int(x) for x in range(40)]
    kv = [rnd(40), rnd(40)]
    ca.insert(0, toks, torch.from_numpy(kv[0]).cuda(), torch.from_numpy(kv[1]).cuda())
    for step in range(100):  # 100 decoded tokens: one full appended chunk and part of another
        k, v = rnd(1), rnd(1)
        q = rnd(1)
        ca.decode_step(np.array([1000 + step], np.int32), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.from_numpy(q).cuda())
        toks.append(1000 + step)
        kv = [np.concatenate([kv[0], k]), np.concatenate([kv[1], v])]
    torch.cuda.synchronize()
    rows0, order0 = ca.export_table()
    st0 = ca.stats()
    assert st0["row_chunks"] >= 2
    cut = 40 + 64 + 20  # inside the second appended chunk
    new_k, new_v = rnd(80), rnd(80)
    t9 = toks[:cut] + list(range(7000, 7080))
    k9 = np.concatenate([kv[0][:cut], new_k])
    v9 = np.concatenate([kv[1][:cut], new_v])
    k9t, v9t = torch.from_numpy(k9).cuda(), torch.from_numpy(v9).cuda()
    ca.set_option(_capi.CA_OPT_FAIL_AFTER_DEVICE_OPS, succeed_first)
    ca.set_option(_capi.CA_OPT_FAIL_DEVICE_OPS, 1)
    with pytest.raises(CaError) as ei:
        ca.insert(9, t9, k9t, v9t)
    assert ei.value.name == "hip"
    rows1, order1 = ca.export_table()
    assert np.array_equal(rows0, rows1) and order0 == order1
    st1 = ca.stats()
    for key in ("live_sequences", "chunks", "free_slots", "unique_tokens"):
        assert st1[key] == st0[key], key
    if succeed_first:
        assert st1["row_chunks"] < st0["row_chunks"]
    else:
        assert st1["row_chunks"] == st0["row_chunks"]
    q = rnd(1)
    _parity(_step(ca, q), A.decode_step(q, [kv]), "after the failed insert")
    assert ca.insert(9, t9, k9t, v9t) == cut
    q = rnd(2)
    _parity(_step(ca, q), A.decode_step(q, [kv, [k9, v9]]), "after the insert")


def test_decode_step_whose_launch_fails_stores_the_tokens():
    """ca_decode_step with in-kernel appends whose launch fails: the tokens go
    to the pool by a write launch, the call returns CA_E_HIP, and the next
    step (over the grown sequences) matches the oracle.  When the write launch
    fails too, the context refuses further work (CA_E_STATE) but still
    reports its state."""
    _say("failed decode step")
    import torch
    from decode_attention_prefix_tree_amd import CaError, _capi
    wl = make_prefix_suffix(128, [10, 20, 30], heads=2, seed=303)
    ca = _ctx(wl)
    rng = np.random.default_rng(304)
    kv = [[x.copy() for x in wl.seq_kv(i)] for i in range(3)]
    _step(ca, wl.q)  # the table is on the device: the next tokens are written in the kernel

    def draw():
        return [rng.standard_normal((3, 2, 128), dtype=np.float32).astype(np.float16) for _ in range(3)]

    k, v, q = draw()
    kt, vt, qt = (torch.from_numpy(x).cuda() for x in (k, v, q))
    patched = ca.stats()["patched_appends"]
    ca.set_option(_capi.CA_OPT_FAIL_DEVICE_OPS, 1)
    with pytest.raises(CaError) as ei:
        ca.decode_step(np.array([11, 12, 13], np.int32), kt, vt, qt)
    assert ei.value.name == "hip"
    assert ca.stats()["patched_appends"] == patched + 1  # it was the in-kernel path
    for i in range(3):
        kv[i] = [np.concatenate([a, b[i:i + 1]]) for a, b in zip(kv[i], (k, v))]
    q2 = draw()[2]
    _parity(_step(ca, q2), A.decode_step(q2, kv), "after the failed decode step")

    k, v, q = draw()
    kt, vt, qt = (torch.from_numpy(x).cuda() for x in (k, v, q))
    ca.set_option(_capi.CA_OPT_FAIL_DEVICE_OPS, 2)
    with pytest.raises(CaError) as ei:
        ca.decode_step(np.array([21, 22, 23], np.int32), kt, vt, qt)
    assert ei.value.name == "hip"
    for call in (lambda: _step(ca, q), lambda: ca.append_batch([0], [5], kt[:1], vt[:1]),
                 lambda: ca.remove(0)):
        with pytest.raises(CaError) as ei:
            call()
        assert ei.value.name == "state"
    assert ca.stats()["live_sequences"] == 3 and ca.sequences() == [0, 1, 2]


def test_failed_append_makes_the_context_refuse_work():
    _say("failed append")
    import torch
    from decode_attention_prefix_tree_amd import CaError, _capi
    wl = make_config(1)
    ca = _ctx(wl)
    k = torch.zeros((1, wl.heads, 128), dtype=torch.float16, device="cuda:0")
    ca.set_option(_capi.CA_OPT_FAIL_DEVICE_OPS, 1)
    with pytest.raises(CaError) as ei:
        ca.append(0, [99], k, k)
    assert ei.value.name == "hip"
    with pytest.raises(CaError) as ei:
        _step(ca, wl.q)
    assert ei.value.name == "state"
    assert ca.stats()["attended_tokens"] == wl.attended_tokens() + 1
