"""ca_attend_noalloc (the step with its workspace in the library's static
device scratch) against ca_attend (the caller's workspace) through the C ABI:
same bits, and the oracle's bar, on two calls in a row, the second with a
smaller input; contexts alternating on the one scratch; appends patched into
the scratch's table; the one-launch step; and the size limit."""

import ctypes
import sys

import numpy as np
import pytest

from oracle import attention as A
from workloads import make_config, make_prefix_suffix

pytestmark = pytest.mark.gpu

ATOL, RTOL, REL_L2 = 2e-3, 1e-2, 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ctx(wl, **kw):
    import torch
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slots_needed
    ca = ChunkAttention(wl.heads, slots_needed(wl) + 4, device="cuda:0", **kw)
    load_workload(ca, wl, device="cuda:0")
    torch.cuda.synchronize()
    return ca


def _noalloc(ca, q, out):
    """ca_attend_noalloc called directly through the C ABI."""
    return ca.lib.ca_attend_noalloc(ca.ctx, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                    ca._stream())


def _both(ca, q_np):
    """(ca_attend result, ca_attend_noalloc result) on the same q."""
    import torch
    q = torch.from_numpy(np.ascontiguousarray(q_np)).cuda()
    ref = ca.attend(q)
    out = torch.full_like(q, float("nan"))
    assert _noalloc(ca, q, out) == 0, ca.lib.ca_last_error(ca.ctx)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def _parity(got, ref, label):
    rep = A.allclose_report(got, ref, ATOL, RTOL)
    _say(f"{label}: max_abs={rep['max_abs']:.3e} rel_l2={rep['rel_l2']:.3e} bad={rep['n_bad']}")
    assert rep["ok"] and rep["rel_l2"] <= REL_L2, (label, rep)


def test_noalloc_equals_attend_then_a_smaller_input():
    """Workload 2 (32 sequences x 32 heads, 1.5 MiB of workspace), then the
    tiny workload 1 (4 x 8 heads) on another context in the same scratch."""
    _say("noalloc: workload 2 then workload 1")
    big, small = make_config(2), make_config(1)
    a = _ctx(big)
    ref, got = _both(a, big.q)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    _parity(got, A.decode_workload(big), "noalloc workload 2")
    b = _ctx(small)
    ref, got = _both(b, small.q)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    _parity(got, A.decode_workload(small), "noalloc workload 1")


def test_contexts_alternating_on_the_scratch():
    """Two contexts take turns: each finds the other's table in the scratch and
    uploads its own again; results stay those of ca_attend."""
    _say("noalloc: alternating contexts")
    import torch
    w1 = make_prefix_suffix(300, [40, 70, 129], heads=4, seed=91)
    w2 = make_prefix_suffix(0, [65, 1, 200, 33, 64], heads=4, seed=92)
    c1, c2 = _ctx(w1), _ctx(w2)
    r1 = c1.attend(torch.from_numpy(w1.q).cuda()).cpu().numpy()
    r2 = c2.attend(torch.from_numpy(w2.q).cuda()).cpu().numpy()
    for _ in range(3):
        for ca, wl, r in ((c1, w1, r1), (c2, w2, r2)):
            q = torch.from_numpy(wl.q).cuda()
            out = torch.full_like(q, float("nan"))
            assert _noalloc(ca, q, out) == 0
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint16), r.view(np.uint16))


def test_appends_between_noalloc_steps():
    """Decode tokens appended in place patch their fill counts into the table
    in the scratch (no upload); a twin context runs ca_attend on the same
    tokens, and both match bit for bit and the oracle every few steps."""
    _say("noalloc: appends between steps")
    import torch
    wl = make_prefix_suffix(128, [10, 61, 3], heads=2, seed=93)
    a, b = _ctx(wl), _ctx(wl)
    rng = np.random.default_rng(94)
    kv = [[x.copy() for x in wl.seq_kv(i)] for i in range(wl.n_seq)]
    ids = list(range(wl.n_seq))
    for step in range(70):
        k = rng.standard_normal((wl.n_seq, 2, 128), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((wl.n_seq, 2, 128), dtype=np.float32).astype(np.float16)
        q = rng.standard_normal((wl.n_seq, 2, 128), dtype=np.float32).astype(np.float16)
        kt, vt, qt = (torch.from_numpy(x).cuda() for x in (k, v, q))
        toks = np.full(wl.n_seq, 5000 + step, np.int32)
        for ca in (a, b):
            ca.append_batch(ids, toks, kt, vt)
        ref = b.attend(qt)
        out = torch.full_like(qt, float("nan"))
        rc = _noalloc(a, qt, out)
        assert rc == 0, a.lib.ca_last_error(a.ctx)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), ref.cpu().numpy().view(np.uint16)), step
        for i in range(wl.n_seq):
            kv[i] = [np.concatenate([x, y[i:i + 1]]) for x, y in zip(kv[i], (k, v))]
        if step % 23 == 0 or step == 69:
            _parity(out.cpu().numpy(), A.decode_step(q, kv), f"noalloc decode step {step}")
    assert a.stats()["patched_appends"] > 50


def test_one_launch_step_in_the_scratch():
    """The one-launch step (merge blocks wait on arrival counters in the
    scratch): repeated steps, then a smaller tree, each equal to ca_attend."""
    _say("noalloc: one-launch step")
    from decode_attention_prefix_tree_amd import _capi
    for wl in (make_config(1), make_prefix_suffix(64, [1, 2, 3], heads=3, seed=95)):
        ca = _ctx(wl)
        ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
        for _ in range(3):
            ref, got = _both(ca, wl.q)
            assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
        _parity(got, A.decode_workload(wl), f"noalloc one launch {wl.name}")


def test_noalloc_limits():
    """A workspace beyond the scratch (workload 4 with one private chunk per
    sequence-first task: 16.3 MiB) is refused with CA_E_WORKSPACE and nothing
    is written; without attached staging a table upload is refused with
    CA_E_STATE."""
    _say("noalloc: limits")
    import torch
    from decode_attention_prefix_tree_amd import _capi
    wl = make_config(4)
    ca = _ctx(wl)
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 1)
    assert ca.workspace_bytes() > _capi.CA_NOALLOC_SCRATCH_BYTES
    q = torch.from_numpy(wl.q).cuda()
    out = torch.zeros_like(q)
    assert _noalloc(ca, q, out) == -7
    assert b"static scratch" in ca.lib.ca_last_error(ca.ctx)
    torch.cuda.synchronize()
    assert not out.any()
    del ca
    small = make_config(1)
    cb = _ctx(small)
    assert cb.lib.ca_attach_staging(cb.ctx, None, 0) == 0
    q = torch.from_numpy(small.q).cuda()
    out = torch.zeros_like(q)
    assert _noalloc(cb, q, out) == -10
    cb._lend_staging(3 << 16)
    assert _noalloc(cb, q, out) == 0
    torch.cuda.synchronize()
    _parity(out.cpu().numpy(), A.decode_workload(small), "noalloc after staging")
