"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (elementwise): |gpu - oracle| <= 2e-3 + 1e-2 * |oracle| for fp16 I/O with
fp32 accumulation; rel-L2 is also reported and gated at 1e-3.  Cases: the
five seeded workloads at full size (every row), tiny trees that exercise padded MFMA rows (ranges 2-15,
16, 32, > 32), partial chunks, sequences ending inside the tree, duplicates,
appends and removals, the unshared comparator layout, and every task-size
setting.  Inputs come from the seeded generators in ``workloads``."""

import functools
import sys

import numpy as np
import pytest

from oracle import attention as A
from workloads import from_token_lists, make_config, make_long_sequence, make_prefix_suffix

pytestmark = pytest.mark.gpu

ATOL, RTOL, REL_L2 = 2e-3, 1e-2, 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def cached_config(k):
    return make_config(k)


def _torch():
    import torch
    return torch


def build_ca(wl, share=True, cf_group=None, sf_group=None, capacity=None, two_phase=True, chunk=64):
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slots_needed
    from decode_attention_prefix_tree_amd import _capi
    cap = capacity or slots_needed(wl, chunk=chunk, share=share) + 4
    ca = ChunkAttention(wl.heads, cap, device="cuda:0", share=share, two_phase=two_phase, chunk_size=chunk)
    if cf_group:
        ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, cf_group)
    if sf_group:
        ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, sf_group)
    load_workload(ca, wl, device="cuda:0")
    torch.cuda.synchronize()
    return ca


def run_step(ca, q_np):
    torch = _torch()
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to("cuda:0")
    out = ca.attend(q)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_parity(got, ref, label):
    rep = A.allclose_report(got, ref, ATOL, RTOL)
    _say(f"{label}: max_abs={rep['max_abs']:.3e} rel_l2={rep['rel_l2']:.3e} bad={rep['n_bad']}")
    assert rep["ok"], (label, rep)
    assert rep["rel_l2"] <= REL_L2, (label, rep)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_full(k):
    """Every output row of workloads 1-4 against the oracle, in the launch
    configuration the benchmark times (partials + merge launches), then the
    same bits from repeated steps and from the one-launch step."""
    _say(f"workload {k}")
    from decode_attention_prefix_tree_amd import _capi
    wl = cached_config(k)
    ca = build_ca(wl)
    assert ca.stats()["one_launch_step"] == 0
    got = run_step(ca, wl.q)
    ref = A.decode_workload(wl)
    assert_parity(got, ref, f"config{k}")
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    for _ in range(3):
        assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("case", ["w3_cf32", "w3_cf64", "p2048x96_cf32"])
def test_long_chunk_first_tasks(case):
    """Chunk-first tasks of 32 and 64 chunks (the automatic choice once a
    step streams for about 80 us or more): workload 3's 64-chunk prompt as
    two tasks or one per head, and a 2,048-token prompt under 96 sequences
    (three 32-row blocks of 32-chunk tasks); every output row against the
    oracle."""
    _say(f"long chunk-first tasks {case}")
    if case.startswith("w3"):
        wl = cached_config(3)
    else:
        wl = make_prefix_suffix(2048, [512] * 96, heads=8, seed=2048)
    group = int(case.split("cf")[1])
    ca = build_ca(wl, cf_group=group)
    assert ca.stats()["cf_chunks_per_task"] == group
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), case)


@pytest.mark.parametrize("two_phase", [True, False])
def test_non_aligned_prefix_full(two_phase):
    """A 1,766-token shared prefix (not a multiple of 64) with 512-token
    suffixes, 32 sequences x 32 heads, every output row: the last shared
    chunk holds 38 tokens and one private tail starts with a 26-token chunk."""
    _say(f"prefix 1766 + 512, two_phase={two_phase}")
    wl = make_prefix_suffix(1766, [512] * 32, heads=32, seed=2001)
    ca = build_ca(wl, two_phase=two_phase)
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), "prefix1766")


def test_non_aligned_prefix_ragged_suffixes():
    """The same prefix with suffix lengths 1..700 drawn per sequence, and with
    no shared prefix at all (every sequence private, ragged)."""
    rng = np.random.default_rng(2002)
    for lp in (1766, 0):
        suffix = [int(x) for x in rng.integers(1, 701, size=40)]
        _say(f"prefix {lp} + ragged suffixes")
        wl = make_prefix_suffix(lp, suffix, heads=8, seed=2003 + lp)
        ca = build_ca(wl)
        assert_parity(run_step(ca, wl.q), A.decode_workload(wl), f"prefix{lp} ragged")


def test_insert_remove_churn():
    """Random inserts (a prefix of a live sequence, cut anywhere, plus fresh
    tokens, or an exact duplicate), removals and multi-token appends, with a
    step after every operation checked against the oracle and the exported
    table checked against the independent tree model.  Token ids never repeat
    outside a copied prefix, so every stored prefix has one set of K/V rows."""
    _say("churn")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention
    from oracle.tree_model import PrefixTreeModel
    rng = np.random.default_rng(404)
    H, cap = 4, 160
    ca = ChunkAttention(H, cap, device="cuda:0")
    model = PrefixTreeModel(64, cap)
    live = {}          # seq id -> (tokens list, K [L,H,d], V [L,H,d])
    fresh = iter(range(1, 1 << 30))
    next_id = 0

    def rows(n):
        return (rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16),
                rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")

    for it in range(70):
        r = rng.random()
        if not live or (r < 0.45 and len(live) < 12):
            if live and rng.random() < 0.8:
                src = list(live)[int(rng.integers(len(live)))]
                t0, k0, v0 = live[src]
                p = int(rng.integers(1, len(t0) + 1))
                extra = 0 if rng.random() < 0.15 else int(rng.integers(1, 200))
            else:
                t0, k0, v0, p, extra = [], None, None, 0, int(rng.integers(1, 300))
            kn, vn = rows(extra)
            toks = t0[:p] + [next(fresh) for _ in range(extra)]
            k = np.concatenate([k0[:p], kn]) if p else kn
            v = np.concatenate([v0[:p], vn]) if p else vn
            if model.free_slots() < (len(toks) + 63) // 64 + 1:
                continue
            assert ca.insert(next_id, toks, dev(k), dev(v)) == model.insert(next_id, toks)
            live[next_id] = (toks, k, v)
            next_id += 1
        elif r < 0.7 and len(live) > 1:
            s = list(live)[int(rng.integers(len(live)))]
            ca.remove(s)
            model.remove(s)
            del live[s]
        else:
            s = list(live)[int(rng.integers(len(live)))]
            n = int(rng.integers(1, 90))
            if model.free_slots() < (n + 63) // 64 + 1:
                continue
            kn, vn = rows(n)
            toks = [next(fresh) for _ in range(n)]
            ca.append(s, toks, dev(kn), dev(vn))
            model.append(s, toks)
            t0, k0, v0 = live[s]
            live[s] = (t0 + toks, np.concatenate([k0, kn]), np.concatenate([v0, vn]))
        order = sorted(live)
        q = rng.standard_normal((len(order), H, 128), dtype=np.float32).astype(np.float16)
        got = run_step(ca, q)
        assert_parity(got, A.decode_step(q, [(live[s][1], live[s][2]) for s in order]), f"churn {it}")
        want_rows, want_order = model.table()
        got_rows, got_order = ca.export_table()
        assert [tuple(int(x) for x in row) for row in got_rows] == want_rows, it
        assert got_order == want_order, it


def test_multi_branch_all_rows():
    """Workload 5 at full size (128 sequences x 32 heads: the default step
    is one launch), every output row against the oracle, then the same bits
    from repeated steps and from the two-launch step."""
    _say("workload 5")
    from decode_attention_prefix_tree_amd import _capi
    wl = cached_config(5)
    ca = build_ca(wl)
    assert ca.stats()["one_launch_step"] == 1
    got = run_step(ca, wl.q)
    assert_parity(got, A.decode_workload(wl), "config5")
    for _ in range(2):
        assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))


def tiny_tree_cases():
    rng = np.random.default_rng(77)
    cases = {}
    # one shared prefix, range R for R in 2..15, 16, 32, 40 (two row blocks), ragged suffixes
    for R in (2, 3, 7, 15, 16, 17, 31, 32, 33, 40, 70):
        pre = list(rng.integers(0, 50, size=int(rng.integers(1, 200))))
        seqs = [pre + [1000 + i] + list(rng.integers(0, 50, size=int(rng.integers(0, 150)))) for i in range(R)]
        cases[f"shared_R{R}"] = seqs
    # interior-ending sequences and duplicates
    base = list(rng.integers(0, 9, size=300))
    cases["interior_and_dups"] = [base[:70], base[:70], base, base[:128], base[:129], base[:1], base + [3, 3]]
    # a deep random tree: divergences inside chunks at many depths
    seqs = []
    for i in range(24):
        parent = seqs[int(rng.integers(0, len(seqs)))] if seqs else []
        cut = int(rng.integers(0, len(parent) + 1))
        seqs.append(parent[:cut] + [2000 + i] + list(rng.integers(0, 5, size=int(rng.integers(1, 180)))))
    cases["deep_random"] = seqs
    # single sequence of a single token; and all-private short sequences
    cases["single_token"] = [[5]]
    cases["all_private"] = [[100 * i + j for j in range(int(rng.integers(1, 140)))] for i in range(9)]
    return cases


@pytest.mark.parametrize("name", list(tiny_tree_cases()))
def test_tiny_trees(name):
    _say(f"tiny tree {name}")
    seqs = tiny_tree_cases()[name]
    wl = from_token_lists(seqs, heads=3, seed=len(name))
    ca = build_ca(wl)
    got = run_step(ca, wl.q)
    ref = A.decode_workload(wl)
    assert_parity(got, ref, name)


@pytest.mark.parametrize("cf_group,sf_group", [(1, 1), (2, 3), (8, 8), (16, 2), (64, 256)])
def test_task_sizes(cf_group, sf_group):
    _say(f"task sizes {cf_group} {sf_group}")
    wl = cached_config(1)
    ca = build_ca(wl, cf_group=cf_group, sf_group=sf_group)
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), f"cf{cf_group}/sf{sf_group}")
    seqs = tiny_tree_cases()["deep_random"]
    wl2 = from_token_lists(seqs, heads=2, seed=9)
    ca2 = build_ca(wl2, cf_group=cf_group, sf_group=sf_group)
    assert_parity(run_step(ca2, wl2.q), A.decode_workload(wl2), f"deep cf{cf_group}/sf{sf_group}")


def test_unshared_comparator_layout():
    _say("unshared")
    wl = cached_config(1)
    ca = build_ca(wl, share=False)
    st = ca.stats()
    assert st["shared_chunks"] == 0 and st["unique_tokens"] == wl.attended_tokens()
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), "unshared config1")


@pytest.mark.parametrize("name", ["config1", "config2", "deep_random", "interior_and_dups"])
def test_shared_pages_without_chunk_first(name):
    """PagedAttn*-style comparator: shared storage, every path streamed per sequence."""
    _say(f"no chunk-first {name}")
    if name.startswith("config"):
        wl = cached_config(int(name[-1]))
    else:
        wl = from_token_lists(tiny_tree_cases()[name], heads=3, seed=5)
    ca = build_ca(wl, two_phase=False)
    st = ca.stats()
    assert st["cf_units"] == 0
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), f"no-cf {name}")


def test_deterministic_bitwise():
    _say("determinism")
    wl = cached_config(1)
    ca = build_ca(wl)
    a = run_step(ca, wl.q)
    b = run_step(ca, wl.q)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_append_and_remove_between_steps():
    _say("append/remove")
    torch = _torch()
    rng = np.random.default_rng(3)
    H = 4
    pre = list(range(100))
    seqs = [pre + [500 + i] * int(rng.integers(1, 90)) for i in range(6)]
    wl = from_token_lists(seqs, heads=H, seed=11)
    ca = build_ca(wl, capacity=64)
    kv = {i: list(wl.seq_kv(i)) for i in range(wl.n_seq)}
    live = list(range(wl.n_seq))
    for step in range(6):
        # append 1..70 tokens to some sequences (in place and across chunk edges)
        for i in list(live):
            if rng.random() < 0.7:
                n = int(rng.integers(1, 70))
                k = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
                v = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
                ca.append(i, list(rng.integers(0, 9, size=n)), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
                kv[i][0] = np.concatenate([kv[i][0], k])
                kv[i][1] = np.concatenate([kv[i][1], v])
        if step == 2:
            ca.remove(live.pop(1))
        if step == 4:
            ca.remove(live.pop(0))
        q = rng.standard_normal((len(live), H, 128), dtype=np.float32).astype(np.float16)
        got = run_step(ca, q)
        ref = A.decode_step(q, [kv[i] for i in live])
        assert_parity(got, ref, f"append step {step}")


def test_phases_equal_fused_call():
    _say("phases")
    torch = _torch()
    from decode_attention_prefix_tree_amd import _capi
    wl = cached_config(1)
    ca = build_ca(wl)
    q = torch.from_numpy(wl.q).cuda()
    ref = ca.attend(q).clone()
    out = torch.empty_like(q)
    ca.prepare()
    for ph in (_capi.CA_PHASE_CHUNK_FIRST, _capi.CA_PHASE_SEQUENCE_FIRST, _capi.CA_PHASE_MERGE):
        ca.attend_phase(ph, q, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    out2 = torch.empty_like(q)
    for ph in (_capi.CA_PHASE_PARTIALS, _capi.CA_PHASE_MERGE):
        ca.attend_phase(ph, q, out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref)


def test_errors_on_device_context():
    _say("errors")
    torch = _torch()
    from decode_attention_prefix_tree_amd import CaError, ChunkAttention
    ca = ChunkAttention(2, 2, device="cuda:0")
    q = torch.zeros((0, 2, 128), dtype=torch.float16, device="cuda:0")
    with pytest.raises(CaError) as ei:
        ca.attend(q)
    assert ei.value.name == "empty"
    k = torch.zeros((200, 2, 128), dtype=torch.float16, device="cuda:0")
    with pytest.raises(CaError) as ei:
        ca.insert(1, list(range(200)), k, k)
    assert ei.value.name == "no_capacity"
    # a decode step with no query or output pointer changes nothing
    import ctypes
    ca.insert(1, list(range(40)), k[:40], k[:40])
    one = torch.ones((1, 2, 128), dtype=torch.float16, device="cuda:0")
    ca.attend(one)
    tok = (ctypes.c_int32 * 1)(7)
    p = ctypes.c_void_p(one.data_ptr())
    for qp, op in ((None, p), (p, None)):
        rc = ca.lib.ca_decode_step(ca.ctx, tok, p, p, qp, op, ca._stream())
        assert rc == -1, rc
    assert ca.stats()["unique_tokens"] == 40
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["config1", "shared_R70", "deep_random", "interior_and_dups"])
def test_fused_merge_matches_two_launch_step(name):
    """The one-launch step (merge blocks at the end of the grid) equals the
    partials + merge launches bit for bit, step after step (the arrival
    counters keep growing by each sequence's partial count) and after the
    tree changes (the upload restarts them)."""
    _say(f"fused merge {name}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import _capi
    if name == "config1":
        wl = cached_config(1)
    else:
        wl = from_token_lists(tiny_tree_cases()[name], heads=3, seed=21)
    ca = build_ca(wl, capacity=None)
    q = torch.from_numpy(np.ascontiguousarray(wl.q)).cuda()
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    ref = ca.attend(q).clone()
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    for _ in range(4):
        got = ca.attend(q)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
    assert_parity(got.cpu().numpy(), A.decode_workload(wl), f"fused {name}")
    # a tree change re-uploads the table (and zeroed counters)
    extra = [10**6 + j for j in range(70)]
    k = torch.zeros((70, wl.heads, 128), dtype=torch.float16, device="cuda:0")
    ca.insert(10**5, extra, k, k)
    q2 = torch.cat([q, torch.zeros((1, wl.heads, 128), dtype=torch.float16, device="cuda:0")])
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    ref2 = ca.attend(q2).clone()
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    for _ in range(3):
        assert torch.equal(ca.attend(q2), ref2)


def test_more_than_64_partials_per_sequence():
    """One private chunk per sequence-first task and long sequences: the merge
    folds more than 64 partials per (sequence, head) in several rounds."""
    _say("many partials")
    torch = _torch()
    from decode_attention_prefix_tree_amd import _capi
    rng = np.random.default_rng(8)
    shared = list(range(64 * 3 + 7))
    seqs = [shared + [9000 + i] + list(rng.integers(0, 7, size=64 * 70 + int(rng.integers(0, 64))))
            for i in range(3)]
    wl = from_token_lists(seqs, heads=2, seed=4)
    ca = build_ca(wl, cf_group=1, sf_group=1)
    assert ca.stats()["partials"] > 3 * 64
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    got = run_step(ca, wl.q)
    assert_parity(got, A.decode_workload(wl), "many partials")
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("k", [15, 16])
def test_dense_and_compact_partial_slots(k):
    """One shared run plus k private chunks (one per task) gives 1 + k
    partials: 16 keeps the dense partial slots, 17 switches to compact ids.
    Both merges against the oracle, and the one-launch step bit for bit."""
    _say(f"partial slots, k={k}")
    from decode_attention_prefix_tree_amd import _capi
    rng = np.random.default_rng(30 + k)
    shared = list(range(128))
    seqs = [shared + [9000 + i] + [int(x) for x in rng.integers(0, 7, size=64 * n - 1)]
            for i, n in enumerate((k, 3, 1))]
    wl = from_token_lists(seqs, heads=4, seed=31 + k)
    ca = build_ca(wl, cf_group=8, sf_group=1)
    st = ca.stats()
    assert st["partials"] == (3 * 16 if k == 15 else 3 + k + 3 + 1), st["partials"]
    got = run_step(ca, wl.q)
    assert_parity(got, A.decode_workload(wl), f"slots k={k}")
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("heads", [1, 64, 128])
def test_head_counts(heads):
    """One head and 64 heads (the kernels index heads only through the
    tile base and the record layout): a shared prefix with ragged private
    tails against the oracle, two launches and one launch bit for bit."""
    _say(f"heads={heads}")
    from decode_attention_prefix_tree_amd import _capi
    suffix = [int(x) for x in np.random.default_rng(40 + heads).integers(1, 300, size=12)]
    wl = make_prefix_suffix(700, suffix, heads=heads, seed=41 + heads)
    ca = build_ca(wl)
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    got = run_step(ca, wl.q)
    assert_parity(got, A.decode_workload(wl), f"heads={heads}")
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("mode", ["two_launch", "one_launch", "shared_pages"])
def test_decode_step_equals_append_then_attend(mode, chunk):
    """ca_decode_step (tokens written by the step's own blocks while chunks
    grow in place, a separate write launch when a chunk fills up or a
    sequence's last chunk is shared) against ca_append_batch + ca_attend on a
    twin context: the same bits at every one of 140 steps, the same tables,
    and the oracle over the grown sequences every 35 steps.  One sequence
    ends inside the shared prefix, so its first append grows a new chunk.
    With 128-token chunks the growing chunk also moves on to its second
    64-key tile (a new tile in the plan: a rebuild, not a patch); with 32,
    two sequences' chunks may share a tile and grow in the same step."""
    _say(f"decode step, {mode}, chunk {chunk}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import _capi
    rng = np.random.default_rng(50)
    H = 4
    shared = list(range(100))
    seqs = [shared + [5000 + i] + [int(x) for x in rng.integers(0, 9, size=n)]
            for i, n in enumerate((0, 30, 62, 63, 130, 10))]
    seqs.append(shared[:40])
    wl = from_token_lists(seqs, heads=H, seed=51)
    two_phase = mode != "shared_pages"
    from decode_attention_prefix_tree_amd import slots_needed
    cap = slots_needed(wl, chunk=chunk) + 40
    a = build_ca(wl, capacity=cap, two_phase=two_phase, chunk=chunk)
    b = build_ca(wl, capacity=cap, two_phase=two_phase, chunk=chunk)
    for ca in (a, b):
        ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1 if mode == "one_launch" else 0)
    n = wl.n_seq
    kv = [[x.copy() for x in wl.seq_kv(i)] for i in range(n)]
    for step in range(140):
        toks = (10**6 + step * 100 + np.arange(n)).astype(np.int32)
        k = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        q = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        kt, vt, qt = (torch.from_numpy(x).cuda() for x in (k, v, q))
        a.append_batch(list(range(n)), toks, kt, vt)
        ra = a.attend(qt).clone()
        rb = b.decode_step(toks, kt, vt, qt).clone()
        torch.cuda.synchronize()
        assert torch.equal(ra, rb), (mode, chunk, step)
        for i in range(n):
            kv[i][0] = np.concatenate([kv[i][0], k[i:i + 1]])
            kv[i][1] = np.concatenate([kv[i][1], v[i:i + 1]])
        if step % 35 == 0 or step == 139:
            assert_parity(rb.cpu().numpy(), A.decode_step(q, kv), f"decode {mode} chunk {chunk} step {step}")
    ta, oa = a.export_table()
    tb, ob = b.export_table()
    assert oa == ob and np.array_equal(ta, tb)
    st = b.stats()
    assert st["patched_appends"] >= 100, st


def _host_shadow(wl, two_phase):
    """A context without a device pool that receives the same tree calls: its
    exported table is the reference for the device context's."""
    from decode_attention_prefix_tree_amd import ChunkAttention
    sh = ChunkAttention(wl.heads, 4096, device=None, two_phase=two_phase)
    for i in range(wl.n_seq):
        sh.insert(i, wl.seq_tokens(i))
    return sh


def _same_table(a, b, label):
    ra, oa = a.export_table()
    rb, ob = b.export_table()
    assert oa == ob, label
    assert np.array_equal(ra, rb), label


@pytest.mark.parametrize("two_phase", [True, False])
def test_decode_progression_batched_appends(two_phase):
    """One token per sequence per step through ca_append_batch, attended each
    step and checked against the oracle on the sequences' full K/V.  Appends
    that land in place have their fill counts stored into the device table by
    the write launch (no upload); a chunk that fills up, or a removal, rebuilds
    and uploads the table.  The exported table matches a host-only context
    that saw the same calls."""
    _say(f"decode progression two_phase={two_phase}")
    torch = _torch()
    rng = np.random.default_rng(12)
    H = 2
    shared = list(range(130))
    seqs = [shared + [700 + i] * int(rng.integers(1, 40)) for i in range(7)]
    wl = from_token_lists(seqs, heads=H, seed=13)
    ca = build_ca(wl, capacity=80, two_phase=two_phase)
    sh = _host_shadow(wl, two_phase)
    kv = {i: list(wl.seq_kv(i)) for i in range(wl.n_seq)}
    live = list(range(wl.n_seq))
    for step in range(90):
        k = rng.standard_normal((len(live), H, 128), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((len(live), H, 128), dtype=np.float32).astype(np.float16)
        toks = list(rng.integers(0, 50, size=len(live)))
        ca.append_batch(live, toks, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        sh.append_batch(live, toks)
        for j, s in enumerate(live):
            kv[s][0] = np.concatenate([kv[s][0], k[j:j + 1]])
            kv[s][1] = np.concatenate([kv[s][1], v[j:j + 1]])
        if step == 45:
            ca.remove(live[2])
            sh.remove(live.pop(2))
        q = rng.standard_normal((len(live), H, 128), dtype=np.float32).astype(np.float16)
        got = run_step(ca, q)
        assert_parity(got, A.decode_step(q, [kv[s] for s in live]), f"decode step {step}")
        if step % 30 == 29:
            _same_table(ca, sh, f"table after step {step}")
    st = ca.stats()
    _say(f"uploads={st['table_uploads']} rebuilds={st['table_rebuilds']} patched={st['patched_appends']}")
    assert st["patched_appends"] > 60
    assert st["table_uploads"] <= st["table_rebuilds"] + 2
    _same_table(ca, sh, "final table")


@pytest.mark.parametrize("sf_group", [1, 8])
def test_patched_single_appends_deep_private_tails(sf_group):
    """ca_append of one token at a time onto sequences whose private tails span
    several chunks, so the growing chunk sits at every position of its task
    (with 8 chunks per task, past the refs carried inline in the record).
    Midway a fresh workspace is attached: that step uploads the host plan,
    whose fill counts were refreshed from the tree, and later appends patch
    the new copy."""
    _say(f"patched single appends sf_group={sf_group}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import _capi
    rng = np.random.default_rng(31)
    H = 3
    shared = list(range(70))
    seqs = [shared + [900 + i] * n for i, n in enumerate([3, 64 * 4 + 10, 64 * 6 + 62, 64 * 7 + 1])]
    wl = from_token_lists(seqs, heads=H, seed=32)
    ca = build_ca(wl, capacity=80, sf_group=sf_group)
    kv = {i: list(wl.seq_kv(i)) for i in range(wl.n_seq)}
    uploads0 = None
    for step in range(12):
        for s in range(wl.n_seq):
            k = rng.standard_normal((1, H, 128), dtype=np.float32).astype(np.float16)
            v = rng.standard_normal((1, H, 128), dtype=np.float32).astype(np.float16)
            ca.append(s, [5], torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
            kv[s][0] = np.concatenate([kv[s][0], k])
            kv[s][1] = np.concatenate([kv[s][1], v])
        if step == 6:
            ws = torch.empty(ca.ws.numel(), dtype=torch.uint8, device="cuda:0")
            torch.cuda.synchronize()
            ca.ws = ws
            assert ca.lib.ca_attach_workspace(ca.ctx, ws.data_ptr(), ws.numel()) == _capi.CA_OK
        q = rng.standard_normal((wl.n_seq, H, 128), dtype=np.float32).astype(np.float16)
        got = run_step(ca, q)
        assert_parity(got, A.decode_step(q, [kv[s] for s in range(wl.n_seq)]), f"step {step}")
        st = ca.stats()
        if step == 1:
            uploads0 = st["table_uploads"]
        if step > 1:
            # one upload when the 3rd sequence grows a new chunk (step 2),
            # one for the new workspace (step 6); the rest are patched
            assert st["table_uploads"] == uploads0 + (1 if step < 6 else 2), (step, st)
    assert ca.stats()["patched_appends"] >= 4 * 9


@pytest.mark.parametrize("chunk", [32, 128])
@pytest.mark.parametrize("two_phase", [True, False])
@pytest.mark.parametrize("name", ["shared_R40", "shared_R70", "deep_random", "interior_and_dups", "all_private",
                                  "single_token"])
def test_chunk_sizes_tiny_trees(name, two_phase, chunk):
    """128-token chunks are one or two 64-key tiles in the plan; 32-token
    chunks are halves of a tile (two chunks per tile, read half by half).
    Divergences split chunks anywhere."""
    _say(f"chunk {chunk} tiny tree {name} two_phase={two_phase}")
    seqs = tiny_tree_cases()[name]
    wl = from_token_lists(seqs, heads=3, seed=len(name) + chunk)
    ca = build_ca(wl, chunk=chunk, two_phase=two_phase)
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), f"c{chunk} {name}")


@pytest.mark.parametrize("chunk", [32, 128])
def test_chunk_sizes_non_aligned_prefix_ragged_suffixes(chunk):
    """A 1766-token shared prefix (ending mid-chunk at 32 and at 128) with
    suffixes of 1..700 tokens, 8 heads, against the oracle."""
    rng = np.random.default_rng(2128)
    suffix = [int(x) for x in rng.integers(1, 701, size=40)]
    wl = make_prefix_suffix(1766, suffix, heads=8, seed=2129)
    _say(f"chunk {chunk} prefix 1766 + ragged suffixes")
    ca = build_ca(wl, chunk=chunk)
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), f"c{chunk} prefix1766 ragged")


def _k_off(key, dim):
    """Position of K[key][dim] in a 64-key tile (the MFMA A-operand order)."""
    return ((((key >> 5) * 8 + (dim >> 4)) * 2 + ((dim >> 3) & 1)) * 32 + (key & 31)) * 8 + (dim & 7)


def _v_off(key, dim):
    """Position of V[key][dim] in a 64-key tile."""
    return ((((dim >> 5) * 4 + (key >> 4)) * 2 + ((key >> 2) & 1)) * 32 + (dim & 31)) * 8 + \
        ((key & 3) | (((key >> 3) & 1) << 2))


def _pool_tiles(ca, heads):
    """The pool as [tile][head][K|V][64 x 128 halves]: tiles lie
    ca_slot_bytes(heads, 128, 64) apart (one head's pair more when the head
    count is a power of two from 16 up), heads and K/V contiguous inside a
    tile."""
    from decode_attention_prefix_tree_amd import slot_bytes
    torch = _torch()
    flat = ca.pool.view(torch.float16).cpu().numpy()
    stride = slot_bytes(heads, 128, 64) // 2
    used = heads * 2 * 64 * 128
    assert stride >= used
    return flat[:flat.size // stride * stride].reshape(-1, stride)[:, :used].reshape(-1, heads, 2, 64 * 128)


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("name", ["deep_random", "interior_and_dups"])
def test_pool_holds_each_chunks_kv(name, chunk):
    """KV scatter: after the inserts (divergences split chunks anywhere, so
    split tails are copied pool to pool, across tile boundaries at 128), key
    j of every table row sits at global pool key slot * chunk + j, in tile
    order, bit for bit equal to the caller's K and V of that token."""
    _say(f"pool contents {name} chunk {chunk}")
    wl = from_token_lists(tiny_tree_cases()[name], heads=3, seed=9)
    ca = build_ca(wl, chunk=chunk)
    rows, order = ca.export_table()
    pool = _pool_tiles(ca, wl.heads)
    keys = np.arange(64)[:, None]
    dims = np.arange(128)[None, :]
    koff, voff = _k_off(keys, dims), _v_off(keys, dims)
    n_keys = 0
    for r in rows:
        start, n, sb, slot = int(r[2]), int(r[3]), int(r[4]), int(r[6])
        k, v = wl.seq_kv(order[sb])
        for j in range(n):
            t, kk = divmod(slot * chunk + j, 64)
            assert np.array_equal(pool[t][:, 0][:, koff[kk]], k[start + j]), (r, j)
            assert np.array_equal(pool[t][:, 1][:, voff[kk]], v[start + j]), (r, j)
            n_keys += 1
    assert n_keys == sum(int(r[3]) for r in rows)


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_pool_room_past_the_heads_is_never_written(chunk):
    """With a power-of-two head count from 16 up each pool tile has one
    head's K/V room more than its heads use.  Inserts (splits, pool-to-pool copies), decode
    steps (tokens stored by the step, chunks opened), an insert that shares
    decoded chunks (their conversion to tiles) and a removal leave that room
    as it was, and the output still matches the oracle."""
    _say(f"pool room past the heads, chunk {chunk}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slot_bytes, slots_needed
    H = 16
    rng = np.random.default_rng(700 + chunk)
    shared = list(range(150))
    seqs = [shared + [9000 + i] + [int(x) for x in rng.integers(0, 9, size=n)] for i, n in enumerate((3, 40, 77))]
    seqs.append(shared[:70])
    wl = from_token_lists(seqs, heads=H, seed=701)
    cap = slots_needed(wl, chunk=chunk) + 40
    ca = ChunkAttention(H, cap, device="cuda:0", chunk_size=chunk)
    sentinel = 0x5A5A
    ca.pool.view(torch.int16).fill_(sentinel)
    load_workload(ca, wl, device="cuda:0")
    toks = {i: [int(t) for t in wl.seq_tokens(i)] for i in range(wl.n_seq)}
    kv = {i: [x.copy() for x in wl.seq_kv(i)] for i in range(wl.n_seq)}
    ids = list(range(wl.n_seq))

    def steps(n_steps, base):
        q = None
        for step in range(n_steps):
            t = (base + step * 100 + np.arange(len(ids))).astype(np.int32)
            k = rng.standard_normal((len(ids), H, 128), dtype=np.float32).astype(np.float16)
            v = rng.standard_normal((len(ids), H, 128), dtype=np.float32).astype(np.float16)
            q = rng.standard_normal((len(ids), H, 128), dtype=np.float32).astype(np.float16)
            out = ca.decode_step(t, *(torch.from_numpy(x).cuda() for x in (k, v, q)))
            for r, i in enumerate(ids):
                toks[i].append(int(t[r]))
                kv[i][0] = np.concatenate([kv[i][0], k[r:r + 1]])
                kv[i][1] = np.concatenate([kv[i][1], v[r:r + 1]])
        torch.cuda.synchronize()
        return q, out.cpu().numpy()

    steps(70, 10**6)
    # a new sequence that shares sequence 1's decoded tokens up to the middle
    # of a grown chunk, then diverges
    cut = len(toks[1]) - 23
    new_tok = toks[1][:cut] + [777000 + j for j in range(9)]
    nk = rng.standard_normal((9, H, 128), dtype=np.float32).astype(np.float16)
    nv = rng.standard_normal((9, H, 128), dtype=np.float32).astype(np.float16)
    k_new = np.concatenate([kv[1][0][:cut], nk])
    v_new = np.concatenate([kv[1][1][:cut], nv])
    ca.insert(10, np.asarray(new_tok, np.int32), torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda())
    toks[10] = new_tok
    kv[10] = [k_new, v_new]
    ca.remove(2)
    ids = [0, 1, 3, 10]
    q, got = steps(40, 2 * 10**6)
    assert_parity(got, A.decode_step(q, [kv[i] for i in ids]), f"pool room chunk {chunk}")
    flat = ca.pool.view(torch.int16).cpu().numpy()
    stride = slot_bytes(H, 128, 64) // 2
    used = H * 2 * 64 * 128
    assert stride == (H + 1) * 2 * 64 * 128
    tiles = flat[:flat.size // stride * stride].reshape(-1, stride)
    assert (tiles[:, used:] == sentinel).all(), np.argwhere(tiles[:, used:] != sentinel)[:4]


def _k_row_off(key, dim):
    """Position of K[key][dim] of a row-major chunk in its 64-key tile."""
    return key * 128 + dim


def _v_row_off(key, dim):
    """Position of V[key][dim] of a row-major chunk in its 64-key tile: rows
    of keys 0..31 and 32..63 stay inside the V units of their tile half."""
    return (4 * ((key & 31) >> 3) + 2 * (key >> 5)) * 512 + (key & 7) * 128 + dim


def _check_pool(ca, heads, chunk, kv_of, row_rows):
    """Every key of every table row against the K/V the caller supplied:
    table rows in row_rows are read in the row layout, the others in the tile
    layout."""
    rows, order = ca.export_table()
    pool = _pool_tiles(ca, heads)
    keys = np.arange(64)[:, None]
    dims = np.arange(128)[None, :]
    offs = {False: (_k_off(keys, dims), _v_off(keys, dims)), True: (_k_row_off(keys, dims), _v_row_off(keys, dims))}
    n_keys = 0
    for ri, r in enumerate(rows):
        start, n, sb, slot = int(r[2]), int(r[3]), int(r[4]), int(r[6])
        k, v = kv_of(order[sb])
        koff, voff = offs[ri in row_rows]
        for j in range(n):
            t, kk = divmod(slot * chunk + j, 64)
            assert np.array_equal(pool[t][:, 0][:, koff[kk]], k[start + j]), (ri, r, j)
            assert np.array_equal(pool[t][:, 1][:, voff[kk]], v[start + j]), (ri, r, j)
            n_keys += 1
    assert n_keys == sum(int(r[3]) for r in rows)
    return rows, order


def _check_pool_either_layout(ca, heads, chunk, kv_of):
    """Every key of every table row against the caller's K/V, reading each
    chunk in the layout (row-major or tiles) in which all its keys match:
    after removals the layout of a chunk is not known from the table alone,
    and a chunk whose keys match in neither fails."""
    rows, order = ca.export_table()
    pool = _pool_tiles(ca, heads)
    keys = np.arange(64)[:, None]
    dims = np.arange(128)[None, :]
    layouts = [(_k_off(keys, dims), _v_off(keys, dims)), (_k_row_off(keys, dims), _v_row_off(keys, dims))]
    for r in rows:
        start, n, sb, slot = int(r[2]), int(r[3]), int(r[4]), int(r[6])
        k, v = kv_of(order[sb])
        ok = False
        for koff, voff in layouts:
            good = True
            for j in range(n):
                t, kk = divmod(slot * chunk + j, 64)
                if not (np.array_equal(pool[t][:, 0][:, koff[kk]], k[start + j]) and
                        np.array_equal(pool[t][:, 1][:, voff[kk]], v[start + j])):
                    good = False
                    break
            ok = ok or good
        assert ok, r


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_pool_rows_of_appended_chunks_and_their_conversion(chunk):
    """Chunks made by appends hold their keys row-major (ca_stats counts
    them), chunks made by inserts hold tiles; an insert that shares a
    sequence's appended chunks, and one that diverges inside one of them,
    first rewrite those chunks as tiles.  Every key is compared with the
    caller's K/V bit for bit after each stage, and each step with the
    oracle."""
    _say(f"row chunks and conversions, chunk {chunk}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention
    rng = np.random.default_rng(500 + chunk)
    H = 2
    ca = ChunkAttention(H, 64, device="cuda:0", chunk_size=chunk)
    toks, kvs = {}, {}

    def rnd_kv(n):
        return [rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16) for _ in range(2)]

    def put(sid, t, k, v):
        ca.insert(sid, t, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        toks[sid], kvs[sid] = list(t), [k, v]

    base = [int(x) for x in rng.integers(0, 50, size=2 * chunk)]
    kb, vb = rnd_kv(2 * chunk)
    put(0, base, kb, vb)
    k1, v1 = rnd_kv(chunk)
    put(1, base[:chunk] + [777] * chunk, np.concatenate([kb[:chunk], k1]), np.concatenate([vb[:chunk], v1]))
    inserted = {0: 2 * chunk, 1: 2 * chunk}
    # appends: single tokens and a multi-token append, crossing chunk ends
    for step in range(chunk + 7):
        for sid in (0, 1):
            n = 3 if step == 5 else 1
            k, v = rnd_kv(n)
            t = [1000 + step * 10 + j for j in range(n)]
            ca.append(sid, t, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
            toks[sid] += t
            kvs[sid] = [np.concatenate([kvs[sid][0], k]), np.concatenate([kvs[sid][1], v])]
    torch.cuda.synchronize()
    st = ca.stats()
    assert st["row_chunks"] >= 4, st["row_chunks"]

    def rows_in_row_layout(rows, order, row_seqs):
        # chunks that only appends made: past the inserted length of a sequence in row_seqs
        out = set()
        for ri, r in enumerate(rows):
            if r[5] - r[4] == 1 and order[r[4]] in row_seqs and r[2] >= inserted[order[r[4]]]:
                out.add(ri)
        return out

    def check(row_seqs, label):
        rows, order = ca.export_table()
        rr = rows_in_row_layout(rows, order, row_seqs)
        _check_pool(ca, H, chunk, lambda s: kvs[s], rr)
        q = rng.standard_normal((len(toks), H, 128), dtype=np.float32).astype(np.float16)
        got = run_step(ca, q)
        ids = sorted(toks)
        assert_parity(got, A.decode_step(q, [kvs[s] for s in ids]), label)
        return len(rr)

    assert check({0, 1}, "appended chunks in rows") == st["row_chunks"]
    # sequence 2 shares all of sequence 0 (its appended chunks become shared)
    put(2, list(toks[0]), *[x.copy() for x in kvs[0]])
    assert ca.stats()["row_chunks"] < st["row_chunks"]
    check({1}, "after sharing sequence 0's chunks")
    # sequence 3 diverges inside sequence 1's last appended chunk
    cut = len(toks[1]) - 3
    k3, v3 = rnd_kv(5)
    put(3, toks[1][:cut] + [4242] * 5, np.concatenate([kvs[1][0][:cut], k3]), np.concatenate([kvs[1][1][:cut], v3]))
    check(set(), "after splitting sequence 1's last chunk")
    assert ca.stats()["row_chunks"] == 0


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("rows_on", [1, 0])
def test_decode_with_inserts_into_decoded_chunks(chunk, rows_on):
    """Decode steps (ca_decode_step) interleaved with inserts of sequences
    that copy a prefix of a decoding sequence, cut anywhere (sharing its
    appended chunks, or splitting one), and removals; every step against the
    oracle, with row-major appended chunks on and off."""
    _say(f"decode with inserts, chunk {chunk}, rows {rows_on}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    rng = np.random.default_rng(600 + chunk + rows_on)
    H = 2
    ca = ChunkAttention(H, 400, device="cuda:0", chunk_size=chunk)
    ca.set_option(_capi.CA_OPT_ROW_APPENDS, rows_on)
    live = {}
    nid = [0]

    def rnd(n):
        return rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)

    def insert(t, k, v):
        sid = nid[0]
        nid[0] += 1
        ca.insert(sid, t, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        live[sid] = (list(t), k, v)

    pre = [int(x) for x in rng.integers(0, 30, size=100)]
    kp, vp = rnd(100), rnd(100)
    for i in range(3):
        n = int(rng.integers(1, 70))
        insert(pre + [900 + i] * n, np.concatenate([kp, rnd(n)]), np.concatenate([vp, rnd(n)]))
    for step in range(150):
        ids = sorted(live)
        k, v, q = rnd(len(ids)), rnd(len(ids)), rnd(len(ids))
        # distinct token ids per (step, sequence), so an insert that copies a
        # prefix follows its source's path and carries the same K/V
        t = [100_000 + 64 * step + j for j in range(len(ids))]
        out = ca.decode_step(np.array(t, np.int32), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                             torch.from_numpy(q).cuda())
        for j, s_ in enumerate(ids):
            tt, kk, vv = live[s_]
            live[s_] = (tt + [t[j]], np.concatenate([kk, k[j:j + 1]]), np.concatenate([vv, v[j:j + 1]]))
        if step % 10 == 0 or step == 149:
            torch.cuda.synchronize()
            assert_parity(out.cpu().numpy(), A.decode_step(q, [live[s_][1:] for s_ in ids]), f"decode {step}")
        if step % 17 == 8:
            src = live[ids[int(rng.integers(0, len(ids)))]]
            cut = int(rng.integers(1, len(src[0]) + 1))
            extra = int(rng.integers(0, 4))
            insert(src[0][:cut] + [5000 + step] * extra, np.concatenate([src[1][:cut], rnd(extra)]),
                   np.concatenate([src[2][:cut], rnd(extra)]))
        if step % 29 == 20 and len(live) > 2:
            victim = ids[int(rng.integers(0, len(ids)))]
            ca.remove(victim)
            del live[victim]
    assert (ca.stats()["row_chunks"] > 0) == bool(rows_on)


def test_one_sequence_of_65536_tokens():
    """The longest single context here: one private sequence of 65,536 tokens
    (1,024 chunks, 256 sequence-first tasks per head, 256 partials merged
    through the compact list), 8 heads, against the oracle."""
    _say("one sequence of 65536 tokens")
    wl = make_long_sequence(65536, heads=8, seed=65536)
    ca = build_ca(wl)
    assert ca.stats()["partials"] == 256
    assert_parity(run_step(ca, wl.q), A.decode_workload(wl), "65536 tokens")


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_256_sequences_one_launch(chunk):
    """A large batch: 256 sequences x 16 heads (4,096 merges, so the default
    step is one launch) sharing a 2,048-token prefix, private suffixes of
    1..300 tokens, at each chunk size; every row against the oracle and
    against the two-launch step bit for bit."""
    _say(f"256 sequences, one launch, chunk {chunk}")
    from decode_attention_prefix_tree_amd import _capi
    rng = np.random.default_rng(256)
    wl = make_prefix_suffix(2048, [int(x) for x in rng.integers(1, 301, size=256)], heads=16, seed=257)
    ca = build_ca(wl, chunk=chunk)
    assert ca.stats()["one_launch_step"] == 1
    got = run_step(ca, wl.q)
    assert_parity(got, A.decode_workload(wl), f"256 seq, chunk {chunk}")
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    assert np.array_equal(run_step(ca, wl.q).view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("chunk", [32, 64])
def test_decode_step_growing_chunk_past_inline_refs(chunk):
    """ca_decode_step with 16 private refs per sequence-first task and private
    tails of 5..11 chunks: the chunk that takes each step's token sits past
    the 4 refs a task record carries inline, so the step's blocks read and
    grow its fill count in the chunk table.  Same bits as append + attend at
    every one of 70 steps, oracle every 35."""
    _say(f"decode step past inline refs, chunk {chunk}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import _capi, slots_needed
    rng = np.random.default_rng(61)
    H = 2
    shared = list(range(70))
    seqs = [shared + [9000 + i] + [int(x) for x in rng.integers(0, 7, size=n)]
            for i, n in enumerate((300, 450, 700, 520, 333))]
    wl = from_token_lists(seqs, heads=H, seed=62)
    cap = slots_needed(wl, chunk=chunk) + 40
    a = build_ca(wl, capacity=cap, chunk=chunk, sf_group=16)
    b = build_ca(wl, capacity=cap, chunk=chunk, sf_group=16)
    n = wl.n_seq
    kv = [[x.copy() for x in wl.seq_kv(i)] for i in range(n)]
    for step in range(70):
        toks = (2 * 10**6 + step * 100 + np.arange(n)).astype(np.int32)
        k = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        q = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        kt, vt, qt = (torch.from_numpy(x).cuda() for x in (k, v, q))
        a.append_batch(list(range(n)), toks, kt, vt)
        ra = a.attend(qt).clone()
        rb = b.decode_step(toks, kt, vt, qt).clone()
        torch.cuda.synchronize()
        assert torch.equal(ra, rb), (chunk, step)
        for i in range(n):
            kv[i][0] = np.concatenate([kv[i][0], k[i:i + 1]])
            kv[i][1] = np.concatenate([kv[i][1], v[i:i + 1]])
        if step % 35 == 0 or step == 69:
            assert_parity(rb.cpu().numpy(), A.decode_step(q, kv), f"decode past inline chunk {chunk} step {step}")
    st = b.stats()
    assert st["sf_chunks_per_task"] == 16 and st["patched_appends"] >= 40, st


def test_one_launch_merge_that_gives_up_writes_nan():
    """The one-launch step's merge waits for its partials for a bounded number
    of polls.  With the bound cut to one poll from the host, merge waves whose
    producers are still running give up: every (sequence, head) is then either
    the two-launch result bit for bit or all NaN, never a merge of incomplete
    partials.  With the default bound restored the next step is exact."""
    _say("one-launch merge with a one-poll wait")
    from decode_attention_prefix_tree_amd import _capi
    wl = cached_config(2)
    ca = build_ca(wl)
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    ref = run_step(ca, wl.q)
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    ca.set_option(_capi.CA_OPT_MERGE_POLL_LIMIT, 1)
    got = run_step(ca, wl.q)
    nan_pairs = 0
    for s_ in range(wl.n_seq):
        for h in range(wl.heads):
            if np.isnan(got[s_, h].astype(np.float32)).all():
                nan_pairs += 1
            else:
                assert np.array_equal(got[s_, h].view(np.uint16), ref[s_, h].view(np.uint16)), (s_, h)
    _say(f"pairs that gave up: {nan_pairs} of {wl.n_seq * wl.heads}")
    ca.set_option(_capi.CA_OPT_MERGE_POLL_LIMIT, 0)
    for _ in range(2):
        assert np.array_equal(run_step(ca, wl.q).view(np.uint16), ref.view(np.uint16))


def test_random_trees_options_and_decode_steps():
    """30 seeded random trees (1..40 sequences, each a prefix of an earlier one
    cut anywhere plus a fresh tail, so divergences split chunks at every
    depth) at random chunk sizes, head counts, launch modes, task groups and
    with or without the chunk-first phase; each attended and then advanced by
    up to three decode steps, every result against the oracle."""
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, load_workload, slots_needed, _capi
    rng = np.random.default_rng(4242)
    for case in range(30):
        seqs = []
        for i in range(int(rng.integers(1, 41))):
            if seqs and rng.random() < 0.7:
                parent = seqs[int(rng.integers(0, len(seqs)))]
                cut = int(rng.integers(0, len(parent) + 1))
            else:
                parent, cut = [], 0
            seqs.append(parent[:cut] + [10000 + i] + [int(x) for x in rng.integers(0, 6, size=int(rng.integers(0, 400)))])
        heads = int(rng.choice([1, 2, 3, 5, 8]))
        chunk = int(rng.choice([32, 64, 128]))
        fused, cfg, sfg = int(rng.choice([0, 1, 2])), int(rng.choice([0, 1, 2, 4, 16])), int(rng.choice([0, 1, 3, 4, 16]))
        two_phase = bool(rng.random() < 0.85)
        label = (f"random case {case}: {len(seqs)} seq, {heads} heads, chunk {chunk}, fused {fused}, "
                 f"cf {cfg}, sf {sfg}, two_phase {two_phase}")
        _say(label)
        wl = from_token_lists(seqs, heads=heads, seed=int(rng.integers(0, 1 << 30)))
        ca = ChunkAttention(heads, slots_needed(wl, chunk=chunk) + 8 + 4 * wl.n_seq, device="cuda:0",
                            two_phase=two_phase, chunk_size=chunk)
        ca.set_option(_capi.CA_OPT_FUSED_MERGE, fused)
        ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, cfg)
        ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, sfg)
        load_workload(ca, wl, device="cuda:0")
        assert_parity(run_step(ca, wl.q), A.decode_workload(wl), label)
        kv = [[x.copy() for x in wl.seq_kv(i)] for i in range(wl.n_seq)]
        n = wl.n_seq
        for step in range(int(rng.integers(0, 4))):
            k = rng.standard_normal((n, heads, 128), dtype=np.float32).astype(np.float16)
            v = rng.standard_normal((n, heads, 128), dtype=np.float32).astype(np.float16)
            q = rng.standard_normal((n, heads, 128), dtype=np.float32).astype(np.float16)
            toks = (3 * 10**6 + step * 1000 + np.arange(n)).astype(np.int32)
            out = ca.decode_step(toks, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(q).cuda())
            torch.cuda.synchronize()
            for i in range(n):
                kv[i][0] = np.concatenate([kv[i][0], k[i:i + 1]])
                kv[i][1] = np.concatenate([kv[i][1], v[i:i + 1]])
            assert_parity(out.cpu().numpy(), A.decode_step(q, kv), f"{label}, decode step {step}")
        del ca


def test_workspace_too_small():
    """With a workspace below ca_workspace_bytes, ca_attend returns
    CA_E_WORKSPACE and launches nothing; ca_decode_step returns it after the
    tokens were stored, and attaching a large enough workspace and calling
    ca_attend finishes that step (oracle over the grown sequences)."""
    _say("workspace too small")
    torch = _torch()
    import ctypes
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    rng = np.random.default_rng(77)
    seqs = [list(range(100)) + [500 + i] * int(rng.integers(1, 90)) for i in range(6)]
    wl = from_token_lists(seqs, heads=2, seed=78)
    ca = build_ca(wl, capacity=64)
    lib, ctx = ca.lib, ca.ctx
    need = ctypes.c_size_t(0)
    assert lib.ca_workspace_bytes(ctx, ctypes.byref(need)) == 0 and need.value > 4096
    tiny = torch.empty(4096, dtype=torch.uint8, device="cuda:0")
    assert lib.ca_attach_workspace(ctx, ctypes.c_void_p(tiny.data_ptr()), tiny.numel()) == 0
    q = torch.from_numpy(np.ascontiguousarray(wl.q)).cuda()
    out = torch.zeros_like(q)
    rc = lib.ca_attend(ctx, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr()), ca._stream())
    torch.cuda.synchronize()
    assert rc == -7 and not out.any()
    # a decode step: the tokens are stored, the attention is not run
    n = wl.n_seq
    k = rng.standard_normal((n, 2, 128), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, 2, 128), dtype=np.float32).astype(np.float16)
    q2 = rng.standard_normal((n, 2, 128), dtype=np.float32).astype(np.float16)
    kt, vt, qt = (torch.from_numpy(x).cuda() for x in (k, v, q2))
    toks = (ctypes.c_int32 * n)(*range(9000, 9000 + n))
    before = ca.stats()["unique_tokens"]
    rc = lib.ca_decode_step(ctx, toks, ctypes.c_void_p(kt.data_ptr()), ctypes.c_void_p(vt.data_ptr()),
                            ctypes.c_void_p(qt.data_ptr()), ctypes.c_void_p(out.data_ptr()), ca._stream())
    assert rc == -7
    assert ca.stats()["unique_tokens"] == before + n
    assert lib.ca_workspace_bytes(ctx, ctypes.byref(need)) == 0
    big = torch.empty(need.value, dtype=torch.uint8, device="cuda:0")
    assert lib.ca_attach_workspace(ctx, ctypes.c_void_p(big.data_ptr()), big.numel()) == 0
    rc = lib.ca_attend(ctx, ctypes.c_void_p(qt.data_ptr()), ctypes.c_void_p(out.data_ptr()), ca._stream())
    torch.cuda.synchronize()
    assert rc == 0
    kv = [[np.concatenate([a, b[i:i + 1]]) for a, b in zip(wl.seq_kv(i), (k, v))] for i in range(n)]
    assert_parity(out.cpu().numpy(), A.decode_step(q2, kv), "after growing the workspace")
    ca.ws = big  # keep it alive with the context


@pytest.mark.parametrize("fused", [0, 1])
def test_captured_step_replays_equal_eager_steps(fused):
    """A step captured in a HIP graph (torch.cuda.graph around ca_attend) and
    replayed with new queries copied into the captured q: every replay equals
    an eager step on the same q bit for bit and matches the oracle, with eager
    steps and host syncs between replays; tokens appended in place between
    replays (fill counts stored on the device) are seen by the replays.  In
    the one-launch step nothing carries over between replays (arrival
    counters return to zero).  A step that would upload the table while the
    stream captures is refused (CA_E_STATE), and so is every call that
    changes the tree, which then stays as it was."""
    _say(f"graph capture, fused={fused}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import CaError, _capi
    rng = np.random.default_rng(400 + fused)
    wl = make_prefix_suffix(200, [int(x) for x in rng.integers(5, 50, size=24)], heads=4, seed=401)
    ca = build_ca(wl, capacity=80)
    ca.set_option(_capi.CA_OPT_FUSED_MERGE, fused)
    twin = build_ca(wl, capacity=80)
    n, H = wl.n_seq, wl.heads
    q = torch.from_numpy(wl.q).cuda()
    out = torch.empty_like(q)
    ca.ensure_workspace()
    ca.attend(q, out)  # the table is on the device: the step only launches kernels
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ca.attend(q, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ca.attend(q, out)
    torch.cuda.synchronize()
    kv = [[x.copy() for x in wl.seq_kv(i)] for i in range(n)]
    for rep in range(6):
        if rep in (2, 4):
            # one token per sequence, in place (every last chunk has room)
            k = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
            v = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
            kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
            toks = np.full(n, 9000 + rep, np.int32)
            ca.append_batch(list(range(n)), toks, kt, vt)
            twin.append_batch(list(range(n)), toks, kt, vt)
            for i in range(n):
                kv[i] = [np.concatenate([a, b[i:i + 1]]) for a, b in zip(kv[i], (k, v))]
        qn = rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)
        q.copy_(torch.from_numpy(qn).cuda())
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        eager = run_step(twin, qn)
        assert np.array_equal(got.view(np.uint16), eager.view(np.uint16)), rep
        assert_parity(got, A.decode_step(qn, kv), f"graph replay {rep}")
    assert ca.stats()["table_uploads"] == 1
    # a structural change: the next step must upload, which a capture refuses
    ca.insert(n, list(range(40)), torch.zeros((40, H, 128), dtype=torch.float16, device="cuda:0"),
              torch.zeros((40, H, 128), dtype=torch.float16, device="cuda:0"))
    q2 = torch.zeros((n + 1, H, 128), dtype=torch.float16, device="cuda:0")
    out2 = torch.empty_like(q2)
    ca.ensure_workspace()
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(CaError) as ei:
        with torch.cuda.graph(g2):
            ca.attend(q2, out2)
    assert ei.value.name == "state"
    torch.cuda.synchronize()
    ca.attend(q2, out2)
    torch.cuda.synchronize()
    assert torch.isfinite(out2).all()
    # calls that change the tree refuse a capturing stream and change nothing
    table = ca.export_table()
    kz = torch.zeros((n + 1, H, 128), dtype=torch.float16, device="cuda:0")
    attempts = [lambda: ca.decode_step(np.zeros(n + 1, np.int32), kz, kz, q2, out2),
                lambda: ca.append_batch(list(range(n + 1)), np.zeros(n + 1, np.int32), kz, kz),
                lambda: ca.append(0, [5], kz[:1], kz[:1]),
                lambda: ca.insert(n + 7, [1, 2, 3], kz[:3], kz[:3])]
    for call in attempts:
        g3 = torch.cuda.CUDAGraph()
        with pytest.raises(CaError) as ei:
            with torch.cuda.graph(g3):
                call()
        assert ei.value.name == "state"
        torch.cuda.synchronize()
        after = ca.export_table()
        assert all(np.array_equal(x, y) for x, y in zip(table, after))
    ca.decode_step(np.zeros(n + 1, np.int32), kz, kz, q2, out2)
    torch.cuda.synchronize()
    assert torch.isfinite(out2).all()


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("rows_on", [1, 0])
def test_tables_built_and_uploaded_ahead(chunk, rows_on):
    """Decode steps with tables built ahead (and copied into the workspace
    after the step that built them, with each sequence's last chunk at its
    fill before the next token) against a twin context that builds and
    uploads every table in the step that needs it: bit for bit at every step,
    through structural steps (last chunks fill up at different steps; the
    step's own blocks store the tokens of the chunks they open when those are
    row-major, the write launch otherwise), an insert that makes a prediction
    stale, and extra ca_attend calls between steps that upload the current
    table over the one copied ahead; the oracle every few steps, and every
    stored key against the caller's K/V at the end."""
    _say(f"tables built ahead, chunk {chunk}, rows {rows_on}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    rng = np.random.default_rng(800 + chunk)
    H = 2
    cas = [ChunkAttention(H, 300, device="cuda:0", chunk_size=chunk) for _ in range(2)]
    cas[1].set_option(_capi.CA_OPT_PREBUILD_PLAN, 0)
    for ca in cas:
        ca.set_option(_capi.CA_OPT_ROW_APPENDS, rows_on)
    live, inserted = {}, {}

    def rnd(n):
        return rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)

    def insert(sid, t, k, v):
        for ca in cas:
            ca.insert(sid, t, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        live[sid] = (list(t), k, v)
        inserted[sid] = len(t)

    pre = list(range(3 * chunk))
    kp, vp = rnd(3 * chunk), rnd(3 * chunk)
    for i, n in enumerate((0, 5, chunk - 1, chunk // 2)):
        insert(i, pre + [700 + i] * n, np.concatenate([kp, rnd(n)]), np.concatenate([vp, rnd(n)]))
    for step in range(3 * chunk + 10):
        ids = sorted(live)
        k, v, q = rnd(len(ids)), rnd(len(ids)), rnd(len(ids))
        t = np.array([int(x) for x in rng.integers(0, 40, size=len(ids))], np.int32)
        outs = [ca.decode_step(t, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                               torch.from_numpy(q).cuda()).cpu().numpy() for ca in cas]
        assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16)), step
        for j, s_ in enumerate(ids):
            tt, kk, vv = live[s_]
            live[s_] = (tt + [int(t[j])], np.concatenate([kk, k[j:j + 1]]), np.concatenate([vv, v[j:j + 1]]))
        if step % 23 == 0:
            assert_parity(outs[0], A.decode_step(q, [live[s_][1:] for s_ in ids]), f"ahead {step}")
        if step % 31 == 7:
            # a step of attention alone: it uploads the current table (over a
            # table copied ahead for the next tree, if any)
            q2 = rnd(len(ids))
            o2 = [ca.attend(torch.from_numpy(q2).cuda()).cpu().numpy() for ca in cas]
            assert np.array_equal(o2[0].view(np.uint16), o2[1].view(np.uint16)), step
        if step == 2 * chunk:
            src = live[1]
            insert(9, src[0][:chunk + 3] + [4321], np.concatenate([src[1][:chunk + 3], rnd(1)]),
                   np.concatenate([src[2][:chunk + 3], rnd(1)]))
    st, st1 = cas[0].stats(), cas[1].stats()
    assert st["prebuilt_plans"] >= 3 and st1["prebuilt_plans"] == 0
    assert st["table_uploads"] < st1["table_uploads"] + 4
    # the structural steps that found their table in place stored their
    # fill counts there instead of uploading a new table
    assert st["patched_appends"] >= st1["patched_appends"] + 3, (st["patched_appends"], st1["patched_appends"])
    for ca in cas:
        rows, order = ca.export_table()
        # chunks that appends opened: private, past the sequence's inserted length
        rr = {ri for ri, r in enumerate(rows)
              if rows_on and r[5] - r[4] == 1 and r[2] >= inserted[order[r[4]]]}
        _check_pool(ca, H, chunk, lambda s_: live[s_][1:], rr)


@pytest.mark.parametrize("chunk,mode", [(32, "tree"), (64, "tree"), (128, "tree"), (64, "unshared"),
                                        (64, "no_chunk_first")])
def test_decode_loop_with_churn_matches_a_twin_without_tables_ahead(chunk, mode):
    """A randomized serving loop on two contexts, one building (and copying)
    tables ahead and one not: decode steps, append_batch + attend steps,
    attention alone, inserts that share a decoding sequence's prefix cut
    anywhere, and removals, in random order over 260 steps.  Both contexts
    must give the same output bit for bit at every step and the same chunk
    table; the oracle checks every 20th step, and every stored key is
    compared with the caller's K/V at the end.  Also with the unshared layout
    and with the prefix tree but no chunk-first phase."""
    _say(f"serving loop with churn, chunk {chunk}, {mode}")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    rng = np.random.default_rng(1200 + chunk)
    H = 2
    cas = [ChunkAttention(H, 500 if mode != "unshared" else 900, device="cuda:0", chunk_size=chunk,
                          share=mode != "unshared", two_phase=mode != "no_chunk_first") for _ in range(2)]
    cas[1].set_option(_capi.CA_OPT_PREBUILD_PLAN, 0)
    live = {}
    nid = [0]

    def rnd(n):
        return rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16)

    def insert(t, k, v):
        sid = nid[0]
        nid[0] += 1
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        for ca in cas:
            ca.insert(sid, t, kd, vd)
        live[sid] = (list(t), k, v)

    def same(outs, label):
        assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16)), label

    pre = [int(x) for x in rng.integers(0, 30, size=2 * chunk + 5)]
    kp, vp = rnd(len(pre)), rnd(len(pre))
    for i in range(5):
        n = int(rng.integers(1, 2 * chunk))
        insert(pre + [900 + i] * n, np.concatenate([kp, rnd(n)]), np.concatenate([vp, rnd(n)]))
    prebuilt_seen = 0
    for step in range(260):
        ids = sorted(live)
        q = rnd(len(ids))
        qd = torch.from_numpy(q).cuda()
        op = rng.random()
        if op < 0.85:
            k, v = rnd(len(ids)), rnd(len(ids))
            # a token id per (step, sequence): an insert that copies a prefix
            # then matches exactly its source's path (two sequences whose
            # tokens agree but whose K/V do not would share the first one's
            # K/V, which the oracle of the second would not see)
            t = [100_000 + 64 * step + j for j in range(len(ids))]
            kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
            if op < 0.7:
                outs = [ca.decode_step(np.array(t, np.int32), kd, vd, qd).cpu().numpy() for ca in cas]
            else:
                outs = []
                for ca in cas:
                    ca.append_batch(ids, np.array(t, np.int32), kd, vd)
                    outs.append(ca.attend(qd).cpu().numpy())
            for j, s_ in enumerate(ids):
                tt, kk, vv = live[s_]
                live[s_] = (tt + [t[j]], np.concatenate([kk, k[j:j + 1]]), np.concatenate([vv, v[j:j + 1]]))
        else:
            outs = [ca.attend(qd).cpu().numpy() for ca in cas]
        same(outs, step)
        if step % 20 == 0:
            assert_parity(outs[0], A.decode_step(q, [live[s_][1:] for s_ in ids]), f"churn {step}")
        prebuilt_seen = cas[0].stats()["prebuilt_plans"]
        r = rng.random()
        if r < 0.05:
            src = live[ids[int(rng.integers(0, len(ids)))]]
            cut = int(rng.integers(1, len(src[0]) + 1))
            extra = int(rng.integers(0, 4))
            insert(src[0][:cut] + [5000 + step] * extra, np.concatenate([src[1][:cut], rnd(extra)]),
                   np.concatenate([src[2][:cut], rnd(extra)]))
        elif r < 0.08 and len(live) > 2:
            victim = ids[int(rng.integers(0, len(ids)))]
            for ca in cas:
                ca.remove(victim)
            del live[victim]
    assert prebuilt_seen >= 3 and cas[1].stats()["prebuilt_plans"] == 0
    tables = [ca.export_table() for ca in cas]
    assert np.array_equal(tables[0][0], tables[1][0]) and tables[0][1] == tables[1][1]
    for ca in cas:
        _check_pool_either_layout(ca, H, chunk, lambda s_: live[s_][1:])


def test_binding_rejects_bad_tensors():
    """The binding's argument checks (a fast path, then the detailed one for
    the message): wrong dtype or device raise TypeError, wrong shape or a
    non-contiguous tensor ValueError, for q, out and the decode step's K/V;
    nothing is launched and the context stays usable."""
    _say("binding argument checks")
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention
    H, n = 2, 3
    ca = ChunkAttention(H, 16, device="cuda:0")
    kv = torch.zeros((10, H, 128), dtype=torch.float16, device="cuda:0")
    for i in range(n):
        ca.insert(i, [100 * i + j for j in range(10)], kv, kv)
    good = torch.zeros((n, H, 128), dtype=torch.float16, device="cuda:0")
    toks = np.arange(n, dtype=np.int32)
    bad_type = [good.float(), good.cpu(), good.numpy(force=True) if hasattr(good, "numpy") else None]
    bad_value = [good[:2], torch.zeros((n, H, 64), dtype=torch.float16, device="cuda:0"),
                 torch.zeros((n, 128, H), dtype=torch.float16, device="cuda:0").transpose(1, 2)]
    for b in bad_type:
        if b is None:
            continue
        with pytest.raises(TypeError):
            ca.attend(b)
        with pytest.raises(TypeError):
            ca.decode_step(toks, b, good, good)
    for b in bad_value:
        with pytest.raises(ValueError):
            ca.attend(b)
        with pytest.raises(ValueError):
            ca.attend(good, b)
        with pytest.raises(ValueError):
            ca.decode_step(toks, good, b, good)
    with pytest.raises(ValueError):
        ca.decode_step(toks[:2], good, good, good)
    assert ca.stats()["unique_tokens"] == 10 * n
    out = ca.attend(good)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # tokens given as a list, a wider integer array or a strided view are converted
    for t in ([5, 6, 7], np.arange(3, dtype=np.int64), np.arange(6, dtype=np.int32)[::2]):
        ca.decode_step(t, good, good, good)
    torch.cuda.synchronize()
    assert ca.stats()["unique_tokens"] == 13 * n


def test_workspace_swapped_after_a_table_was_copied_ahead():
    """A table copied ahead into the workspace is forgotten once the caller
    attaches another workspace, also when it later attaches the first buffer
    again (whose contents are then the caller's, here zeros): the structural
    step uploads its own table and matches a twin without tables built ahead
    bit for bit, and the oracle."""
    _say("workspace swapped after a copy ahead")
    import ctypes
    torch = _torch()
    from decode_attention_prefix_tree_amd import ChunkAttention, _capi
    rng = np.random.default_rng(901)
    H, n = 2, 3
    cas = [ChunkAttention(H, 32, device="cuda:0") for _ in range(2)]
    cas[1].set_option(_capi.CA_OPT_PREBUILD_PLAN, 0)
    kv = []
    for i in range(n):
        k, v = [rng.standard_normal((63, H, 128), dtype=np.float32).astype(np.float16) for _ in range(2)]
        for ca in cas:
            ca.insert(i, [1000 * i + j for j in range(63)], torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        kv.append([k, v])

    def step():
        k, v, q = [rng.standard_normal((n, H, 128), dtype=np.float32).astype(np.float16) for _ in range(3)]
        t = np.arange(n, dtype=np.int32) + 7
        outs = [ca.decode_step(t, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                               torch.from_numpy(q).cuda()).cpu().numpy() for ca in cas]
        for i in range(n):
            kv[i] = [np.concatenate([kv[i][0], k[i:i + 1]]), np.concatenate([kv[i][1], v[i:i + 1]])]
        assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))
        assert_parity(outs[0], A.decode_step(q, kv), "swapped workspace")

    for ca in cas:
        ca.ensure_workspace()
    up0 = cas[0].stats()["table_uploads"]
    step()  # every last chunk is full now: the next step's table was copied ahead
    torch.cuda.synchronize()
    st = cas[0].stats()
    assert st["prebuilt_plans"] == 0 and st["table_uploads"] == up0 + 2  # this step's table, the one ahead
    ca = cas[0]
    first = ca.ws
    other = torch.empty_like(first)
    assert ca.lib.ca_attach_workspace(ca.ctx, ctypes.c_void_p(other.data_ptr()), other.numel()) == 0
    first.zero_()
    assert ca.lib.ca_attach_workspace(ca.ctx, ctypes.c_void_p(first.data_ptr()), first.numel()) == 0
    uploads = ca.stats()["table_uploads"]
    step()  # structural: every sequence opens a chunk
    torch.cuda.synchronize()
    assert ca.stats()["prebuilt_plans"] == 1 and ca.stats()["table_uploads"] == uploads + 1
    step()
