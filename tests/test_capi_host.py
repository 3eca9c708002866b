"""The C-ABI library on the CPU: it loads, exports what the header declares,
and its host-side tree and chunk table match the hand-worked golden cases and
the independent Python model bit for bit.  No device work is done here: the
contexts have no device pool."""

import ctypes

import numpy as np
import pytest

from decode_attention_prefix_tree_amd import CaError, ChunkAttention, _capi
from oracle.tree_model import PrefixTreeModel, TreeError
from tests.golden_cases import load_cases
from workloads import make_config, make_prefix_suffix


def test_library_exports_every_declared_symbol():
    lib = _capi.load()
    names = _capi.header_symbols()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_capi._SIGS), "binding and header disagree"


def test_create_rejects_unsupported_shapes():
    lib = _capi.load()
    ctx = ctypes.c_void_p()
    assert lib.ca_create(8, 64, 64, ctypes.byref(ctx)) == -2
    for c in (0, 65, 96, 129):
        assert lib.ca_create(8, 128, c, ctypes.byref(ctx)) == -2
    for c in (32, 128):
        assert lib.ca_create(8, 128, c, ctypes.byref(ctx)) == 0
        lib.ca_destroy(ctx)
    # any size up to 64 serves the tree and tables; a device pool needs 32, 64 or 128
    assert lib.ca_create(8, 128, 3, ctypes.byref(ctx)) == 0
    assert lib.ca_attach_pool(ctx, None, 10) == 0
    assert lib.ca_attach_pool(ctx, ctypes.c_void_p(1 << 20), 10) == -2
    lib.ca_destroy(ctx)
    assert lib.ca_create(0, 128, 64, ctypes.byref(ctx)) == -1
    assert lib.ca_create_ex(8, 128, 64, 0x100, ctypes.byref(ctx)) == -2



def test_slot_bytes_pad_power_of_two_head_counts():
    """A slot holds K and V of every head (4 * H * C * d bytes), and of one
    head more when H is a power of two from 16 up, so that tiles of one head
    in tiles allocated a power of two apart do not lie a power of two apart;
    slots of 32 tokens are half a tile and of 128 two."""
    lib = _capi.load()
    for heads, stored in ((32, 33), (16, 17), (64, 65), (8, 8), (4, 4), (1, 1), (3, 3), (24, 24), (40, 40)):
        for chunk in (32, 64, 128):
            assert lib.ca_slot_bytes(heads, 128, chunk) == 4 * stored * chunk * 128, (heads, chunk)
    assert lib.ca_slot_bytes(0, 128, 64) == 0 and lib.ca_slot_bytes(8, 128, 0) == 0


def _apply(ca, op):
    try:
        if op.kind == "insert":
            return str(ca.insert(op.seq, op.tokens))
        if op.kind == "append":
            ca.append(op.seq, op.tokens)
        else:
            ca.remove(op.seq)
        return None
    except CaError as e:
        return e.name


def model_and_lib_agree(m, ca):
    rows, order = m.table()
    got_rows, got_order = ca.export_table()
    assert [tuple(int(x) for x in r) for r in got_rows] == rows
    assert got_order == order
    st = ca.stats()
    assert st["unique_tokens"] == sum(r[3] for r in rows)
    assert st["chunks"] == len(rows)
    assert st["free_slots"] == m.free_slots()
    assert ca.sequences() == m.sequences()


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c.name)
def test_golden_scripts_lib_equals_model_at_chunk64(case):
    m = PrefixTreeModel(64, case.capacity, case.share)
    ca = ChunkAttention(2, case.capacity, device=None, share=case.share)
    for op in case.ops:
        if op.kind == "table":
            model_and_lib_agree(m, ca)
            continue
        before = ca.export_table()
        got = _apply(ca, op)
        try:
            if op.kind == "insert":
                want = str(m.insert(op.seq, op.tokens))
            elif op.kind == "append":
                m.append(op.seq, op.tokens)
                want = None
            else:
                m.remove(op.seq)
                want = None
        except TreeError as e:
            want = e.code
            after = ca.export_table()
            assert np.array_equal(before[0], after[0]) and before[1] == after[1]
        assert got == want
        model_and_lib_agree(m, ca)


def expand(tokens, rep):
    return [t for t in tokens for _ in range(rep)]


@pytest.mark.parametrize("case", [c for c in load_cases()], ids=lambda c: c.name)
def test_golden_tables_at_chunk64_by_token_expansion(case):
    """Repeating every token 64/C times turns a chunk-C golden case into a
    chunk-64 case with the same tree shape, so the hand-worked rows carry
    over with token_start and n_tokens scaled (splits in the golden cases
    fall on token boundaries, which stay chunk-relative after expansion)."""
    rep = 64 // case.chunk
    if 64 % case.chunk:
        pytest.skip("chunk does not divide 64")
    ca = ChunkAttention(2, case.capacity, device=None, share=case.share)
    for op in case.ops:
        if op.kind == "table":
            rows, order = ca.export_table()
            want = [(r[0], r[1], r[2] * rep, r[3] * rep, r[4], r[5], r[6]) for r in op.rows]
            assert [tuple(int(x) for x in r) for r in rows] == want
            assert order == op.order
            continue
        got = _apply(ca, type(op)(op.kind, op.seq, expand(op.tokens, rep), op.expect))
        if op.kind == "insert" and op.expect is not None and op.expect.lstrip("-").isdigit():
            assert got == str(int(op.expect) * rep)
        else:
            assert got == op.expect


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_random_ops_bit_exact_against_model(chunk):
    rng = np.random.default_rng(1234)
    for trial in range(25):
        cap = int(rng.integers(5, 60))
        if chunk == 32:
            cap -= cap % 2  # 32-token chunks pair up in 64-key tiles: even capacities
        share = bool(rng.random() < 0.85)
        m = PrefixTreeModel(chunk, cap, share)
        ca = ChunkAttention(4, cap, device=None, share=share, chunk_size=chunk)
        ids = []
        for step in range(80):
            r = rng.random()
            # tokens from a small alphabet in runs, so prefixes collide often and
            # divergences land inside chunks
            def toks(n):
                base = rng.integers(0, 3, size=max(1, n // 16))
                return list(np.repeat(base, 16)[:n] if n >= 16 else rng.integers(0, 3, size=n))
            if r < 0.45 or not ids:
                sid = int(rng.integers(0, 1000))
                t = toks(int(rng.integers(1, 300)))
                op = ("insert", sid, t)
            elif r < 0.75:
                op = ("append", int(rng.choice(ids)), toks(int(rng.integers(1, 100))))
            elif r < 0.95:
                op = ("remove", int(rng.choice(ids)), [])
            else:
                op = ("remove", 5000, [])  # unknown
            kind, sid, t = op
            try:
                getattr(m, kind)(sid, t) if kind != "remove" else m.remove(sid)
                want = None
            except TreeError as e:
                want = e.code
            try:
                getattr(ca, kind)(sid, t) if kind != "remove" else ca.remove(sid)
                got = None
            except CaError as e:
                got = e.name
            assert got == want, (kind, sid)
            ids = m.sequences()
            model_and_lib_agree(m, ca)


def test_errors_leave_state_unchanged():
    ca = ChunkAttention(2, 3, device=None)
    ca.insert(1, list(range(130)))   # 3 chunks: full pool
    snap = ca.export_table()
    for fn, code in ((lambda: ca.insert(1, [5]), "dup_seq"),
                     (lambda: ca.insert(2, []), "invalid_arg"),
                     (lambda: ca.insert(2, [7]), "no_capacity"),
                     (lambda: ca.append(9, [1]), "unknown_seq"),
                     (lambda: ca.append(1, list(range(63))), "no_capacity"),
                     (lambda: ca.remove(9), "unknown_seq")):
        with pytest.raises(CaError) as ei:
            fn()
        assert ei.value.name == code
        after = ca.export_table()
        assert np.array_equal(snap[0], after[0]) and snap[1] == after[1]
    ca.append(1, list(range(62)))     # fills the last chunk (2 + 62 = 64)
    assert ca.stats()["unique_tokens"] == 192


def test_attach_pool_only_while_empty_and_attend_needs_device():
    lib = _capi.load()
    ca = ChunkAttention(2, 4, device=None)
    ca.insert(1, [1, 2])
    assert lib.ca_attach_pool(ca.ctx, None, 8) == -10
    assert lib.ca_attend(ca.ctx, ctypes.c_void_p(256), ctypes.c_void_p(256), None) == -9
    ca.remove(1)
    assert lib.ca_attach_pool(ca.ctx, None, 8) == 0
    assert lib.ca_attend(ca.ctx, ctypes.c_void_p(256), ctypes.c_void_p(256), None) == -9


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_tables_and_plan_sizes(k):
    wl = make_config(k, heads=1)
    m = PrefixTreeModel(64, 10_000)
    ca = ChunkAttention(32, 10_000, device=None)
    for i in range(wl.n_seq):
        t = wl.seq_tokens(i)
        assert ca.insert(i, t) == m.insert(i, t)
    model_and_lib_agree(m, ca)
    st = ca.stats()
    assert st["attended_tokens"] == wl.attended_tokens()
    assert st["unique_kv_bytes"] == st["unique_tokens"] * 4 * 32 * 128
    rows, _ = m.table()
    shared = [r for r in rows if r[5] - r[4] >= 2]
    private = [r for r in rows if r[5] - r[4] == 1]
    assert st["shared_chunks"] == len(shared)
    # every shared chunk is read once per 32-row block, every private chunk once
    assert st["cf_chunk_reads"] == sum((r[5] - r[4] + 31) // 32 for r in shared)
    assert st["sf_chunk_reads"] == len(private)


def test_non_aligned_prefix_at_scale():
    """A 1,766-token shared prefix: the first insert cuts 27 full chunks and
    a chunk holding the prefix's last 38 tokens and 26 suffix tokens; the
    second insert splits that chunk at the divergence, so the tree shares 28
    chunks, the last one partial, and the first sequence's tail starts with a
    26-token chunk."""
    wl = make_prefix_suffix(1766, [512] * 32, heads=1, seed=2001)
    m = PrefixTreeModel(64, 10_000)
    ca = ChunkAttention(32, 10_000, device=None)
    for i in range(wl.n_seq):
        t = wl.seq_tokens(i)
        assert ca.insert(i, t) == m.insert(i, t)
    model_and_lib_agree(m, ca)
    st = ca.stats()
    rows, _ = m.table()
    shared = [r for r in rows if r[5] - r[4] >= 2]
    assert len(shared) == 28 and st["shared_chunks"] == 28
    assert sorted(r[3] for r in shared)[0] == 38 and sum(r[3] for r in shared) == 1766
    assert st["unique_tokens"] == 1766 + 32 * 512
    assert st["attended_tokens"] == 32 * 2278
    tail0 = sorted((r for r in rows if r[5] - r[4] == 1 and r[4] == 0), key=lambda r: r[2])
    assert [r[3] for r in tail0] == [26] + [64] * 7 + [38]
    assert st["cf_chunk_reads"] == 28 and st["sf_chunk_reads"] == 9 + 31 * 8


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("case,want", [("w1", 4), ("p1024x256", 8), ("w2", 16), ("w3", 16),
                                       ("p2048x96", 32), ("w5", 64)])
def test_automatic_chunk_first_group(case, want, chunk):
    """With the group left open, the longest chunk-first chain (2 halves per
    chunk of a wave, about 2.5 us each) must fit in half of the step's
    streaming time at 6 TB/s (32 heads): the tiny workload (6.3 MB) allows one
    chunk per wave, 1024 shared + 32 x 256 private tokens (151 MB) two,
    285-335 MB four, 2048 shared + 96 x 512 private (839 MB) eight and the
    multi-branch tree (1.26 GB) sixteen.  At 32-token chunks a ref is half a
    tile, so the same chains take twice the refs, at most 64.  An explicit
    setting wins."""
    if case.startswith("w"):
        wl = make_config(int(case[1:]), heads=1)
    elif case == "p2048x96":
        wl = make_prefix_suffix(2048, [512] * 96, heads=1, seed=6)
    else:
        wl = make_prefix_suffix(1024, [256] * 32, heads=1, seed=5)
    ca = ChunkAttention(32, 20_000, device=None, chunk_size=chunk)
    for i in range(wl.n_seq):
        ca.insert(i, wl.seq_tokens(i))
    want = min(64, want * 2) if chunk == 32 else want
    assert ca.stats()["cf_chunks_per_task"] == want
    ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, 8)
    assert ca.stats()["cf_chunks_per_task"] == 8
    ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, 0)
    assert ca.stats()["cf_chunks_per_task"] == want
    with pytest.raises(CaError):
        ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, 65)


@pytest.mark.parametrize("k", [2, 5])
def test_no_chunk_first_mode_keeps_tree_and_streams_whole_paths(k):
    """The PagedAttn*-style mode shares storage exactly like the two-phase
    context but plans every path chunk, shared ones included, per sequence."""
    wl = make_config(k, heads=1)
    ca2 = ChunkAttention(32, 10_000, device=None)
    ca1 = ChunkAttention(32, 10_000, device=None, two_phase=False)
    for i in range(wl.n_seq):
        t = wl.seq_tokens(i)
        assert ca1.insert(i, t) == ca2.insert(i, t)
    r1, o1 = ca1.export_table()
    r2, o2 = ca2.export_table()
    assert np.array_equal(r1, r2) and o1 == o2
    s1, s2 = ca1.stats(), ca2.stats()
    assert s1["unique_tokens"] == s2["unique_tokens"] and s1["shared_chunks"] == s2["shared_chunks"] > 0
    assert s1["cf_tasks"] == 0 and s1["cf_units"] == 0
    # every (sequence, chunk-on-its-path) pair is one chunk read per head
    assert s1["sf_chunk_reads"] == int(sum((r[5] - r[4]) for r in r1))
    assert s2["sf_chunk_reads"] + s2["shared_chunks"] < s1["sf_chunk_reads"]


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_append_batch_matches_model_through_fill_refreshes(chunk):
    rng = np.random.default_rng(77)
    m = PrefixTreeModel(chunk, 400)
    ca = ChunkAttention(2, 400, device=None, chunk_size=chunk)
    shared = list(range(100))
    ids = [3, 9, 11, 20, 21]
    for n, s in enumerate(ids):
        t = shared + [1000 + n] * int(rng.integers(1, 70))
        assert ca.insert(s, t) == m.insert(s, t)
    ca.insert(50, shared[:40])          # ends inside a shared chunk
    m.insert(50, shared[:40])
    model_and_lib_agree(m, ca)
    live = ids + [50]
    for step in range(150):
        batch = [s for s in live if rng.random() < 0.8] or [live[0]]
        toks = [int(x) for x in rng.integers(0, 5, size=len(batch))]
        ca.append_batch(batch, toks)
        for s, t in zip(batch, toks):
            m.append(s, [t])
        model_and_lib_agree(m, ca)
        if step == 60:
            ca.remove(11)
            m.remove(11)
            live.remove(11)
    st = ca.stats()
    assert st["fill_refreshes"] > 50 and st["table_rebuilds"] > 3


def test_append_batch_errors_change_nothing():
    ca = ChunkAttention(2, 3, device=None)
    ca.insert(1, list(range(64)))      # full private chunk
    ca.insert(2, list(range(100, 130)))
    snap = ca.export_table()
    for args, code in (([[1, 7], [5, 5]], "unknown_seq"),
                       ([[2, 2], [5, 5]], "invalid_arg"),
                       ([[], []], "invalid_arg")):
        with pytest.raises(CaError) as ei:
            ca.append_batch(*args)
        assert ei.value.name == code
        after = ca.export_table()
        assert np.array_equal(snap[0], after[0]) and snap[1] == after[1]
    # seq 1 needs a new chunk (its chunk is full), seq 2 appends in place: one free slot is enough
    ca.append_batch([1, 2], [5, 6])
    assert ca.stats()["free_slots"] == 0
    ca.insert(4, list(range(64)))       # shares seq 1's first chunk, needs no slot
    snap = ca.export_table()
    # seq 4 ends on a shared full chunk -> needs a new chunk, none free
    with pytest.raises(CaError) as ei:
        ca.append_batch([2, 4], [7, 8])
    assert ei.value.name == "no_capacity"
    after = ca.export_table()
    assert np.array_equal(snap[0], after[0]) and snap[1] == after[1]


@pytest.mark.parametrize("n_chunks,expect", [(16, 32), (17, 18)])
def test_partial_slots_dense_up_to_16_per_sequence(n_chunks, expect):
    """Partial ids are dense (sequence x list position) while no sequence has
    more than 16 partials, compact beyond: one sequence with n_chunks private
    chunks (one per task) and one with a single chunk."""
    ca = ChunkAttention(2, 64, device=None)
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 1)
    ca.insert(0, list(range(64 * n_chunks)))
    ca.insert(1, [10**6 + j for j in range(10)])
    assert ca.stats()["partials"] == expect


def test_partial_slots_of_a_shared_prefix_batch():
    """32 sequences of 1024 shared + 512 private tokens, 4 chunks per task on
    both sides: 4 shared runs and 2 private tasks per sequence, 6 partials each."""
    ca = ChunkAttention(2, 4096, device=None)
    ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, 4)
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 4)
    shared = list(range(1024))
    for i in range(32):
        ca.insert(i, shared + [(1 << 20) + i * 1000 + j for j in range(512)])
    st = ca.stats()
    assert st["cf_tasks"] == 4 and st["sf_tasks"] == 64
    assert st["partials"] == 32 * 6


def test_launch_mode_follows_merge_pair_count():
    """By default a step is one launch from 3072 (sequence, head) pairs up
    (96 sequences at 32 heads), two launches below; the option overrides."""
    def ctx(n_seq):
        ca = ChunkAttention(32, 1024, device=None)
        for i in range(n_seq):
            ca.insert(i, [i * 100 + j for j in range(3)])
        return ca
    assert ctx(95).stats()["one_launch_step"] == 0
    big = ctx(96)
    assert big.stats()["one_launch_step"] == 1
    big.set_option(_capi.CA_OPT_FUSED_MERGE, 0)
    assert big.stats()["one_launch_step"] == 0
    small = ctx(4)
    small.set_option(_capi.CA_OPT_FUSED_MERGE, 1)
    assert small.stats()["one_launch_step"] == 1
    with pytest.raises(CaError):
        small.set_option(_capi.CA_OPT_FUSED_MERGE, 3)
    # the merge's poll bound: 0 (the library's own) or any positive count
    for value in (1, 1000, 0):
        small.set_option(_capi.CA_OPT_MERGE_POLL_LIMIT, value)
    with pytest.raises(CaError):
        small.set_option(_capi.CA_OPT_MERGE_POLL_LIMIT, -1)
    with pytest.raises(CaError):
        small.set_option(99, 0)


def test_partial_slots_compact_when_dense_would_waste_memory():
    """One sequence with 16 partials among 99 with one: dense slots would
    take 1600 entries for 115 partials, so the ids stay compact."""
    ca = ChunkAttention(2, 512, device=None)
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 1)
    ca.insert(0, list(range(64 * 16)))
    for i in range(1, 100):
        ca.insert(i, [10**6 + i * 100 + j for j in range(10)])
    assert ca.stats()["partials"] == 16 + 99


def _tile_reads(rows):
    """Per-head tile reads of a plan, from the canonical table: a chunk of n
    tokens is ceil(n / 64) tiles of 64 keys; a shared chunk (range >= 2) is
    read once per 32 query rows, a private one once."""
    cf = sf = 0
    for r in rows:
        tiles = max(1, -(-r[3] // 64))
        rng_ = r[5] - r[4]
        if rng_ >= 2:
            cf += tiles * -(-rng_ // 32)
        else:
            sf += tiles
    return cf, sf


def test_chunk128_plan_lists_64_key_tiles():
    m = PrefixTreeModel(128, 64)
    ca = ChunkAttention(2, 64, device=None, chunk_size=128)
    shared = list(range(300))
    for s, n in enumerate([100, 1, 64, 65, 200]):
        t = shared + [1000 + s] * n
        assert ca.insert(s, t) == m.insert(s, t)
    model_and_lib_agree(m, ca)
    rows, _ = m.table()
    st = ca.stats()
    assert (st["cf_chunk_reads"], st["sf_chunk_reads"]) == _tile_reads(rows)
    # 300 shared tokens: chunks of 128, 128 and 44 (split at the divergence)
    assert sorted(r[3] for r in rows if r[5] - r[4] >= 2) == [44, 128, 128]


def test_chunk128_append_into_second_tile_rebuilds_the_plan():
    ca = ChunkAttention(2, 8, device=None, chunk_size=128)
    ca.insert(1, list(range(60)))
    ca.insert(2, [7] * 10)
    st0 = ca.stats()
    for t in range(4):                      # keys 60..63: still the first tile
        ca.append_batch([1, 2], [500 + t, 600 + t])
        ca.stats()
    st1 = ca.stats()
    assert st1["table_rebuilds"] == st0["table_rebuilds"]
    assert st1["fill_refreshes"] > st0["fill_refreshes"]
    ca.append_batch([1, 2], [700, 701])     # key 64 of sequence 1: a second tile
    st2 = ca.stats()
    assert st2["table_rebuilds"] == st1["table_rebuilds"] + 1
    assert st2["sf_chunk_reads"] == 3 and st2["chunks"] == 2


def test_chunk32_capacity_in_pairs_and_plan():
    """32-token chunks pair up in 64-key tiles: an odd last slot is left out,
    and the plan lists one ref per chunk."""
    ca = ChunkAttention(2, 7, device=None, chunk_size=32)
    assert ca.stats()["capacity_slots"] == 6
    m = PrefixTreeModel(32, 6)
    for s, t in enumerate([list(range(70)), list(range(40)) + [9] * 5, [5] * 20]):
        assert ca.insert(s, t) == m.insert(s, t)
    model_and_lib_agree(m, ca)
    rows, _ = m.table()
    cf = sum(-(-(r[5] - r[4]) // 32) for r in rows if r[5] - r[4] >= 2)
    sf = sum(1 for r in rows if r[5] - r[4] < 2)
    st = ca.stats()
    assert (st["cf_chunk_reads"], st["sf_chunk_reads"]) == (cf, sf)


@pytest.mark.parametrize("case,want", [("w1", 4), ("w2", 3), ("w3", 3), ("w4", 16), ("w5", 16)])
def test_automatic_sequence_first_group(case, want):
    """With the group left open, the largest of 16, 8 and 4 private refs per
    task that still gives 1920 / heads tasks (about 2.5 rounds of blocks over
    3 x 256 resident block slots; 8/5 of that behind chunk-first units):
    32 sequences with 8 private chunks each under a shared prefix fall back
    to 3 (3 + 3 + 2 chunks: 3072 blocks at 32 heads); 32 chunks each
    (workload 4) and the multi-branch tree's ragged suffixes reach 16.  An
    explicit setting wins."""
    wl = make_config(int(case[1:]), heads=1)
    ca = ChunkAttention(32, 10_000, device=None)
    for i in range(wl.n_seq):
        ca.insert(i, wl.seq_tokens(i))
    st = ca.stats()
    assert st["sf_chunks_per_task"] == want
    # every sequence's private refs cut into tasks of that size
    rows, _ = ca.export_table()
    assert st["sf_tasks"] >= 1920 // 32 or want in (3, 4)
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 2)
    assert ca.stats()["sf_chunks_per_task"] == 2
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 0)
    assert ca.stats()["sf_chunks_per_task"] == want
    with pytest.raises(CaError):
        ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 257)


@pytest.mark.parametrize("private,want", [(512, 3), (704, 3), (320, 4), (256, 4), (448, 4)])
def test_sequence_first_fallback_three_without_single_chunk_tasks(private, want):
    """Behind chunk-first units, where neither 16 nor 8 refs per task reach
    the task target, 3 replaces 4 when it makes more tasks and no sequence
    is left a one-chunk remainder: 8 and 11 private chunks take 3 (3 + 3 + 2,
    3 + 3 + 3 + 2); 5 stays at 4 (two tasks either way), 4 and 7 too (3 + 1
    and 3 + 3 + 1 would leave one)."""
    ca = ChunkAttention(32, 10_000, device=None)
    for i in range(32):
        ca.insert(i, list(range(1024)) + [100_000 + 1000 * i + j for j in range(private)])
    st = ca.stats()
    assert st["sf_chunks_per_task"] == want
    n = -(-private // 64)
    assert st["sf_tasks"] == 32 * -(-n // want)


@pytest.mark.parametrize("chunk,shared,group,want", [
    (64, 1766, 16, [14, 14]), (64, 4096, 16, [16, 16, 16, 16]), (64, 1024, 16, [16]),
    (64, 2112, 16, [11, 11, 11]), (128, 1766, 16, [14, 14]), (64, 1766, 5, [5, 5, 5, 5, 4, 4])])
def test_chunk_first_runs_cut_evenly(chunk, shared, group, want):
    """A chain of shared chunks longer than the chunk-first group is cut into
    as few runs as the group allows, of equal length to within one chunk:
    28 tiles (1,766 tokens at chunk 64) in two runs of 14, not 16 + 12; 33 in
    three of 11; a 128-token chunk's two tiles stay in one run."""
    ca = ChunkAttention(8, 10_000, device=None, chunk_size=chunk)
    ca.set_option(_capi.CA_OPT_CF_CHUNKS_PER_TASK, group)
    for i in range(32):
        ca.insert(i, list(range(shared)) + [100_000 + 1000 * i + j for j in range(200)])
    st = ca.stats()
    img = np.frombuffer(ca.export_plan(), dtype=np.int32)
    units = img[:32 * int(st["cf_units"])].reshape(-1, 32)
    assert sorted(units[:, 1].tolist(), reverse=True) == want
    assert sum(want) == -(-shared // 64)


@pytest.mark.parametrize("shared,want", [(1024, 8), (0, 16)])
def test_sequence_first_group_with_chunk_first_units(shared, want):
    """The automatic sequence-first group asks for 8/5 as many tasks when
    chunk-first units share the launch: 64 sequences of 16 private chunks at
    32 heads make 64 tasks with 16 refs each, enough alone (60) but short of
    96 behind a 1024-token shared prefix, where 8 refs each (128 tasks) win."""
    ca = ChunkAttention(32, 10_000, device=None)
    for i in range(64):
        ca.insert(i, list(range(shared)) + [100_000 + 2000 * i + j for j in range(1024)])
    st = ca.stats()
    assert (st["cf_chunk_reads"] > 0) == (shared > 0)
    assert st["sf_chunks_per_task"] == want
    assert st["sf_tasks"] == 64 * 16 // want


@pytest.mark.parametrize("chunk", [2, 3, 4])
def test_tiny_chunks_random_ops_bit_exact_against_model(chunk):
    """Chunks of 2, 3 and 4 tokens, a vocabulary of 2 or 3 and sequences of at
    most 12 tokens, with inserts, appends (single and batched) and removals
    interleaved: nearly every call splits, shares or opens chunks.  Tables,
    DFS order, counts and free slots bit for bit equal to the tree model; a
    failing call (unknown id, no capacity) fails alike and changes nothing.
    A batch of appends is all or nothing: the model applies it to a copy."""
    import copy
    rng = np.random.default_rng(100 + chunk)
    for trial in range(40):
        vocab = int(rng.integers(2, 4))
        cap = int(rng.integers(8, 60))
        share = bool(rng.random() < 0.9)
        m = PrefixTreeModel(chunk, cap, share)
        ca = ChunkAttention(2, cap, device=None, share=share, chunk_size=chunk)
        for step in range(60):
            live = m.sequences()
            r = rng.random()
            toks = [int(x) for x in rng.integers(0, vocab, size=int(rng.integers(1, 13)))]
            if r < 0.4 or not live:
                kind, args = "insert", (int(rng.integers(0, 30)), toks)
            elif r < 0.6:
                kind, args = "append", (int(rng.choice(live)), toks[:int(rng.integers(1, 4))])
            elif r < 0.8:
                batch = [int(x) for x in rng.choice(live, size=int(rng.integers(1, len(live) + 1)), replace=False)]
                kind, args = "append_batch", (batch, [int(x) for x in rng.integers(0, vocab, size=len(batch))])
            else:
                kind, args = "remove", (int(rng.choice(live)),)
            try:
                if kind == "append_batch":
                    trial_model = copy.deepcopy(m)
                    for sid, t in zip(*args):
                        trial_model.append(sid, [t])
                    m = trial_model
                else:
                    getattr(m, kind)(*args)
                want = None
            except TreeError as e:
                want = e.code
            try:
                getattr(ca, kind)(*args)
                got = None
            except CaError as e:
                got = e.name
            assert got == want, (chunk, trial, step, kind)
            model_and_lib_agree(m, ca)


def test_staging_size_and_attach_checks():
    """ca_staging_bytes is three 256-byte aligned parts, each holding the
    table (the table alone is what ca_workspace_bytes holds besides the
    partials); a misaligned staging pointer is refused; NULL detaches."""
    lib = _capi.load()
    ca = ChunkAttention(8, 64, device=None)
    for i in range(5):
        ca.insert(i, list(range(100)) + [1000 + i] * (10 + 30 * i))
    need = ctypes.c_size_t(0)
    assert lib.ca_staging_bytes(ca.ctx, ctypes.byref(need)) == 0
    assert need.value > 0 and need.value % (3 * 256) == 0
    assert need.value // 3 < ca.workspace_bytes()
    assert lib.ca_staging_bytes(ca.ctx, None) == -1
    assert lib.ca_attach_staging(ca.ctx, ctypes.c_void_p(4096 + 8), 1 << 16) == -1
    assert lib.ca_attach_staging(ca.ctx, None, 0) == 0


def test_failure_injection_option():
    lib = _capi.load()
    ca = ChunkAttention(2, 16, device=None)
    assert lib.ca_set_option(ca.ctx, _capi.CA_OPT_FAIL_DEVICE_OPS, -1) == -1
    assert lib.ca_set_option(ca.ctx, _capi.CA_OPT_FAIL_DEVICE_OPS, 3) == 0
    assert lib.ca_set_option(ca.ctx, _capi.CA_OPT_FAIL_AFTER_DEVICE_OPS, -1) == -1
    assert lib.ca_set_option(ca.ctx, _capi.CA_OPT_FAIL_AFTER_DEVICE_OPS, 2) == 0
    # a host-only context runs no device operation: inserts are unaffected
    ca.insert(1, list(range(70)))
    assert ca.sequences() == [1]


def test_insert_with_failed_copy_changes_nothing():
    """An insert whose K/V copy cannot be enqueued (injected failure, before any
    HIP call) returns CA_E_HIP and leaves the tree as it was."""
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("uses a stand-in pool address: only where no GPU is visible")
    lib = _capi.load()
    ctx = ctypes.c_void_p()
    assert lib.ca_create(2, 128, 64, ctypes.byref(ctx)) == 0
    try:
        assert lib.ca_attach_pool(ctx, ctypes.c_void_p(1 << 20), 32) == 0
        assert lib.ca_set_option(ctx, _capi.CA_OPT_FAIL_DEVICE_OPS, 1 << 20) == 0
        toks = (ctypes.c_int32 * 150)(*range(150))
        matched = ctypes.c_int32(-7)
        rc = lib.ca_insert(ctx, 5, toks, 150, ctypes.c_void_p(1 << 21), ctypes.c_void_p(1 << 22), None,
                           ctypes.byref(matched))
        assert rc == -8 and b"injected" in lib.ca_last_error(ctx)
        assert matched.value == -7
        assert lib.ca_list_sequences(ctx, None, 0) == 0
        st = _capi.ca_stats_t()
        assert lib.ca_stats(ctx, ctypes.byref(st)) == 0
        assert st.free_slots == 32 and st.chunks == 0 and st.unique_tokens == 0
        # the same id can be tried again (it was not left half inserted)
        rc = lib.ca_insert(ctx, 5, toks, 150, ctypes.c_void_p(1 << 21), ctypes.c_void_p(1 << 22), None, None)
        assert rc == -8 and lib.ca_list_sequences(ctx, None, 0) == 0
    finally:
        lib.ca_destroy(ctx)


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_prebuilt_plans_equal_fresh_builds(chunk):
    """Two host contexts run the same script, one building the next table
    ahead of structural decode steps (in the call before), one building every
    table in the call that needs it: after every call their chunk tables,
    device table images and plan statistics are equal byte for byte, and the
    first one did take prebuilt tables.  The script decodes one token per
    live sequence (so last chunks fill up, chunks of 128 open their second
    tile, shared last chunks get private children) with inserts that share
    and split chunks, duplicates, removals and partial batches mixed in."""
    rng = np.random.default_rng(700 + chunk)
    a = ChunkAttention(3, 6000, device=None, chunk_size=chunk)
    b = ChunkAttention(3, 6000, device=None, chunk_size=chunk)
    b.set_option(_capi.CA_OPT_PREBUILD_PLAN, 0)
    live = {}
    next_id = [0]
    keys = ("chunks", "shared_chunks", "unique_tokens", "attended_tokens", "cf_tasks", "cf_units", "sf_tasks",
            "partials", "cf_chunks_per_task", "sf_chunks_per_task", "free_slots")

    def insert(toks):
        sid = next_id[0]
        next_id[0] += 1
        for ca in (a, b):
            ca.insert(sid, toks)
        live[sid] = list(toks)

    base = [int(x) for x in rng.integers(0, 1000, size=int(rng.integers(chunk, 3 * chunk)))]
    for i in range(6):
        insert(base + [5000 + i] * int(rng.integers(0, chunk + 5)))
    insert(list(live[2]))  # a duplicate: its last chunk is shared
    step = 0
    for it in range(260):
        u = rng.random()
        ids = sorted(live)
        if u < 0.82:
            toks = [int(x) for x in rng.integers(0, 1000, size=len(ids))]
            for ca in (a, b):
                ca.append_batch(ids, toks)
            for s_, t in zip(ids, toks):
                live[s_].append(t)
            step += 1
        elif u < 0.88:
            src = live[ids[int(rng.integers(0, len(ids)))]]
            cut = int(rng.integers(1, len(src) + 1))
            insert(src[:cut] + ([int(rng.integers(2000, 3000))] if rng.random() < 0.7 else []))
        elif u < 0.93 and len(ids) > 3:
            victim = ids[int(rng.integers(0, len(ids)))]
            for ca in (a, b):
                ca.remove(victim)
            del live[victim]
        else:
            sub = sorted(rng.choice(ids, size=max(1, len(ids) // 2), replace=False).tolist())
            toks = [int(x) for x in rng.integers(0, 1000, size=len(sub))]
            for ca in (a, b):
                ca.append_batch(sub, toks)
            for s_, t in zip(sub, toks):
                live[s_].append(t)
        ra, oa = a.export_table()
        rb, ob = b.export_table()
        assert np.array_equal(ra, rb) and oa == ob, it
        assert a.export_plan() == b.export_plan(), it
        sa, sb = a.stats(), b.stats()
        for k in keys:
            assert sa[k] == sb[k], (it, k)
    assert a.stats()["prebuilt_plans"] >= 3, a.stats()["prebuilt_plans"]
    assert b.stats()["prebuilt_plans"] == 0


def _sf_records(ca):
    """The sequence-first task records of the plan's device table: after the
    chunk-first records (128 bytes each), at the next 256-byte boundary, 16
    int32 each (chunk refs begin, count, DFS position, partial id, caller row,
    reuse, append index, pad, 4 inline slots, 4 inline fill counts)."""
    img = np.frombuffer(ca.export_plan(), dtype=np.int32)
    st = ca.stats()
    off = (int(st["cf_units"]) * 128 + 255) // 256 * 256 // 4
    n = int(st["sf_tasks"])
    return img[off:off + 16 * n].reshape(n, 16)


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_sequence_first_tasks_longest_first_then_by_slot(chunk):
    """Decoding gives every sequence one new chunk per chunk_size tokens, so
    the sequences' chunks interleave in the pool.  The plan lists the
    sequence-first tasks longest first and, among tasks of one length, by
    the slot of their first chunk (not by sequence), so that blocks running
    together read slots close together; every private chunk ref is in exactly
    one task."""
    ca = ChunkAttention(8, 4000, device=None, chunk_size=chunk)
    ca.set_option(_capi.CA_OPT_SF_CHUNKS_PER_TASK, 4)
    prompt = list(range(3 * chunk))
    n = 12
    for i in range(n):
        ca.insert(i, prompt + [10_000 + i])
    rng = np.random.default_rng(3)
    for step in range(9 * chunk + 5):
        ids = list(range(n)) if step < 6 * chunk else list(range(0, n, 2))
        ca.append_batch(ids, [int(x) for x in 20_000 + step * 100 + np.arange(len(ids))])
    recs = _sf_records(ca)
    counts, first_slot = recs[:, 1], recs[:, 8]
    assert (np.diff(counts) <= 0).all()
    for c in np.unique(counts):
        sl = first_slot[counts == c]
        assert (np.diff(sl) > 0).all(), (c, sl)
    # the tasks of one sequence (DFS position) cover its private refs once
    refs = sorted(int(b) + k for b, cnt in zip(recs[:, 0], counts) for k in range(int(cnt)))
    assert refs == list(range(min(refs), min(refs) + len(refs)))
    # interleaved: some task's first slot lies below a task of a sequence
    # that comes earlier in DFS order
    pos = recs[:, 2]
    assert any(pos[j] > pos[k] and first_slot[j] < first_slot[k]
               for j in range(len(pos)) for k in range(len(pos)) if counts[j] == counts[k])


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_large_three_level_tree_matches_model(chunk):
    """512 sequences in a three-level tree (a 1,000-token root, 8 branches of
    500 tokens, suffixes of 1..300 tokens, so every level ends inside a
    chunk), then removals of every third sequence and 200 decode rounds that
    grow the survivors: the library's table, slot use and DFS order equal the
    independent tree model's after each phase."""
    rng = np.random.default_rng(900 + chunk)
    root = [int(x) for x in 100_000 + np.arange(1000)]
    branches = [[int(x) for x in 200_000 + 1000 * b + np.arange(500)] for b in range(8)]
    m = PrefixTreeModel(chunk, 60_000)
    ca = ChunkAttention(32, 60_000, device=None, chunk_size=chunk)
    for i in range(512):
        toks = root + branches[i % 8] + [int(x) for x in 300_000 + 1000 * i + np.arange(int(rng.integers(1, 301)))]
        assert ca.insert(i, toks) == m.insert(i, toks)
    model_and_lib_agree(m, ca)
    for i in range(0, 512, 3):
        ca.remove(i)
        m.remove(i)
    model_and_lib_agree(m, ca)
    ids = m.sequences()
    for step in range(200):
        toks = [int(x) for x in 10_000_000 + 1000 * step + np.arange(len(ids))]
        ca.append_batch(ids, toks)
        for s_, t in zip(ids, toks):
            m.append(s_, [t])
    model_and_lib_agree(m, ca)
