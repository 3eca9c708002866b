"""Seeded synthetic inputs for one decode step over a prefix-shared KV cache.

This module only draws token ids, keys, values and queries.  It holds none of
the attention arithmetic and none of the prefix-tree logic: both the fp64
oracle (``oracle/``) and the HIP path take what it returns as plain arrays.

Workload shapes follow the microkernel evaluation of ChunkAttention
(paperlayer.ai summary of arXiv 2402.15220v4, section 4.1 and Table 3: chunk
size 64, batch 32, shared tokens 0 to 4096; Figure 3: 512 completion tokens).
The pages measure on synthetic shapes, not on a dataset.

Draw order for workload ``k`` with ``rng = numpy.random.default_rng(1000 + k)``:

1. (multi-branch tree only) the 128 private suffix lengths,
   ``rng.integers(64, 1025, size=128)`` (inclusive bounds 64 and 1024);
2. for every trie segment in DFS pre-order (root prefix, then each branch
   followed by the private suffixes below it, sequences in index order):
   keys, then values, each ``standard_normal((len, H, d), float32)`` rounded
   to float16 (round to nearest even);
3. the queries, ``standard_normal((N, H, d), float32)`` rounded to float16.

Token ids: token ``j`` of segment ``s`` is ``(s << 13) | j``, so distinct
segments never share a token and sharing happens only where the structure says.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
CHUNK = 64
_TOKEN_BITS = 13  # up to 8192 tokens per segment

__all__ = [
    "HEAD_DIM",
    "CHUNK",
    "Segment",
    "Workload",
    "TokenListWorkload",
    "CONFIG_NAMES",
    "make_config",
    "make_prefix_suffix",
    "make_long_sequence",
    "from_token_lists",
    "segment_tokens",
]


def segment_tokens(seg_id: int, length: int) -> np.ndarray:
    """Token ids of segment ``seg_id``: ``(seg_id << 13) | j`` for j < length."""
    if length > (1 << _TOKEN_BITS):
        raise ValueError("segment longer than 8192 tokens")
    return ((seg_id << _TOKEN_BITS) | np.arange(length, dtype=np.int64)).astype(np.int32)


@dataclass
class Segment:
    seg_id: int
    tokens: np.ndarray  # int32 [len]
    k: np.ndarray  # float16 [len, H, d]
    v: np.ndarray  # float16 [len, H, d]

    @property
    def length(self) -> int:
        return int(self.tokens.shape[0])


@dataclass
class Workload:
    """A batch of sequences, each a path of segments, with one query per sequence.

    Sequence ``i`` has ``seq_id == i``; rows of ``q`` are in ascending seq_id.
    """

    name: str
    heads: int
    head_dim: int
    chunk: int
    seed: int
    segments: List[Segment]
    paths: List[List[int]]  # segment ids per sequence, root first
    q: np.ndarray  # float16 [N, H, d]
    description: str = ""

    @property
    def n_seq(self) -> int:
        return len(self.paths)

    def seq_tokens(self, i: int) -> np.ndarray:
        return np.concatenate([self.segments[s].tokens for s in self.paths[i]])

    def seq_kv(self, i: int) -> Tuple[np.ndarray, np.ndarray]:
        segs = [self.segments[s] for s in self.paths[i]]
        return (np.concatenate([s.k for s in segs], axis=0),
                np.concatenate([s.v for s in segs], axis=0))

    def seq_len(self, i: int) -> int:
        return int(sum(self.segments[s].length for s in self.paths[i]))

    def lengths(self) -> np.ndarray:
        return np.array([self.seq_len(i) for i in range(self.n_seq)], dtype=np.int64)

    def unique_tokens(self) -> int:
        used = sorted({s for p in self.paths for s in p})
        return int(sum(self.segments[s].length for s in used))

    def attended_tokens(self) -> int:
        return int(self.lengths().sum())


def _draw_segments(rng: np.random.Generator, lengths: Sequence[int], heads: int,
                   head_dim: int) -> List[Segment]:
    segs = []
    for sid, n in enumerate(lengths):
        k = rng.standard_normal((n, heads, head_dim), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((n, heads, head_dim), dtype=np.float32).astype(np.float16)
        segs.append(Segment(sid, segment_tokens(sid, n), k, v))
    return segs


CONFIG_NAMES = {
    1: "tiny: 4 seq, 8 heads, shared prefix 256 + private suffix 32",
    2: "llama7b-like: 32 seq, 32 heads, shared prefix 1024 + private suffix 512",
    3: "long-prompt: 32 seq, 32 heads, shared prefix 4096 + private suffix 512",
    4: "no-sharing: 32 seq, 32 heads, 2048 private tokens each",
    5: "multi-branch: 128 seq, 32 heads, root 1024 -> 4 x 1024 -> private U[64,1024]",
}


def make_config(k: int, heads: int | None = None) -> Workload:
    """Build workload ``k`` (1..5).  ``heads`` overrides the head count (used to
    run one head shard of a workload at its real sequence shape)."""
    rng = np.random.default_rng(1000 + k)
    d = HEAD_DIM
    if k in (1, 2, 3):
        n, h, lp, ls = {1: (4, 8, 256, 32), 2: (32, 32, 1024, 512), 3: (32, 32, 4096, 512)}[k]
        h = heads or h
        segs = _draw_segments(rng, [lp] + [ls] * n, h, d)
        paths = [[0, 1 + i] for i in range(n)]
    elif k == 4:
        n, h = 32, heads or 32
        segs = _draw_segments(rng, [2048] * n, h, d)
        paths = [[i] for i in range(n)]
    elif k == 5:
        n, h, branches = 128, heads or 32, 4
        per_branch = n // branches
        suffix = rng.integers(64, 1025, size=n)
        # DFS pre-order of the segment tree: root, then branch b and its suffixes.
        lengths, paths = [1024], [None] * n
        for b in range(branches):
            bseg = len(lengths)
            lengths.append(1024)
            for i in range(b * per_branch, (b + 1) * per_branch):
                paths[i] = [0, bseg, len(lengths)]
                lengths.append(int(suffix[i]))
        segs = _draw_segments(rng, lengths, h, d)
    else:
        raise ValueError(f"unknown workload {k}")
    q = rng.standard_normal((len(paths), h, d), dtype=np.float32).astype(np.float16)
    return Workload(name=f"config{k}", heads=h, head_dim=d, chunk=CHUNK, seed=1000 + k,
                    segments=segs, paths=paths, q=q, description=CONFIG_NAMES[k])


def make_prefix_suffix(prefix_len: int, suffix_lens: Sequence[int], heads: int, seed: int,
                       name: str | None = None) -> Workload:
    """One shared prefix of ``prefix_len`` tokens (0 for none) and one private
    suffix per sequence, drawn like the single-prefix workloads above: with
    ``rng = default_rng(seed)``, K then V of the prefix, then of each suffix in
    sequence order, then the queries.  Neither length needs to be a multiple
    of the chunk size (a shared system prompt with six plugins reaches 1,766
    tokens: paperlayer.ai summary of arXiv 2402.15220v4, sections 1 and 2.1)."""
    rng = np.random.default_rng(seed)
    d, n = HEAD_DIM, len(suffix_lens)
    if prefix_len > 0:
        segs = _draw_segments(rng, [prefix_len] + [int(x) for x in suffix_lens], heads, d)
        paths = [[0, 1 + i] for i in range(n)]
    else:
        segs = _draw_segments(rng, [int(x) for x in suffix_lens], heads, d)
        paths = [[i] for i in range(n)]
    q = rng.standard_normal((n, heads, d), dtype=np.float32).astype(np.float16)
    desc = f"{n} seq, {heads} heads, shared prefix {prefix_len} + private suffixes " + (
        f"{suffix_lens[0]}" if len(set(int(x) for x in suffix_lens)) == 1 else
        f"{min(suffix_lens)}..{max(suffix_lens)}")
    return Workload(name=name or f"prefix{prefix_len}", heads=heads, head_dim=d, chunk=CHUNK, seed=seed,
                    segments=segs, paths=paths, q=q, description=desc)


def make_long_sequence(length: int, heads: int, seed: int) -> Workload:
    """One private sequence of ``length`` tokens, longer than a segment may
    be: a chain of segments of at most 8,192 tokens, K then V of each drawn in
    order with ``rng = default_rng(seed)``, then the query."""
    rng = np.random.default_rng(seed)
    pieces = [min(1 << _TOKEN_BITS, length - i) for i in range(0, length, 1 << _TOKEN_BITS)]
    segs = _draw_segments(rng, pieces, heads, HEAD_DIM)
    q = rng.standard_normal((1, heads, HEAD_DIM), dtype=np.float32).astype(np.float16)
    return Workload(name=f"long{length}", heads=heads, head_dim=HEAD_DIM, chunk=CHUNK, seed=seed,
                    segments=segs, paths=[list(range(len(pieces)))], q=q,
                    description=f"1 seq of {length} tokens, {heads} heads")


@dataclass
class TokenListWorkload:
    """Sequences given as explicit token lists (small tests).

    Keys/values are drawn once per distinct prefix, in order of first
    appearance scanning sequences in index order, so every sequence that shares
    a prefix supplies identical K/V rows for it (as a causal model would).
    """

    name: str
    heads: int
    head_dim: int
    chunk: int
    seed: int
    tokens: List[np.ndarray]
    k_rows: List[np.ndarray]  # per sequence, float16 [L, H, d]
    v_rows: List[np.ndarray]
    q: np.ndarray
    prefix_rows: Dict[Tuple[int, ...], int] = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        return len(self.tokens)

    def seq_tokens(self, i: int) -> np.ndarray:
        return self.tokens[i]

    def seq_kv(self, i: int):
        return self.k_rows[i], self.v_rows[i]

    def seq_len(self, i: int) -> int:
        return int(self.tokens[i].shape[0])

    def lengths(self) -> np.ndarray:
        return np.array([self.seq_len(i) for i in range(self.n_seq)], dtype=np.int64)

    def attended_tokens(self) -> int:
        return int(self.lengths().sum())


def from_token_lists(token_lists: Sequence[Sequence[int]], heads: int, seed: int,
                     head_dim: int = HEAD_DIM, chunk: int = CHUNK,
                     name: str = "tokens") -> TokenListWorkload:
    rng = np.random.default_rng(seed)
    table: Dict[Tuple[int, ...], int] = {}
    rows_k: List[np.ndarray] = []
    rows_v: List[np.ndarray] = []
    toks = [np.asarray(t, dtype=np.int32) for t in token_lists]
    per_seq_idx = []
    for t in toks:
        idx = []
        for j in range(len(t)):
            key = tuple(int(x) for x in t[: j + 1])
            if key not in table:
                table[key] = len(rows_k)
                rows_k.append(rng.standard_normal((heads, head_dim), dtype=np.float32).astype(np.float16))
                rows_v.append(rng.standard_normal((heads, head_dim), dtype=np.float32).astype(np.float16))
            idx.append(table[key])
        per_seq_idx.append(idx)
    ks = np.stack(rows_k) if rows_k else np.zeros((0, heads, head_dim), np.float16)
    vs = np.stack(rows_v) if rows_v else np.zeros((0, heads, head_dim), np.float16)
    k_rows = [ks[np.asarray(ix, dtype=np.int64)] for ix in per_seq_idx]
    v_rows = [vs[np.asarray(ix, dtype=np.int64)] for ix in per_seq_idx]
    q = rng.standard_normal((len(toks), heads, head_dim), dtype=np.float32).astype(np.float16)
    return TokenListWorkload(name=name, heads=heads, head_dim=head_dim, chunk=chunk, seed=seed,
                             tokens=toks, k_rows=k_rows, v_rows=v_rows, q=q, prefix_rows=table)
