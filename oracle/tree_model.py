"""Plain-Python model of the prefix-aware KV cache.  TEST INFRASTRUCTURE ONLY.

Follows the prefix-aware KV cache (PAKV) description: keys/values are cut into
chunks; chunks are the nodes of a prefix tree in which every root-to-node path
is a token prefix and every live sequence is a path (paperlayer.ai summary of
arXiv 2402.15220v4, section 3.1 and Figure 1); a shared prefix is stored once
and referenced by every sequence that has it (explainer, "Prefix-Aware KV
Cache" diagram); sharing only happens for prompts at the start of a sequence
(summary, section 7); a matched prefix gains a reference on arrival and loses
it on completion, and a chunk nobody references is freed (explainer, "dynamic
prefix detection"); decoding appends to leaf chunks or grows new chunks
(summary, section 3.1).

Where the pages are silent the model takes these readings (the C++ manager
implements the same readings independently):

* a node holds at most ``chunk`` tokens; a new path is cut into full chunks
  from its divergence point, the last one possibly partial;
* divergence inside a node splits it: the node keeps the matched head (same
  slot), the tail moves to a newly allocated slot as its only child and takes
  over the node's children and the sequences that ended in it;
* children are kept in creation order; matching follows the first child (in
  that order) whose first token equals the next token;
* a sequence that ends at a node with children sits before those children in
  DFS order; several sequences ending at one node keep arrival order;
* append writes into the sequence's last chunk only if that chunk is private
  (referenced by this sequence alone) and not full; otherwise it grows new
  private chunks below it.  Appended tokens are never deduplicated;
* slots are taken lowest free index first; on a split the tail slot is taken
  before the slots of new tokens, which are taken in token order;
* a failed call (duplicate or unknown sequence, empty token list, too few free
  slots) changes nothing.

The canonical chunk table: one row per chunk node in DFS pre-order,
``(node_id, parent_row, token_start, n_tokens, seq_begin, seq_end, slot)`` with
``parent_row = -1`` under the root and ``[seq_begin, seq_end)`` the node's
contiguous range in the DFS sequence order, which is returned alongside.
"""

from __future__ import annotations

import heapq
from typing import Dict, List, Optional, Sequence, Tuple


class TreeError(Exception):
    code = "error"


class DuplicateSeq(TreeError):
    code = "dup_seq"


class UnknownSeq(TreeError):
    code = "unknown_seq"


class InvalidArg(TreeError):
    code = "invalid_arg"


class NoCapacity(TreeError):
    code = "no_capacity"


class _Node:
    __slots__ = ("nid", "parent", "tokens", "slot", "children", "ended", "start", "ref")

    def __init__(self, nid: int, parent: Optional["_Node"], tokens: List[int], slot: int, start: int):
        self.nid = nid
        self.parent = parent
        self.tokens = tokens
        self.slot = slot
        self.children: List[_Node] = []
        self.ended: List[int] = []
        self.start = start
        self.ref = 0


class PrefixTreeModel:
    def __init__(self, chunk: int, capacity: int, share: bool = True):
        if chunk < 1 or capacity < 0:
            raise InvalidArg("chunk >= 1 and capacity >= 0 required")
        self.chunk = chunk
        self.capacity = capacity
        self.share = share
        self.root = _Node(-1, None, [], -1, 0)
        self._next_id = 0
        self._free = list(range(capacity))
        heapq.heapify(self._free)
        self._end: Dict[int, _Node] = {}

    # -- helpers --------------------------------------------------------------
    def _alloc(self) -> int:
        return heapq.heappop(self._free)

    def _new_node(self, parent: _Node, tokens: List[int], start: int) -> _Node:
        n = _Node(self._next_id, parent, tokens, self._alloc(), start)
        self._next_id += 1
        return n

    def _chunks_for(self, n_tokens: int) -> int:
        return (n_tokens + self.chunk - 1) // self.chunk

    def free_slots(self) -> int:
        return len(self._free)

    # -- mutations ------------------------------------------------------------
    def insert(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Add a sequence; returns the number of leading tokens already stored."""
        if seq_id in self._end:
            raise DuplicateSeq(seq_id)
        T = [int(t) for t in tokens]
        L = len(T)
        if L < 1:
            raise InvalidArg("empty sequence")
        # Walk without mutating.
        cur, pos, split = self.root, 0, None
        while pos < L and self.share:
            nxt = None
            for c in cur.children:
                if c.tokens[0] == T[pos]:
                    nxt = c
                    break
            if nxt is None:
                break
            k = 0
            lim = min(len(nxt.tokens), L - pos)
            while k < lim and nxt.tokens[k] == T[pos + k]:
                k += 1
            if k < len(nxt.tokens):
                split = (nxt, k)
                pos += k
                break
            cur, pos = nxt, pos + k
        need = (1 if split else 0) + self._chunks_for(L - pos)
        if need > len(self._free):
            raise NoCapacity(f"need {need} slots, {len(self._free)} free")
        matched = pos
        if split:
            node, k = split
            tail = self._new_node(node, node.tokens[k:], node.start + k)
            tail.children, node.children = node.children, [tail]
            for c in tail.children:
                c.parent = tail
            tail.ended, node.ended = node.ended, []
            for s in tail.ended:
                self._end[s] = tail
            tail.ref = node.ref
            node.tokens = node.tokens[:k]
            cur = node
        while pos < L:
            piece = T[pos: pos + self.chunk]
            n = self._new_node(cur, piece, pos)
            cur.children.append(n)
            cur, pos = n, pos + len(piece)
        cur.ended.append(seq_id)
        self._end[seq_id] = cur
        x = cur
        while x is not self.root:
            x.ref += 1
            x = x.parent
        return matched

    def append(self, seq_id: int, tokens: Sequence[int]) -> None:
        if seq_id not in self._end:
            raise UnknownSeq(seq_id)
        T = [int(t) for t in tokens]
        if len(T) < 1:
            raise InvalidArg("empty append")
        e = self._end[seq_id]
        room = self.chunk - len(e.tokens) if e.ref == 1 else 0
        take = min(room, len(T))
        need = self._chunks_for(len(T) - take)
        if need > len(self._free):
            raise NoCapacity(f"need {need} slots, {len(self._free)} free")
        e.tokens.extend(T[:take])
        pos = e.start + len(e.tokens)
        rest = T[take:]
        if not rest:
            return
        e.ended.remove(seq_id)
        cur = e
        i = 0
        while i < len(rest):
            piece = rest[i: i + self.chunk]
            n = self._new_node(cur, piece, pos)
            n.ref = 1
            cur.children.append(n)
            cur, pos, i = n, pos + len(piece), i + len(piece)
        cur.ended.append(seq_id)
        self._end[seq_id] = cur

    def remove(self, seq_id: int) -> None:
        if seq_id not in self._end:
            raise UnknownSeq(seq_id)
        e = self._end.pop(seq_id)
        e.ended.remove(seq_id)
        x = e
        while x is not self.root:
            x.ref -= 1
            p = x.parent
            if x.ref == 0:
                p.children.remove(x)
                heapq.heappush(self._free, x.slot)
            x = p

    # -- views ----------------------------------------------------------------
    def sequences(self) -> List[int]:
        return sorted(self._end)

    def table(self) -> Tuple[List[Tuple[int, ...]], List[int]]:
        rows: List[List[int]] = []
        order: List[int] = []
        # iterative pre-order; a marker closes a node's range after its subtree
        stack: List[Tuple[_Node, int, bool]] = [(c, -1, False) for c in reversed(self.root.children)]
        while stack:
            node, prow, closing = stack.pop()
            if closing:
                rows[prow][5] = len(order)
                continue
            r = len(rows)
            rows.append([node.nid, prow, node.start, len(node.tokens), len(order), -1, node.slot])
            order.extend(node.ended)
            stack.append((node, r, True))
            for c in reversed(node.children):
                stack.append((c, r, False))
        return [tuple(r) for r in rows], order

    def unique_tokens(self) -> int:
        rows, _ = self.table()
        return sum(r[3] for r in rows)

    def refcounts(self) -> Dict[int, int]:
        out = {}
        stack = list(self.root.children)
        while stack:
            n = stack.pop()
            out[n.nid] = n.ref
            stack.extend(n.children)
        return out

    def seq_path(self, seq_id: int) -> List[Tuple[int, int, int]]:
        """(slot, token_start, n_tokens) of the chunks on a sequence's path, root first."""
        x = self._end[seq_id]
        out = []
        while x is not self.root:
            out.append((x.slot, x.start, len(x.tokens)))
            x = x.parent
        return out[::-1]
