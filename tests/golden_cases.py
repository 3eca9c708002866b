"""Parser for tests/golden/tree_cases.txt (hand-worked prefix-tree cases)."""
import os
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))


@dataclass
class Op:
    kind: str  # insert / append / remove / table
    seq: int = 0
    tokens: List[int] = field(default_factory=list)
    expect: Optional[str] = None  # matched count as text, or an error code
    rows: List[Tuple[int, ...]] = field(default_factory=list)
    order: List[int] = field(default_factory=list)
    unique: Optional[int] = None


@dataclass
class Case:
    name: str
    chunk: int
    capacity: int
    share: bool
    ops: List[Op]


def load_cases(path: str = os.path.join(HERE, "golden", "tree_cases.txt")) -> List[Case]:
    cases, cur, tab = [], None, None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        w = line.split()
        if w[0] == "case":
            kv = dict(zip(w[2::2], w[3::2]))
            cur = Case(w[1], int(kv["chunk"]), int(kv["capacity"]), kv["share"] == "1", [])
            tab = None
        elif w[0] == "end":
            cases.append(cur)
            cur, tab = None, None
        elif w[0] in ("insert", "append", "remove"):
            expect = None
            if "->" in w:
                i = w.index("->")
                expect = w[i + 1]
                w = w[:i]
            cur.ops.append(Op(w[0], int(w[1]), [int(x) for x in w[2:]], expect))
            tab = None
        elif w[0] == "table":
            tab = Op("table")
            cur.ops.append(tab)
        elif w[0] == "row":
            tab.rows.append(tuple(int(x) for x in w[1:]))
        elif w[0] == "order":
            tab.order = [int(x) for x in w[1:]]
        elif w[0] == "unique":
            tab.unique = int(w[1])
        else:
            raise ValueError(f"bad line: {raw!r}")
    return cases
