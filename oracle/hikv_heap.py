"""Model of HiKV's important bank as its accelerator keeps it: a min-heap
whose nodes are vectors of w (score, token) entries.

TEST INFRASTRUCTURE ONLY.  The GPU library keeps no heap (it finds the
lowest frozen score with block-wide minima); this model exists so that the
tests can hold the oracle's dual-bank eviction against the data structure the
pages describe.  Only the test suite may import it.

Source: HiKV: Hierarchical Importance-Aware KV Cache with Hardware
Acceleration, Sec. IV-C and Fig. 11 (HEAPIFY_UP, HEAPIFY_DOWN), Sec. III-B
(promotion iff the ejected token's score beats the bank's lowest).

A node is a list of (score, token) pairs.  Its lowest score sits in the first
entry, its highest in the last, the others in no set order.  Node i has
children 2i+1 and 2i+2; the heap property is that no parent's highest score
exceeds a child's lowest, so the root's first entry is the bank's minimum.
"""

from __future__ import annotations

from typing import List, Optional, Tuple

Entry = Tuple[float, int]
Node = List[Entry]


def pick(node: Node) -> Node:
    """The max-min picker: the lowest entry (first one among equals) moves to
    the front, then the highest (last one among equals) to the back; the
    entries they trade places with take the freed positions."""
    n = list(node)
    lo = min(range(len(n)), key=lambda i: (n[i][0], i))
    n[0], n[lo] = n[lo], n[0]
    hi = max(range(len(n)), key=lambda i: (n[i][0], i))
    n[-1], n[hi] = n[hi], n[-1]
    return n


def sort_pair(a: Node, b: Node) -> Tuple[Node, Node]:
    """The parallel sorter: a ascending, b descending by score (stable)."""
    return sorted(a, key=lambda e: e[0]), sorted(b, key=lambda e: e[0], reverse=True)


def partial_merge(asc: Node, desc: Node) -> Tuple[Node, Node]:
    """One compare stage on position pairs of an ascending and a descending
    vector: the smaller of each pair (the ascending one among equals) goes to
    the first group, the larger to the second.  For sorted inputs the groups
    are exactly the lower and upper halves of the union."""
    lo, hi = [], []
    for x, y in zip(asc, desc):
        if y[0] < x[0]:
            lo.append(y), hi.append(x)
        else:
            lo.append(x), hi.append(y)
    return lo, hi


def split(parent: Node, child: Node) -> Tuple[Node, Node]:
    """Compare two nodes: the lower half goes to the parent, the upper half
    to the child, each through the picker."""
    lo, hi = partial_merge(*sort_pair(parent, child))
    return pick(lo), pick(hi)


class VectorHeap:
    def __init__(self, width: int):
        if width < 1:
            raise ValueError("node width must be positive")
        self.w = width
        self.nodes: List[Node] = []
        self.visited = 0  # nodes touched by the last offer

    # -- construction (HEAPIFY_UP) -----------------------------------------
    def insert_node(self, entries: Node) -> None:
        """Add one node at the end and compare it upwards until its lowest
        score is no less than its parent's highest."""
        if len(entries) != self.w:
            raise ValueError("a node holds exactly `width` entries")
        self.nodes.append(pick(entries))
        i = len(self.nodes) - 1
        while i > 0:
            p = (i - 1) // 2
            if self.nodes[i][0][0] >= self.nodes[p][-1][0]:
                break
            self.nodes[p], self.nodes[i] = split(self.nodes[p], self.nodes[i])
            i = p

    @classmethod
    def build(cls, entries: Node, width: int) -> "VectorHeap":
        if len(entries) % width:
            raise ValueError("the bank size must be a multiple of the node width")
        h = cls(width)
        for s in range(0, len(entries), width):
            h.insert_node(list(entries[s:s + width]))
        return h

    # -- maintenance (HEAPIFY_DOWN) ----------------------------------------
    def offer(self, entry: Entry) -> Optional[Entry]:
        """The recent bank ejects `entry`.  If its score beats the bank's
        lowest it replaces that entry, which is returned as evicted;
        otherwise `entry` itself is returned (discarded)."""
        self.visited = 0
        if not self.nodes or not entry[0] > self.nodes[0][0][0]:
            return entry
        evicted = self.nodes[0][0]
        root = list(self.nodes[0])
        root[0] = entry
        self.nodes[0] = pick(root)
        self.visited = 1
        i = 0
        while True:
            kids = [c for c in (2 * i + 1, 2 * i + 2) if c < len(self.nodes)]
            if not kids:
                break
            c = min(kids, key=lambda k: self.nodes[k][0][0])
            if self.nodes[i][-1][0] <= self.nodes[c][0][0]:
                break
            # the node's highest and the child's lowest trade places
            node, kid = list(self.nodes[i]), list(self.nodes[c])
            node[-1], kid[0] = kid[0], node[-1]
            self.nodes[i] = node
            self.nodes[c] = pick(kid)
            self.visited += 1
            i = c
        return evicted

    # -- inspection --------------------------------------------------------
    def entries(self) -> Node:
        return [e for n in self.nodes for e in n]

    def minimum(self) -> Entry:
        return self.nodes[0][0]

    def depth(self) -> int:
        return len(self.nodes).bit_length()

    def check(self) -> None:
        """Raise AssertionError unless every node and the heap are well formed."""
        for i, n in enumerate(self.nodes):
            s = [e[0] for e in n]
            assert s[0] == min(s) and s[-1] == max(s), ("node order", i, n)
            for c in (2 * i + 1, 2 * i + 2):
                if c < len(self.nodes):
                    assert s[-1] <= self.nodes[c][0][0], ("heap order", i, c)
