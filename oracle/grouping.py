"""Prefix-group discovery as a dictionary trie over block IDs (test only).

The method first finds groups of requests that share a KV-cache prefix
(ZoRRo Inference & Forest Cascade Attention page, "Core Mechanism", step 1),
so that each shared block can be read once per group.  The page does not say
how sharing is recognised; the reading used here is the one a paged cache
makes natural: requests that start with the same prompt reference the same
physical blocks (PagedAttention vs. RadixAttention page, "How PagedAttention
Works", step 4), so two requests share their first j blocks exactly when the
first j entries of their block tables are equal.

Rules (readings of what the pages leave open):

* only full blocks take part: request i contributes the path
  ``table[i][0 : L_i // block_size]``; a partly filled last block is never
  shared (copy-on-write gives a diverging request its own copy);
* every node of the compressed trie of these paths that at least two requests
  pass through is a group; a maximal run of trie nodes with the same request
  set is one group spanning that run's block range -- groups therefore nest
  and form a forest;
* a group's depth is the number of groups strictly above it; its parent is
  the nearest one;
* a request's suffix starts at the end of the deepest group it is in (block
  0 if none) and covers the rest of its L_i tokens.

Canonical form: groups sorted by (smallest member, depth) -- unique because
two groups with a common member are nested and differ in depth.  Each group
gives (depth, parent index in that order or -1, block_begin, block_end,
ascending members, the block IDs of its range read from its smallest member).
Each request gives (suffix_block_begin, suffix_tokens, deepest group or -1).
"""

from __future__ import annotations


class _TrieNode:
    __slots__ = ("pos", "children", "members")

    def __init__(self, pos):
        self.pos = pos
        self.children = {}
        self.members = []


def group(block_tables, seq_lens, block_size, cascade=True):
    """Canonical prefix grouping of a batch (see module docstring)."""
    B = len(seq_lens)
    root = _TrieNode(-1)
    for i in range(B):
        nfull = int(seq_lens[i]) // block_size
        node = root
        for j in range(nfull):
            b = int(block_tables[i][j])
            nxt = node.children.get(b)
            if nxt is None:
                nxt = node.children[b] = _TrieNode(j)
            nxt.members.append(i)
            node = nxt

    raw = []  # dict(members, begin, end, parent_raw)
    deepest_raw = [-1] * B

    def walk(node, parent_raw):
        # node is the first trie node of a run; extend while the single child
        # carries the same request set.
        begin = node.pos
        cur = node
        while len(cur.children) == 1:
            (child,) = cur.children.values()
            if len(child.members) != len(cur.members):
                break
            cur = child
        end = cur.pos + 1
        here = parent_raw
        if len(node.members) >= 2:
            here = len(raw)
            raw.append(dict(members=tuple(sorted(node.members)), begin=begin, end=end, parent=parent_raw))
            for i in node.members:
                deepest_raw[i] = here
        for child in cur.children.values():
            walk(child, here)

    if cascade:
        for child in root.children.values():
            walk(child, -1)

    depth_raw = []
    for g in raw:
        d, p = 0, g["parent"]
        while p >= 0:
            d += 1
            p = raw[p]["parent"]
        depth_raw.append(d)

    order = sorted(range(len(raw)), key=lambda k: (raw[k]["members"][0], depth_raw[k]))
    index = {k: n for n, k in enumerate(order)}
    groups = []
    for k in order:
        g = raw[k]
        first = g["members"][0]
        groups.append(
            dict(
                depth=depth_raw[k],
                parent=index[g["parent"]] if g["parent"] >= 0 else -1,
                block_begin=g["begin"],
                block_end=g["end"],
                members=g["members"],
                block_ids=tuple(int(block_tables[first][j]) for j in range(g["begin"], g["end"])),
            )
        )
    requests = []
    for i in range(B):
        d = deepest_raw[i]
        if d < 0:
            requests.append((0, int(seq_lens[i]), -1))
        else:
            sb = raw[d]["end"]
            requests.append((sb, int(seq_lens[i]) - block_size * sb, index[d]))
    return dict(groups=groups, requests=requests)
