"""Batch structure: prefix forests, block tables and sequence lengths.

A batch is built from a small forest spec.  Every tree node owns a run of
shared prompt tokens (a whole number of cache blocks); the samples hanging off
a leaf each own a private suffix.  Requests that hang off the same node share
that node's physical blocks, which is how a paged cache with prefix reuse hands
the attention layer identical block IDs for identical prompts (PagedAttention
vs. RadixAttention page, "How PagedAttention Works", step 4: requests that
start with the same prompt reference the same physical blocks).

The draw order of every seeded batch is fixed:

1. suffix lengths (construction order),
2. request-order shuffle (groups are not contiguous in the batch),
3. physical block permutation of the pool,
4. block-table padding past each request's last block (random int32),
5. (values, in ``values.py``) K/V pool, then queries.

``Batch.truth`` is the prefix grouping the construction implies, in the
canonical order used across the project: groups sorted by (smallest member,
depth).  It comes from the construction, not from any grouping algorithm.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class AttnShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    block_size: int
    scale: float
    v_aliases_k: bool = False

    @property
    def gqa_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_token(self) -> int:
        """bf16 bytes one cached token occupies in one layer."""
        if self.v_aliases_k:
            return self.num_kv_heads * self.head_dim_qk * 2
        return self.num_kv_heads * (self.head_dim_qk + self.head_dim_v) * 2


@dataclass
class Node:
    """A run of shared prompt tokens and what hangs below it."""

    prefix_tokens: int
    children: List["Node"] = field(default_factory=list)
    samples: int = 0
    suffix: Optional[Tuple[int, int]] = None  # inclusive uniform range


@dataclass
class Config:
    name: str
    shape: AttnShape
    trees: List[Node]
    singletons: int = 0
    singleton_len: Optional[Tuple[int, int]] = None
    pool_blocks: Optional[int] = None  # None: ceil(1.25 x blocks needed)
    seed: int = 0
    description: str = ""


GQA_LLAMA = AttnShape(32, 8, 128, 128, 16, 1.0 / math.sqrt(128.0))


def _prompts(n_prompts, prefix, samples, suffix):
    return [Node(prefix, samples=samples, suffix=suffix) for _ in range(n_prompts)]


CONFIGS = {
    "tiny": Config(
        name="tiny",
        shape=AttnShape(8, 2, 128, 128, 16, 1.0 / math.sqrt(128.0)),
        trees=_prompts(1, 512, 8, (32, 96)),
        pool_blocks=256,
        seed=1,
        description="8 requests sharing one 512-token prefix, suffix U{32..96}, "
        "GQA 8/2, D 128, block 16, 256-block pool",
    ),
    "llama3_8b": Config(
        name="llama3_8b",
        shape=GQA_LLAMA,
        trees=_prompts(8, 4096, 8, (256, 1024)),
        seed=2,
        description="64 requests = 8 prompts x 8 samples, prefix 4096, suffix "
        "U{256..1024}, GQA 32/8, D 128, block 16",
    ),
    "long_rl": Config(
        name="long_rl",
        shape=GQA_LLAMA,
        trees=_prompts(16, 16384, 16, (1, 4096)),
        seed=3,
        description="256 requests = 16 prompts x 16 samples, prefix 16384, "
        "suffix U{1..4096}, GQA 32/8, D 128, block 16",
    ),
    "forest_mixed": Config(
        name="forest_mixed",
        shape=GQA_LLAMA,
        trees=[Node(2048, children=_prompts(32, 4096, 16, (512, 2048)))],
        singletons=64,
        singleton_len=(1024, 8192),
        seed=4,
        description="2048-token system prefix -> 32 branches of 4096 -> 16 "
        "samples each (suffix U{512..2048}), plus 64 unshared requests of "
        "length U{1024..8192}; GQA 32/8, D 128, block 16",
    ),
    "mla": Config(
        name="mla",
        shape=AttnShape(128, 1, 576, 512, 64, 1.0 / math.sqrt(576.0), v_aliases_k=True),
        trees=_prompts(4, 32768, 16, (512, 2048)),
        seed=5,
        description="64 requests = 4 prompts x 16 samples, prefix 32768, suffix "
        "U{512..2048}, 128 q heads on one 576-wide latent (V = first 512), "
        "block 64",
    ),
}

CONFIG_ORDER = ["tiny", "llama3_8b", "long_rl", "forest_mixed", "mla"]


def config_by_name(name: str) -> Config:
    return CONFIGS[name]


@dataclass
class Batch:
    config: Config
    shape: AttnShape
    block_tables: np.ndarray  # int32 [B, max_blocks]
    seq_lens: np.ndarray  # int32 [B]
    num_blocks: int  # pool size
    used_blocks: np.ndarray  # bool [num_blocks]
    truth: dict  # canonical grouping implied by the construction
    rng: np.random.Generator  # positioned after the structure draws

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])


def _max_len(node: Node, above: int) -> int:
    here = above + node.prefix_tokens
    best = 0
    if node.samples:
        best = here + node.suffix[1]
    for c in node.children:
        best = max(best, _max_len(c, here))
    return best


def build_batch(cfg: Config, seed: Optional[int] = None) -> Batch:
    """Draw one batch's structure (tables, lengths, pool size, truth)."""
    shape = cfg.shape
    bs = shape.block_size
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))

    # Walk the forest in construction order: nodes pre-order, samples at leaves.
    nodes = []  # (node, parent_index, start_block)
    leaves = []  # (node_index, sample k)

    def visit(node, parent, start):
        assert node.prefix_tokens > 0 and node.prefix_tokens % bs == 0
        idx = len(nodes)
        nodes.append((node, parent, start))
        n_blocks = node.prefix_tokens // bs
        if node.samples:
            assert not node.children and node.samples >= 2
            for k in range(node.samples):
                leaves.append((idx, k))
        else:
            assert len(node.children) >= 2, "a single child would merge with its parent"
        for c in node.children:
            visit(c, idx, start + n_blocks)

    for t in cfg.trees:
        visit(t, -1, 0)

    # 1. suffix lengths, construction order (tree samples, then singletons).
    suffix = [int(rng.integers(nodes[ni][0].suffix[0], nodes[ni][0].suffix[1] + 1)) for ni, _ in leaves]
    single = [
        int(rng.integers(cfg.singleton_len[0], cfg.singleton_len[1] + 1)) for _ in range(cfg.singletons)
    ]
    n_req = len(leaves) + cfg.singletons

    # 2. request-order shuffle: construction index c sits at batch position pos[c].
    pos = rng.permutation(n_req)

    # Blocks needed.
    node_blocks = [n.prefix_tokens // bs for n, _, _ in nodes]
    own_blocks = [-(-s // bs) for s in suffix] + [-(-s // bs) for s in single]
    needed = sum(node_blocks) + sum(own_blocks)
    pool = cfg.pool_blocks if cfg.pool_blocks is not None else int(math.ceil(1.25 * needed))
    assert pool >= needed

    # 3. physical block permutation; IDs are taken in construction order.
    perm = rng.permutation(pool).astype(np.int64)
    cursor = 0
    node_ids = []
    for nb in node_blocks:
        node_ids.append(perm[cursor : cursor + nb])
        cursor += nb
    own_ids = []
    for nb in own_blocks:
        own_ids.append(perm[cursor : cursor + nb])
        cursor += nb

    max_len = max([_max_len(t, 0) for t in cfg.trees] + ([cfg.singleton_len[1]] if cfg.singletons else []))
    max_blocks = -(-max_len // bs)

    # 4. padding past each request's last block: arbitrary int32 values.
    tables = rng.integers(-(2**31), 2**31, size=(n_req, max_blocks), dtype=np.int64).astype(np.int32)
    lens = np.zeros(n_req, dtype=np.int32)

    def path_of(ni):
        chain = []
        while ni >= 0:
            chain.append(ni)
            ni = nodes[ni][1]
        return chain[::-1]

    for c in range(n_req):
        p = pos[c]
        if c < len(leaves):
            ni, _ = leaves[c]
            ids = [node_ids[a] for a in path_of(ni)] + [own_ids[c]]
            row = np.concatenate(ids)
            L = sum(nodes[a][0].prefix_tokens for a in path_of(ni)) + suffix[c]
        else:
            row = own_ids[c]
            L = single[c - len(leaves)]
        tables[p, : row.shape[0]] = row
        lens[p] = L

    used = np.zeros(pool, dtype=bool)
    for i in range(n_req):
        nb = -(-int(lens[i]) // bs)
        used[tables[i, :nb]] = True

    truth = _construction_truth(cfg, nodes, leaves, pos, tables, lens, bs)
    return Batch(cfg, shape, tables, lens, pool, used, truth, rng)


def _construction_truth(cfg, nodes, leaves, pos, tables, lens, bs):
    """Canonical grouping implied by the forest spec (every node is a group)."""
    n_req = lens.shape[0]
    members = {i: [] for i in range(len(nodes))}
    leaf_of = {}
    for c, (ni, _) in enumerate(leaves):
        leaf_of[int(pos[c])] = ni
        a = ni
        while a >= 0:
            members[a].append(int(pos[c]))
            a = nodes[a][1]
    depth = {}
    for i, (_, parent, _) in enumerate(nodes):
        depth[i] = 0 if parent < 0 else depth[parent] + 1
    order = sorted(range(len(nodes)), key=lambda i: (min(members[i]), depth[i]))
    index = {ni: k for k, ni in enumerate(order)}
    groups = []
    for ni in order:
        node, parent, start = nodes[ni]
        mem = sorted(members[ni])
        b0, b1 = start, start + node.prefix_tokens // bs
        groups.append(
            dict(
                depth=depth[ni],
                parent=index[parent] if parent >= 0 else -1,
                block_begin=b0,
                block_end=b1,
                members=tuple(mem),
                block_ids=tuple(int(x) for x in tables[mem[0], b0:b1]),
            )
        )
    requests = []
    for i in range(n_req):
        if i in leaf_of:
            g = index[leaf_of[i]]
            sb = groups[g]["block_end"]
            requests.append((sb, int(lens[i]) - bs * sb, g))
        else:
            requests.append((0, int(lens[i]), -1))
    return dict(groups=groups, requests=requests)
