"""Seeded synthetic inputs for the EAGLE-3 tree-verify workloads.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic (no attention, no projection, no argmax, no acceptance).
Both the CPU oracle and the GPU path consume what it produces, so a mismatch
between them can never come from the inputs.

Every array is drawn from its own child generator
``numpy.random.default_rng([workload_id, seed, component])`` so a test that
needs only one component (say the prefix KV) does not pay for the others
(say the 1 GB LM-head matrix).

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even
from float32, done here with integer arithmetic on the bit pattern).

Tree shapes follow the pages' description of draft trees: the root is the
last committed token (node 0); drafts are expanded level by level with at
most ``branch`` (top-k) children per node and numbered in BFS order, so
``parent[n] < n`` (EAGLE-3 course lesson, "Tree draft vs chain draft"; the
news write-up of the EAGLE-3 paper, EAGLE-2 dynamic trees).
"""
from __future__ import annotations

import dataclasses

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# component ids of the child generators
C_TREE, C_PLEN, C_WLM, C_KPRE, C_VPRE, C_Q, C_KTREE, C_VTREE, C_PERM, C_PLANT = range(10)
C_WEIGHTS, C_PROMPT, C_FEAT, C_CTX, C_EMB, C_VOCAB = range(10, 16)


def child_rng(workload_id: int, seed: int, component: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(seed), int(component)])


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even.

    NaN inputs stay NaN (quiet). Works in chunks to bound the temporaries.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, flat.size, step):
        u = flat[s:s + step].view(np.uint32)
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(flat[s:s + step])
        if nan.any():
            r[nan] = BF16_NAN
        out[s:s + step] = r
    return out.reshape(x.shape)


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16, generated in float32 chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        m = min(step, n - s)
        v = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:s + m] = f32_to_bf16(v)
    return out.reshape(shape)


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v.reshape(shape)


# ---------------------------------------------------------------- trees

def chain_tree(n_drafts: int) -> np.ndarray:
    """Root plus a chain of n drafts: parent = [-1, 0, 1, ..., n-1]."""
    return np.arange(-1, n_drafts, dtype=np.int32)


def levels_tree(level_sizes, fanout) -> np.ndarray:
    """Complete tree from level sizes where every node of level d has `fanout`
    children on level d+1 (until the level is full), BFS numbering."""
    parent = [-1]
    prev = [0]
    for size in level_sizes:
        cur = []
        for i in range(size):
            p = prev[i // fanout] if fanout else prev[0]
            parent.append(p)
            cur.append(len(parent) - 1)
        prev = cur
    return np.asarray(parent, dtype=np.int32)


def binary_tree_15() -> np.ndarray:
    """15 drafts in levels 1, 2, 4, 8 (depths 1..4) under the root: T = 16."""
    return levels_tree([1, 2, 4, 8], 2)


def lesson_tree_7() -> np.ndarray:
    """The course lesson's example: d1 -> {d2a, d2b}; d2a -> {d3a, d3b};
    d2b -> {d3c, d3d}; plus the root.  Node order: root, d1, d2a, d2b, d3a..d3d."""
    return np.asarray([-1, 0, 1, 1, 2, 2, 3, 3], dtype=np.int32)


def topk_level_sizes(rng: np.random.Generator, n_drafts: int, depth: int, branch: int) -> list:
    """Level sizes n_1..n_depth, each >= 1, summing to n_drafts, with
    n_1 <= branch and n_{d+1} <= branch * n_d."""
    if not (depth <= n_drafts):
        raise ValueError("depth exceeds the number of drafts")
    sizes = [1] * depth
    for _ in range(n_drafts - depth):
        ok = []
        for d in range(depth):
            cap = branch if d == 0 else branch * sizes[d - 1]
            if sizes[d] < cap:
                ok.append(d)
        sizes[ok[int(rng.integers(len(ok)))]] += 1
    return sizes


def ranked_tree(p: float, n_drafts: int = 60, depth: int = 8, branch: int = 10) -> np.ndarray:
    """The tree a confidence-ranked drafter keeps when its confidence is
    calibrated to the ranked match model (plant_tokens_ranked): the rank-j
    child of a node is on the target's path with probability
    p (1 - p)^(j - 1) given its parent is, so a node's path probability is
    the product over its path; the tree is the n_drafts nodes of highest path
    probability (ties: first created first) with at most `branch` children
    per node and depth at most `depth`, grown best-first. Creation order is
    the numbering, so parents precede children and a node's children appear
    in rank order."""
    import heapq
    parent = [-1]
    heap, made = [], 0        # entries: (-path probability, creation counter, parent node, rank)

    def push_children(node, prob):
        nonlocal made
        for j in range(1, branch + 1):
            heapq.heappush(heap, (-prob * p * (1.0 - p) ** (j - 1), made, node, j))
            made += 1

    depth_of = [0]
    prob_of = [1.0]
    push_children(0, 1.0)
    while len(parent) < n_drafts + 1:
        negp, _, par, _ = heapq.heappop(heap)
        node = len(parent)
        parent.append(par)
        depth_of.append(depth_of[par] + 1)
        prob_of.append(-negp)
        if depth_of[node] < depth:
            push_children(node, -negp)
    return np.asarray(parent, dtype=np.int32)


def topk_tree(rng: np.random.Generator, n_drafts: int = 60, depth: int = 7, branch: int = 10) -> np.ndarray:
    """Random parent[] consistent with top-`branch` expansion, BFS numbered.

    Level d+1 nodes each pick a uniform parent among level-d nodes that still
    have fewer than `branch` children; children are then numbered grouped by
    parent (BFS order)."""
    sizes = topk_level_sizes(rng, n_drafts, depth, branch)
    parent = [-1]
    prev = [0]
    for size in sizes:
        kids = {p: 0 for p in prev}
        chosen = []
        for _ in range(size):
            avail = [p for p in prev if kids[p] < branch]
            p = avail[int(rng.integers(len(avail)))]
            kids[p] += 1
            chosen.append(p)
        chosen.sort()
        cur = []
        for p in chosen:
            parent.append(p)
            cur.append(len(parent) - 1)
        prev = cur
    return np.asarray(parent, dtype=np.int32)


def random_tree(rng: np.random.Generator, T: int, max_children: int = 64) -> np.ndarray:
    """Uniform random recursive tree on T nodes (parent[n] uniform in [0, n))."""
    parent = np.empty(T, dtype=np.int32)
    parent[0] = -1
    kids = np.zeros(T, dtype=np.int64)
    for n in range(1, T):
        while True:
            p = int(rng.integers(n))
            if kids[p] < max_children:
                break
        kids[p] += 1
        parent[n] = p
    return parent


# ---------------------------------------------------------------- paged KV

@dataclasses.dataclass
class PagedKV:
    k_cache: np.ndarray      # uint16 [num_blocks, Hkv, block_size, D]
    v_cache: np.ndarray      # uint16 [num_blocks, Hkv, D, block_size]  (key index fastest)
    block_table: np.ndarray  # int32  [B, max_blocks]
    prefix_len: np.ndarray   # int32  [B]
    block_size: int

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]


def paged_kv(workload_id: int, seed: int, prefix_len, Hkv: int, D: int,
             block_size: int = 16, spare_blocks: int = 1, max_blocks: int | None = None,
             dtype: str = "bf16") -> PagedKV:
    """Prefix K/V ~ N(0,1) (bf16 bit patterns, or float32 with dtype="f32"),
    scattered into a shuffled block pool.

    Logical rows are drawn in (sequence, position, head, dim) order. Slots
    past a sequence's prefix, spare blocks and unused block-table entries
    point at NaN-filled memory so that a read of them shows up in results.
    """
    f32 = dtype == "f32"
    draw = normal_f32 if f32 else normal_bf16
    nan = np.float32(np.nan) if f32 else BF16_NAN
    npdt = np.float32 if f32 else np.uint16
    prefix_len = np.asarray(prefix_len, dtype=np.int32)
    B = prefix_len.shape[0]
    nb = [(int(L) + block_size - 1) // block_size for L in prefix_len]
    used = sum(nb)
    nblk = used + spare_blocks
    if max_blocks is None:
        max_blocks = max(1, max(nb) if nb else 1)
    perm = child_rng(workload_id, seed, C_PERM).permutation(nblk).astype(np.int32)
    k_cache = np.full((nblk, Hkv, block_size, D), nan, dtype=npdt)
    v_cache = np.full((nblk, Hkv, D, block_size), nan, dtype=npdt)
    spare = int(perm[used]) if spare_blocks > 0 else 0
    table = np.full((B, max_blocks), spare, dtype=np.int32)
    rk = child_rng(workload_id, seed, C_KPRE)
    rv = child_rng(workload_id, seed, C_VPRE)
    nxt = 0
    for b in range(B):
        L = int(prefix_len[b])
        kb = draw(rk, (L, Hkv, D))
        vb = draw(rv, (L, Hkv, D))
        for j in range(nb[b]):
            phys = int(perm[nxt]); nxt += 1
            table[b, j] = phys
            lo, hi = j * block_size, min(L, (j + 1) * block_size)
            n = hi - lo
            k_cache[phys, :, :n, :] = kb[lo:hi].transpose(1, 0, 2)
            v_cache[phys, :, :, :n] = vb[lo:hi].transpose(1, 2, 0)
    return PagedKV(k_cache, v_cache, table, prefix_len, block_size)


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass
class VerifyShape:
    """One tree-verify step: tree attention -> RMSNorm -> LM head -> accept."""
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    D: int
    V: int
    n_drafts: int
    depth: int
    branch: int = 10
    prefix: tuple = (1024, 1024)   # inclusive range of prefix lengths
    p_match: tuple = (0.88, 0.88)  # per-sequence match probability range
    dtype: str = "bf16"
    tree: str = "topk"             # "topk" (random top-`branch` expansion), "chain" or "ranked" (ranked_tree)
    planting: str = "independent"  # "independent" or "ranked" (see plant_tokens_ranked)

    @property
    def T(self):
        return self.n_drafts + 1

    @property
    def K(self):
        return self.Hq * self.D


LLAMA8B_B1 = VerifyShape("llama8b-b1", 2, B=1, Hq=32, Hkv=8, D=128, V=128256, n_drafts=60, depth=7)
LLAMA8B_B64 = VerifyShape("llama8b-b64", 3, B=64, Hq=32, Hkv=8, D=128, V=128256, n_drafts=60, depth=7,
                          prefix=(200, 1500), p_match=(0.6, 0.95))
LLAMA70B_B8 = VerifyShape("llama70b-b8", 4, B=8, Hq=64, Hkv=8, D=128, V=128256, n_drafts=60, depth=8,
                          prefix=(4096, 4096))
# chain vs tree at equal node budgets (60 and 40 draft tokens), 8B shapes at
# batch 64, per-sequence match probability uniform in 0.6-0.95; siblings of a
# tree are alternatives (at most one of them is the target's token) and the
# tree is the one a calibrated drafter keeps (ranked_tree: depth <= 8, the
# number of draft steps; top-10 children). A chain and a tree of one budget
# share the workload id, so their prefixes, match probabilities and planting
# draws are the same: a paired comparison
CHAIN_TREE = tuple(
    VerifyShape(f"{kind}{n}-b64", wid, B=64, Hq=32, Hkv=8, D=128, V=128256, n_drafts=n,
                depth=n if kind == "chain" else 8, branch=1 if kind == "chain" else 10, prefix=(200, 1500),
                p_match=(0.6, 0.95), tree=kind if kind == "chain" else "ranked", planting="ranked")
    for wid, (kind, n) in ((5, ("chain", 60)), (5, ("tree", 60)), (7, ("chain", 40)), (7, ("tree", 40))))
VERIFY_SHAPES = {s.name: s for s in (LLAMA8B_B1, LLAMA8B_B64, LLAMA70B_B8) + CHAIN_TREE}


@dataclasses.dataclass
class VerifyInputs:
    shape: VerifyShape
    seed: int
    parent: np.ndarray      # int32 [B, T]
    kv: PagedKV
    q: np.ndarray           # uint16 [B, T, Hq, D]
    k_tree: np.ndarray      # uint16 [B, T, Hkv, D]
    v_tree: np.ndarray      # uint16 [B, T, Hkv, D]
    p_seq: np.ndarray       # float64 [B] planted match probability
    plant_u: np.ndarray     # float64 [B, T] uniforms for planting
    plant_id: np.ndarray    # int32 [B, T] random token ids for planting


def verify_inputs(shape: VerifyShape, seed: int, batch: slice | None = None) -> VerifyInputs:
    """Draw every verify-step input except the LM-head matrix (see lm_head_weight).

    ``batch`` restricts the draw to a subset of sequences while keeping their
    values identical to the full draw (generators are per component and the
    per-sequence loops consume them in order, so the full draw is made and
    then sliced for the small arrays; the prefix KV, the only large one, is
    drawn for every sequence up to the last requested one)."""
    B, T = shape.B, shape.T
    rl = child_rng(shape.wid, seed, C_PLEN)
    lo, hi = shape.prefix
    plen = rl.integers(lo, hi + 1, size=B).astype(np.int32)
    rp = child_rng(shape.wid, seed, C_PLANT)
    plo, phi = shape.p_match
    p_seq = rp.uniform(plo, phi, size=B) if phi > plo else np.full(B, plo)
    plant_u = rp.random((B, T))
    plant_id = rp.integers(0, shape.V, size=(B, T)).astype(np.int32)
    rt = child_rng(shape.wid, seed, C_TREE)
    if shape.tree == "chain":
        parent = np.stack([chain_tree(shape.n_drafts) for _ in range(B)])
    elif shape.tree == "ranked":
        parent = np.stack([ranked_tree(float(p_seq[b]), shape.n_drafts, shape.depth, shape.branch)
                           for b in range(B)])
    else:
        parent = np.stack([topk_tree(rt, shape.n_drafts, shape.depth, shape.branch) for _ in range(B)])
    q = normal_bf16(child_rng(shape.wid, seed, C_Q), (B, T, shape.Hq, shape.D))
    kt = normal_bf16(child_rng(shape.wid, seed, C_KTREE), (B, T, shape.Hkv, shape.D))
    vt = normal_bf16(child_rng(shape.wid, seed, C_VTREE), (B, T, shape.Hkv, shape.D))
    sel = np.arange(B) if batch is None else np.arange(B)[batch]
    max_blocks = max(1, (int(plen.max()) + 15) // 16)
    if batch is not None:
        # draw the KV of the selected sequences only: the per-sequence draws
        # come from one stream, so draw (and discard) the earlier ones
        last = int(sel.max()) + 1
        kv_all = paged_kv(shape.wid, seed, plen[:last], shape.Hkv, shape.D, max_blocks=max_blocks)
        kv = _select_kv(kv_all, sel)
    else:
        kv = paged_kv(shape.wid, seed, plen, shape.Hkv, shape.D, max_blocks=max_blocks)
    return VerifyInputs(shape, seed, parent[sel], kv, q[sel], kt[sel], vt[sel], p_seq[sel],
                        plant_u[sel], plant_id[sel])


def _select_kv(kv: PagedKV, sel: np.ndarray) -> PagedKV:
    """Keep the block pool (physical ids unchanged) and the selected rows."""
    return PagedKV(kv.k_cache, kv.v_cache, kv.block_table[sel].copy(), kv.prefix_len[sel].copy(), kv.block_size)


def lm_head_weight(shape_or_wid, V: int, K: int, std: float = 0.02, threads: int | None = None) -> np.ndarray:
    """LM-head matrix [V, K] (vocabulary-major), N(0, std^2) in bf16. The model
    is fixed per workload: seeds vary the inputs, not the weights.

    Rows come in blocks of 2048, block i from its own generator
    default_rng([workload_id, 0, C_WLM, i]), so blocks can be drawn in
    parallel threads with identical results."""
    import concurrent.futures
    import os
    wid = shape_or_wid.wid if hasattr(shape_or_wid, "wid") else int(shape_or_wid)
    out = np.empty((V, K), dtype=np.uint16)
    RB = 2048

    def block(i):
        r0 = i * RB
        r1 = min(V, r0 + RB)
        rng = np.random.default_rng([wid, 0, C_WLM, i])
        out[r0:r1] = normal_bf16(rng, (r1 - r0, K), std=std)

    nthreads = threads or min(16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(block, range((V + RB - 1) // RB)))
    return out


def plant_tokens(parent: np.ndarray, target_idx: np.ndarray, p_seq, plant_u, plant_id) -> np.ndarray:
    """Draft tokens planted against a target argmax array.

    For each non-root node n: tok[n] = target_idx[parent[n]] when the node's
    uniform is below the sequence's match probability, else the node's random
    id (which can still match by chance). The root's token is the random id.
    ``target_idx`` must come from the oracle, never from the GPU path."""
    parent = np.atleast_2d(parent)
    target_idx = np.atleast_2d(target_idx)
    B, T = parent.shape
    tok = np.array(np.atleast_2d(plant_id), dtype=np.int32, copy=True)
    p_seq = np.broadcast_to(np.asarray(p_seq, dtype=np.float64), (B,))
    for b in range(B):
        for n in range(1, T):
            if plant_u[b][n] < p_seq[b]:
                tok[b, n] = target_idx[b, parent[b, n]]
    return tok


def plant_tokens_ranked(parent: np.ndarray, target_idx: np.ndarray, p_seq, plant_u, plant_id) -> np.ndarray:
    """Draft tokens planted with siblings as alternatives.

    The children of a node, in index order, are its draft's ranked
    candidates: child j (rank j) carries the target's token at the parent
    when its uniform is below the sequence's match probability and no earlier
    sibling does (so rank j matches with probability p (1 - p)^(j - 1), and at
    most one sibling matches); every other child carries its random id (which
    can still match by chance). For a chain this is plant_tokens. The root's
    token is its random id. ``target_idx`` must come from the oracle."""
    parent = np.atleast_2d(parent)
    target_idx = np.atleast_2d(target_idx)
    B, T = parent.shape
    tok = np.array(np.atleast_2d(plant_id), dtype=np.int32, copy=True)
    p_seq = np.broadcast_to(np.asarray(p_seq, dtype=np.float64), (B,))
    for b in range(B):
        taken = np.zeros(T, dtype=bool)   # parent already has its matching child
        for n in range(1, T):
            p = parent[b, n]
            if not taken[p] and plant_u[b][n] < p_seq[b]:
                tok[b, n] = target_idx[b, p]
                taken[p] = True
    return tok


def plant_for(inp, target_idx) -> np.ndarray:
    """Draft tokens of a verify workload, by its planting rule."""
    f = plant_tokens_ranked if inp.shape.planting == "ranked" else plant_tokens
    return f(inp.parent, target_idx, inp.p_seq, inp.plant_u, inp.plant_id)


# ---------------------------------------------------------------- toy decoder

@dataclasses.dataclass
class ToyShape:
    name: str = "toy-lossless"
    wid: int = 1
    layers: int = 2
    K: int = 256
    H: int = 4
    D: int = 64
    V: int = 4096
    F: int = 896
    prompt: int = 128
    new_tokens: int = 64
    p_match: float = 0.88
    theta: float = 500000.0
    eps: float = 1e-5
    std: float = 0.02


TOY = ToyShape()


def toy_weights(shape: ToyShape = TOY, seed: int = 0) -> dict:
    """fp32 N(0, std^2) weights of a Llama-style decoder, untied embedding/head.

    Matrices are stored output-major ([out, in]) so that y = x @ W.T."""
    r = child_rng(shape.wid, seed, C_WEIGHTS)
    K, F, V = shape.K, shape.F, shape.V
    HD = shape.H * shape.D
    w = {"embed": normal_f32(r, (V, K), shape.std)}
    for i in range(shape.layers):
        w[f"l{i}.wqkv"] = normal_f32(r, (3 * HD, K), shape.std)
        w[f"l{i}.wo"] = normal_f32(r, (K, HD), shape.std)
        w[f"l{i}.wgu"] = normal_f32(r, (2 * F, K), shape.std)   # rows [0,F) gate, [F,2F) up
        w[f"l{i}.wd"] = normal_f32(r, (K, F), shape.std)
    w["lm_head"] = normal_f32(r, (V, K), shape.std)
    return w


def toy_prompt(shape: ToyShape = TOY, seed: int = 0) -> np.ndarray:
    return child_rng(shape.wid, seed, C_PROMPT).integers(0, shape.V, size=shape.prompt).astype(np.int32)


def toy_plant_stream(shape: ToyShape = TOY, seed: int = 0):
    return child_rng(shape.wid, seed, C_PLANT)


# ---------------------------------------------------------------- draft head

@dataclasses.dataclass
class DraftShape:
    """EAGLE-3 draft head + tree growth (news write-up of the EAGLE-3 paper,
    draft-stage paragraphs; top-k 10 and 60 draft tokens from the Spec-Bench
    blog post's inference table)."""
    name: str = "draft-b64"
    wid: int = 5
    B: int = 64
    k: int = 4096
    V: int = 128256
    ctx: int = 1024
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    F: int = 14336
    steps: int = 8
    topk: int = 10
    n_drafts: int = 60
    theta: float = 500000.0
    eps: float = 1e-5
    std: float = 0.02
    lm_std: float = 0.02
    vocab_keep: int = 0          # rows of a trimmed draft LM head (0: the full vocabulary)

    @property
    def pool_len(self):
        return self.topk + (self.steps - 1) * self.topk * self.topk


DRAFT_B64 = DraftShape()
# small draft head for element-wise parity; a 15x larger LM-head scale spreads
# the draft logits so fewer selection boundaries are near-ties
DRAFT_SMALL = DraftShape("draft-small", 25, B=6, k=256, V=2000, ctx=96, Hq=4, Hkv=2, D=128, F=512, lm_std=0.3)
# trimmed draft vocabularies (Spec-Bench blog post, sections 1 and 5.1: the
# draft's search space shrinks by 40-60%): half of the rows kept; same weights
DRAFT_B64_TRIM = dataclasses.replace(DRAFT_B64, name="draft-b64-trim", vocab_keep=64128)
DRAFT_SMALL_TRIM = dataclasses.replace(DRAFT_SMALL, name="draft-small-trim", vocab_keep=1000)


def draft_vocab(shape: DraftShape) -> np.ndarray | None:
    """The kept ids of a trimmed draft vocabulary: vocab_keep distinct ids of
    [0, V), ascending, drawn uniformly (a stand-in for a frequency-ranked
    subset, which needs corpus statistics); None for the full vocabulary."""
    if not shape.vocab_keep:
        return None
    rng = child_rng(shape.wid, 0, C_VOCAB)
    return np.sort(rng.choice(shape.V, shape.vocab_keep, replace=False)).astype(np.int32)


def _blocks_bf16(wid: int, comp: int, shape, std: float, rb: int = 2048, threads: int | None = None) -> np.ndarray:
    """bf16 N(0, std^2) matrix drawn in row blocks from their own generators
    default_rng([wid, 0, comp, i]), in parallel threads."""
    import concurrent.futures
    import os
    rows, cols = int(shape[0]), int(np.prod(shape[1:]))
    out = np.empty((rows, cols), dtype=np.uint16)

    def block(i):
        r0, r1 = i * rb, min(rows, (i + 1) * rb)
        out[r0:r1] = normal_bf16(np.random.default_rng([wid, 0, comp, i]), (r1 - r0, cols), std=std)

    with concurrent.futures.ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(block, range((rows + rb - 1) // rb)))
    return out.reshape(shape)


def draft_weights(shape: DraftShape) -> dict:
    """bf16 weights of the draft head, output-major ([out, in]); the LM head is
    the target's. Fixed per workload."""
    k, V, F = shape.k, shape.V, shape.F
    qd, kvd = shape.Hq * shape.D, shape.Hkv * shape.D
    spec = {"embed": ((V, k), shape.std), "w_fuse": ((k, 3 * k), shape.std), "w_in": ((k, 2 * k), shape.std),
            "wqkv": ((qd + 2 * kvd, k), shape.std), "wo": ((k, qd), shape.std), "wgu": ((2 * F, k), shape.std),
            "wd": ((k, F), shape.std), "lm_head": ((V, k), shape.lm_std)}
    return {name: _blocks_bf16(shape.wid, 100 + i, shp, std) for i, (name, (shp, std)) in enumerate(spec.items())}


def draft_inputs(shape: DraftShape, seed: int, batch: slice | None = None):
    """Target features l, m, h [B, ctx, k] ~ N(0, 1) (bf16) and the token one
    step ahead of every context row, ctx_tok [B, ctx]; the last entry of each
    row is the root (the token the target just emitted)."""
    B = shape.B
    sel = np.arange(B) if batch is None else np.arange(B)[batch]
    feats = []
    for c in range(3):
        # per-sequence draws, so a subset of sequences costs only what it uses
        rows = [normal_bf16(np.random.default_rng([shape.wid, seed, C_FEAT, c, int(b)]), (shape.ctx, shape.k))
                for b in sel]
        feats.append(np.stack(rows))
    tok = child_rng(shape.wid, seed, C_CTX).integers(0, shape.V, size=(B, shape.ctx)).astype(np.int32)[sel]
    return feats[0], feats[1], feats[2], tok


def ceil_div(a, b):
    return (a + b - 1) // b



@dataclasses.dataclass
class AttnInputs:
    q: np.ndarray        # [B, Tq, Hq, D]
    k_tree: np.ndarray   # [B, Tk, Hkv, D]
    v_tree: np.ndarray   # [B, Tk, Hkv, D]
    kv: PagedKV


def attn_inputs(workload_id: int, seed: int, B: int, Tq: int, Tk: int, Hq: int, Hkv: int, D: int,
                prefix_len, dtype: str = "bf16", q_scale: float = 1.0) -> AttnInputs:
    """Generic tree-attention inputs with N(0,1) values (q times q_scale)."""
    draw = normal_f32 if dtype == "f32" else normal_bf16
    kv = paged_kv(workload_id, seed, prefix_len, Hkv, D, dtype=dtype)
    q = draw(child_rng(workload_id, seed, C_Q), (B, Tq, Hq, D), q_scale)
    kt = draw(child_rng(workload_id, seed, C_KTREE), (B, Tk, Hkv, D))
    vt = draw(child_rng(workload_id, seed, C_VTREE), (B, Tk, Hkv, D))
    return AttnInputs(q, kt, vt, kv)


# ---------------------------------------------------------------- target model

@dataclasses.dataclass(frozen=True)
class TargetShape:
    """A Llama-style target decoder run over a batch of draft trees (the
    verify pass with the target's own layers: QKV / O / MLP GEMMs at
    M = B * T rows, RoPE at P + depth, tree attention over a paged prefix per
    layer). 8B shapes by default (LLaMA-3-8B: 32 layers, hidden 4096, 32 / 8
    heads of 128, FFN 14336, vocab 128256); random weights."""
    name: str = "target8b-b64"
    wid: int = 9
    layers: int = 32
    B: int = 64
    k: int = 4096
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    F: int = 14336
    V: int = 128256
    n_drafts: int = 60
    depth: int = 7
    branch: int = 10
    prefix: tuple = (200, 1500)
    theta: float = 500000.0
    eps: float = 1e-5
    std: float = 0.02
    # the layers whose outputs feed a draft head as low / mid / high features
    features: tuple = (2, 16, 29)

    @property
    def T(self):
        return self.n_drafts + 1


TARGET_8B = TargetShape()
# small shapes for element-wise parity: two layers, several tiles, ragged tails
TARGET_SMALL = TargetShape("target-small", 31, layers=2, B=3, k=256, Hq=4, Hkv=2, D=128, F=512, V=2000,
                           n_drafts=40, depth=6, prefix=(37, 300), features=(0, 1))


def target_weights(shape: TargetShape) -> dict:
    """bf16 N(0, std^2) weights, output-major ([out, in]): embed [V, k],
    lm_head [V, k], and per layer i: l{i}.wqkv [(Hq + 2 Hkv) D, k] (q rows,
    then k, then v), l{i}.wo [k, Hq D], l{i}.wgu [2F, k] (gate rows, then up),
    l{i}.wd [k, F]. Each matrix from its own row-block streams."""
    k, F, V = shape.k, shape.F, shape.V
    qd, kvd = shape.Hq * shape.D, shape.Hkv * shape.D
    W = {"embed": _blocks_bf16(shape.wid, 300, (V, k), shape.std),
         "lm_head": _blocks_bf16(shape.wid, 301, (V, k), shape.std)}
    for i in range(shape.layers):
        for j, (name, shp) in enumerate((("wqkv", (qd + 2 * kvd, k)), ("wo", (k, qd)), ("wgu", (2 * F, k)),
                                         ("wd", (k, F)))):
            W[f"l{i}.{name}"] = _blocks_bf16(shape.wid, 400 + 4 * i + j, shp, shape.std)
    return W


@dataclasses.dataclass
class TargetInputs:
    shape: TargetShape
    seed: int
    parent: np.ndarray      # int32 [B, T]
    tokens: np.ndarray      # int32 [B, T] (node 0: the last committed token)
    prefix_len: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks], shared by every layer
    k_cache: list           # per layer [num_blocks, Hkv, 16, D]
    v_cache: list           # per layer [num_blocks, Hkv, D, 16]

    def kv(self, layer: int, batch=None) -> PagedKV:
        bt, pl = self.block_table, self.prefix_len
        if batch is not None:
            bt, pl = bt[batch], pl[batch]
        return PagedKV(self.k_cache[layer], self.v_cache[layer], bt, pl, 16)


def target_inputs(shape: TargetShape, seed: int, batch: slice | None = None, dtype: str = "bf16",
                  threads: int | None = None, reserve: int = 16) -> TargetInputs:
    """Trees (random top-`branch` expansion), uniform random tokens and a
    per-layer prefix K/V ~ N(0, 1) standing in for a committed context of
    prefix_len tokens (uniform in shape.prefix). One shuffled block pool per
    layer under one block table; every sequence owns blocks for `reserve`
    more tokens after its prefix (room to commit accepted rows); unused slots
    hold NaN. Each (layer, sequence) prefix comes from its own stream, so
    ``batch`` draws only the sequences it keeps (the block table is still the
    full batch's)."""
    import concurrent.futures
    import os
    B, T, bs = shape.B, shape.T, 16
    rt = child_rng(shape.wid, seed, C_TREE)
    parent = np.stack([topk_tree(rt, shape.n_drafts, shape.depth, shape.branch) for _ in range(B)])
    tokens = child_rng(shape.wid, seed, C_PROMPT).integers(0, shape.V, size=(B, T)).astype(np.int32)
    lo, hi = shape.prefix
    plen = child_rng(shape.wid, seed, C_PLEN).integers(lo, hi + 1, size=B).astype(np.int32)
    nb = (plen + bs - 1) // bs
    own = (plen + reserve + bs - 1) // bs            # blocks a sequence owns
    nblk = int(own.sum()) + 1
    perm = child_rng(shape.wid, seed, C_PERM).permutation(nblk).astype(np.int32)
    max_blocks = int(own.max())
    table = np.full((B, max_blocks), perm[-1], np.int32)
    off = np.concatenate([[0], np.cumsum(own)])
    for b in range(B):
        table[b, :own[b]] = perm[off[b]:off[b + 1]]
    keep = np.arange(B) if batch is None else np.arange(B)[batch]
    f32 = dtype == "f32"
    npdt, nan = (np.float32, np.float32(np.nan)) if f32 else (np.uint16, BF16_NAN)
    draw = normal_f32 if f32 else normal_bf16
    Hkv, D = shape.Hkv, shape.D
    kc = [np.full((nblk, Hkv, bs, D), nan, npdt) for _ in range(shape.layers)]
    vc = [np.full((nblk, Hkv, D, bs), nan, npdt) for _ in range(shape.layers)]

    def fill(job):
        layer, b = job
        L = int(plen[b])
        kb = draw(np.random.default_rng([shape.wid, seed, C_KPRE, layer, b]), (L, Hkv, D))
        vb = draw(np.random.default_rng([shape.wid, seed, C_VPRE, layer, b]), (L, Hkv, D))
        for j in range(nb[b]):
            phys = table[b, j]
            r0, r1 = j * bs, min(L, (j + 1) * bs)
            kc[layer][phys, :, :r1 - r0, :] = kb[r0:r1].transpose(1, 0, 2)
            vc[layer][phys, :, :, :r1 - r0] = vb[r0:r1].transpose(1, 2, 0)

    jobs = [(layer, int(b)) for layer in range(shape.layers) for b in keep]
    with concurrent.futures.ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, jobs))
    return TargetInputs(shape, seed, parent, tokens, plen, table, kc, vc)


# device-resident speculative loop: a target and a draft head sharing the
# vocabulary (the draft uses the target's embedding and LM head). The small
# pair has 16 tokens, so a top-10 draft often holds the target's choice and
# multi-token acceptances occur; both contexts hold `ctx` committed tokens.
LOOP_TARGET_SMALL = TargetShape("loop-target-small", 33, layers=2, B=3, k=256, Hq=4, Hkv=2, D=128, F=512, V=16,
                                n_drafts=20, depth=4, prefix=(96, 96), features=(0, 1, 1))
LOOP_DRAFT_SMALL = DraftShape("loop-draft-small", 34, B=3, k=256, V=16, ctx=96, Hq=4, Hkv=2, D=128, F=512, steps=4,
                              topk=10, n_drafts=20, lm_std=0.3)
LOOP_TARGET_8B = dataclasses.replace(TARGET_8B, name="loop-target8b", prefix=(1024, 1024))
