"""Seeded input generators (host side, NumPy).

Everything here builds *inputs*: draft-tree topologies, draft tokens, target
logits with a chosen per-node maximum, and KV caches in the three storage
formats the library reads (fp32, bf16 bits, int8 codes + fp16 per-token
scales). None of the verification steps is computed here.

Streams: every tensor draws from its own ``numpy.random.Generator`` built from
``SeedSequence(seed, spawn_key=(stream ids...))`` so adding a tensor never
shifts the values of another.
"""

from __future__ import annotations

import heapq
import math

import numpy as np

__all__ = [
    "rng_for",
    "chain_tree",
    "binary_tree_7",
    "sary_tree",
    "random_tree",
    "confidence_tree",
    "children_lists",
    "random_descent",
    "plant_walk",
    "planted_logits",
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "quantize_int8_per_token",
    "unique_fp16_scales",
    "make_kv_cache",
    "make_queries",
    "draft_rows",
    "lm_head_inputs",
    "quantize_q4_groups",
    "lm_head_q4_inputs",
    "lm_head_q4_random",
]


def rng_for(seed: int, *stream: int) -> np.random.Generator:
    """Independent generator for (seed, stream ids)."""
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(int(s) for s in stream)))


# ----------------------------------------------------------------------------
# Topologies. Nodes are labelled in a topological order (parent[i] < i), node 0
# is the root (the last committed token) with parent -1.
# ----------------------------------------------------------------------------

def chain_tree(T: int) -> np.ndarray:
    """Linear tree: parent[i] = i - 1."""
    return np.arange(-1, T - 1, dtype=np.int32)


def binary_tree_7(rng: np.random.Generator) -> np.ndarray:
    """Root + 2 + 4 binary tree with a random topological labelling.

    The shape is fixed (root r; children a, b; a has a1, a2; b has b1, b2); the
    labels are a uniformly drawn linear extension of the parent-before-child
    order, so labellings such as a, a1, b, ... occur as well as plain BFS.
    """
    shape_parent = {0: -1, 1: 0, 2: 0, 3: 1, 4: 1, 5: 2, 6: 2}  # shape ids
    kids = {u: [v for v, p in shape_parent.items() if p == u] for u in shape_parent}
    order = [0]
    frontier = list(kids[0])
    while frontier:
        pick = frontier.pop(int(rng.integers(0, len(frontier))))
        order.append(pick)
        frontier.extend(kids[pick])
    label = {shape: i for i, shape in enumerate(order)}
    parent = np.full(7, -1, dtype=np.int32)
    for shape, p in shape_parent.items():
        parent[label[shape]] = -1 if p < 0 else label[p]
    return parent


def sary_tree(s: int, depth: int) -> np.ndarray:
    """Full s-ary tree of the given depth (levels below the root), BFS labels."""
    parent = [-1]
    level = [0]
    for _ in range(depth):
        nxt = []
        for u in level:
            for _ in range(s):
                parent.append(u)
                nxt.append(len(parent) - 1)
        level = nxt
    return np.asarray(parent, dtype=np.int32)


def random_tree(rng: np.random.Generator, T: int) -> np.ndarray:
    """Random recursive tree: parent[i] ~ U{0..i-1}."""
    parent = np.empty(T, dtype=np.int32)
    parent[0] = -1
    for i in range(1, T):
        parent[i] = int(rng.integers(0, i))
    return parent


def confidence_tree(rng: np.random.Generator, n_nodes: int = 16, max_depth: int = 8,
                    vocab: int = 248320, topk: int = 4):
    """EAGLE-2-like draft tree grown best-first by cumulative drafter probability.

    Each expanded node draws ``topk`` distinct candidate tokens and drafter
    logits for them (N(0, 2^2)); a candidate's score is the sum of log
    probabilities along its root path (the drafter softmax leaves a seeded
    share of the mass to unlisted tokens). The best candidate is inserted next,
    so labels are topological and siblings carry distinct tokens.

    Returns (parent int32 [n], tokens int64 [n]); tokens[0] is the root token.
    """
    parent = [-1]
    depth = [0]
    tokens = [int(rng.integers(0, vocab))]
    score = [0.0]
    heap: list = []
    tie = 0

    def expand(u: int) -> None:
        nonlocal tie
        if depth[u] >= max_depth:
            return
        cand = rng.choice(vocab, size=topk, replace=False)
        z = rng.standard_normal(topk) * 2.0
        z = z - z.max()
        p = np.exp(z) / np.exp(z).sum() * rng.uniform(0.5, 1.0)
        for tok, pi in zip(cand, p):
            heapq.heappush(heap, (-(score[u] + math.log(pi)), tie, u, int(tok)))
            tie += 1

    expand(0)
    while len(parent) < n_nodes and heap:
        neg, _, u, tok = heapq.heappop(heap)
        parent.append(u)
        depth.append(depth[u] + 1)
        tokens.append(tok)
        score.append(-neg)
        expand(len(parent) - 1)
    return np.asarray(parent, dtype=np.int32), np.asarray(tokens, dtype=np.int64)


def children_lists(parent) -> list:
    """Children of every node in ascending label order."""
    kids = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        kids[int(parent[i])].append(i)
    return kids


def random_descent(parent, rng: np.random.Generator, first_child_not=None) -> list:
    """Random root-to-leaf descent (list of node ids starting with 0).

    ``first_child_not`` excludes one child of the root from the first step when
    the root has another child (used to build paths whose first step is not
    node 1, the worst case for an in-place rollback).
    """
    kids = children_lists(parent)
    path = [0]
    u = 0
    while kids[u]:
        options = kids[u]
        if u == 0 and first_child_not is not None and len(options) > 1:
            options = [c for c in options if c != first_child_not]
        u = options[int(rng.integers(0, len(options)))]
        path.append(u)
    return path


# ----------------------------------------------------------------------------
# Draft tokens and target argmaxes consistent with a chosen accepted path.
# ----------------------------------------------------------------------------

def plant_walk(parent, path, rng: np.random.Generator, vocab: int, tokens=None,
               equal_sibling: bool = False):
    """Choose draft tokens and per-node target argmaxes so that ``path`` is the
    accepted root path.

    Constraints set up here (the walk itself is not evaluated):
    * for consecutive path nodes u -> n: target[u] = token[n], and no child of u
      with a lower label than n carries token[n];
    * at the last path node e: target[e] differs from every child's token.
    Off-path targets are uniform draws. With ``equal_sibling`` one path node n
    that has a higher-labelled sibling s gets that sibling's token duplicated
    (token[s] = token[n]), so two siblings both carry the target's token.

    Returns (tokens int64 [T], targets int64 [T], dup) where dup is the
    (n, s) pair used for the duplicate, or None.
    """
    T = len(parent)
    kids = children_lists(parent)
    tok = (rng.integers(0, vocab, size=T) if tokens is None else np.array(tokens, dtype=np.int64)).astype(np.int64)
    tgt = rng.integers(0, vocab, size=T).astype(np.int64)

    def fresh(avoid) -> int:
        while True:
            x = int(rng.integers(0, vocab))
            if x not in avoid:
                return x

    for k in range(len(path) - 1):
        u, n = path[k], path[k + 1]
        for c in kids[u]:
            if c < n and tok[c] == tok[n]:
                tok[c] = fresh({int(tok[n])})
        tgt[u] = tok[n]
    dup = None
    if equal_sibling:
        for k in range(1, len(path)):
            n = path[k]
            sibs = [c for c in kids[path[k - 1]] if c > n]
            if sibs:
                s = sibs[int(rng.integers(0, len(sibs)))]
                tok[s] = tok[n]
                dup = (n, s)
                break
        if dup is None:
            raise ValueError("no path node has a higher-labelled sibling")
    end = path[-1]
    tgt[end] = fresh({int(tok[c]) for c in kids[end]})
    return tok, tgt, dup


def planted_logits(rng: np.random.Generator, targets, vocab: int, sigma: float) -> np.ndarray:
    """fp32 logits [N, vocab] ~ N(0, sigma^2) whose unique row maximum sits at
    targets[n] (that entry is set to the row's largest draw plus 1)."""
    targets = np.asarray(targets)
    N = len(targets)
    x = rng.standard_normal((N, vocab), dtype=np.float32)
    x *= np.float32(sigma)
    rows = np.arange(N)
    x[rows, targets] = x.max(axis=1) + np.float32(1.0)
    return x


# ----------------------------------------------------------------------------
# Storage formats.
# ----------------------------------------------------------------------------

def to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_int8_per_token(x):
    """Symmetric per-token int8: scale = fp16(max|x| / 127) (RNE),
    code = clip(rint(x / scale), -127, 127) with half-to-even rint; a zero
    scale gives zero codes. x: float32 [..., D] -> (int8 [..., D], float16 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float16)
    s32 = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(x / np.where(s32 > 0, s32, 1)), 0)
    return np.clip(q, -127, 127).astype(np.int8), scale


def unique_fp16_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """Positive finite fp16 scales, pairwise distinct along the last axis
    (needs last axis <= 26,623)."""
    shape = tuple(shape)
    n = shape[-1]
    lo, hi = 0x1400, 0x7BFF
    if n > hi - lo:
        raise ValueError("too many tokens for distinct fp16 scales")
    lead = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    bits = np.empty((lead, n), dtype=np.uint16)
    for r in range(lead):
        bits[r] = lo + rng.permutation(hi - lo)[:n]
    return bits.reshape(shape).view(np.float16)


def make_kv_cache(seed: int, stream: int, B: int, Hkv: int, cap: int, D: int, dtype: str,
                  unique_scales: bool = False):
    """One layer's K and V, layout [B, Hkv, cap, D], values N(0, 1).

    dtype 'f32' -> float32 arrays; 'bf16' -> uint16 bf16 bit patterns (RNE);
    'i8' -> int8 codes plus float16 scales [B, Hkv, cap] (per token, per KV
    head). With ``unique_scales`` the int8 scales are replaced by pairwise
    distinct values per (b, head) (codes unchanged) so a gather that moves
    codes without their scales cannot match.
    """
    out = {}
    for name, sid in (("k", 0), ("v", 1)):
        g = rng_for(seed, stream, sid)
        x = g.standard_normal((B, Hkv, cap, D), dtype=np.float32)
        if dtype == "f32":
            out[name] = x
        elif dtype == "bf16":
            out[name] = to_bf16_bits(x)
        elif dtype == "i8":
            code, scale = quantize_int8_per_token(x)
            if unique_scales:
                scale = unique_fp16_scales(rng_for(seed, stream, sid, 7), (B, Hkv, cap))
            out[name] = code
            out[name + "_scale"] = scale
        else:
            raise ValueError(dtype)
    return out


def make_queries(seed: int, stream: int, n_nodes: int, Hq: int, D: int, dtype: str) -> np.ndarray:
    """Q [n_nodes, Hq, D] ~ N(0, 1): float32, or bf16 bit patterns."""
    x = rng_for(seed, stream).standard_normal((n_nodes, Hq, D), dtype=np.float32)
    return x if dtype == "f32" else to_bf16_bits(x)


def draft_rows(seed: int, B: int, n_depths: int, top_k: int, vocab: int, sigma: float = 2.0) -> list:
    """Synthetic drafter logits for confidence branching, fp32 N(0, sigma^2):
    entry d is [B, F_d, vocab] with F_0 = 1 (the root's row) and F_d = top_k
    after (one row per frontier slot). The rows stand in for a drafter run on
    the frontier; they do not depend on which candidates the frontier holds."""
    out = []
    for d in range(n_depths):
        F = 1 if d == 0 else top_k
        r = rng_for(seed, 40, d)
        out.append((r.standard_normal((B, F, vocab), dtype=np.float32) * np.float32(sigma)).astype(np.float32))
    return out


def lm_head_inputs(seed: int, N: int, H: int, V: int, planted=None, duplicate=None):
    """Synthetic LM-head operands as bf16 bit patterns: hidden states [N, H]
    N(0, 1) and a head weight [V, H] N(0, 1/H) (unit-variance logits).
    planted: {node n: vocab row t} makes row t a multiple of hidden[n]'s
    direction, so t carries node n's largest logit by a wide margin.
    duplicate: [(a, b)] copies weight row a onto row b (equal logits)."""
    r = rng_for(seed, 50)
    X = r.standard_normal((N, H), dtype=np.float32)
    W = r.standard_normal((V, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    hb = to_bf16_bits(X)
    if planted:
        for n, t in planted.items():
            W[t] = bf16_bits_to_f32(hb[n]) * np.float32(4.0 / np.sqrt(H))
    wb = to_bf16_bits(W)
    if duplicate:
        for a, b in duplicate:
            wb[b] = wb[a]
    return hb, wb


def quantize_q4_groups(W) -> tuple:
    """Affine 4-bit quantisation of W [V, H] in groups of 64 along H: per
    group scale = (max - min) / 15 and bias = min, both rounded to bf16, codes
    round((w - bias) / scale) clipped to 0..15 (a constant group gets scale 0
    and code 0). Returns (wq uint32 [V, H/8], element i in bits 4 (i mod 8) of
    word i / 8; sb bf16 bits [H/64, V, 2] holding (scale, bias))."""
    W = np.asarray(W, dtype=np.float32)
    V, H = W.shape
    G = H // 64
    g = W.reshape(V, G, 64)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    s_bits = to_bf16_bits((hi - lo) / np.float32(15))
    b_bits = to_bf16_bits(lo)
    s = bf16_bits_to_f32(s_bits).astype(np.float64)[:, :, None]
    b = bf16_bits_to_f32(b_bits).astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((g - b) / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, 15).astype(np.uint32).reshape(V, H)
    wq = np.zeros((V, H // 8), dtype=np.uint32)
    for j in range(8):
        wq |= q[:, j::8] << np.uint32(4 * j)
    sb = np.stack([s_bits.T, b_bits.T], axis=2).astype(np.uint16)
    return wq, np.ascontiguousarray(sb)


def lm_head_q4_inputs(seed: int, N: int, H: int, V: int, planted=None):
    """Hidden states [N, H] N(0, 1) as bf16 bits and a 4-bit head quantised
    from N(0, 1/H) weights. planted: {node n: vocab row t} quantises row t
    from a multiple of hidden[n], so t carries node n's largest logit by a
    wide margin."""
    r = rng_for(seed, 51)
    X = r.standard_normal((N, H), dtype=np.float32)
    W = r.standard_normal((V, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    hb = to_bf16_bits(X)
    if planted:
        for n, t in planted.items():
            W[t] = bf16_bits_to_f32(hb[n]) * np.float32(4.0 / np.sqrt(H))
    wq, sb = quantize_q4_groups(W)
    return hb, wq, sb


def lm_head_q4_random(seed: int, N: int, H: int, V: int, planted=None):
    """A 4-bit head drawn directly in packed form (no float copy of the
    weight, so the full 248,320 x 5,120 head fits in host memory): uniform
    codes 0..15, per group scale s ~ U(0.5, 1.5) / (4.6 sqrt(H)) and bias
    about -7.5 s (values centred, unit-variance logits), both bf16; hidden
    states N(0, 1). planted: {node n: row t} re-quantises row t from a
    multiple of hidden[n]."""
    r = rng_for(seed, 52)
    X = r.standard_normal((N, H), dtype=np.float32)
    hb = to_bf16_bits(X)
    G = H // 64
    wq = r.integers(0, 2 ** 32, size=(V, H // 8), dtype=np.uint32)
    sc = (r.uniform(0.5, 1.5, size=(G, V)) / (4.6 * np.sqrt(H))).astype(np.float32)
    bi = (-7.5 * sc * r.uniform(0.9, 1.1, size=(G, V))).astype(np.float32)
    sb = np.stack([to_bf16_bits(sc), to_bf16_bits(bi)], axis=2).astype(np.uint16)
    if planted:
        for n, t in planted.items():
            row = bf16_bits_to_f32(hb[n]) * np.float32(4.0 / np.sqrt(H))
            q1, sb1 = quantize_q4_groups(row[None, :])
            wq[t] = q1[0]
            sb[:, t, :] = sb1[:, 0, :]
    return hb, wq, np.ascontiguousarray(sb)

