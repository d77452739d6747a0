"""The five synthetic workloads, as seeded recipes.

Shapes and distributions follow the workloads the pages describe (draft trees
of up to 64 nodes over a long KV prefix, 40 query / 8 KV heads with head_dim
128, vocab 248,320, bf16 or int8 KV with per-token fp16 scales). The pages
measure on model checkpoints and prompt cohorts; these seeded synthetics stand
in for them.

``RoundSpec`` carries the per-round metadata (topologies, draft tokens, target
argmax plants, prefix lengths, planned accept paths); it is small and always
built on the host. Bulk tensors (KV caches, queries, logits) come either from
``host_tensors`` (NumPy, small configs) or from ``workloads.device`` (torch on
the GPU, large configs).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import (binary_tree_7, chain_tree, confidence_tree, make_kv_cache, make_queries,
                  plant_walk, planted_logits, random_descent, random_tree, rng_for, sary_tree)

__all__ = ["RoundSpec", "config1_round", "config2_round", "config3_round", "config4_round",
           "config5_round", "config5_schedule", "host_tensors", "CONFIG_TEXT"]

CONFIG_TEXT = {
    1: "tiny fp32 round: B=1, 1 layer, Hq=4/Hkv=2, D=64, prefix 64, 7-node binary tree, vocab 1024",
    2: "linear chains T=3/4/8: B=1, bf16, Hq=40/Hkv=8, D=128, prefix 2048, vocab 248320",
    3: "16-node confidence tree: B=1, 16 layers, int8 KV + fp16 scales, Hq=40/Hkv=8, D=128, prefix 4096, vocab 248320",
    4: "batched ragged rounds: B=32, bf16, Hq=40/Hkv=8, D=128, prefixes U{1024..32768}, trees of 8-64 nodes, vocab 248320",
    5: "long-context stress: B=8, 8 layers, int8 KV + fp16 scales, Hq=40/Hkv=8, D=128, prefix 131072, 16-node trees, vocab 248320",
}


@dataclass
class RoundSpec:
    seed: int
    B: int
    L: int
    Hq: int
    Hkv: int
    D: int
    vocab: int
    sigma: float
    kv_dtype: str          # 'f32' | 'bf16' | 'i8'
    q_dtype: str           # 'f32' | 'bf16'
    hist_len: np.ndarray   # int32 [B]
    parents: list          # per sequence int32 [T_b]
    tokens: list           # per sequence int64 [T_b]
    targets: list          # per sequence int64 [T_b] (planted per-node argmax)
    paths: list            # per sequence planned accepted path (node ids from 0)
    cap: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def node_off(self) -> np.ndarray:
        off = np.zeros(self.B + 1, dtype=np.int32)
        off[1:] = np.cumsum([len(p) for p in self.parents])
        return off

    @property
    def n_nodes(self) -> int:
        return int(sum(len(p) for p in self.parents))

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def flat(self, name: str) -> np.ndarray:
        arrs = getattr(self, name)
        dt = np.int32 if name == "parents" else np.int64
        return np.concatenate([np.asarray(a, dtype=dt) for a in arrs]) if arrs else np.zeros(0, dt)

    @property
    def flat_targets(self) -> np.ndarray:
        return self.flat("targets")


def _spec(seed, B, L, Hq, Hkv, D, vocab, sigma, kv, q, hist, parents, tokens, targets, paths, note=""):
    hist = np.asarray(hist, dtype=np.int32)
    cap = int(max(int(h) + len(p) for h, p in zip(hist, parents))) if B else 0
    return RoundSpec(seed, B, L, Hq, Hkv, D, vocab, sigma, kv, q, hist, list(parents), list(tokens),
                     list(targets), list(paths), cap=cap, note=note)


def config1_round(accepted: int | None = None, equal_sibling: bool = False, seed: int = 1) -> RoundSpec:
    """Tiny fp32 round. The tree (root + 2 + 4) has depth 2 and node 0 is the
    committed token, so an accepted count of 0, 1 or 2 is reachable; it is drawn
    uniformly unless given. ``equal_sibling`` duplicates the on-path node's
    token onto a higher-labelled sibling."""
    r = rng_for(seed, 0)
    parent = binary_tree_7(rng_for(seed, 1))
    if accepted is None:
        accepted = int(r.integers(0, 3))
    descent_rng = rng_for(seed, 2, accepted, int(equal_sibling))
    # choose a descent where the step after the root has a higher sibling when
    # the duplicate-sibling case is requested
    while True:
        d = random_descent(parent, descent_rng)
        path = d[: accepted + 1]
        if not equal_sibling:
            break
        kids0 = [i for i in range(1, 7) if parent[i] == path[0]]
        if len(path) > 1 and any(c > path[1] for c in kids0):
            break
    tok, tgt, dup = plant_walk(parent, path, rng_for(seed, 3, accepted, int(equal_sibling)), 1024,
                               equal_sibling=equal_sibling)
    s = _spec(seed, 1, 1, 4, 2, 64, 1024, 1.0, "f32", "f32", [64], [parent], [tok], [tgt], [path],
              note=f"accepted={accepted} equal_sibling={equal_sibling}")
    s.extra["dup"] = dup
    return s


def config2_round(T: int, accepted: int, seed: int = 2) -> RoundSpec:
    """Chain of T nodes (parent[i] = i-1) with the given accept length."""
    parent = chain_tree(T)
    path = list(range(accepted + 1))
    tok, tgt, _ = plant_walk(parent, path, rng_for(seed, 10, T, accepted), 248320)
    return _spec(seed, 1, 1, 40, 8, 128, 248320, 2.0, "bf16", "bf16", [2048], [parent], [tok], [tgt],
                 [path], note=f"chain T={T} accepted={accepted}")


def config3_round(seed: int = 3, P: int = 4096, L: int = 16, worst_case: bool = False,
                  stream: int = 0) -> RoundSpec:
    """16-node confidence-branching tree, depth <= 8, int8 KV, 16 layers."""
    parent, tokens = confidence_tree(rng_for(seed, 20, stream), 16, 8, 248320, 4)
    r = rng_for(seed, 21, stream)
    d = random_descent(parent, r, first_child_not=1 if worst_case else None)
    acc = len(d) - 1 if worst_case else int(r.integers(0, len(d)))
    path = d[: acc + 1]
    tok, tgt, _ = plant_walk(parent, path, rng_for(seed, 22, stream), 248320, tokens=tokens)
    return _spec(seed, 1, L, 40, 8, 128, 248320, 2.0, "i8", "bf16", [P], [parent], [tok], [tgt],
                 [path], note="confidence tree")


def config4_round(seed: int = 4, B: int = 32, pmin: int = 1024, pmax: int = 32768) -> RoundSpec:
    """Batched ragged round: per sequence a 3-ary depth-3 tree (40 nodes) or a
    random recursive tree of U{8..64} nodes (seeded coin), prefix U{pmin..pmax},
    accepted count uniform over 0..depth of a random leaf."""
    r = rng_for(seed, 30)
    parents, tokens, targets, paths, hist = [], [], [], [], []
    for b in range(B):
        if r.integers(0, 2) == 0:
            parent = sary_tree(3, 3)
        else:
            parent = random_tree(rng_for(seed, 31, b), int(r.integers(8, 65)))
        d = random_descent(parent, rng_for(seed, 32, b))
        acc = int(r.integers(0, len(d)))
        path = d[: acc + 1]
        tok, tgt, _ = plant_walk(parent, path, rng_for(seed, 33, b), 248320)
        parents.append(parent)
        tokens.append(tok)
        targets.append(tgt)
        paths.append(path)
        hist.append(int(r.integers(pmin, pmax + 1)))
    return _spec(seed, B, 1, 40, 8, 128, 248320, 2.0, "bf16", "bf16", hist, parents, tokens, targets,
                 paths, note="ragged batch")


def config5_schedule(n_rounds: int = 100, seed: int = 5) -> list:
    """Round types for the long-context stress run: 'tree' (confidence tree,
    worst-case scattered path: first step is not node 1), 'full' (chain-16,
    full accept: identity selection), 'partial' (chain-16, partial accept:
    prefix selection). Rounds 0, 1, 2 are one of each; the rest are drawn."""
    r = rng_for(seed, 40)
    kinds = ["tree", "full", "partial"]
    sched = kinds[:]
    while len(sched) < n_rounds:
        sched.append(kinds[int(r.integers(0, 3))])
    return sched[:n_rounds]


def config5_round(round_idx: int, hist_len, kind: str, seed: int = 5, B: int = 8, L: int = 8,
                  T: int = 16, Hq: int = 40, Hkv: int = 8, vocab: int = 248320) -> RoundSpec:
    parents, tokens, targets, paths = [], [], [], []
    for b in range(B):
        if kind == "tree":
            parent, tok0 = confidence_tree(rng_for(seed, 50, round_idx, b), T, 8, vocab, 4)
            d = random_descent(parent, rng_for(seed, 51, round_idx, b), first_child_not=1)
            path = d
            tok, tgt, _ = plant_walk(parent, path, rng_for(seed, 52, round_idx, b), vocab, tokens=tok0)
        else:
            parent = chain_tree(T)
            acc = T - 1 if kind == "full" else int(rng_for(seed, 53, round_idx, b).integers(0, T - 1))
            path = list(range(acc + 1))
            tok, tgt, _ = plant_walk(parent, path, rng_for(seed, 54, round_idx, b), vocab)
        parents.append(parent)
        tokens.append(tok)
        targets.append(tgt)
        paths.append(path)
    return _spec(seed, B, L, Hq, Hkv, 128, vocab, 2.0, "i8", "bf16", hist_len, parents, tokens,
                 targets, paths, note=f"round {round_idx} {kind}")


def host_tensors(spec: RoundSpec, cap: int | None = None, unique_scales: bool = False) -> dict:
    """NumPy bulk inputs for a round: per layer q [n_nodes, Hq, D] and a KV
    cache [B, Hkv, cap, D] (+ scales), and logits [n_nodes, vocab] with each
    row's maximum planted at the spec's target."""
    cap = spec.cap if cap is None else cap
    layers = []
    for l in range(spec.L):
        kv = make_kv_cache(spec.seed, 100 + l, spec.B, spec.Hkv, cap, spec.D, spec.kv_dtype,
                           unique_scales=unique_scales)
        kv["q"] = make_queries(spec.seed, 200 + l, spec.n_nodes, spec.Hq, spec.D, spec.q_dtype)
        layers.append(kv)
    logits = planted_logits(rng_for(spec.seed, 300), spec.flat_targets, spec.vocab, spec.sigma)
    return {"layers": layers, "logits": logits, "cap": cap}
