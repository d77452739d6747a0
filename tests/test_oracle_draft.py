"""Pins of the oracle's confidence-branching tree construction (expand by
top-k per frontier row, frontier = top-k of the new candidates by path score,
rerank over every depth) against a hand-worked example, the degenerate
linear tree, a closed form, and a brute force written over path
probabilities."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O
from workloads import draft_rows, rng_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLDEN, "draft_worked.json")) as f:
        return json.load(f)


def test_worked_example_by_hand():
    g = _worked()
    rows = [np.log(np.asarray(r, np.float64)).astype(np.float32) for r in g["depth_probs"]]
    st = O.draft_tree_new(g["root_token"])
    for d, r in enumerate(rows):
        O.draft_tree_expand(st, r, g["top_k"])
        assert st["frontier"] == g["frontiers"][d], f"frontier after depth {d + 1}"
    for case in g["cases"]:
        parent, token, score = O.draft_tree_select(st, case["n_nodes"])
        assert parent.tolist() == case["parent"]
        assert token.tolist() == case["token"]
        np.testing.assert_allclose(np.exp(score), case["prob"], rtol=1e-6)


def test_top1_is_the_linear_chain_of_argmaxes():
    # a drafter that does not branch yields its chain as a linear tree
    for seed in range(5):
        depths = 1 + seed
        rows = draft_rows(100 + seed, 1, depths, 1, 300)
        parent, token, score, _ = O.draft_tree(5, [r[0] for r in rows], 1, depths + 1)
        assert parent.tolist() == [-1] + list(range(depths))
        assert token[0] == 5
        assert token[1:].tolist() == [int(np.argmax(r[0, 0])) for r in rows]
        assert np.all(np.diff(score) <= 0)


def test_uniform_rows_closed_form():
    # every row uniform: each node's children are tokens 0..k-1, every score
    # is -depth * ln V, and equal scores keep creation order
    V, k, depths = 10, 3, 3
    st = O.draft_tree_new(0)
    for d in range(depths):
        O.draft_tree_expand(st, np.zeros((1 if d == 0 else k, V), np.float32), k)
    parent, token, score = O.draft_tree_select(st, 1 + k + k * k)
    assert token[1:].tolist() == [0, 1, 2] + [0, 1, 2] * 3
    assert parent.tolist() == [-1, 0, 0, 0, 1, 1, 1, 2, 2, 2, 3, 3, 3]
    np.testing.assert_allclose(score[1:4], -math.log(V), rtol=1e-14)
    np.testing.assert_allclose(score[4:], -2 * math.log(V), rtol=1e-14)


def brute_force_tree(root, depth_rows, k, n_nodes):
    """The same construction over path probabilities: products of scipy
    softmax probabilities, frontiers and the final set chosen by sorting on
    (-probability, creation index). Returns (parent, token, log prob)."""
    cands = []  # (prob, parent index or -1, token)
    frontier = [(-1, 1.0)]
    for rows in depth_rows:
        rows = np.asarray(rows, np.float32)
        made = []
        for f, (u, pu) in enumerate(frontier):
            p = softmax(rows[f].astype(np.float64))
            toks = sorted(range(len(p)), key=lambda t: (-float(rows[f][t]), t))[:k]
            for t in toks:
                cands.append((pu * p[t], u, t))
                made.append(len(cands) - 1)
        made.sort(key=lambda c: (-cands[c][0], c))
        frontier = [(c, cands[c][0]) for c in made[:k]]
    best = sorted(range(len(cands)), key=lambda c: (-cands[c][0], c))[: n_nodes - 1]
    lab = {c: i + 1 for i, c in enumerate(best)}
    parent = [-1] + [0 if cands[c][1] < 0 else lab[cands[c][1]] for c in best]
    token = [root] + [cands[c][2] for c in best]
    return parent, token, [0.0] + [math.log(cands[c][0]) for c in best]


@pytest.mark.parametrize("k,depths,n_nodes,V", [(2, 3, 6, 40), (3, 4, 12, 50), (4, 8, 16, 200), (5, 3, 20, 64),
                                                (8, 4, 64, 300)])
def test_matches_brute_force_over_probabilities(k, depths, n_nodes, V):
    for seed in range(4):
        rows = draft_rows(7 * seed + k, 1, depths, k, V)
        parent, token, score, _ = O.draft_tree(3, [r[0] for r in rows], k, n_nodes)
        bp, bt, bs = brute_force_tree(3, [r[0] for r in rows], k, n_nodes)
        assert parent.tolist() == bp and token.tolist() == bt
        np.testing.assert_allclose(score, bs, rtol=0, atol=1e-9)


@pytest.mark.parametrize("k,depths,n_nodes", [(4, 8, 16), (2, 6, 10), (6, 5, 64)])
def test_invariants(k, depths, n_nodes):
    V = 500
    for seed in range(3):
        rows = draft_rows(50 + seed, 1, depths, k, V)
        parent, token, score, st = O.draft_tree(11, [r[0] for r in rows], k, n_nodes)
        n = len(parent)
        assert n == n_nodes and parent[0] == -1
        assert all(0 <= parent[i] < i for i in range(1, n))  # topological, closed under parents
        assert all(score[i] <= score[parent[i]] for i in range(1, n))
        assert len({(int(parent[i]), int(token[i])) for i in range(1, n)}) == n - 1  # unique prefixes
        # every chosen candidate outranks every one left out
        left = sorted(st["score"], reverse=True)[n - 1:]
        if left:
            assert min(score[1:]) >= max(left)
        # siblings never repeat a token, so the walk has one way down
        for u in range(n):
            kids = [int(token[i]) for i in range(1, n) if parent[i] == u]
            assert len(kids) == len(set(kids))
        # the tree feeds the mask and the walk
        bits = O.ancestor_bits(parent)
        assert all(int(bits[i]) >> i & 1 for i in range(n))
        # targets follow each node's first-labelled child: the walk descends
        # those children to a leaf
        first = [next((int(token[i]) for i in range(1, n) if parent[i] == u), -1) for u in range(n)]
        path, emitted = O.tree_accept_walk(parent, token, np.asarray(first, np.int32))
        assert all(parent[path[j]] == path[j - 1] for j in range(1, len(path)))
        assert first[path[-1]] == -1 and len(path) == O.node_depths(parent)[path[-1]] + 1


def test_refusals():
    st = O.draft_tree_new(0)
    bad = np.zeros((1, 8), np.float32)
    bad[0, 3] = np.nan
    with pytest.raises(ValueError):
        O.draft_tree_expand(st, bad, 2)
    st = O.draft_tree_new(0)
    O.draft_tree_expand(st, np.zeros((1, 8), np.float32), 2)
    with pytest.raises(ValueError):
        O.draft_tree_select(st, 4)  # two candidates cannot make four nodes
    with pytest.raises(AssertionError):
        O.draft_tree_expand(st, np.zeros((1, 8), np.float32), 2)  # the frontier holds two nodes


def test_ties_within_a_row_go_to_the_lower_token():
    row = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]], np.float32)
    st = O.draft_tree_expand(O.draft_tree_new(9), row, 2)
    assert st["token"] == [1, 2] and st["frontier"] == [0, 1]
    assert st["score"][0] == st["score"][1]
