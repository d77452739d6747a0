"""GPU parity of the confidence-branching draft tree (draft_tree_expand,
draft_tree_select) against the CPU oracle. Tokens, parents, frontiers and the
final trees must match bit for bit; scores (float64 path log-probabilities)
to 1e-9. The choices are decided by float64 score comparisons whose two
sides differ only in summation order (~1e-16 relative), so a random case
asserts its decisive gaps exceed 1e-9 before the comparison is trusted;
planted ties are exact on both sides (same row, or identical rows reduced in
the same fixed order)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import draft_rows, rng_for

from gpu_util import log, run_walk, status, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

V5 = 248320
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def gpu_expand(ttv, table, depth, rows, stride_pad=0, ws_fill=0xA5):
    """rows: float32 [B, F, V]; stride_pad > 0 places the rows at a padded
    (possibly unaligned) stride."""
    B, F, V = rows.shape
    if stride_pad:
        buf = np.full((B * F, V + stride_pad), 7.0, np.float32)
        buf[:, :V] = rows.reshape(B * F, V)
        Xd = to_dev(buf)
        Xd = Xd[:, :V]
    else:
        Xd = to_dev(np.ascontiguousarray(rows))
    st = status()
    ws = zeros_ws(ttv.draft_tree_expand_ws(B * F, V, table.top_k))
    ws.fill_(ws_fill)  # contents on entry are irrelevant
    ttv.draft_tree_expand(table, depth, Xd, st, ws)
    return int(to_host(st)[0])


def gpu_select(ttv, table, n_nodes, roots):
    B = table.B
    parent = torch.full((B * n_nodes,), -5, dtype=torch.int32, device="cuda")
    token = torch.full((B * n_nodes,), -5, dtype=torch.int32, device="cuda")
    score = torch.full((B * n_nodes,), 9.0, dtype=torch.float64, device="cuda")
    st = status()
    ttv.draft_tree_select(table, n_nodes, to_dev(np.asarray(roots, np.int32)), parent, token, st, score)
    return (to_host(parent).reshape(B, n_nodes), to_host(token).reshape(B, n_nodes),
            to_host(score).reshape(B, n_nodes), int(to_host(st)[0]))


def oracle_states(roots, depth_rows, k):
    states = []
    for b, r in enumerate(roots):
        st = O.draft_tree_new(int(r))
        for rows in depth_rows:
            O.draft_tree_expand(st, rows[b], k)
        states.append(st)
    return states


def decisive_gap(st, k, n_nodes):
    """Smallest score gap at any boundary a choice depends on: each depth's
    frontier cut and the final cut (inf where a cut takes everything)."""
    gaps = []
    sc = np.asarray(st["score"])
    d = np.asarray(st["depth"])
    for depth in range(1, int(d.max()) + 1):
        s = np.sort(sc[d == depth])[::-1]
        if len(s) > k:
            gaps.append(s[k - 1] - s[k])
    s = np.sort(sc)[::-1]
    if len(s) > n_nodes - 1 >= 1:
        gaps.append(s[n_nodes - 2] - s[n_nodes - 1])
    return min(gaps) if gaps else np.inf


def check_table(ttv, table, states):
    cnt = to_host(table.cand_count)
    tok = to_host(table.cand_token)
    par = to_host(table.cand_parent)
    sco = to_host(table.cand_score)
    fr = to_host(table.frontier)
    for b, st in enumerate(states):
        n = len(st["token"])
        assert cnt[b] == n, f"seq {b}: count {cnt[b]} != {n}"
        assert tok[b, :n].tolist() == st["token"], f"seq {b}: tokens"
        assert par[b, :n].tolist() == st["parent"], f"seq {b}: parents"
        np.testing.assert_allclose(sco[b, :n], st["score"], rtol=0, atol=1e-9)
        assert fr[b].tolist() == st["frontier"], f"seq {b}: frontier"


def test_worked_example(ttv):
    with open(os.path.join(GOLDEN, "draft_worked.json")) as f:
        g = json.load(f)
    k = g["top_k"]
    table = ttv.DraftTable(1, k, 64)
    for d, probs in enumerate(g["depth_probs"]):
        rows = np.log(np.asarray(probs, np.float64)).astype(np.float32)[None]
        assert gpu_expand(ttv, table, d + 1, rows) == 0
        assert to_host(table.frontier)[0].tolist() == g["frontiers"][d]
    for case in g["cases"]:
        parent, token, score, st = gpu_select(ttv, table, case["n_nodes"], [g["root_token"]])
        assert st == 0
        assert parent[0].tolist() == case["parent"] and token[0].tolist() == case["token"]
        np.testing.assert_allclose(np.exp(score[0]), case["prob"], rtol=1e-6)


CASES = [  # (B, top_k, depths, n_nodes, V, stride_pad)
    (1, 4, 8, 16, V5, 0),       # one 16-node tree over the full vocabulary
    (8, 4, 8, 16, V5, 0),       # a batch of 16-node trees
    (3, 1, 5, 6, 5000, 0),      # no branching: the chain of argmaxes
    (2, 16, 3, 64, 70000, 0),   # widest frontier, largest tree
    (4, 8, 4, 64, 4097 + 13, 0),  # a ragged last chunk
    (2, 4, 3, 16, 2048 + 5, 0),   # one full 2,048-logit chunk and a 5-logit tail
    (3, 4, 4, 16, 3 * 2048, 0),   # whole chunks only
    (2, 2, 6, 12, 100, 0),      # a vocabulary smaller than one chunk
    (3, 4, 3, 16, 9001, 3),     # unaligned row stride
    (5, 3, 2, 13, 12288, 0),    # every candidate chosen (1 + 3 + 9)
    (128, 16, 2, 64, 1000, 0),  # the largest batch with the widest frontier (1024-thread merge)
    (3, 3, 3, 13, 3, 0),        # vocabulary == top_k: every token is a child
]


@pytest.mark.parametrize("B,k,depths,n_nodes,V,pad", CASES)
def test_parity_random(ttv, B, k, depths, n_nodes, V, pad):
    seed = 1000 + 97 * B + 13 * k + depths + V % 1000
    log(f"draft parity B={B} k={k} depths={depths} n={n_nodes} V={V} pad={pad} seed={seed}")
    rows = draft_rows(seed, B, depths, k, V)
    roots = rng_for(seed, 1).integers(0, V, size=B)
    states = oracle_states(roots, rows, k)
    for st in states:
        assert decisive_gap(st, k, n_nodes) > 1e-9, "a near-tie would make the comparison ambiguous"
    cap = k + (depths - 1) * k * k
    table = ttv.DraftTable(B, k, cap)
    for d, r in enumerate(rows):
        assert gpu_expand(ttv, table, d + 1, r, stride_pad=pad) == 0
    check_table(ttv, table, states)
    parent, token, score, st = gpu_select(ttv, table, n_nodes, roots)
    assert st == 0
    for b in range(B):
        wp, wt, ws = O.draft_tree_select(states[b], n_nodes)
        assert parent[b].tolist() == wp.tolist(), f"seq {b}: parents"
        assert token[b].tolist() == wt.tolist(), f"seq {b}: tokens"
        np.testing.assert_allclose(score[b], ws, rtol=0, atol=1e-9)


def test_restart_and_reuse(ttv):
    # a depth-1 call starts a table afresh; the same table serves a second tree
    B, k, V = 2, 4, 30000
    table = ttv.DraftTable(B, k, 64)
    for seed in (11, 12):
        rows = draft_rows(seed, B, 3, k, V)
        roots = [5, 6]
        for d, r in enumerate(rows):
            assert gpu_expand(ttv, table, d + 1, r) == 0
        check_table(ttv, table, oracle_states(roots, rows, k))


def test_ties_exact(ttv):
    # uniform rows: equal logits within a row and identical rows across the
    # frontier give exactly equal scores on both sides; ties go to the lower
    # token and then to the earlier candidate
    B, k, V = 2, 3, 10000
    rows = [np.zeros((B, 1 if d == 0 else k, V), np.float32) for d in range(3)]
    table = ttv.DraftTable(B, k, 64)
    for d, r in enumerate(rows):
        assert gpu_expand(ttv, table, d + 1, r) == 0
    check_table(ttv, table, oracle_states([1, 2], rows, k))
    parent, token, score, st = gpu_select(ttv, table, 13, [1, 2])
    assert st == 0
    for b in range(B):
        assert token[b, 1:].tolist() == [0, 1, 2] * 4
        assert parent[b].tolist() == [-1, 0, 0, 0, 1, 1, 1, 2, 2, 2, 3, 3, 3]


def test_ties_across_chunks(ttv):
    # the row maximum appears in three chunks (and at the tail): the lowest
    # index wins; a second value tied across chunk boundaries likewise
    V = 3 * 4096 + 77
    r = rng_for(5, 2).standard_normal((1, 1, V)).astype(np.float32)
    for i in (8191, 4096, V - 1):
        r[0, 0, i] = 9.0
    for i in (12287, 4095, 100, 2047, 2048):
        r[0, 0, i] = 8.5
    table = ttv.DraftTable(1, 4, 16)
    assert gpu_expand(ttv, table, 1, r) == 0
    st = oracle_states([0], [r], 4)
    check_table(ttv, table, st)
    assert to_host(table.cand_token)[0, :4].tolist() == [4096, 8191, V - 1, 100]


def test_bad_logits_leave_the_table(ttv):
    B, k, V = 3, 2, 5000
    rows = draft_rows(21, B, 2, k, V)
    roots = [0, 1, 2]
    table = ttv.DraftTable(B, k, 32)
    assert gpu_expand(ttv, table, 1, rows[0]) == 0
    states = oracle_states(roots, rows[:1], k)
    bad = rows[1].copy()
    bad[1, 1, 4321] = np.nan
    bad[2, 0, 7] = np.inf
    assert gpu_expand(ttv, table, 2, bad) == ttv.TTV_DEV_BAD_LOGITS
    O.draft_tree_expand(states[0], bad[0], k)  # sequence 0 proceeds
    check_table(ttv, table, states)


def test_capacity_and_state_refusals(ttv):
    B, k, V = 2, 4, 3000
    rows = draft_rows(31, B, 3, k, V)
    table = ttv.DraftTable(B, k, 20)  # 4 + 16 fit, a third depth does not
    assert gpu_expand(ttv, table, 1, rows[0]) == 0
    assert gpu_expand(ttv, table, 2, rows[1]) == 0
    states = oracle_states([3, 4], rows[:2], k)
    assert gpu_expand(ttv, table, 3, rows[2]) == ttv.TTV_DEV_DRAFT_STATE
    check_table(ttv, table, states)
    # more nodes than candidates: nothing written
    parent, token, score, st = gpu_select(ttv, table, 22, [3, 4])
    assert st == ttv.TTV_DEV_DRAFT_STATE and (parent == -5).all() and (token == -5).all()
    # a deeper call on a table that was never started
    fresh = ttv.DraftTable(B, k, 64)
    assert gpu_expand(ttv, fresh, 2, rows[1]) == ttv.TTV_DEV_DRAFT_STATE
    assert (to_host(fresh.cand_count) == 0).all()


def test_tree_feeds_mask_and_walk(ttv):
    # the selected trees go straight into steps 1 and 4 on the device
    B, k, depths, n = 4, 4, 8, 16
    V = 50000
    rows = draft_rows(41, B, depths, k, V)
    roots = [9, 8, 7, 6]
    table = ttv.DraftTable(B, k, k + (depths - 1) * k * k)
    for d, r in enumerate(rows):
        assert gpu_expand(ttv, table, d + 1, r) == 0
    parent_d = torch.empty(B * n, dtype=torch.int32, device="cuda")
    token_d = torch.empty(B * n, dtype=torch.int32, device="cuda")
    st = status()
    ttv.draft_tree_select(table, n, to_dev(np.asarray(roots, np.int32)), parent_d, token_d, st)
    batch = ttv.Batch(np.arange(B + 1) * n, np.full(B, 100))
    anc = torch.empty(B * n, dtype=torch.int64, device="cuda")
    depth = torch.empty(B * n, dtype=torch.int32, device="cuda")
    ttv.tree_build_mask(batch, parent_d, anc, depth, st)
    # targets follow each node's first-labelled child
    states = oracle_states(roots, rows, k)
    targets = []
    for b in range(B):
        wp, wt, _ = O.draft_tree_select(states[b], n)
        targets += [next((int(wt[i]) for i in range(1, n) if wp[i] == u), -1) for u in range(n)]
        assert (to_host(anc)[b * n:(b + 1) * n].view(np.uint64) == O.ancestor_bits(wp)).all()
    path, plen, emitted, _, _, wst = run_walk(ttv, batch, parent_d, token_d,
                                              to_dev(np.asarray(targets, np.int32)))
    assert int(to_host(st)[0]) == 0 and int(to_host(wst)[0]) == 0
    for b in range(B):
        wp, wt, _ = O.draft_tree_select(states[b], n)
        want, _ = O.tree_accept_walk(wp, wt, np.asarray(targets[b * n:(b + 1) * n], np.int32))
        assert to_host(path)[b, :len(want)].tolist() == list(want)


def test_wide_logit_ranges(ttv):
    # rows whose terms exp(x - max) underflow to subnormals and to zero, and a
    # row dominated by one huge logit: the float64 normalisers must still
    # agree with the oracle's
    B, k, V = 2, 4, 9000
    rows = draft_rows(61, B, 2, k, V)
    r0 = rows[0].copy()
    r0[0, 0, :100] = -720.0     # subnormal terms
    r0[0, 0, 100:200] = -1e4    # zero terms
    r0[1, 0, 5] = 600.0         # everything else ~e^-600
    r1 = rows[1].copy()
    r1[:, :, 7::3] -= 730.0
    table = ttv.DraftTable(B, k, 64)
    assert gpu_expand(ttv, table, 1, r0) == 0
    assert gpu_expand(ttv, table, 2, r1) == 0
    check_table(ttv, table, oracle_states([0, 1], [r0, r1], k))
