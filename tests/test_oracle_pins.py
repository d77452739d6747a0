"""Pins of the CPU oracle against things other than itself: the pages'
equivalences and worked examples, closed forms, brute force on tiny inputs,
and library routines (torch SDPA in float64, Python's max/index)."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import (binary_tree_7, chain_tree, config1_round, config2_round, config3_round,
                       confidence_tree, plant_walk, planted_logits, quantize_int8_per_token,
                       random_descent, random_tree, rng_for, sary_tree, to_bf16_bits,
                       unique_fp16_scales)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MASKED = np.float32(-1e9)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------

def closure_ancestors(parent):
    """Reflexive-transitive closure of the child->parent relation by repeated
    boolean matrix products (a different algorithm from chain walking)."""
    T = len(parent)
    A = np.zeros((T, T), dtype=bool)
    for i in range(1, T):
        A[i, parent[i]] = True
    R = np.eye(T, dtype=bool)
    while True:
        R2 = R | ((R.astype(np.int64) @ A.astype(np.int64)) > 0)
        if (R2 == R).all():
            return R
        R = R2


def causal_mask(T, offset):
    """Textbook causal mask with history: row q (position q + offset) sees
    columns c <= q + offset."""
    m = np.full((T, offset + T), MASKED, dtype=np.float32)
    for q in range(T):
        m[q, : q + offset + 1] = 0.0
    return m


def speculative_walk(drafts, target):
    """Chain acceptance: the longest prefix of the drafts where draft k (node
    k, k >= 1) equals the target's token at node k-1; emitted are the target's
    tokens at nodes 0..accepted."""
    a = 0
    while a + 1 < len(drafts) and drafts[a + 1] == target[a]:
        a += 1
    return a, [int(t) for t in target[: a + 1]]


def sdpa_reference(qf, K, V, P, open_mask, G, scale):
    """torch SDPA (float64) for one sequence: qf [T, Hq, D], K, V [Hkv, P+T, D],
    open_mask [T, T] boolean over block columns (history always open)."""
    T, Hq, D = qf.shape
    Hkv = K.shape[0]
    q = torch.from_numpy(qf).permute(1, 0, 2)[None]                      # [1, Hq, T, D]
    k = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]              # [1, Hq, S, D]
    v = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
    allow = torch.ones(T, P + T, dtype=torch.bool)
    allow[:, P:] = torch.from_numpy(open_mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=allow, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# Step 1: mask
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", range(0, 6))
def test_linear_tree_masks_as_causal_offset0(T):
    np.testing.assert_array_equal(O.additive_mask_with_history(chain_tree(T), 0), causal_mask(T, 0))


@pytest.mark.parametrize("T,offset", itertools.product(range(0, 6), [1, 3, 64]))
def test_linear_tree_history_mask_equals_causal(T, offset):
    np.testing.assert_array_equal(O.additive_mask_with_history(chain_tree(T), offset), causal_mask(T, offset))


def test_mask_golden_binary7():
    g = _golden("mask_binary7_p2.json")
    rows = g["rows_open_o_masked_x"]
    want = np.array([[0.0 if ch == "o" else MASKED for ch in rows[2 * i] + rows[2 * i + 1]]
                     for i in range(len(g["parent"]))], dtype=np.float32)
    np.testing.assert_array_equal(O.additive_mask_with_history(g["parent"], g["offset"]), want)
    np.testing.assert_array_equal(O.node_depths(g["parent"]), g["depth"])


def _trees():
    out = [chain_tree(1), chain_tree(64), sary_tree(3, 3), sary_tree(2, 5)]
    for s in range(6):
        out.append(binary_tree_7(rng_for(900, s)))
        out.append(random_tree(rng_for(901, s), int(rng_for(902, s).integers(2, 65))))
        out.append(confidence_tree(rng_for(903, s), 16, 8, 1000, 4)[0])
    return out


@pytest.mark.parametrize("idx", range(22))
def test_ancestors_brute_force(idx):
    parent = _trees()[idx]
    R = closure_ancestors(parent)
    sets = O.ancestor_sets(parent)
    for i in range(len(parent)):
        assert sets[i] == frozenset(np.nonzero(R[i])[0].tolist())
    bits = O.ancestor_bits(parent)
    for i in range(len(parent)):
        assert int(bits[i]) == sum(1 << int(j) for j in np.nonzero(R[i])[0])
    np.testing.assert_array_equal(O.node_depths(parent), R.sum(axis=1) - 1)


@pytest.mark.parametrize("idx", range(22))
def test_mask_invariants(idx):
    parent = _trees()[idx]
    T = len(parent)
    for P in (0, 5):
        m = O.additive_mask_with_history(parent, P)
        assert (m[:, :P] == 0).all()                         # history open to every node
        for i in range(T):
            assert m[i, P + i] == 0                          # self
            assert (m[i] == 0).any()                         # no fully masked row
        for i, j in itertools.combinations(range(1, T), 2):
            if parent[i] == parent[j]:                       # siblings never see each other
                assert m[i, P + j] == MASKED and m[j, P + i] == MASKED
        assert set(np.unique(m)) <= {0.0, MASKED}
        np.testing.assert_array_equal((m[:, P:] == 0).sum(axis=1), O.node_depths(parent) + 1)


def test_invalid_parent_rejected():
    for bad in ([0, 0], [-1, 1], [-1, 0, 2], [-1, -1]):
        with pytest.raises(ValueError):
            O.ancestor_sets(bad)


# ---------------------------------------------------------------------------
# Step 4: walk
# ---------------------------------------------------------------------------

def test_walk_golden_cases():
    for c in _golden("walk_cases.json")["cases"]:
        path, em = O.tree_accept_walk(c["parent"], c["token"], c["argmax"])
        assert path == c["path"], c["name"]
        assert em == c["emitted"], c["name"]


@pytest.mark.parametrize("T", range(1, 9))
def test_linear_tree_walks_as_speculative_walk(T):
    # every accept length, with planted tokens
    for acc in range(T):
        tok, tgt, _ = plant_walk(chain_tree(T), list(range(acc + 1)), rng_for(910, T, acc), 50)
        path, em = O.tree_accept_walk(chain_tree(T), tok, tgt)
        a, em2 = speculative_walk(list(tok), list(tgt))
        assert a == acc and len(path) - 1 == a and em == em2 and path == list(range(a + 1))
    # and on unplanted tokens over a 2-token vocabulary (many chance matches)
    r = rng_for(911, T)
    for _ in range(50):
        tok = r.integers(0, 2, size=T)
        tgt = r.integers(0, 2, size=T)
        path, em = O.tree_accept_walk(chain_tree(T), tok, tgt)
        a, em2 = speculative_walk(list(tok), list(tgt))
        assert len(path) - 1 == a and em == em2


def brute_force_walk(parent, token, target):
    """All root paths whose every step matches (token[child] == target[parent]);
    of the maximal ones, the lexicographically smallest label sequence."""
    T = len(parent)
    kids = [[c for c in range(1, T) if parent[c] == u] for u in range(T)]
    paths = []

    def dfs(p):
        ext = [c for c in kids[p[-1]] if token[c] == target[p[-1]]]
        if not ext:
            paths.append(p)
        for c in ext:
            dfs(p + [c])

    dfs([0])
    return min(paths)


@pytest.mark.parametrize("seed", range(40))
def test_walk_brute_force(seed):
    r = rng_for(920, seed)
    T = int(r.integers(1, 40))
    parent = random_tree(r, T)
    token = r.integers(0, 3, size=T)
    target = r.integers(0, 3, size=T)
    path, em = O.tree_accept_walk(parent, token, target)
    assert path == brute_force_walk(parent, token, target)
    for k in range(1, len(path)):
        assert parent[path[k]] == path[k - 1]
        assert token[path[k]] == target[path[k - 1]]
    assert em == [int(target[n]) for n in path] and len(em) == len(path)


def test_equal_token_siblings_single_path():
    for s in range(20):
        spec = config1_round(accepted=2, equal_sibling=True, seed=1000 + s)
        n, sib = spec.extra["dup"]
        path, _ = O.tree_accept_walk(spec.parents[0], spec.tokens[0], spec.targets[0])
        assert spec.tokens[0][n] == spec.tokens[0][sib] and n < sib
        assert n in path and sib not in path
        assert path == spec.paths[0]


@pytest.mark.parametrize("make", ["c1", "c2", "c3", "rand"])
def test_walk_follows_planted_path(make):
    for s in range(10):
        if make == "c1":
            spec = config1_round(seed=2000 + s)
        elif make == "c2":
            spec = config2_round(8, s % 8, seed=2000 + s)
        elif make == "c3":
            spec = config3_round(seed=2000 + s, P=8, L=1)
        else:
            parent = random_tree(rng_for(930, s), 30)
            path = random_descent(parent, rng_for(931, s))
            tok, tgt, _ = plant_walk(parent, path, rng_for(932, s), 5)
            assert O.tree_accept_walk(parent, tok, tgt)[0] == path
            continue
        assert O.tree_accept_walk(spec.parents[0], spec.tokens[0], spec.targets[0])[0] == spec.paths[0]


def test_pages_round_arithmetic():
    """emitted = accepted + 1 per round reproduces the pages' printed 2.4359
    emitted per verify from 56 accepted over 39 rounds."""
    g = _golden("round_stats_pages.json")
    assert round((g["accepted"] + g["rounds"]) / g["rounds"], 4) == g["emitted_per_verify"]
    assert g["zero"] + g["partial"] + g["full"] == g["rounds"]


# ---------------------------------------------------------------------------
# Step 3: argmax
# ---------------------------------------------------------------------------

def first_max_index(row):
    row = [float(x) for x in row]
    for i, x in enumerate(row):
        if x != x:
            return i
    return row.index(max(row))


def test_argmax_ties_zero_nan_against_python():
    r = rng_for(940)
    rows = []
    V = 1031
    for k in range(40):
        x = r.integers(-3, 4, size=V).astype(np.float32)      # many exact ties
        rows.append(x)
    z = np.zeros(V, np.float32); z[5] = -0.0; z[:] = -1; z[7] = -0.0; z[9] = 0.0; rows.append(z)
    z = np.full(V, -1, np.float32); z[11] = 0.0; z[3] = -0.0; rows.append(z)
    z = r.standard_normal(V).astype(np.float32); z[600] = np.nan; z[900] = np.nan; rows.append(z)
    z = r.standard_normal(V).astype(np.float32); z[V - 1] = 50; z[V - 2] = 50; rows.append(z)
    z = np.full(V, -np.inf, np.float32); rows.append(z)
    z = r.standard_normal(V).astype(np.float32); z[17] = np.inf; z[400] = np.inf; rows.append(z)
    X = np.stack(rows)
    got = O.vocab_argmax(X)
    assert got.dtype == np.int32
    for i, row in enumerate(X):
        assert got[i] == first_max_index(row), i


def test_argmax_planted_rows():
    tg = rng_for(941).integers(0, 248320, size=6)
    X = planted_logits(rng_for(942), tg, 248320, 2.0)
    np.testing.assert_array_equal(O.vocab_argmax(X), tg)
    # ties planted across the row, including the last element of the 248,320 tail
    X[0, [3, 70000, 248319]] = X[0].max()
    X[1, [248319, 248318]] = X[1].max() + 5
    got = O.vocab_argmax(X)
    assert got[0] == min(3, tg[0]) and got[1] == 248318
    for i in range(len(X)):
        assert got[i] == first_max_index(X[i])


# ---------------------------------------------------------------------------
# Step 2: attention
# ---------------------------------------------------------------------------

def _small_case(seed, kv_dtype, T=None, P=None, Hq=4, Hkv=2, D=16, tree="random"):
    r = rng_for(950, seed)
    T = int(r.integers(1, 12)) if T is None else T
    P = int(r.integers(0, 20)) if P is None else P
    parent = random_tree(r, T) if tree == "random" else chain_tree(T)
    from workloads import make_kv_cache, make_queries
    kv = make_kv_cache(951, seed, 1, Hkv, P + T, D, kv_dtype)
    q = make_queries(952, seed, T, Hq, D, "f32" if kv_dtype == "f32" else "bf16")
    return parent, kv, q, P, T


def _decode_with_torch(kv, q, kv_dtype):
    """Library decoding for the reference side: torch's bfloat16 / float16."""
    if kv_dtype == "bf16":
        K = torch.from_numpy(kv["k"][0].view(np.int16)).view(torch.bfloat16).double().numpy()
        V = torch.from_numpy(kv["v"][0].view(np.int16)).view(torch.bfloat16).double().numpy()
    elif kv_dtype == "i8":
        ks = torch.from_numpy(kv["k_scale"][0]).double()[..., None]
        vs = torch.from_numpy(kv["v_scale"][0]).double()[..., None]
        K = (torch.from_numpy(kv["k"][0]).double() * ks).numpy()
        V = (torch.from_numpy(kv["v"][0]).double() * vs).numpy()
    else:
        K, V = kv["k"][0].astype(np.float64), kv["v"][0].astype(np.float64)
    if q.dtype == np.uint16:
        qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    else:
        qf = q.astype(np.float64)
    return qf, K, V


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_attention_matches_sdpa_with_closure_mask(seed, kv_dtype):
    parent, kv, q, P, T = _small_case(seed, kv_dtype)
    scale = 1 / math.sqrt(16)
    node_off = np.array([0, T])
    got = O.tree_verify_attention(q, kv, node_off, [P], [parent], scale,
                                  "f32" if kv_dtype == "f32" else "bf16", kv_dtype)
    qf, K, V = _decode_with_torch(kv, q, kv_dtype)
    want = sdpa_reference(qf, K, V, P, closure_ancestors(parent), 2, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_attention_dense_form_agrees(seed):
    parent, kv, q, P, T = _small_case(seed, "bf16")
    scale = 0.25
    got = O.tree_verify_attention(q, kv, [0, T], [P], [parent], scale, "bf16", "bf16")
    qf = O.decode_bf16(q)
    dense = O.tree_verify_attention_dense(qf, O.decode_bf16(kv["k"][0]), O.decode_bf16(kv["v"][0]),
                                          O.additive_mask_with_history(parent, P), scale, 2)
    np.testing.assert_allclose(got, dense, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_attention_zero_query_is_mean_over_visible_set(seed):
    """q = 0 makes every visible key equally likely, so the output is the
    plain mean of V over exactly the visible rows; one-hot V rows expose the
    set itself."""
    r = rng_for(960, seed)
    T, P = int(r.integers(1, 10)), int(r.integers(0, 8))
    parent = random_tree(r, T)
    S = P + T
    D = S
    k = r.standard_normal((1, 1, S, D)).astype(np.float32)
    v = np.eye(S, D, dtype=np.float32)[None, None]
    q = np.zeros((T, 1, D), np.float32)
    got = O.tree_verify_attention(q, {"k": k, "v": v}, [0, T], [P], [parent], 0.3, "f32", "f32")
    R = closure_ancestors(parent)
    for i in range(T):
        want = np.zeros(D)
        vis = list(range(P)) + [P + j for j in range(T) if R[i, j]]
        want[vis] = 1.0 / len(vis)
        np.testing.assert_allclose(got[i, 0], want, atol=1e-15)


def test_attention_T1_is_single_query_decode():
    parent, kv, q, P, T = _small_case(3, "f32", T=1, P=13)
    got = O.tree_verify_attention(q, kv, [0, 1], [P], [parent], 0.2, "f32", "f32")
    qf, K, V = _decode_with_torch(kv, q, "f32")
    for h in range(4):
        g = h // 2
        qt = torch.from_numpy(qf[0, h])[None, None, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, torch.from_numpy(K[g, : P + 1])[None, None], torch.from_numpy(V[g, : P + 1])[None, None], scale=0.2)
        np.testing.assert_allclose(got[0, h], o[0, 0, 0].numpy(), atol=1e-13)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_linear_tree_attention_is_causal(kv_dtype):
    parent, kv, q, P, T = _small_case(7, kv_dtype, T=9, P=11, tree="chain")
    qd = "f32" if kv_dtype == "f32" else "bf16"
    tree = O.tree_verify_attention(q, kv, [0, T], [P], [parent], 0.25, qd, kv_dtype)
    causal = O.tree_verify_attention(q, kv, [0, T], [P], None, 0.25, qd, kv_dtype)
    np.testing.assert_array_equal(tree, causal)
    qf, K, V = _decode_with_torch(kv, q, kv_dtype)
    tril = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(tree, sdpa_reference(qf, K, V, P, tril, 2, 0.25), atol=1e-12)


def test_gqa_head_map():
    """Query head h reads KV head h // G: with q = 0 and V constant per KV
    head the output of head h is that head's constant."""
    Hq, Hkv, D, P, T = 6, 3, 4, 5, 3
    k = rng_for(970).standard_normal((1, Hkv, P + T, D)).astype(np.float32)
    v = np.zeros((1, Hkv, P + T, D), np.float32)
    for g in range(Hkv):
        v[0, g] = g + 1
    q = np.zeros((T, Hq, D), np.float32)
    got = O.tree_verify_attention(q, {"k": k, "v": v}, [0, T], [P], [chain_tree(T)], 1.0, "f32", "f32")
    for h in range(Hq):
        np.testing.assert_allclose(got[:, h], h // 2 + 1, atol=1e-15)


def test_int8_quantiser_and_dequant():
    x = rng_for(980).standard_normal((64, 128)).astype(np.float32)
    code, scale = quantize_int8_per_token(x)
    deq = O.decode_kv(code, "i8", scale)
    s = scale.astype(np.float64)[:, None]
    assert (np.abs(deq - x) <= s / 2 + 1e-12).all()
    assert (np.abs(code) <= 127).all() and (np.abs(code).max(axis=1) >= 126).all()
    # a single-valued token maps every element to the same code (pages, gather_positions commit)
    c, sc = quantize_int8_per_token(np.full((3, 128), 0.37, np.float32))
    assert (c == c[:, :1]).all() and (c == 127).all()
    # the zero token gives a zero scale and zero codes
    c, sc = quantize_int8_per_token(np.zeros((1, 8), np.float32))
    assert sc[0] == 0 and (c == 0).all()


def test_bf16_decode_and_rounding():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3e-30, 65504.0], np.float32)
    bits = to_bf16_bits(x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    np.testing.assert_array_equal(bits.view(np.int16), t.view(torch.int16).numpy())
    np.testing.assert_array_equal(O.decode_bf16(bits), t.double().numpy())


# ---------------------------------------------------------------------------
# Step 5: gather
# ---------------------------------------------------------------------------

def _cache(seed, dtype="i8", B=2, H=3, cap=40, D=8, unique=True):
    from workloads import make_kv_cache
    return make_kv_cache(990, seed, B, H, cap, D, dtype, unique_scales=unique)


def test_prefix_selection_equals_trim_to():
    c = _cache(0)
    for n in (0, 1, 17, 40):
        got = O.gather_layer(c, [np.arange(n)] * 2)
        for name in c:
            trimmed = c[name][:, :, :n]                  # trim_to(n): keep the first n rows
            np.testing.assert_array_equal(got[name][:, :, :n], trimmed)
            np.testing.assert_array_equal(got[name][:, :, n:], c[name][:, :, n:])


def test_identity_selection_is_noop():
    c = _cache(1)
    got = O.gather_layer(c, [np.arange(40), np.arange(40)])
    for name in c:
        np.testing.assert_array_equal(got[name], c[name])


def test_absolute_selection_equals_tail_form():
    """gather_within_tail(tail_len, kept) keeps [0, tail_start) and writes the
    kept block offsets to [tail_start, tail_start + len(kept)); the same
    selection in absolute positions must give the same cache."""
    c = _cache(2)
    tail_start, kept = 30, np.array([0, 2, 3, 7, 9])
    tail = {n: c[n].copy() for n in c}
    for n in c:
        tail[n][:, :, tail_start: tail_start + len(kept)] = c[n][:, :, tail_start + kept]
    absolute = np.concatenate([np.arange(tail_start), tail_start + kept])
    got = O.gather_layer(c, [absolute, absolute])
    for n in c:
        np.testing.assert_array_equal(got[n], tail[n])
    # the oracle's tail form (live 40, tail 10 -> tail_start 30) gives the same cache
    via_tail = O.gather_within_tail(c, [40, 40], [10, 10], [kept, kept])
    for n in c:
        np.testing.assert_array_equal(via_tail[n], tail[n])


def test_tail_gather_worked_example():
    """Worked by hand: rows 10..15 with live 6 and tail 4 (tail_start 2);
    kept offsets [1, 3] move rows 3 and 5 to rows 2 and 3, and rows 4, 5
    keep their old contents (the live length becomes 4)."""
    k = np.arange(10, 16, dtype=np.float32).reshape(1, 1, 6, 1)
    got = O.gather_within_tail({"k": k}, [6], [4], [[1, 3]])["k"].ravel().tolist()
    assert got == [10, 11, 13, 15, 14, 15]
    # an empty kept set and the identity prefix move nothing
    assert O.gather_within_tail({"k": k}, [6], [4], [[]])["k"].ravel().tolist() == list(range(10, 16))
    assert O.gather_within_tail({"k": k}, [6], [4], [[0, 1]])["k"].ravel().tolist() == list(range(10, 16))


@pytest.mark.parametrize("seed", range(4))
def test_tail_gather_equals_absolute_selection(seed):
    """Per-sequence tails of different lengths: the tail form equals the
    in-place absolute gather of [0, s) ++ (s + kept), scales included, and a
    prefix of the tail is the trim (nothing moves)."""
    r = rng_for(996, seed)
    c = _cache(10 + seed, B=3, cap=80)
    live = [80, 61, 9]
    tails = [16, 64 if seed % 2 else 5, 9]
    tails[1] = min(tails[1], live[1])
    kept, sels = [], []
    for b in range(3):
        k = np.sort(r.choice(tails[b], size=int(r.integers(0, tails[b] + 1)), replace=False))
        kept.append(k)
        s = live[b] - tails[b]
        sels.append(np.concatenate([np.arange(s), s + k]))
    got = O.gather_within_tail(c, live, tails, kept)
    want = O.gather_layer(c, sels)
    for n in c:
        np.testing.assert_array_equal(got[n], want[n])
    # scales travel with their rows: every moved row's scale is its source's
    for b in range(3):
        s = live[b] - tails[b]
        for j, kj in enumerate(kept[b]):
            assert np.array_equal(got["k_scale"][b, :, s + j], c["k_scale"][b, :, s + kj])
    prefix = [np.arange(int(r.integers(0, t + 1))) for t in tails]
    same = O.gather_within_tail(c, live, tails, prefix)
    for n in c:
        np.testing.assert_array_equal(same[n], c[n])


@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_linear_tree_path_selection_equals_trim(T):
    P = 20
    c = _cache(3, cap=P + T)
    for acc in range(T):
        tok, tgt, _ = plant_walk(chain_tree(T), list(range(acc + 1)), rng_for(991, T, acc), 9)
        path, _ = O.tree_accept_walk(chain_tree(T), tok, tgt)
        sel = O.rollback_selection(P, path)
        got = O.gather_layer(c, [sel, sel])
        n = acc + 1                                    # chain rollback keeps P + n rows
        trim = T - n
        live = P + T - trim
        for name in c:
            np.testing.assert_array_equal(got[name][:, :, :live], c[name][:, :, :live])


def test_scales_move_with_tokens():
    c = _cache(4, unique=True)
    sel = np.array([0, 1, 2, 5, 9, 10, 23, 39])
    got = O.gather_layer(c, [sel, sel[:5]])
    for b, s in enumerate([sel, sel[:5]]):
        for h in range(3):
            for j, src in enumerate(s):
                assert got["k_scale"][b, h, j] == c["k_scale"][b, h, src]
                assert (got["k"][b, h, j] == c["k"][b, h, src]).all()
                assert got["v_scale"][b, h, j] == c["v_scale"][b, h, src]
    # the scales are distinct per token, so leaving them behind is visible
    assert (got["k_scale"][0, :, 3:8] != c["k_scale"][0, :, 3:8]).all()
    assert len(np.unique(c["k_scale"][0, 0])) == 40


def test_take_matches_row_loop():
    c = _cache(5, dtype="bf16", unique=False)
    sel = np.array([1, 4, 5, 6, 30])
    got = O.gather_positions(c["k"][1], sel, axis=1)
    for h in range(3):
        for j, s in enumerate(sel):
            np.testing.assert_array_equal(got[h, j], c["k"][1, h, s])


def test_unique_scales_are_distinct():
    s = unique_fp16_scales(rng_for(1), (2, 3, 500))
    for row in s.reshape(-1, 500):
        assert len(np.unique(row.view(np.uint16))) == 500 and np.isfinite(row).all() and (row > 0).all()


# ---------------------------------------------------------------------------
# Round: a linear tree behaves as the chain round
# ---------------------------------------------------------------------------

def test_linear_tree_round_equals_chain_round():
    T, P, Hq, Hkv, D = 6, 12, 4, 2, 8
    script = [T - 1, 2, 0, T - 1, 4, 0, 1]            # full, partial, zero accepts
    kinds = set()
    c = _cache(6, dtype="i8", B=1, H=Hkv, cap=P + T, D=D)
    for r, acc in enumerate(script):
        tok, tgt, _ = plant_walk(chain_tree(T), list(range(acc + 1)), rng_for(995, r), 40)
        logits = planted_logits(rng_for(996, r), tgt, 40, 1.0)
        am = O.vocab_argmax(logits)
        path, emitted = O.tree_accept_walk(chain_tree(T), tok, am)
        a, em_chain = speculative_walk(list(tok), list(am))
        assert emitted == em_chain and len(path) - 1 == a == acc
        kinds.add("full" if a == T - 1 else "zero" if a == 0 else "partial")
        tree_cache = O.gather_layer(c, [O.rollback_selection(P, path)])
        n = a + 1
        live = P + T - (T - n)                         # kv.trim(block_size - n)
        for name in c:
            np.testing.assert_array_equal(tree_cache[name][:, :, :live], c[name][:, :, :live])
    assert kinds == {"full", "partial", "zero"}


# ---------------------------------------------------------------------------
# sampled selection (nucleus-filtered draw per node)
# ---------------------------------------------------------------------------

def test_sample_golden_worked():
    g = _golden("sample_worked.json")
    x = np.array([g["logits"]], np.float32)
    for c in g["cases"]:
        got = O.vocab_sample(x, [c["u"]], 0, c["temperature"], c["top_k"], c["top_p"])
        assert int(got[0]) == c["token"], c


def _nucleus_reference(x, T, k, p):
    """Kept tokens and their renormalised probabilities, via numpy's sort and
    cumsum (a library route, not the oracle's loop)."""
    order = np.argsort(-x.astype(np.float64), kind="stable")[:k]
    z = x[order].astype(np.float64) / T
    w = np.exp(z - z.max())
    C = np.cumsum(w) / w.sum()
    n = int(np.searchsorted(C, p, side="left")) + 1
    return order[:n], w[:n] / w[:n].sum()


@pytest.mark.parametrize("seed", range(4))
def test_sample_top1_and_tiny_top_p_are_argmax(seed):
    r = np.random.default_rng(700 + seed)
    X = r.integers(-4, 5, size=(40, 300)).astype(np.float32)  # many ties
    X[0, 7] = -0.0
    X[0, 3] = 0.0
    U = r.random(40).astype(np.float32)
    want = np.argmax(X, axis=1)
    assert (O.vocab_sample(X, U, 1, 1.0, 1, 0.95) == want).all()
    assert (O.vocab_sample(X, U, 1, 0.7, 20, 1e-9) == want).all()


@pytest.mark.parametrize("seed", range(4))
def test_sample_full_softmax_is_inverse_cdf(seed):
    """top-k = V and top-p = 1: the draw is the inverse CDF of softmax(x / T),
    i.e. numpy's searchsorted on the cumulative softmax (distinct logits)."""
    r = np.random.default_rng(710 + seed)
    V = 50
    X = (r.standard_normal((30, V)) * 2).astype(np.float32)
    U = r.random(30).astype(np.float32)
    T = 0.8
    got = O.vocab_sample(X, U, 1, T, V, 1.0)
    for n in range(30):
        order = np.argsort(-X[n].astype(np.float64), kind="stable")
        w = np.exp(X[n, order].astype(np.float64) / T - X[n, order[0]] / T)
        C = np.cumsum(w) / w.sum()
        i = int(np.searchsorted(C, float(U[n]), side="right"))
        assert got[n] == order[i], n


def test_sample_stratified_frequencies_match_nucleus():
    """Equally spaced uniforms hit every kept token in proportion to its
    renormalised nucleus probability, to within one draw."""
    r = np.random.default_rng(720)
    x = (r.standard_normal((1, 2000)) * 2).astype(np.float32)
    M = 20000
    U = ((np.arange(M) + 0.5) / M).astype(np.float32)
    X = np.repeat(x, M, axis=0)
    got = O.vocab_sample(X, U, 1, 1.0, 20, 0.95)
    kept, prob = _nucleus_reference(x[0], 1.0, 20, 0.95)
    counts = {int(t): int((got == t).sum()) for t in np.unique(got)}
    assert set(counts) <= set(int(t) for t in kept)
    for t, pr in zip(kept, prob):
        assert abs(counts.get(int(t), 0) - M * pr) <= 1.5, (int(t), counts.get(int(t), 0), M * pr)


def test_sample_chi_square_random_uniforms():
    """The pages' check for sampled exactness: a chi-square test of drawn
    tokens against the nucleus distribution (seeded uniforms)."""
    from scipy.stats import chisquare
    r = np.random.default_rng(730)
    x = (r.standard_normal((1, 5000)) * 2).astype(np.float32)
    M = 20000
    U = r.random(M).astype(np.float32)
    got = O.vocab_sample(np.repeat(x, M, axis=0), U, 1, 1.0, 20, 0.95)
    kept, prob = _nucleus_reference(x[0], 1.0, 20, 0.95)
    obs = np.array([(got == t).sum() for t in kept], np.float64)
    assert obs.sum() == M
    assert chisquare(obs, M * prob).pvalue > 1e-3


def test_sample_uniform_stride_and_monotone_in_u():
    r = np.random.default_rng(740)
    X = (r.standard_normal((6, 100)) * 2).astype(np.float32)
    U = r.random(12).astype(np.float32)
    s0 = O.vocab_sample(X, U, 0, 1.0, 20, 0.95)
    s2 = O.vocab_sample(X, U, 2, 1.0, 20, 0.95)
    for n in range(6):
        assert s0[n] == O.vocab_sample(X[n:n + 1], U[:1], 0, 1.0, 20, 0.95)[0]
        assert s2[n] == O.vocab_sample(X[n:n + 1], U[2 * n:2 * n + 1], 0, 1.0, 20, 0.95)[0]
    # a larger uniform never picks a higher-ranked (larger-logit) token
    row = X[:1]
    order = list(np.argsort(-row[0].astype(np.float64), kind="stable"))
    ranks = [order.index(int(O.vocab_sample(row, [u], 0, 1.0, 20, 0.95)[0])) for u in np.linspace(0, 0.999, 200)]
    assert ranks == sorted(ranks)


def test_sample_nonfinite_top_selects_it():
    X = np.zeros((3, 10), np.float32)
    X[0, 4] = np.nan
    X[0, 6] = np.nan
    X[1, 2] = np.inf
    X[2, 5] = -np.inf
    X[2, 1] = 3.0
    got = O.vocab_sample(X, [0.99, 0.99, 0.0], 1, 1.0, 5, 0.95)
    assert list(got) == [4, 2, 1]


def test_sampled_walk_commits_the_samples():
    """A round with sampled targets: every emitted token is the sample at its
    path node and the path is the one the walk takes for those targets."""
    r = rng_for(750)
    parent = random_tree(r, 30)
    X = (r.standard_normal((30, 64)) * 2).astype(np.float32)
    U = r.random(30).astype(np.float32)
    tgt = O.vocab_sample(X, U, 1, 1.0, 20, 0.95)
    token = np.array([0] + [int(tgt[parent[i]]) if r.random() < 0.5 else 63 for i in range(1, 30)])
    path, emitted = O.tree_accept_walk(parent, token, tgt)
    assert emitted == [int(tgt[n]) for n in path]
    for a, b in zip(path, path[1:]):
        assert parent[b] == a and token[b] == tgt[a]


# ---------------------------------------------------------------------------
# sliding window: caller mask intersected with the band
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_sliding_mask_properties(seed):
    """The three properties the pages state for sliding_mask_from_caller."""
    r = np.random.default_rng(800 + seed)
    T = int(r.integers(1, 20))
    parent = random_tree(r, T)
    offset = int(r.integers(0, 60))
    caller = O.additive_mask_with_history(parent, offset)
    # below the window the caller mask comes back untouched
    W_big = offset + T + int(r.integers(0, 5))
    assert np.array_equal(O.sliding_mask_from_caller(caller, offset, W_big), caller)
    # past the window an all-attend caller mask reduces to the band
    W = int(r.integers(1, offset + T)) if offset + T > 1 else 1
    allow = np.zeros_like(caller)
    band = O.sliding_mask_from_caller(allow, offset, W)
    for q in range(T):
        for c in range(offset + T):
            want = 0.0 if (offset + q - W < c <= offset + q) else MASKED
            assert band[q, c] == np.float32(want)
    # a mask that already carries the band is unchanged by intersecting again
    once = O.sliding_mask_from_caller(caller, offset, W)
    assert np.array_equal(O.sliding_mask_from_caller(once, offset, W), once)
    # every row keeps its own position
    for q in range(T):
        assert once[q, offset + q] == 0.0


@pytest.mark.parametrize("seed,window", [(0, 5), (1, 40), (2, 70), (3, 1), (4, 200)])
def test_sliding_attention_explicit_equals_dense_band(seed, window):
    """The explicit key-set form with a window equals the dense form under
    the intersected mask (two independent routes to the same set)."""
    r = np.random.default_rng(820 + seed)
    T, P, Hq, Hkv, D = 12, 64, 4, 2, 16
    parent = random_tree(r, T)
    K = r.standard_normal((1, Hkv, P + T, D)).astype(np.float32)
    V = r.standard_normal((1, Hkv, P + T, D)).astype(np.float32)
    q = r.standard_normal((T, Hq, D)).astype(np.float32)
    got = O.tree_verify_attention(q, {"k": K, "v": V}, [0, T], [P], [parent], 0.25, "f32", "f32", window=window)
    mask = O.sliding_mask_from_caller(O.additive_mask_with_history(parent, P), P, window)
    want = O.tree_verify_attention_dense(q.astype(np.float64), K[0].astype(np.float64), V[0].astype(np.float64),
                                         mask, 0.25, Hq // Hkv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    if window >= P + T:
        full = O.tree_verify_attention(q, {"k": K, "v": V}, [0, T], [P], [parent], 0.25, "f32", "f32")
        assert np.array_equal(got, full)


@pytest.mark.parametrize("seed", range(6))
def test_sliding_band_holds_window_keys(seed):
    """Count pin for the band edge: a window of W tokens holds W keys, the
    query's own included. Under an all-open caller past the window, row q (at
    position offset + q) keeps exactly min(W, offset + q + 1) columns, and
    they are the newest ones, counted back from its own position. The
    expected set is built by counting back, not from the band inequality, so
    a band one key too wide or too narrow fails here."""
    r = np.random.default_rng(840 + seed)
    T = int(r.integers(1, 20))
    offset = int(r.integers(0, 60))
    W = int(r.integers(1, offset + T + 1))
    if offset + T <= W:
        W = max(1, offset + T - 1)
        if offset + T <= W:
            pytest.skip("no row past the window")
    got = O.sliding_mask_from_caller(np.zeros((T, offset + T), np.float32), offset, W)
    for q in range(T):
        open_cols = [c for c in range(offset + T) if got[q, c] == 0.0]
        assert len(open_cols) == min(W, offset + q + 1), (q, W, offset)
        expect, pos = [], offset + q
        while len(expect) < W and pos >= 0:
            expect.append(pos)
            pos -= 1
        assert open_cols == sorted(expect)


@pytest.mark.parametrize("window", [1, 5, 20, 63])
def test_sliding_attention_ignores_the_key_just_past_the_window(window):
    """Windowed attention at the band edge: node i (cache row P + i) of a chain
    sees the W newest rows, down to P + i - W + 1. A key planted at
    P + i - W with a huge score for node i must not move node i's output; the
    same spike one row later (P + i - W + 1), and the planted key as seen by
    the earlier node i - 1, must move it (so the check is not vacuous)."""
    r = np.random.default_rng(860 + window)
    T, P, Hq, Hkv, D = 8, 64, 2, 1, 16
    parent = chain_tree(T)
    K = r.standard_normal((1, Hkv, P + T, D))
    V = r.standard_normal((1, Hkv, P + T, D))
    q = r.standard_normal((T, Hq, D))
    base = O.tree_verify_attention(q, {"k": K, "v": V}, [0, T], [P], [parent], 0.25, "f32", "f32", window=window)
    for i in range(T):
        edge = P + i - window
        if edge < 0:
            continue
        for key, moves in ((edge, False), (edge + 1, True)):
            Kp = K.copy()
            Kp[0, 0, key] = 40.0 * q[i, 0]            # score ~ 10 |q|^2: dominates node i's row if visible
            Vp = V.copy()
            Vp[0, 0, key] = 25.0
            got = O.tree_verify_attention(q, {"k": Kp, "v": Vp}, [0, T], [P], [parent], 0.25, "f32", "f32",
                                          window=window)
            delta = float(np.abs(got[i, 0] - base[i, 0]).max())
            if moves:
                assert delta > 1.0, (i, key, window, delta)
            else:
                assert delta == 0.0, (i, key, window, delta)
            if not moves and i > 0 and edge > P + (i - 1) - window:
                # the earlier node's window still holds the planted row
                assert float(np.abs(got[i - 1] - base[i - 1]).max()) > 0.0
