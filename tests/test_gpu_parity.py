"""GPU parity: every step of the HIP path against the CPU oracle on the same
seeded inputs. Integer/index/byte outputs must match bit for bit; attention
within max-abs 2e-3 (bf16 or int8 KV, fp32 accumulation) or 1e-5 (fp32)."""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from workloads import (binary_tree_7, chain_tree, config1_round, config2_round, config3_round, config4_round,
                       config5_round, config5_schedule, confidence_tree, host_tensors, make_kv_cache, make_queries, plant_walk, planted_logits,
                       random_descent, random_tree, rng_for, sary_tree)

from gpu_util import (layer_to_dev, layer_to_host, log, run_argmax, run_attention, run_mask, run_walk, spec_batch,
                      status, to_dev, to_host, zeros_ws)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
TOL_F32 = 1e-5


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def _batch_of(ttv, parents, hist):
    node_off = np.zeros(len(parents) + 1, np.int32)
    node_off[1:] = np.cumsum([len(p) for p in parents])
    return ttv.Batch(node_off, hist), node_off


def _trees(n=40):
    out = [chain_tree(1), chain_tree(2), chain_tree(64), sary_tree(3, 3), sary_tree(2, 5), np.zeros(0, np.int32)]
    for s in range(n):
        out.append(binary_tree_7(rng_for(1100, s)))
        out.append(random_tree(rng_for(1101, s), int(rng_for(1102, s).integers(1, 65))))
        out.append(confidence_tree(rng_for(1103, s), 16, 8, 1000, 4)[0])
    return out


# ---------------------------------------------------------------- mask ----

def test_mask_matches_oracle(ttv):
    trees = _trees()
    batch, off = _batch_of(ttv, trees, [0] * len(trees))
    log(f"mask: {len(trees)} trees, {off[-1]} nodes")
    par = to_dev(np.concatenate(trees).astype(np.int32))
    anc, depth, st = run_mask(ttv, batch, par)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got_a = to_host(anc).view(np.uint64)
    got_d = to_host(depth)
    for b, p in enumerate(trees):
        if len(p) == 0:
            continue
        np.testing.assert_array_equal(got_a[off[b]:off[b + 1]], O.ancestor_bits(p))
        np.testing.assert_array_equal(got_d[off[b]:off[b + 1]], O.node_depths(p))


def test_mask_invalid_parent_writes_nothing_for_that_tree(ttv):
    good = binary_tree_7(rng_for(1110))
    bad = np.array([-1, 0, 2, 1], np.int32)       # parent[2] = 2 is not an earlier node
    trees = [good, bad, chain_tree(5)]
    batch, off = _batch_of(ttv, trees, [3, 3, 3])
    anc, depth, st = run_mask(ttv, batch, to_dev(np.concatenate(trees)))
    torch.cuda.synchronize()
    assert int(st.item()) == ttv.TTV_DEV_BAD_PARENT
    a = to_host(anc)
    assert (a[off[1]:off[2]] == -1).all()
    np.testing.assert_array_equal(a.view(np.uint64)[off[2]:off[3]], O.ancestor_bits(chain_tree(5)))
    np.testing.assert_array_equal(a.view(np.uint64)[:off[1]], O.ancestor_bits(good))


def test_mask_expand_additive_matches_oracle(ttv):
    for s in range(6):
        parent = random_tree(rng_for(1120, s), int(rng_for(1121, s).integers(1, 65)))
        P = [0, 1, 7, 64, 200, 1000][s]
        batch, off = _batch_of(ttv, [chain_tree(3), parent], [5, P])
        anc, depth, st = run_mask(ttv, batch, to_dev(np.concatenate([chain_tree(3), parent])))
        out = torch.zeros(len(parent), P + len(parent), dtype=torch.float32, device="cuda")
        ttv.tree_mask_expand_additive(batch, 1, anc, -1e9, out)
        np.testing.assert_array_equal(to_host(out), O.additive_mask_with_history(parent, P))


# ---------------------------------------------------------------- walk ----

def _walk_cases():
    cases = []
    for acc in range(3):
        cases.append(config1_round(accepted=acc))
    cases.append(config1_round(accepted=2, equal_sibling=True))
    cases.append(config1_round(accepted=1, equal_sibling=True))
    for T in (3, 4, 8):
        for acc in range(T):
            cases.append(config2_round(T, acc))
    cases.append(config3_round(P=8, L=1))
    cases.append(config3_round(P=8, L=1, worst_case=True, stream=3))
    trees, toks, tgts, hist = [], [], [], []
    for c in cases:
        trees.append(c.parents[0])
        toks.append(c.tokens[0])
        tgts.append(c.targets[0])
        hist.append(int(c.hist_len[0]))
    spec4 = config4_round(B=32, pmin=1, pmax=300)
    trees += spec4.parents
    toks += spec4.tokens
    tgts += spec4.targets
    hist += [int(h) for h in spec4.hist_len]
    for s in range(30):   # unplanted tokens over a 3-token vocabulary: many equal-token siblings
        r = rng_for(1130, s)
        T = int(r.integers(1, 65))
        trees.append(random_tree(r, T))
        toks.append(r.integers(0, 3, size=T))
        tgts.append(r.integers(0, 3, size=T))
        hist.append(int(r.integers(0, 50)))
    return trees, toks, tgts, hist


def test_walk_matches_oracle(ttv):
    trees, toks, tgts, hist = _walk_cases()
    trees, toks, tgts, hist = trees[:128], toks[:128], tgts[:128], hist[:128]
    batch, off = _batch_of(ttv, trees, hist)
    log(f"walk: {len(trees)} trees")
    path, plen, em, sel, sel_len, st = run_walk(
        ttv, batch, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(np.concatenate(toks).astype(np.int32)),
        to_dev(np.concatenate(tgts).astype(np.int32)))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    path, plen, em, sel, sel_len = map(to_host, (path, plen, em, sel, sel_len))
    n_partial = n_zero = n_full = 0
    for b in range(len(trees)):
        want_path, want_em = O.tree_accept_walk(trees[b], toks[b], tgts[b])
        L = len(want_path)
        assert plen[b] == L, b
        assert list(path[b, :L]) == want_path, b
        assert list(em[b, :L]) == want_em, b
        assert (path[b, L:] == -3).all() and (em[b, L:] == -3).all()
        want_sel = O.rollback_selection(hist[b], want_path)
        assert sel_len[b] == len(want_sel)
        np.testing.assert_array_equal(sel[b, :len(want_sel)], want_sel)
        n_zero += L == 1
        n_partial += 1 < L < len(trees[b])
    assert n_zero > 0 and n_partial > 0


def test_walk_invalid_parent(ttv):
    trees = [chain_tree(4), np.array([0, 0, 1], np.int32)]   # second tree has no root
    batch, off = _batch_of(ttv, trees, [2, 2])
    flat = np.concatenate(trees)
    path, plen, em, sel, sel_len, st = run_walk(ttv, batch, to_dev(flat), to_dev(np.zeros(len(flat), np.int32)),
                                                 to_dev(np.zeros(len(flat), np.int32)))
    torch.cuda.synchronize()
    assert int(st.item()) == ttv.TTV_DEV_BAD_PARENT
    assert to_host(plen)[1] == -3 and to_host(plen)[0] == 4


# -------------------------------------------------------------- argmax ----

def _check_argmax(ttv, X, label):
    log(f"argmax: {label} {X.shape}")
    got = to_host(run_argmax(ttv, to_dev(X)))
    np.testing.assert_array_equal(got, O.vocab_argmax(X))


def test_argmax_config_shapes(ttv):
    c1 = config1_round()
    _check_argmax(ttv, host_tensors(c1)["logits"], "config 1")
    c2 = config2_round(8, 3)
    X = planted_logits(rng_for(1140), c2.flat_targets, 248320, 2.0)
    _check_argmax(ttv, X, "config 2")
    c3 = config3_round(P=8, L=1)
    _check_argmax(ttv, planted_logits(rng_for(1141), c3.flat_targets, 248320, 2.0), "config 3")


def test_argmax_ties_zero_nan_and_tails(ttv):
    V = 248320
    r = rng_for(1150)
    X = (r.standard_normal((24, V)).astype(np.float32) * 2)
    m = float(X.max()) + 3
    for i in range(8):              # ties across many candidate chunk boundaries and the tail
        pos = np.unique(np.concatenate([r.integers(0, V, 3), [V - 1, V - 2, 2047, 2048, 4095, 4096,
                                                             15519, 15520, 124159, 124160]]))
        X[i, pos[i % len(pos):]] = m
    X[8, :] = -np.inf
    X[9, :] = -np.inf; X[9, V - 1] = -1
    X[10, 100] = np.nan; X[10, 50000] = np.nan
    X[11, :] = 0.0; X[11, :1000] = -0.0; X[11, 0] = -0.0
    X[12, :] = -1.0; X[12, 70001] = -0.0; X[12, 70000] = 0.0; X[12, 9] = -0.0
    X[13, 200000] = np.inf; X[13, 7] = np.inf
    X[14, :] = 5.0
    X[15, ::2] = np.nan
    X[16] = -X[16]; X[16, V - 1] = m
    _check_argmax(ttv, X, "ties/zero/nan")
    # unaligned row stride forces the scalar path
    Y = np.ascontiguousarray(X[:, :V - 3])
    Yd = to_dev(np.ascontiguousarray(np.pad(Y, ((0, 0), (0, 1)), constant_values=np.nan)))  # never read
    out = torch.full((24,), -7, dtype=torch.int32, device="cuda")
    ttv.vocab_argmax(Yd, out, zeros_ws(ttv.vocab_argmax_ws(24, V - 3)), vocab=V - 3)
    np.testing.assert_array_equal(to_host(out), O.vocab_argmax(Y))


def test_argmax_many_rows_and_small_vocab(ttv):
    r = rng_for(1160)
    _check_argmax(ttv, r.integers(-2, 3, size=(1500, 257)).astype(np.float32), "1500 x 257 ints")
    _check_argmax(ttv, r.standard_normal((3, 5)).astype(np.float32), "3 x 5")
    X = r.standard_normal((1150, 248320)).astype(np.float32)
    _check_argmax(ttv, X, "config 4 rows")


# -------------------------------------------------------------- gather ----

def _gather_case(ttv, dtype, in_place, sels, B=3, L=2, H=2, D=64, cap=700, seed=0, unique=True):
    # distinct per-token scales prove that scales move with their tokens (fp16 has ~26k of them)
    host = [make_kv_cache(1170 + seed, l, B, H, cap, D, dtype, unique_scales=unique and dtype == "i8")
            for l in range(L)]
    devs, layers = zip(*[layer_to_dev(ttv, h) for h in host])
    live = np.array([cap - 3 * b for b in range(B)], np.int32)
    stride = cap + 5
    sel = np.full((B, stride), -1, np.int32)
    for b, s in enumerate(sels):
        sel[b, :len(s)] = s
    sel_len = np.array([len(s) for s in sels], np.int32)
    if in_place:
        dst_layers, dst_devs = None, devs
        base = host
    else:
        dst_host = [{n: np.zeros_like(a) for n, a in h.items()} for h in host]
        for h in dst_host:          # poison
            for n, a in h.items():
                a.view(np.uint8)[...] = 0xA5
        dst_devs, dst_layers = zip(*[layer_to_dev(ttv, h) for h in dst_host])
        base = dst_host
    st = status()
    ttv.kv_gather_positions(list(layers), None if in_place else list(dst_layers), to_dev(sel), to_dev(sel_len),
                            live, st, zeros_ws(ttv.kv_gather_positions_ws(B)))
    torch.cuda.synchronize()
    got = [layer_to_host(d) for d in dst_devs]
    return host, base, got, int(st.item()), live


def _selections(rng, live, kind):
    out = []
    for b, n in enumerate(live):
        if kind == "rollback":
            P = int(n) - 16
            path = [0] + sorted(rng.choice(np.arange(1, 16), size=int(rng.integers(0, 8)), replace=False).tolist())
            out.append(O.rollback_selection(P, path))
        elif kind == "prefix":
            out.append(np.arange(int(rng.integers(0, n + 1))))
        elif kind == "identity":
            out.append(np.arange(n))
        elif kind == "scatter":
            out.append(np.sort(rng.choice(n, size=n // 2, replace=False)))
        elif kind == "wide":  # long in-place span: moved rows exceed one chunk
            keep = np.ones(n, bool)
            keep[5:n:3] = False
            out.append(np.nonzero(keep)[0])
        elif kind == "empty":
            out.append(np.zeros(0, np.int64))
    return out


@pytest.mark.parametrize("dtype,D", [("i8", 64), ("i8", 128), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("in_place", [True, False])
@pytest.mark.parametrize("kind", ["rollback", "prefix", "identity", "scatter", "wide", "empty"])
def test_gather_matches_oracle(ttv, dtype, D, in_place, kind):
    rng = rng_for(1180, zlib.crc32(repr((dtype, D, in_place, kind)).encode()) % 1000)
    B, cap = 3, 700
    live = np.array([cap - 3 * b for b in range(B)])
    sels = _selections(rng, live, kind)
    log(f"gather: {dtype} D={D} in_place={in_place} {kind}")
    host, base, got, st, live = _gather_case(ttv, dtype, in_place, sels, B=B, D=D, cap=cap)
    assert st == 0
    for l in range(len(host)):
        kv = {n: a for n, a in host[l].items()}
        want = O.gather_layer(kv, sels, base=base[l])
        for n in want:
            np.testing.assert_array_equal(got[l][n], want[n], err_msg=f"layer {l} {n}")


@pytest.mark.parametrize("in_place", [True, False])
def test_gather_more_layers_than_one_launch(ttv, in_place):
    """37 layers: the copies run as launches of 16 layers each (16, 16, 5)
    after one validation, every layer gathered as the oracle's take."""
    rng = rng_for(1185, int(in_place))
    B, cap, L = 3, 300, 37
    live = np.array([cap - 3 * b for b in range(B)])
    sels = _selections(rng, live, "rollback")
    host, base, got, st, live = _gather_case(ttv, "i8", in_place, sels, B=B, L=L, D=64, cap=cap)
    assert st == 0
    for l in range(L):
        want = O.gather_layer(dict(host[l]), sels, base=base[l])
        for n in want:
            np.testing.assert_array_equal(got[l][n], want[n], err_msg=f"layer {l} {n}")


@pytest.mark.parametrize("in_place", [True, False])
def test_gather_bad_selection_writes_nothing(ttv, in_place):
    rng = rng_for(1190)
    live = np.array([700, 697, 694])
    sels = _selections(rng, live, "rollback")
    sels[1] = sels[1].copy()
    sels[1][-1], sels[1][-2] = sels[1][-2], sels[1][-1]      # not increasing
    host, base, got, st, _ = _gather_case(ttv, "i8", in_place, sels)
    assert st == ttv.TTV_DEV_BAD_SELECTION
    for l in range(len(host)):
        for n in host[l]:
            np.testing.assert_array_equal(got[l][n], base[l][n])
    sels = _selections(rng, live, "prefix")
    sels[2] = np.array([0, 5, 694])                            # out of range (live 694)
    host, base, got, st, _ = _gather_case(ttv, "bf16", in_place, sels, D=128)
    assert st == ttv.TTV_DEV_BAD_SELECTION
    for l in range(len(host)):
        for n in host[l]:
            np.testing.assert_array_equal(got[l][n], base[l][n])


@pytest.mark.parametrize("in_place", [True, False])
def test_gather_long_selection_many_chunks(ttv, in_place):
    """Selections of ~140k entries: the validation runs over many workgroups per
    sequence; a defect in a late chunk (or right at a chunk seam) still stops
    every write."""
    rng = rng_for(1195)
    B, cap = 2, 140000
    live = np.array([cap - 3 * b for b in range(B)])
    sels = [O.rollback_selection(int(live[0]) - 16, [0, 3, 9, 14]), np.sort(rng.choice(live[1], 90001, replace=False))]
    log(f"gather: long selections in_place={in_place}")
    host, base, got, st, _ = _gather_case(ttv, "i8", in_place, sels, B=B, L=1, H=1, D=64, cap=cap, seed=7,
                                             unique=False)
    assert st == 0
    want = O.gather_layer(dict(host[0]), sels, base=base[0])
    for n in want:
        np.testing.assert_array_equal(got[0][n], want[n], err_msg=n)
    for where in (4096, 2 * 2304, 57 * 2304, len(sels[0]) - 1):   # 2304 entries per chunk at this size
        bad = [sels[0].copy(), sels[1]]
        bad[0][where] = bad[0][where - 1]                       # repeated entry: not increasing
        host, base, got, st, _ = _gather_case(ttv, "i8", in_place, bad, B=B, L=1, H=1, D=64, cap=cap, seed=7,
                                                 unique=False)
        assert st == ttv.TTV_DEV_BAD_SELECTION, where
        for n in host[0]:
            np.testing.assert_array_equal(got[0][n], base[0][n], err_msg=f"{where} {n}")


# ----------------------------------------------------------- attention ----

def _attn_check(ttv, spec, tensors, tol, layers=None, anc_mode="tree", label=""):
    batch = spec_batch(ttv, spec)
    scale = 1.0 / math.sqrt(spec.D)
    par = to_dev(spec.flat("parents"))
    anc, _, st = run_mask(ttv, batch, par)
    worst = 0.0
    for li in (range(spec.L) if layers is None else layers):
        host = tensors["layers"][li]
        dev, kvl = layer_to_dev(ttv, host)
        q = to_dev(host["q"], "bf16" if spec.q_dtype == "bf16" else None)
        out, ws = run_attention(ttv, batch, q, kvl, None if anc_mode == "causal" else anc, scale)
        torch.cuda.synchronize()
        parents = None if anc_mode == "causal" else spec.parents
        want = O.tree_verify_attention(host["q"], {k: v for k, v in host.items() if k != "q"}, spec.node_off,
                                       spec.hist_len, parents, scale, spec.q_dtype, spec.kv_dtype)
        g = to_host(out)
        assert np.isfinite(g).all()
        err = float(np.abs(g - want).max()) if g.size else 0.0
        worst = max(worst, err)
        log(f"attention {label} layer {li}: max|err| {err:.3e}")
        assert err <= tol, (label, li, err)
    assert int(st.item()) == 0
    return worst


def test_attention_config1_fp32(ttv):
    for acc in range(3):
        spec = config1_round(accepted=acc)
        _attn_check(ttv, spec, host_tensors(spec), TOL_F32, label=f"config1 acc={acc}")


@pytest.mark.parametrize("T", [3, 4, 8])
def test_attention_config2_chain_equals_causal(ttv, T):
    spec = config2_round(T, T // 2)
    tensors = host_tensors(spec)
    _attn_check(ttv, spec, tensors, TOL_BF16, label=f"config2 T={T} tree")
    _attn_check(ttv, spec, tensors, TOL_BF16, anc_mode="causal", label=f"config2 T={T} causal")
    # the linear tree's bitsets and anc = NULL give bit-identical outputs
    batch = spec_batch(ttv, spec)
    host = tensors["layers"][0]
    dev, kvl = layer_to_dev(ttv, host)
    q = to_dev(host["q"], "bf16")
    anc, _, _ = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    o1, _ = run_attention(ttv, batch, q, kvl, anc, 1 / math.sqrt(128))
    o2, _ = run_attention(ttv, batch, q, kvl, None, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_attention_config3_int8_16_layers(ttv):
    spec = config3_round()
    _attn_check(ttv, spec, host_tensors(spec), TOL_BF16, label="config3")


GRID = [
    # (kv dtype, T, P, tree kind, Hq, Hkv)
    ("bf16", 1, 0, "chain", 40, 8), ("bf16", 1, 1, "chain", 40, 8), ("bf16", 2, 31, "random", 40, 8),
    ("bf16", 16, 32, "random", 40, 8), ("bf16", 33, 33, "random", 40, 8), ("bf16", 64, 100, "random", 40, 8),
    ("bf16", 64, 5000, "random", 40, 8), ("bf16", 40, 3000, "sary", 40, 8), ("bf16", 13, 777, "random", 16, 16),
    ("i8", 1, 0, "chain", 40, 8), ("i8", 3, 65, "random", 40, 8), ("i8", 16, 4095, "conf", 40, 8),
    ("i8", 64, 2000, "random", 40, 8), ("i8", 7, 9000, "random", 32, 4),
    ("f32", 7, 64, "binary", 4, 2), ("f32", 64, 300, "random", 8, 2), ("f32", 1, 0, "chain", 4, 2),
    # int8 splits with exactly two tiles: a ragged last split (one partial prefix
    # tile + one block tile) and two block tiles with no prefix at all
    ("i8", 5, 276, "random", 40, 8), ("i8", 40, 0, "random", 40, 8),
    # a wide bf16 unit whose keys split into 64 partials: the merge takes its
    # many-partials form over 48-row chunks
    ("bf16", 64, 16384, "random", 40, 8),
]


@pytest.mark.parametrize("case", range(len(GRID)))
def test_attention_grid(ttv, case):
    kv, T, P, kind, Hq, Hkv = GRID[case]
    r = rng_for(1200, case)
    parent = {"chain": chain_tree(T), "random": random_tree(r, T), "sary": sary_tree(3, 3)[:T],
              "conf": confidence_tree(r, T, 8, 1000, 4)[0], "binary": binary_tree_7(r)[:T]}[kind]
    D = 64 if kv == "f32" else 128
    qd = "f32" if kv == "f32" else "bf16"
    from workloads.configs import _spec
    spec = _spec(1200 + case, 1, 1, Hq, Hkv, D, 16, 1.0, kv, qd, [P], [parent], [np.zeros(T, np.int64)],
                 [np.zeros(T, np.int64)], [[0]])
    tensors = {"layers": [dict(make_kv_cache(1201, case, 1, Hkv, P + T + 3, D, kv),
                               q=make_queries(1202, case, T, Hq, D, qd))]}
    _attn_check(ttv, spec, tensors, TOL_F32 if kv == "f32" else TOL_BF16, label=f"grid {GRID[case]}")


@pytest.mark.parametrize("kv", ["i8", "bf16"])
def test_attention_peaked_scores(ttv, kv):
    """Scores far above a split's first tile: a few planted keys aligned with
    their query (scaled queries make every row sharper too). The kernels fix
    each row's reference from the first tile of a split and run the split again
    with raised references when a later score exceeds it by more than the fp16
    headroom; the result must still match the float64 oracle."""
    from workloads.configs import _spec
    from workloads.gen import bf16_bits_to_f32, quantize_int8_per_token, to_bf16_bits
    r = rng_for(1250, 0 if kv == "i8" else 1)
    T, P, Hq, Hkv, D = 16, 3000, 40, 8, 128
    parent = confidence_tree(r, T, 8, 1000, 4)[0]
    spec = _spec(1250, 1, 1, Hq, Hkv, D, 16, 1.0, kv, "bf16", [P], [parent], [np.zeros(T, np.int64)],
                 [np.zeros(T, np.int64)], [[0]])
    q = bf16_bits_to_f32(make_queries(1251, 0, T, Hq, D, "bf16")) * 3.0
    cache = make_kv_cache(1252, 0, 1, Hkv, P + T + 3, D, "f32")
    G = Hq // Hkv
    for key, node, h in ((1500, 0, 0), (2900, 3, 7), (700, 15, 39), (2047, 9, 12)):
        cache["k"][0, h // G, key] = 0.5 * q[node, h]            # score ~ 0.5 |q|^2 / sqrt(D): a spike
    if kv == "i8":
        layer = {}
        for n in ("k", "v"):
            code, scale = quantize_int8_per_token(cache[n])
            layer[n], layer[n + "_scale"] = code, scale
    else:
        layer = {n: to_bf16_bits(cache[n]) for n in ("k", "v")}
    layer["q"] = to_bf16_bits(q)
    log(f"attention peaked {kv}")
    _attn_check(ttv, spec, {"layers": [layer]}, TOL_BF16, label=f"peaked {kv}")


@pytest.mark.parametrize("kv", ["i8", "bf16"])
@pytest.mark.parametrize("qscale", [1e-6, 8.0, 30.0, 300.0])
def test_attention_query_magnitudes(ttv, kv, qscale):
    """Queries far from unit size: N(0, s^2) for s from 1e-6 (entries below
    fp16's normal range) to 300 (scores hundreds of log units apart, row sums
    of |q| past the offset code conversion's bound on the int8 path). The
    int8 path scales each row chunk's queries by a power of two into fp16
    range (a call this small converts every code exactly, in one launch; the
    offset form and its flagged second launch are checked at full size
    below); both KV dtypes must stay within the tolerance of the float64
    oracle."""
    from workloads.configs import _spec
    from workloads.gen import bf16_bits_to_f32, to_bf16_bits
    r = rng_for(1260, int(qscale * 1000) % 997, 0 if kv == "i8" else 1)
    T, P, Hq, Hkv, D = 16, 3000, 40, 8, 128
    parent = confidence_tree(r, T, 8, 1000, 4)[0]
    spec = _spec(1260, 1, 1, Hq, Hkv, D, 16, 1.0, kv, "bf16", [P], [parent], [np.zeros(T, np.int64)],
                 [np.zeros(T, np.int64)], [[0]])
    q = to_bf16_bits(bf16_bits_to_f32(make_queries(1261, 0, T, Hq, D, "bf16")) * np.float32(qscale))
    layer = dict(make_kv_cache(1262, 0, 1, Hkv, P + T + 3, D, kv), q=q)
    log(f"attention query scale {qscale} {kv}")
    _attn_check(ttv, spec, {"layers": [layer]}, TOL_BF16, label=f"qscale {qscale} {kv}")


@pytest.mark.parametrize("spread", [4, 8, 12])
def test_int8_spread_scales_error_relative_to_abs_values(ttv, spread):
    """int8 KV whose per-token k- and v-scales spread log-uniformly over a
    factor 2^spread within each head (outputs up to ~200 instead of ~3):
    P and P' = P * v_scale are rounded to fp16, so the error of an output
    row is bounded relative to the largest element of sum_j p_j |v_j|, the
    attention of |V| (the oracle run on the codes' absolute values), not
    absolutely."""
    from workloads.configs import _spec
    r = rng_for(1270, spread)
    B, Hq, Hkv, D = 6, 40, 8, 128
    parents = [confidence_tree(rng_for(1271, spread, b), 16, 8, 1000, 4)[0] for b in range(B)]
    hist = [int(r.integers(0, 1200)) for _ in range(B)]
    spec = _spec(1270, B, 1, Hq, Hkv, D, 16, 1.0, "i8", "bf16", hist, parents, [np.zeros(16, np.int64)] * B,
                 [np.zeros(16, np.int64)] * B, [[0]] * B)
    layer = make_kv_cache(1272, spread, B, Hkv, spec.cap, D, "i8")
    for n in ("k_scale", "v_scale"):
        f = np.exp2(r.uniform(-spread / 2, spread / 2, layer[n].shape))
        layer[n] = (layer[n].astype(np.float64) * f).astype(np.float16)
    layer["q"] = make_queries(1273, spread, spec.n_nodes, Hq, D, "bf16")
    batch = spec_batch(ttv, spec)
    anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    dev, kvl = layer_to_dev(ttv, layer)
    out, _ = run_attention(ttv, batch, to_dev(layer["q"], "bf16"), kvl, anc, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    kv = {k: v for k, v in layer.items() if k != "q"}
    want = O.tree_verify_attention(layer["q"], kv, spec.node_off, spec.hist_len, spec.parents, 1 / math.sqrt(D),
                                   "bf16", "i8")
    absv = dict(kv, v=np.abs(kv["v"].astype(np.int16)).astype(np.int8))
    cond = O.tree_verify_attention(layer["q"], absv, spec.node_off, spec.hist_len, spec.parents, 1 / math.sqrt(D),
                                   "bf16", "i8")
    g = to_host(out)
    assert np.isfinite(g).all() and int(st.item()) == 0
    # per output row: the largest element of the attention of |V| (an element
    # whose dominant keys hold code 0 is itself near zero, and the keys whose
    # fp16 P' underflows still leave an error of that row's scale)
    rel = float((np.abs(g - want) / np.maximum(cond.max(axis=2, keepdims=True), 1e-30)).max())
    log(f"int8 scales spread 2^{spread}: max|out| {np.abs(want).max():.3e}, max|err| {np.abs(g - want).max():.3e}, "
        f"max err / (attention of |V|) {rel:.3e}")
    assert rel <= TOL_BF16


@pytest.mark.parametrize("spread,T", [(6, 16), (10, 16), (10, 40)])
def test_bf16_spread_magnitudes_error_relative_to_abs_values(ttv, spread, T):
    """bf16 KV whose per-token key and value magnitudes spread log-uniformly
    over a factor 2^spread within each head: scores then span hundreds of
    log2 units (references raised by redo passes) and outputs reach ~100.
    As for int8 KV the error of an output row is bounded relative to the
    largest element of the attention of |V| (the oracle on |v|)."""
    from workloads.configs import _spec
    from workloads.gen import bf16_bits_to_f32, to_bf16_bits
    r = rng_for(1280, spread, T)
    B, Hq, Hkv, D = 6, 40, 8, 128
    parents = [confidence_tree(rng_for(1281, spread, T, b), T, 8, 1000, 4)[0] for b in range(B)]
    hist = [int(r.integers(0, 3000)) for _ in range(B)]
    spec = _spec(1280, B, 1, Hq, Hkv, D, 16, 1.0, "bf16", "bf16", hist, parents, [np.zeros(T, np.int64)] * B,
                 [np.zeros(T, np.int64)] * B, [[0]] * B)
    layer = make_kv_cache(1282, spread, B, Hkv, spec.cap, D, "bf16")
    for n in ("k", "v"):
        f = np.exp2(r.uniform(-spread / 2, spread / 2, layer[n].shape[:3]))[..., None]
        layer[n] = to_bf16_bits(bf16_bits_to_f32(layer[n]) * f.astype(np.float32))
    q = make_queries(1283, spread, spec.n_nodes, Hq, D, "bf16")
    batch = spec_batch(ttv, spec)
    anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    dev, kvl = layer_to_dev(ttv, layer)
    out, _ = run_attention(ttv, batch, to_dev(q, "bf16"), kvl, anc, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    want = O.tree_verify_attention(q, layer, spec.node_off, spec.hist_len, spec.parents, 1 / math.sqrt(D), "bf16",
                                   "bf16")
    absv = dict(layer, v=layer["v"] & np.uint16(0x7FFF))  # clear the bf16 sign bit
    cond = O.tree_verify_attention(q, absv, spec.node_off, spec.hist_len, spec.parents, 1 / math.sqrt(D), "bf16",
                                   "bf16")
    g = to_host(out)
    assert np.isfinite(g).all() and int(st.item()) == 0
    rel = float((np.abs(g - want) / np.maximum(cond.max(axis=2, keepdims=True), 1e-30)).max())
    log(f"bf16 magnitudes spread 2^{spread}, T={T}: max|out| {np.abs(want).max():.3e}, "
        f"max|err| {np.abs(g - want).max():.3e}, max err / (attention of |V|) {rel:.3e}")
    assert rel <= TOL_BF16


@pytest.mark.parametrize("kv,D,T", [("i8", 128, 16), ("bf16", 128, 16), ("bf16", 128, 40), ("i8", 64, 16),
                                    ("f32", 64, 16)])
def test_attention_ignores_cache_rows_past_live_length(ttv, kv, D, T):
    """Cache rows past each sequence's P_b + T_b are not part of the call:
    filled with NaN / infinity (scales, bf16 and fp32 values) or arbitrary
    codes, they must leave the output finite and equal to the oracle's, which
    never reads them. Boundary tiles load whole 8-key scale groups and clamp
    code rows, so those rows do reach the kernels' registers."""
    from workloads.configs import _spec
    r = rng_for(1290, D, {"i8": 0, "bf16": 1, "f32": 2}[kv])
    B, Hq, Hkv = 3, (40 if kv != "f32" else 4), (8 if kv != "f32" else 2)
    parents = [confidence_tree(rng_for(1291, b), T, 8, 1000, 4)[0] for b in range(B)]
    hist = [37, 130, 203]
    spec = _spec(1290, B, 1, Hq, Hkv, D, 16, 1.0, kv, "f32" if kv == "f32" else "bf16", hist, parents,
                 [np.zeros(T, np.int64)] * B, [np.zeros(T, np.int64)] * B, [[0]] * B)
    cap = spec.cap + 45
    layer = make_kv_cache(1292, D, B, Hkv, cap, D, kv)
    layer["q"] = make_queries(1293, D, spec.n_nodes, Hq, D, "f32" if kv == "f32" else "bf16")
    host = {k: v.copy() for k, v in layer.items()}
    for b in range(B):
        live = hist[b] + T
        for n in ("k", "v"):
            if kv == "i8":
                host[n][b, :, live:] = r.integers(-127, 128, host[n][b, :, live:].shape, dtype=np.int8)
                sc = host[n + "_scale"].view(np.uint16)
                sc[b, :, live:] = np.where(r.integers(0, 2, sc[b, :, live:].shape) == 0, 0x7C00, 0x7E00)
            elif kv == "bf16":
                host[n][b, :, live:] = 0x7FC0
            else:
                host[n][b, :, live:] = np.float32(np.nan)
    batch = spec_batch(ttv, spec)
    anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    dev, kvl = layer_to_dev(ttv, host)
    q = to_dev(host["q"], None if kv == "f32" else "bf16")
    out, _ = run_attention(ttv, batch, q, kvl, anc, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    want = O.tree_verify_attention(layer["q"], {k: v for k, v in layer.items() if k != "q"}, spec.node_off,
                                   spec.hist_len, spec.parents, 1 / math.sqrt(D), "f32" if kv == "f32" else "bf16",
                                   kv)
    g = to_host(out)
    assert np.isfinite(g).all(), f"{kv}: non-finite output from rows past the live length"
    err = float(np.abs(g - want).max())
    log(f"garbage past live length {kv} D={D} T={T}: max|err| {err:.3e}")
    assert err <= (TOL_F32 if kv == "f32" else TOL_BF16)


def _oracle_node_rows(slab: dict, kv: str, qrows, P: int, parent, t: int, scale: float):
    """The oracle's attention rows of one node and one KV head from that
    head's cache slab ({'k','v'[, scales]} [P + T, D] / [P + T]): the node's
    explicit key set, decoded keys and values, float64 softmax."""
    keys = O.visible_keys(P, O.ancestor_sets(parent)[t])
    K = O.decode_kv(slab["k"], kv, slab.get("k_scale"))
    V = O.decode_kv(slab["v"], kv, slab.get("v_scale"))
    return O.attention_rows(O.decode_bf16(qrows), K, V, keys, scale)


@pytest.mark.parametrize("T", [64, 40])
def test_wide_bf16_long_prefix_sampled(ttv, T):
    """One sequence of T nodes (T * 5 = 320 or 200 query rows per KV head, the
    wide bf16 layout) over a 131,072-token bf16 prefix: 64 key splits per
    unit, merged in the many-partials form. Sampled (node, KV head) rows of
    every row chunk are checked against the oracle."""
    from workloads.device import dev_kv_cache, dev_queries
    P, Hq, Hkv, D = 131072, 40, 8, 128
    parent = random_tree(rng_for(1270, T), T)
    node_off = np.array([0, T], np.int32)
    batch = ttv.Batch(node_off, np.array([P], np.int32))
    c = dev_kv_cache(1270, T, 1, Hkv, P + T, D, "bf16", "cuda")
    layer = ttv.KVLayer(c["k"], c["v"])
    q = dev_queries(1271, T, T, Hq, D, "bf16", "cuda")
    anc, _, st = run_mask(ttv, batch, to_dev(parent))
    out, _ = run_attention(ttv, batch, q, layer, anc, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    G = Hq // Hkv
    r = rng_for(1272, T)
    worst = 0.0
    # nodes spread over the tree, so every row chunk of the unit is sampled; random KV heads
    for t in sorted({0, T // 4, T // 2, (3 * T) // 4, T - 1, int(r.integers(0, T))}):
        g = int(r.integers(0, Hkv))
        slab = {n: to_host(c[n][0, g, :P + T]) for n in ("k", "v")}
        qrows = to_host(q[t, g * G:(g + 1) * G])
        want = _oracle_node_rows(slab, "bf16", qrows, P, parent, t, 1 / math.sqrt(D))
        got = to_host(out[t, g * G:(g + 1) * G])
        err = float(np.abs(got - want).max())
        log(f"wide long-prefix T={T}: node {t} kv head {g}: max|err| {err:.3e}")
        worst = max(worst, err)
    assert worst <= TOL_BF16
    assert np.isfinite(to_host(out)).all()


def test_attention_ragged_batch(ttv):
    spec = config4_round(B=12, pmin=0, pmax=2500)
    spec.parents[3] = np.zeros(0, np.int32)        # an empty tree in the middle of the batch
    spec.tokens[3] = np.zeros(0, np.int64)
    spec.targets[3] = np.zeros(0, np.int64)
    _attn_check(ttv, spec, host_tensors(spec), TOL_BF16, label="ragged B=12")
    _attn_check(ttv, spec, host_tensors(spec), TOL_BF16, anc_mode="causal", label="ragged causal")


def test_attention_workspace_reuse_across_shapes(ttv):
    """One workspace, poisoned first, serves calls of different shapes back to
    back: nothing in it is read before the call writes it."""
    big = config3_round(P=6000, L=1)
    small = config2_round(8, 2)
    tb, ts = host_tensors(big), host_tensors(small)
    ws = zeros_ws(64 << 20)
    ws.fill_(0xA5)
    for spec, tens in ((big, tb), (small, ts), (big, tb)):
        batch = spec_batch(ttv, spec)
        anc, _, _ = run_mask(ttv, batch, to_dev(spec.flat("parents")))
        host = tens["layers"][0]
        dev, kvl = layer_to_dev(ttv, host)
        out, _ = run_attention(ttv, batch, to_dev(host["q"], "bf16"), kvl, anc, 1 / math.sqrt(128), ws=ws)
        torch.cuda.synchronize()
        want = O.tree_verify_attention(host["q"], {k: v for k, v in host.items() if k != "q"}, spec.node_off,
                                       spec.hist_len, spec.parents, 1 / math.sqrt(128), "bf16", spec.kv_dtype)
        assert float(np.abs(to_host(out) - want).max()) <= TOL_BF16


# --------------------------------------------------------------- round ----

@pytest.mark.parametrize("acc,dup", [(0, False), (1, False), (2, False), (2, True)])
def test_round_config1_end_to_end(ttv, acc, dup):
    spec = config1_round(accepted=acc, equal_sibling=dup)
    tens = host_tensors(spec)
    want = O.verify_round(spec, tens)
    batch = spec_batch(ttv, spec)
    par = to_dev(spec.flat("parents"))
    anc, depth, st = run_mask(ttv, batch, par)
    host = tens["layers"][0]
    dev, kvl = layer_to_dev(ttv, host)
    out, _ = run_attention(ttv, batch, to_dev(host["q"]), kvl, anc, 1 / math.sqrt(spec.D))
    am = run_argmax(ttv, to_dev(tens["logits"]))
    path, plen, em, sel, sel_len, st2 = run_walk(ttv, batch, par, to_dev(spec.flat("tokens").astype(np.int32)), am)
    st3 = status()
    ttv.kv_gather_positions([kvl], None, sel, sel_len, spec.hist_len + np.diff(spec.node_off), st3,
                            zeros_ws(ttv.kv_gather_positions_ws(1)))
    torch.cuda.synchronize()
    assert int(st.item()) == int(st2.item()) == int(st3.item()) == 0
    np.testing.assert_array_equal(to_host(anc).view(np.uint64), want["anc"])
    assert float(np.abs(to_host(out) - want["attn"][0]).max()) <= TOL_F32
    np.testing.assert_array_equal(to_host(am), want["argmax"])
    L = int(to_host(plen)[0])
    assert list(to_host(path)[0, :L]) == want["paths"][0] == spec.paths[0]
    assert list(to_host(em)[0, :L]) == want["emitted"][0]
    got = layer_to_host(dev)
    for n in want["caches"][0]:
        np.testing.assert_array_equal(got[n], want["caches"][0][n])


# -------------------------------------------------------- long-context ----

def test_long_context_rounds_cache_tracks_oracle(ttv):
    """The long-context stress loop at reduced size (B=2, 2 layers, 10/2 heads,
    4096-token start, 16-node trees): every round appends the block's 16 rows,
    runs mask -> attention -> argmax -> walk -> in-place rollback on the GPU,
    and the paths, emitted tokens, attention and the whole cache (codes and
    scales) must equal the oracle's, round after round. The schedule mixes
    scattered tree paths, full accepts (identity selection) and partial
    accepts (prefix selection)."""
    from workloads.gen import quantize_int8_per_token
    B, L, T, Hq, Hkv, D, V = 2, 2, 16, 10, 2, 128, 4096
    rounds = 12
    sched = config5_schedule(rounds, seed=77)
    hist = np.array([4096, 4096 - 40], np.int64)
    cap = int(hist.max()) + T * rounds + 64
    mirror = [make_kv_cache(1300, l, B, Hkv, cap, D, "i8") for l in range(L)]
    devs, layers = zip(*[layer_to_dev(ttv, m) for m in mirror])
    scale = 1.0 / math.sqrt(D)
    for r, kind in enumerate(sched):
        spec = config5_round(r, hist.copy(), kind, seed=77, B=B, L=L, T=T, Hq=Hq, Hkv=Hkv, vocab=V)
        # the block's 16 rows are appended at P_b (both copies)
        for l in range(L):
            for b in range(B):
                P = int(hist[b])
                for n in ("k", "v"):
                    x = rng_for(1301, r, l, b, 0 if n == "k" else 1).standard_normal((Hkv, T, D), dtype=np.float32)
                    code, sc = quantize_int8_per_token(x)
                    mirror[l][n][b, :, P:P + T] = code
                    mirror[l][n + "_scale"][b, :, P:P + T] = sc
                    devs[l][n][b, :, P:P + T] = to_dev(code)
                    devs[l][n + "_scale"][b, :, P:P + T] = to_dev(sc)
        qs = [make_queries(1302, r * L + l, spec.n_nodes, Hq, D, "bf16") for l in range(L)]
        logits = planted_logits(rng_for(1303, r), spec.flat_targets, V, 2.0)
        want = O.verify_round(spec, {"layers": [dict(mirror[l], q=qs[l]) for l in range(L)], "logits": logits})
        # GPU round
        batch = spec_batch(ttv, spec)
        par = to_dev(spec.flat("parents"))
        anc, _, st = run_mask(ttv, batch, par)
        for l in range(L):
            out, _ = run_attention(ttv, batch, to_dev(qs[l], "bf16"), layers[l], anc, scale)
            err = float(np.abs(to_host(out) - want["attn"][l]).max())
            assert err <= TOL_BF16, (r, kind, l, err)
        am = run_argmax(ttv, to_dev(logits))
        path, plen, emitted, sel, sel_len, st2 = run_walk(ttv, batch, par, to_dev(spec.flat("tokens").astype(np.int32)), am)
        live = (spec.hist_len + np.diff(spec.node_off)).astype(np.int32)
        gst = status()
        ttv.kv_gather_positions(list(layers), None, sel, sel_len, live, gst, zeros_ws(ttv.kv_gather_positions_ws(B)))
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and int(st2.item()) == 0 and int(gst.item()) == 0
        pl = to_host(plen)
        for b in range(B):
            assert list(to_host(path)[b, :pl[b]]) == list(want["paths"][b]), (r, kind, b)
            assert list(to_host(emitted)[b, :pl[b]]) == list(want["emitted"][b]), (r, kind, b)
        assert list(to_host(sel_len)) == [len(x) for x in want["sels"]]
        for l in range(L):
            got = layer_to_host(devs[l])
            for n in got:
                np.testing.assert_array_equal(got[n], want["caches"][l][n], err_msg=f"round {r} {kind} layer {l} {n}")
            mirror[l] = want["caches"][l]
        log(f"long-context round {r} {kind}: paths {[len(x) - 1 for x in want['paths']]} ok")
        hist = np.array([len(x) for x in want["sels"]], np.int64)


def test_long_context_full_size_sampled(ttv):
    """The long-context workload at full size (B=8, 131,072-token prefix,
    16-node trees, int8 KV, 40/8 heads) in the bench's launch configuration:
    sampled output rows checked one by one against the oracle."""
    from workloads.device import dev_kv_cache, dev_queries
    spec = config5_round(0, [131072] * 8, "tree", L=1)
    cap = int(max(spec.hist_len + np.diff(spec.node_off)))
    c = dev_kv_cache(spec.seed, 100, spec.B, spec.Hkv, cap, spec.D, "i8", "cuda")
    layer = ttv.KVLayer(c["k"], c["v"], c["k_scale"], c["v_scale"])
    q = dev_queries(spec.seed, 200, spec.n_nodes, spec.Hq, spec.D, "bf16", "cuda")
    batch = spec_batch(ttv, spec)
    anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    out, _ = run_attention(ttv, batch, q, layer, anc, 1 / math.sqrt(spec.D))
    torch.cuda.synchronize()
    r = rng_for(1310)
    worst = 0.0
    for _ in range(6):
        b = int(r.integers(0, spec.B))
        t = int(r.integers(0, 16))
        g = int(r.integers(0, spec.Hkv))
        node = int(spec.node_off[b]) + t
        P = int(spec.hist_len[b])
        lay = {n: c[n][b:b + 1, g:g + 1, :P + 16].cpu().numpy() for n in ("k", "v", "k_scale", "v_scale")}
        qh = q[node:node + 1, g * spec.G:(g + 1) * spec.G].view(torch.int16).cpu().numpy().view(np.uint16)
        par = spec.parents[b]
        # the whole tree, one KV head: the oracle's row for (node t, each head of the group)
        qt = np.zeros((16, spec.G, spec.D), np.uint16)
        qt[t] = qh[0]
        want = O.tree_verify_attention(qt, lay, np.array([0, 16]), np.array([P]), [par], 1 / math.sqrt(spec.D),
                                       "bf16", "i8")[t]
        got = to_host(out[node, g * spec.G:(g + 1) * spec.G])
        worst = max(worst, float(np.abs(got - want).max()))
    log(f"full-size sampled rows: max|err| {worst:.3e}")
    assert worst <= TOL_BF16
    assert np.isfinite(to_host(out)).all()


def test_int8_offset_and_flagged_exact_launches(ttv):
    """An int8 call above the single-launch size (2 sequences x 8 KV heads x
    140,016 keys x 260 B = 582 MB) with unit-size queries on sequence 0 (the
    offset code conversion) and queries scaled by 300 on sequence 1 (row sums
    of |q| past the offset form's bound: those workgroups are flagged by the
    first launch and run exact in the second). Sampled rows of both sequences
    against the oracle."""
    from workloads.device import dev_kv_cache, dev_queries
    P, T, Hq, Hkv, D = 140000, 16, 40, 8, 128
    G = Hq // Hkv
    parents = [random_tree(rng_for(1320, b), T) for b in range(2)]
    node_off = np.array([0, T, 2 * T], np.int32)
    batch = ttv.Batch(node_off, np.array([P, P], np.int32))
    c = dev_kv_cache(1320, 0, 2, Hkv, P + T, D, "i8", "cuda")
    layer = ttv.KVLayer(c["k"], c["v"], c["k_scale"], c["v_scale"])
    q = dev_queries(1321, 0, 2 * T, Hq, D, "bf16", "cuda")
    q[T:] = (q[T:].float() * 300.0).to(torch.bfloat16)
    anc, _, st = run_mask(ttv, batch, to_dev(np.concatenate(parents)))
    scale = 1 / math.sqrt(D)
    out, _ = run_attention(ttv, batch, q, layer, anc, scale)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    r = rng_for(1322)
    worst = [0.0, 0.0]
    for b in (0, 1):
        for _ in range(2):
            g = int(r.integers(0, Hkv))
            slab = {n: to_host(c[n][b, g, :P + T]) for n in ("k", "v", "k_scale", "v_scale")}
            for t in sorted({int(r.integers(0, T)), T - 1}):
                node = b * T + t
                qrows = to_host(q[node, g * G:(g + 1) * G])
                want = _oracle_node_rows(slab, "i8", qrows, P, parents[b], t, scale)
                got = to_host(out[node, g * G:(g + 1) * G])
                worst[b] = max(worst[b], float(np.abs(got - want).max()))
    log(f"int8 two-launch: max|err| offset rows {worst[0]:.3e}, exact rows {worst[1]:.3e}")
    assert max(worst) <= TOL_BF16
    assert np.isfinite(to_host(out)).all()


def test_ragged_batch_full_size_sampled(ttv):
    """The batched ragged workload at full size (B=32, bf16, prefixes up to
    32,768, trees of 8-64 nodes, so up to 320 rows per KV head) in the bench's
    launch configuration: sampled output rows checked one by one against the
    oracle."""
    from workloads.device import dev_kv_cache, dev_queries
    spec = config4_round()
    T_b = np.diff(spec.node_off)
    cap = int(max(spec.hist_len + T_b))
    c = dev_kv_cache(spec.seed, 100, spec.B, spec.Hkv, cap, spec.D, "bf16", "cuda")
    layer = ttv.KVLayer(c["k"], c["v"])
    q = dev_queries(spec.seed, 200, spec.n_nodes, spec.Hq, spec.D, "bf16", "cuda")
    batch = spec_batch(ttv, spec)
    anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    out, _ = run_attention(ttv, batch, q, layer, anc, 1 / math.sqrt(spec.D))
    torch.cuda.synchronize()
    r = rng_for(1320)
    worst = 0.0
    big = [b for b in range(spec.B) if T_b[b] * spec.G > 96]  # sequences with more than one row chunk
    for i in range(8):
        b = int(big[int(r.integers(0, len(big)))]) if i % 2 == 0 else int(r.integers(0, spec.B))
        T = int(T_b[b])
        t = int(r.integers(0, T))
        g = int(r.integers(0, spec.Hkv))
        node = int(spec.node_off[b]) + t
        P = int(spec.hist_len[b])
        lay = {n: c[n][b:b + 1, g:g + 1, :P + T].view(torch.int16).cpu().numpy().view(np.uint16) for n in ("k", "v")}
        qh = q[node:node + 1, g * spec.G:(g + 1) * spec.G].view(torch.int16).cpu().numpy().view(np.uint16)
        qt = np.zeros((T, spec.G, spec.D), np.uint16)
        qt[t] = qh[0]
        want = O.tree_verify_attention(qt, lay, np.array([0, T]), np.array([P]), [spec.parents[b]],
                                       1 / math.sqrt(spec.D), "bf16", "bf16")[t]
        got = to_host(out[node, g * spec.G:(g + 1) * spec.G])
        worst = max(worst, float(np.abs(got - want).max()))
    log(f"ragged full-size sampled rows: max|err| {worst:.3e}")
    assert worst <= TOL_BF16
    assert np.isfinite(to_host(out)).all()
