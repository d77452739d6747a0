"""A seeded sweep of ragged attention calls against the float64 oracle: every
case draws its own batch (1-5 sequences; trees of 0-64 nodes, random, chain
or 3-ary; histories of 0-4,000 keys, some empty), head layout, KV dtype
(bf16 / int8 with D = 128, f32 with D = 64), mask form (tree bitsets or
causal) and, for some, a sliding window drawn around the histories' lengths.
Together the cases reach the planner's paths: the narrow and wide bf16
layouts with their dispatch order, the int8 kernel, the vector kernel,
windows on the matrix cores (with edge tiles) and off them, one split or
many, empty trees and empty histories in one batch. A second sweep draws
larger batches (1-8 sequences, more 64-node trees), longer histories (up to
12,000 keys for a quarter of the cases) and, for a third of the cases, fills
every cache row past a sequence's live length with NaN or infinity. The whole
output of every call is compared."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from workloads import chain_tree, make_kv_cache, make_queries, random_tree, rng_for, sary_tree

from gpu_util import layer_to_dev, log, run_mask, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "i8": 2e-3, "f32": 1e-5}
N_CASES = 64
N_WIDE = 96


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def _case(i):
    r = rng_for(1700, i)
    kv = ["bf16", "bf16", "i8", "i8", "f32"][int(r.integers(0, 5))]
    D = 64 if kv == "f32" else 128
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 3, 5, 8]))
    B = int(r.integers(1, 6))
    parents, hist = [], []
    for b in range(B):
        kind = int(r.integers(0, 6))
        if kind == 0:
            T = 0
        elif kind == 1:
            T = int(r.integers(1, 5))
        else:
            T = int(r.integers(5, 65))
        tree = int(r.integers(0, 3))
        if T == 0:
            p = np.zeros(0, np.int32)
        elif tree == 0:
            p = chain_tree(T)
        elif tree == 1 and T <= 40:
            p = sary_tree(3, 3)[:T]
        else:
            p = random_tree(rng_for(1701, i, b), T)
        parents.append(np.asarray(p, np.int32))
        hist.append(0 if int(r.integers(0, 6)) == 0 else int(r.integers(1, 4001)))
    if sum(len(p) for p in parents) == 0:
        parents[0] = chain_tree(3)
    window = 0
    if int(r.integers(0, 5)) < 2:
        # around a drawn sequence's history: inside, at, or past it
        ref = hist[int(r.integers(0, B))] + 1
        window = int(max(1, r.choice([ref // 4, ref // 2, ref - 30, ref + 40, 63, 64, 97, 128, 1024])))
    causal = int(r.integers(0, 4)) == 0
    return kv, D, Hkv, G, parents, hist, window, causal


def _wide_case(i):
    r = rng_for(2700, i)
    kv = ["bf16", "bf16", "i8", "i8", "f32"][int(r.integers(0, 5))]
    D = 64 if kv == "f32" else 128
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 5, 8]))
    B = int(r.integers(1, 9))
    big = int(r.integers(0, 4)) == 0
    parents, hist = [], []
    for b in range(B):
        kind = int(r.integers(0, 7))
        T = 0 if kind == 0 else int(r.integers(1, 5)) if kind == 1 else 64 if kind == 2 else int(r.integers(5, 65))
        tree = int(r.integers(0, 3))
        if T == 0:
            p = np.zeros(0, np.int32)
        elif tree == 0:
            p = chain_tree(T)
        elif tree == 1 and T <= 40:
            p = sary_tree(3, 3)[:T]
        else:
            p = random_tree(rng_for(2701, i, b), T)
        parents.append(np.asarray(p, np.int32))
        hist.append(0 if int(r.integers(0, 6)) == 0 else int(r.integers(1, 12001 if big else 3001)))
    if sum(len(p) for p in parents) == 0:
        parents[0] = chain_tree(3)
    window = 0
    if int(r.integers(0, 5)) < 2:
        ref = hist[int(r.integers(0, B))] + 1
        window = int(max(1, r.choice([ref // 4, ref // 2, ref - 30, ref + 40, 63, 64, 97, 128, 1024])))
    causal = int(r.integers(0, 4)) == 0
    garbage = int(r.integers(0, 3)) == 0
    return kv, D, Hkv, G, parents, hist, window, causal, garbage


@pytest.mark.parametrize("i", range(N_CASES))
def test_attention_sweep(ttv, i):
    _run_case(ttv, i, *_case(i), garbage=False, seeds=(1702, 1703))


@pytest.mark.parametrize("i", range(N_WIDE))
def test_attention_sweep_wide(ttv, i):
    kv, D, Hkv, G, parents, hist, window, causal, garbage = _wide_case(i)
    _run_case(ttv, i, kv, D, Hkv, G, parents, hist, window, causal, garbage=garbage, seeds=(2702, 2703))


def _run_case(ttv, i, kv, D, Hkv, G, parents, hist, window, causal, garbage, seeds):
    Hq = Hkv * G
    qd = "f32" if kv == "f32" else "bf16"
    B = len(parents)
    node_off = np.zeros(B + 1, np.int32)
    node_off[1:] = np.cumsum([len(p) for p in parents])
    n = int(node_off[-1])
    cap = int(max(h + len(p) for h, p in zip(hist, parents))) + (37 if garbage else 5)
    host = make_kv_cache(seeds[0], i, B, Hkv, cap, D, kv)
    q = make_queries(seeds[1], i, n, Hq, D, qd)
    dev_host = {k: v.copy() for k, v in host.items()}
    if garbage:  # rows past each live length are not part of the call
        for b in range(B):
            live = hist[b] + len(parents[b])
            for nm in ("k", "v"):
                if kv == "i8":
                    dev_host[nm + "_scale"].view(np.uint16)[b, :, live:] = 0x7E00
                elif kv == "bf16":
                    dev_host[nm][b, :, live:] = 0x7F80
                else:
                    dev_host[nm][b, :, live:] = np.float32(np.inf)
    _, kvl = layer_to_dev(ttv, dev_host)
    batch = ttv.Batch(node_off, np.asarray(hist, np.int32))
    anc, _, st = run_mask(ttv, batch, to_dev(np.concatenate(parents)))
    scale = 1.0 / math.sqrt(D)
    qdev = to_dev(q, "bf16" if qd == "bf16" else None)
    out = torch.full((n, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    a = None if causal else anc
    if window:
        ws = zeros_ws(ttv.tree_verify_attention_window_ws(batch, Hq, kvl, qd, window))
        ws.fill_(0x3C)
        ttv.tree_verify_attention_window(batch, qdev, kvl, a, scale, window, out, ws)
    else:
        ws = zeros_ws(ttv.tree_verify_attention_ws(batch, Hq, kvl, qd))
        ws.fill_(0x3C)
        ttv.tree_verify_attention(batch, qdev, kvl, a, scale, out, ws)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    want = O.tree_verify_attention(q, host, node_off, hist, None if causal else parents, scale, qd, kv,
                                   window=window)
    got = to_host(out)
    assert np.isfinite(got).all()
    err = float(np.abs(got - want).max())
    log(f"sweep {seeds[0]}/{i}: {kv} D={D} {Hq}/{Hkv} B={B} T={[len(p) for p in parents]} P={hist} "
        f"window={window} {'causal' if causal else 'tree'}{' garbage' if garbage else ''}: max|err| {err:.3e}")
    assert err <= TOL[kv], (i, err)
