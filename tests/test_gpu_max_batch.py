"""A whole verify round at the largest batch the boundary takes (128
sequences): ragged trees of 1 to 64 nodes (3-ary depth-3 trees, random
recursive trees, chains of 64 and single nodes), prefixes of 0 to 400 keys,
40/8 heads, bf16 and int8 KV. Mask, attention, argmax, walk and the in-place
rollback gather run on the GPU and are compared with the oracle's round:
masks, argmaxes, paths, emitted tokens and the gathered cache bit for bit,
attention within the bf16 bound."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from workloads import host_tensors, plant_walk, random_descent, random_tree, rng_for, sary_tree
from workloads.configs import _spec

from gpu_util import (layer_to_dev, layer_to_host, log, run_argmax, run_attention, run_mask, run_walk, spec_batch,
                      status, to_dev, to_host, zeros_ws)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
VOCAB = 1000


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def max_batch_spec(ttv, kv: str, seed: int = 61):
    B = ttv.MAX_BATCH
    r = rng_for(seed, 0)
    parents, tokens, targets, paths, hist = [], [], [], [], []
    for b in range(B):
        kind = b % 4
        if kind == 0:
            parent = sary_tree(3, 3)
        elif kind == 1:
            parent = random_tree(rng_for(seed, 1, b), int(r.integers(8, 65)))
        elif kind == 2:
            parent = np.arange(-1, 63, dtype=np.int32) if b % 8 == 2 else np.array([-1], np.int32)
        else:
            parent = random_tree(rng_for(seed, 2, b), 64)
        d = random_descent(parent, rng_for(seed, 3, b))
        path = d[: int(r.integers(0, len(d))) + 1]
        tok, tgt, _ = plant_walk(parent, path, rng_for(seed, 4, b), VOCAB)
        parents.append(parent)
        tokens.append(tok)
        targets.append(tgt)
        paths.append(path)
        hist.append(int(r.integers(0, 401)))
    return _spec(seed, B, 1, 40, 8, 128, VOCAB, 2.0, kv, "bf16", hist, parents, tokens, targets, paths,
                 note=f"max batch {kv}")


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_round_at_max_batch(ttv, kv):
    spec = max_batch_spec(ttv, kv)
    T_b = np.diff(spec.node_off)
    assert spec.B == ttv.MAX_BATCH and T_b.max() == 64 and T_b.min() == 1
    tens = host_tensors(spec)
    want = O.verify_round(spec, tens)
    log(f"max batch {kv}: {spec.B} trees, {spec.n_nodes} nodes, paths of {sorted(set(len(p) for p in spec.paths))}")
    batch = spec_batch(ttv, spec)
    par = to_dev(spec.flat("parents"))
    anc, depth, st = run_mask(ttv, batch, par)
    host = tens["layers"][0]
    dev, kvl = layer_to_dev(ttv, host)
    out, _ = run_attention(ttv, batch, to_dev(host["q"], "bf16"), kvl, anc, 1 / math.sqrt(spec.D))
    am = run_argmax(ttv, to_dev(tens["logits"]))
    path, plen, em, sel, sel_len, st2 = run_walk(ttv, batch, par, to_dev(spec.flat("tokens").astype(np.int32)), am)
    st3 = status()
    ttv.kv_gather_positions([kvl], None, sel, sel_len, spec.hist_len + T_b, st3,
                            zeros_ws(ttv.kv_gather_positions_ws(spec.B)))
    torch.cuda.synchronize()
    assert int(st.item()) == int(st2.item()) == int(st3.item()) == 0
    np.testing.assert_array_equal(to_host(anc).view(np.uint64), want["anc"])
    np.testing.assert_array_equal(to_host(depth), want["depth"])
    g = to_host(out)
    assert np.isfinite(g).all()
    err = float(np.abs(g - want["attn"][0]).max())
    log(f"max batch {kv}: attention max|err| {err:.3e}")
    assert err <= TOL_BF16
    np.testing.assert_array_equal(to_host(am), want["argmax"])
    hp, hl, he = to_host(path), to_host(plen), to_host(em)
    for b in range(spec.B):
        n = int(hl[b])
        assert list(hp[b, :n]) == want["paths"][b] == spec.paths[b], b
        assert list(he[b, :n]) == want["emitted"][b], b
    got = layer_to_host(dev)
    for name in want["caches"][0]:
        np.testing.assert_array_equal(got[name], want["caches"][0][name])
