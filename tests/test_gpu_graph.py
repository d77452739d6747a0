"""A whole verify round captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capturing stream) and replayed: every replay,
with eager work and synchronisations between replays, must reproduce the
eager round bit for bit (same kernels, same inputs, no atomics in any
reduction). The round: ancestor mask, attention over every layer, vocabulary
argmax, accept walk with its selection, and the out-of-place gather of every
layer into a second cache. Two shapes: the 16-layer int8 tree round and a
ragged bf16 batch whose larger trees take the wide attention layout."""

import math

import numpy as np
import pytest
import torch

from workloads import config3_round, config4_round
from workloads.device import dev_kv_cache, dev_planted_logits, dev_queries

from gpu_util import spec_batch, to_dev, zeros_ws

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def _round(ttv, spec, kv):
    dev = "cuda"
    B, L, n = spec.B, spec.L, spec.n_nodes
    cap = int(max(spec.hist_len + np.diff(spec.node_off)))
    caches = [dev_kv_cache(spec.seed, 300 + l, B, spec.Hkv, cap, spec.D, kv, dev) for l in range(L)]
    layers = [ttv.KVLayer(c["k"], c["v"], c.get("k_scale"), c.get("v_scale")) for c in caches]
    dst = [{k: torch.zeros_like(t) for k, t in c.items()} for c in caches]
    dst_layers = [ttv.KVLayer(c["k"], c["v"], c.get("k_scale"), c.get("v_scale")) for c in dst]
    qs = [dev_queries(spec.seed, 400 + l, n, spec.Hq, spec.D, "bf16", dev) for l in range(L)]
    logits = dev_planted_logits(spec.seed, spec.flat_targets, spec.vocab, spec.sigma, dev)
    batch = spec_batch(ttv, spec)
    parent = to_dev(spec.flat("parents"))
    token = to_dev(spec.flat("tokens").astype(np.int32))
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    anc = torch.empty(n, dtype=torch.int64, device=dev)
    outs = [torch.empty(n, spec.Hq, spec.D, dtype=torch.float32, device=dev) for _ in range(L)]
    ws = zeros_ws(ttv.tree_verify_attention_ws(batch, spec.Hq, layers[0], "bf16"))
    am = torch.empty(n, dtype=torch.int32, device=dev)
    aws = zeros_ws(max(1, ttv.vocab_argmax_ws(n, spec.vocab)))
    path = torch.empty(B, 64, dtype=torch.int32, device=dev)
    plen = torch.empty(B, dtype=torch.int32, device=dev)
    emitted = torch.empty(B, 64, dtype=torch.int32, device=dev)
    sel = torch.empty(B, cap, dtype=torch.int32, device=dev)
    sel_len = torch.empty(B, dtype=torch.int32, device=dev)
    live = (spec.hist_len + np.diff(spec.node_off)).astype(np.int32)
    gws = zeros_ws(ttv.kv_gather_positions_ws(B))
    scale = 1.0 / math.sqrt(spec.D)

    def step():
        ttv.tree_build_mask(batch, parent, anc, None, st)
        for l in range(L):
            ttv.tree_verify_attention(batch, qs[l], layers[l], anc, scale, outs[l], ws)
        ttv.vocab_argmax(logits, am, aws)
        ttv.tree_accept_walk(batch, parent, token, am, path, plen, emitted, st, sel, sel_len)
        ttv.kv_gather_positions(layers, dst_layers, sel, sel_len, live, st, gws)

    def results():
        r = {f"out{l}": t.clone() for l, t in enumerate(outs)}
        r.update(anc=anc.clone(), argmax=am.clone(), path=path.clone(), plen=plen.clone(), emitted=emitted.clone(),
                 sel_len=sel_len.clone(), status=st.clone())
        for l, c in enumerate(dst):
            r.update({f"dst{l}_{k}": t.clone() for k, t in c.items()})
        return r

    def scrub():
        # outputs overwritten between runs, so a replay that skipped a launch shows
        for t in outs:
            t.fill_(float("nan"))
        for t in (anc, am, path, plen, emitted, sel_len):
            t.fill_(-7)
        for c in dst:
            for t in c.values():
                t.zero_()
        ws.fill_(0x5A)

    return step, results, scrub


@pytest.mark.parametrize("shape", ["int8_16_layers", "bf16_ragged"])
def test_round_graph_replays_match_eager(ttv, shape):
    if shape == "int8_16_layers":
        spec, kv = config3_round(), "i8"
    else:
        spec, kv = config4_round(B=6, pmin=500, pmax=3000), "bf16"   # trees up to 64 nodes: the wide layout
    step, results, scrub = _round(ttv, spec, kv)
    # eager reference (twice: the round is deterministic)
    scrub()
    step()
    torch.cuda.synchronize()
    want = results()
    assert int(want["status"].item()) == 0
    assert int(want["plen"].min().item()) >= 1
    scrub()
    step()
    torch.cuda.synchronize()
    again = results()
    for k in want:
        assert torch.equal(want[k], again[k]), k
    # capture (torch's capture stream is the binding's current stream)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        scrub()
        x = torch.randn(1 << 20, device="cuda")   # eager work between replays
        (x * 2).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = results()
        for k in want:
            assert torch.equal(want[k], got[k]), (shape, rep, k)
