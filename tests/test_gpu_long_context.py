"""The long-context stress workload at its stated size, round after round:
B=8 sequences, 8 layers of int8 KV with fp16 per-token scales, 40/8 heads,
head_dim 128, a 131,072-token prefix, 16-node trees, vocab 248,320, and 100
rounds of mask -> attention (every layer) -> argmax -> walk -> in-place
rollback, on the seeded schedule that mixes scattered tree paths, full
accepts (the identity selection) and partial accepts (prefix selections).

Every round the GPU state is compared with the oracle:
  * ancestor bitsets, argmax, paths, emitted tokens and selection lengths,
    bit for bit;
  * every cache row past the initial prefix (codes and scales, every layer,
    sequence and KV head), bit for bit, against the oracle's gather applied
    to its own copy of those rows;
  * attention of two seeded nodes of one seeded (layer, sequence, KV head);
    a whole (sequence, layer) slab (16 nodes x 40 heads) on round 0 and every
    tenth round after it (rounds 9, 19, ..., 99), round 49 among them.
Every 10 rounds the untouched prefix of every layer is compared with a fresh
draw of the generator. The oracle's inputs are the generator's draws and its
own copy of the appended rows: nothing it reads comes from the HIP path."""

import math
import time

import numpy as np
import pytest
import torch

import oracle as O
from workloads import config5_round, config5_schedule, rng_for
from workloads.device import dev_kv_cache, dev_planted_logits, dev_queries
from workloads.gen import quantize_int8_per_token

from gpu_util import log, run_argmax, run_mask, run_walk, spec_batch, status, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
P0 = 131072
ROUNDS = 100
T = 16
SEED = 5
FULL_CHECK_ROUNDS = (0, 9, 19, 29, 39, 49, 59, 69, 79, 89, 99)
NAMES = ("k", "v", "k_scale", "v_scale")


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def test_long_context_100_rounds_cache_tracks_oracle(ttv):
    t_start = time.time()
    sched = config5_schedule(ROUNDS, seed=SEED)
    spec0 = config5_round(0, [P0] * 8, sched[0], seed=SEED)
    B, L, Hq, Hkv, D, V, G = spec0.B, spec0.L, spec0.Hq, spec0.Hkv, spec0.D, spec0.vocab, spec0.G
    cap = P0 + T * (ROUNDS + 1)
    scale = 1.0 / math.sqrt(D)

    def draw_layer(l):
        # the generator's draw of layer l's cache (the same one every time)
        return dev_kv_cache(SEED, 100 + l, B, Hkv, cap, D, "i8", "cuda")

    caches = [draw_layer(l) for l in range(L)]
    layers = [ttv.KVLayer(c["k"], c["v"], c["k_scale"], c["v_scale"]) for c in caches]
    # the oracle's copy of every row at and past P0 (all of them change hands
    # during the run), starting from the generator's draw
    mirror = [{n: to_host(c[n][:, :, P0:]) for n in NAMES} for c in caches]
    torch.cuda.synchronize()
    log(f"long-context: {L} layers x {B} sequences x {Hkv} KV heads, cap {cap}, set up in "
        f"{time.time() - t_start:.1f} s")

    ws = zeros_ws(32 << 20)
    gws = zeros_ws(ttv.kv_gather_positions_ws(B))
    hist = np.full(B, P0, np.int64)
    kinds_seen, accepts = {}, []
    worst = 0.0
    for r, kind in enumerate(sched):
        t_round = time.time()
        spec = config5_round(r, hist.copy(), kind, seed=SEED)
        n = spec.n_nodes
        # the block's 16 quantised rows of every (layer, sequence) are appended at P_b, on both copies
        for l in range(L):
            for b in range(B):
                P = int(hist[b])
                o = P - P0
                for nm, sid in (("k", 0), ("v", 1)):
                    x = rng_for(1400, r, l, b, sid).standard_normal((Hkv, T, D), dtype=np.float32)
                    code, sc = quantize_int8_per_token(x)
                    mirror[l][nm][b, :, o:o + T] = code
                    mirror[l][nm + "_scale"][b, :, o:o + T] = sc
                    caches[l][nm][b, :, P:P + T] = to_dev(code)
                    caches[l][nm + "_scale"][b, :, P:P + T] = to_dev(sc)
        qs = [dev_queries(14000 + r, l, n, Hq, D, "bf16", "cuda") for l in range(L)]
        logits = dev_planted_logits(15000 + r, spec.flat_targets, V, spec.sigma, "cuda")

        # ---- the GPU round
        batch = spec_batch(ttv, spec)
        par = to_dev(spec.flat("parents"))
        anc, _, st = run_mask(ttv, batch, par)
        assert ttv.tree_verify_attention_ws(batch, Hq, layers[0], "bf16") <= ws.numel()
        outs = []
        for l in range(L):
            out = torch.empty(n, Hq, D, dtype=torch.float32, device="cuda")
            ttv.tree_verify_attention(batch, qs[l], layers[l], anc, scale, out, ws)
            outs.append(out)
        am = run_argmax(ttv, logits)
        path, plen, emitted, sel, sel_len, st2 = run_walk(ttv, batch, par,
                                                          to_dev(spec.flat("tokens").astype(np.int32)), am)
        live = (hist + T).astype(np.int32)
        gst = status()
        ttv.kv_gather_positions(layers, None, sel, sel_len, live, gst, gws)
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and int(st2.item()) == 0 and int(gst.item()) == 0, r

        # ---- steps 1, 3, 4 against the oracle, bit for bit
        node_off = spec.node_off
        np.testing.assert_array_equal(to_host(anc).view(np.uint64),
                                      np.concatenate([O.ancestor_bits(p) for p in spec.parents]))
        am_o = O.vocab_argmax(to_host(logits))
        np.testing.assert_array_equal(to_host(am), am_o)
        pl, ph, eh = to_host(plen), to_host(path), to_host(emitted)
        sels = []
        for b in range(B):
            o0, o1 = int(node_off[b]), int(node_off[b + 1])
            p_o, e_o = O.tree_accept_walk(spec.parents[b], spec.tokens[b], am_o[o0:o1])
            assert list(ph[b, :pl[b]]) == p_o and list(eh[b, :pl[b]]) == e_o, (r, kind, b)
            assert p_o == list(spec.paths[b]), (r, kind, b)      # the planted path: the round is what it says
            sels.append(O.rollback_selection(int(hist[b]), p_o))
            accepts.append(len(p_o) - 1)
        assert list(to_host(sel_len)) == [len(s) for s in sels]

        # ---- step 2: sampled nodes every round, whole slabs on the full-check rounds
        rs = rng_for(1402, r)
        l_s = int(rs.integers(0, L))
        checks = [(l_s, int(rs.integers(0, B)), int(rs.integers(0, Hkv)), None)]
        if r in FULL_CHECK_ROUNDS:
            b_full = int(rng_for(1403, r).integers(0, B))
            checks += [(l_s, b_full, g, "all") for g in range(Hkv)]
        fresh = draw_layer(l_s)
        for l, b, g, mode in checks:
            P = int(hist[b])
            slab = {}
            for nm in NAMES:
                head = to_host(fresh[nm][b:b + 1, g:g + 1, :P0])
                tail = mirror[l][nm][b:b + 1, g:g + 1, :P - P0 + T]
                slab[nm] = np.concatenate([head, tail], axis=2)
            o0 = int(node_off[b])
            qh = to_host(qs[l][o0:o0 + T, g * G:(g + 1) * G])
            got = to_host(outs[l][o0:o0 + T, g * G:(g + 1) * G])
            if mode == "all":
                want = O.tree_verify_attention(qh, slab, np.array([0, T]), np.array([P]), [spec.parents[b]], scale,
                                               "bf16", "i8")
                err = float(np.abs(got - want).max())
            else:
                K = O.decode_kv(slab["k"][0, 0], "i8", slab["k_scale"][0, 0])
                Vv = O.decode_kv(slab["v"][0, 0], "i8", slab["v_scale"][0, 0])
                sets = O.ancestor_sets(spec.parents[b])
                err = 0.0
                for t in sorted({int(rs.integers(0, T)), int(rs.integers(0, T))}):
                    want = O.attention_rows(O.decode_bf16(qh[t]), K, Vv, O.visible_keys(P, sets[t]), scale)
                    err = max(err, float(np.abs(got[t] - want).max()))
            worst = max(worst, err)
            assert err <= TOL_BF16, (r, kind, l, b, g, mode, err)
        del fresh

        # ---- step 5: the oracle's gather on its copy; every row past P0 must match
        rel = [s[P0:] - P0 for s in sels]
        mirror = [O.gather_layer(m, rel) for m in mirror]
        for l in range(L):
            for nm in NAMES:
                got = to_host(caches[l][nm][:, :, P0:])
                if not np.array_equal(got, mirror[l][nm]):
                    bad = np.argwhere(got != mirror[l][nm])[:4]
                    raise AssertionError(f"round {r} {kind}: layer {l} {nm} differs at {bad.tolist()}")
        # the untouched prefix, against a fresh draw of the generator
        if r % 10 == 9 or r == 0:
            for l in range(L):
                fresh = draw_layer(l)
                for nm in NAMES:
                    assert torch.equal(caches[l][nm][:, :, :P0], fresh[nm][:, :, :P0]), (r, l, nm)
                del fresh
        kinds_seen[kind] = kinds_seen.get(kind, 0) + 1
        hist = np.array([len(s) for s in sels], np.int64)
        log(f"long-context round {r:3d} {kind:7s}: accepted {[len(s) - int(h) - 1 for s, h in zip(sels, spec.hist_len)]}"
            f", attention max|err| {worst:.2e}{' (whole slab)' if r in FULL_CHECK_ROUNDS else ''}, cache rows past "
            f"P0 equal, {time.time() - t_round:.1f} s")
        del qs, logits, outs

    # the run covered what the schedule promises: scattered tree paths, full
    # accepts (identity selections) and partial ones (prefix selections,
    # zero accepts among them)
    assert set(kinds_seen) == {"tree", "full", "partial"}
    assert 0 in accepts and T - 1 in accepts
    log(f"long-context: {ROUNDS} rounds {kinds_seen}, worst attention error {worst:.2e}, "
        f"{time.time() - t_start:.0f} s in all")
