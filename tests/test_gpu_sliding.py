"""GPU parity of the sliding-window layers' variants against the CPU oracle:
the caller mask intersected with the window band (bit-exact float32) and the
rollback confined to the verify block, including the refusal of a wrapped
rotating cache (bit-exact bytes)."""

import zlib

import numpy as np
import pytest
import torch

import oracle as O
from workloads import make_kv_cache, random_tree, rng_for

from gpu_util import layer_to_dev, layer_to_host, log, status, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

MASKED = np.float32(-1e9)


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


# ------------------------------------------------------------ band mask ----

def _band(ttv, caller, offset, window, in_place=False):
    c = to_dev(np.ascontiguousarray(caller, np.float32))
    out = c if in_place else torch.full_like(c, 7.0)
    ttv.sliding_mask_from_caller(c, offset, window, float(MASKED), out)
    return to_host(out)


@pytest.mark.parametrize("T,offset", [(1, 0), (7, 3), (16, 100), (64, 1000), (33, 4097)])
def test_band_of_tree_mask_matches_oracle(ttv, T, offset):
    parent = random_tree(rng_for(1500, T), T)
    caller = O.additive_mask_with_history(parent, offset)
    for window in sorted({1, 2, max(1, (offset + T) // 2), offset + T - 1 if offset + T > 1 else 1, offset + T,
                          offset + T + 9, 1024}):
        want = O.sliding_mask_from_caller(caller, offset, window)
        for in_place in (False, True):
            got = _band(ttv, caller, offset, window, in_place)
            np.testing.assert_array_equal(got, want, err_msg=f"T={T} P={offset} W={window} in_place={in_place}")
    log(f"band: T={T} offset={offset} ok")


def test_band_general_caller_values(ttv):
    """Arbitrary float callers (positive entries, NaN, the masked value itself,
    more columns than offset + T) and the pages' three properties on device."""
    r = rng_for(1510)
    T, offset = 40, 700
    S = offset + T + 37
    caller = (r.standard_normal((T, S)) * 3).astype(np.float32)
    caller[3, 690] = np.nan
    caller[5, :100] = MASKED
    caller[9, 720] = np.inf
    for window in (1, 17, 256, 739, 740, 741, 5000):
        want = O.sliding_mask_from_caller(caller, offset, window)
        np.testing.assert_array_equal(_band(ttv, caller, offset, window), want, err_msg=f"W={window}")
    W = 256
    allow = np.zeros((T, offset + T), np.float32)
    band = _band(ttv, allow, offset, W)
    q = np.arange(T)[:, None] + offset
    c = np.arange(offset + T)[None, :]
    np.testing.assert_array_equal(band, np.where((c > q - W) & (c <= q), 0.0, MASKED).astype(np.float32))
    once = _band(ttv, caller, offset, W)
    np.testing.assert_array_equal(_band(ttv, once, offset, W), once)
    # below the window: untouched, also in place (nothing launches then)
    np.testing.assert_array_equal(_band(ttv, caller, offset, offset + T), caller)
    np.testing.assert_array_equal(_band(ttv, caller, offset, offset + T, in_place=True), caller)


def test_band_expand_then_intersect_in_place(ttv):
    """The tree mask expanded on device, then intersected in place: equals the
    oracle's sliding form of the history mask, for every sequence of a batch."""
    parents = [random_tree(rng_for(1520, s), n) for s, n in enumerate((5, 64, 17, 1))]
    hist = np.array([1030, 0, 2000, 40], np.int32)
    node_off = np.zeros(len(parents) + 1, np.int32)
    node_off[1:] = np.cumsum([len(p) for p in parents])
    batch = ttv.Batch(node_off, hist)
    anc = to_dev(np.concatenate([O.ancestor_bits(p) for p in parents]))
    for b, par in enumerate(parents):
        T, P = len(par), int(hist[b])
        out = torch.empty(T, P + T, dtype=torch.float32, device="cuda")
        ttv.tree_mask_expand_additive(batch, b, anc, float(MASKED), out)
        ttv.sliding_mask_from_caller(out, P, 1024, float(MASKED), out)
        want = O.sliding_mask_from_caller(O.additive_mask_with_history(par, P), P, 1024)
        np.testing.assert_array_equal(to_host(out), want, err_msg=f"sequence {b}")


# ----------------------------------------------------------- tail gather ----

def _tail_case(ttv, dtype, D, kept, live, tails, L=2, H=2, cap=200, seed=0, wrapped=None):
    B = len(kept)
    host = [make_kv_cache(1530 + seed, l, B, H, cap, D, dtype, unique_scales=dtype == "i8") for l in range(L)]
    devs, layers = zip(*[layer_to_dev(ttv, h) for h in host])
    stride = 64 + 3
    kp = np.full((B, stride), -1, np.int32)
    for b, k in enumerate(kept):
        kp[b, :len(k)] = k
    kl = np.array([len(k) for k in kept], np.int32)
    st = status()
    err = None
    try:
        ttv.kv_gather_within_tail(list(layers), to_dev(kp), to_dev(kl), np.asarray(live, np.int32),
                                  np.asarray(tails, np.int32), st, zeros_ws(ttv.kv_gather_within_tail_ws(B)),
                                  ring_wrapped=wrapped)
    except ttv.TTVError as e:
        err = e
    torch.cuda.synchronize()
    return host, [layer_to_host(d) for d in devs], int(st.item()), err


def _kept_sets(r, tails, kind):
    out = []
    for t in tails:
        if kind == "random":
            out.append(np.sort(r.choice(t, size=int(r.integers(0, t + 1)), replace=False)))
        elif kind == "path":      # a root-first accepted path: 0 then increasing labels
            rest = r.choice(np.arange(1, t), size=int(r.integers(0, min(t - 1, 9) + 1)), replace=False) if t > 1 else []
            out.append(np.array([0] + sorted(int(x) for x in rest), np.int64) if t else np.zeros(0, np.int64))
        elif kind == "prefix":
            out.append(np.arange(int(r.integers(0, t + 1))))
        elif kind == "full":
            out.append(np.arange(t))
        elif kind == "last":      # only the block's last row survives
            out.append(np.array([t - 1]) if t else np.zeros(0, np.int64))
    return out


@pytest.mark.parametrize("dtype,D", [("i8", 64), ("i8", 128), ("bf16", 128), ("f32", 64), ("f32", 256)])
@pytest.mark.parametrize("kind", ["random", "path", "prefix", "full", "last"])
def test_tail_gather_matches_oracle(ttv, dtype, D, kind):
    r = rng_for(1540, zlib.crc32(repr((dtype, D, kind)).encode()) % 1000)
    live = [200, 150, 64, 7, 120]
    tails = [16, 64, 64, 7, 0]
    kept = _kept_sets(r, tails, kind)
    log(f"tail gather: {dtype} D={D} {kind}")
    host, got, st, err = _tail_case(ttv, dtype, D, kept, live, tails)
    assert err is None and st == 0
    for l in range(len(host)):
        want = O.gather_within_tail(host[l], live, tails, kept)
        for n in want:
            np.testing.assert_array_equal(got[l][n], want[n], err_msg=f"layer {l} {n}")


def test_tail_gather_many_layers_and_sequences(ttv):
    """18 layers (two launches of 16 layers at most) over 128 sequences."""
    r = rng_for(1550)
    B = 128
    live = [int(x) for x in r.integers(64, 100, size=B)]
    tails = [int(x) for x in r.integers(0, 65, size=B)]
    kept = _kept_sets(r, tails, "random")
    host, got, st, err = _tail_case(ttv, "i8", 64, kept, live, tails, L=18, H=1, cap=100, seed=1)
    assert err is None and st == 0
    for l in range(18):
        want = O.gather_within_tail(host[l], live, tails, kept)
        for n in want:
            np.testing.assert_array_equal(got[l][n], want[n], err_msg=f"layer {l} {n}")


def test_tail_gather_equals_absolute_gather(ttv):
    """The same rollback said in absolute positions through kv_gather_positions
    gives the same bytes."""
    r = rng_for(1560)
    live, tails = [200, 180, 90], [33, 64, 5]
    kept = _kept_sets(r, tails, "path")
    host, got, st, err = _tail_case(ttv, "bf16", 128, kept, live, tails, seed=2)
    assert err is None and st == 0
    sels = [np.concatenate([np.arange(lv - t), lv - t + np.asarray(k, np.int64)]) for lv, t, k in zip(live, tails, kept)]
    devs, layers = zip(*[layer_to_dev(ttv, h) for h in host])
    sel = np.full((3, 201), -1, np.int32)
    for b, s in enumerate(sels):
        sel[b, :len(s)] = s
    st2 = status()
    ttv.kv_gather_positions(list(layers), None, to_dev(sel), to_dev(np.array([len(s) for s in sels], np.int32)),
                            np.asarray(live, np.int32), st2, zeros_ws(ttv.kv_gather_positions_ws(3)))
    torch.cuda.synchronize()
    assert int(st2.item()) == 0
    for l, d in enumerate(devs):
        absolute = layer_to_host(d)
        for n in absolute:
            np.testing.assert_array_equal(got[l][n], absolute[n], err_msg=f"layer {l} {n}")


def test_tail_gather_bad_kept_writes_nothing(ttv):
    r = rng_for(1570)
    live, tails = [200, 150, 64], [16, 20, 64]
    for bad_case in range(4):
        kept = _kept_sets(r, tails, "path")
        if bad_case == 0:
            kept[1] = np.array([0, 5, 5])                  # not strictly increasing
        elif bad_case == 1:
            kept[2] = np.array([0, 64])                    # outside the tail
        elif bad_case == 2:
            kept[0] = np.array([-1, 3])                    # negative
        else:
            kept[1] = np.arange(21)                        # longer than the tail
        host, got, st, err = _tail_case(ttv, "i8", 64, kept, live, tails, seed=3)
        assert err is None and st == ttv.TTV_DEV_BAD_SELECTION, bad_case
        for l in range(len(host)):
            for n in host[l]:
                np.testing.assert_array_equal(got[l][n], host[l][n], err_msg=f"case {bad_case} layer {l} {n}")


def test_tail_gather_refuses_wrapped_ring(ttv):
    r = rng_for(1580)
    live, tails = [200, 150], [16, 16]
    kept = _kept_sets(r, tails, "path")
    host, got, st, err = _tail_case(ttv, "bf16", 64, kept, live, tails, seed=4, wrapped=[0, 1])
    assert err is not None and err.status == ttv.TTV_ERR_UNSUPPORTED and "wrapped" in str(err)
    assert st == 0
    for l in range(len(host)):
        for n in host[l]:
            np.testing.assert_array_equal(got[l][n], host[l][n])
    # an unwrapped (buffered) ring is gathered as usual
    host, got, st, err = _tail_case(ttv, "bf16", 64, kept, live, tails, seed=4, wrapped=[0, 0])
    assert err is None and st == 0
    want = O.gather_within_tail(host[0], live, tails, kept)
    for n in want:
        np.testing.assert_array_equal(got[0][n], want[n])


# ---------------------------------------------------- windowed attention ----

TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def _window_check(ttv, kv, parents, hist, Hq, Hkv, windows, seed, causal=False):
    from workloads import make_queries
    D = 64 if kv == "f32" else 128
    qd = "f32" if kv == "f32" else "bf16"
    B = len(parents)
    node_off = np.zeros(B + 1, np.int32)
    node_off[1:] = np.cumsum([len(p) for p in parents])
    cap = int(max(h + len(p) for h, p in zip(hist, parents))) + 3
    host = make_kv_cache(1590, seed, B, Hkv, cap, D, kv)
    q = make_queries(1591, seed, int(node_off[-1]), Hq, D, qd)
    _, kvl = layer_to_dev(ttv, host)
    qd_dev = to_dev(q, "bf16" if qd == "bf16" else None)
    batch = ttv.Batch(node_off, np.asarray(hist, np.int32))
    anc = None if causal else to_dev(np.concatenate([O.ancestor_bits(p) for p in parents]))
    scale = 1.0 / np.sqrt(D)
    tol = TOL_F32 if kv == "f32" else TOL_BF16
    for W in windows:
        need = ttv.tree_verify_attention_window_ws(batch, Hq, kvl, qd, W)
        assert need > 0, ttv.last_error()
        ws = zeros_ws(need)
        ws.fill_(0x7F)     # any contents on entry
        out = torch.full((int(node_off[-1]), Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        ttv.tree_verify_attention_window(batch, qd_dev, kvl, anc, float(scale), W, out, ws)
        torch.cuda.synchronize()
        want = O.tree_verify_attention(q, host, node_off, hist, None if causal else parents, scale, qd, kv, window=W)
        g = to_host(out)
        assert np.isfinite(g).all(), W
        err = float(np.abs(g - want).max()) if g.size else 0.0
        log(f"window attention {kv} W={W}: max|err| {err:.3e}")
        assert err <= tol, (kv, W, err)


@pytest.mark.parametrize("kv", ["bf16", "i8", "f32"])
def test_window_attention_matches_oracle(ttv, kv):
    """Windows below the block (W < T: ancestors drop out too), inside the
    history, and beyond P + T (the plain key sets), over a ragged batch with an
    empty tree and an empty history."""
    parents = [random_tree(rng_for(1600, s), n) for s, n in enumerate((64, 16, 1, 40))] + [np.zeros(0, np.int32)]
    parents.append(random_tree(rng_for(1600, 9), 20))
    hist = [3000, 1100, 0, 257, 12, 0]
    Hq, Hkv = (8, 2) if kv == "f32" else (40, 8)
    _window_check(ttv, kv, parents, hist, Hq, Hkv, [1, 5, 63, 64, 300, 1024, 2999, 3064, 5000],
                  seed=zlib.crc32(kv.encode()) % 97)


def test_window_attention_long_history_many_splits(ttv):
    """A 4096-token window over histories of 20k-40k: the history below the
    window is never read, the window spans several splits."""
    parents = [random_tree(rng_for(1610, s), 64) for s in range(3)]
    _window_check(ttv, "i8", parents, [40000, 20000, 4000], 32, 8, [4096, 1024], seed=3)


def test_window_attention_causal_block(ttv):
    """anc = NULL (the linear block) under a window: equals the oracle's chain."""
    from workloads import chain_tree
    parents = [chain_tree(33), chain_tree(8)]
    _window_check(ttv, "bf16", parents, [500, 70], 16, 4, [10, 40, 200], seed=5, causal=True)


def test_window_attention_small_trees_edge_tiles(ttv):
    """Trees of at most 19 nodes and a chain (the narrow bf16 kernel, and the
    int8 one) under windows whose first keys are hidden from some rows: 64
    and 65 (one hidden-key tile; at history 129 the window of 64 leaves no
    whole tile behind it, so that call takes the vector path), 96/97/128
    around the second tile, and windows reaching the start of the history."""
    from workloads import chain_tree
    parents = [random_tree(rng_for(1620, s), n) for s, n in enumerate((19, 7, 12))] + [chain_tree(3)]
    hist = [5000, 2000, 700, 129]
    _window_check(ttv, "bf16", parents, hist, 40, 8, [64, 65, 96, 97, 128, 500, 1999, 2000, 2020], seed=7)
    _window_check(ttv, "i8", parents, hist, 40, 8, [64, 65, 100, 1000, 2010], seed=8)
