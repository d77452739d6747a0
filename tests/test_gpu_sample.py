"""GPU parity of the sampled selection (vocab_sample) against the CPU oracle:
the drawn index must match the oracle's draw for every row. The draw is an
integer decided by float64 comparisons; the two sides compute the same
float64 expressions in the same order, and may only part where a uniform
falls within 1e-12 of a cumulative boundary (checked, never seen)."""

import numpy as np
import pytest
import torch

import oracle as O
from workloads import confidence_tree, random_descent, random_tree, rng_for, sary_tree

from gpu_util import log, run_walk, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

V5 = 248320


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def run_sample(ttv, X, U, stride, T, k, p, vocab=None):
    Xd = to_dev(np.ascontiguousarray(X, np.float32))
    Ud = to_dev(np.ascontiguousarray(U, np.float32))
    n = X.shape[0]
    V = X.shape[1] if vocab is None else vocab
    out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    ws = zeros_ws(ttv.vocab_sample_ws(n, V, k))
    ws.fill_(0xA5)  # contents on entry are irrelevant
    ttv.vocab_sample(Xd, Ud, out, ws, T, k, p, uniform_stride=stride, vocab=V)
    return to_host(out)


def boundary_margin(x, u, T, k, p):
    """Distance of the draw's decisions from their thresholds (float64)."""
    x = np.asarray(x, np.float64)
    order = np.argsort(-x, kind="stable")[: min(k, len(x))]
    z = x[order] / np.float64(np.float32(T))
    e = np.exp(z - z[0])
    C = np.cumsum(e) / e.sum()
    pp = np.float64(np.float32(p))
    i_star = int(np.argmax(C >= pp))
    tgt = np.float64(np.float32(u)) * C[i_star]
    return min(np.min(np.abs(C - pp)), np.min(np.abs(C[: i_star + 1] - tgt)))


def check(ttv, X, U, stride, T, k, p, label, vocab=None):
    got = run_sample(ttv, X, U, stride, T, k, p, vocab)
    Xo = X if vocab is None else X[:, :vocab]
    want = O.vocab_sample(Xo, U, stride, T, k, p)
    bad = np.nonzero(got != want)[0]
    for n in bad:
        m = boundary_margin(Xo[n], U[n * stride], T, k, p)
        assert m < 1e-12, (label, int(n), int(got[n]), int(want[n]), m)
    log(f"sample {label}: {X.shape[0]} rows, {len(bad)} boundary ties")
    return got


@pytest.mark.parametrize("T,k,p", [(1.0, 20, 0.95), (0.7, 64, 0.9), (1.5, 1, 0.95), (1.0, 5, 1.0), (2.0, 33, 0.5)])
def test_sample_matches_oracle_vocab_248320(ttv, T, k, p):
    r = rng_for(1400, int(T * 10) + k)
    X = (r.standard_normal((24, V5)) * 2).astype(np.float32)
    U = r.random(24).astype(np.float32)
    check(ttv, X, U, 1, T, k, p, f"V={V5} T={T} k={k} p={p}")


@pytest.mark.parametrize("n,V", [(7, 1024), (3, 2049), (5, 100), (2, 1), (40, 4097), (3, 20)])
def test_sample_small_and_ragged_vocab(ttv, n, V):
    r = rng_for(1410, V)
    X = (r.standard_normal((n, V)) * 2).astype(np.float32)
    U = r.random(n).astype(np.float32)
    check(ttv, X, U, 1, 1.0, 20, 0.95, f"{n} x {V}")
    check(ttv, X, U, 1, 0.5, 64, 0.99, f"{n} x {V} k=64")


def test_sample_uniform_stride(ttv):
    r = rng_for(1420)
    X = (r.standard_normal((9, 5000)) * 2).astype(np.float32)
    U = r.random(30).astype(np.float32)
    check(ttv, X, U, 0, 1.0, 20, 0.95, "stride 0")
    check(ttv, X, U, 3, 1.0, 20, 0.95, "stride 3")


def test_sample_ties_nonfinite_and_unaligned(ttv):
    r = rng_for(1430)
    X = (r.standard_normal((16, V5)) * 2).astype(np.float32)
    m = float(X.max()) + 1
    X[0, [5, 2047, 2048, 4095, 100000, V5 - 1]] = m           # ties at the top across chunk boundaries
    X[1, ::7] = m                                              # thousands of tied top values
    X[2, :] = 1.0                                              # every value tied
    X[3, 100] = np.nan
    X[3, 5] = np.nan
    X[4, 77] = np.inf
    X[5, :] = -np.inf
    X[6, :] = -np.inf
    X[6, 1234] = 0.5
    X[6, 999] = 0.5
    X[7, :1000] = -0.0
    X[7, 1000:] = -5.0
    X[7, 500] = 0.0
    X[8, :] = np.round(X[8, :])                               # many ties everywhere
    U = r.random(16).astype(np.float32)
    U[9] = 0.0
    U[10] = np.float32(0.99999994)
    check(ttv, X, U, 1, 1.0, 20, 0.95, "ties/non-finite")
    check(ttv, X, U, 1, 1.0, 64, 1.0, "ties/non-finite k=64")
    # unaligned rows take the scalar loads
    Y = np.ascontiguousarray(np.pad(X[:, : V5 - 3], ((0, 0), (0, 1)), constant_values=np.inf))  # never read
    check(ttv, Y, U, 1, 1.0, 20, 0.95, "unaligned", vocab=V5 - 3)


def test_sample_chi_square_on_device(ttv):
    """The pages' check: drawn tokens against the nucleus distribution."""
    from scipy.stats import chisquare
    r = rng_for(1440)
    x = (r.standard_normal((1, 8192)) * 2).astype(np.float32)
    M = 4096
    X = np.repeat(x, M, axis=0)
    U = r.random(M).astype(np.float32)
    got = check(ttv, X, U, 1, 1.0, 20, 0.95, "chi-square rows")
    order = np.argsort(-x[0].astype(np.float64), kind="stable")[:20]
    w = np.exp(x[0, order].astype(np.float64) - x[0, order[0]])
    C = np.cumsum(w) / w.sum()
    n_keep = int(np.searchsorted(C, np.float64(np.float32(0.95)), side="left")) + 1
    kept, prob = order[:n_keep], w[:n_keep] / w[:n_keep].sum()
    obs = np.array([(got == t).sum() for t in kept], np.float64)
    assert obs.sum() == M
    pv = chisquare(obs, M * prob).pvalue
    log(f"sample chi-square: {n_keep} kept tokens, p = {pv:.3f}")
    assert pv > 1e-3


def test_sampled_round_walk(ttv):
    """Sampled targets drive the walk: the device's draws and path equal the
    oracle's on confidence trees and random trees."""
    r = rng_for(1450)
    parents = [confidence_tree(rng_for(1451, s), 16, 8, 1000, 4)[0] for s in range(6)]
    parents += [random_tree(rng_for(1452, s), 40) for s in range(4)] + [sary_tree(3, 3)]
    n = sum(len(p) for p in parents)
    X = (r.standard_normal((n, 4096)) * 2).astype(np.float32)
    U = r.random(n).astype(np.float32)
    tgt = O.vocab_sample(X, U, 1, 1.0, 20, 0.95)
    got = run_sample(ttv, X, U, 1, 1.0, 20, 0.95)
    np.testing.assert_array_equal(got, tgt)
    # draft tokens: random, except that along a random descent each node
    # carries its parent's sampled target (so walks go deep)
    tokens, off = [], 0
    for s_, par in enumerate(parents):
        rr = rng_for(1453, s_)
        tok = rr.integers(0, 4096, size=len(par)).astype(np.int64)
        d = random_descent(par, rng_for(1454, s_))
        for a, b in zip(d[:-1], d[1:]):
            tok[b] = tgt[off + a]
        tokens.append(tok)
        off += len(par)
    node_off = np.zeros(len(parents) + 1, np.int32)
    node_off[1:] = np.cumsum([len(p) for p in parents])
    batch = ttv.Batch(node_off, np.full(len(parents), 64, np.int32))
    path, plen, emitted, _, _, st = run_walk(ttv, batch, to_dev(np.concatenate(parents).astype(np.int32)),
                                             to_dev(np.concatenate(tokens).astype(np.int32)), to_dev(got))
    assert int(to_host(st)[0]) == 0
    deep = 0
    for b, par in enumerate(parents):
        o = int(node_off[b])
        want_path, want_emit = O.tree_accept_walk(par, tokens[b], tgt[o:o + len(par)])
        L = int(to_host(plen)[b])
        assert list(to_host(path)[b, :L]) == want_path, b
        assert list(to_host(emitted)[b, :L]) == want_emit, b
        deep += len(want_path) > 2
    assert deep >= 5  # the walks are not vacuous
