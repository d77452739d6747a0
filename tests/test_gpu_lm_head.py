"""GPU parity of the fused LM-head projection + argmax (lm_head_argmax)
against the CPU oracle's float64 logits.

The kernel takes the decision on fp32 logits accumulated from exact bf16
products, so its logits differ from the float64 ones by at most
gamma * sum_i |x_i w_vi| with gamma = H * 2^-24 (a bound on any summation
order). Per node, with tol = gamma * max_v sum_i |x_i w_vi|: where the top two
float64 logits are more than 2 tol apart the index must equal the oracle's
argmax exactly, and in every case the chosen logit must lie within 2 tol of
the maximum. Planted winners and equal rows (identical weight rows give
bit-identical logits on both sides) are checked exactly."""

import numpy as np
import pytest
import torch

import oracle as O
from workloads import bf16_bits_to_f32, lm_head_inputs, rng_for

from gpu_util import log, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

V5 = 248320


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def run(ttv, hb, wb, hs_pad=0, ws_pad=0):
    N, H = hb.shape
    V = wb.shape[0]
    if hs_pad:  # the padding holds NaN: no element past H may be read
        buf = np.full((N, H + hs_pad), 0x7FC0, np.uint16)
        buf[:, :H] = hb
        Xd = to_dev(buf, "bf16")[:, :H]
    else:
        Xd = to_dev(hb, "bf16")
    if ws_pad:
        buf = np.full((V, H + ws_pad), 0x7FC0, np.uint16)
        buf[:, :H] = wb
        Wd = to_dev(buf, "bf16")[:, :H]
    else:
        Wd = to_dev(wb, "bf16")
    out = torch.full((max(N, 1),), -3, dtype=torch.int32, device="cuda")
    ws = zeros_ws(ttv.lm_head_argmax_ws(N, V))
    ws.fill_(0x5A)  # contents on entry are irrelevant
    ttv.lm_head_argmax(Xd, Wd, out, ws)
    return to_host(out)[:N]


def oracle_rows(hb, wb, rows, block=16384):
    """float64 logits and absolute-product sums of the given rows, the
    oracle's projection taken over vocabulary blocks to bound memory."""
    L, A = [], []
    Xa = np.abs(bf16_bits_to_f32(hb[rows]).astype(np.float64))
    for v0 in range(0, wb.shape[0], block):
        L.append(O.lm_head_logits(hb[rows], wb[v0:v0 + block]))
        A.append(Xa @ np.abs(bf16_bits_to_f32(wb[v0:v0 + block]).astype(np.float64)).T)
    return np.concatenate(L, axis=1), np.concatenate(A, axis=1)


def check(got, hb, wb, rows):
    H = hb.shape[1]
    L, A = oracle_rows(hb, wb, rows)
    want = np.argmax(L, axis=1)
    gamma = H * 2.0 ** -24
    decided = 0
    for r, n in enumerate(rows):
        tol = gamma * A[r].max()
        top = np.sort(L[r])[-2:] if L.shape[1] > 1 else np.array([-np.inf, L[r, 0]])
        assert 0 <= got[n] < wb.shape[0], f"node {n}: index {got[n]} out of range"
        assert L[r, got[n]] >= top[-1] - 2 * tol, f"node {n}: logit {L[r, got[n]]} vs max {top[-1]} (tol {tol})"
        if top[-1] - top[-2] > 2 * tol:
            assert got[n] == want[r], f"node {n}: {got[n]} != {want[r]} (gap {top[-1] - top[-2]}, tol {tol})"
            decided += 1
    return decided


SMALL = [  # (N, H, V)
    (1, 64, 1), (5, 128, 17), (16, 64, 511), (16, 640, 512), (40, 128, 513), (128, 256, 5000), (130, 64, 3000),
    (300, 128, 1500), (7, 1024, 4096 + 77),
    # up to 112 nodes a workgroup covers 512 vocabulary rows, above that 384:
    # both sides of the switch, with vocabularies ending inside a slab
    (112, 192, 1500), (113, 192, 1500), (127, 128, 385), (97, 64, 513),
]


@pytest.mark.parametrize("N,H,V", SMALL)
def test_small_against_oracle(ttv, N, H, V):
    log(f"lm_head N={N} H={H} V={V}")
    hb, wb = lm_head_inputs(N * 7 + H + V, N, H, V)
    got = run(ttv, hb, wb)
    decided = check(got, hb, wb, list(range(N)))
    assert V == 1 or decided >= N // 2, f"only {decided} of {N} rows decided exactly"


def test_padded_strides(ttv):
    N, H, V = 20, 192, 2000
    hb, wb = lm_head_inputs(8, N, H, V)
    got = run(ttv, hb, wb, hs_pad=8, ws_pad=24)
    assert check(got, hb, wb, list(range(N))) >= N // 2


def test_planted_and_equal_rows(ttv):
    N, H, V = 24, 256, 20000
    plant = {n: (n * 811 + 5) % V for n in range(N)}
    dup = [(plant[0], plant[0] + 1), (plant[3], 2), (plant[7], plant[7] - 1), (plant[9], V - 1)]
    hb, wb = lm_head_inputs(9, N, H, V, planted=plant, duplicate=dup)
    want = O.lm_head_argmax(hb, wb)
    got = run(ttv, hb, wb)
    assert (got == want).all()
    assert want[3] == 2 and want[7] == plant[7] - 1 and want[0] == plant[0]


def test_empty(ttv):
    hb, wb = lm_head_inputs(1, 1, 64, 10)
    out = torch.full((1,), -3, dtype=torch.int32, device="cuda")
    ttv.lm_head_argmax(to_dev(hb, "bf16")[:0], to_dev(wb, "bf16"), out, zeros_ws(1))
    assert to_host(out)[0] == -3


@pytest.mark.parametrize("N", [16, 128])
def test_full_size_sampled(ttv, N):
    # the pages' head: 248,320 vocabulary rows of a 5,120-wide hidden state;
    # planted rows for a few nodes, sampled rows checked against the oracle
    H, V = 5120, V5
    plant = {1: 0, N - 1: V - 1, N // 2: 123457}
    log(f"lm_head full size N={N}")
    hb, wb = lm_head_inputs(100 + N, N, H, V, planted=plant)
    got = run(ttv, hb, wb)
    for n, t in plant.items():
        assert got[n] == t
    rows = sorted(set([0, N // 3, N - 2] + list(rng_for(N, 3).choice(N, size=min(N, 5), replace=False))))
    rows = [n for n in rows if n not in plant]
    assert check(got, hb, wb, rows) >= len(rows) // 2


# ---------------------------------------------------------------------------
# the 4-bit head
# ---------------------------------------------------------------------------

from workloads import lm_head_q4_inputs, lm_head_q4_random  # noqa: E402


def run_q4(ttv, hb, wq, sb, hs_pad=0):
    N, H = hb.shape
    V = wq.shape[0]
    if hs_pad:  # the padding holds NaN: no element past H may be read
        buf = np.full((N, H + hs_pad), 0x7FC0, np.uint16)
        buf[:, :H] = hb
        Xd = to_dev(buf, "bf16")[:, :H]
    else:
        Xd = to_dev(hb, "bf16")
    out = torch.full((max(N, 1),), -3, dtype=torch.int32, device="cuda")
    ws = zeros_ws(ttv.lm_head_q4_argmax_ws(N, V, H))
    ws.fill_(0x5A)
    ttv.lm_head_q4_argmax(Xd, torch.from_numpy(wq.view(np.int32)).to("cuda"), to_dev(sb, "bf16"), out, ws)
    return to_host(out)[:N]


def check_q4(got, hb, wq, sb, rows, block=16384):
    """Exact where the top two float64 logits are further apart than twice
    the bound on the kernel's error, and within the bound everywhere. Bound:
    each group's 64 products accumulate in fp32 (64 roundings) and the group
    is folded into the running logit with one fma (G roundings); each
    group's hidden sum accumulates in fp32 (63 roundings) and enters the bias
    product as three exact bf16 terms, whose 3 G exact products accumulate
    onto the same running logit (3 G roundings). Every rounding is at most
    2^-24 of a partial sum bounded by sum_k |x_k| (s q_k + |b|), so the error
    is at most 2^-24 (64 + 4 G + 8) sum_k |x_k| (s q_k + |b|) (G groups)."""
    H = hb.shape[1]
    G = H // 64
    Xa = np.abs(bf16_bits_to_f32(hb[rows]).astype(np.float64))
    L, A = [], []
    for v0 in range(0, wq.shape[0], block):
        wqb, sbb = wq[v0:v0 + block], sb[:, v0:v0 + block]
        L.append(O.lm_head_q4_logits(hb[rows], wqb, sbb))
        Wv = O.lm_head_q4_weight(wqb, sbb)
        Bv = np.repeat(np.abs(bf16_bits_to_f32(sbb[:, :, 1]).astype(np.float64)).T, 64, axis=1)
        A.append(Xa @ (np.abs(Wv - np.repeat(bf16_bits_to_f32(sbb[:, :, 1]).astype(np.float64).T, 64, axis=1))
                       + Bv).T)
    L, A = np.concatenate(L, axis=1), np.concatenate(A, axis=1)
    want = np.argmax(L, axis=1)
    decided = 0
    for r, n in enumerate(rows):
        tol = 2.0 ** -24 * (64 + 4 * G + 8) * A[r].max()
        top = np.sort(L[r])[-2:]
        assert 0 <= got[n] < wq.shape[0]
        assert L[r, got[n]] >= top[-1] - 2 * tol, f"node {n}: {L[r, got[n]]} vs {top[-1]} (tol {tol})"
        if top[-1] - top[-2] > 2 * tol:
            assert got[n] == want[r], f"node {n}: {got[n]} != {want[r]}"
            decided += 1
    return decided


Q4_SMALL = [(1, 64, 4), (5, 128, 20), (16, 64, 512), (40, 128, 516), (64, 256, 5000), (65, 64, 3000),
            (130, 128, 1500), (7, 1024, 4100), (20, 320, 1000), (32, 192, 772),
            # 65..128 nodes share one slice (32 vocabulary rows per wave): ragged node and row tails
            (100, 192, 2048), (128, 64, 3108), (80, 320, 1000), (257, 64, 516)]


@pytest.mark.parametrize("N,H,V", Q4_SMALL)
def test_q4_small_against_oracle(ttv, N, H, V):
    log(f"lm_head_q4 N={N} H={H} V={V}")
    hb, wq, sb = lm_head_q4_inputs(N * 3 + H + V, N, H, V)
    got = run_q4(ttv, hb, wq, sb)
    assert check_q4(got, hb, wq, sb, list(range(N))) >= N // 2


def test_q4_padded_hidden_stride(ttv):
    N, H, V = 20, 192, 1000
    hb, wq, sb = lm_head_q4_inputs(9, N, H, V)
    got = run_q4(ttv, hb, wq, sb, hs_pad=40)
    assert check_q4(got, hb, wq, sb, list(range(N))) >= N // 2


def test_q4_planted(ttv):
    N, H, V = 24, 256, 20000
    plant = {n: (n * 811 + 5) % V for n in range(N)}
    hb, wq, sb = lm_head_q4_inputs(19, N, H, V, planted=plant)
    assert (run_q4(ttv, hb, wq, sb) == O.lm_head_q4_argmax(hb, wq, sb)).all()
    assert [plant[n] for n in range(N)] == O.lm_head_q4_argmax(hb, wq, sb).tolist()


@pytest.mark.parametrize("N", [16, 128])
def test_q4_full_size_sampled(ttv, N):
    # the pages' head: 248,320 rows of 5,120 four-bit codes (80 groups)
    H, V = 5120, V5
    plant = {0: V - 1, N // 2: 4097, N - 1: 0}
    log(f"lm_head_q4 full size N={N}")
    hb, wq, sb = lm_head_q4_random(200 + N, N, H, V, planted=plant)
    got = run_q4(ttv, hb, wq, sb)
    for n, t in plant.items():
        assert got[n] == t
    rows = sorted(set([1, N // 3, N - 2] + list(rng_for(N, 4).choice(N, size=min(N, 5), replace=False))))
    rows = [n for n in rows if n not in plant]
    assert check_q4(got, hb, wq, sb, rows) >= len(rows) // 2
