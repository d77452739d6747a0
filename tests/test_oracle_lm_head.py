"""Pins of the oracle's LM-head projection and fused argmax against a
brute force with exactly rounded sums, planted winners, equal rows, and the
plain argmax over materialised logits."""

import math

import numpy as np

import oracle as O
from workloads import bf16_bits_to_f32, lm_head_inputs


def test_brute_force_exact_sums():
    # tiny, non-square: rows of fsum-exact dot products, then Python's max/index
    N, H, V = 3, 40, 23
    hb, wb = lm_head_inputs(1, N, H, V)
    X = bf16_bits_to_f32(hb).astype(float).tolist()
    W = bf16_bits_to_f32(wb).astype(float).tolist()
    L = O.lm_head_logits(hb, wb)
    assert L.shape == (N, V)
    for n in range(N):
        row = [math.fsum(X[n][i] * W[v][i] for i in range(H)) for v in range(V)]
        np.testing.assert_allclose(L[n], row, rtol=1e-13, atol=1e-13)
        assert O.lm_head_argmax(hb, wb)[n] == row.index(max(row))


def test_planted_winners():
    N, H, V = 6, 256, 5000
    plant = {0: 4999, 1: 0, 2: 1234, 3: 1235, 4: 77, 5: 4096}
    hb, wb = lm_head_inputs(2, N, H, V, planted=plant)
    assert O.lm_head_argmax(hb, wb).tolist() == [plant[n] for n in range(N)]


def test_equal_rows_go_to_the_lower_index():
    N, H, V = 4, 128, 3000
    plant = {0: 2500, 1: 10, 2: 2999, 3: 1500}
    hb, wb = lm_head_inputs(3, N, H, V, planted=plant, duplicate=[(2500, 2501), (2999, 5), (1500, 1499)])
    # row 2501 equals 2500 (2500 wins); row 5 equals 2999 (5 wins); 1499 equals 1500 (1499 wins)
    assert O.lm_head_argmax(hb, wb).tolist() == [2500, 10, 5, 1499]


def test_fused_equals_argmax_of_materialised_logits():
    N, H, V = 8, 512, 20000
    hb, wb = lm_head_inputs(4, N, H, V)
    L = O.lm_head_logits(hb, wb)
    s = np.sort(L, axis=1)
    assert (s[:, -1] - s[:, -2] > 1e-6).all()  # no near ties: float32 rounding keeps the order
    assert (O.lm_head_argmax(hb, wb) == O.vocab_argmax(L.astype(np.float32))).all()
    # the logits have unit variance under this recipe
    assert 0.8 < L.std() < 1.2


# ---------------------------------------------------------------------------
# the 4-bit head (affine, groups of 64)
# ---------------------------------------------------------------------------

from workloads import lm_head_q4_inputs, quantize_q4_groups, to_bf16_bits  # noqa: E402


def test_q4_unpacking_brute_force():
    # every element's code read bit by bit from its word, times its group's
    # scale plus bias, on a tiny non-square head
    V, H = 5, 128
    rng = np.random.default_rng(3)
    wq = rng.integers(0, 2 ** 32, size=(V, H // 8), dtype=np.uint64).astype(np.uint32)
    sb = to_bf16_bits(rng.standard_normal((H // 64, V, 2)).astype(np.float32))
    W = O.lm_head_q4_weight(wq, sb)
    for v in range(V):
        for i in range(H):
            word = int(wq[v, i // 8])
            code = sum(((word >> (4 * (i % 8) + bit)) & 1) << bit for bit in range(4))
            sc = float(bf16_bits_to_f32(sb[i // 64, v, 0]))
            bi = float(bf16_bits_to_f32(sb[i // 64, v, 1]))
            assert W[v, i] == sc * code + bi


def test_q4_equals_bf16_head_when_exact():
    # scale 1/16 and bias -1/2 make every value (code - 8) / 16 exactly a
    # bf16 number: the 4-bit head then equals the bf16 head of those values
    N, V, H = 6, 700, 256
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, size=(V, H)).astype(np.uint32)
    wq = np.zeros((V, H // 8), np.uint32)
    for j in range(8):
        wq |= codes[:, j::8] << np.uint32(4 * j)
    sb = np.zeros((H // 64, V, 2), np.uint16)
    sb[:, :, 0] = to_bf16_bits(np.float32(1 / 16))
    sb[:, :, 1] = to_bf16_bits(np.float32(-0.5))
    wb = to_bf16_bits(((codes.astype(np.float32) - 8) / 16).astype(np.float32))
    hb = to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    np.testing.assert_array_equal(O.lm_head_q4_logits(hb, wq, sb), O.lm_head_logits(hb, wb))
    assert (O.lm_head_q4_argmax(hb, wq, sb) == O.lm_head_argmax(hb, wb)).all()


def test_q4_quantiser_bounds_and_planted_winners():
    N, H, V = 5, 256, 4000
    plant = {0: 3999, 1: 0, 2: 777, 3: 2048, 4: 1}
    hb, wq, sb = lm_head_q4_inputs(5, N, H, V, planted=plant)
    assert O.lm_head_q4_argmax(hb, wq, sb).tolist() == [plant[n] for n in range(N)]
    # reconstruction error within half a step (plus the bf16 rounding of scale and bias)
    W = np.random.default_rng(6).standard_normal((40, H)).astype(np.float32)
    wq2, sb2 = quantize_q4_groups(W)
    R = O.lm_head_q4_weight(wq2, sb2)
    step = np.repeat(bf16_bits_to_f32(sb2[:, :, 0]).T, 64, axis=1)
    assert (np.abs(R - W) <= 0.5 * step + 0.02 * np.abs(W) + 1e-6).all()
    # fsum-exact logits of a tiny case
    hb3, wq3, sb3 = lm_head_q4_inputs(7, 2, 64, 9)
    L = O.lm_head_q4_logits(hb3, wq3, sb3)
    Wt = O.lm_head_q4_weight(wq3, sb3).tolist()
    X = bf16_bits_to_f32(hb3).astype(float).tolist()
    for n in range(2):
        row = [math.fsum(X[n][i] * Wt[v][i] for i in range(64)) for v in range(9)]
        np.testing.assert_allclose(L[n], row, rtol=1e-13, atol=1e-13)
