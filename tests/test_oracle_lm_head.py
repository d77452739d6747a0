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
