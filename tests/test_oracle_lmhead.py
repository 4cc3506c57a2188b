"""Pins of the oracle's greedy prediction from hidden states (summary §2.3:
both views predict greedily): logits = hidden . W^T, argmax with the lowest
index on ties.  Checked against brute force, selector inputs that read one
weight column, planted ties and the orientation of the product."""
import numpy as np

import oracle
import workloads as W


def test_brute_force_small():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((5, 7))
    w = rng.standard_normal((11, 7))
    ref = [max(range(11), key=lambda v: (sum(h[r, k] * w[v, k] for k in range(7)), -v))
           for r in range(5)]
    assert oracle.lmhead_argmax(h, w).tolist() == ref
    np.testing.assert_allclose(oracle.lmhead_logits(h, w, chunk=4), h @ w.T, rtol=1e-14)


def test_one_hot_rows_select_a_weight_column():
    # hidden row r = e_k reads column k of W: the argmax is numpy's first
    # occurrence of that column's maximum
    rng = np.random.default_rng(5)
    w = rng.standard_normal((300, 16))
    ks = [0, 3, 15, 7]
    h = np.zeros((len(ks), 16))
    for r, k in enumerate(ks):
        h[r, k] = 1.0
    assert oracle.lmhead_argmax(h, w).tolist() == [int(np.argmax(w[:, k])) for k in ks]


def test_planted_tie_takes_the_lowest_index_and_scaling_is_invariant():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((200, 8)) * 0.1
    h = rng.standard_normal((3, 8))
    # rows 150 and 40 both equal 10 * h[0]: the largest logit for row 0, twice
    w[150] = w[40] = 10 * h[0]
    got = oracle.lmhead_argmax(h, w)
    assert got[0] == 40
    assert oracle.lmhead_argmax(2.0 * h, w).tolist() == got.tolist()


def test_generator_shapes_and_scale():
    h, w = W.lmhead_inputs(4, 256, 1000, seed=1)
    assert tuple(h.shape) == (4, 256) and tuple(w.shape) == (1000, 256)
    assert abs(float(w.float().std()) - 256 ** -0.5) < 0.01
    h2, w2 = W.lmhead_inputs(4, 256, 1000, seed=1)
    assert h.view(-1).equal(h2.view(-1)) and w.view(-1).equal(w2.view(-1))
