"""Pins for the oracle's argmax, consensus and KV append (CPU only).

* argmax: numpy.argmax (documented to return the first occurrence of the
  maximum) and brute force over tiny arrays with ties, signed zeros and -inf.
* consensus: exhaustive enumeration of tiny token arrays against two
  formulations written independently of the oracle's scan, hand-worked cases
  (tests/golden/consensus_cases.json) and special cases.
* append: sentinel-filled caches (only the accepted rows change), paged
  placement, lens_out, and the losslessness loop in test_oracle_lossless.py.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
rng = np.random.default_rng(777)


# ---------------------------------------------------------------- argmax

def test_argmax_matches_numpy_first_occurrence():
    x = rng.standard_normal((50, 1001))
    x[3, 10] = x[3, 900] = 99.0                  # tie: first wins
    x[7, -1] = 50.0                              # max at the last index
    np.testing.assert_array_equal(oracle.argmax_rows(x), np.argmax(x, axis=1))


def test_argmax_bf16_ties_match_numpy():
    import torch
    xb = torch.randn(200, 151936, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    x = xb.double().numpy()
    got = oracle.argmax_rows(x)
    np.testing.assert_array_equal(got, np.argmax(x, axis=1))
    ties = sum(int((x[r] == x[r].max()).sum() > 1) for r in range(200))
    assert ties > 0                               # bf16 rows at this width do tie


def test_argmax_bruteforce_tiny_with_signed_zero_and_inf():
    vals = [-np.inf, -1.0, -0.0, 0.0, 1.0]
    for V in range(1, 5):
        for combo in itertools.product(vals, repeat=V):
            x = np.array(combo)
            best = [v for v in range(V) if all(x[v] >= x[u] for u in range(V))][0]
            assert oracle.argmax_rows(x[None])[0] == best, combo


def test_argmax_rejects_nan():
    with pytest.raises(ValueError):
        oracle.argmax_rows(np.array([[0.0, np.nan, 1.0]]))


# ---------------------------------------------------------------- consensus

def accept_len_leading(d, a):
    """1 + number of leading matches, capped at K."""
    K = len(d)
    m = 0
    for x, y in zip(d, a):
        if x != y:
            break
        m += 1
    return min(m + 1, K)


def accept_len_largest(d, a):
    """Largest n <= K such that d[i] == a[i] for every i < n - 1."""
    K = len(d)
    return max(n for n in range(1, K + 1) if all(d[i] == a[i] for i in range(n - 1)))


def test_consensus_exhaustive_tiny():
    for K in range(1, 5):
        for V in range(1, 4):
            seqs = list(itertools.product(range(V), repeat=K))
            pairs = [(d, a) for d in seqs for a in seqs]
            d = np.array([p[0] for p in pairs], np.int32)
            a = np.array([p[1] for p in pairs], np.int32)
            r = oracle.consensus(d, a)
            off = 0
            for b, (db, ab) in enumerate(pairs):
                n1, n2 = accept_len_leading(db, ab), accept_len_largest(db, ab)
                assert n1 == n2 == r["n"][b]
                j = next((i for i in range(K) if db[i] != ab[i]), K)
                assert r["j"][b] == j
                assert r["emit_off"][b] == off
                em = list(r["emitted"][off:off + n1])
                # emitted = accepted candidates, then the AR correction
                want = list(db[:j]) + ([ab[j]] if j < K else [])
                assert em == want[:n1] == list(ab[:n1])
                assert r["next_anchor"][b] == ab[n1 - 1]
                off += n1
            assert r["emit_off"][-1] == off


def test_consensus_special_cases():
    r = oracle.consensus(np.array([[4]]), np.array([[9]]))          # K = 1
    assert r["n"][0] == 1 and list(r["emitted"]) == [9]
    r = oracle.consensus(np.array([[1, 2, 3]]), np.array([[0, 2, 3]]))  # first differs
    assert r["n"][0] == 1 and r["j"][0] == 0 and list(r["emitted"]) == [0]
    r = oracle.consensus(np.array([[1, 2, 3]]), np.array([[1, 2, 3]]))  # all match
    assert r["n"][0] == 3 and r["j"][0] == 3 and list(r["emitted"]) == [1, 2, 3]


def test_consensus_golden_cases():
    with open(os.path.join(HERE, "golden", "consensus_cases.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        r = oracle.consensus(np.array(case["d"], np.int32), np.array(case["a"], np.int32))
        assert r["j"].tolist() == case["j"], case["name"]
        assert r["n"].tolist() == case["n"], case["name"]
        assert r["emit_off"].tolist() == case["emit_off"], case["name"]
        assert r["emitted"].tolist() == case["emitted"], case["name"]
        assert r["next_anchor"].tolist() == case["next_anchor"], case["name"]


# ---------------------------------------------------------------- append

SENT = -12345


def test_append_contiguous_sentinel_tail():
    layers, B, K, Hkv, D, cap = 3, 4, 5, 2, 3, 20
    lens = np.array([0, 7, 15, 3], np.int32)
    n = np.array([5, 1, 5, 2], np.int32)
    kc = np.full((layers, B, Hkv, cap, D), SENT, np.int32)
    vc = np.full((layers, B, Hkv, cap, D), SENT - 1, np.int32)
    kb = rng.integers(0, 1000, (layers, B, K, Hkv, D)).astype(np.int32)
    vb = rng.integers(0, 1000, (layers, B, K, Hkv, D)).astype(np.int32)
    k2, v2, lo = oracle.kv_append(kc, vc, kb, vb, n, lens)
    np.testing.assert_array_equal(lo, lens + n)
    for l in range(layers):
        for b in range(B):
            for t in range(cap):
                i = t - lens[b]
                if 0 <= i < n[b]:
                    np.testing.assert_array_equal(k2[l, b, :, t], kb[l, b, i])
                    np.testing.assert_array_equal(v2[l, b, :, t], vb[l, b, i])
                else:
                    assert (k2[l, b, :, t] == SENT).all() and (v2[l, b, :, t] == SENT - 1).all()


def test_append_paged_placement():
    layers, B, K, Hkv, D, ps = 2, 3, 4, 2, 2, 16
    lens = np.array([14, 0, 31], np.int32)
    n = np.array([4, 2, 3], np.int32)
    maxp = 3
    P = B * maxp
    table = rng.permutation(P).reshape(B, maxp).astype(np.int32)
    kc = np.full((layers, P, Hkv, ps, D), SENT, np.int16)
    vc = np.full((layers, P, Hkv, ps, D), SENT, np.int16)
    kb = rng.integers(0, 1000, (layers, B, K, Hkv, D)).astype(np.int16)
    vb = rng.integers(0, 1000, (layers, B, K, Hkv, D)).astype(np.int16)
    k2, v2, lo = oracle.kv_append(kc, vc, kb, vb, n, lens, layout=oracle.PAGED, page_table=table)
    np.testing.assert_array_equal(lo, lens + n)
    touched = np.zeros((P, ps), bool)
    for b in range(B):
        for i in range(n[b]):
            t = lens[b] + i
            page, slot = table[b, t // ps], t % ps
            touched[page, slot] = True
            for l in range(layers):
                np.testing.assert_array_equal(k2[l, page, :, slot], kb[l, b, i])
                np.testing.assert_array_equal(v2[l, page, :, slot], vb[l, b, i])
    for l in range(layers):
        for page in range(P):
            for slot in range(ps):
                if not touched[page, slot]:
                    assert (k2[l, page, :, slot] == SENT).all()
                    assert (v2[l, page, :, slot] == SENT).all()


def test_append_rejects_overflow_and_bad_n():
    kc = np.zeros((1, 1, 1, 4, 2), np.int32)
    kb = np.zeros((1, 1, 3, 1, 2), np.int32)
    with pytest.raises(ValueError):
        oracle.kv_append(kc, kc, kb, kb, np.array([3], np.int32), np.array([2], np.int32))
    with pytest.raises(ValueError):
        oracle.kv_append(kc, kc, kb, kb, np.array([4], np.int32), np.array([0], np.int32))
