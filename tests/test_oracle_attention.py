"""Pins for the oracle's block attention (CPU only).

Each check ties the oracle to something other than itself: torch's
scaled_dot_product_attention (a library routine) on the special cases the
method reduces to, a hand-derived closed form, and invariants of the
definition (cache-order permutation, constant V, GQA head mapping, block-row
equivariance, paged == contiguous).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
rng = np.random.default_rng(12345)


def rand(*shape):
    return rng.standard_normal(shape)


def make(B=1, K=4, Hq=4, Hkv=2, D=16, L=(13,), cap=None):
    L = np.array(L, np.int32)
    cap = cap or int(L.max()) + K
    return dict(q=rand(B, K, Hq, D), kc=rand(B, Hkv, cap, D), vc=rand(B, Hkv, cap, D),
                kb=rand(B, K, Hkv, D), vb=rand(B, K, Hkv, D), lens=L)


def run(t, mask, scale=0.25, **kw):
    return oracle.block_attn(t["q"], t["kc"], t["vc"], t["kb"], t["vb"], t["lens"],
                             mask=mask, scale=scale, **kw)


def sdpa_row(t, b, i, h, nblk, scale):
    """Library attention for one query over cache rows 0..L-1 + block rows 0..nblk-1."""
    G = t["q"].shape[2] // t["kb"].shape[2]
    g = h // G
    L = int(t["lens"][b])
    keys = np.concatenate([t["kc"][b, g, :L], t["kb"][b, :nblk, g]], 0)
    vals = np.concatenate([t["vc"][b, g, :L], t["vb"][b, :nblk, g]], 0)
    q = torch.from_numpy(t["q"][b, i, h][None, None, None])
    o = F.scaled_dot_product_attention(q, torch.from_numpy(keys)[None, None],
                                       torch.from_numpy(vals)[None, None], scale=scale)
    return o[0, 0, 0].numpy()


@pytest.mark.parametrize("mask", [oracle.BIDIR, oracle.CAUSAL])
def test_k1_is_ordinary_decode_attention(mask):
    # K = 1: the block is the anchor alone, which is plain decode attention over
    # L + 1 keys (both masks coincide).
    t = make(B=2, K=1, Hq=6, Hkv=3, D=32, L=(37, 5))
    out, lse = run(t, mask, scale=1 / math.sqrt(32))
    for b in range(2):
        for h in range(6):
            ref = sdpa_row(t, b, 0, h, 1, 1 / math.sqrt(32))
            np.testing.assert_allclose(out[b, 0, h], ref, rtol=0, atol=1e-12)


def test_causal_row_is_full_attention_over_prefix_and_block_upto_i():
    t = make(B=2, K=6, Hq=4, Hkv=2, D=16, L=(9, 21))
    out, _ = run(t, oracle.CAUSAL)
    for b in range(2):
        for i in range(6):
            for h in range(4):
                ref = sdpa_row(t, b, i, h, i + 1, 0.25)
                np.testing.assert_allclose(out[b, i, h], ref, rtol=0, atol=1e-12)


def test_bidir_row_is_full_attention_over_prefix_and_whole_block():
    t = make(B=2, K=5, Hq=4, Hkv=1, D=8, L=(3, 17))
    out, _ = run(t, oracle.BIDIR)
    for b in range(2):
        for i in range(5):
            for h in range(4):
                ref = sdpa_row(t, b, i, h, 5, 0.25)
                np.testing.assert_allclose(out[b, i, h], ref, rtol=0, atol=1e-12)


def test_lse_is_logsumexp_of_scores():
    from scipy.special import logsumexp
    t = make(B=1, K=3, Hq=2, Hkv=1, D=8, L=(11,))
    for mask in (oracle.BIDIR, oracle.CAUSAL):
        _, lse = run(t, mask, scale=0.5)
        for h in range(2):
            for i in range(3):
                nblk = 3 if mask == oracle.BIDIR else i + 1
                keys = np.concatenate([t["kc"][0, 0, :11], t["kb"][0, :nblk, 0]], 0)
                s = 0.5 * (keys @ t["q"][0, i, h])
                assert abs(lse[0, h, i] - logsumexp(s)) < 1e-12


def test_closed_form_two_keys_golden():
    # Hand-derived: one cache row, one block row, scale 1 (see fixture).
    with open(os.path.join(HERE, "golden", "attn_two_keys.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], float).reshape(1, 1, 1, -1)
    kc = np.array(g["k_cache"], float).reshape(1, 1, 1, -1)
    vc = np.array(g["v_cache"], float).reshape(1, 1, 1, -1)
    kb = np.array(g["k_block"], float).reshape(1, 1, 1, -1)
    vb = np.array(g["v_block"], float).reshape(1, 1, 1, -1)
    for mask in (oracle.BIDIR, oracle.CAUSAL):
        out, lse = oracle.block_attn(q, kc, vc, kb, vb, np.array([1], np.int32), mask=mask,
                                     scale=g["scale"])
        np.testing.assert_allclose(out[0, 0, 0], g["out"], rtol=0, atol=1e-14)
        assert abs(lse[0, 0, 0] - g["lse"]) < 1e-14


def test_cache_order_permutation_invariance():
    t = make(B=1, K=4, Hq=2, Hkv=1, D=16, L=(40,))
    out, lse = run(t, oracle.CAUSAL)
    perm = rng.permutation(40)
    t2 = dict(t)
    t2["kc"] = t["kc"].copy()
    t2["vc"] = t["vc"].copy()
    t2["kc"][:, :, :40] = t["kc"][:, :, perm]
    t2["vc"][:, :, :40] = t["vc"][:, :, perm]
    out2, lse2 = run(t2, oracle.CAUSAL)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mask", [oracle.BIDIR, oracle.CAUSAL])
def test_identical_v_rows_return_that_row(mask):
    t = make(B=2, K=5, Hq=4, Hkv=2, D=8, L=(7, 30))
    v = rand(8)
    t["vc"][:] = v
    t["vb"][:] = v
    out, _ = run(t, mask)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=0, atol=1e-13)


def test_gqa_head_mapping_contiguous_groups():
    # V constant c_g within KV head g: query head h must read head h // G.
    t = make(B=1, K=3, Hq=8, Hkv=2, D=4, L=(10,))
    c = np.array([[1.0, 2.0, 3.0, 4.0], [-5.0, 6.0, -7.0, 8.0]])
    for g in range(2):
        t["vc"][:, g] = c[g]
        t["vb"][:, :, g] = c[g]
    out, _ = run(t, oracle.BIDIR)
    for h in range(8):
        np.testing.assert_allclose(out[0, :, h], np.broadcast_to(c[h // 4], (3, 4)),
                                   rtol=0, atol=1e-13)


def test_causal_last_row_equals_bidir_last_row():
    t = make(B=2, K=7, Hq=4, Hkv=2, D=16, L=(12, 3))
    oc, lc = run(t, oracle.CAUSAL)
    ob, lb = run(t, oracle.BIDIR)
    np.testing.assert_allclose(oc[:, -1], ob[:, -1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lc[:, :, -1], lb[:, :, -1], rtol=0, atol=1e-13)
    assert np.abs(oc[:, 0] - ob[:, 0]).max() > 1e-3      # masks do differ on row 0


def test_bidir_equivariant_under_joint_block_permutation():
    t = make(B=1, K=6, Hq=2, Hkv=1, D=8, L=(9,))
    out, lse = run(t, oracle.BIDIR)
    perm = rng.permutation(6)
    t2 = dict(t, q=t["q"][:, perm], kb=t["kb"][:, perm], vb=t["vb"][:, perm])
    out2, lse2 = run(t2, oracle.BIDIR)
    np.testing.assert_allclose(out2, out[:, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, perm], rtol=0, atol=1e-13)


def test_empty_prefix_attends_block_only():
    t = make(B=1, K=1, Hq=2, Hkv=1, D=8, L=(0,), cap=4)
    for mask in (oracle.BIDIR, oracle.CAUSAL):
        out, lse = run(t, mask)
        np.testing.assert_allclose(out[0, 0], np.broadcast_to(t["vb"][0, 0, 0], (2, 8)),
                                   rtol=0, atol=1e-15)


def test_paged_equals_contiguous():
    B, K, Hq, Hkv, D, ps = 3, 4, 4, 2, 8, 16
    lens = np.array([5, 40, 17], np.int32)
    t = make(B=B, K=K, Hq=Hq, Hkv=Hkv, D=D, L=tuple(lens))
    cap = t["kc"].shape[2]
    maxp = (cap + ps - 1) // ps
    P = B * maxp
    perm = rng.permutation(P)
    table = perm.reshape(B, maxp).astype(np.int32)
    kp = np.zeros((P, Hkv, ps, D))
    vp = np.zeros((P, Hkv, ps, D))
    for b in range(B):
        for tkn in range(cap):
            page, slot = table[b, tkn // ps], tkn % ps
            kp[page, :, slot] = t["kc"][b, :, tkn]
            vp[page, :, slot] = t["vc"][b, :, tkn]
    for mask in (oracle.BIDIR, oracle.CAUSAL):
        oc, lc = run(t, mask)
        op, lp = oracle.block_attn(t["q"], kp, vp, t["kb"], t["vb"], lens, mask=mask,
                                   scale=0.25, layout=oracle.PAGED, page_table=table)
        assert np.array_equal(oc, op) and np.array_equal(lc, lp)


def test_bad_page_index_rejected():
    t = make(B=1, K=2, Hq=2, Hkv=1, D=4, L=(20,))
    kp = np.zeros((2, 1, 16, 4))
    table = np.array([[0, 7]], np.int32)     # page 7 does not exist
    with pytest.raises(ValueError):
        oracle.block_attn(t["q"], kp, kp, t["kb"], t["vb"], t["lens"], mask=0, scale=1.0,
                          layout=oracle.PAGED, page_table=table)
