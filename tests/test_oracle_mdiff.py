"""Pins for the oracle's training-time block-mask attention M_diff (CPU only).

The summary's §2.2 states the mask in two rules: a block's positions see the
clean AR context before the block's anchor (causally), and the positions of
one block see each other (bidirectionally).  The oracle is tied to:
  * torch's scaled_dot_product_attention (a library routine) over ONE packed
    problem -- all blocks' queries against [context ++ all blocks' keys] --
    with a dense boolean mask built from the two rules;
  * the decode step it generalises: one block whose anchor is the whole
    context is the diffusion view's block attention;
  * invariants: a context row at or after an anchor is invisible to that
    block; blocks are independent (permuting them permutes the outputs);
    anchor 0 leaves the block alone with itself (a closed-form softmax).
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle

rng = np.random.default_rng(2024)


def rand(*shape):
    return rng.standard_normal(shape)


def make(B=2, NB=3, K=4, Hq=4, Hkv=2, D=16, cap=40, anchors=None):
    if anchors is None:
        anchors = np.sort(rng.integers(0, cap + 1, size=(B, NB)), axis=1)
    return dict(q=rand(B, NB, K, Hq, D), kc=rand(B, Hkv, cap, D), vc=rand(B, Hkv, cap, D),
                kb=rand(B, NB, K, Hkv, D), vb=rand(B, NB, K, Hkv, D),
                anchors=np.asarray(anchors, np.int32))


def run(t, scale=0.25):
    return oracle.mdiff_attn(t["q"], t["kc"], t["vc"], t["anchors"], t["kb"], t["vb"],
                             scale=scale)


def test_equals_library_attention_with_the_dense_mdiff_mask():
    t = make(B=2, NB=3, K=4, Hq=6, Hkv=3, D=16, cap=33,
             anchors=[[0, 7, 33], [12, 12, 30]])
    B, NB, K, Hq, D = t["q"].shape
    Hkv, cap = t["kb"].shape[3], t["kc"].shape[2]
    G = Hq // Hkv
    out, lse = run(t, scale=1 / math.sqrt(D))
    for b in range(B):
        # keys: the context rows, then every block's rows (block-major)
        nq, nk = NB * K, cap + NB * K
        allowed = np.zeros((nq, nk), bool)
        for j in range(NB):
            for i in range(K):
                r = j * K + i
                allowed[r, :t["anchors"][b, j]] = True            # rule 1: t < anchor
                allowed[r, cap + j * K:cap + (j + 1) * K] = True  # rule 2: own block only
        for h in range(Hq):
            g = h // G
            q = torch.from_numpy(t["q"][b, :, :, h].reshape(nq, D))
            k = torch.from_numpy(np.concatenate([t["kc"][b, g],
                                                 t["kb"][b, :, :, g].reshape(NB * K, D)]))
            v = torch.from_numpy(np.concatenate([t["vc"][b, g],
                                                 t["vb"][b, :, :, g].reshape(NB * K, D)]))
            ref = F.scaled_dot_product_attention(q[None], k[None], v[None],
                                                 attn_mask=torch.from_numpy(allowed)[None],
                                                 scale=1 / math.sqrt(D))[0].numpy()
            np.testing.assert_allclose(out[b, :, :, h].reshape(nq, D), ref, rtol=0, atol=1e-12)
            s = (q.numpy() @ k.numpy().T) / math.sqrt(D)
            s[~allowed] = -np.inf
            m = s.max(axis=1)
            ref_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
            np.testing.assert_allclose(lse[b, :, h, :].reshape(nq), ref_lse, rtol=0, atol=1e-12)


def test_one_block_at_the_end_of_the_context_is_the_decode_step():
    # a single block whose anchor is the whole context is the diffusion view
    # of a decode step over that context as the cache (bidirectional block)
    t = make(B=2, NB=1, K=5, Hq=4, Hkv=2, D=8, cap=21, anchors=[[21], [9]])
    out, lse = run(t)
    lens = t["anchors"][:, 0].copy()
    o2, l2 = oracle.block_attn(t["q"][:, 0], t["kc"], t["vc"], t["kb"][:, 0], t["vb"][:, 0],
                               lens, mask=oracle.BIDIR, scale=0.25)
    np.testing.assert_allclose(out[:, 0], o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:, 0], l2, rtol=0, atol=1e-13)


def test_context_at_or_after_the_anchor_is_invisible():
    t = make(B=1, NB=2, K=3, cap=20, anchors=[[5, 14]])
    out, _ = run(t)
    u = {k: v.copy() for k, v in t.items()}
    u["kc"][:, :, 5] += 3.0      # row 5: the anchor of block 0 itself
    u["vc"][:, :, 5] -= 2.0
    o2, _ = run(u)
    np.testing.assert_array_equal(out[0, 0], o2[0, 0])     # block 0: rows t < 5 only
    assert np.abs(out[0, 1] - o2[0, 1]).max() > 1e-3       # block 1 sees row 5
    u = {k: v.copy() for k, v in t.items()}
    u["kc"][:, :, 4] += 3.0      # the last row block 0 sees
    o3, _ = run(u)
    assert np.abs(out[0, 0] - o3[0, 0]).max() > 1e-3


def test_blocks_are_independent():
    t = make(B=1, NB=4, K=3, cap=25)
    out, lse = run(t)
    perm = np.array([2, 0, 3, 1])
    u = dict(t)
    for k in ("q", "kb", "vb"):
        u[k] = t[k][:, perm]
    u["anchors"] = t["anchors"][:, perm]
    o2, l2 = run(u)
    np.testing.assert_array_equal(o2, out[:, perm])
    np.testing.assert_array_equal(l2, lse[:, perm])


def test_anchor_zero_block_attends_only_to_itself():
    t = make(B=1, NB=1, K=3, Hq=2, Hkv=1, D=4, cap=10, anchors=[[0]])
    out, lse = run(t, scale=0.5)
    q, kb, vb = t["q"][0, 0], t["kb"][0, 0, :, 0], t["vb"][0, 0, :, 0]
    for i in range(3):
        for h in range(2):
            s = 0.5 * kb @ q[i, h]
            w = np.exp(s - s.max())
            np.testing.assert_allclose(out[0, 0, i, h], w @ vb / w.sum(), rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, h, i], s.max() + np.log(w.sum()), atol=1e-14)


def test_bad_anchor_rejected():
    t = make(B=1, NB=1, cap=8, anchors=[[9]])
    try:
        run(t)
    except ValueError:
        return
    raise AssertionError("anchor beyond the context was accepted")
