"""Pins for the oracle's decode step around the kernels (oracle/model.py),
CPU only: the pieces against library routines and closed forms, the layer
against an independent torch formulation, and the lossless property -- the
Orthrus loop (diffusion candidates, AR verification, consensus, commit)
emits exactly the sequential greedy stream of the AR view."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W
from oracle import model as M

SMALL = M.Dims(H=64, Hq=4, Hkv=2, D=16, I=96, V=50, layers=2, eps=1e-6, theta=1e4)


def test_rmsnorm_matches_the_library():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)) * 3
    w = rng.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(M.rmsnorm(x, w, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rope_is_a_complex_rotation_and_relative():
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal((3, 2, D))
    pos = np.array([0, 7, 123])
    y = M.rope(x, pos, 1e4)
    # (a + i b) * e^{i pos theta^(-2d/D)} for the pair (d, d + D/2)
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(
        1j * pos[:, None, None] * 1e4 ** (-2.0 * np.arange(D // 2) / D))
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # <rope(q, m), rope(k, n)> depends on m - n only
    q, k = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    a = (M.rope(q, [5], 1e4) * M.rope(k, [2], 1e4)).sum()
    b = (M.rope(q, [105], 1e4) * M.rope(k, [102], 1e4)).sum()
    assert abs(a - b) < 1e-11
    np.testing.assert_array_equal(M.rope(x, [0, 0, 0], 1e4), x)


def test_silu_matches_the_library():
    g = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(M.silu(g), F.silu(torch.from_numpy(g)).numpy(), rtol=1e-14,
                               atol=1e-300)


def torch_layer(w, l, view, h, kc, vc, lens, K, mask, d):
    """The same layer written with torch fp64 library calls (rms_norm,
    scaled_dot_product_attention with an explicit mask, silu), one request."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    W_ = {k: t(v.double().numpy()) for k, v in w.items() if k.startswith(f"l{l}.")}
    h = t(h)
    x = F.rms_norm(h, (d.H,), W_[f"l{l}.in_norm"], eps=d.eps)
    qkv = x @ W_[f"l{l}.{view}.wqkv"].T
    q = qkv[:, :d.Hq * d.D].reshape(K, d.Hq, d.D)
    k = qkv[:, d.Hq * d.D:(d.Hq + d.Hkv) * d.D].reshape(K, d.Hkv, d.D)
    v = qkv[:, (d.Hq + d.Hkv) * d.D:].reshape(K, d.Hkv, d.D)
    pos = np.arange(K) + lens
    q = t(M.rope(F.rms_norm(q, (d.D,), W_[f"l{l}.q_norm"], eps=d.eps).numpy(), pos, d.theta))
    k = t(M.rope(F.rms_norm(k, (d.D,), W_[f"l{l}.k_norm"], eps=d.eps).numpy(), pos, d.theta))
    keys = torch.cat([t(kc[0, :, :lens]).permute(1, 0, 2), k], 0)      # [L+K, Hkv, D]
    vals = torch.cat([t(vc[0, :, :lens]).permute(1, 0, 2), v], 0)
    G = d.Hq // d.Hkv
    allowed = torch.ones((K, lens + K), dtype=torch.bool)
    if mask == oracle.CAUSAL:
        allowed[:, lens:] = torch.tril(torch.ones((K, K), dtype=torch.bool))
    o = F.scaled_dot_product_attention(
        q.permute(1, 0, 2), keys.repeat_interleave(G, 1).permute(1, 0, 2),
        vals.repeat_interleave(G, 1).permute(1, 0, 2), attn_mask=allowed,
        scale=d.D ** -0.5).permute(1, 0, 2).reshape(K, d.Hq * d.D)
    h = h + o @ W_[f"l{l}.{view}.wo"].T
    x = F.rms_norm(h, (d.H,), W_[f"l{l}.post_norm"], eps=d.eps)
    gu = x @ W_[f"l{l}.wgu"].T
    return (h + (F.silu(gu[:, :d.I]) * gu[:, d.I:]) @ W_[f"l{l}.wdown"].T).numpy()


@pytest.mark.parametrize("view,mask", [("ar", oracle.CAUSAL), ("diff", oracle.BIDIR)])
def test_layer_equals_an_independent_torch_formulation(view, mask):
    d = SMALL
    w = W.model_weights(d, seed=1)
    m = M.Model(d, w)
    rng = np.random.default_rng(2)
    L, K = 9, 5
    kc = rng.standard_normal((1, d.Hkv, L + K, d.D))
    vc = rng.standard_normal((1, d.Hkv, L + K, d.D))
    h = rng.standard_normal((K, d.H))
    pos = np.arange(K) + L
    got, _, _ = m.layer(0, h, view, kc, vc, np.array([L], np.int32), pos, mask)
    ref = torch_layer(w, 0, view, h, kc, vc, L, K, mask, d)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_causal_block_rows_equal_sequential_rows():
    # the AR view's block pass: row i equals the one-token pass at position
    # lens + i once rows 0..i-1 are in the cache (what makes verification exact)
    d = SMALL
    m = M.Model(d, W.model_weights(d, seed=2), keep_f64=True)
    caches = M.new_caches(d, 1, 64)
    lens, _ = M.prefill(m, [[3, 1, 4, 1, 5, 9, 2]], caches)
    toks = np.array([[6, 5, 3, 5]])
    x_blk, lg_blk, _ = m.forward(toks, "ar", caches, lens, oracle.CAUSAL)
    seq = M.new_caches(d, 1, 64)
    l2, _ = M.prefill(m, [[3, 1, 4, 1, 5, 9, 2]], seq)
    for i in range(4):
        xi, lgi, kv = m.forward(toks[:, i:i + 1], "ar", seq, l2, oracle.CAUSAL)
        np.testing.assert_allclose(lg_blk[i], lgi[0], rtol=1e-11, atol=1e-11)
        l2 = M.append(seq, kv, l2, [1])


@pytest.mark.parametrize("K", [1, 3, 8])
@pytest.mark.parametrize("drafter", ["model", "noisy-greedy"])
def test_orthrus_loop_is_lossless(K, drafter):
    """Emitted stream == sequential greedy decoding of the AR view, whatever
    the diffusion candidates are (the model's own, or the true continuation
    with random corruptions, which exercises long acceptance)."""
    d = SMALL
    m = M.Model(d, W.model_weights(d, seed=3), keep_f64=True)
    prompts = [[1, 2, 3, 4, 5], [7, 7, 8, 9, 10]]
    n_tok = 30
    ref = M.greedy(m, prompts, n_tok + 2 * K + 1, cap=128)
    rng = np.random.default_rng(K)
    caches = M.new_caches(d, 2, 160)
    lens, lg = M.prefill(m, prompts, caches)
    anchor = oracle.argmax_rows(lg)
    streams = [[int(a)] for a in anchor]
    accepted = []
    while min(len(s) for s in streams) < n_tok:
        draft = None
        if drafter == "noisy-greedy":
            draft = np.zeros((2, K), np.int32)
            for b in range(2):
                p = len(streams[b])
                true = ref[b, p:p + K]
                noisy = np.where(rng.random(K) < 0.8, true, rng.integers(0, d.V, K))
                draft[b] = noisy
        emitted, lens, anchor, dd, aa = M.orthrus_step(m, caches, lens, anchor, K, d.V, draft)
        for b in range(2):
            streams[b] += [int(t) for t in emitted[b]]
            accepted.append(len(emitted[b]))
    for b in range(2):
        n = min(len(streams[b]), ref.shape[1])
        assert streams[b][:n] == list(ref[b, :n]), (b, streams[b][:n], list(ref[b, :n]))
    if drafter == "noisy-greedy" and K > 1:
        assert max(accepted) > 1          # long acceptance actually happened
