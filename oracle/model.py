"""fp64 reference of the decode step around the Orthrus kernels.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): the tests, smoke()
and the benchmark's CPU baseline use it; the HIP path never does.

The pages describe one frozen AR Transformer of the Qwen3 family and a light
diffusion module with its own attention, initialised from the AR attention
(agents-report core design); both views read one KV cache (summary §2.1).
Inference (summary §2.3): the diffusion view takes the anchor and K-1
<mask> tokens and projects K candidates in one forward pass (bidirectional
block); the AR view takes the anchor and the first K-1 candidates and
verifies all K positions in one causal pass; consensus keeps the agreed
prefix plus the AR correction, and the accepted AR rows' K/V join the cache.

The layer is the Qwen3 one (the pages name the Qwen3 family; the layer
itself is the plainest reading of that name): RMSNorm, Q/K/V projection,
per-head RMSNorm of q and k, rotary embedding (pairs (d, d + D/2), angle
position * theta^(-2d/D)), attention, output projection + residual,
RMSNorm, SwiGLU MLP + residual; a final RMSNorm and the LM head.  The
diffusion view differs in its Q/K/V and O weights and in the block mask;
its <mask> token is one extra embedding row (index V).

Everything here is fp64 on the exact values of the (bf16) weights: numpy
matrix products and the oracle's fp64 block attention.  No rounding to bf16
anywhere -- that is the GPU path's business.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle


@dataclass
class Dims:
    H: int = 4096          # hidden size
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    I: int = 12288         # MLP intermediate size
    V: int = 151936
    layers: int = 2
    eps: float = 1e-6
    theta: float = 1e6


def f64(t):
    return np.asarray(t.double().numpy() if hasattr(t, "double") else t, dtype=np.float64)


def exact32(t):
    """The weight's values in fp32 (bf16 values are exact there): half the
    memory of fp64 for the large matrices, widened to fp64 per use."""
    return np.asarray(t.float().numpy() if hasattr(t, "float") else t, dtype=np.float32)


def mm(x, w, chunk: int = 8192):
    """x [R, Kin] (fp64) times w^T, w [N, Kin] holding exact values: an fp64
    library matrix product per block of w's rows."""
    if w.dtype == np.float64:
        return x @ w.T
    out = np.empty((x.shape[0], w.shape[0]), np.float64)
    for n0 in range(0, w.shape[0], chunk):
        out[:, n0:n0 + chunk] = x @ w[n0:n0 + chunk].astype(np.float64).T
    return out


def rmsnorm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope(x, pos, theta):
    """Rotary embedding of x [R, heads, D] at positions pos [R]: the pair
    (d, d + D/2) is rotated by the angle pos * theta^(-2d/D)."""
    D = x.shape[-1]
    d = np.arange(D // 2)
    ang = np.asarray(pos, np.float64)[:, None] * theta ** (-2.0 * d / D)     # [R, D/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(g):
    return g / (1.0 + np.exp(-g))


class Model:
    """fp64 copy of one random-weight model (weights: a dict of torch bf16
    tensors, see workloads.model_weights)."""

    def __init__(self, dims: Dims, weights: dict, keep_f64: bool = False):
        """keep_f64: hold every weight in fp64 (faster repeated passes, twice
        the memory of the default fp32 copies)."""
        self.d = dims
        self.w = {k: (f64(v) if keep_f64 else exact32(v)) for k, v in weights.items()}

    def layer(self, l, h, view, kc, vc, lens, pos, mask):
        """One layer over the block rows h [B*K, H] of B requests (K rows
        each, positions pos [B*K]) against the caches kc, vc [B, Hkv, cap, D]
        with lens [B].  Returns (h', k_blk, v_blk) with k_blk, v_blk
        [B, K, Hkv, D] (the rows' own keys/values, post-rotary)."""
        d, w = self.d, self.w
        B = len(lens)
        K = h.shape[0] // B
        x = rmsnorm(h, w[f"l{l}.in_norm"].astype(np.float64), d.eps)
        qkv = mm(x, w[f"l{l}.{view}.wqkv"])
        q = qkv[:, :d.Hq * d.D].reshape(-1, d.Hq, d.D)
        k = qkv[:, d.Hq * d.D:(d.Hq + d.Hkv) * d.D].reshape(-1, d.Hkv, d.D)
        v = qkv[:, (d.Hq + d.Hkv) * d.D:].reshape(-1, d.Hkv, d.D)
        q = rope(rmsnorm(q, w[f"l{l}.q_norm"].astype(np.float64), d.eps), pos, d.theta)
        k = rope(rmsnorm(k, w[f"l{l}.k_norm"].astype(np.float64), d.eps), pos, d.theta)
        kb, vb = k.reshape(B, K, d.Hkv, d.D), v.reshape(B, K, d.Hkv, d.D)
        o, _ = oracle.block_attn(q.reshape(B, K, d.Hq, d.D), kc, vc, kb, vb, lens, mask=mask,
                                 scale=d.D ** -0.5)
        h = h + mm(o.reshape(B * K, d.Hq * d.D), w[f"l{l}.{view}.wo"])
        x = rmsnorm(h, w[f"l{l}.post_norm"].astype(np.float64), d.eps)
        gu = mm(x, w[f"l{l}.wgu"])
        h = h + mm(silu(gu[:, :d.I]) * gu[:, d.I:], w[f"l{l}.wdown"])
        return h, kb, vb

    def forward(self, tokens, view, caches, lens, mask):
        """Both views' pass over a block: tokens [B, K] at positions lens[b] +
        i; caches: per layer (kc, vc) [B, Hkv, cap, D].  Returns (final
        normed hidden [B*K, H], logits [B*K, V], per-layer (k_blk, v_blk))."""
        d, w = self.d, self.w
        B, K = tokens.shape
        pos = (np.asarray(lens)[:, None] + np.arange(K)[None, :]).reshape(-1)
        h = w["embed"][np.asarray(tokens).reshape(-1)].astype(np.float64)
        kv = []
        for l in range(d.layers):
            kc, vc = caches[l]
            h, kb, vb = self.layer(l, h, view, kc, vc, lens, pos, mask)
            kv.append((kb, vb))
        x = rmsnorm(h, w["final_norm"].astype(np.float64), d.eps)
        return x, mm(x, w["lm_head"]), kv


def new_caches(dims: Dims, B: int, cap: int):
    return [(np.zeros((B, dims.Hkv, cap, dims.D)), np.zeros((B, dims.Hkv, cap, dims.D)))
            for _ in range(dims.layers)]


def append(caches, kv, lens, n):
    """Rows 0..n[b]-1 of every layer's block keys/values at cache rows
    lens[b].. (the commit; summary §2.3 step 3)."""
    for (kc, vc), (kb, vb) in zip(caches, kv):
        for b in range(len(lens)):
            for i in range(int(n[b])):
                kc[b, :, lens[b] + i] = kb[b, i]
                vc[b, :, lens[b] + i] = vb[b, i]
    return np.asarray(lens) + np.asarray(n)


def prefill(model: Model, prompts, caches, chunk: int = 64):
    """The AR view over the prompts [B, P] in causal blocks of up to `chunk`
    rows, every row appended.  Returns (lens, last row's logits [B, V])."""
    prompts = np.asarray(prompts)
    B, P = prompts.shape
    lens = np.zeros(B, np.int32)
    logits = None
    for s in range(0, P, chunk):
        blk = prompts[:, s:s + chunk]
        _, lg, kv = model.forward(blk, "ar", caches, lens, oracle.CAUSAL)
        lens = append(caches, kv, lens, np.full(B, blk.shape[1]))
        logits = lg.reshape(B, blk.shape[1], -1)[:, -1]
    return lens, logits


def greedy(model: Model, prompts, steps: int, cap: int):
    """Sequential greedy decoding with the AR view (one token per forward):
    returns the generated tokens [B, steps] (the first is the prefill's)."""
    caches = new_caches(model.d, len(prompts), cap)
    lens, lg = prefill(model, prompts, caches)
    tok = oracle.argmax_rows(lg)
    out = [tok]
    for _ in range(steps - 1):
        _, lg, kv = model.forward(tok[:, None], "ar", caches, lens, oracle.CAUSAL)
        lens = append(caches, kv, lens, np.ones(len(lens), np.int32))
        tok = oracle.argmax_rows(lg)
        out.append(tok)
    return np.stack(out, axis=1)


def orthrus_step(model: Model, caches, lens, anchor, K: int, mask_token: int, draft=None):
    """One Orthrus decode step (summary §2.3).  anchor [B]: the last emitted
    token, not yet in the cache.  The diffusion view projects K candidates
    from [anchor, <mask> x (K-1)] (bidirectional block); draft [B, K], if
    given, replaces them (a stand-in drafter, to exercise long acceptance);
    the AR view verifies [anchor, d_0..d_{K-2}] (causal block); consensus;
    the accepted AR rows' K/V are appended.  Returns (emitted tokens per
    request, new lens, next anchor, d, a)."""
    B = len(lens)
    blk = np.full((B, K), mask_token, np.int64)
    blk[:, 0] = anchor
    _, lg_d, _ = model.forward(blk, "diff", caches, lens, oracle.BIDIR)
    d = oracle.argmax_rows(lg_d).reshape(B, K)
    if draft is not None:
        d = np.asarray(draft, np.int32)
    ar_in = np.concatenate([np.asarray(anchor)[:, None], d[:, :K - 1]], axis=1)
    _, lg_a, kv = model.forward(ar_in, "ar", caches, lens, oracle.CAUSAL)
    a = oracle.argmax_rows(lg_a).reshape(B, K)
    r = oracle.consensus(d, a)
    lens = append(caches, kv, lens, r["n"])
    emitted = [r["emitted"][r["emit_off"][b]:r["emit_off"][b + 1]] for b in range(B)]
    return emitted, lens, r["next_anchor"], d, a
