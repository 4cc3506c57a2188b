"""The Orthrus decode step on the GPU, end to end, over the C ABI.

A random-weight Qwen3-style model (the layer is described at
orthrus_gemm in include/orthrus.h) drives the library's kernels through one
decode step (the Orthrus summary's §2.3):

 1. the diffusion view's pass over [anchor, <mask> x (K-1)] with its own
    attention weights and the bidirectional block (orthrus_block_attn,
    BIDIR) -> K candidates d (orthrus_lmhead_argmax);
 2. the AR view's pass over [anchor, d_0 .. d_{K-2}] with the frozen weights
    and the causal block -> the AR tokens a, and each layer's block K/V;
 3. orthrus_consensus_tokens(d, a) -> accepted count n and the next anchor;
    orthrus_kv_append of the AR block rows 0..n-1 of every layer, in place.

Every step runs in the library's kernels: this module only allocates torch
buffers and marshals arguments; nothing is computed with torch.  A step
never synchronises with the host (it can be captured in a HIP graph).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _binding as B_
from . import api


@dataclass
class Dims:
    H: int = 4096
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    I: int = 12288
    V: int = 151936
    layers: int = 2
    eps: float = 1e-6
    theta: float = 1e6


def _ok(fn, st):
    B_.check(fn, st)


# prompt rows per prefill block (the block attention takes up to 64 rows)
PREFILL_CHUNK = 64


_PACKED = (".wqkv", ".wo", ".wgu", ".wdown", "lm_head")


class DecodeModel:
    """Weights on the GPU plus per-batch buffers.  The row buffers hold a
    block of B x max(K, PREFILL_CHUNK) rows: a decode block, or one prefill
    block of the prompt."""

    def __init__(self, dims: Dims, weights: dict, B: int, K: int, cap: int, device="cuda"):
        self.d, self.B, self.K, self.cap = dims, B, K, cap
        dev = torch.device(device)
        # the projection and LM-head matrices in the packed tile layout the
        # weight-streaming kernels read (packed once, here)
        self.w = {}
        for k, v in weights.items():
            t = v.to(dev).contiguous()
            if k.endswith(".wgu"):
                self.w[k] = api.pack_weight_gate_up(t)   # SwiGLU in the projection
            else:
                self.w[k] = api.pack_weight(t) if k.endswith(_PACKED) else t
        d = dims
        self.mask_token = d.V                      # the extra embedding row
        R = B * max(K, PREFILL_CHUNK)              # rows of the largest block
        self.R_max = R
        f32 = dict(dtype=torch.float32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        nqkv = (d.Hq + 2 * d.Hkv) * d.D
        # caches of all layers in one block each (the multi-layer append)
        self.kc = torch.zeros((d.layers, B, d.Hkv, cap, d.D), **bf)
        self.vc = torch.zeros_like(self.kc)
        self.lens = torch.zeros(B, **i32)
        # host-side upper bound on every request's length, so that no append
        # can pass the caches' capacity (checked before anything is launched)
        self.upper = 0
        self.caches = [api.make_cache(self.kc[l], self.vc[l], self.lens, max_len=cap)
                       for l in range(d.layers)]
        # the AR pass's block K/V of every layer (the rows an append commits)
        self.kb = torch.empty((d.layers, B, K, d.Hkv, d.D), **bf)
        self.vb = torch.empty_like(self.kb)
        self.kb_scratch = torch.empty((B, K, d.Hkv, d.D), **bf)   # the diffusion view's
        self.vb_scratch = torch.empty_like(self.kb_scratch)
        self.h = torch.empty((R, d.H), **f32)
        self.x = torch.empty((R, d.H), **bf)
        self.q = torch.empty((B, K, d.Hq, d.D), **bf)
        self.o = torch.empty((B, K, d.Hq, d.D), **bf)
        self.lse = torch.empty((B, d.Hq, K), **f32)
        self.act = torch.empty((R, d.I), **bf)
        self.tok = torch.empty((B, K), **i32)          # a decode block
        self.d_tok = torch.empty((B, K), **i32)
        self.a_tok = torch.empty((B, K), **i32)
        self.anchor = torch.zeros(B, **i32)
        self.n_match = torch.empty(B, **i32)
        self.n_emit = torch.empty(B, **i32)
        self.emit_off = torch.empty(B + 1, **i32)
        self.emitted = torch.empty(B * K, **i32)
        # the projections' partial sums (each projection's epilogue reads them)
        gws = max(B_.orthrus_gemm_epilogue_workspace_bytes(R, n, k) for n, k in
                  ((nqkv, d.H), (d.H, d.Hq * d.D), (2 * d.I, d.H), (d.H, d.I)))
        self.gws = torch.empty(max(gws, 16), dtype=torch.uint8, device=dev)
        self.aws, _ = api.block_attn_workspace(self.caches[0], B, K, d.Hq, d.Hkv, d.D, B_.BF16,
                                               0, dev)
        lmn = B_.orthrus_lmhead_argmax_workspace_bytes(B * K, d.H, d.V, B_.BF16)
        self.lws = torch.empty(max(lmn, 8), dtype=torch.uint8, device=dev)
        self.views_attn = {}

    # ------------------------------------------------------------ kernels
    def _layer(self, l, view, mask, kb, vb, K, next_norm):
        """Layer l on the block rows, whose normed input x = rmsnorm(h) the
        previous projection's epilogue wrote; ends with x = next_norm(h)."""
        d, w = self.d, self.w
        R = self.B * K
        h, x = self.h[:R], self.x[:R]
        ws, wn = self.gws, self.gws.numel()
        q = self.q[:, :K] if K == self.K else torch.empty((self.B, K, d.Hq, d.D),
                                                          dtype=torch.bfloat16,
                                                          device=self.h.device)
        _ok("orthrus_gemm_qk_norm_rope",
            B_.orthrus_gemm_qk_norm_rope(x, w[f"l{l}.{view}.wqkv"], w[f"l{l}.q_norm"],
                                         w[f"l{l}.k_norm"], self.lens, K, q, kb, vb, R, d.Hq,
                                         d.Hkv, d.D, d.H, d.eps, d.theta, ws, wn))
        o = self.o if K == self.K else torch.empty_like(q)
        lse = self.lse if K == self.K else torch.empty((self.B, d.Hq, K), dtype=torch.float32,
                                                       device=self.h.device)
        api.block_attn(q, kb, vb, self.caches[l], mask=mask, scale=d.D ** -0.5, out=o, lse=lse,
                       workspace=self.aws if K == self.K else None)
        # h += o Wo^T (in place), x = post_norm(h); then the MLP
        _ok("orthrus_gemm_rmsnorm",
            B_.orthrus_gemm_rmsnorm(o.view(R, d.Hq * d.D), w[f"l{l}.{view}.wo"], h,
                                    w[f"l{l}.post_norm"], x, R, d.H, d.Hq * d.D, d.eps, ws, wn))
        _ok("orthrus_gemm_swiglu",
            B_.orthrus_gemm_swiglu(x, w[f"l{l}.wgu"], self.act[:R], R, d.I, d.H, ws, wn))
        _ok("orthrus_gemm_rmsnorm",
            B_.orthrus_gemm_rmsnorm(self.act[:R], w[f"l{l}.wdown"], h, next_norm, x, R, d.H, d.I,
                                    d.eps, ws, wn))

    def forward(self, tokens, view, mask, kv_out=None, idx=None):
        """One view's pass over the block tokens [B, K'] (device int32) at
        positions lens[b] + i.  kv_out: (k, v) per layer [B, K', Hkv, D] to
        keep the block K/V (the AR view), else scratch.  Writes the greedy
        tokens to idx [B, K'] and returns the final normed hidden rows."""
        d, w = self.d, self.w
        B, K = tokens.shape
        R = B * K
        # every row buffer below is sliced to R rows: never beyond its size
        if B != self.B or R > self.R_max:
            raise ValueError(f"a block of {B} x {K} rows does not fit the {self.R_max}-row "
                             f"buffers of this {self.B}-request model")
        _ok("orthrus_embed", B_.orthrus_embed(tokens, w["embed"], self.h[:R], R, d.H))
        x = self.x[:R]
        _ok("orthrus_rmsnorm", B_.orthrus_rmsnorm(self.h[:R], w["l0.in_norm"], x, R, d.H, d.eps))
        for l in range(d.layers):
            if kv_out is not None:
                kb, vb = kv_out[l]
            elif K == self.K:
                kb, vb = self.kb_scratch, self.vb_scratch
            else:
                kb = torch.empty((B, K, d.Hkv, d.D), dtype=torch.bfloat16, device=self.h.device)
                vb = torch.empty_like(kb)
            nxt = w[f"l{l + 1}.in_norm"] if l + 1 < d.layers else w["final_norm"]
            self._layer(l, view, mask, kb, vb, K, nxt)
        if idx is not None:
            api.lmhead_argmax(x, w["lm_head"], idx=idx.view(-1),
                              workspace=self.lws if K == self.K else None)
        return x

    def _reserve(self, rows: int):
        if self.upper + rows > self.cap:
            raise ValueError(f"{rows} more rows could pass the cache capacity {self.cap} "
                             f"(up to {self.upper} used)")

    def sync_lengths(self):
        """Tighten the host-side bound to the true lengths (a device read)."""
        self.upper = int(self.lens.max())

    def set_lengths(self, L: int):
        """All requests' caches hold L rows (filled by the caller)."""
        self._reserve(L - self.upper)
        self.lens.fill_(L)
        self.upper = L

    # -------------------------------------------------------- the method
    def prefill(self, prompts, chunk: int = PREFILL_CHUNK):
        """The AR view over the prompts [B, P] (device int32) in causal blocks
        of up to `chunk` rows, all appended; the anchor becomes the greedy
        token after the prompt."""
        d = self.d
        B, P = prompts.shape
        self._reserve(P)
        for s in range(0, P, chunk):
            blk = prompts[:, s:s + chunk].contiguous()
            k = blk.shape[1]
            kv = [(torch.empty((B, k, d.Hkv, d.D), dtype=torch.bfloat16, device=blk.device),
                   torch.empty((B, k, d.Hkv, d.D), dtype=torch.bfloat16, device=blk.device))
                  for _ in range(d.layers)]
            idx = torch.empty((B, k), dtype=torch.int32, device=blk.device)
            self.forward(blk, "ar", B_.CAUSAL, kv_out=kv, idx=idx)
            n = torch.full((B,), k, dtype=torch.int32, device=blk.device)
            for l in range(d.layers):
                api.kv_append(self.caches[l], kv[l][0], kv[l][1], n, lens_out=self.lens
                              if l == d.layers - 1 else torch.empty_like(self.lens))
            self.anchor.copy_(idx[:, -1])
        self.upper += P

    def greedy_step(self):
        """Plain AR decoding of one token: the anchor's pass (K = 1), its K/V
        appended, the next anchor its greedy token."""
        d = self.d
        B = self.B
        self._reserve(1)
        tok = self.anchor.view(B, 1).clone()
        kv = [(torch.empty((B, 1, d.Hkv, d.D), dtype=torch.bfloat16, device=tok.device),
               torch.empty((B, 1, d.Hkv, d.D), dtype=torch.bfloat16, device=tok.device))
              for _ in range(d.layers)]
        idx = torch.empty((B, 1), dtype=torch.int32, device=tok.device)
        self.forward(tok, "ar", B_.CAUSAL, kv_out=kv, idx=idx)
        one = torch.ones(B, dtype=torch.int32, device=tok.device)
        for l in range(d.layers):
            api.kv_append(self.caches[l], kv[l][0], kv[l][1], one,
                          lens_out=self.lens if l == d.layers - 1 else torch.empty_like(self.lens))
        self.anchor.copy_(idx[:, 0])
        self.upper += 1
        return tok.view(-1)

    def orthrus_step(self, draft=None, keep_hidden=False, advance=True):
        """One Orthrus step (module doc).  draft [B, K] (device int32), if
        given, replaces the diffusion view's candidates (the diffusion pass
        still runs).  Outputs: n_emit, emit_off, emitted (packed), anchor.
        keep_hidden: also keep both views' final normed hidden rows
        (x_diff, x_ar; a copy, for inspection).  advance=False writes the new
        lengths to lens_next instead of lens (the accepted rows are still
        written), so that a replayed step repeats the same work."""
        d = self.d
        B, K = self.B, self.K
        self._reserve(K)              # at most K rows are accepted
        _ok("orthrus_block_tokens",
            B_.orthrus_block_tokens(self.anchor, None, self.mask_token, self.tok, B, K))
        x = self.forward(self.tok, "diff", B_.BIDIR, idx=self.d_tok)
        if keep_hidden:
            self.x_diff = x.clone()
        cand = self.d_tok if draft is None else draft
        _ok("orthrus_block_tokens",
            B_.orthrus_block_tokens(self.anchor, cand, 0, self.tok, B, K))
        kv = [(self.kb[l], self.vb[l]) for l in range(d.layers)]
        x = self.forward(self.tok, "ar", B_.CAUSAL, kv_out=kv, idx=self.a_tok)
        if keep_hidden:
            self.x_ar = x.clone()
        _ok("orthrus_consensus_tokens",
            B_.orthrus_consensus_tokens(cand, self.a_tok, B, K, self.n_match, self.n_emit,
                                        self.emit_off, self.emitted, self.anchor))
        # the accepted AR rows of every layer, lengths advanced in place
        if not advance and not hasattr(self, "lens_next"):
            self.lens_next = torch.empty_like(self.lens)
        api.kv_append(self.caches[0], self.kb[0], self.vb[0], self.n_emit,
                      lens_out=self.lens if advance else self.lens_next,
                      num_layers=d.layers, cache_layer_stride=self.kc[0].numel(),
                      blk_layer_stride=self.kb[0].numel())
        if advance:
            self.upper += K
