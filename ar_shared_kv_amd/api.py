"""Tensor-level wrappers over the C ABI: allocate outputs and workspaces with
torch on the inputs' device, call the library, raise on a non-zero status.
No arithmetic happens here."""
from __future__ import annotations

import torch

from . import _binding as B_

_DT = {torch.float32: B_.F32, torch.bfloat16: B_.BF16}


def dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def make_cache(k, v, lens, *, page_table=None, max_len=0):
    return B_.make_cache(k, v, lens, page_table=page_table, max_len=max_len)


def block_attn_workspace(cache, B, K, Hq, Hkv, D, dtype, num_splits=0, device=None):
    n = B_.orthrus_block_attn_workspace_bytes(cache, B, K, Hq, Hkv, D, dtype, num_splits)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def block_attn(q, k_blk, v_blk, cache, *, mask, scale=None, num_splits=0, out=None, lse=None,
               want_lse=True, workspace=None, stream=None):
    """Shared-KV block attention of one layer; returns (out, lse)."""
    Bn, K, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    dt = dtype_code(q)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Bn, Hq, K), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace, nbytes = block_attn_workspace(cache, Bn, K, Hq, Hkv, D, dt, num_splits, q.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    st = B_.orthrus_block_attn(cache, q, k_blk, v_blk, out, lse, Bn, K, Hq, Hkv, D, dt, mask,
                               scale, num_splits, workspace, nbytes, stream)
    B_.check("orthrus_block_attn", st)
    return out, lse


class ConsensusBuffers:
    """Outputs + workspace of orthrus_consensus for a fixed (B, K, V, dtype)."""

    def __init__(self, B, K, V, dtype, device):
        i32 = dict(dtype=torch.int32, device=device)
        self.B, self.K, self.V, self.dtype = B, K, V, dtype
        self.diff_tok = torch.empty((B, K), **i32)
        self.ar_tok = torch.empty((B, K), **i32)
        self.n_match = torch.empty(B, **i32)
        self.n_emit = torch.empty(B, **i32)
        self.emit_off = torch.empty(B + 1, **i32)
        self.emitted = torch.empty(B * K, **i32)
        self.next_anchor = torch.empty(B, **i32)
        self.ws_bytes = B_.orthrus_consensus_workspace_bytes(B, K, V, dtype)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def as_dict(self):
        total = int(self.emit_off[-1])
        return {"diff_tok": self.diff_tok, "ar_tok": self.ar_tok, "j": self.n_match,
                "n": self.n_emit, "emit_off": self.emit_off, "emitted": self.emitted[:total],
                "next_anchor": self.next_anchor}


def consensus(diff_logits, ar_logits, bufs: ConsensusBuffers | None = None, stream=None):
    Bn, K, V = ar_logits.shape
    dt = dtype_code(ar_logits)
    if bufs is None:
        bufs = ConsensusBuffers(Bn, K, V, dt, ar_logits.device)
    st = B_.orthrus_consensus(diff_logits, ar_logits, Bn, K, V, dt, bufs.diff_tok, bufs.ar_tok,
                              bufs.n_match, bufs.n_emit, bufs.emit_off, bufs.emitted,
                              bufs.next_anchor, bufs.ws, bufs.ws_bytes, stream)
    B_.check("orthrus_consensus", st)
    return bufs


def argmax(logits, stream=None):
    V = logits.shape[-1]
    rows = logits.numel() // V
    dt = dtype_code(logits)
    idx = torch.empty(rows, dtype=torch.int32, device=logits.device)
    n = B_.orthrus_argmax_workspace_bytes(rows, V, dt)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=logits.device)
    st = B_.orthrus_argmax(logits, rows, V, dt, idx, ws, n, stream)
    B_.check("orthrus_argmax", st)
    return idx.view(logits.shape[:-1])


def lmhead_argmax(hidden, weight, idx=None, workspace=None, stream=None):
    """Greedy tokens of hidden [..., H] under the LM head weight [V, H] (bf16)."""
    H = hidden.shape[-1]
    R = hidden.numel() // H
    V = weight.shape[0]
    dt = dtype_code(hidden)
    if idx is None:
        idx = torch.empty(R, dtype=torch.int32, device=hidden.device)
    n = B_.orthrus_lmhead_argmax_workspace_bytes(R, H, V, dt)
    if workspace is None:
        workspace = torch.empty(max(n, 8), dtype=torch.uint8, device=hidden.device)
    st = B_.orthrus_lmhead_argmax(hidden, weight, R, H, V, dt, idx, workspace,
                                  workspace.numel(), stream)
    B_.check("orthrus_lmhead_argmax", st)
    return idx.view(hidden.shape[:-1])


def kv_append(cache, k_blk, v_blk, n_emit, lens_out=None, *, num_layers=1,
              cache_layer_stride=0, blk_layer_stride=0, stream=None):
    """Append accepted AR rows; k_blk/v_blk are layer 0's [B, K, Hkv, D]."""
    Bn, K, Hkv, D = k_blk.shape[-4:]
    if lens_out is None:
        lens_out = torch.empty(Bn, dtype=torch.int32, device=k_blk.device)
    st = B_.orthrus_kv_append(cache, k_blk, v_blk, n_emit, lens_out, Bn, K, Hkv, D,
                              dtype_code(k_blk), num_layers, cache_layer_stride, blk_layer_stride,
                              stream)
    B_.check("orthrus_kv_append", st)
    return lens_out
