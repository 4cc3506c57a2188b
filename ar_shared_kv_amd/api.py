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


def _need(name, t, *, dtype=None, shape=None, device=None):
    """Host-side checks before a device pointer crosses the C ABI: the library
    reads dense row-major buffers, so a view with other strides, another
    element type or another device would be read as garbage."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (call .contiguous())")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return t


def make_cache(k, v, lens, *, page_table=None, max_len=0, k_scale=None, v_scale=None):
    """orthrus_cache over k, v [B, Hkv, cap, D] (or paged [pages, Hkv, 16, D]
    with page_table [B, max_pages]).  With k_scale/v_scale (float32, the
    cache shape without D) k and v are uint8 tensors of OCP E4M3 codes."""
    _need("k_cache", k)
    _need("v_cache", v, dtype=k.dtype, shape=k.shape, device=k.device)
    if k.dim() != 4:
        raise ValueError("cache tensors are [B, Hkv, cap, D] or [pages, Hkv, page, D]")
    _need("lens", lens, dtype=torch.int32, device=k.device)
    if page_table is not None:
        _need("page_table", page_table, dtype=torch.int32, device=k.device)
        if page_table.dim() != 2 or page_table.shape[0] != lens.shape[0]:
            raise ValueError("page_table must be [B, max_pages] with B = len(lens)")
    if (k_scale is None) != (v_scale is None):
        raise ValueError("an E4M3 cache needs both k_scale and v_scale")
    if k_scale is not None:
        if k.dtype != torch.uint8:
            raise TypeError("an E4M3 cache holds uint8 codes")
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            _need(name, t, dtype=torch.float32, shape=k.shape[:-1], device=k.device)
    return B_.make_cache(k, v, lens, page_table=page_table, max_len=max_len, k_scale=k_scale,
                         v_scale=v_scale)


def _cache_matches(cache, dtype, device, Hkv, D):
    ck = cache._keep[0]
    fp8 = cache.kv_dtype == B_.FP8_E4M3
    ok = (ck.dtype == torch.uint8 and dtype == torch.bfloat16) if fp8 else ck.dtype == dtype
    return ok and ck.device == device and ck.shape[1] == Hkv and ck.shape[3] == D


def block_attn_workspace(cache, B, K, Hq, Hkv, D, dtype, num_splits=0, device=None):
    n = B_.orthrus_block_attn_workspace_bytes(cache, B, K, Hq, Hkv, D, dtype, num_splits)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def block_attn(q, k_blk, v_blk, cache, *, mask, scale=None, num_splits=0, out=None, lse=None,
               want_lse=True, workspace=None, stream=None):
    """Shared-KV block attention of one layer; returns (out, lse)."""
    if q.dim() != 4 or k_blk.dim() != 4:
        raise ValueError("q is [B, K, Hq, D] and k_blk/v_blk [B, K, Hkv, D]")
    Bn, K, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    dt = dtype_code(q)
    _need("q", q)
    _need("k_blk", k_blk, dtype=q.dtype, shape=(Bn, K, Hkv, D), device=q.device)
    _need("v_blk", v_blk, dtype=q.dtype, shape=(Bn, K, Hkv, D), device=q.device)
    if not _cache_matches(cache, q.dtype, q.device, Hkv, D):
        ck = cache._keep[0]
        raise ValueError(f"cache {tuple(ck.shape)} {ck.dtype} does not match q/k_blk "
                         f"(Hkv={Hkv}, D={D}, {q.dtype})")
    if cache._keep[2].shape[0] != Bn:
        raise ValueError("cache lens has another batch size than q")
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _need("out", out, dtype=q.dtype, shape=q.shape, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Bn, Hq, K), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need("lse", lse, dtype=torch.float32, shape=(Bn, Hq, K), device=q.device)
    if workspace is None:
        workspace, nbytes = block_attn_workspace(cache, Bn, K, Hq, Hkv, D, dt, num_splits, q.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    st = B_.orthrus_block_attn(cache, q, k_blk, v_blk, out, lse, Bn, K, Hq, Hkv, D, dt, mask,
                               scale, num_splits, workspace, nbytes, stream)
    B_.check("orthrus_block_attn", st)
    return out, lse


def mdiff_attn(q, k_blk, v_blk, k_ctx, v_ctx, anchors, *, scale=None, max_anchor=0,
               num_splits=0, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Training-time block-mask (M_diff) attention, forward: q [B, NB, K, Hq, D],
    k_blk/v_blk [B, NB, K, Hkv, D], k_ctx/v_ctx [B, Hkv, cap, D], anchors
    int32 [B, NB].  Returns (out, lse)."""
    if q.dim() != 5 or k_blk.dim() != 5 or k_ctx.dim() != 4:
        raise ValueError("q/k_blk/v_blk are [B, NB, K, H, D] and k_ctx/v_ctx [B, Hkv, cap, D]")
    Bn, NB, K, Hq, D = q.shape
    Hkv = k_blk.shape[3]
    cap = k_ctx.shape[2]
    dt = dtype_code(q)
    _need("q", q)
    for name, t in (("k_blk", k_blk), ("v_blk", v_blk)):
        _need(name, t, dtype=q.dtype, shape=(Bn, NB, K, Hkv, D), device=q.device)
    for name, t in (("k_ctx", k_ctx), ("v_ctx", v_ctx)):
        _need(name, t, dtype=q.dtype, shape=(Bn, Hkv, cap, D), device=q.device)
    _need("anchors", anchors, dtype=torch.int32, shape=(Bn, NB), device=q.device)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _need("out", out, dtype=q.dtype, shape=q.shape, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Bn, NB, Hq, K), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need("lse", lse, dtype=torch.float32, shape=(Bn, NB, Hq, K), device=q.device)
    n = B_.orthrus_mdiff_attn_workspace_bytes(cap, max_anchor, Bn, NB, K, Hq, Hkv, D, dt,
                                              num_splits)
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = B_.orthrus_mdiff_attn(k_ctx, v_ctx, cap, anchors, max_anchor, q, k_blk, v_blk, out, lse,
                               Bn, NB, K, Hq, Hkv, D, dt, scale, num_splits, workspace, nbytes,
                               stream)
    B_.check("orthrus_mdiff_attn", st)
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
    _need("ar_logits", ar_logits)
    _need("diff_logits", diff_logits, dtype=ar_logits.dtype, shape=ar_logits.shape,
          device=ar_logits.device)
    if bufs is not None and (bufs.B, bufs.K, bufs.V, bufs.dtype) != (Bn, K, V, dt):
        raise ValueError("ConsensusBuffers were made for another (B, K, V, dtype)")
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
    _need("logits", logits)
    idx = torch.empty(rows, dtype=torch.int32, device=logits.device)
    n = B_.orthrus_argmax_workspace_bytes(rows, V, dt)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=logits.device)
    st = B_.orthrus_argmax(logits, rows, V, dt, idx, ws, n, stream)
    B_.check("orthrus_argmax", st)
    return idx.view(logits.shape[:-1])


class PackedWeight:
    """A bf16 weight of N rows x Kin columns in the library's packed tile
    layout (orthrus_pack_weight), as the projections and the LM head read it.
    ``data`` is the flat bf16 storage (ceil(N / 128) * 128 * Kin values);
    the object passes for a tensor in the binding's calls (``data_ptr``)."""

    def __init__(self, data: torch.Tensor, N: int, Kin: int, gate_up: bool = False):
        self.data, self.N, self.Kin, self.gate_up = data, int(N), int(Kin), gate_up

    @property
    def device(self):
        return self.data.device

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def pack_weight(w, out=None, stream=None) -> PackedWeight:
    """Packs a row-major bf16 weight [N, Kin] for orthrus_gemm* and
    lmhead_argmax (a one-time layout step, not part of a decode step)."""
    _need("weight", w, dtype=torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("weight is [N, Kin]")
    N, Kin = w.shape
    n = B_.orthrus_packed_weight_bytes(N, Kin)
    if n == 0:
        raise ValueError(f"weight [{N}, {Kin}]: Kin must be a positive multiple of 64")
    if out is None:
        out = torch.empty(n // 2, dtype=torch.bfloat16, device=w.device)
    _need("out", out, dtype=torch.bfloat16, device=w.device)
    B_.check("orthrus_pack_weight",
             B_.orthrus_pack_weight(w, N, Kin, out, out.numel() * 2, stream))
    return PackedWeight(out, N, Kin)


def pack_weight_gate_up(w, out=None, stream=None) -> PackedWeight:
    """Packs the MLP's gate/up weight [2I, Kin] (gate rows, then up rows) in
    the paired order orthrus_gemm_swiglu reads."""
    _need("weight", w, dtype=torch.bfloat16)
    if w.dim() != 2 or w.shape[0] % 8:
        raise ValueError("gate/up weight is [2I, Kin] with I a multiple of 4")
    N, Kin = w.shape
    n = B_.orthrus_packed_weight_bytes(N, Kin)
    if n == 0:
        raise ValueError(f"weight [{N}, {Kin}]: Kin must be a positive multiple of 64")
    if out is None:
        out = torch.empty(n // 2, dtype=torch.bfloat16, device=w.device)
    _need("out", out, dtype=torch.bfloat16, device=w.device)
    B_.check("orthrus_pack_weight_gate_up",
             B_.orthrus_pack_weight_gate_up(w, N // 2, Kin, out, out.numel() * 2, stream))
    return PackedWeight(out, N, Kin, gate_up=True)


def lmhead_argmax(hidden, weight, idx=None, workspace=None, stream=None):
    """Greedy tokens of hidden [..., H] under the LM head weight (V rows of
    H, bf16) packed by pack_weight."""
    H = hidden.shape[-1]
    R = hidden.numel() // H
    dt = dtype_code(hidden)
    _need("hidden", hidden)
    if not isinstance(weight, PackedWeight) or weight.gate_up:
        raise TypeError("weight: pack it first with pack_weight(w)")
    if weight.Kin != H or weight.device != hidden.device:
        raise ValueError(f"weight packs {weight.Kin} columns on {weight.device}; hidden has "
                         f"{H} on {hidden.device}")
    V = weight.N
    if idx is None:
        idx = torch.empty(R, dtype=torch.int32, device=hidden.device)
    _need("idx", idx, dtype=torch.int32, device=hidden.device)
    if idx.numel() != R:
        raise ValueError(f"idx holds {idx.numel()} entries for {R} rows")
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
    _need("k_blk", k_blk)
    _need("v_blk", v_blk, dtype=k_blk.dtype, shape=k_blk.shape, device=k_blk.device)
    _need("n_emit", n_emit, dtype=torch.int32, shape=(Bn,), device=k_blk.device)
    if not _cache_matches(cache, k_blk.dtype, k_blk.device, Hkv, D):
        raise ValueError("cache and block rows differ in dtype, device, Hkv or D")
    if lens_out is None:
        lens_out = torch.empty(Bn, dtype=torch.int32, device=k_blk.device)
    _need("lens_out", lens_out, dtype=torch.int32, shape=(Bn,), device=k_blk.device)
    st = B_.orthrus_kv_append(cache, k_blk, v_blk, n_emit, lens_out, Bn, K, Hkv, D,
                              dtype_code(k_blk), num_layers, cache_layer_stride, blk_layer_stride,
                              stream)
    B_.check("orthrus_kv_append", st)
    return lens_out
