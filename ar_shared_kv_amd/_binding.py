"""ctypes binding of liborthrus.so (the C ABI in include/orthrus.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and streams; torch
is imported before the library is loaded so that both use the one HIP runtime
already in the process (torch's libamdhip64 carries the same soname the
library was linked against).  There is no fallback: if the library is missing
every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch  # noqa: F401  (must precede the library load; see module doc)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liborthrus.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "orthrus.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = range(7)
F32, BF16, FP8_E4M3 = 0, 1, 2
BIDIR, CAUSAL = 0, 1
CONTIGUOUS, PAGED = 0, 1


class OrthrusError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class orthrus_cache(ctypes.Structure):
    """Mirror of ``struct orthrus_cache`` (include/orthrus.h)."""
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("capacity", ctypes.c_int64),
        ("num_pages", ctypes.c_int64),
        ("page_table", ctypes.c_void_p),
        ("max_pages_per_req", ctypes.c_int64),
        ("lens", ctypes.c_void_p),
        ("max_len", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


_lock = threading.Lock()
_lib = None

_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_CP = ctypes.POINTER(orthrus_cache)
SIGNATURES = {
    "orthrus_block_attn": (_I, [_CP, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                _P, _SZ, _P]),
    "orthrus_block_attn_workspace_bytes": (_SZ, [_CP, _I, _I, _I, _I, _I, _I, _I]),
    "orthrus_block_attn_noalloc": (_I, [_CP, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                        _I, _P]),
    "orthrus_block_attn_noalloc_max_workspace": (_SZ, []),
    "orthrus_mdiff_attn": (_I, [_P, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                _I, _I, _F, _I, _P, _SZ, _P]),
    "orthrus_mdiff_attn_workspace_bytes": (_SZ, [_I64, _I64, _I, _I, _I, _I, _I, _I, _I, _I]),
    "orthrus_consensus": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_consensus_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "orthrus_argmax": (_I, [_P, _I64, _I, _I, _P, _P, _SZ, _P]),
    "orthrus_argmax_workspace_bytes": (_SZ, [_I64, _I, _I]),
    "orthrus_lmhead_argmax": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "orthrus_lmhead_argmax_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "orthrus_kv_append": (_I, [_CP, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _I64, _P]),
    "orthrus_stream_read": (_I, [_P, _SZ, _I, _P, _P]),
    "orthrus_consensus_tokens": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _P, _P]),
    "orthrus_gemm": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "orthrus_gemm_workspace_bytes": (_SZ, [_I, _I, _I]),
    "orthrus_rmsnorm": (_I, [_P, _P, _P, _I, _I, _F, _P]),
    "orthrus_gemm_epilogue_workspace_bytes": (_SZ, [_I, _I, _I]),
    "orthrus_gemm_rmsnorm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _SZ, _P]),
    "orthrus_gemm_swiglu": (_I, [_P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "orthrus_gemm_qk_norm_rope": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I,
                                       _F, _F, _P, _SZ, _P]),
    "orthrus_qk_norm_rope": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F, _F, _P]),
    "orthrus_block_tokens": (_I, [_P, _P, _I, _P, _I, _I, _P]),
    "orthrus_swiglu": (_I, [_P, _P, _I, _I, _P]),
    "orthrus_embed": (_I, [_P, _P, _P, _I, _I, _P]),
    "orthrus_pack_weight": (_I, [_P, _I, _I, _P, _SZ, _P]),
    "orthrus_packed_weight_bytes": (_SZ, [_I, _I]),
    "orthrus_pack_weight_gate_up": (_I, [_P, _I, _I, _P, _SZ, _P]),
    "orthrus_status_string": (ctypes.c_char_p, [_I]),
    "orthrus_version": (_I, []),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m ar_shared_kv_amd.build`")
            l = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                f = getattr(l, name)
                f.restype = res
                f.argtypes = args
            _lib = l
    return _lib


def header_functions() -> list:
    """Names of the functions include/orthrus.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(orthrus_[a-z_0-9]+)\s*\(",
                                 txt, re.M)))


def status_string(status: int) -> str:
    return lib().orthrus_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != OK:
        raise OrthrusError(fn, status, status_string(status))


def ptr(t) -> int | None:
    """Device address of a tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_cache(k, v, lens, *, page_table=None, capacity=None, max_len=0, page_size=16,
               k_scale=None, v_scale=None):
    """orthrus_cache for torch tensors.

    Contiguous: k, v [B, Hkv, cap, D].  Paged: k, v [num_pages, Hkv, page, D]
    with page_table [B, max_pages].  With k_scale/v_scale (fp32, the cache's
    shape without D) the cache holds fp8 e4m3 codes (uint8 tensors).  The
    returned struct keeps references to the tensors it points at.
    """
    c = orthrus_cache()
    if page_table is None:
        c.layout = CONTIGUOUS
        c.capacity = int(capacity if capacity is not None else k.shape[2])
        c.page_size = page_size
    else:
        c.layout = PAGED
        c.page_size = int(k.shape[2])
        c.num_pages = int(k.shape[0])
        c.page_table = ptr(page_table)
        c.max_pages_per_req = int(page_table.shape[1])
    c.k, c.v, c.lens = ptr(k), ptr(v), ptr(lens)
    c.max_len = int(max_len)
    if k_scale is not None:
        c.kv_dtype = FP8_E4M3
        c.k_scale, c.v_scale = ptr(k_scale), ptr(v_scale)
    c._keep = (k, v, lens, page_table, k_scale, v_scale)
    return c


# ---------------------------------------------------------------- raw ABI

def orthrus_block_attn(cache, q, k_blk, v_blk, out, lse, B, K, Hq, Hkv, D, dtype, mask, scale,
                       num_splits, workspace, workspace_bytes, stream=None) -> int:
    return lib().orthrus_block_attn(ctypes.byref(cache), ptr(q), ptr(k_blk), ptr(v_blk), ptr(out),
                                    ptr(lse), B, K, Hq, Hkv, D, dtype, mask, scale, num_splits,
                                    ptr(workspace), workspace_bytes,
                                    stream if isinstance(stream, int) else stream_handle(stream))


def orthrus_block_attn_workspace_bytes(cache, B, K, Hq, Hkv, D, dtype, num_splits) -> int:
    return lib().orthrus_block_attn_workspace_bytes(ctypes.byref(cache), B, K, Hq, Hkv, D, dtype,
                                                    num_splits)


def orthrus_block_attn_noalloc(cache, q, k_blk, v_blk, out, lse, B, K, Hq, Hkv, D, dtype, mask,
                               scale, num_splits, stream=None) -> int:
    return lib().orthrus_block_attn_noalloc(ctypes.byref(cache), ptr(q), ptr(k_blk), ptr(v_blk),
                                            ptr(out), ptr(lse), B, K, Hq, Hkv, D, dtype, mask,
                                            scale, num_splits,
                                            stream if isinstance(stream, int)
                                            else stream_handle(stream))


def orthrus_block_attn_noalloc_max_workspace() -> int:
    return lib().orthrus_block_attn_noalloc_max_workspace()


def orthrus_mdiff_attn(k_ctx, v_ctx, ctx_capacity, anchors, max_anchor, q, k_blk, v_blk, out,
                       lse, B, NB, K, Hq, Hkv, D, dtype, scale, num_splits, workspace,
                       workspace_bytes, stream=None) -> int:
    return lib().orthrus_mdiff_attn(ptr(k_ctx), ptr(v_ctx), ctx_capacity, ptr(anchors),
                                    max_anchor, ptr(q), ptr(k_blk), ptr(v_blk), ptr(out), ptr(lse),
                                    B, NB, K, Hq, Hkv, D, dtype, scale, num_splits, ptr(workspace),
                                    workspace_bytes,
                                    stream if isinstance(stream, int) else stream_handle(stream))


def orthrus_mdiff_attn_workspace_bytes(ctx_capacity, max_anchor, B, NB, K, Hq, Hkv, D, dtype,
                                       num_splits) -> int:
    return lib().orthrus_mdiff_attn_workspace_bytes(ctx_capacity, max_anchor, B, NB, K, Hq, Hkv,
                                                    D, dtype, num_splits)


def orthrus_consensus(diff_logits, ar_logits, B, K, V, dtype, diff_tok, ar_tok, n_match, n_emit,
                      emit_off, emitted, next_anchor, workspace, workspace_bytes,
                      stream=None) -> int:
    return lib().orthrus_consensus(ptr(diff_logits), ptr(ar_logits), B, K, V, dtype, ptr(diff_tok),
                                   ptr(ar_tok), ptr(n_match), ptr(n_emit), ptr(emit_off),
                                   ptr(emitted), ptr(next_anchor), ptr(workspace), workspace_bytes,
                                   stream if isinstance(stream, int) else stream_handle(stream))


def orthrus_consensus_workspace_bytes(B, K, V, dtype) -> int:
    return lib().orthrus_consensus_workspace_bytes(B, K, V, dtype)


def orthrus_argmax(logits, rows, V, dtype, idx, workspace, workspace_bytes, stream=None) -> int:
    return lib().orthrus_argmax(ptr(logits), rows, V, dtype, ptr(idx), ptr(workspace),
                                workspace_bytes,
                                stream if isinstance(stream, int) else stream_handle(stream))


def orthrus_argmax_workspace_bytes(rows, V, dtype) -> int:
    return lib().orthrus_argmax_workspace_bytes(rows, V, dtype)


def orthrus_lmhead_argmax(hidden, weight, R, H, V, dtype, idx, workspace, workspace_bytes,
                          stream=None) -> int:
    return lib().orthrus_lmhead_argmax(ptr(hidden), ptr(weight), R, H, V, dtype, ptr(idx),
                                       ptr(workspace), workspace_bytes,
                                       stream if isinstance(stream, int) else stream_handle(stream))


def orthrus_lmhead_argmax_workspace_bytes(R, H, V, dtype) -> int:
    return lib().orthrus_lmhead_argmax_workspace_bytes(R, H, V, dtype)


def orthrus_kv_append(cache, k_blk, v_blk, n_emit, lens_out, B, K, Hkv, D, dtype, num_layers,
                      cache_layer_stride, blk_layer_stride, stream=None) -> int:
    return lib().orthrus_kv_append(ctypes.byref(cache), ptr(k_blk), ptr(v_blk), ptr(n_emit),
                                   ptr(lens_out), B, K, Hkv, D, dtype, num_layers,
                                   cache_layer_stride, blk_layer_stride,
                                   stream if isinstance(stream, int) else stream_handle(stream))


def orthrus_stream_read(src, nbytes, work_groups, sink, stream=None) -> int:
    return lib().orthrus_stream_read(ptr(src), nbytes, work_groups, ptr(sink),
                                     stream if isinstance(stream, int) else stream_handle(stream))


def _st(stream):
    return stream if isinstance(stream, int) else stream_handle(stream)


def orthrus_consensus_tokens(diff_tok, ar_tok, B, K, n_match, n_emit, emit_off, emitted,
                             next_anchor, stream=None) -> int:
    return lib().orthrus_consensus_tokens(ptr(diff_tok), ptr(ar_tok), B, K, ptr(n_match),
                                          ptr(n_emit), ptr(emit_off), ptr(emitted),
                                          ptr(next_anchor), _st(stream))


def orthrus_gemm(x, w, residual, y, R, N, Kin, out_dtype, workspace, workspace_bytes,
                 stream=None) -> int:
    return lib().orthrus_gemm(ptr(x), ptr(w), ptr(residual), ptr(y), R, N, Kin, out_dtype,
                              ptr(workspace), workspace_bytes, _st(stream))


def orthrus_gemm_workspace_bytes(R, N, Kin) -> int:
    return lib().orthrus_gemm_workspace_bytes(R, N, Kin)


def orthrus_rmsnorm(x, weight, y, R, H, eps, stream=None) -> int:
    return lib().orthrus_rmsnorm(ptr(x), ptr(weight), ptr(y), R, H, eps, _st(stream))


def orthrus_qk_norm_rope(qkv, q_norm, k_norm, lens, K, q, k, v, R, Hq, Hkv, D, eps, theta,
                         stream=None) -> int:
    return lib().orthrus_qk_norm_rope(ptr(qkv), ptr(q_norm), ptr(k_norm), ptr(lens), K, ptr(q),
                                      ptr(k), ptr(v), R, Hq, Hkv, D, eps, theta, _st(stream))


def orthrus_block_tokens(anchor, cand, fill, out, B, K, stream=None) -> int:
    return lib().orthrus_block_tokens(ptr(anchor), ptr(cand), fill, ptr(out), B, K, _st(stream))


def orthrus_gemm_epilogue_workspace_bytes(R, N, Kin) -> int:
    return lib().orthrus_gemm_epilogue_workspace_bytes(R, N, Kin)


def orthrus_gemm_rmsnorm(x, w, h, norm_weight, xn, R, H, Kin, eps, workspace, workspace_bytes,
                         stream=None) -> int:
    return lib().orthrus_gemm_rmsnorm(ptr(x), ptr(w), ptr(h), ptr(norm_weight), ptr(xn), R, H,
                                      Kin, eps, ptr(workspace), workspace_bytes, _st(stream))


def orthrus_gemm_swiglu(x, w_gate_up, act, R, I, Kin, workspace, workspace_bytes,
                        stream=None) -> int:
    return lib().orthrus_gemm_swiglu(ptr(x), ptr(w_gate_up), ptr(act), R, I, Kin, ptr(workspace),
                                     workspace_bytes, _st(stream))


def orthrus_gemm_qk_norm_rope(x, w_qkv, q_norm, k_norm, lens, K, q, k, v, R, Hq, Hkv, D, Kin,
                              eps, theta, workspace, workspace_bytes, stream=None) -> int:
    return lib().orthrus_gemm_qk_norm_rope(ptr(x), ptr(w_qkv), ptr(q_norm), ptr(k_norm),
                                           ptr(lens), K, ptr(q), ptr(k), ptr(v), R, Hq, Hkv, D,
                                           Kin, eps, theta, ptr(workspace), workspace_bytes,
                                           _st(stream))


def orthrus_swiglu(gate_up, act, R, I, stream=None) -> int:
    return lib().orthrus_swiglu(ptr(gate_up), ptr(act), R, I, _st(stream))


def orthrus_embed(tokens, table, h, R, H, stream=None) -> int:
    return lib().orthrus_embed(ptr(tokens), ptr(table), ptr(h), R, H, _st(stream))


def orthrus_pack_weight(w, N, Kin, packed, packed_bytes, stream=None) -> int:
    return lib().orthrus_pack_weight(ptr(w), N, Kin, ptr(packed), packed_bytes, _st(stream))


def orthrus_pack_weight_gate_up(w, I, Kin, packed, packed_bytes, stream=None) -> int:
    return lib().orthrus_pack_weight_gate_up(ptr(w), I, Kin, ptr(packed), packed_bytes,
                                             _st(stream))


def orthrus_packed_weight_bytes(N, Kin) -> int:
    return lib().orthrus_packed_weight_bytes(N, Kin)


def orthrus_status_string(status: int) -> str:
    return status_string(status)


def orthrus_version() -> int:
    return lib().orthrus_version()
