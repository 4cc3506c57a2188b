"""fp64 CPU oracle for the Orthrus decode step.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this package; the product path
(``ar_shared_kv_amd``) never imports it, and the two share no code.

The arithmetic lives in ``orthrus_oracle.c`` (plain C, fp64, compiled with
gcc); this module only marshals numpy arrays.  Each function cites the passage
of the pages it follows (see the C file's header for the source list):

* ``block_attn``  -- shared-KV block attention, bidirectional (diffusion view)
  or causal (AR verification) inside the block; summary §2.1-§2.3.
* ``mdiff_attn``  -- the training-time block mask M_diff (forward): several
  blocks per sequence, each causal to the clean context before its anchor and
  bidirectional inside itself; summary §2.2.
* ``argmax_rows`` -- greedy prediction per row, lowest index on ties;
  summary §2.3 step 3.
* ``lmhead_logits`` / ``lmhead_argmax`` -- the greedy prediction from final
  hidden states (logits = hidden . W^T in fp64, then ``argmax_rows``);
  summary §2.3.
* ``consensus``   -- left-to-right exact consensus; summary §2.3 step 3.
* ``kv_append``   -- commit of the accepted rows' KV; summary §2.3 step 3 and
  the agents-report core-design section.
* ``e4m3_decode`` / ``e4m3_encode`` / ``fp8_scale_exp`` / ``dequant_fp8`` /
  ``kv_append_fp8`` -- the FP8 (OCP E4M3) KV cache: decoding and
  round-to-nearest-even encoding from the format's definition, the per-row
  power-of-two scale, and the quantizing commit; the agents-report outlook
  (low-precision kernels).  Attention over an FP8 cache is ``block_attn``
  on the dequantized values.

Parity pins: every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (library routines, closed forms, invariants and
brute force); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orthrus_oracle.c")
_LIB = os.path.join(_HERE, "liborthrus_oracle.so")
_lock = threading.Lock()
_lib = None

CONTIGUOUS, PAGED = 0, 1
BIDIR, CAUSAL = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (portable flags, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_double
            lib.oracle_block_attn.argtypes = [P, P, P, I, L, I, P, I, I, P, P, P,
                                              I, I, I, I, I, I, D, P, P]
            lib.oracle_block_attn.restype = I
            lib.oracle_argmax_rows.argtypes = [P, L, L, P]
            lib.oracle_argmax_rows.restype = I
            lib.oracle_consensus.argtypes = [P, P, I, I, P, P, P, P, P]
            lib.oracle_consensus.restype = None
            lib.oracle_kv_append.argtypes = [P, P, I, L, I, P, I, I, P, P, P, P, P,
                                             I, I, I, I, I, I, L, L]
            lib.oracle_kv_append.restype = I
            lib.oracle_mdiff_attn.argtypes = [P, P, P, L, P, P, P, I, I, I, I, I, I, D, P, P]
            lib.oracle_mdiff_attn.restype = I
            lib.oracle_e4m3_decode.argtypes = [I]
            lib.oracle_e4m3_decode.restype = D
            lib.oracle_e4m3_encode.argtypes = [D]
            lib.oracle_e4m3_encode.restype = I
            lib.oracle_fp8_scale_exp.argtypes = [D]
            lib.oracle_fp8_scale_exp.restype = I
            lib.oracle_e4m3_decode_array.argtypes = [P, L, P]
            lib.oracle_e4m3_decode_array.restype = None
            lib.oracle_kv_append_fp8.argtypes = [P, P, P, P, I, L, I, P, I, I, P, P, P, P, P,
                                                 I, I, I, I, I, L, L]
            lib.oracle_kv_append_fp8.restype = I
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = I
            lib.oracle_set_num_threads.argtypes = [I]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the C oracle's OpenMP loops for later calls."""
    _load().oracle_set_num_threads(int(n))


def block_attn(q, k_cache, v_cache, k_blk, v_blk, lens, *, mask, scale,
               layout=CONTIGUOUS, page_table=None, page_size=16):
    """Block attention of one layer in fp64.

    q, k_blk, v_blk: [B, K, H, D]; contiguous caches [B, Hkv, cap, D] or paged
    caches [num_pages, Hkv, page_size, D] with page_table [B, max_pages].
    Returns (out [B, K, Hq, D], lse [B, Hq, K]) as float64 arrays.
    """
    q, kc, vc, kb, vb = map(_f64, (q, k_cache, v_cache, k_blk, v_blk))
    lens = _i32(lens)
    B, K, Hq, D = q.shape
    Hkv = kb.shape[2]
    if layout == CONTIGUOUS:
        cap, num_pages, max_pages, pt = kc.shape[2], 0, 0, None
    else:
        pt = _i32(page_table)
        cap, num_pages, max_pages = 0, kc.shape[0], pt.shape[1]
        page_size = kc.shape[2]
    out = np.empty((B, K, Hq, D), np.float64)
    lse = np.empty((B, Hq, K), np.float64)
    rc = _load().oracle_block_attn(_ptr(q), _ptr(kc), _ptr(vc), layout, cap, page_size,
                                   _ptr(pt), max_pages, num_pages, _ptr(lens), _ptr(kb),
                                   _ptr(vb), B, K, Hq, Hkv, D, mask, float(scale),
                                   _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_block_attn rejected its arguments")
    return out, lse


def mdiff_attn(q, k_ctx, v_ctx, anchors, k_blk, v_blk, *, scale):
    """Diffusion-view attention under the training block mask M_diff (forward),
    in fp64.  q, k_blk, v_blk: [B, NB, K, H, D]; k_ctx, v_ctx: [B, Hkv, cap, D]
    (the clean context of each sequence); anchors: [B, NB].  Block j of
    sequence b sees context rows t < anchors[b, j] and its own K block rows.
    Returns (out [B, NB, K, Hq, D], lse [B, NB, Hq, K])."""
    q, kc, vc, kb, vb = map(_f64, (q, k_ctx, v_ctx, k_blk, v_blk))
    anchors = _i32(anchors)
    B, NB, K, Hq, D = q.shape
    Hkv = kb.shape[3]
    cap = kc.shape[2]
    out = np.empty((B, NB, K, Hq, D), np.float64)
    lse = np.empty((B, NB, Hq, K), np.float64)
    rc = _load().oracle_mdiff_attn(_ptr(q), _ptr(kc), _ptr(vc), cap, _ptr(anchors), _ptr(kb),
                                   _ptr(vb), B, NB, K, Hq, Hkv, D, float(scale), _ptr(out),
                                   _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_mdiff_attn rejected its arguments")
    return out, lse


def argmax_rows(x):
    """Row argmax of x[..., V] (lowest index on ties); returns int32 [...]."""
    x = _f64(x)
    V = x.shape[-1]
    rows = x.size // V
    idx = np.empty(rows, np.int32)
    if _load().oracle_argmax_rows(_ptr(x), rows, V, _ptr(idx)) != 0:
        raise ValueError("argmax undefined: NaN in logits")
    return idx.reshape(x.shape[:-1])


def lmhead_logits(hidden, weight, chunk: int = 8192):
    """fp64 logits hidden [R, H] . weight[V, H]^T -> [R, V] (a library matmul
    per block of vocabulary rows, so that weight never exists whole in fp64)."""
    def f64(a):   # numpy, or a tensor-like with .double().numpy() (bf16 inputs)
        return _f64(a.double().numpy() if hasattr(a, "double") else a)
    h = f64(hidden)
    R, H = h.shape
    V = weight.shape[0]
    out = np.empty((R, V), np.float64)
    for v0 in range(0, V, chunk):
        w = f64(weight[v0:v0 + chunk])
        out[:, v0:v0 + w.shape[0]] = h @ w.T
    return out


def lmhead_argmax(hidden, weight):
    """Greedy tokens: argmax_v of the fp64 logits, lowest index on ties."""
    return argmax_rows(lmhead_logits(hidden, weight))


def e4m3_decode(code: int) -> float:
    """Value of one OCP FP8 E4M3 code (NaN for S.1111.111)."""
    return float(_load().oracle_e4m3_decode(int(code)))


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code to x, ties to even; raises beyond +-448."""
    c = _load().oracle_e4m3_encode(float(x))
    if c < 0:
        raise ValueError(f"{x} is outside the E4M3 range")
    return c


def fp8_scale_exp(amax: float) -> int:
    """Smallest e >= -120 with 448 * 2^e >= amax (0 for amax = 0)."""
    return int(_load().oracle_fp8_scale_exp(float(amax)))


def dequant_fp8(codes, scales):
    """fp64 values of an E4M3 cache: decode(codes) * scale of the row.  codes
    [..., D] uint8, scales [...] float32 (one per row)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out * np.asarray(scales, dtype=np.float64)[..., None]


def kv_append_fp8(k_codes, v_codes, k_scale, v_scale, k_blk, v_blk, n, lens, *,
                  layout=CONTIGUOUS, page_table=None):
    """Append accepted AR rows into copies of an E4M3 cache, quantizing each
    (row, KV head): k_codes/v_codes [layers, ...cache layout...] uint8,
    k_scale/v_scale [layers, ...rows...] float32, k_blk/v_blk [layers, B, K,
    Hkv, D] (any real type; converted to fp64 exactly).  Returns (k_codes',
    v_codes', k_scale', v_scale', lens_out)."""
    kc = np.array(k_codes, dtype=np.uint8, copy=True, order="C")
    vc = np.array(v_codes, dtype=np.uint8, copy=True, order="C")
    ks = np.array(k_scale, dtype=np.float32, copy=True, order="C")
    vs = np.array(v_scale, dtype=np.float32, copy=True, order="C")
    kb, vb = _f64(k_blk), _f64(v_blk)
    layers, B, K, Hkv, D = kb.shape
    n, lens = _i32(n), _i32(lens)
    if layout == CONTIGUOUS:
        cap, page_size, num_pages, max_pages, pt = kc.shape[3], 16, 0, 0, None
    else:
        pt = _i32(page_table)
        cap, num_pages, page_size, max_pages = 0, kc.shape[1], kc.shape[3], pt.shape[1]
    lens_out = np.empty(B, np.int32)
    rc = _load().oracle_kv_append_fp8(_ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), layout, cap,
                                      page_size, _ptr(pt), max_pages, num_pages, _ptr(lens),
                                      _ptr(kb), _ptr(vb), _ptr(n), _ptr(lens_out), B, K, Hkv, D,
                                      layers, kc[0].size, kb[0].size)
    if rc != 0:
        raise ValueError("oracle_kv_append_fp8 rejected its arguments")
    return kc, vc, ks, vs, lens_out


def consensus(d_tok, a_tok):
    """Exact consensus over [B, K] token arrays.

    Returns dict with j, n, emit_off [B+1], emitted [sum n], next_anchor.
    """
    d, a = _i32(d_tok), _i32(a_tok)
    B, K = d.shape
    j = np.empty(B, np.int32)
    n = np.empty(B, np.int32)
    off = np.empty(B + 1, np.int32)
    emitted = np.empty(B * K, np.int32)
    anchor = np.empty(B, np.int32)
    _load().oracle_consensus(_ptr(d), _ptr(a), B, K, _ptr(j), _ptr(n), _ptr(off),
                             _ptr(emitted), _ptr(anchor))
    return {"j": j, "n": n, "emit_off": off, "emitted": emitted[: off[B]].copy(),
            "next_anchor": anchor}


def kv_append(k_cache, v_cache, k_blk, v_blk, n, lens, *, layout=CONTIGUOUS,
              page_table=None):
    """Append accepted AR block rows into copies of the caches.

    k_cache/v_cache: [layers, ...cache layout...] numpy arrays of any element
    type (copied as bytes); k_blk/v_blk: [layers, B, K, Hkv, D].
    Returns (k_cache', v_cache', lens_out).
    """
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    kb = np.ascontiguousarray(k_blk)
    vb = np.ascontiguousarray(v_blk)
    if kb.dtype != kc.dtype or vb.dtype != kc.dtype or vc.dtype != kc.dtype:
        raise ValueError("cache and block element types differ")
    layers, B, K, Hkv, D = kb.shape
    n, lens = _i32(n), _i32(lens)
    if layout == CONTIGUOUS:
        cap, page_size, num_pages, max_pages, pt = kc.shape[3], 16, 0, 0, None
    else:
        pt = _i32(page_table)
        cap, num_pages, page_size, max_pages = 0, kc.shape[1], kc.shape[3], pt.shape[1]
    lens_out = np.empty(B, np.int32)
    rc = _load().oracle_kv_append(_ptr(kc), _ptr(vc), layout, cap, page_size, _ptr(pt),
                                  max_pages, num_pages, _ptr(lens), _ptr(kb), _ptr(vb),
                                  _ptr(n), _ptr(lens_out), B, K, Hkv, D, kc.itemsize,
                                  layers, kc[0].size, kb[0].size)
    if rc != 0:
        raise ValueError("oracle_kv_append rejected its arguments")
    return kc, vc, lens_out
