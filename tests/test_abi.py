"""The C ABI on the host (CPU only): the library loads, exports every function
include/orthrus.h declares, and rejects every invalid argument with its
status code before touching a device (no call here reaches a launch)."""
import ctypes

import pytest

from ar_shared_kv_amd import _binding as B

FAKE = 1 << 20           # a non-null, 16-byte-aligned stand-in address (never dereferenced)


def cache(layout=B.CONTIGUOUS, capacity=8224, max_len=8192, pages=0, maxp=0, page_size=16):
    c = B.orthrus_cache()
    c.layout, c.capacity, c.max_len = layout, capacity, max_len
    c.k = c.v = c.lens = FAKE
    c.page_size = page_size
    if layout == B.PAGED:
        c.page_table, c.num_pages, c.max_pages_per_req, c.capacity = FAKE, pages, maxp, 0
    return c


def attn(c, **kw):
    a = dict(q=FAKE, kb=FAKE, vb=FAKE, out=FAKE, lse=None, B=1, K=32, Hq=32, Hkv=8, D=128,
             dtype=B.BF16, mask=B.CAUSAL, scale=0.088, splits=0, ws=None, wsb=0)
    a.update(kw)
    return B.lib().orthrus_block_attn(ctypes.byref(c) if c is not None else None, a["q"], a["kb"],
                                      a["vb"], a["out"], a["lse"], a["B"], a["K"], a["Hq"],
                                      a["Hkv"], a["D"], a["dtype"], a["mask"], a["scale"],
                                      a["splits"], a["ws"], a["wsb"], None)


def test_exports_every_declared_function():
    declared = B.header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(B.lib(), name), name
    assert set(declared) == set(B.SIGNATURES)


def test_status_strings_complete():
    names = [B.status_string(s) for s in range(7)]
    assert len(set(names)) == 7 and "unknown" not in " ".join(names)
    assert B.status_string(99) == "unknown status"
    assert B.orthrus_version() == 10000


def test_block_attn_validation_codes():
    c = cache()
    assert attn(None) == B.ERR_NULL
    assert attn(c, q=None) == B.ERR_NULL
    assert attn(c, out=None) == B.ERR_NULL
    assert attn(c, B=0) == B.ERR_SHAPE
    assert attn(c, Hq=30) == B.ERR_SHAPE            # Hq % Hkv != 0
    assert attn(c, K=0) == B.ERR_SHAPE
    assert attn(c, scale=float("nan")) == B.ERR_SHAPE
    assert attn(c, K=65) == B.ERR_UNSUPPORTED
    assert attn(c, D=96) == B.ERR_UNSUPPORTED
    assert attn(c, Hq=8 * 17) == B.ERR_UNSUPPORTED  # G = 17 > 16
    assert attn(c, dtype=2) == B.ERR_DTYPE
    assert attn(c, mask=3) == B.ERR_DTYPE
    assert attn(c, q=FAKE + 2) == B.ERR_UNSUPPORTED  # misaligned
    assert attn(cache(layout=7)) == B.ERR_DTYPE
    assert attn(cache(max_len=9000)) == B.ERR_SHAPE  # hint beyond capacity
    # split-KV needs a workspace
    need = B.orthrus_block_attn_workspace_bytes(c, 1, 32, 32, 8, 128, B.BF16, 0)
    assert need > 0
    assert attn(c) == B.ERR_WORKSPACE
    assert attn(c, ws=FAKE, wsb=need - 1) == B.ERR_WORKSPACE
    pc = cache(layout=B.PAGED, pages=100, maxp=10, max_len=0, page_size=8)
    assert attn(pc) == B.ERR_UNSUPPORTED            # page size must be 16
    pc = cache(layout=B.PAGED, pages=100, maxp=10, max_len=0)
    pc.page_table = None
    assert attn(pc) == B.ERR_NULL


def test_block_attn_workspace_formula():
    c = cache(capacity=131136, max_len=131072)
    # 64 splits of 2048 keys: bf16 partials [B*Hkv][M][S][D] (256-byte aligned
    # end) + fp32 lse [B*Hkv][M][S]
    n = B.orthrus_block_attn_workspace_bytes(c, 1, 64, 32, 8, 128, B.BF16, 64)
    rows = 1 * 8 * 64 * 256
    assert n == -(-rows * 128 * 2 // 256) * 256 + rows * 4
    nf = B.orthrus_block_attn_workspace_bytes(c, 1, 64, 32, 8, 128, B.F32, 64)
    assert nf == -(-rows * 128 * 4 // 256) * 256 + rows * 4
    # one split -> no workspace (fp32 splits go down to 64 keys, bf16 to 256)
    small = cache(capacity=128, max_len=64)
    assert B.orthrus_block_attn_workspace_bytes(small, 1, 8, 2, 1, 64, B.F32, 0) == 0
    assert B.orthrus_block_attn_workspace_bytes(small, 1, 8, 2, 1, 64, B.BF16, 0) == 0
    # 128 keys in fp32: two splits of 64; M = 16 rows padded to 32
    small = cache(capacity=128, max_len=128)
    rows = 1 * 1 * 2 * 32
    assert B.orthrus_block_attn_workspace_bytes(small, 1, 8, 2, 1, 64, B.F32, 0) == \
        rows * 64 * 4 + rows * 4
    assert B.orthrus_block_attn_workspace_bytes(c, 1, 64, 32, 8, 96, B.BF16, 0) == 0   # invalid


def _splits(c, B_, K, Hq, Hkv, D=128, dtype=B.BF16, num_splits=0):
    """Split count of the automatic plan, read back from the workspace size."""
    n = B.orthrus_block_attn_workspace_bytes(c, B_, K, Hq, Hkv, D, dtype, num_splits)
    if n == 0:
        return 1
    mpad = -(-(Hq // Hkv) * K // 32) * 32
    per_split = B_ * Hkv * mpad
    for s in range(1, 4097):
        if -(-per_split * s * D * 2 // 256) * 256 + per_split * s * 4 == n:
            return s
    raise AssertionError(f"no split count gives {n} bytes")


def test_automatic_split_plan_of_the_workloads():
    # Qwen3-8B shape, L = 8,192, K = 32: 26 splits of 320 keys -> 208 work-groups
    assert _splits(cache(capacity=8224, max_len=8192), 1, 32, 32, 8) == 26
    # Qwen3-1.7B layer, L = 2,048: the 128-key minimum decides (16 splits)
    assert _splits(cache(capacity=2080, max_len=2048), 1, 32, 16, 8) == 16
    # 131,072 keys with the workload's explicit 64 partitions
    assert _splits(cache(capacity=131136, max_len=131072), 1, 32, 32, 8, num_splits=64) == 64
    # paged, 32 requests up to 8,192 keys (+32 appended rows): work-list items of
    # at most 3,584 keys -> 3 split slots per request over the page table's range
    pc = cache(layout=B.PAGED, pages=20000, maxp=515, max_len=0)
    assert _splits(pc, 32, 32, 32, 8) == 3
    # no split below two tiles of keys
    assert _splits(cache(capacity=200, max_len=128), 1, 32, 32, 8) == 1


def test_consensus_validation_and_workspace():
    f = B.lib().orthrus_consensus
    args = [FAKE, FAKE, 1, 32, 151936, B.BF16] + [FAKE] * 7
    need = B.orthrus_consensus_workspace_bytes(1, 32, 151936, B.BF16)
    chunks = -(-151936 * 2 // 16384)
    assert need == 2 * 32 * chunks * 8
    assert f(*args, FAKE, need - 8, None) == B.ERR_WORKSPACE
    assert f(*args, None, need, None) == B.ERR_WORKSPACE
    bad = list(args)
    bad[0] = None
    assert f(*bad, FAKE, need, None) == B.ERR_NULL
    bad = list(args)
    bad[5] = 9
    assert f(*bad, FAKE, need, None) == B.ERR_DTYPE
    bad = list(args)
    bad[3] = 65
    assert f(*bad, FAKE, need, None) == B.ERR_UNSUPPORTED
    bad = list(args)
    bad[4] = 0
    assert f(*bad, FAKE, need, None) == B.ERR_SHAPE
    assert B.orthrus_argmax_workspace_bytes(10, 1000, B.F32) == 10 * 1 * 8
    assert B.lib().orthrus_argmax(FAKE, 0, 10, B.F32, FAKE, FAKE, 8, None) == B.ERR_SHAPE


def test_lmhead_argmax_validation_and_workspace():
    f = B.lib().orthrus_lmhead_argmax
    ws_bytes = B.orthrus_lmhead_argmax_workspace_bytes
    # R rows x ceil(V / 128) vocabulary blocks of 64-bit keys
    assert ws_bytes(32, 4096, 151936, B.BF16) == 32 * 1187 * 8
    assert ws_bytes(1, 128, 1, B.BF16) == 8
    assert ws_bytes(32, 4096, 151936, B.F32) == 0        # bf16 only
    assert ws_bytes(32, 100, 1000, B.BF16) == 0          # H not a multiple of 128
    need = ws_bytes(32, 4096, 151936, B.BF16)

    def call(hidden=FAKE, weight=FAKE, R=32, H=4096, V=151936, dtype=B.BF16, idx=FAKE, ws=FAKE,
             wsb=need):
        return f(hidden, weight, R, H, V, dtype, idx, ws, wsb, None)

    assert call(hidden=None) == B.ERR_NULL
    assert call(weight=None) == B.ERR_NULL
    assert call(idx=None) == B.ERR_NULL
    assert call(dtype=7) == B.ERR_DTYPE
    assert call(R=0) == B.ERR_SHAPE
    assert call(V=0) == B.ERR_SHAPE
    assert call(dtype=B.F32) == B.ERR_UNSUPPORTED
    assert call(H=4000) == B.ERR_UNSUPPORTED
    assert call(H=96) == B.ERR_UNSUPPORTED
    assert call(H=32) == B.ERR_UNSUPPORTED
    assert call(hidden=FAKE + 2) == B.ERR_UNSUPPORTED      # misaligned
    assert call(ws=None) == B.ERR_WORKSPACE
    assert call(wsb=need - 1) == B.ERR_WORKSPACE


def test_kv_append_validation():
    c = cache(capacity=100, max_len=0)
    f = B.lib().orthrus_kv_append
    base = [FAKE, FAKE, FAKE, FAKE + 4096, 1, 32, 8, 128, B.BF16, 1, 0, 0, None]
    b = list(base)
    b[2] = None
    assert f(ctypes.byref(c), *b) == B.ERR_NULL
    b = list(base)
    b[7] = 80
    assert f(ctypes.byref(c), *b) == B.ERR_UNSUPPORTED
    b = list(base)
    b[9] = 0
    assert f(ctypes.byref(c), *b) == B.ERR_SHAPE
    b = list(base)
    b[9], b[10] = 2, 3        # layer stride not a multiple of 16 bytes
    assert f(ctypes.byref(c), *b) == B.ERR_UNSUPPORTED


def test_mdiff_attn_validation():
    f = B.lib().orthrus_mdiff_attn

    def call(**kw):
        a = dict(kc=FAKE, vc=FAKE, cap=4096, anchors=FAKE, hint=4096, q=FAKE, kb=FAKE, vb=FAKE,
                 out=FAKE, lse=None, B=1, NB=128, K=32, Hq=32, Hkv=8, D=128, dtype=B.BF16,
                 scale=0.088, splits=0, ws=None, wsb=0)
        a.update(kw)
        return f(a["kc"], a["vc"], a["cap"], a["anchors"], a["hint"], a["q"], a["kb"], a["vb"],
                 a["out"], a["lse"], a["B"], a["NB"], a["K"], a["Hq"], a["Hkv"], a["D"],
                 a["dtype"], a["scale"], a["splits"], a["ws"], a["wsb"], None)

    assert call(kc=None) == B.ERR_NULL
    assert call(anchors=None) == B.ERR_NULL
    assert call(q=None) == B.ERR_NULL
    assert call(NB=0) == B.ERR_SHAPE
    assert call(hint=5000) == B.ERR_SHAPE           # hint beyond the context
    assert call(cap=-1) == B.ERR_SHAPE
    assert call(K=65) == B.ERR_UNSUPPORTED
    assert call(D=96) == B.ERR_UNSUPPORTED
    assert call(dtype=7) == B.ERR_DTYPE
    assert call(q=FAKE + 8) == B.ERR_UNSUPPORTED     # misaligned
    # 1 x 128 blocks x 8 heads fill the chip without splits: no workspace
    assert B.lib().orthrus_mdiff_attn_workspace_bytes(4096, 4096, 1, 128, 32, 32, 8, 128,
                                                      B.BF16, 0) == 0
    need = B.lib().orthrus_mdiff_attn_workspace_bytes(4096, 4096, 1, 2, 32, 32, 8, 128,
                                                      B.BF16, 0)
    assert need > 0
    assert call(NB=2, ws=None, wsb=0) == B.ERR_WORKSPACE
    assert call(NB=2, ws=FAKE, wsb=need - 1) == B.ERR_WORKSPACE


def test_stream_read_validation():
    f = B.lib().orthrus_stream_read
    assert f(None, 1024, 4, FAKE, None) == B.ERR_NULL
    assert f(FAKE, 1024, 4, None, None) == B.ERR_NULL
    assert f(FAKE, 1000, 4, FAKE, None) == B.ERR_SHAPE        # not a multiple of 16
    assert f(FAKE, 0, 4, FAKE, None) == B.ERR_SHAPE
    assert f(FAKE, 1024, 0, FAKE, None) == B.ERR_SHAPE
    assert f(FAKE + 8, 1024, 4, FAKE, None) == B.ERR_UNSUPPORTED
    assert f(FAKE, 1024, 70000, FAKE, None) == B.ERR_UNSUPPORTED


def test_layer_validation_codes():
    L = B.lib()
    # orthrus_rmsnorm: H a multiple of 4, at most 16384; eps > 0
    assert L.orthrus_rmsnorm(None, FAKE, FAKE, 4, 4096, 1e-6, None) == B.ERR_NULL
    assert L.orthrus_rmsnorm(FAKE, FAKE, FAKE, 0, 4096, 1e-6, None) == B.ERR_SHAPE
    assert L.orthrus_rmsnorm(FAKE, FAKE, FAKE, 4, 4096, 0.0, None) == B.ERR_SHAPE
    assert L.orthrus_rmsnorm(FAKE, FAKE, FAKE, 4, 4094, 1e-6, None) == B.ERR_UNSUPPORTED
    assert L.orthrus_rmsnorm(FAKE, FAKE, FAKE, 4, 16388, 1e-6, None) == B.ERR_UNSUPPORTED
    assert L.orthrus_rmsnorm(FAKE + 8, FAKE, FAKE, 4, 4096, 1e-6, None) == B.ERR_UNSUPPORTED
    assert L.orthrus_swiglu(FAKE, FAKE, 4, 1002, None) == B.ERR_UNSUPPORTED
    # the fused projections: partial sums always written
    ew = B.orthrus_gemm_epilogue_workspace_bytes
    assert ew(32, 4096, 4096) == 8 * 32 * 4096 * 4            # split 8 ways
    assert ew(32, 24576, 4096) == 1 * 32 * 24576 * 4           # not split, still written
    assert ew(32, 6144, 4096) == 4 * 32 * 6144 * 4             # split 4 ways
    assert ew(32, 4096, 12288) == 8 * 32 * 4096 * 4           # split 8 ways
    assert ew(7, 264, 64) == 7 * 264 * 4                        # not split, still written
    assert ew(32, 4096, 100) == 0
    assert B.orthrus_gemm_workspace_bytes(7, 264, 64) == 0
    g = L.orthrus_gemm_rmsnorm
    need = ew(32, 4096, 4096)
    assert g(None, FAKE, FAKE, FAKE, FAKE, 32, 4096, 4096, 1e-6, FAKE, need, None) == B.ERR_NULL
    assert g(FAKE, FAKE, None, FAKE, FAKE, 32, 4096, 4096, 1e-6, FAKE, need, None) == B.ERR_NULL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4096, 4000, 1e-6, FAKE, need,
             None) == B.ERR_UNSUPPORTED                          # Kin not a multiple of 64
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4098, 4096, 1e-6, FAKE, need,
             None) == B.ERR_UNSUPPORTED                          # H not a multiple of 4
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4096, 4096, 1e-6, FAKE, need - 4,
             None) == B.ERR_WORKSPACE
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4096, 4096, 1e-6, None, need,
             None) == B.ERR_WORKSPACE
    sw = L.orthrus_gemm_swiglu
    need = ew(32, 24576, 4096)
    assert sw(FAKE, FAKE, None, 32, 12288, 4096, FAKE, need, None) == B.ERR_NULL
    assert sw(FAKE, FAKE, FAKE, 32, 0, 4096, FAKE, need, None) == B.ERR_SHAPE
    assert sw(FAKE, FAKE, FAKE, 32, 1 << 30, 4096, FAKE, need, None) == B.ERR_SHAPE  # 2I overflows
    assert sw(FAKE, FAKE, FAKE, 32, 12286, 4096, FAKE, need, None) == B.ERR_UNSUPPORTED
    assert sw(FAKE, FAKE, FAKE, 32, 12288, 4096, FAKE, need - 1, None) == B.ERR_WORKSPACE
    qk = L.orthrus_gemm_qk_norm_rope
    need = ew(32, 6144, 4096)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, 32, 32, 8, 128, 4096, 1e-6, 1e6,
            FAKE, need, None]
    bad = list(args); bad[4] = None
    assert qk(*bad) == B.ERR_NULL                                # lens
    bad = list(args); bad[9] = 33
    assert qk(*bad) == B.ERR_SHAPE                               # R not a multiple of K
    bad = list(args); bad[12] = 64
    assert qk(*bad) == B.ERR_UNSUPPORTED                         # D = 128 only
    bad = list(args); bad[10] = 1 << 20
    assert qk(*bad) == B.ERR_UNSUPPORTED                         # absurd head counts
    bad = list(args); bad[17] = need - 4
    assert qk(*bad) == B.ERR_WORKSPACE


def test_pack_weight_sizes_and_validation():
    pb = B.orthrus_packed_weight_bytes
    assert pb(6144, 4096) == 6144 * 4096 * 2                   # whole 128-row blocks
    assert pb(151936, 4096) == 1187 * 128 * 4096 * 2           # the Qwen3 vocabulary: 1,187 blocks
    assert pb(132, 64) == 256 * 64 * 2                          # ragged: padded to 256 rows
    assert pb(1, 192) == 128 * 192 * 2
    assert pb(0, 64) == 0 and pb(128, 0) == 0 and pb(128, 100) == 0 and pb(128, 32) == 0
    P = B.lib().orthrus_pack_weight
    need = pb(132, 64)
    assert P(None, 132, 64, FAKE, need, None) == B.ERR_NULL
    assert P(FAKE, 132, 64, None, need, None) == B.ERR_NULL
    assert P(FAKE, 0, 64, FAKE, need, None) == B.ERR_SHAPE
    assert P(FAKE, 132, 100, FAKE, need, None) == B.ERR_UNSUPPORTED   # Kin not a multiple of 64
    assert P(FAKE + 8, 132, 64, FAKE, need, None) == B.ERR_UNSUPPORTED
    assert P(FAKE, 132, 64, FAKE + 8, need, None) == B.ERR_UNSUPPORTED
    assert P(FAKE, 132, 64, FAKE, need - 2, None) == B.ERR_WORKSPACE
    G = B.lib().orthrus_pack_weight_gate_up
    need = pb(2 * 132, 64)
    assert G(None, 132, 64, FAKE, need, None) == B.ERR_NULL
    assert G(FAKE, 0, 64, FAKE, need, None) == B.ERR_SHAPE
    assert G(FAKE, 1 << 30, 64, FAKE, need, None) == B.ERR_SHAPE       # 2I would overflow an int
    assert G(FAKE, 130, 64, FAKE, need, None) == B.ERR_UNSUPPORTED    # I not a multiple of 4
    assert G(FAKE, 132, 96, FAKE, need, None) == B.ERR_UNSUPPORTED    # Kin not a multiple of 64
    assert G(FAKE, 132, 64, FAKE, need - 2, None) == B.ERR_WORKSPACE


def test_single_hip_runtime_in_process():
    import torch  # noqa: F401
    B.lib()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths
