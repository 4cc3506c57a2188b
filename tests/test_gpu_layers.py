"""GPU parity of the decode step's layer kernels against fp64 references
(oracle.model's pieces and numpy fp64 matrix products on the same bf16
values), through the C ABI.  Bounds: fp32 accumulation over n terms is
within n * 2^-24 * sum|terms| (plus 1% slack), and a bf16 output carries
half an ulp (2^-9 relative); the copies and the token kernels are exact."""
import numpy as np
import pytest
import torch

import oracle
from ar_shared_kv_amd import _binding as B_
from ar_shared_kv_amd import api
from gpu_util import record, say
from oracle import model as M

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bf(shape, gen, std=1.0):
    return (torch.randn(shape, generator=gen) * std).to(torch.bfloat16)


@pytest.mark.parametrize("R,N,Kin,out", [
    (32, 6144, 4096, "f32"),      # QKV projection, split 4 ways
    (32, 4096, 4096, "f32"),      # output projection, split 8 ways
    (32, 24576, 4096, "f32"),     # gate/up projection
    (32, 4096, 12288, "f32"),     # down projection
    (1, 6144, 4096, "f32"),       # one row (plain decoding)
    (50, 1000, 256, "bf16"),      # 64-row blocks, ragged N blocks, no split
    (200, 512, 1024, "f32"),      # 128-row blocks
    (7, 132, 64, "bf16"),         # one chunk, ragged N
])
def test_gemm_matches_fp64(R, N, Kin, out):
    gen = torch.Generator().manual_seed(R * 7 + N)
    x, w = bf((R, Kin), gen), bf((N, Kin), gen, Kin ** -0.5)
    res = torch.randn((R, N), generator=gen)
    ref = x.double().numpy() @ w.double().numpy().T + res.double().numpy()
    mag = np.abs(x.double().numpy()) @ np.abs(w.double().numpy()).T
    bound = 1.01 * Kin * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(ref)
    if out == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref)
    xd, wd, rd = x.to(DEV), api.pack_weight(w.to(DEV)), res.to(DEV)
    y = torch.empty((R, N), dtype=torch.float32 if out == "f32" else torch.bfloat16, device=DEV)
    n = B_.orthrus_gemm_workspace_bytes(R, N, Kin)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
    dt = B_.F32 if out == "f32" else B_.BF16
    say(f"gemm R={R} N={N} Kin={Kin} out={out} workspace={n}")
    B_.check("orthrus_gemm", B_.orthrus_gemm(xd, wd, rd, y, R, N, Kin, dt, ws, ws.numel()))
    torch.cuda.synchronize()
    err = np.abs(y.double().cpu().numpy() - ref)
    record("gemm", f"R={R} N={N} Kin={Kin} {out}", max_err=float(err.max()),
           bound=float(bound.max()), worst_ratio=float((err / bound).max()))
    assert (err <= bound).all(), float((err / bound).max())
    # in place: y = y + x W^T with the residual in y
    if out == "f32":
        y2 = rd.clone()
        B_.check("orthrus_gemm", B_.orthrus_gemm(xd, wd, y2, y2, R, N, Kin, dt, ws, ws.numel()))
        torch.cuda.synchronize()
        assert torch.equal(y2, y)


@pytest.mark.parametrize("N,Kin", [(6144, 4096), (132, 64), (1, 192), (300, 128)])
def test_pack_weight_is_the_tile_permutation(N, Kin):
    """The packed layout is a pure rearrangement: tile (block, chunk) holds
    rows 128*block.. and columns 64*chunk.. in row order, blocks padded with
    zero rows; checked bit for bit against a numpy reshape of the weight."""
    gen = torch.Generator().manual_seed(N + Kin)
    w = bf((N, Kin), gen)
    pw = api.pack_weight(w.to(DEV))
    torch.cuda.synchronize()
    nb = (N + 127) // 128
    assert pw.data.numel() * 2 == B_.orthrus_packed_weight_bytes(N, Kin) == nb * 128 * Kin * 2
    wp = np.zeros((nb * 128, Kin), np.uint16)
    wp[:N] = w.view(torch.int16).numpy().view(np.uint16)
    ref = wp.reshape(nb, 128, Kin // 64, 64).transpose(0, 2, 1, 3).reshape(-1)
    got = pw.data.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("I,Kin", [(12288, 64), (132, 64), (4, 128)])
def test_pack_weight_gate_up_pairs_gate_and_up_rows(I, Kin):
    """Every 8 packed rows are gate rows 4g..4g+3 and then up rows
    I+4g..I+4g+3, packed as orthrus_pack_weight packs; bit for bit."""
    gen = torch.Generator().manual_seed(I + Kin)
    w = bf((2 * I, Kin), gen)
    pw = api.pack_weight_gate_up(w.to(DEV))
    torch.cuda.synchronize()
    g = np.arange(2 * I) // 8
    j = np.arange(2 * I) % 8
    src = np.where(j < 4, 4 * g + j, I + 4 * g + j - 4)
    paired = w[torch.from_numpy(src)].contiguous()
    ref = api.pack_weight(paired.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(pw.data, ref.data)
    assert pw.gate_up and not ref.gate_up


def test_gemm_rows_do_not_depend_on_the_batch():
    gen = torch.Generator().manual_seed(3)
    x, w = bf((32, 4096), gen), bf((6144, 4096), gen, 4096 ** -0.5)
    xd, wd = x.to(DEV), api.pack_weight(w.to(DEV))
    ws = torch.empty(B_.orthrus_gemm_workspace_bytes(32, 6144, 4096) + 16, dtype=torch.uint8,
                     device=DEV)
    y32 = torch.empty((32, 6144), dtype=torch.float32, device=DEV)
    B_.check("gemm", B_.orthrus_gemm(xd, wd, None, y32, 32, 6144, 4096, B_.F32, ws, ws.numel()))
    for r in (0, 17, 31):
        y1 = torch.empty((1, 6144), dtype=torch.float32, device=DEV)
        x1 = xd[r:r + 1].contiguous()
        B_.check("gemm", B_.orthrus_gemm(x1, wd, None, y1, 1, 6144, 4096, B_.F32, ws, ws.numel()))
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y32[r])
    # 64- and 128-row work-groups add in the same order
    for R in (50, 100):
        xr = torch.cat([xd, bf((R - 32, 4096), gen).to(DEV)])
        wsr = torch.empty(B_.orthrus_gemm_workspace_bytes(R, 6144, 4096) + 16, dtype=torch.uint8,
                          device=DEV)
        yr = torch.empty((R, 6144), dtype=torch.float32, device=DEV)
        B_.check("gemm", B_.orthrus_gemm(xr, wd, None, yr, R, 6144, 4096, B_.F32, wsr,
                                         wsr.numel()))
        torch.cuda.synchronize()
        assert torch.equal(yr[:32], y32)


def test_rmsnorm_swiglu_embed():
    gen = torch.Generator().manual_seed(4)
    R, H, I = 33, 4096, 12288
    x = torch.randn((R, H), generator=gen) * 3
    w = bf((H,), gen)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=DEV)
    B_.check("rmsnorm", B_.orthrus_rmsnorm(x.to(DEV), w.to(DEV), y, R, H, 1e-6))
    ref = M.rmsnorm(x.double().numpy(), w.double().numpy(), 1e-6)
    err = np.abs(y.double().cpu().numpy() - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()).all()
    gu = torch.randn((R, 2 * I), generator=gen) * 4
    act = torch.empty((R, I), dtype=torch.bfloat16, device=DEV)
    B_.check("swiglu", B_.orthrus_swiglu(gu.to(DEV), act, R, I))
    g, u = gu[:, :I].double().numpy(), gu[:, I:].double().numpy()
    ref = M.silu(g) * u
    err = np.abs(act.double().cpu().numpy() - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6).all()
    table = bf((100, H), gen)
    tok = torch.tensor([5, 0, 99, 5], dtype=torch.int32)
    h = torch.empty((4, H), dtype=torch.float32, device=DEV)
    B_.check("embed", B_.orthrus_embed(tok.to(DEV), table.to(DEV), h, 4, H))
    torch.cuda.synchronize()
    assert torch.equal(h.cpu(), table[tok.long()].float())


@pytest.mark.parametrize("B,K,lens", [(1, 32, [8192]), (3, 5, [0, 17, 100000])])
def test_qk_norm_rope(B, K, lens):
    gen = torch.Generator().manual_seed(5)
    Hq, Hkv, D = 32, 8, 128
    R = B * K
    qkv = torch.randn((R, (Hq + 2 * Hkv) * D), generator=gen) * 2
    wq, wk = bf((D,), gen), bf((D,), gen)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    q = torch.empty((R, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((R, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((R, Hkv, D), dtype=torch.bfloat16, device=DEV)
    B_.check("qk_norm_rope", B_.orthrus_qk_norm_rope(qkv.to(DEV), wq.to(DEV), wk.to(DEV),
                                                    lens_t.to(DEV), K, q, k, v, R, Hq, Hkv, D,
                                                    1e-6, 1e6))
    torch.cuda.synchronize()
    a = qkv.double().numpy()
    pos = (np.asarray(lens)[:, None] + np.arange(K)[None, :]).reshape(-1)
    rq = M.rope(M.rmsnorm(a[:, :Hq * D].reshape(R, Hq, D), wq.double().numpy(), 1e-6), pos, 1e6)
    rk = M.rope(M.rmsnorm(a[:, Hq * D:(Hq + Hkv) * D].reshape(R, Hkv, D), wk.double().numpy(),
                          1e-6), pos, 1e6)
    rv = a[:, (Hq + Hkv) * D:].reshape(R, Hkv, D)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        err = np.abs(got.double().cpu().numpy() - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 2e-5 * np.abs(ref).max()
        record("qk_norm_rope", f"{name} B={B} K={K}", max_err=float(err.max()),
               bound=float(bound.max()))
        assert (err <= bound).all(), (name, float((err / bound).max()))


def _ws(n):
    return torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("R,H,Kin", [
    (32, 4096, 4096),      # output projection: split 8 ways
    (32, 4096, 12288),     # down projection: split 8 ways
    (5, 256, 64),          # not split; one float4 group per thread, most threads idle
    (3, 8192, 128),        # two groups per thread
    (2, 16384, 64),        # four groups per thread (the largest H)
])
def test_gemm_rmsnorm_equals_gemm_then_rmsnorm(R, H, Kin):
    gen = torch.Generator().manual_seed(R * 13 + H + Kin)
    x, w = bf((R, Kin), gen).to(DEV), api.pack_weight(bf((H, Kin), gen, Kin ** -0.5).to(DEV))
    nw = bf((H,), gen).to(DEV)
    h0 = (torch.randn((R, H), generator=gen) * 2).to(DEV)
    say(f"gemm_rmsnorm R={R} H={H} Kin={Kin}")
    ha, xa = h0.clone(), torch.empty((R, H), dtype=torch.bfloat16, device=DEV)
    ws = _ws(B_.orthrus_gemm_workspace_bytes(R, H, Kin))
    B_.check("gemm", B_.orthrus_gemm(x, w, ha, ha, R, H, Kin, B_.F32, ws, ws.numel()))
    B_.check("rmsnorm", B_.orthrus_rmsnorm(ha, nw, xa, R, H, 1e-6))
    hb, xb = h0.clone(), torch.empty((R, H), dtype=torch.bfloat16, device=DEV)
    ws2 = _ws(B_.orthrus_gemm_epilogue_workspace_bytes(R, H, Kin))
    B_.check("gemm_rmsnorm", B_.orthrus_gemm_rmsnorm(x, w, hb, nw, xb, R, H, Kin, 1e-6, ws2,
                                                     ws2.numel()))
    torch.cuda.synchronize()
    assert torch.equal(ha, hb)
    assert torch.equal(xa, xb)
    # and the norm itself against fp64
    ref = M.rmsnorm(hb.double().cpu().numpy(), nw.double().cpu().numpy(), 1e-6)
    err = np.abs(xb.double().cpu().numpy() - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()).all()


@pytest.mark.parametrize("R,I,Kin", [
    (32, 12288, 4096),     # the Qwen3-8B MLP: not split, SwiGLU in the projection's epilogue
    (7, 132, 64),          # not split, ragged last block (264 rows in 3 blocks)
    (40, 1024, 512),       # split 2 ways: paired partial sums, separate SwiGLU pass
    (100, 256, 4096),      # 128-row work-groups, split 16 ways
    (70, 96, 128),         # 128-row work-groups, not split, one ragged block
])
def test_gemm_swiglu_equals_gemm_then_swiglu(R, I, Kin):
    gen = torch.Generator().manual_seed(R + I + Kin)
    wr = bf((2 * I, Kin), gen, Kin ** -0.5).to(DEV)
    x, w = bf((R, Kin), gen).to(DEV), api.pack_weight(wr)
    wp = api.pack_weight_gate_up(wr)
    say(f"gemm_swiglu R={R} I={I} Kin={Kin}")
    gu = torch.empty((R, 2 * I), dtype=torch.float32, device=DEV)
    ws = _ws(B_.orthrus_gemm_workspace_bytes(R, 2 * I, Kin))
    B_.check("gemm", B_.orthrus_gemm(x, w, None, gu, R, 2 * I, Kin, B_.F32, ws, ws.numel()))
    a1 = torch.empty((R, I), dtype=torch.bfloat16, device=DEV)
    B_.check("swiglu", B_.orthrus_swiglu(gu, a1, R, I))
    a2 = torch.empty_like(a1)
    ws2 = _ws(B_.orthrus_gemm_epilogue_workspace_bytes(R, 2 * I, Kin))
    B_.check("gemm_swiglu", B_.orthrus_gemm_swiglu(x, wp, a2, R, I, Kin, ws2, ws2.numel()))
    torch.cuda.synchronize()
    assert torch.equal(a1, a2)


@pytest.mark.parametrize("B,K,Kin,lens", [(1, 32, 4096, [8192]), (3, 5, 256, [0, 17, 100000])])
def test_gemm_qk_norm_rope_equals_gemm_then_qk_norm_rope(B, K, Kin, lens):
    gen = torch.Generator().manual_seed(B * 100 + K)
    Hq, Hkv, D = 32, 8, 128
    R, N = B * K, (Hq + 2 * Hkv) * D
    x, w = bf((R, Kin), gen).to(DEV), api.pack_weight(bf((N, Kin), gen, Kin ** -0.5).to(DEV))
    wq, wk = bf((D,), gen).to(DEV), bf((D,), gen).to(DEV)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    say(f"gemm_qk_norm_rope B={B} K={K} Kin={Kin}")
    qkv = torch.empty((R, N), dtype=torch.float32, device=DEV)
    ws = _ws(B_.orthrus_gemm_workspace_bytes(R, N, Kin))
    B_.check("gemm", B_.orthrus_gemm(x, w, None, qkv, R, N, Kin, B_.F32, ws, ws.numel()))
    outs = []
    for fused in (False, True):
        q = torch.empty((R, Hq, D), dtype=torch.bfloat16, device=DEV)
        k = torch.empty((R, Hkv, D), dtype=torch.bfloat16, device=DEV)
        v = torch.empty((R, Hkv, D), dtype=torch.bfloat16, device=DEV)
        if fused:
            ws2 = _ws(B_.orthrus_gemm_epilogue_workspace_bytes(R, N, Kin))
            B_.check("gemm_qk", B_.orthrus_gemm_qk_norm_rope(x, w, wq, wk, lens_t, K, q, k, v, R,
                                                             Hq, Hkv, D, Kin, 1e-6, 1e6, ws2,
                                                             ws2.numel()))
        else:
            B_.check("qk", B_.orthrus_qk_norm_rope(qkv, wq, wk, lens_t, K, q, k, v, R, Hq, Hkv,
                                                   D, 1e-6, 1e6))
        outs.append((q, k, v))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_block_tokens_and_consensus_tokens():
    B, K = 3, 6
    anchor = torch.tensor([7, 8, 9], dtype=torch.int32, device=DEV)
    cand = torch.arange(B * K, dtype=torch.int32, device=DEV).view(B, K) + 100
    out = torch.empty((B, K), dtype=torch.int32, device=DEV)
    B_.check("block_tokens", B_.orthrus_block_tokens(anchor, None, 999, out, B, K))
    torch.cuda.synchronize()
    assert out[:, 0].tolist() == [7, 8, 9] and (out[:, 1:] == 999).all()
    B_.check("block_tokens", B_.orthrus_block_tokens(anchor, cand, 999, out, B, K))
    torch.cuda.synchronize()
    assert torch.equal(out[:, 1:], cand[:, :K - 1])
    rng = np.random.default_rng(6)
    d = rng.integers(0, 3, (B, K)).astype(np.int32)
    a = d.copy()
    a[0, 2] = 5
    a[2, 0] = 4
    bufs = {k: torch.empty(s, dtype=torch.int32, device=DEV) for k, s in
            (("j", B), ("n", B), ("off", B + 1), ("em", B * K), ("anc", B))}
    B_.check("consensus_tokens", B_.orthrus_consensus_tokens(
        torch.from_numpy(d).to(DEV), torch.from_numpy(a).to(DEV), B, K, bufs["j"], bufs["n"],
        bufs["off"], bufs["em"], bufs["anc"]))
    torch.cuda.synchronize()
    r = oracle.consensus(d, a)
    assert bufs["n"].tolist() == r["n"].tolist() and bufs["j"].tolist() == r["j"].tolist()
    assert bufs["off"].tolist() == r["emit_off"].tolist()
    assert bufs["em"][:int(r["emit_off"][-1])].tolist() == r["emitted"].tolist()
    assert bufs["anc"].tolist() == r["next_anchor"].tolist()
