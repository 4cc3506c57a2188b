"""The whole decode step on the GPU (ar_shared_kv_amd.decode: layers, both
views' block attention, fused LM-head argmax, consensus, multi-layer append)
against the fp64 oracle model, and the lossless loop on the GPU.

One step at the Qwen3-8B shapes (hidden 4,096, 32 query / 8 KV heads of 128,
MLP 12,288, vocabulary 151,936, two layers) from a synthetic cache of 300
tokens: the final hidden rows of both views, the appended K/V rows of both
layers and the greedy tokens are compared with the oracle.  Tokens must match
wherever the oracle's top-2 logit gap exceeds twice the bound on the logit
error that the measured hidden-state error allows (Cauchy-Schwarz with the
largest LM-head row norm, plus the fp32 accumulation bound).

The loop (hidden 4,096, the same heads, vocabulary 32,000, two layers):
Orthrus steps with candidates from a noisy copy of the greedy continuation
(so that long prefixes are accepted) emit exactly the stream of plain greedy
decoding run with the same kernels, and that stream matches the oracle's
greedy stream for as long as the oracle's margins are clear."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from ar_shared_kv_amd import _binding as B_
from ar_shared_kv_amd.decode import DecodeModel, Dims
from gpu_util import record, say
from oracle import model as M

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dims_of(d: Dims) -> M.Dims:
    return M.Dims(H=d.H, Hq=d.Hq, Hkv=d.Hkv, D=d.D, I=d.I, V=d.V, layers=d.layers, eps=d.eps,
                  theta=d.theta)


def token_check(name, gpu_tok, x_gpu, x_ref, logits_ref, w_lm):
    """Greedy tokens against the oracle's, row by row.  The GPU decides on
    w_v . x_gpu (fp32), the oracle on w_v . x_ref (fp64); with dx = x_gpu -
    x_ref, the logit difference of two tokens u, v moves by (w_u - w_v) . dx
    plus the fp32 accumulation error, at most b = H 2^-24 sum_k |x_k w_vk|
    <= H 2^-24 |x| max_v |w_v|.
    The worst case |w_u - w_v| |dx| is far above the gaps of a random head,
    so rows are classed by the size that error takes for a dx not aligned
    with the weight rows: standard deviation s = |dx| max|w_v| / sqrt(H).
    Where the oracle's top-2 gap exceeds 2 (6 s + b) the tokens must be
    equal; every other row must pick a token whose oracle logit is within
    2 (|dx| max|w_v| + b) of the maximum (the worst-case bound)."""
    dx = np.linalg.norm(x_gpu - x_ref, axis=1)
    wmax = np.sqrt((w_lm.astype(np.float64) ** 2).sum(axis=1).max())
    H = x_ref.shape[1]
    clear = equal = 0
    for r in range(len(gpu_tok)):
        top = np.sort(logits_ref[r])[-2:]
        b = H * 2.0 ** -24 * np.linalg.norm(x_gpu[r]) * wmax
        sigma = dx[r] * wmax / np.sqrt(H)
        ref_tok = int(np.argmax(logits_ref[r]))
        equal += int(gpu_tok[r] == ref_tok)
        if top[1] - top[0] > 2 * (6 * sigma + b):
            assert gpu_tok[r] == ref_tok, (name, r, gpu_tok[r], ref_tok, top, sigma)
            clear += 1
        else:
            worst = dx[r] * wmax + b
            assert logits_ref[r, gpu_tok[r]] >= top[1] - 2 * worst, (name, r)
    say(f"  {name}: {equal}/{len(gpu_tok)} rows equal to the oracle's token; "
        f"{clear} with a margin above 6 sigma, all of those equal")
    record("decode-tokens", name, rows=len(gpu_tok), equal_rows=equal, clear_rows=clear,
           mismatches_on_clear_rows=0)
    return clear


def test_one_step_qwen3_8b_shapes_against_oracle():
    d = Dims(layers=2)
    md = dims_of(d)
    w = W.model_weights(md, seed=7)
    B, K, L = 1, 32, 300
    cap = L + K
    gen = torch.Generator().manual_seed(9)
    kc = (torch.randn((d.layers, B, d.Hkv, cap, d.D), generator=gen)).to(torch.bfloat16)
    vc = (torch.randn((d.layers, B, d.Hkv, cap, d.D), generator=gen)).to(torch.bfloat16)
    draft = torch.randint(0, d.V, (B, K), generator=gen, dtype=torch.int32)
    anchor = torch.tensor([1234], dtype=torch.int32)
    say("decode step: building the GPU model")
    gm = DecodeModel(d, w, B, K, cap)
    gm.kc.copy_(kc)
    gm.vc.copy_(vc)
    gm.set_lengths(L)
    gm.anchor.copy_(anchor)
    gm.orthrus_step(draft=draft.to(DEV), keep_hidden=True)
    torch.cuda.synchronize()
    x_diff, x_ar = gm.x_diff.double().cpu().numpy(), gm.x_ar.double().cpu().numpy()
    d_tok, a_tok = gm.d_tok.cpu().numpy(), gm.a_tok.cpu().numpy()
    n = gm.n_emit.cpu().numpy()
    say("decode step: oracle")
    om = M.Model(md, w)
    caches = [(kc[l].double().numpy(), vc[l].double().numpy()) for l in range(d.layers)]
    lens = np.array([L], np.int32)
    blk = np.full((B, K), d.V, np.int64)
    blk[:, 0] = anchor.numpy()
    xd_ref, lg_d, _ = om.forward(blk, "diff", caches, lens, oracle.BIDIR)
    ar_in = np.concatenate([anchor.numpy()[:, None], draft.numpy()[:, :K - 1]], axis=1)
    xa_ref, lg_a, kv = om.forward(ar_in, "ar", caches, lens, oracle.CAUSAL)
    for name, xg, xr in (("diffusion", x_diff, xd_ref), ("AR", x_ar, xa_ref)):
        rel = np.linalg.norm(xg - xr, axis=1) / np.linalg.norm(xr, axis=1)
        record("decode-hidden", f"{name} view final hidden", max_rel=float(rel.max()),
               bound=0.05)
        say(f"  {name} final hidden: max relative error {rel.max():.3e}")
        assert rel.max() <= 0.05
    wl = w["lm_head"].float().numpy()
    clear = token_check("diffusion tokens", d_tok.reshape(-1), x_diff, xd_ref, lg_d, wl)
    clear += token_check("AR tokens", a_tok.reshape(-1), x_ar, xa_ref, lg_a, wl)
    assert clear >= 32          # at least half of the 64 rows are decided by the test
    # consensus of the GPU's own tokens, and the appended rows of both layers
    r = oracle.consensus(draft.numpy(), a_tok)
    assert n.tolist() == r["n"].tolist()
    assert gm.lens.cpu().tolist() == [L + int(n[0])]
    for l in range(d.layers):
        for name, got, ref in (("k", gm.kc[l], kv[l][0]), ("v", gm.vc[l], kv[l][1])):
            rows = got[0, :, L:L + int(n[0])].double().cpu().numpy()          # [Hkv, n, D]
            refr = np.transpose(ref[0, :int(n[0])], (1, 0, 2))
            err = np.abs(rows - refr).max()
            scale = np.abs(refr).max()
            record("decode-append", f"layer {l} {name}", max_err=float(err),
                   bound=float(0.03 * scale))
            assert err <= 0.03 * scale, (l, name, err, scale)
            # nothing past the accepted rows was written
            assert torch.equal(got[0, :, L + int(n[0]):].cpu(),
                               (kc if name == "k" else vc)[l, 0, :, L + int(n[0]):])


def test_orthrus_loop_equals_greedy_on_gpu_and_oracle():
    d = Dims(layers=2, V=32000)
    md = dims_of(d)
    w = W.model_weights(md, seed=8)
    B, K, P, n_tok = 2, 8, 40, 48
    cap = P + n_tok + 3 * K
    gen = torch.Generator().manual_seed(10)
    prompts = torch.randint(0, d.V, (B, P), generator=gen, dtype=torch.int32)
    say("loop: GPU greedy")
    gg = DecodeModel(d, w, B, K, cap)
    gg.prefill(prompts.to(DEV))
    greedy = [gg.anchor.cpu().clone()]
    for _ in range(n_tok + 2 * K):
        gg.greedy_step()
        greedy.append(gg.anchor.cpu().clone())
    greedy = torch.stack(greedy, 1).numpy()                   # [B, n_tok + 2K + 1]
    say("loop: GPU Orthrus")
    go = DecodeModel(d, w, B, K, cap)
    go.prefill(prompts.to(DEV))
    streams = [[int(t)] for t in go.anchor.cpu()]
    rng = np.random.default_rng(11)
    accepted = []
    while min(len(s) for s in streams) < n_tok:
        draft = np.zeros((B, K), np.int32)
        for b in range(B):
            p = len(streams[b])
            draft[b] = np.where(rng.random(K) < 0.8, greedy[b, p:p + K], rng.integers(0, d.V, K))
        go.orthrus_step(draft=torch.from_numpy(draft).to(DEV))
        off = go.emit_off.cpu().tolist()
        em = go.emitted.cpu().tolist()
        go.sync_lengths()
        for b in range(B):
            streams[b] += em[off[b]:off[b + 1]]
            accepted.append(off[b + 1] - off[b])
    say(f"  accepted per step: mean {np.mean(accepted):.2f}, max {max(accepted)}")
    record("decode-loop", "orthrus vs greedy on GPU", steps=len(accepted),
           mean_accepted=float(np.mean(accepted)), max_accepted=int(max(accepted)))
    for b in range(B):
        m = min(len(streams[b]), greedy.shape[1])
        assert streams[b][:m] == greedy[b, :m].tolist(), b
    assert max(accepted) > 1
    say("loop: oracle greedy")
    om = M.Model(md, w, keep_f64=True)
    ref = M.greedy(om, prompts.numpy(), 16, cap)
    # equal up to the first position whose oracle margin is within the logit
    # error that the one-step test's hidden-state tolerance (5% relative)
    # allows; at least the first 8 tokens must agree
    wl = w["lm_head"].float().numpy().astype(np.float64)
    wmax = np.sqrt((wl ** 2).sum(axis=1).max())
    caches = M.new_caches(md, B, cap)
    lens, lg = M.prefill(om, prompts.numpy(), caches)
    x = None
    agree = np.zeros(B, int)
    done = np.zeros(B, bool)
    for t in range(16):
        top = np.sort(lg, axis=1)[:, -2:]
        for b in range(B):
            if done[b]:
                continue
            if greedy[b, t] == ref[b, t]:
                agree[b] += 1
            else:
                xn = np.sqrt(md.H) * 1.5 if x is None else np.linalg.norm(x[b])
                assert top[b, 1] - top[b, 0] < 2 * 0.05 * xn * wmax, (b, t, top[b])
                done[b] = True
        x, lg, kv = om.forward(ref[:, t:t + 1], "ar", caches, lens, oracle.CAUSAL)
        lens = M.append(caches, kv, lens, np.ones(B, np.int32))
    say(f"  GPU greedy == oracle greedy for the first {agree.tolist()} tokens")
    record("decode-loop", "GPU greedy vs oracle greedy", agreeing_prefix=agree.tolist())
    assert agree.min() >= 8


def test_orthrus_step_graph_replays_match_eager():
    """One whole Orthrus step (two layers, both views, the fused LM head,
    consensus, the multi-layer append) captured in a HIP graph: every replay,
    with its outputs scrambled and the step's inputs restored by eager work
    in between, reproduces the eager step bit for bit."""
    d = Dims(H=512, Hq=4, Hkv=2, D=128, I=1024, V=1000, layers=2)
    w = W.model_weights(dims_of(d), seed=21)
    B, K, L = 2, 8, 40
    gm = DecodeModel(d, w, B, K, L + K, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(22)
    gm.kc.copy_(torch.randn(gm.kc.shape, generator=g, device=DEV).to(torch.bfloat16))
    gm.vc.copy_(torch.randn(gm.vc.shape, generator=g, device=DEV).to(torch.bfloat16))
    gm.set_lengths(L)
    anchor0 = torch.tensor([7, 11], dtype=torch.int32, device=DEV)

    def prepare():
        gm.anchor.copy_(anchor0)
        gm.kc[:, :, :, L:].fill_(float("nan"))
        gm.vc[:, :, :, L:].fill_(float("nan"))
        for t in (gm.n_emit, gm.emit_off, gm.emitted, gm.d_tok, gm.a_tok):
            t.fill_(-7)
        gm.kb.fill_(float("nan"))
        gm.vb.fill_(float("nan"))
        gm.x.fill_(float("nan"))
        if hasattr(gm, "lens_next"):
            gm.lens_next.fill_(-7)

    def results():
        n = gm.n_emit.cpu().tolist()
        r = {k: getattr(gm, k).clone() for k in ("n_emit", "emit_off", "d_tok", "a_tok", "anchor",
                                                  "lens_next")}
        r["emitted"] = gm.emitted[: int(gm.emit_off[-1])].clone()
        r["kb"], r["vb"] = gm.kb.view(torch.int16).clone(), gm.vb.view(torch.int16).clone()
        r["x"] = gm.x[: B * K].view(torch.int16).clone()
        for b in range(B):
            r[f"kc{b}"] = gm.kc[:, b, :, L:L + n[b]].view(torch.int16).clone()
            r[f"vc{b}"] = gm.vc[:, b, :, L:L + n[b]].view(torch.int16).clone()
        return r

    prepare()
    gm.orthrus_step(advance=False)
    torch.cuda.synchronize()
    ref = results()
    say(f"graph decode step: eager n_emit {ref['n_emit'].tolist()}")
    assert int(gm.lens.max()) == L                          # the replayable form leaves lens
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        gm.orthrus_step(advance=False)
    for rep in range(3):
        prepare()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = results()
        say(f"graph decode step: replay {rep}")
        for k, v in ref.items():
            assert torch.equal(got[k], v), (rep, k)
