"""GPU parity of orthrus_kv_append (bit-exact against the oracle), a whole
decode step (both attention views + consensus + append) against the oracle,
and the losslessness loop run through the GPU consensus and append."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attn_close, cache_for, dev, f64, gpu_attn, oracle_attn, say
from ar_shared_kv_amd import api

pytestmark = pytest.mark.gpu


def raw(t):
    return t.detach().cpu().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_multi_layer_bit_exact(paged, dtype):
    layers, Bn, K, Hkv, D = 3, 5, 9, 2, 128
    lens = [0, 15, 16, 400, 77]
    step = W.custom_step(Bn, 4, Hkv, D, K, lens, dtype=dtype, paged=paged, seed=40)
    tdt = step.cfg.torch_dtype
    cshape = step.layers[0].k_cache.shape
    gen = torch.Generator().manual_seed(1)
    kc = torch.randn((layers, *cshape), generator=gen).to(tdt)
    vc = torch.randn((layers, *cshape), generator=gen).to(tdt)
    kb = torch.randn((layers, Bn, K, Hkv, D), generator=gen).to(tdt)
    vb = torch.randn((layers, Bn, K, Hkv, D), generator=gen).to(tdt)
    n = torch.tensor([9, 1, 4, 0, 7], dtype=torch.int32)
    kc_d, vc_d = dev(kc), dev(vc)
    c = api.make_cache(kc_d[0], vc_d[0], dev(step.lens),
                       page_table=dev(step.page_table) if paged else None)
    say(f"append paged={paged} dtype={dtype}")
    lens_out = api.kv_append(c, dev(kb)[0], dev(vb)[0], dev(n), num_layers=layers,
                             cache_layer_stride=kc[0].numel(), blk_layer_stride=kb[0].numel())
    torch.cuda.synchronize()
    rk, rv, rl = oracle.kv_append(raw(kc), raw(vc), raw(kb), raw(vb), n.numpy(),
                                  step.lens.numpy(),
                                  layout=oracle.PAGED if paged else oracle.CONTIGUOUS,
                                  page_table=step.page_table.numpy() if paged else None)
    np.testing.assert_array_equal(lens_out.cpu().numpy(), rl)
    assert np.array_equal(raw(kc_d), rk) and np.array_equal(raw(vc_d), rv)


@pytest.mark.parametrize("paged", [False, True])
def test_append_in_place_lens(paged):
    """lens_out may be the cache's own lens: rows land where the old lengths
    say, then the lengths advance."""
    layers, Bn, K, Hkv, D = 2, 6, 8, 2, 128
    lens = [0, 15, 16, 400, 77, 1000]
    step = W.custom_step(Bn, 4, Hkv, D, K, lens, paged=paged, seed=41)
    cshape = step.layers[0].k_cache.shape
    gen = torch.Generator().manual_seed(2)
    kc = torch.randn((layers, *cshape), generator=gen).to(torch.bfloat16)
    vc = torch.randn((layers, *cshape), generator=gen).to(torch.bfloat16)
    kb = torch.randn((layers, Bn, K, Hkv, D), generator=gen).to(torch.bfloat16)
    vb = torch.randn((layers, Bn, K, Hkv, D), generator=gen).to(torch.bfloat16)
    n = torch.tensor([8, 1, 4, 0, 7, 3], dtype=torch.int32)
    kc_d, vc_d, lens_d = dev(kc), dev(vc), dev(step.lens)
    c = api.make_cache(kc_d[0], vc_d[0], lens_d,
                       page_table=dev(step.page_table) if paged else None)
    say(f"append in place paged={paged}")
    out = api.kv_append(c, dev(kb)[0], dev(vb)[0], dev(n), lens_out=lens_d, num_layers=layers,
                        cache_layer_stride=kc[0].numel(), blk_layer_stride=kb[0].numel())
    torch.cuda.synchronize()
    assert out.data_ptr() == lens_d.data_ptr()
    rk, rv, rl = oracle.kv_append(raw(kc), raw(vc), raw(kb), raw(vb), n.numpy(),
                                  step.lens.numpy(),
                                  layout=oracle.PAGED if paged else oracle.CONTIGUOUS,
                                  page_table=step.page_table.numpy() if paged else None)
    np.testing.assert_array_equal(lens_d.cpu().numpy(), rl)
    assert np.array_equal(raw(kc_d), rk) and np.array_equal(raw(vc_d), rv)


@pytest.mark.parametrize("cid", [1, 2])
def test_full_step_against_oracle(cid):
    """One decode step: BIDIR pass, CAUSAL pass, consensus, append."""
    cfg = W.CONFIGS[cid]
    step = W.step_inputs(cfg)
    lay = step.layers[0]
    say(f"full step config{cid}")
    for view in ("diff", "ar"):
        o, l = gpu_attn(step, lay, view)
        ro, rl = oracle_attn(step, lay, view)
        assert_attn_close(o, l, ro, rl, cfg.torch_dtype, f"step config{cid} {view}")
    bufs = api.consensus(dev(step.diff_logits), dev(step.ar_logits))
    c = cache_for(step, lay)
    lens_out = api.kv_append(c, dev(lay.k_blk_ar), dev(lay.v_blk_ar), bufs.n_emit)
    torch.cuda.synchronize()
    d_ref = oracle.argmax_rows(f64(step.diff_logits))
    a_ref = oracle.argmax_rows(f64(step.ar_logits))
    r = oracle.consensus(d_ref, a_ref)
    np.testing.assert_array_equal(bufs.n_emit.cpu().numpy(), r["n"])
    rk, rv, rl = oracle.kv_append(raw(lay.k_cache)[None], raw(lay.v_cache)[None],
                                  raw(lay.k_blk_ar)[None], raw(lay.v_blk_ar)[None], r["n"],
                                  step.lens.numpy())
    np.testing.assert_array_equal(lens_out.cpu().numpy(), rl)
    assert np.array_equal(raw(c._keep[0])[None], rk) and np.array_equal(raw(c._keep[1])[None], rv)


VOCAB = 11


def _h(seq):
    x = 1469598103
    for t in seq:
        x = ((x ^ (int(t) + 1)) * 1099511) % 2147483647
    return x


def _next(seq):
    return _h(seq) % VOCAB


def _kv(seq):
    # exactly representable in fp32: integers below 2^24
    return [float(_h(seq) % 16777216), float(len(seq) * 64 + int(seq[-1]))]


def test_lossless_loop_through_gpu_consensus_and_append():
    """Toy AR/diffusion models driven through the GPU consensus and append
    emit the sequential greedy stream and build the sequential cache."""
    rng = np.random.default_rng(9)
    Bn, K, D, n_gen, p = 3, 6, 64, 30, 0.7
    prompts = [list(rng.integers(0, VOCAB, size=s)) for s in (1, 4, 9)]
    cap = max(map(len, prompts)) + n_gen * K + 2 * K
    kc = torch.zeros((Bn, 1, cap, D), dtype=torch.float32, device=DEV)
    vc = torch.zeros_like(kc)
    for b, pr in enumerate(prompts):
        for t in range(len(pr)):
            kv = _kv(pr[:t + 1])
            kc[b, 0, t, :2] = torch.tensor(kv)
            vc[b, 0, t, :2] = torch.tensor(kv) + 7
    seqs = [list(pr) for pr in prompts]
    lens = torch.tensor([len(pr) for pr in prompts], dtype=torch.int32, device=DEV)
    anchor = [_next(s) for s in seqs]
    while min(len(s) - len(pr) for s, pr in zip(seqs, prompts)) < n_gen:
        dl = torch.zeros((Bn, K, VOCAB))
        al = torch.zeros((Bn, K, VOCAB))
        kb = torch.zeros((Bn, K, 1, D))
        vb = torch.zeros((Bn, K, 1, D))
        for b in range(Bn):
            ctx = seqs[b] + [anchor[b]]
            cont = []
            for _ in range(K):
                cont.append(_next(ctx + cont))
            d = [c if rng.random() < p else int(rng.integers(0, VOCAB)) for c in cont]
            block = [anchor[b]] + d[:K - 1]
            for i in range(K):
                dl[b, i, d[i]] = 5.0
                pre = seqs[b] + block[:i + 1]
                al[b, i, _next(pre)] = 5.0
                kb[b, i, 0, :2] = torch.tensor(_kv(pre))
                vb[b, i, 0, :2] = torch.tensor(_kv(pre)) + 7
        bufs = api.consensus(dev(dl), dev(al))
        c = api.make_cache(kc, vc, lens)
        lens = api.kv_append(c, dev(kb), dev(vb), bufs.n_emit)
        g = bufs.as_dict()
        off, em, na = g["emit_off"].cpu().tolist(), g["emitted"].cpu().tolist(), \
            g["next_anchor"].cpu().tolist()
        for b in range(Bn):
            e = em[off[b]:off[b + 1]]
            seqs[b] = seqs[b] + [anchor[b]] + e[:-1]
            anchor[b] = na[b]
    torch.cuda.synchronize()
    lens_h = lens.cpu().tolist()
    kh, vh = kc.cpu(), vc.cpu()
    for b in range(Bn):
        full = seqs[b] + [anchor[b]]
        ref = list(prompts[b])
        while len(ref) < len(full):
            ref.append(_next(ref))
        assert full == ref
        assert lens_h[b] == len(seqs[b])
        for t in range(lens_h[b]):
            assert kh[b, 0, t, :2].tolist() == _kv(ref[:t + 1])
            assert vh[b, 0, t, :2].tolist() == [x + 7 for x in _kv(ref[:t + 1])]
