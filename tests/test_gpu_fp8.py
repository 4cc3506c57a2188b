"""GPU parity of the FP8 (OCP E4M3) KV cache against the fp64 oracle, through
the C ABI: block attention over an E4M3 cache with per-row power-of-two
scales equals the oracle's attention over the dequantized values (within the
bf16 tolerance) at the Qwen3-8B layer shape, the 32-request paged batch and
the 131,072-token context, plus edge cases; the quantizing append is
bit-exact (codes and scales) against the oracle's quantizer."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from ar_shared_kv_amd import _binding as B_
from ar_shared_kv_amd import api
from gpu_util import assert_attn_close, dev, f64, record, say

pytestmark = pytest.mark.gpu


def fp8_layer(step, lay, seed):
    kc8, ks = W.fp8_cache(lay.k_cache, seed)
    vc8, vs = W.fp8_cache(lay.v_cache, seed + 1)
    return kc8, ks, vc8, vs


def run_fp8(step, lay, view, kc8, ks, vc8, vs, num_splits=0, max_len=0, what=""):
    cfg = step.cfg
    lens = dev(step.lens)
    pt = dev(step.page_table) if cfg.paged else None
    cache = api.make_cache(dev(kc8), dev(vc8), lens, page_table=pt, max_len=max_len,
                           k_scale=dev(ks), v_scale=dev(vs))
    q = dev(getattr(lay, f"q_{view}"))
    kb = dev(getattr(lay, f"k_blk_{view}"))
    vb = dev(getattr(lay, f"v_blk_{view}"))
    out = torch.full_like(q, float("nan"))
    out, lse = api.block_attn(q, kb, vb, cache, mask=B_.BIDIR if view == "diff" else B_.CAUSAL,
                              scale=cfg.scale, num_splits=num_splits, out=out)
    torch.cuda.synchronize()
    kd, vd = oracle.dequant_fp8(kc8.numpy(), ks.numpy()), oracle.dequant_fp8(vc8.numpy(),
                                                                             vs.numpy())
    kw = dict(mask=oracle.BIDIR if view == "diff" else oracle.CAUSAL, scale=cfg.scale)
    if cfg.paged:
        kw.update(layout=oracle.PAGED, page_table=step.page_table.numpy())
    ro, rl = oracle.block_attn(f64(getattr(lay, f"q_{view}")), kd, vd,
                               f64(getattr(lay, f"k_blk_{view}")),
                               f64(getattr(lay, f"v_blk_{view}")), step.lens.numpy(), **kw)
    return assert_attn_close(out, lse, ro, rl, torch.bfloat16, what)


@pytest.mark.parametrize("view", ["diff", "ar"])
def test_fp8_qwen3_8b_layer(view):
    step = W.step_inputs(W.CONFIGS[3], layers=1, with_logits=False)
    lay = step.layers[0]
    say(f"fp8 config3 {view}")
    run_fp8(step, lay, view, *fp8_layer(step, lay, 300), max_len=8192,
            what=f"fp8 config3 {view}")


@pytest.mark.parametrize("view", ["diff", "ar"])
def test_fp8_paged_serving_all_requests(view):
    step = W.step_inputs(W.CONFIGS[4], with_logits=False)
    lay = step.layers[0]
    say(f"fp8 config4 {view}")
    run_fp8(step, lay, view, *fp8_layer(step, lay, 400), max_len=8192,
            what=f"fp8 config4 all requests {view}")


@pytest.mark.parametrize("K", [32, 64])
def test_fp8_long_context(K):
    cfg = W.CONFIGS[5].with_(K=K)
    L = 131072
    kc = W.normal((1, 8, L + 64, 128), torch.bfloat16, W.seed_of(cfg, W.T_KC))
    vc = W.normal((1, 8, L + 64, 128), torch.bfloat16, W.seed_of(cfg, W.T_VC))
    lay = W.LayerInputs(
        q_diff=W.normal((1, K, 32, 128), torch.bfloat16, W.seed_of(cfg, W.T_Q_DIFF, K)),
        q_ar=W.normal((1, K, 32, 128), torch.bfloat16, W.seed_of(cfg, W.T_Q_AR, K)),
        k_cache=kc, v_cache=vc,
        k_blk_diff=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_KB_DIFF, K)),
        v_blk_diff=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_VB_DIFF, K)),
        k_blk_ar=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_KB_AR, K)),
        v_blk_ar=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_VB_AR, K)))
    step = W.StepInputs(cfg, torch.tensor([L], dtype=torch.int32), None, 0, L + 64, [lay],
                        None, None)
    say(f"fp8 config5 K={K}")
    run_fp8(step, lay, "ar", *fp8_layer(step, lay, 500 + K), num_splits=64, max_len=L,
            what=f"fp8 config5 K={K} ar all heads")


EDGE = [
    # (name, B, Hq, Hkv, K, lens, paged, splits)
    ("empty-prefix", 2, 4, 2, 4, [0, 0], False, 0),
    ("ragged-tails", 3, 16, 4, 7, [64, 1000, 129], False, 0),
    ("K1", 3, 8, 8, 1, [1, 5, 63], False, 0),
    ("M32", 2, 8, 8, 32, [700, 90], False, 0),
    ("M64", 2, 8, 4, 32, [333, 1200], False, 0),
    ("M256-K64", 1, 32, 8, 64, [700], False, 0),
    ("forced-splits", 2, 8, 2, 12, [3000, 2200], False, 16),
    ("paged-ragged", 4, 8, 2, 9, [0, 17, 300, 1100], True, 0),
    ("paged-B64-worklist", 64, 8, 2, 8, [100 * ((7 * i) % 9) for i in range(64)], True, 0),
    ("paged-M256", 3, 32, 8, 64, [16, 2049, 500], True, 0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_fp8_edge_cases(case):
    name, Bn, Hq, Hkv, K, lens, paged, splits = case
    step = W.custom_step(Bn, Hq, Hkv, 128, K, lens, paged=paged, seed=len(name) + 50)
    lay = step.layers[0]
    for view in ("diff", "ar"):
        say(f"fp8 edge {name} {view}")
        run_fp8(step, lay, view, *fp8_layer(step, lay, 600 + len(name)), num_splits=splits,
                what=f"fp8 {name} {view}")


def test_fp8_subnormal_codes_with_large_scales():
    """Every value of this cache is a subnormal E4M3 code (m * 2^-9, m < 8)
    times a large scale (2^4 .. 2^6): values up to ~0.9, so a decode that
    flushed subnormal codes would read an all-zero cache."""
    step = W.custom_step(2, 8, 2, 128, 16, [900, 333], seed=77)
    lay = step.layers[0]
    gen = torch.Generator().manual_seed(12)
    shape = tuple(lay.k_cache.shape)
    mk = lambda: (torch.randint(0, 8, shape, generator=gen, dtype=torch.uint8)  # noqa: E731
                  | (torch.randint(0, 2, shape, generator=gen, dtype=torch.uint8) << 7))
    kc8, vc8 = mk(), mk()
    ks = torch.exp2(torch.randint(4, 7, shape[:-1], generator=gen).float())
    vs = torch.exp2(torch.randint(4, 7, shape[:-1], generator=gen).float())
    for view in ("diff", "ar"):
        run_fp8(step, lay, view, kc8, ks, vc8, vs, what=f"fp8 subnormal codes {view}")


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_append_bit_exact(paged):
    layers, Bn, K, Hkv, D = 3, 5, 9, 8, 128
    lens = [0, 15, 16, 400, 77]
    step = W.custom_step(Bn, 32, Hkv, D, K, lens, paged=paged, seed=61)
    cshape = tuple(step.layers[0].k_cache.shape)
    gen = torch.Generator().manual_seed(3)
    kc = torch.randint(0, 0x7E, (layers, *cshape), generator=gen, dtype=torch.uint8)
    vc = torch.randint(0, 0x7E, (layers, *cshape), generator=gen, dtype=torch.uint8)
    ks = torch.full((layers, *cshape[:-1]), 0.25)
    vs = torch.full((layers, *cshape[:-1]), 0.5)
    kb = torch.randn((layers, Bn, K, Hkv, D), generator=gen).to(torch.bfloat16)
    # rows spanning the whole range: large, tiny, all zero, one nonzero value
    vb = (torch.randn((layers, Bn, K, Hkv, D), generator=gen) * 300).to(torch.bfloat16)
    kb[0, 0, 1, 3] = 0
    kb[1, 3, 0, 0] = (torch.randn(D, generator=gen) * 1e-30).to(torch.bfloat16)
    kb[2, 4, 2, 7] = 0
    kb[2, 4, 2, 7, 5] = -3.0
    n = torch.tensor([9, 1, 4, 0, 7], dtype=torch.int32)
    kc_d, vc_d, ks_d, vs_d = dev(kc), dev(vc), dev(ks), dev(vs)
    c = api.make_cache(kc_d[0], vc_d[0], dev(step.lens),
                       page_table=dev(step.page_table) if paged else None,
                       k_scale=ks_d[0], v_scale=vs_d[0])
    say(f"fp8 append paged={paged}")
    lo = api.kv_append(c, dev(kb)[0], dev(vb)[0], dev(n), num_layers=layers,
                       cache_layer_stride=kc[0].numel(), blk_layer_stride=kb[0].numel())
    torch.cuda.synchronize()
    rk, rv, rks, rvs, rl = oracle.kv_append_fp8(
        kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), kb.double().numpy(),
        vb.double().numpy(), n.numpy(), step.lens.numpy(),
        layout=oracle.PAGED if paged else oracle.CONTIGUOUS,
        page_table=step.page_table.numpy() if paged else None)
    np.testing.assert_array_equal(lo.cpu().numpy(), rl)
    bad = int((kc_d.cpu().numpy() != rk).sum() + (vc_d.cpu().numpy() != rv).sum())
    record("fp8-append", f"paged={paged}", code_mismatches=bad)
    np.testing.assert_array_equal(ks_d.cpu().numpy(), rks)
    np.testing.assert_array_equal(vs_d.cpu().numpy(), rvs)
    assert bad == 0
