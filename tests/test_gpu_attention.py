"""GPU parity of orthrus_block_attn against the fp64 oracle (through the C ABI).

Covers the five workloads at full size, every request and every head, in the
launch configuration the benchmark uses, edge cases (empty prefix, ragged tails, K=1 and K=64, D=64,
G=1 and G=16, ragged contiguous batches, a wrong max_len hint), and GPU
metamorphic properties (split-count invariance, paged == contiguous,
run-to-run determinism, causal last row == bidirectional last row).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (DEV, assert_attn_close, cache_for, dev, f64, gpu_attn, oracle_attn, say)
from ar_shared_kv_amd import api
from ar_shared_kv_amd import _binding as B_

pytestmark = pytest.mark.gpu

VIEWS = ["diff", "ar"]


@pytest.mark.parametrize("view", VIEWS)
def test_config1_tiny_fp32(view):
    step = W.step_inputs(W.CONFIGS[1])
    say(f"config1 fp32 view={view}")
    out, lse = gpu_attn(step, step.layers[0], view)
    ro, rl = oracle_attn(step, step.layers[0], view)
    assert_attn_close(out, lse, ro, rl, torch.float32, "config1")


@pytest.mark.parametrize("view", VIEWS)
def test_config2_qwen3_1p7b_layer(view):
    step = W.step_inputs(W.CONFIGS[2])
    say(f"config2 view={view}")
    out, lse = gpu_attn(step, step.layers[0], view, max_len=2048)
    ro, rl = oracle_attn(step, step.layers[0], view)
    assert_attn_close(out, lse, ro, rl, torch.bfloat16, "config2")


@pytest.mark.parametrize("view", VIEWS)
def test_config3_qwen3_8b_layer_full_shape(view):
    # one of the 36 layers at full shape, automatic split plan as in the benchmark
    step = W.step_inputs(W.CONFIGS[3], layers=1, with_logits=False)
    say(f"config3 layer view={view}")
    out, lse = gpu_attn(step, step.layers[0], view, max_len=8192)
    ro, rl = oracle_attn(step, step.layers[0], view)
    assert_attn_close(out, lse, ro, rl, torch.bfloat16, "config3")


@pytest.fixture(scope="module")
def config4_step():
    return W.step_inputs(W.CONFIGS[4], with_logits=False)


@pytest.mark.parametrize("view", VIEWS)
def test_config4_paged_all_requests(view, config4_step):
    step = config4_step
    say(f"config4 paged view={view} lens={step.lens.tolist()[:8]}...")
    out, lse = gpu_attn(step, step.layers[0], view, max_len=8192)
    ro, rl = oracle_attn(step, step.layers[0], view)
    assert_attn_close(out, lse, ro, rl, torch.bfloat16, f"config4 all 32 requests {view}")


@pytest.fixture(scope="module")
def long_cache():
    L, Hkv, D = 131072, 8, 128
    cfg = W.CONFIGS[5]
    kc = W.normal((1, Hkv, L + 64, D), torch.bfloat16, W.seed_of(cfg, W.T_KC))
    vc = W.normal((1, Hkv, L + 64, D), torch.bfloat16, W.seed_of(cfg, W.T_VC))
    return kc, vc


@pytest.mark.parametrize("K", W.LONG_CONTEXT_K_SWEEP)
@pytest.mark.parametrize("view", VIEWS)
def test_config5_long_context_64_splits(K, view, long_cache):
    cfg = W.CONFIGS[5].with_(K=K)
    kc, vc = long_cache
    lens = torch.tensor([131072], dtype=torch.int32)
    lay = W.LayerInputs(
        q_diff=W.normal((1, K, 32, 128), torch.bfloat16, W.seed_of(cfg, W.T_Q_DIFF, K)),
        q_ar=W.normal((1, K, 32, 128), torch.bfloat16, W.seed_of(cfg, W.T_Q_AR, K)),
        k_cache=kc, v_cache=vc,
        k_blk_diff=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_KB_DIFF, K)),
        v_blk_diff=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_VB_DIFF, K)),
        k_blk_ar=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_KB_AR, K)),
        v_blk_ar=W.normal((1, K, 8, 128), torch.bfloat16, W.seed_of(cfg, W.T_VB_AR, K)))
    step = W.StepInputs(cfg, lens, None, 0, L_cap := kc.shape[2], [lay], None, None)
    say(f"config5 K={K} view={view}")
    out, lse = gpu_attn(step, lay, view, num_splits=64, max_len=131072)
    # every KV head (all 32 query heads), against the whole 131,072-key cache
    ro, rl = oracle_attn(step, lay, view)
    assert_attn_close(out, lse, ro, rl, torch.bfloat16, f"config5 K={K} {view} all heads")
    assert L_cap == 131136


EDGE = [
    # (name, B, Hq, Hkv, D, K, lens, dtype, paged)
    ("empty-prefix", 2, 4, 2, 128, 4, [0, 0], "bf16", False),
    ("tiny-prefix-K1", 3, 8, 8, 128, 1, [1, 5, 63], "bf16", False),
    ("ragged-tails", 3, 16, 4, 128, 7, [64, 1000, 129], "bf16", False),
    ("K64-M256", 1, 32, 8, 128, 64, [700], "bf16", False),
    ("K64-G16-M1024", 1, 16, 1, 64, 64, [300], "bf16", False),
    ("D64", 2, 8, 2, 64, 16, [333, 90], "bf16", False),
    ("G1", 1, 4, 4, 128, 32, [500], "bf16", False),
    ("M96-rowblock-tail", 1, 24, 8, 128, 32, [900], "bf16", False),
    ("M48", 2, 12, 4, 128, 16, [1500, 40], "bf16", False),
    # 320 work-groups of 8 rows: more than the CUs, so two share a CU (2-slot ring)
    ("M8-two-per-CU", 40, 8, 8, 128, 8, [(97 * i) % 700 for i in range(40)], "bf16", False),
    # 288 work-groups of 128 rows (3 splits each): two share a CU, four waves
    # each taking whole 64-key tiles
    ("M128-two-per-CU", 12, 32, 8, 128, 32, [(211 * i) % 1500 for i in range(12)], "bf16", False),
    ("paged-ragged", 4, 8, 2, 128, 9, [0, 17, 300, 1100], "bf16", True),
    # the longest-first work list decodes one request per lane: 64 requests is
    # its limit (equal tails test the rank's tie-break); 65 takes the plain grid
    ("paged-B64-worklist", 64, 8, 2, 128, 8, [100 * ((7 * i) % 9) for i in range(64)], "bf16", True),
    ("paged-B65-plain", 65, 8, 2, 128, 8, [100 * ((7 * i) % 9) for i in range(65)], "bf16", True),
    ("paged-D64", 2, 4, 1, 64, 32, [16, 47], "bf16", True),
    # D = 64 through the work list with several splits per request, and K = 1
    # (one query row per head) on pages
    ("paged-D64-worklist", 24, 8, 2, 64, 16, [(409 * i) % 3000 for i in range(24)], "bf16", True),
    ("paged-K1", 5, 8, 8, 128, 1, [1, 700, 64, 0, 2049], "bf16", True),
    ("fp32-ragged", 2, 4, 2, 128, 5, [70, 3], "f32", False),
    ("fp32-paged", 2, 2, 1, 64, 8, [130, 0], "f32", True),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
@pytest.mark.parametrize("view", VIEWS)
def test_edge_cases(case, view):
    name, Bn, Hq, Hkv, D, K, lens, dt, paged = case
    step = W.custom_step(Bn, Hq, Hkv, D, K, lens, dtype=dt, paged=paged, seed=len(name))
    say(f"edge {name} view={view}")
    out, lse = gpu_attn(step, step.layers[0], view)
    ro, rl = oracle_attn(step, step.layers[0], view)
    assert_attn_close(out, lse, ro, rl, step.cfg.torch_dtype, name)


def test_forced_splits_and_wrong_hint():
    # many splits, and a max_len hint below the true length (last split takes the rest)
    step = W.custom_step(2, 8, 2, 128, 12, [3000, 2200], seed=7)
    for ns, ml in [(1, 0), (3, 0), (16, 0), (0, 0), (8, 1000)]:
        say(f"splits={ns} max_len={ml}")
        for view in VIEWS:
            out, lse = gpu_attn(step, step.layers[0], view, num_splits=ns, max_len=ml)
            ro, rl = oracle_attn(step, step.layers[0], view)
            assert_attn_close(out, lse, ro, rl, torch.bfloat16, f"splits={ns} hint={ml} {view}")


def test_split_count_invariance_and_determinism():
    """Results for 1, 2, 8 and 32 splits agree with each other and with the
    oracle, and each is bit-identical from run to run.

    Two split plans differ by the rounding of the split partials (bf16, half
    an ulp: |O_s| * 2^-9, with |O_s| <= max |V| since a partial is a convex
    combination of V rows) and by the final output rounding (half an ulp of
    |O| each), so |O_a - O_b| <= 2^-9 max|V| + 2^-8 max|O| (+ fp32 terms)."""
    step = W.custom_step(1, 32, 8, 128, 32, [4096], seed=11)
    lay = step.layers[0]
    ro, rl = oracle_attn(step, lay, "ar")
    vmax = max(float(lay.v_cache.float().abs().max()), float(lay.v_blk_ar.float().abs().max()))
    bound = 2.0 ** -9 * vmax + 2.0 ** -8 * float(np.abs(ro).max()) + 1e-5
    outs = []
    for ns in (1, 2, 8, 32):
        o, l = gpu_attn(step, lay, "ar", num_splits=ns)
        o2, l2 = gpu_attn(step, lay, "ar", num_splits=ns)
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "not deterministic"
        assert torch.equal(l, l2)
        assert_attn_close(o, l, ro, rl, torch.bfloat16, f"split invariance splits={ns}")
        outs.append(f64(o))
    for ns, o in zip((2, 8, 32), outs[1:]):
        d = float(np.abs(o - outs[0]).max())
        say(f"  splits={ns} vs 1: max diff {d:.3e} (bound {bound:.3e})")
        assert d <= bound


def test_bf16_partials_error_budget():
    """The split partials are stored in bf16: their rounding adds at most
    2^-9 max|V| to the error.  Measured at the Qwen3-8B layer shape (8,192
    keys, 26 splits) against the single-split launch of the same inputs."""
    step = W.step_inputs(W.CONFIGS[3], layers=1, with_logits=False)
    lay = step.layers[0]
    for view in VIEWS:
        ro, rl = oracle_attn(step, lay, view)
        o1, l1 = gpu_attn(step, lay, view, num_splits=1, max_len=8192)
        oa, la = gpu_attn(step, lay, view, max_len=8192)
        e1 = assert_attn_close(o1, l1, ro, rl, torch.bfloat16, f"config3 {view} one split")
        ea = assert_attn_close(oa, la, ro, rl, torch.bfloat16, f"config3 {view} auto splits")
        vmax = max(float(lay.v_cache.float().abs().max()),
                   float(getattr(lay, f"v_blk_{view}").float().abs().max()))
        say(f"  config3 {view}: bf16 partials add {ea - e1:+.3e} to max|err| "
            f"(budget {2.0 ** -9 * vmax:.3e})")
        assert ea - e1 <= 2.0 ** -9 * vmax


def test_paged_equals_contiguous_bitwise():
    # same logical cache, identity-free shuffled pages: identical tiles -> identical bits
    Bn, Hq, Hkv, D, K = 3, 8, 2, 128, 10
    lens = [900, 64, 333]
    cont = W.custom_step(Bn, Hq, Hkv, D, K, lens, seed=21)
    lay = cont.layers[0]
    ps = 16
    maxp = (max(lens) + K + ps - 1) // ps
    gen = torch.Generator().manual_seed(5)
    P = Bn * maxp
    table = torch.randperm(P, generator=gen).to(torch.int32).view(Bn, maxp)
    kp = torch.zeros((P, Hkv, ps, D), dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    for b in range(Bn):
        for t in range(maxp * ps):
            if t < lay.k_cache.shape[2]:
                kp[table[b, t // ps], :, t % ps] = lay.k_cache[b, :, t]
                vp[table[b, t // ps], :, t % ps] = lay.v_cache[b, :, t]
    lensd = dev(cont.lens)
    for view in VIEWS:
        for ns in (1, 2):
            c_cont = api.make_cache(dev(lay.k_cache), dev(lay.v_cache), lensd, max_len=900)
            c_page = api.make_cache(dev(kp), dev(vp), lensd, page_table=dev(table), max_len=900)
            o1, l1 = gpu_attn(cont, lay, view, num_splits=ns, cache=c_cont)
            o2, l2 = gpu_attn(cont, lay, view, num_splits=ns, cache=c_page)
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
            assert torch.equal(l1, l2)


def test_causal_last_row_equals_bidir_last_row():
    step = W.custom_step(2, 8, 2, 128, 16, [500, 77], seed=3)
    lay = step.layers[0]
    lay.q_ar, lay.k_blk_ar, lay.v_blk_ar = lay.q_diff, lay.k_blk_diff, lay.v_blk_diff
    ob, lb = gpu_attn(step, lay, "diff")
    oc, lc = gpu_attn(step, lay, "ar")
    assert torch.equal(ob[:, -1].view(torch.int16), oc[:, -1].view(torch.int16))
    assert torch.equal(lb[:, :, -1], lc[:, :, -1])
    assert not torch.equal(ob[:, 0], oc[:, 0])


def test_no_lse_output_and_nan_poisoned_outputs_overwritten():
    step = W.custom_step(1, 8, 2, 128, 8, [200], seed=4)
    lay = step.layers[0]
    q = dev(lay.q_ar)
    out = torch.full_like(q, float("nan"))
    c = cache_for(step, lay)
    api.block_attn(q, dev(lay.k_blk_ar), dev(lay.v_blk_ar), c, mask=B_.CAUSAL, out=out,
                   want_lse=False)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ro, _ = oracle_attn(step, lay, "ar")
    assert np.abs(f64(out) - ro).max() <= 1e-2
