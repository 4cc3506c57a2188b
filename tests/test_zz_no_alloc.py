"""orthrus_block_attn_noalloc (the entry point that allocates nothing: the
split partials live in a fixed array of the library on each GPU) against
orthrus_block_attn with a caller workspace, through the C ABI: two calls in
a row, the second with a smaller input, must equal the workspace path bit
for bit (same kernels, same split plan); a call needing more than the array
is refused before anything is launched."""
import pytest
import torch

import workloads as W
from ar_shared_kv_amd import _binding as B_
from ar_shared_kv_amd import api
from gpu_util import cache_for, dev, say

pytestmark = pytest.mark.gpu


def run_both(step, view, num_splits=0, max_len=0):
    cfg = step.cfg
    lay = step.layers[0]
    q = dev(getattr(lay, f"q_{view}"))
    kb = dev(getattr(lay, f"k_blk_{view}"))
    vb = dev(getattr(lay, f"v_blk_{view}"))
    mask = B_.BIDIR if view == "diff" else B_.CAUSAL
    cache = cache_for(step, lay, max_len=max_len)
    ref, ref_lse = api.block_attn(q, kb, vb, cache, mask=mask, scale=cfg.scale,
                                  num_splits=num_splits)
    out = torch.full_like(q, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    dt = api.dtype_code(q)
    st = B_.orthrus_block_attn_noalloc(cache, q, kb, vb, out, lse, cfg.B, cfg.K, cfg.Hq, cfg.Hkv,
                                       cfg.D, dt, mask, cfg.scale, num_splits)
    B_.check("orthrus_block_attn_noalloc", st)
    torch.cuda.synchronize()
    need = B_.orthrus_block_attn_workspace_bytes(cache, cfg.B, cfg.K, cfg.Hq, cfg.Hkv, cfg.D, dt,
                                                 num_splits)
    return ref, ref_lse, out, lse, need


def test_noalloc_two_calls_second_smaller_equal_workspace_path():
    big = W.step_inputs(W.CONFIGS[3], layers=1, with_logits=False)          # 26 splits
    small = W.custom_step(2, 8, 2, 128, 12, [3000, 2200], seed=7)           # fewer, smaller
    for name, step, ns, ml in (("qwen3-8b layer", big, 0, 8192), ("small", small, 8, 0)):
        for view in ("diff", "ar"):
            ref, ref_lse, out, lse, need = run_both(step, view, ns, ml)
            say(f"noalloc {name} {view}: workspace {need} bytes")
            assert need > 0, "the case must use split partials"
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
            assert torch.equal(lse, ref_lse)


def test_noalloc_paged_and_refuses_beyond_its_array():
    step = W.custom_step(5, 8, 8, 128, 1, [1, 700, 64, 0, 2049], paged=True, seed=9)
    ref, ref_lse, out, lse, need = run_both(step, "ar")
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse, ref_lse)
    cap = B_.orthrus_block_attn_noalloc_max_workspace()
    assert cap == 64 << 20
    # 64 requests x 8 KV heads x 256 rows x 64 splits of partials: beyond the array
    lens = torch.full((64,), 131072, dtype=torch.int32, device="cuda")
    kc = torch.empty((64, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    c = api.make_cache(kc, kc, lens, max_len=0)
    c.capacity = 131072 + 64        # host-side plan only: nothing is launched
    q = torch.empty((64, 64, 32, 128), dtype=torch.bfloat16, device="cuda")
    kb = torch.empty((64, 64, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    need = B_.orthrus_block_attn_workspace_bytes(c, 64, 64, 32, 8, 128, B_.BF16, 64)
    assert need > cap
    st = B_.orthrus_block_attn_noalloc(c, q, kb, kb, out, None, 64, 64, 32, 8, 128, B_.BF16,
                                       B_.CAUSAL, 0.088, 64)
    assert st == B_.ERR_WORKSPACE
