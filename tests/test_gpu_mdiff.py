"""GPU parity of orthrus_mdiff_attn (the training-time block mask M_diff,
forward) against the fp64 oracle, through the C ABI: blocks tiling whole
sequences, random (overlapping, unsorted across sequences) anchors including
0 and the full context, several sequences, the Qwen3-8B attention shape, a
wrong max_anchor hint, forced split counts, D = 64, and fp32 inputs."""
import pytest
import torch

import oracle
import workloads as W
from ar_shared_kv_amd import api
from gpu_util import assert_attn_close, dev, f64, say

pytestmark = pytest.mark.gpu


def run_case(name, inp: W.MdiffInputs, dtype, max_anchor=0, num_splits=0):
    D = inp.q.shape[-1]
    scale = D ** -0.5
    say(f"mdiff {name}: q {tuple(inp.q.shape)} ctx {tuple(inp.k_ctx.shape)} "
        f"anchors {inp.anchors.flatten().tolist()[:6]}...")
    q = dev(inp.q)
    out = torch.full_like(q, float("nan"))
    out, lse = api.mdiff_attn(q, dev(inp.k_blk), dev(inp.v_blk), dev(inp.k_ctx), dev(inp.v_ctx),
                              dev(inp.anchors), scale=scale, max_anchor=max_anchor,
                              num_splits=num_splits, out=out)
    torch.cuda.synchronize()
    ro, rl = oracle.mdiff_attn(f64(inp.q), f64(inp.k_ctx), f64(inp.v_ctx),
                               inp.anchors.numpy(), f64(inp.k_blk), f64(inp.v_blk), scale=scale)
    return assert_attn_close(out, lse, ro, rl, dtype, f"mdiff {name}")


CASES = [
    # (name, B, N, K, Hq, Hkv, D, layout, NB, dtype, max_anchor, splits)
    ("tile-small", 2, 320, 8, 8, 2, 128, "tile", 0, "bf16", 0, 0),
    ("random-anchors", 3, 1000, 16, 8, 2, 128, "random", 9, "bf16", 0, 0),
    ("random-K32-G4", 2, 2000, 32, 16, 4, 128, "random", 5, "bf16", 0, 0),
    ("random-wrong-hint", 2, 1500, 16, 8, 2, 128, "random", 6, "bf16", 300, 0),
    ("random-forced-splits", 2, 1500, 16, 8, 2, 128, "random", 6, "bf16", 0, 4),
    ("tile-D64", 1, 640, 16, 8, 2, 64, "tile", 0, "bf16", 0, 0),
    ("K1", 2, 200, 1, 4, 4, 128, "random", 7, "bf16", 0, 0),
    ("fp32-random", 2, 300, 8, 4, 2, 64, "random", 5, "f32", 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mdiff_matches_oracle(case):
    name, Bn, N, K, Hq, Hkv, D, layout, NB, dt, hint, splits = case
    inp = W.mdiff_inputs(Bn, N, K, Hq, Hkv, D, layout=layout, NB=NB, dtype=dt, seed=len(name))
    if layout == "random":
        # the edges of the rule: a block with no context and one with all of it
        inp.anchors[0, 0] = 0
        inp.anchors[-1, -1] = N
    run_case(name, inp, torch.float32 if dt == "f32" else torch.bfloat16, hint, splits)


def test_mdiff_qwen3_8b_training_microbatch_sequence():
    # one sequence of the benchmark's micro-batch at full shape: 4,096 tokens,
    # 128 blocks of K = 32 tiling it, 32 query / 8 KV heads, head_dim 128
    wl = W.MDIFF_WORKLOAD
    inp = W.mdiff_inputs(1, wl["N"], wl["K"], wl["Hq"], wl["Hkv"], wl["D"], layout="tile")
    run_case("qwen3-8b 1x4096 tiled", inp, torch.bfloat16, max_anchor=wl["N"])


def test_mdiff_single_block_equals_decode_block_attention():
    # NB = 1 with the anchor at the end of the context: the same kernels
    # compute the diffusion view of a decode step, bit for bit
    inp = W.mdiff_inputs(2, 700, 16, 8, 2, 128, layout="random", NB=1, seed=3)
    inp.anchors[:, 0] = torch.tensor([700, 515], dtype=torch.int32)
    q = dev(inp.q)
    o1, l1 = api.mdiff_attn(q, dev(inp.k_blk), dev(inp.v_blk), dev(inp.k_ctx), dev(inp.v_ctx),
                            dev(inp.anchors))
    cache = api.make_cache(dev(inp.k_ctx), dev(inp.v_ctx), dev(inp.anchors[:, 0].contiguous()))
    from ar_shared_kv_amd import _binding as B_
    o2, l2 = api.block_attn(q[:, 0].contiguous(), dev(inp.k_blk[:, 0].contiguous()),
                            dev(inp.v_blk[:, 0].contiguous()), cache, mask=B_.BIDIR)
    torch.cuda.synchronize()
    # the same work-groups with the same split plan (2 requests x 8 heads):
    # only the dispatch order differs, which changes no arithmetic
    assert torch.equal(o1[:, 0].view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1[:, 0], l2)
