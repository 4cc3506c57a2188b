"""Greedy prediction from hidden states on the GPU (orthrus_lmhead_argmax)
against the fp64 oracle.  The kernel decides the argmax on fp32
accumulations, so where the oracle's best two logits are closer than the
fp32 accumulation bound either index is a valid answer: rows are compared
exactly when the gap exceeds the bound, and otherwise the GPU's choice must
lie within the bound of the maximum."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from ar_shared_kv_amd import api
from gpu_util import record, say

pytestmark = pytest.mark.gpu

CASES = [
    # (name, R, H, V)
    ("qwen3-8b-head-benched-shape", 32, 4096, 151936),
    ("qwen3-vocab", 32, 1024, 151936),
    ("two-views-64-rows", 64, 4096, 20000),
    ("deep-H-ragged-V", 7, 4096, 1000),
    ("seventy-rows-one-128-row-block", 70, 256, 130),
    ("fifty-rows-64-row-block", 50, 512, 3000),
    ("hundred-rows-one-128-row-block", 100, 512, 2000),
    ("129-rows-one-256-row-block", 129, 256, 700),
    ("serving-rows-two-256-row-blocks", 300, 512, 5000),
    ("one-row-one-block", 1, 128, 1),
    ("one-chunk-H64", 5, 64, 300),
]


def check(name, h, w, got):
    logits = oracle.lmhead_logits(h, w)
    ref = oracle.argmax_rows(logits)
    H = h.shape[1]
    # fp32 accumulation bound per row: H * 2^-24 * sum_k |x_k w_vk|, over v
    mag = np.abs(h.double().numpy()) @ np.abs(w.double().numpy()).T
    bound = 2.0 * H * 2.0 ** -24 * mag.max(axis=1)
    exact = 0
    for r in range(len(ref)):
        top = np.sort(logits[r])[-2:] if logits.shape[1] > 1 else np.array([-np.inf, logits[r, 0]])
        if top[1] - top[0] > 2 * bound[r]:
            assert got[r] == ref[r], f"{name} row {r}: {got[r]} vs {ref[r]} (clear gap)"
            exact += 1
        else:
            assert logits[r, got[r]] >= logits[r, ref[r]] - 2 * bound[r], f"{name} row {r}"
    say(f"  {name}: {exact}/{len(ref)} rows with a clear gap, all equal")
    record("lmhead", name, rows=len(ref), clear_gap_rows=exact, mismatches=0)
    return exact


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lmhead_argmax_matches_oracle(case):
    name, R, H, V = case
    h, w = W.lmhead_inputs(R, H, V, seed=R)
    say(f"lmhead {name} R={R} H={H} V={V}")
    got = api.lmhead_argmax(h.cuda(), api.pack_weight(w.cuda())).cpu().numpy()
    exact = check(name, h, w, got)
    assert exact >= R // 2


@pytest.mark.parametrize("R,H,rows", [
    (4, 512, (2900, 333)),          # 32-row work-groups; vocabulary blocks 22 and 2
    (4, 512, (380, 333)),           # same block, different waves
    (50, 512, (2177, 1)),           # 64-row work-groups (blocks 17 and 0)
    (100, 512, (1999, 5)),          # 128-row work-groups (blocks 15 and 0)
    (300, 512, (4001, 7)),          # 256-row work-groups
    (32, 4096, (151935, 77777)),    # the Qwen3-8B head: the last row and one far away
])
def test_lmhead_argmax_duplicate_rows_take_the_lowest_index(R, H, rows):
    V = max(rows) + 1 if max(rows) + 1 > 3000 else 3000
    h, w = W.lmhead_inputs(R, H, V, seed=11)
    # two weight rows (in different vocabulary blocks but one) are the same
    # vector, aligned with hidden row 0: for row 0 they must carry
    # bitwise-equal fp32 logits, the largest of the row, and the lower index
    # wins
    best = (h[0].float() / h[0].float().norm()).to(torch.bfloat16)
    hi, lo = rows
    w[hi] = best
    w[lo] = best
    say(f"lmhead duplicates R={R} H={H} rows={rows}")
    got = api.lmhead_argmax(h.cuda(), api.pack_weight(w.cuda())).cpu().numpy()
    record("lmhead-ties", f"R={R} H={H} rows {hi}/{lo}", token=int(got[0]), expected=int(lo))
    assert got[0] == lo
    check("duplicates", h, w, got)


def test_lmhead_argmax_graph_replay_equals_eager():
    R, H, V = 32, 1024, 20000
    h, w = W.lmhead_inputs(R, H, V, seed=5)
    hd, wd = h.cuda(), api.pack_weight(w.cuda())
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    from ar_shared_kv_amd import _binding as B_
    n = B_.orthrus_lmhead_argmax_workspace_bytes(R, H, V, B_.BF16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    api.lmhead_argmax(hd, wd, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    ref = idx.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.lmhead_argmax(hd, wd, idx=idx, workspace=ws)
    for _ in range(3):
        idx.fill_(-1)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref)
