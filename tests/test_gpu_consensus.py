"""GPU parity of orthrus_consensus / orthrus_argmax against the oracle:
tokens, divergence index, emitted counts, offsets, packed tokens and next
anchors must be bit-exact, on the workloads' logits and on adversarial rows
(ties, signed zeros, -inf, maxima at the last index and across chunk
boundaries, rows that are not 16-byte aligned, tiny vocabularies)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, dev, f64, say
from ar_shared_kv_amd import api

pytestmark = pytest.mark.gpu


def check_consensus(diff, ar, what):
    say(f"consensus {what}: B,K,V={tuple(ar.shape)} {ar.dtype}")
    bufs = api.consensus(dev(diff), dev(ar))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.as_dict().items()}
    d_ref = oracle.argmax_rows(f64(diff))
    a_ref = oracle.argmax_rows(f64(ar))
    np.testing.assert_array_equal(g["diff_tok"], d_ref, err_msg=what)
    np.testing.assert_array_equal(g["ar_tok"], a_ref, err_msg=what)
    r = oracle.consensus(d_ref, a_ref)
    for k in ("j", "n", "emit_off", "emitted", "next_anchor"):
        np.testing.assert_array_equal(g[k], r[k], err_msg=f"{what}: {k}")
    return r


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workload_logits(cid):
    cfg = W.CONFIGS[cid]
    diff, ar = W.consensus_logits(cfg.B, cfg.K, cfg.V, W.match_probabilities(cfg), cfg.torch_dtype,
                                  W.seed_of(cfg, W.T_LOGITS))
    r = check_consensus(diff, ar, f"config{cid}")
    say(f"  mean accepted n = {r['n'].mean():.2f}")


@pytest.mark.parametrize("K", W.LONG_CONTEXT_K_SWEEP)
def test_long_context_block_sweep(K):
    cfg = W.CONFIGS[5]
    diff, ar = W.consensus_logits(1, K, cfg.V, 0.8, torch.bfloat16, W.seed_of(cfg, W.T_LOGITS, K))
    check_consensus(diff, ar, f"config5 K={K}")


def adversarial(V, dtype, K=12):
    rows = []
    rows.append(torch.zeros(V))                                  # all equal -> 0
    x = torch.full((V,), -1.0); x[V // 3] = -0.0; x[V // 2] = 0.0
    rows.append(x)                                               # signed zeros tie
    rows.append(torch.full((V,), float("-inf")))                 # all -inf -> 0
    x = torch.randn(V); x[V - 1] = 100.0
    rows.append(x)                                               # max at V-1
    chunk = 16384 // (2 if dtype == torch.bfloat16 else 4)
    x = torch.randn(V); b0 = min(chunk, V - 1)
    x[b0] = 50.0; x[b0 - 1] = 50.0
    rows.append(x)                                               # tie across chunk boundary
    x = torch.randn(V); x[min(2 * chunk + 3, V - 1)] = 60.0; x[V - 1] = 60.0
    rows.append(x)                                               # tie, later chunk vs last
    x = torch.full((V,), float("-inf")); x[V - 1] = -5.0
    rows.append(x)
    while len(rows) < K:
        rows.append(torch.randn(V))
    a = torch.stack(rows[:K])[None].to(dtype)
    d = a.clone()
    d[0, 5, 7 % V] = 1000.0                                      # one mismatch at row 5
    return d, a


@pytest.mark.parametrize("V", [1, 7, 1000, 1001, 8193, 151936])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_adversarial_rows(V, dtype):
    d, a = adversarial(V, dtype)
    check_consensus(d, a, f"adversarial V={V}")


def test_argmax_entry_point_matches_oracle():
    x = torch.randn(37, 5003).to(torch.bfloat16)
    x[3, 17] = x[3, 4000] = 20.0
    idx = api.argmax(dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.argmax_rows(f64(x)))


def test_batched_ragged_acceptance():
    # 32 requests with per-request match probability in [0.5, 0.95]
    cfg = W.CONFIGS[4]
    ps = W.match_probabilities(cfg, salt=3)
    diff, ar = W.consensus_logits(cfg.B, cfg.K, 4096, ps, torch.bfloat16, 4242)
    r = check_consensus(diff, ar, "ragged batch")
    assert len(set(r["n"].tolist())) > 3


@pytest.mark.parametrize("B,K", [(1, 64), (16, 32), (65, 8), (300, 4), (1100, 2), (4000, 16)],
                         ids=["B1-K64", "B16", "B65", "B300", "B1100-two-level", "B4000"])
def test_batch_sizes_cover_every_scan_path(B, K):
    # small batches keep tokens in LDS; more than 64 requests use the
    # work-group scan, more than 1024 give each thread a run of requests
    V = 600
    ps = torch.linspace(0.3, 0.97, B).tolist()
    diff, ar = W.consensus_logits(B, K, V, ps, torch.bfloat16, 777 + B)
    r = check_consensus(diff, ar, f"B={B} K={K}")
    assert r["emit_off"][-1] == int(r["n"].sum())


def test_argmax_many_rows_and_chunks():
    # rows not a multiple of the 16 rows a work-group reduces; > 64 chunks per row
    x = torch.randn(41, 600000).to(torch.bfloat16)
    x[5, 599999] = 50.0
    x[40, 0] = 50.0
    idx = api.argmax(dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.argmax_rows(f64(x)))
