"""The seeded input generators (CPU only): reproducible, and shaped as the
workloads describe them."""
import numpy as np
import torch

import oracle
import workloads as W


def test_same_seed_same_bits():
    a = W.normal((3, 5, 7), torch.bfloat16, 42)
    b = W.normal((3, 5, 7), torch.bfloat16, 42)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = W.normal((3, 5, 7), torch.bfloat16, 43)
    assert not torch.equal(a, c)


def test_logits_match_rate_and_plus_ten_construction():
    B, K, V, p = 4, 500, 1000, 0.8
    diff, ar = W.consensus_logits(B, K, V, p, torch.float32, seed=9)
    da = oracle.argmax_rows(diff.double().numpy())
    aa = oracle.argmax_rows(ar.double().numpy())
    same_row = (diff == ar).all(dim=-1).numpy()
    # where the rows are untouched the views agree; where a token got +10 they differ
    assert (da[same_row] == aa[same_row]).all()
    assert (da[~same_row] != aa[~same_row]).all()
    changed = (diff != ar).sum(dim=-1).numpy()
    assert set(np.unique(changed)) <= {0, 1}
    rate = same_row.mean()
    assert abs(rate - p) < 0.03


def test_per_request_probabilities_and_bf16_rounding():
    cfg = W.CONFIGS[4]
    ps = W.match_probabilities(cfg)
    assert len(ps) == cfg.B and all(0.5 <= x <= 0.95 for x in ps)
    diff, ar = W.consensus_logits(2, 8, 64, [1.0, 0.0], torch.bfloat16, seed=3)
    assert torch.equal(diff[0], ar[0])
    d = (diff[1].float() - ar[1].float())
    idx = d.nonzero()
    assert idx.shape[0] == 8
    for i, u in idx.tolist():
        assert diff[1, i, u] == (ar[1, i, u].float() + 10).to(torch.bfloat16)


def test_page_table_is_a_permutation_with_room_for_append():
    cfg = W.CONFIGS[4].with_(B=6, L_range=(5, 100))
    lens = W.prefix_lengths(cfg)
    table, P = W.page_table(cfg, lens)
    used = []
    for b in range(cfg.B):
        need = (int(lens[b]) + cfg.K + 15) // 16
        row = table[b].tolist()
        assert all(x >= 0 for x in row[:need]) and all(x == -1 for x in row[need:])
        used += row[:need]
    assert sorted(used) == list(range(P))


def test_config_shapes():
    c3 = W.CONFIGS[3]
    assert (c3.Hq, c3.Hkv, c3.D, c3.K, c3.L, c3.layers, c3.V) == (32, 8, 128, 32, 8192, 36, 151936)
    st = W.step_inputs(W.CONFIGS[1])
    l0 = st.layers[0]
    assert l0.q_diff.shape == (1, 8, 2, 64) and l0.k_cache.shape == (1, 1, 136, 64)
    assert st.diff_logits.shape == (1, 8, 1000) and st.diff_logits.dtype == torch.float32
