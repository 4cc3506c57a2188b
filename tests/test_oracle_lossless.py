"""Losslessness pin for consensus + append (CPU only).

The summary's §2.3 (and the abstract) state that consensus makes the output
match the frozen AR model's own greedy decoding exactly.  A toy deterministic
"AR model" (next token = hash of the prefix; each position's KV = a hash of
its whole prefix) and a noisy "diffusion model" (the AR continuation with
probability p, a random token otherwise) drive the Orthrus loop through the
oracle's consensus and append.  The emitted stream and the cache it builds
must equal plain sequential greedy decoding for every K and p.  This pins the
row alignment of the two views, the n = min(j+1, K) rule and which block rows
are appended.
"""
import numpy as np
import pytest

import oracle

VOCAB = 5


def h(seq):
    x = 1469598103
    for t in seq:
        x = ((x ^ (int(t) + 1)) * 1099511) % 2147483647
    return x


def ar_next(seq):
    return h(seq) % VOCAB


def kv_of(seq_upto_pos):
    """KV row of the last token of seq_upto_pos given its whole prefix."""
    pos = len(seq_upto_pos) - 1
    return [h(seq_upto_pos) & 0x7FFFFFFF, pos * 1000 + int(seq_upto_pos[-1])]


def sequential(prompt, n_new):
    seq = list(prompt)
    for _ in range(n_new):
        seq.append(ar_next(seq))
    return seq


@pytest.mark.parametrize("K", [1, 2, 4, 8])
@pytest.mark.parametrize("p", [0.0, 0.6, 1.0])
@pytest.mark.parametrize("paged", [False, True])
def test_orthrus_loop_equals_sequential_greedy(K, p, paged):
    rng = np.random.default_rng(K * 100 + int(p * 10))
    B, n_gen, ps = 3, 40, 16
    prompts = [list(rng.integers(0, VOCAB, size=int(s))) for s in (1, 6, 13)]
    cap = max(len(x) for x in prompts) + n_gen * K + 2 * K   # fastest request bound
    # prefill: cache rows for the prompt, anchor = first generated token
    seqs = [list(pr) for pr in prompts]
    lens = np.array([len(pr) for pr in prompts], np.int32)
    if paged:
        maxp = (cap + ps - 1) // ps
        table = rng.permutation(B * maxp).reshape(B, maxp).astype(np.int32)
        kc = np.zeros((1, B * maxp, 1, ps, 2), np.int64)
    else:
        table = None
        kc = np.zeros((1, B, 1, cap, 2), np.int64)
    vc = kc.copy()

    def put(kc, b, t, row):
        if paged:
            kc[0, table[b, t // ps], 0, t % ps] = row
        else:
            kc[0, b, 0, t] = row

    def get(kc, b, t):
        return kc[0, table[b, t // ps], 0, t % ps] if paged else kc[0, b, 0, t]

    for b, pr in enumerate(prompts):
        for t in range(len(pr)):
            put(kc, b, t, kv_of(pr[:t + 1]))
            put(vc, b, t, [x + 7 for x in kv_of(pr[:t + 1])])
    anchor = [ar_next(s) for s in seqs]
    while min(len(s) - len(pr) for s, pr in zip(seqs, prompts)) < n_gen:
        d = np.zeros((B, K), np.int32)
        a = np.zeros((B, K), np.int32)
        kb = np.zeros((1, B, K, 1, 2), np.int64)
        vb = np.zeros((1, B, K, 1, 2), np.int64)
        for b in range(B):
            ctx = seqs[b] + [anchor[b]]
            cont = sequential(ctx, K)[len(ctx):]            # the AR's own continuation
            for i in range(K):
                d[b, i] = cont[i] if rng.random() < p else rng.integers(0, VOCAB)
            block = [anchor[b]] + list(d[b, :K - 1])       # AR verify inputs
            for i in range(K):
                pre = seqs[b] + block[:i + 1]
                a[b, i] = ar_next(pre)
                kb[0, b, i, 0] = kv_of(pre)
                vb[0, b, i, 0] = [x + 7 for x in kv_of(pre)]
        r = oracle.consensus(d, a)
        kc, vc, lens_out = oracle.kv_append(kc, vc, kb, vb, r["n"], lens,
                                            layout=oracle.PAGED if paged else oracle.CONTIGUOUS,
                                            page_table=table)
        for b in range(B):
            em = r["emitted"][r["emit_off"][b]:r["emit_off"][b + 1]]
            seqs[b] = seqs[b] + [anchor[b]] + list(em[:-1])
            anchor[b] = int(r["next_anchor"][b])
        lens = lens_out
    for b in range(B):
        full = seqs[b] + [anchor[b]]
        ref = sequential(prompts[b], len(full) - len(prompts[b]))
        assert full == ref
        assert lens[b] == len(seqs[b])
        for t in range(lens[b]):
            assert list(get(kc, b, t)) == kv_of(ref[:t + 1])
            assert list(get(vc, b, t)) == [x + 7 for x in kv_of(ref[:t + 1])]
