"""One decode step captured in a HIP graph and replayed: every replay must
reproduce the eager results bit for bit.

The step is the one the benchmark times (block attention of both views with
the split-KV merge, consensus, KV append), at small sizes.  Between replays
the outputs are overwritten by eager work and the stream is synchronized, so
that a replay which skipped a launch, or one whose recorded memory operation
went stale, shows up as a mismatch.
"""
from __future__ import annotations

import pytest
import torch

import workloads as W
from ar_shared_kv_amd import api
from ar_shared_kv_amd import _binding as B_
from gpu_util import cache_for, dev, say

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, Hq, Hkv, D, K, lens, paged)
    ("contiguous-splits", 2, 16, 8, 128, 16, [700, 1500], False),
    ("paged-worklist", 3, 8, 2, 128, 32, [900, 64, 2500], True),
]


class Step:
    def __init__(self, st: W.StepInputs):
        cfg = st.cfg
        lay = st.layers[0]
        self.cfg = cfg
        self.cache = cache_for(st, lay)
        self.q = {"diff": dev(lay.q_diff), "ar": dev(lay.q_ar)}
        self.kb = {"diff": dev(lay.k_blk_diff), "ar": dev(lay.k_blk_ar)}
        self.vb = {"diff": dev(lay.v_blk_diff), "ar": dev(lay.v_blk_ar)}
        self.logits = (dev(st.diff_logits), dev(st.ar_logits))
        self.out = {v: torch.empty_like(self.q[v]) for v in ("diff", "ar")}
        self.lse = {v: torch.empty((cfg.B, cfg.Hq, cfg.K), dtype=torch.float32, device="cuda")
                    for v in ("diff", "ar")}
        dcode = api.dtype_code(self.q["ar"])
        self.ws, self.ws_bytes = api.block_attn_workspace(self.cache, cfg.B, cfg.K, cfg.Hq, cfg.Hkv,
                                                          cfg.D, dcode, 0, "cuda")
        self.cbufs = api.ConsensusBuffers(cfg.B, cfg.K, cfg.V, dcode, "cuda")
        self.lens_out = torch.empty(cfg.B, dtype=torch.int32, device="cuda")

    def run(self):
        for view, mask in (("diff", B_.BIDIR), ("ar", B_.CAUSAL)):
            api.block_attn(self.q[view], self.kb[view], self.vb[view], self.cache, mask=mask,
                           scale=self.cfg.scale, out=self.out[view], lse=self.lse[view],
                           workspace=self.ws)
        api.consensus(self.logits[0], self.logits[1], self.cbufs)
        api.kv_append(self.cache, self.kb["ar"], self.vb["ar"], self.cbufs.n_emit, self.lens_out)

    def results(self):
        c = self.cbufs
        r = {f"out_{v}": self.out[v].view(torch.int16) for v in ("diff", "ar")}
        r.update({f"lse_{v}": self.lse[v].view(torch.int32) for v in ("diff", "ar")})
        r.update(diff_tok=c.diff_tok, ar_tok=c.ar_tok, n_match=c.n_match, n_emit=c.n_emit,
                 emit_off=c.emit_off, next_anchor=c.next_anchor, lens_out=self.lens_out,
                 emitted=c.emitted[: int(c.emit_off[-1])])
        return {k: v.clone() for k, v in r.items()}

    def scramble(self):
        """Eager work between replays: overwrite every output."""
        for v in ("diff", "ar"):
            self.out[v].fill_(float("nan"))
            self.lse[v].fill_(float("nan"))
        for t in (self.cbufs.diff_tok, self.cbufs.ar_tok, self.cbufs.n_match, self.cbufs.n_emit,
                  self.cbufs.emit_off, self.cbufs.next_anchor, self.lens_out):
            t.fill_(-7)
        self.cbufs.emitted.fill_(-7)
        if self.ws is not None:
            self.ws.fill_(0xA5)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(case):
    name, Bn, Hq, Hkv, D, K, lens, paged = case
    st = W.custom_step(Bn, Hq, Hkv, D, K, lens, paged=paged, seed=31, V=5003)
    step = Step(st)
    say(f"graph {name}: eager")
    step.run()
    torch.cuda.synchronize()
    ref = step.results()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    for rep in range(3):
        step.scramble()
        torch.cuda.synchronize()
        say(f"graph {name}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = step.results()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"{name}: replay {rep} differs from eager in {k}"
