"""Benchmark of the Orthrus decode-step hot path on one MI355X.

One step (Qwen3-8B shape: 36 layers, 32 query / 8 KV heads, head_dim 128,
prefix L=8192, block K=32, vocabulary 151,936) is:
    36 x block attention, diffusion view (bidirectional block)
    36 x block attention, AR verification view (causal block)
    consensus over both views' logits [1, 32, 151936]
    append of the accepted rows' KV on all 36 layers
Every layer has its own synthetic cache (1.2 GB in total, resident in HBM).
The step is captured in a HIP graph; W warm-up replays, then K timed replays
between two synchronisations.  Prints ONE JSON line.

--config N runs another workload (1 tiny fp32, 2 Qwen3-1.7B layer, 4 paged
serving, 5 long context with --K in {4, 8, 16, 32, 64}).  A workload whose
inputs span less than 512 MiB cycles that many copies of them (one per
consecutive step, each replay runs all of them), so that no step is served
from the 256 MB last-level cache; "steps" then counts the steps timed.

The oracle (fp64 CPU) is timed on the host cores on a bounded sample of the
same step ("cpu_baseline"); it is a reported baseline, not the target.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify steps/s and achieved HBM TB/s, block attn+consensus, K=32, Qwen3-8B shape"
HBM_PEAK_GBPS = 8000.0
# sources that decide what the block-attention launch does (kernel and plan)
ATTN_SOURCES = ("ar_shared_kv_amd/csrc/block_attn.hip", "ar_shared_kv_amd/csrc/kernels.hpp",
                "ar_shared_kv_amd/csrc/common.hpp", "ar_shared_kv_amd/csrc/abi.cpp")
# ... and what the fused LM-head argmax call does
LM_SOURCES = ("ar_shared_kv_amd/csrc/lmhead.hip", "ar_shared_kv_amd/csrc/common.hpp")


def attn_source_hash(sources=ATTN_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, splits, name=None, sources=ATTN_SOURCES):
    """HBM bytes per block-attention launch (or per call of the profile `name`)
    from the committed counter summary of this workload, or None when the
    kernel sources changed since then."""
    path = os.path.join(ROOT, "profiles", name or f"block_attn_{workload}_traffic.txt")
    if splits or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_hash") != attn_source_hash(sources):
        return None
    return int(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload id (3 = the headline one)")
    ap.add_argument("--K", type=int, default=0, help="block size override (long-context sweep)")
    ap.add_argument("--splits", type=int, default=0, help="num_splits passed to block attention")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets cycled by consecutive steps (0 = enough for 512 MiB)")
    ap.add_argument("--lmhead", action="store_true",
                    help="time the fused LM-head argmax (greedy tokens from hidden states) at "
                         "the Qwen3-8B head shape instead of the decode step")
    ap.add_argument("--lmhead-rows", type=int, default=32,
                    help="hidden rows per --lmhead call (32 = one view of one request)")
    ap.add_argument("--calib-bytes", type=int, default=0,
                    help="first run one plain device copy of this many bytes (a known-size "
                         "kernel for scaling hardware byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """Device-resident inputs and outputs of one decode step of a workload."""

    def __init__(self, cfg, splits, sets=0, dev="cuda"):
        import torch
        import workloads as W
        from ar_shared_kv_amd import api
        self.cfg = cfg
        self.splits = splits
        nl = cfg.layers
        st = W.step_inputs(cfg, layers=1, with_logits=True)   # shapes + logits + lens
        # Input sets cycled by consecutive steps, so that a small workload's
        # inputs are not served from the 256 MB last-level cache: enough
        # copies of the step's inputs to span 512 MiB.
        e = 2 if cfg.dtype == "bf16" else 4
        lay0 = st.layers[0]
        per_set = nl * e * sum(getattr(lay0, k).numel() for k in
                               ("k_cache", "v_cache", "q_diff", "q_ar", "k_blk_diff",
                                "v_blk_diff", "k_blk_ar", "v_blk_ar"))
        per_set += e * (st.diff_logits.numel() + st.ar_logits.numel())
        if sets <= 0:
            sets = min(64, max(1, -(-(512 << 20) // per_set)))
        self.sets = sets
        self.set_bytes = per_set
        nt = nl * sets
        self.lens = st.lens.to(dev)
        self.lens_out = torch.empty_like(self.lens)
        self.page_table = st.page_table.to(dev) if cfg.paged else None
        cshape = tuple(st.layers[0].k_cache.shape)
        dt = cfg.torch_dtype
        self.kc = torch.empty((nt, *cshape), dtype=dt, device=dev)
        self.vc = torch.empty_like(self.kc)
        qs = (nt, cfg.B, cfg.K, cfg.Hq, cfg.D)
        bs = (nt, cfg.B, cfg.K, cfg.Hkv, cfg.D)
        self.q = {v: torch.empty(qs, dtype=dt, device=dev) for v in ("diff", "ar")}
        self.kb = {v: torch.empty(bs, dtype=dt, device=dev) for v in ("diff", "ar")}
        self.vb = {v: torch.empty(bs, dtype=dt, device=dev) for v in ("diff", "ar")}
        t0 = time.time()
        for l in range(nl):
            lay = st.layers[0] if l == 0 else W.layer_inputs(cfg, l, st.lens, st.num_pages,
                                                              st.capacity)
            self.kc[l].copy_(lay.k_cache)
            self.vc[l].copy_(lay.v_cache)
            for v in ("diff", "ar"):
                self.q[v][l].copy_(getattr(lay, f"q_{v}"))
                self.kb[v][l].copy_(getattr(lay, f"k_blk_{v}"))
                self.vb[v][l].copy_(getattr(lay, f"v_blk_{v}"))
        for x in [self.kc, self.vc] + [d[v] for d in (self.q, self.kb, self.vb)
                                       for v in ("diff", "ar")]:
            for si in range(1, sets):   # copies: other addresses, same values
                x[si * nl:(si + 1) * nl].copy_(x[:nl])
        log(f"inputs for {nl} layers x {sets} input sets generated in {time.time() - t0:.1f}s")
        self.step_inputs = st
        dl, al = st.diff_logits.to(dev), st.ar_logits.to(dev)
        self.diff_logits = [dl] + [dl.clone() for _ in range(1, sets)]
        self.ar_logits = [al] + [al.clone() for _ in range(1, sets)]
        lmax = int(st.lens.max())
        self.caches = [api.make_cache(self.kc[l], self.vc[l], self.lens,
                                      page_table=self.page_table, max_len=lmax)
                       for l in range(nt)]
        self.out = torch.empty(qs[1:], dtype=dt, device=dev)
        self.lse = torch.empty((cfg.B, cfg.Hq, cfg.K), dtype=torch.float32, device=dev)
        dcode = api.dtype_code(self.q["ar"])
        self.ws, self.ws_bytes = api.block_attn_workspace(self.caches[0], cfg.B, cfg.K, cfg.Hq,
                                                          cfg.Hkv, cfg.D, dcode, splits, dev)
        self.cbufs = api.ConsensusBuffers(cfg.B, cfg.K, cfg.V, dcode, dev)

    def attention(self, view, layer):
        from ar_shared_kv_amd import api
        from ar_shared_kv_amd import _binding as B_
        mask = B_.BIDIR if view == "diff" else B_.CAUSAL
        api.block_attn(self.q[view][layer], self.kb[view][layer], self.vb[view][layer],
                       self.caches[layer], mask=mask, scale=self.cfg.scale,
                       num_splits=self.splits, out=self.out, lse=self.lse, workspace=self.ws)

    def attention_set(self, si):
        nl = self.cfg.layers
        for view in ("diff", "ar"):          # all diffusion layers, then all AR layers
            for l in range(nl):
                self.attention(view, si * nl + l)

    def attention_passes(self):
        """Block attention of `sets` consecutive steps."""
        for si in range(self.sets):
            self.attention_set(si)

    def run(self):
        """`sets` consecutive decode steps, one per input set."""
        from ar_shared_kv_amd import api
        nl = self.cfg.layers
        for si in range(self.sets):
            self.attention_set(si)
            api.consensus(self.diff_logits[si], self.ar_logits[si], self.cbufs)
            api.kv_append(self.caches[si * nl], self.kb["ar"][si * nl], self.vb["ar"][si * nl],
                          self.cbufs.n_emit, self.lens_out, num_layers=nl,
                          cache_layer_stride=self.kc[0].numel(),
                          blk_layer_stride=self.kb["ar"][0].numel())

    # algorithmic bytes: every input read once, every output written once
    def attn_bytes_per_launch(self):
        c = self.cfg
        e = 2 if c.dtype == "bf16" else 4
        cache = int(self.step_inputs.lens.sum()) * c.Hkv * c.D * 2 * e
        blk = c.B * c.K * (2 * c.Hq + 2 * c.Hkv) * c.D * e
        return cache + blk + c.B * c.Hq * c.K * 4

    def attn_flops_per_launch(self):
        c = self.cfg
        return 4 * c.Hq * c.D * sum(c.K * (int(L) + c.K) for L in self.step_inputs.lens)

    def step_bytes(self, n_total):
        c = self.cfg
        e = 2 if c.dtype == "bf16" else 4
        logits = 2 * c.B * c.K * c.V * e
        append = 2 * 2 * c.Hkv * c.D * e * n_total * c.layers
        return 2 * c.layers * self.attn_bytes_per_launch() + logits + append


def timed(fn, steps, warmup, graph):
    import torch
    s = torch.cuda.current_stream()
    if graph:
        g = torch.cuda.CUDAGraph()
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        run = g.replay
    else:
        run = fn
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        run()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, (g if graph else None)


def cpu_baseline(step: Step, budget_s: float):
    """The oracle on the host cores: whole layers of the step until ~budget_s,
    extrapolated to the full step (consensus and append timed once)."""
    import numpy as np
    import oracle
    import workloads as W
    cfg = step.cfg
    st = step.step_inputs
    lens = st.lens.numpy()
    pt = st.page_table.numpy() if cfg.paged else None
    kw = dict(scale=cfg.scale)
    if cfg.paged:
        kw.update(layout=oracle.PAGED, page_table=pt)
    t_layers = 0.0
    done = 0
    while done < cfg.layers:
        lay = st.layers[0] if done == 0 else W.layer_inputs(cfg, done, st.lens, st.num_pages,
                                                            st.capacity)
        arrs = {k: getattr(lay, k).double().numpy() for k in
                ("q_diff", "q_ar", "k_cache", "v_cache", "k_blk_diff", "v_blk_diff",
                 "k_blk_ar", "v_blk_ar")}
        t0 = time.perf_counter()
        oracle.block_attn(arrs["q_diff"], arrs["k_cache"], arrs["v_cache"], arrs["k_blk_diff"],
                          arrs["v_blk_diff"], lens, mask=oracle.BIDIR, **kw)
        oracle.block_attn(arrs["q_ar"], arrs["k_cache"], arrs["v_cache"], arrs["k_blk_ar"],
                          arrs["v_blk_ar"], lens, mask=oracle.CAUSAL, **kw)
        t_layers += time.perf_counter() - t0
        done += 1
        if t_layers >= budget_s:
            break
    dl = st.diff_logits.double().numpy()
    al = st.ar_logits.double().numpy()
    t0 = time.perf_counter()
    r = oracle.consensus(oracle.argmax_rows(dl), oracle.argmax_rows(al))
    t_cons = time.perf_counter() - t0
    raw = lambda t: t.view(torch_int(t)).numpy()  # noqa: E731
    lay = st.layers[0]
    t0 = time.perf_counter()
    oracle.kv_append(raw(lay.k_cache)[None], raw(lay.v_cache)[None], raw(lay.k_blk_ar)[None],
                     raw(lay.v_blk_ar)[None], r["n"], lens,
                     layout=oracle.PAGED if cfg.paged else oracle.CONTIGUOUS, page_table=pt)
    t_app = time.perf_counter() - t0
    step_s = t_layers / done * cfg.layers + t_cons + t_app * cfg.layers
    sample = (f"oracle fp64 on {done} of {cfg.layers} layers (BIDIR+CAUSAL passes at full shape), "
              f"consensus and a 1-layer append; extrapolated to the {cfg.layers}-layer step")
    return {"value": round(1.0 / step_s, 6), "unit": "steps/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds_measured": round(t_layers + t_cons + t_app, 2)}


def torch_int(t):
    import torch
    return torch.int16 if t.element_size() == 2 else torch.int32


def calibrate(nbytes):
    """An elementwise kernel that reads and writes nbytes once each: the
    yardstick that scales the HBM byte counters."""
    if not nbytes:
        return
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def lmhead_main(args):
    """The fused LM-head argmax at the Qwen3-8B head shape: R = B*K = 32 hidden
    rows of H = 4,096 against V = 151,936 vocabulary rows, one view per call.
    Algorithmic bytes: the weight, the hidden rows and the tokens, once."""
    import torch
    import workloads as W
    from ar_shared_kv_amd import api
    from ar_shared_kv_amd import _binding as B_
    R, H, V = args.lmhead_rows, 4096, 151936
    calibrate(args.calib_bytes)
    h, w = W.lmhead_inputs(R, H, V, seed=0)
    hd, wd = h.cuda(), w.cuda()
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    n = B_.orthrus_lmhead_argmax_workspace_bytes(R, H, V, B_.BF16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    call = lambda: api.lmhead_argmax(hd, wd, idx=idx, workspace=ws)
    ms, _ = timed(call, args.steps, args.warmup, not args.no_graph)
    nbytes = V * H * 2 + R * H * 2 + R * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    flops = 2 * R * H * V
    res = {
        "metric": ("fused LM-head argmax calls/s (greedy tokens of one view's 32 block rows)"
                   if R == 32 else f"fused LM-head argmax calls/s (greedy tokens of {R} rows)"),
        "value": round(1e3 / ms, 3), "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3-8b-lmhead" if R == 32 else f"qwen3-8b-lmhead-R{R}",
                   "R": R, "H": H, "V": V,
                   "graph": not args.no_graph},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("qwen3-8b-lmhead", R != 32,
                                                 "lmhead_argmax_qwen3-8b_traffic.txt", LM_SOURCES),
                     "kernel": "lmhead_argmax_kernel + lmhead_finalize_kernel, per call",
                     "us_per_launch": round(ms * 1e3, 3), "bytes_per_launch": nbytes,
                     "mfma_frac": round(flops / (ms * 1e-3) / 2.5e15, 4)},
    }
    if not args.no_cpu:
        import oracle
        # the oracle's fp64 logits over a sample of vocabulary rows, scaled to V
        vs = V // 16
        t0 = time.perf_counter()
        oracle.lmhead_argmax(h, w[:vs])
        t = (time.perf_counter() - t0) * V / vs
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        res["cpu_baseline"] = {"value": round(1.0 / t, 4), "unit": "calls/s",
                               "cores": max(blas) if blas else 1, "kind": "oracle",
                               "sample": f"fp64 logits + argmax over {vs} of {V} vocabulary rows, "
                                         "scaled to the whole head"}
    if flops / 2.5e15 > nbytes / (HBM_PEAK_GBPS * 1e9):
        # many rows: the matrix cores, not one read of the weight, set the floor
        tf = flops / (ms * 1e-3) / 1e12
        res["roofline"].update(bound="mfma", achieved=round(tf, 1), peak=2500.0, unit="TFLOP/s",
                               frac=round(tf / 2500.0, 4), flops_per_launch=flops)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); sharding "
              "over several GPUs is a design, not implemented here", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "needs a GPU"
    if args.lmhead:
        lmhead_main(args)
        return
    cfg = W.CONFIGS[args.config]
    if args.K:
        cfg = cfg.with_(K=args.K)
    splits = args.splits or cfg.num_splits
    log(f"workload {cfg.name} K={cfg.K} splits={splits or 'auto'}")
    calibrate(args.calib_bytes)
    step = Step(cfg, splits, args.sets)
    graph = not args.no_graph

    ms_run, _ = timed(step.run, args.steps, args.warmup, graph)
    ms_step = ms_run / step.sets
    # the dominant kernel: block attention alone, all 2*layers passes per step
    ms_attn_all, _ = timed(step.attention_passes, args.steps, args.warmup, graph)
    us_attn = ms_attn_all * 1e3 / (2 * cfg.layers * step.sets)
    n = step.cbufs.n_emit.cpu()
    n_total = int(n.sum())

    attn_b = step.attn_bytes_per_launch()
    attn_f = step.attn_flops_per_launch()
    achieved_gbps = attn_b / (us_attn * 1e-6) / 1e9
    steps_s = 1e3 / ms_step
    res = {
        "metric": METRIC,
        "value": round(steps_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps * step.sets,
        "warmup": args.warmup * step.sets,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "K": cfg.K, "L": cfg.L if cfg.L_range is None else list(cfg.L_range),
                   "layers": cfg.layers, "V": cfg.V, "paged": cfg.paged,
                   "num_splits": splits or "auto", "graph": graph, "input_sets": step.sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if args.K else measured_traffic(cfg.name, args.splits),
                     "kernel": "block attention (attn_bf16_kernel + split merge), per launch",
                     "us_per_launch": round(us_attn, 3), "bytes_per_launch": attn_b,
                     "mfma_frac": round(attn_f / (us_attn * 1e-6) / 2.5e15, 4)},
        "step_hbm_tbps": round(step.step_bytes(n_total) / (ms_step * 1e-3) / 1e12, 3),
        "accepted_per_step": n.tolist() if cfg.B <= 4 else round(float(n.float().mean()), 3),
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
