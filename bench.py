"""Benchmark of the Orthrus decode-step hot path on one MI355X.

One step (Qwen3-8B shape: 36 layers, 32 query / 8 KV heads, head_dim 128,
prefix L=8192, block K=32, vocabulary 151,936) is:
    36 x block attention, diffusion view (bidirectional block)
    36 x block attention, AR verification view (causal block)
    consensus over both views' logits [1, 32, 151936]
    append of the accepted rows' KV on all 36 layers
Every layer has its own synthetic cache (1.2 GB in total, resident in HBM).
Consecutive steps cycle 16 seeded draws of the consensus logits (match
probability 0.85), so the accepted lengths vary from step to step; the JSON
line reports their mean and histogram.  The steps are captured in a HIP
graph; W warm-up replays, then 5 repeats of K timed replays, each between two
synchronisations; the median repeat is reported.  Prints ONE JSON line.

The block attention (the dominant kernel) is timed alone as well, and next to
it the read-only streaming ceiling of one launch that reads the same number of
bytes (orthrus_stream_read over distinct buffers back to back):
"roofline.frac_of_ceiling".  --stream-ceiling prints only that ceiling.

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
LM_SOURCES = ("ar_shared_kv_amd/csrc/lmhead.hip", "ar_shared_kv_amd/csrc/common.hpp",
              "ar_shared_kv_amd/csrc/wtile.hpp")


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
    ap.add_argument("--steps", type=int, default=50)
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
    ap.add_argument("--draws", type=int, default=0,
                    help="seeded consensus-logits draws cycled by consecutive steps "
                         "(0 = 16 when they fit in 512 MiB, else 1)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed repeats of --steps replays; the median is reported")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only measure the read-only streaming ceiling of one launch "
                         "(34 MB and 537 MB per launch, distinct buffers back to back)")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="KV-cache element type: bf16, or OCP E4M3 codes with a power-of-two "
                         "scale per row and head (half the cache bytes)")
    ap.add_argument("--decode-step", action="store_true",
                    help="time one whole Orthrus decode step of a 36-layer random-weight "
                         "Qwen3-8B-shaped model (both views' passes with every layer, fused "
                         "LM-head argmax, consensus, append) at L=8192, K=32")
    ap.add_argument("--mdiff", action="store_true",
                    help="time the training-time block-mask (M_diff) attention forward on a "
                         "4 x 4,096-token micro-batch at the Qwen3-8B shape instead")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-ceiling measurement of the default run")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """Device-resident inputs and outputs of one decode step of a workload."""

    def __init__(self, cfg, splits, sets=0, draws=0, dev="cuda", kv="bf16"):
        import torch
        import workloads as W
        from ar_shared_kv_amd import api
        self.cfg = cfg
        self.splits = splits
        self.kv8 = kv == "fp8"
        nl = cfg.layers
        st = W.step_inputs(cfg, layers=1, with_logits=True)   # shapes + logits + lens
        # Input sets cycled by consecutive steps, so that a small workload's
        # inputs are not served from the 256 MB last-level cache: enough
        # copies of the step's inputs to span 512 MiB.
        e = 2 if cfg.dtype == "bf16" else 4
        lay0 = st.layers[0]
        per_set = nl * e * sum(getattr(lay0, k).numel() for k in
                               ("q_diff", "q_ar", "k_blk_diff", "v_blk_diff", "k_blk_ar",
                                "v_blk_ar"))
        # the cache: E4M3 codes (one byte) and one fp32 scale per row, or dtype
        ncache = lay0.k_cache.numel() + lay0.v_cache.numel()
        per_set += nl * (ncache + 4 * ncache // cfg.D if self.kv8 else e * ncache)
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
        cdt = torch.uint8 if self.kv8 else dt
        self.kc = torch.empty((nt, *cshape), dtype=cdt, device=dev)
        self.vc = torch.empty_like(self.kc)
        if self.kv8:
            self.ks = torch.empty((nt, *cshape[:-1]), dtype=torch.float32, device=dev)
            self.vs = torch.empty_like(self.ks)
        qs = (nt, cfg.B, cfg.K, cfg.Hq, cfg.D)
        bs = (nt, cfg.B, cfg.K, cfg.Hkv, cfg.D)
        self.q = {v: torch.empty(qs, dtype=dt, device=dev) for v in ("diff", "ar")}
        self.kb = {v: torch.empty(bs, dtype=dt, device=dev) for v in ("diff", "ar")}
        self.vb = {v: torch.empty(bs, dtype=dt, device=dev) for v in ("diff", "ar")}
        t0 = time.time()
        for l in range(nl):
            lay = st.layers[0] if l == 0 else W.layer_inputs(cfg, l, st.lens, st.num_pages,
                                                              st.capacity)
            if self.kv8:
                kc8, ks = W.fp8_cache(lay.k_cache, W.seed_of(cfg, W.T_FP8_KS, l))
                vc8, vs = W.fp8_cache(lay.v_cache, W.seed_of(cfg, W.T_FP8_VS, l))
                self.kc[l].copy_(kc8)
                self.vc[l].copy_(vc8)
                self.ks[l].copy_(ks)
                self.vs[l].copy_(vs)
            else:
                self.kc[l].copy_(lay.k_cache)
                self.vc[l].copy_(lay.v_cache)
            for v in ("diff", "ar"):
                self.q[v][l].copy_(getattr(lay, f"q_{v}"))
                self.kb[v][l].copy_(getattr(lay, f"k_blk_{v}"))
                self.vb[v][l].copy_(getattr(lay, f"v_blk_{v}"))
        scales = [self.ks, self.vs] if self.kv8 else []
        for x in [self.kc, self.vc] + scales + [d[v] for d in (self.q, self.kb, self.vb)
                                                for v in ("diff", "ar")]:
            for si in range(1, sets):   # copies: other addresses, same values
                x[si * nl:(si + 1) * nl].copy_(x[:nl])
        log(f"inputs for {nl} layers x {sets} input sets generated in {time.time() - t0:.1f}s")
        self.step_inputs = st
        # Consensus logits: `draws` independent seeded draws (the workload's
        # match probabilities), cycled by consecutive steps so that the
        # accepted lengths vary as they would over a generation.
        lbytes = e * (st.diff_logits.numel() + st.ar_logits.numel())
        if draws <= 0:
            draws = 16 if 16 * lbytes <= (512 << 20) else 1
        self.draws = draws
        # steps per replay: every input set and every draw at least once
        self.nsteps = max(sets, draws)
        self.diff_logits, self.ar_logits = [], []
        for d in range(draws):
            if d == 0:
                dl, al = st.diff_logits, st.ar_logits
            else:
                dl, al = W.consensus_logits(cfg.B, cfg.K, cfg.V, W.match_probabilities(cfg),
                                            cfg.torch_dtype,
                                            W.seed_of(cfg, W.T_LOGITS, salt=1000 + d))
            self.diff_logits.append(dl.to(dev))
            self.ar_logits.append(al.to(dev))
        lmax = int(st.lens.max())
        self.caches = [api.make_cache(self.kc[l], self.vc[l], self.lens,
                                      page_table=self.page_table, max_len=lmax,
                                      k_scale=self.ks[l] if self.kv8 else None,
                                      v_scale=self.vs[l] if self.kv8 else None)
                       for l in range(nt)]
        self.out = torch.empty(qs[1:], dtype=dt, device=dev)
        self.lse = torch.empty((cfg.B, cfg.Hq, cfg.K), dtype=torch.float32, device=dev)
        dcode = api.dtype_code(self.q["ar"])
        self.ws, self.ws_bytes = api.block_attn_workspace(self.caches[0], cfg.B, cfg.K, cfg.Hq,
                                                          cfg.Hkv, cfg.D, dcode, splits, dev)
        self.cbufs = [api.ConsensusBuffers(cfg.B, cfg.K, cfg.V, dcode, dev)
                      for _ in range(draws)]

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
        """`nsteps` consecutive decode steps: step j uses input set j % sets
        and logits draw j % draws."""
        from ar_shared_kv_amd import api
        nl = self.cfg.layers
        for j in range(self.nsteps):
            si, d = j % self.sets, j % self.draws
            self.attention_set(si)
            bufs = api.consensus(self.diff_logits[d], self.ar_logits[d], self.cbufs[d])
            api.kv_append(self.caches[si * nl], self.kb["ar"][si * nl], self.vb["ar"][si * nl],
                          bufs.n_emit, self.lens_out, num_layers=nl,
                          cache_layer_stride=self.kc[0].numel(),
                          blk_layer_stride=self.kb["ar"][0].numel())

    # algorithmic bytes: every input read once, every output written once
    def attn_bytes_per_launch(self):
        c = self.cfg
        e = 2 if c.dtype == "bf16" else 4
        # K and V rows of the cache: D elements each (E4M3: one byte per code
        # plus the row's fp32 scale)
        row = c.D * 1 + 4 if self.kv8 else c.D * e
        cache = int(self.step_inputs.lens.sum()) * c.Hkv * row * 2
        blk = c.B * c.K * (2 * c.Hq + 2 * c.Hkv) * c.D * e
        return cache + blk + c.B * c.Hq * c.K * 4

    def attn_flops_per_launch(self):
        c = self.cfg
        return 4 * c.Hq * c.D * sum(c.K * (int(L) + c.K) for L in self.step_inputs.lens)

    def step_bytes(self, n_mean_total):
        """Algorithmic bytes of one step with n_mean_total accepted rows (summed
        over the batch, averaged over the steps of a replay)."""
        c = self.cfg
        e = 2 if c.dtype == "bf16" else 4
        logits = 2 * c.B * c.K * c.V * e
        row_out = c.D * 1 + 4 if self.kv8 else c.D * e
        append = 2 * c.Hkv * (c.D * e + row_out) * n_mean_total * c.layers
        return 2 * c.layers * self.attn_bytes_per_launch() + logits + append


def timed(fn, steps, warmup, graph, repeats=1, stream=None):
    """Per-call milliseconds of `fn` (captured in a HIP graph unless graph is
    False): warm-up calls, then `repeats` timed runs of `steps` calls, each
    between two synchronisations and timed with events on the launch stream.
    Returns (median ms, list of per-repeat ms)."""
    import statistics
    import torch
    s = stream or torch.cuda.current_stream()
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
    per = []
    for _ in range(max(1, repeats)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(steps):
            run()
        e1.record(s)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / steps)
    return statistics.median(per), per


def stream_ceiling(nbytes, n_buffers, wgs_list, steps=20, warmup=5):
    """The read-only streaming rate of one launch reading `nbytes`, launches
    back to back over `n_buffers` distinct buffers (so that the 256 MB
    last-level cache cannot serve a repeat), captured in a HIP graph; one
    entry per work-group count.  Every byte is read once per launch."""
    import torch
    from ar_shared_kv_amd import _binding as B_
    nbytes -= nbytes % 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_buffers)]
    sink = torch.empty(max(wgs_list), dtype=torch.int32, device="cuda")
    out = []
    for wgs in wgs_list:
        def launches(wgs=wgs):
            for b in bufs:
                B_.check("orthrus_stream_read", B_.orthrus_stream_read(b, nbytes, wgs, sink))
        ms, _ = timed(launches, steps, warmup, True)
        us = ms * 1e3 / n_buffers
        out.append({"work_groups": wgs, "us_per_launch": round(us, 3),
                    "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)})
    del bufs
    torch.cuda.synchronize()
    return {"bytes_per_launch": nbytes, "buffers": n_buffers, "sweep": out,
            "best_gbps": max(r["gbps"] for r in out)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(step: Step, budget_s: float):
    """The oracle on the host cores: whole layers of the step until ~budget_s
    with every thread, then one layer with one thread; each extrapolated to
    the full step (consensus and a 1-layer append timed once per leg)."""
    import oracle
    import workloads as W
    cfg = step.cfg
    st = step.step_inputs
    lens = st.lens.numpy()
    pt = st.page_table.numpy() if cfg.paged else None
    kw = dict(scale=cfg.scale)
    if cfg.paged:
        kw.update(layout=oracle.PAGED, page_table=pt)
    raw = lambda t: t.view(torch_int(t)).numpy()  # noqa: E731

    def layer_arrays(l):
        lay = st.layers[0] if l == 0 else W.layer_inputs(cfg, l, st.lens, st.num_pages,
                                                        st.capacity)
        return {k: getattr(lay, k).double().numpy() for k in
                ("q_diff", "q_ar", "k_cache", "v_cache", "k_blk_diff", "v_blk_diff",
                 "k_blk_ar", "v_blk_ar")}

    def layer_pair(a):
        oracle.block_attn(a["q_diff"], a["k_cache"], a["v_cache"], a["k_blk_diff"],
                          a["v_blk_diff"], lens, mask=oracle.BIDIR, **kw)
        oracle.block_attn(a["q_ar"], a["k_cache"], a["v_cache"], a["k_blk_ar"],
                          a["v_blk_ar"], lens, mask=oracle.CAUSAL, **kw)

    def tail():
        dl = st.diff_logits.double().numpy()
        al = st.ar_logits.double().numpy()
        t0 = time.perf_counter()
        r = oracle.consensus(oracle.argmax_rows(dl), oracle.argmax_rows(al))
        lay = st.layers[0]
        t1 = time.perf_counter()
        oracle.kv_append(raw(lay.k_cache)[None], raw(lay.v_cache)[None], raw(lay.k_blk_ar)[None],
                         raw(lay.v_blk_ar)[None], r["n"], lens,
                         layout=oracle.PAGED if cfg.paged else oracle.CONTIGUOUS, page_table=pt)
        return t1 - t0, time.perf_counter() - t1

    threads = oracle.num_threads()
    t_layers, done = 0.0, 0
    first = None
    while done < cfg.layers:
        a = layer_arrays(done)
        if first is None:
            first = a
        t0 = time.perf_counter()
        layer_pair(a)
        t_layers += time.perf_counter() - t0
        done += 1
        if t_layers >= budget_s:
            break
    t_cons, t_app = tail()
    step_s = t_layers / done * cfg.layers + t_cons + t_app * cfg.layers
    # one thread: a single layer pair (the cost per layer does not depend on
    # which layer), consensus and the 1-layer append
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        layer_pair(first)
        t1_layer = time.perf_counter() - t0
        t1_cons, t1_app = tail()
    finally:
        oracle.set_num_threads(threads)
    step1_s = t1_layer * cfg.layers + t1_cons + t1_app * cfg.layers
    sample = (f"oracle fp64 on {done} of {cfg.layers} layers (BIDIR+CAUSAL passes at full shape), "
              f"consensus and a 1-layer append, extrapolated to the {cfg.layers}-layer step; "
              f"the 1-thread leg on 1 layer")
    return {"value": round(1.0 / step_s, 6), "unit": "steps/s", "cores": threads,
            "kind": "oracle", "sample": sample, "cpu_model": cpu_model(),
            "value_1thread": round(1.0 / step1_s, 6),
            "seconds_measured": round(t_layers + t_cons + t_app + t1_layer + t1_cons + t1_app, 2)}


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
    hd, wd = h.cuda(), api.pack_weight(w.cuda())     # the layout step, untimed
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    n = B_.orthrus_lmhead_argmax_workspace_bytes(R, H, V, B_.BF16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    call = lambda: api.lmhead_argmax(hd, wd, idx=idx, workspace=ws)
    ms, per = timed(call, args.steps, args.warmup, not args.no_graph, args.repeats)
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
    if args.stream_ceiling:
        ceiling_main(args)
        return
    if args.mdiff:
        mdiff_main(args)
        return
    if args.decode_step:
        decode_step_main(args)
        return
    cfg = W.CONFIGS[args.config]
    if args.K:
        cfg = cfg.with_(K=args.K)
    splits = args.splits or cfg.num_splits
    log(f"workload {cfg.name} K={cfg.K} splits={splits or 'auto'}")
    calibrate(args.calib_bytes)
    step = Step(cfg, splits, args.sets, args.draws, kv=args.kv)
    graph = not args.no_graph

    ms_run, per_run = timed(step.run, args.steps, args.warmup, graph, args.repeats)
    ms_step = ms_run / step.nsteps
    log(f"step: median {ms_step:.5f} ms over {args.repeats} repeats "
        f"({', '.join(f'{m / step.nsteps:.5f}' for m in per_run)})")
    # the dominant kernel: block attention alone, all 2*layers passes per step
    ms_attn_all, per_attn = timed(step.attention_passes, args.steps, args.warmup, graph,
                                  args.repeats)
    us_attn = ms_attn_all * 1e3 / (2 * cfg.layers * step.sets)
    # accepted rows of every draw (each draw's outputs are its own buffers)
    import torch
    n_all = torch.stack([b.n_emit for b in step.cbufs]).cpu()      # [draws, B]
    n_mean_total = float(n_all.sum(dim=1).float().mean())

    attn_b = step.attn_bytes_per_launch()
    attn_f = step.attn_flops_per_launch()
    achieved_gbps = attn_b / (us_attn * 1e-6) / 1e9
    steps_s = 1e3 / ms_step
    hist = torch.bincount(n_all.flatten().long(), minlength=cfg.K + 1).tolist()
    res = {
        "metric": METRIC,
        "value": round(steps_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps * step.nsteps,
        "warmup": args.warmup * step.nsteps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "K": cfg.K, "L": cfg.L if cfg.L_range is None else list(cfg.L_range),
                   "layers": cfg.layers, "V": cfg.V, "paged": cfg.paged,
                   "num_splits": splits or "auto", "graph": graph, "input_sets": step.sets,
                   "logits_draws": step.draws, "kv_cache": args.kv},
        "timing": {"repeats": args.repeats, "statistic": "median",
                   "ms_per_step_repeats": [round(m / step.nsteps, 5) for m in per_run],
                   "us_per_attn_launch_repeats":
                       [round(m * 1e3 / (2 * cfg.layers * step.sets), 3) for m in per_attn]},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if (args.K or step.kv8) else measured_traffic(cfg.name,
                                                                                  args.splits),
                     "kernel": "block attention (attn_bf16_kernel + split merge), per launch"
                               + (", E4M3 cache" if step.kv8 else ""),
                     "us_per_launch": round(us_attn, 3), "bytes_per_launch": attn_b,
                     "mfma_frac": round(attn_f / (us_attn * 1e-6) / 2.5e15, 4)},
        "step_hbm_tbps": round(step.step_bytes(n_mean_total) / (ms_step * 1e-3) / 1e12, 3),
        "accepted": {"mean_n_per_request": round(n_mean_total / cfg.B, 3),
                     "histogram_n": {str(i): c for i, c in enumerate(hist) if c},
                     "samples": int(n_all.numel()),
                     "expected_n": round(expected_n(cfg), 3)},
    }
    if not args.no_ceiling:
        # the same bytes per launch as one attention pass, read with nothing
        # else to do, over enough distinct buffers to span 1 GiB
        nbuf = max(4, -(-(1 << 30) // attn_b))
        ceil = stream_ceiling(attn_b, nbuf, [208, 256, 512, 1024, 2048])
        res["roofline"]["ceiling_gbps"] = ceil["best_gbps"]
        res["roofline"]["frac_of_ceiling"] = round(achieved_gbps / ceil["best_gbps"], 4)
        res["stream_ceiling"] = ceil
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def expected_n(cfg):
    """E[n] = (1 - p^K) / (1 - p) per request, averaged over the batch's p."""
    import workloads as W
    p = W.match_probabilities(cfg)
    ps = p if isinstance(p, (list, tuple)) else [p]
    return sum(cfg.K if q >= 1 else (1 - q ** cfg.K) / (1 - q) for q in ps) / len(ps)


def mdiff_main(args):
    """The training-time block mask M_diff, forward: every block of K = 32
    positions of 4 sequences of 4,096 tokens (Qwen3-8B attention shape) sees
    the clean context before its anchor and its own block.  Bound: the matrix
    cores (the FLOPs at peak take longer than the unique bytes at peak)."""
    import torch
    import workloads as W
    from ar_shared_kv_amd import api
    wl = W.MDIFF_WORKLOAD
    Bn, N, K, Hq, Hkv, D = wl["B"], wl["N"], wl["K"], wl["Hq"], wl["Hkv"], wl["D"]
    inp = W.mdiff_inputs(Bn, N, K, Hq, Hkv, D, layout=wl["layout"])
    d = {k: getattr(inp, k).cuda() for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx", "anchors")}
    out = torch.empty_like(d["q"])
    NB = inp.q.shape[1]
    lse = torch.empty((Bn, NB, Hq, K), dtype=torch.float32, device="cuda")
    call = lambda: api.mdiff_attn(d["q"], d["k_blk"], d["v_blk"], d["k_ctx"], d["v_ctx"],  # noqa
                                  d["anchors"], max_anchor=N, out=out, lse=lse)
    ms, per = timed(call, args.steps, args.warmup, not args.no_graph, args.repeats)
    a = inp.anchors.long()
    flops = 4 * Hq * D * K * int((a + K).sum())
    e = 2
    nbytes = (2 * Bn * Hkv * N * D * e + 2 * inp.q.numel() * e + 2 * inp.k_blk.numel() * e
              + 4 * lse.numel())
    tf = flops / (ms * 1e-3) / 1e12
    gbps = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "M_diff block-mask attention forward calls/s (training micro-batch)",
        "value": round(1e3 / ms, 3), "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "B": Bn, "N": N, "K": K, "blocks_per_seq": NB,
                   "Hq": Hq, "Hkv": Hkv, "D": D, "layout": wl["layout"],
                   "graph": not args.no_graph},
        "timing": {"repeats": args.repeats, "statistic": "median",
                   "ms_repeats": [round(m, 5) for m in per]},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4), "traffic": None,
                     "kernel": "attn_bf16_kernel (blocks as requests over a shared context)",
                     "us_per_launch": round(ms * 1e3, 3), "flops_per_launch": flops,
                     "bytes_per_launch": nbytes, "hbm_gbps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)},
    }
    if flops / 2.5e15 < nbytes / (HBM_PEAK_GBPS * 1e9):
        res["roofline"].update(bound="hbm", achieved=round(gbps, 1), peak=HBM_PEAK_GBPS,
                               unit="GB/s", frac=round(gbps / HBM_PEAK_GBPS, 4))
    if not args.no_cpu:
        import oracle
        # the oracle on every 16th block of the first sequence, scaled by FLOPs
        sel = list(range(NB - 1, -1, -16))
        sub = {k: getattr(inp, k)[:1, sel].contiguous() for k in ("q", "k_blk", "v_blk")}
        anc = inp.anchors[:1, sel].contiguous()
        t0 = time.perf_counter()
        oracle.mdiff_attn(sub["q"].double().numpy(), inp.k_ctx[:1].double().numpy(),
                          inp.v_ctx[:1].double().numpy(), anc.numpy(),
                          sub["k_blk"].double().numpy(), sub["v_blk"].double().numpy(),
                          scale=D ** -0.5)
        t = time.perf_counter() - t0
        sub_flops = 4 * Hq * D * K * int((anc.long() + K).sum())
        res["cpu_baseline"] = {"value": round(sub_flops / flops / t, 6), "unit": "calls/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "cpu_model": cpu_model(),
                               "sample": f"fp64 oracle on {len(sel)} of {Bn * NB} blocks "
                                         "(every 16th block of sequence 0), scaled by FLOPs"}
    print(json.dumps(res), flush=True)


def decode_step_main(args):
    """One whole decode step of a 36-layer Qwen3-8B-shaped model with random
    weights (drawn on the GPU, seeded), B = 1, K = 32, a synthetic 8,192-row
    cache per layer: the diffusion pass (36 layers, bidirectional block), its
    greedy candidates, the AR pass (36 layers, causal block), consensus, the
    36-layer append.  Algorithmic bytes: every weight matrix each pass reads
    (the views' own attention projections, the shared MLP, the LM head), the
    caches twice, the block rows, and the append.  The weight-streaming
    projections dominate."""
    import torch
    import workloads as W
    from ar_shared_kv_amd.decode import DecodeModel, Dims
    d = Dims(layers=36)
    B, K, L = 1, 32, 8192
    cap = L + K
    t0 = time.time()
    w = W.model_weights(d, seed=0, device="cuda")
    gm = DecodeModel(d, w, B, K, cap)
    g = torch.Generator(device="cuda").manual_seed(77)
    gm.kc.copy_(torch.randn(gm.kc.shape, generator=g, device="cuda").to(torch.bfloat16))
    gm.vc.copy_(torch.randn(gm.vc.shape, generator=g, device="cuda").to(torch.bfloat16))
    gm.set_lengths(L)
    gm.anchor.fill_(1234)
    log(f"36-layer model and caches ready in {time.time() - t0:.1f}s")
    step = lambda: gm.orthrus_step(advance=False)  # noqa: E731
    ms, per = timed(step, args.steps, args.warmup, not args.no_graph, args.repeats)
    nqkv = (d.Hq + 2 * d.Hkv) * d.D
    layer_w = 2 * (nqkv * d.H + d.H * d.Hq * d.D + 2 * d.I * d.H + d.H * d.I)    # bytes, per view
    kv_bytes = L * d.Hkv * d.D * 2 * 2                                          # one layer's cache
    blk = B * K * (2 * d.Hq + 2 * d.Hkv) * d.D * 2                              # q, o, block K/V
    step_bytes = 2 * (d.layers * (layer_w + kv_bytes + blk) + 2 * d.V * d.H) \
        + d.layers * 2 * d.Hkv * d.D * 2 * 2 * B                                 # + the append
    gbps = step_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "Orthrus decode steps/s, whole model (36-layer Qwen3-8B shape, random weights)",
        "value": round(1e3 / ms, 3), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3-8b-36layers-decode-step", "B": B, "K": K, "L": L,
                   "layers": d.layers, "H": d.H, "I": d.I, "V": d.V, "graph": not args.no_graph},
        "timing": {"repeats": args.repeats, "statistic": "median",
                   "ms_repeats": [round(m, 5) for m in per]},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "whole step (weight-streaming projections dominate)",
                     "bytes_per_step": step_bytes},
        "accepted_n": gm.n_emit.cpu().tolist(),
    }
    print(json.dumps(res), flush=True)


def ceiling_main(args):
    """Only the streaming ceiling: one launch reading one attention pass's bytes
    at the Qwen3-8B shape (34 MB), and a long launch (537 MB)."""
    res = {"metric": "read-only streaming ceiling of one launch", "unit": "GB/s", "n_gpus": 1,
           "higher_is_better": True, "data": "synthetic", "dtype": "u8",
           "config": {"workload": "stream-read"}, "launches": []}
    for nbytes, nbuf in ((34213888, 36), (536870912, 4)):
        res["launches"].append(stream_ceiling(nbytes, nbuf, [208, 256, 512, 1024, 2048],
                                              steps=args.steps, warmup=args.warmup))
    res["value"] = res["launches"][0]["best_gbps"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
