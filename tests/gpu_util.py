"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, run the fp64 oracle on the same inputs,
and compare to the tolerances the method's target fixes (bf16 inputs with
fp32 accumulation: max abs error <= 1e-2; fp32 inputs: <= 1e-5; tokens,
counts and the appended cache: bit-exact)."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import oracle
import workloads as W
from ar_shared_kv_amd import api
from ar_shared_kv_amd import _binding as B_

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}
# extra guards, so that a dropped tile cannot hide under the absolute bound:
# relative to the largest |O|, and on lse.  The bf16 path's row sum is the sum
# of the bf16-rounded weights (so that O is an exact convex combination of V
# rows); each carries a relative rounding error of at most 2^-8, so its lse
# may differ from the exact one by up to -ln(1 - 2^-8) = 3.91e-3 plus fp32
# terms.  Dropping 1/32 of 2,048 keys moves lse by about 0.03.
REL_GUARD = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
LSE_TOL = {torch.bfloat16: 4e-3, torch.float32: 1e-5}
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def dev(t):
    return None if t is None else t.to(DEV)


def cache_for(step: W.StepInputs, layer: W.LayerInputs, max_len=0):
    cfg = step.cfg
    lens = dev(step.lens)
    kc, vc = dev(layer.k_cache), dev(layer.v_cache)
    if cfg.paged:
        return api.make_cache(kc, vc, lens, page_table=dev(step.page_table), max_len=max_len)
    return api.make_cache(kc, vc, lens, max_len=max_len)


def oracle_attn(step: W.StepInputs, layer: W.LayerInputs, view: str, requests=None, kv_heads=None):
    """Oracle block attention for view 'diff' (BIDIR) or 'ar' (CAUSAL).

    ``requests``/``kv_heads`` restrict the computation to a sample (the
    oracle then sees a sliced problem); outputs are for that sample only.
    """
    cfg = step.cfg
    q = layer.q_diff if view == "diff" else layer.q_ar
    kb = layer.k_blk_diff if view == "diff" else layer.k_blk_ar
    vb = layer.v_blk_diff if view == "diff" else layer.v_blk_ar
    mask = oracle.BIDIR if view == "diff" else oracle.CAUSAL
    lens = step.lens.numpy()
    kc, vc = layer.k_cache, layer.v_cache
    pt = step.page_table.numpy() if cfg.paged else None
    if requests is not None:
        rq = list(requests)
        q, kb, vb, lens = q[rq], kb[rq], vb[rq], lens[rq]
        if cfg.paged:
            pt = pt[rq]
        else:
            kc, vc = kc[rq], vc[rq]
    if kv_heads is not None:
        hs = list(kv_heads)
        qh = [g * cfg.G + j for g in hs for j in range(cfg.G)]
        q = q[:, :, qh]
        kb, vb = kb[:, :, hs], vb[:, :, hs]
        kc, vc = kc[:, hs], vc[:, hs]
    kw = dict(mask=mask, scale=cfg.scale)
    if cfg.paged:
        kw.update(layout=oracle.PAGED, page_table=pt)
    return oracle.block_attn(f64(q), f64(kc), f64(vc), f64(kb), f64(vb), lens, **kw)


def gpu_attn(step: W.StepInputs, layer: W.LayerInputs, view: str, num_splits=0, max_len=0,
             cache=None):
    cfg = step.cfg
    q = dev(layer.q_diff if view == "diff" else layer.q_ar)
    kb = dev(layer.k_blk_diff if view == "diff" else layer.k_blk_ar)
    vb = dev(layer.v_blk_diff if view == "diff" else layer.v_blk_ar)
    mask = B_.BIDIR if view == "diff" else B_.CAUSAL
    if cache is None:
        cache = cache_for(step, layer, max_len=max_len)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((cfg.B, cfg.Hq, cfg.K), float("nan"), dtype=torch.float32, device=DEV)
    out, lse = api.block_attn(q, kb, vb, cache, mask=mask, scale=cfg.scale,
                              num_splits=num_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def half_ulp(x: np.ndarray, dtype) -> np.ndarray:
    """Half a unit in the last place of the output dtype at |x| (the rounding
    any output of that dtype carries; 8 significant bits for bf16).  Printed
    as a diagnostic only: the assertion is the plain max |err| bound."""
    if dtype == torch.float32:
        return np.zeros_like(x)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


# Per-case parity record: every comparison is kept in RESULTS (the test
# session's summary prints the worst margin of each kind) and, when
# ORTHRUS_PARITY_RECORD names a file, appended to it as one JSON line (case
# name, max |err|, error relative to max |O|, lse error, the bound).
RECORD = os.environ.get("ORTHRUS_PARITY_RECORD")
RESULTS: list = []


def record(kind: str, what: str, **fields):
    row = {"kind": kind, "case": what, **fields}
    RESULTS.append(row)
    if not RECORD:
        return
    try:
        if os.path.dirname(RECORD):
            os.makedirs(os.path.dirname(RECORD), exist_ok=True)
        with open(RECORD, "a") as fh:
            fh.write(json.dumps(row) + "\n")
    except OSError:
        pass


def assert_attn_close(out, lse, ref_out, ref_lse, dtype, what=""):
    """max |out - ref| <= TOL (1e-2 for bf16 inputs, 1e-5 for fp32), plus the
    relative and lse guards.  The error beyond the output's own rounding is
    printed and recorded next to it."""
    o = f64(out)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    diff = np.abs(o - ref_out)
    err = float(diff.max()) if diff.size else 0.0
    excess = float((diff - half_ulp(ref_out, dtype)).max()) if diff.size else 0.0
    omax = float(np.abs(ref_out).max()) if diff.size else 0.0
    rel = err / max(omax, 1e-30)
    lerr = float(np.abs(f64(lse) - ref_lse).max()) if lse is not None and diff.size else 0.0
    say(f"  {what}: max|err| {err:.3e} (bound {TOL[dtype]:.0e})  beyond-rounding {excess:.3e}  "
        f"max|O| {omax:.3e}  rel {rel:.3e}  lse err {lerr:.3e}")
    record("attention", what, max_err=err, bound=TOL[dtype], beyond_rounding=excess,
           max_abs_ref=omax, rel_err=rel, lse_err=lerr, lse_bound=LSE_TOL[dtype],
           dtype=str(dtype).replace("torch.", ""))
    assert err <= TOL[dtype], f"{what}: max|err| {err} > {TOL[dtype]}"
    assert rel <= REL_GUARD[dtype], f"{what}: error {rel} of max |O|"
    assert lerr <= LSE_TOL[dtype], f"{what}: lse error {lerr}"
    return err
