"""Pins for the oracle's FP8 (OCP E4M3) KV-cache functions (CPU only).

* decode: all 256 codes against torch's float8_e4m3fn (a library
  implementation of the same format);
* encode (round to nearest, ties to even): every code's value, every
  midpoint between neighbouring codes (the tie cases), points just off the
  midpoints, and a dense random sweep, against torch's conversion;
* the scale exponent against the definition checked by brute force and a
  closed form at the binade edges;
* the quantizing append: only the appended rows change, codes decode to
  within half a unit of the format's precision, the scale is the power of
  two the definition picks;
* attention over the dequantized cache equals attention over a cache that
  holds those values in fp64 (the definition the GPU path is tested
  against).
"""
import math

import numpy as np
import pytest
import torch

import oracle

F8 = torch.float8_e4m3fn


def torch_decode(codes):
    return torch.tensor(codes, dtype=torch.uint8).view(F8).float().double().numpy()


def torch_encode(xs):
    # from fp32 (every test point is an fp32 value): one rounding, to E4M3
    x32 = np.asarray(xs, dtype=np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(xs, dtype=np.float64))
    return torch.from_numpy(x32).to(F8).view(torch.uint8).numpy().astype(int)


def test_decode_every_code_matches_the_library():
    ref = torch_decode(list(range(256)))
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    assert oracle.e4m3_decode(0x7E) == 448.0 and oracle.e4m3_decode(0x01) == 2.0 ** -9


def finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_encode_exact_values_and_ties_to_even():
    vals = sorted({oracle.e4m3_decode(c) for c in finite_codes()})
    pts = list(vals)
    for a, b in zip(vals, vals[1:]):
        mid = np.float32((a + b) / 2)          # exact (3 mantissa bits + 1)
        pts += [float(mid), float(np.nextafter(mid, np.float32(-np.inf))),
                float(np.nextafter(mid, np.float32(np.inf)))]
    ref = torch_encode(pts)
    got = [oracle.e4m3_encode(x) for x in pts]
    # +0 and -0 both decode to zero; compare by code except for the sign of zero
    for x, g, r in zip(pts, got, ref):
        if oracle.e4m3_decode(r) == 0.0:
            assert oracle.e4m3_decode(g) == 0.0 and math.copysign(1, x) * 1 == \
                (-1 if g & 0x80 else 1), (x, g, r)
        else:
            assert g == r, (x, hex(g), hex(r))


def test_encode_random_sweep_matches_the_library():
    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.uniform(-448, 448, 20000),
                         rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)])
    xs = np.clip(xs, -448, 448).astype(np.float32).astype(np.float64)
    ref = torch_encode(xs)
    got = np.array([oracle.e4m3_encode(x) for x in xs])
    nz = np.array([oracle.e4m3_decode(r) != 0.0 for r in ref])
    np.testing.assert_array_equal(got[nz], ref[nz])
    with pytest.raises(ValueError):
        oracle.e4m3_encode(449.0)


def test_scale_exponent_definition():
    rng = np.random.default_rng(3)
    amaxes = np.concatenate([[448.0, 448.0 * 2 ** -5, 1.0, 1.75, 1.7500001, 3.5, 2.0 ** -140,
                              3.0e38], np.abs(rng.standard_normal(2000)) * 10.0 ** rng.uniform(
                                  -8, 8, 2000)])
    for a in amaxes:
        e = oracle.fp8_scale_exp(a)
        assert e >= -120
        assert 448.0 * 2.0 ** e >= a
        if e > -120:
            assert 448.0 * 2.0 ** (e - 1) < a
    assert oracle.fp8_scale_exp(0.0) == 0
    assert oracle.fp8_scale_exp(448.0) == 0 and oracle.fp8_scale_exp(448.0001) == 1
    assert oracle.fp8_scale_exp(1.75) == -8 and oracle.fp8_scale_exp(1.751) == -7


def test_append_fp8_touches_only_the_appended_rows_and_quantizes_by_definition():
    rng = np.random.default_rng(4)
    layers, B, K, Hkv, D, cap = 2, 3, 5, 2, 128, 40
    kc = rng.integers(0, 0x7E, (layers, B, Hkv, cap, D)).astype(np.uint8)
    vc = rng.integers(0, 0x7E, (layers, B, Hkv, cap, D)).astype(np.uint8)
    ks = np.full((layers, B, Hkv, cap), 0.25, np.float32)
    vs = np.full((layers, B, Hkv, cap), 0.5, np.float32)
    kb = torch.randn((layers, B, K, Hkv, D), dtype=torch.float64).to(torch.bfloat16)
    vb = (torch.randn((layers, B, K, Hkv, D), dtype=torch.float64) * 100).to(torch.bfloat16)
    kb[0, 0, 2, 1] = 0.0                        # an all-zero row: scale 1, codes 0
    n = np.array([5, 0, 2], np.int32)
    lens = np.array([0, 17, 38], np.int32)
    kbd, vbd = kb.double().numpy(), vb.double().numpy()
    k2, v2, ks2, vs2, lo = oracle.kv_append_fp8(kc, vc, ks, vs, kbd, vbd, n, lens)
    np.testing.assert_array_equal(lo, lens + n)
    changed = np.zeros((layers, B, Hkv, cap), bool)
    for b in range(B):
        changed[:, b, :, lens[b]:lens[b] + n[b]] = True
    np.testing.assert_array_equal(k2[~changed], kc[~changed])
    np.testing.assert_array_equal(ks2[~changed], ks[~changed])
    for l in range(layers):
        for b in range(B):
            for i in range(n[b]):
                for g in range(Hkv):
                    for src, codes, sc in ((kbd, k2, ks2), (vbd, v2, vs2)):
                        x = src[l, b, i, g]
                        e = oracle.fp8_scale_exp(np.abs(x).max())
                        assert sc[l, b, g, lens[b] + i] == 2.0 ** e
                        deq = oracle.dequant_fp8(codes[l, b, g, lens[b] + i],
                                                 sc[l, b, g, lens[b] + i])
                        # round to nearest: within half a step of the format
                        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(
                            np.abs(x) / 2.0 ** e, 2.0 ** -6))) - 3), 2.0 ** -9) * 2.0 ** e
                        assert np.all(np.abs(deq - x) <= step / 2 + 1e-300)
    assert np.all(k2[0, 0, 1, 2] == 0) and ks2[0, 0, 1, 2] == 1.0
    np.testing.assert_array_equal(k2[:, 1], kc[:, 1])           # n[1] = 0: untouched


def test_attention_over_dequantized_cache():
    rng = np.random.default_rng(5)
    B, K, Hq, Hkv, D, cap = 2, 4, 4, 2, 128, 50
    codes_k = rng.integers(0, 0x7E, (B, Hkv, cap, D)).astype(np.uint8) | \
        (rng.integers(0, 2, (B, Hkv, cap, D)) << 7).astype(np.uint8)
    codes_v = rng.integers(0, 0x7E, (B, Hkv, cap, D)).astype(np.uint8)
    sk = 2.0 ** rng.integers(-9, -5, (B, Hkv, cap)).astype(np.float32)
    sv = 2.0 ** rng.integers(-9, -5, (B, Hkv, cap)).astype(np.float32)
    kd, vd = oracle.dequant_fp8(codes_k, sk), oracle.dequant_fp8(codes_v, sv)
    ref = torch_decode(list(range(256)))
    np.testing.assert_array_equal(kd, ref[codes_k] * sk[..., None])
    q = rng.standard_normal((B, K, Hq, D))
    kb, vb = rng.standard_normal((B, K, Hkv, D)), rng.standard_normal((B, K, Hkv, D))
    lens = np.array([50, 13], np.int32)
    o1, l1 = oracle.block_attn(q, kd, vd, kb, vb, lens, mask=oracle.CAUSAL, scale=D ** -0.5)
    assert np.isfinite(o1).all() and np.isfinite(l1).all()
