"""Pins the oracle's number formats and its cache writer.

Expected values come from library conversions (torch float8_e4m3fn and
bfloat16, numpy float16) and from the OCP E4M3 definition points stored in
tests/golden/ocp_e4m3_points.json, never from the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from pool_util import build_pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _h(s):
    return int(s, 16)


def test_e4m3_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_definition_points(orc):
    g = json.load(open(os.path.join(GOLDEN, "ocp_e4m3_points.json")))
    for code, val in g["decode"]:
        got = orc.e4m3_decode(np.array([_h(code)], np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert np.isnan(orc.e4m3_decode(np.array([_h(code)], np.uint8))[0])
    for val, code in g["encode"]:
        x = np.array([float(val)], np.float32)
        assert orc.e4m3_encode(x)[0] == _h(code), (val, code)


def test_e4m3_encode_matches_torch_below_overflow(orc):
    """torch rounds to nearest even but turns overflow into NaN; in the range
    where no overflow happens (|x| <= 464 rounds to at most 448) both rules
    coincide, so every bf16 value there and a random fp32 sample must agree."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = workloads.bf16_values(bits)
    rng = np.random.default_rng(0)
    y = np.concatenate([x, (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)])
    keep = np.isfinite(y) & (np.abs(y) <= 464.0)
    y = y[keep]
    ours = orc.e4m3_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_roundtrip_and_saturation(orc):
    codes = np.arange(256, dtype=np.uint8)
    finite = np.array([c not in (0x7F, 0xFF) for c in codes])
    vals = orc.e4m3_decode(codes[finite]).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), codes[finite])
    big = np.array([448.0, 449.0, 500.0, 1e30, np.inf], np.float32)
    assert np.all(orc.e4m3_encode(big) == 0x7E)
    assert np.all(orc.e4m3_encode(-big) == 0xFE)
    assert orc.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


def test_e4m3_midpoints_round_to_even(orc):
    codes = np.arange(0, 0x7E, dtype=np.uint8)          # positive finite, below max
    lo = orc.e4m3_decode(codes)
    hi = orc.e4m3_decode(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)   # exact in fp32
    got = orc.e4m3_encode(mid)
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, even)


def test_bf16_widening_matches_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f16_widening_matches_numpy(orc):
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ours = orc.widen(x, "f16")
    ref = x.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# --- cache writer ---------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_writer_same_dtype_matches_slice_scatter(orc, dtype):
    """Bit copy into slot//bs, slot%bs; skipped slots (negative, past the
    pool) and every other byte stay untouched."""
    rng = np.random.default_rng(31)
    NB, bs, H, D, T = 12, 8, 3, 64, 20
    k = workloads.draw(rng, (T, H, D), dtype)
    v = workloads.draw(rng, (T, H, D), dtype)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    slots[3] = -1
    slots[7] = NB * bs + 5
    kc = workloads.draw(rng, (NB, bs, H, D), dtype)
    vc = workloads.draw(rng, (NB, bs, H, D), dtype)
    ek, ev = kc.copy(), vc.copy()
    for i, sl in enumerate(slots):
        if 0 <= sl < NB * bs:
            ek.reshape(NB * bs, H, D)[sl] = k[i]
            ev.reshape(NB * bs, H, D)[sl] = v[i]
    orc.reshape_and_cache(k, v, kc, vc, slots, src_dtype=dtype, cache_dtype=dtype)
    assert kc.tobytes() == ek.tobytes() and vc.tobytes() == ev.tobytes()


@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
def test_writer_fp8_matches_torch_quantisation(orc, src):
    rng = np.random.default_rng(32)
    NB, bs, H, D, T = 6, 16, 2, 128, 40
    k = workloads.draw(rng, (T, H, D), src)
    v = workloads.draw(rng, (T, H, D), src)
    ks, vs = workloads.amax_scale(k, src), workloads.amax_scale(v, src)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    kc = np.full((NB, bs, H, D), 0x7F, np.uint8)
    vc = np.full((NB, bs, H, D), 0x7F, np.uint8)
    orc.reshape_and_cache(k, v, kc, vc, slots, src_dtype=src, cache_dtype="fp8",
                          k_scale=ks, v_scale=vs)
    for x, sc, cache in ((k, ks, kc), (v, vs, vc)):
        xf = torch.from_numpy(workloads._as_float32(x, src))
        q = (xf / torch.tensor(sc, dtype=torch.float32))          # fp32 divide
        assert float(q.abs().max()) <= 448.0 + 1e-3
        ref = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = cache.reshape(NB * bs, H, D)[slots]
        assert np.array_equal(got, ref)
    untouched = np.ones(NB * bs, bool)
    untouched[slots] = False
    assert np.all(kc.reshape(NB * bs, H, D)[untouched] == 0x7F)


def test_writer_then_gather_roundtrip(orc):
    """Write a whole sequence through the writer, gather it back through the
    block table: the logical K/V come back bit for bit."""
    rng = np.random.default_rng(33)
    c = workloads.make_case("rt", 34, [45, 3, 64], 4, 2, 64, 16, q_dtype="bf16",
                            cache_dtype="bf16")
    kc = np.full_like(c.k_cache, workloads.POISON["bf16"])
    vc = np.full_like(c.v_cache, workloads.POISON["bf16"])
    for s in range(c.S):
        L = int(c.seq_lens[s])
        K = workloads.draw(rng, (L, 2, 64), "bf16")
        V = workloads.draw(rng, (L, 2, 64), "bf16")
        slots = np.array([c.block_tables[s, t // 16] * 16 + t % 16 for t in range(L)], np.int64)
        orc.reshape_and_cache(K, V, kc, vc, slots, src_dtype="bf16", cache_dtype="bf16")
        for h in range(2):
            Kg, Vg = orc.gather_sequence(kc, vc, c.block_tables, c.seq_lens, s, h,
                                         cache_dtype="bf16")
            assert np.array_equal(Kg, workloads.bf16_values(K[:, h]).astype(np.float64))
            assert np.array_equal(Vg, workloads.bf16_values(V[:, h]).astype(np.float64))


def test_fp8_decode_uses_scaled_codes(orc):
    """fp8 cache: the oracle attends over decode(code) * scale; pinned by
    building the same K/V in f32 from torch-decoded codes."""
    c = workloads.shared_prefix_fp8(bs=16, S=4)
    kc, vc = c.k_cache.copy(), c.v_cache.copy()
    orc.reshape_and_cache(c.new_key, c.new_value, kc, vc, c.slot_mapping,
                          src_dtype="bf16", cache_dtype="fp8",
                          k_scale=c.k_scale, v_scale=c.v_scale)
    out = orc.paged_decode(c.query, kc, vc, c.block_tables, c.seq_lens,
                           q_dtype="bf16", cache_dtype="fp8", scale=c.scale,
                           k_scale=c.k_scale, v_scale=c.v_scale)
    assert np.isfinite(out).all()
    dk = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * c.k_scale
    dv = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * c.v_scale
    q = workloads.bf16_values(c.query).astype(np.float64)
    for s in range(c.S):
        L = int(c.seq_lens[s])
        nb = -(-L // 16)
        K = np.concatenate([dk[c.block_tables[s, j]] for j in range(nb)])[:L]
        V = np.concatenate([dv[c.block_tables[s, j]] for j in range(nb)])[:L]
        for hq in range(0, c.Hq, 7):
            h = hq // c.G
            z = (K[:, h] @ q[s, hq]) * c.scale
            p = np.exp(z - z.max())
            np.testing.assert_allclose(out[s, hq], p @ V[:, h] / p.sum(), atol=1e-12)
