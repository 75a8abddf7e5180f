"""Pins the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a worked example printed on
the pages (tests/golden/), a library routine (scipy softmax, numpy matmul,
torch/numpy format conversions), a closed form, or an invariant the method
guarantees.  Pages cited:
  [P4] "vLLM 推理引擎源码级拆解" (chenxutan.com/d/5333)
  [P2] "vLLM 深度实战" (chenxutan.com/d/3332)
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import workloads
from pool_util import build_pool, relabel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense_attention_fp64(q, K, V, scale):
    """Library-routine brute force: softmax(scale * K q) V in float64."""
    z = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    p = scipy.special.softmax(z)
    return p @ V.astype(np.float64)


def rand_logical(rng, lens, Hkv, D, dtype):
    Ks = [workloads.draw(rng, (L, Hkv, D), dtype) for L in lens]
    Vs = [workloads.draw(rng, (L, Hkv, D), dtype) for L in lens]
    return Ks, Vs


def widen(x, dtype, orc):
    return orc.widen(x, dtype)


# --- dense attention on tiny inputs (library routine) ---------------------

@pytest.mark.parametrize("seed", range(6))
def test_decode_matches_dense_softmax_on_tiny_inputs(orc, seed):
    rng = np.random.default_rng(100 + seed)
    dtype = ["f32", "f16", "bf16"][seed % 3]
    bs = [8, 16, 32][seed % 3]
    Hkv = [1, 2, 4][seed % 3]
    G = [1, 2, 4, 8][seed % 4]
    D = [64, 128][seed % 2]
    S = 3
    lens = rng.integers(1, 90, size=S)
    Ks, Vs = rand_logical(rng, lens, Hkv, D, dtype)
    kc, vc, tables, sl = build_pool(Ks, Vs, bs, dtype=dtype, rng=rng)
    q = workloads.draw(rng, (S, Hkv * G, D), dtype)
    scale = 1.0 / math.sqrt(D)
    out = orc.paged_decode(q, kc, vc, tables, sl, q_dtype=dtype,
                           cache_dtype=dtype, scale=scale)
    assert np.isfinite(out).all()
    for s in range(S):
        for hq in range(Hkv * G):
            h = hq // G
            ref = dense_attention_fp64(widen(q[s, hq], dtype, orc),
                                       widen(Ks[s][:, h], dtype, orc),
                                       widen(Vs[s][:, h], dtype, orc), scale)
            np.testing.assert_allclose(out[s, hq], ref, rtol=0, atol=1e-12)


def test_tiny_workload_matches_dense_softmax(orc):
    """Config 1 (tiny fp32): every row against the library brute force on the
    K/V the test reads back block by block through its own indexing."""
    c = workloads.tiny_f32()
    out = orc.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables,
                           c.seq_lens, q_dtype="f32", cache_dtype="f32",
                           scale=c.scale)
    assert np.isfinite(out).all()
    for s in range(c.S):
        L = int(c.seq_lens[s])
        nb = -(-L // c.bs)
        K = np.concatenate([c.k_cache[c.block_tables[s, j]] for j in range(nb)])[:L]
        V = np.concatenate([c.v_cache[c.block_tables[s, j]] for j in range(nb)])[:L]
        for hq in range(c.Hq):
            ref = dense_attention_fp64(c.query[s, hq], K[:, hq], V[:, hq], c.scale)
            np.testing.assert_allclose(out[s, hq], ref, rtol=0, atol=1e-12)


# --- closed forms ----------------------------------------------------------

def _single_seq(orc, K, V, q, bs=16, scale=0.125, dtype="f32"):
    kc, vc, tables, sl = build_pool([K], [V], bs, dtype=dtype)
    return orc.paged_decode(q[None], kc, vc, tables, sl, q_dtype=dtype,
                            cache_dtype=dtype, scale=scale)[0]


def test_identical_keys_give_mean_of_values(orc):
    rng = np.random.default_rng(7)
    L, H, D = 77, 2, 64
    k = rng.standard_normal((1, H, D), dtype=np.float32)
    K = np.repeat(k, L, axis=0)
    V = rng.standard_normal((L, H, D), dtype=np.float32)
    q = rng.standard_normal((H, D), dtype=np.float32)
    out = _single_seq(orc, K, V, q)
    np.testing.assert_allclose(out, V.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_single_token_returns_its_value_exactly(orc):
    rng = np.random.default_rng(8)
    K = rng.standard_normal((1, 3, 64), dtype=np.float32)
    V = rng.standard_normal((1, 3, 64), dtype=np.float32)
    q = rng.standard_normal((3, 64), dtype=np.float32)
    out = _single_seq(orc, K, V, q)
    assert np.array_equal(out, V[0].astype(np.float64))


def test_zero_scale_gives_mean_of_values(orc):
    rng = np.random.default_rng(9)
    K = rng.standard_normal((50, 1, 64), dtype=np.float32)
    V = rng.standard_normal((50, 1, 64), dtype=np.float32)
    q = rng.standard_normal((1, 64), dtype=np.float32)
    out = _single_seq(orc, K, V, q, scale=0.0)
    np.testing.assert_allclose(out, V.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_are_returned(orc):
    rng = np.random.default_rng(10)
    K = rng.standard_normal((40, 2, 64), dtype=np.float32)
    V = np.broadcast_to(rng.standard_normal((1, 2, 64), dtype=np.float32), (40, 2, 64)).copy()
    q = rng.standard_normal((2, 64), dtype=np.float32)
    out = _single_seq(orc, K, V, q)
    np.testing.assert_allclose(out, V[0].astype(np.float64), rtol=1e-14, atol=0)


def test_two_tokens_closed_form(orc):
    """L=2 with unequal scores: out = v0 + sigmoid(z1 - z0) (v1 - v0).

    By hand: z0 = 2 * (0.5*1 + 0.75*0) = 1 and z1 = 2 * (0.5*0 + 0.75*2) = 3,
    so the second token's weight is sigmoid(2) = 0.8807970779778823.  A
    dropped scale gives sigmoid(1) = 0.73, swapped scores sigmoid(-2) =
    0.12, and query components paired with the wrong key components
    (z0 = 1.5, z1 = 2) sigmoid(0.5) = 0.62."""
    K = np.array([[[1.0, 0.0]], [[0.0, 2.0]]], np.float32)   # [2,1,2]
    V = np.array([[[3.0, -1.0]], [[-2.0, 5.0]]], np.float32)
    q = np.array([[0.5, 0.75]], np.float32)
    out = _single_seq(orc, K, V, q, bs=8, scale=2.0)[0]
    w1 = 0.8807970779778823                                  # 1 / (1 + e^-2)
    expect = np.array([3.0 + w1 * (-5.0), -1.0 + w1 * 6.0])   # v0 + w1 (v1 - v0)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-15)


def test_zero_length_gives_zeros(orc):
    c = workloads.tiny_f32()
    sl = c.seq_lens.copy()
    sl[1] = 0
    out = orc.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables, sl,
                           q_dtype="f32", cache_dtype="f32", scale=c.scale)
    assert np.all(out[1] == 0.0)
    assert np.isfinite(out).all()


# --- paging invariants (bit-exact) ---------------------------------------

def test_block_permutation_is_bit_invariant(orc):
    c = workloads.tiny_f32()
    base = orc.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables,
                            c.seq_lens, q_dtype="f32", cache_dtype="f32", scale=c.scale)
    rng = np.random.default_rng(11)
    for _ in range(3):
        k2, v2, t2 = relabel(c.k_cache, c.v_cache, c.block_tables, rng)
        out = orc.paged_decode(c.query, k2, v2, t2, c.seq_lens, q_dtype="f32",
                               cache_dtype="f32", scale=c.scale)
        assert np.array_equal(out, base)


def test_block_size_is_bit_invariant(orc):
    rng = np.random.default_rng(12)
    lens = [5, 64, 97]
    Ks, Vs = rand_logical(rng, lens, 2, 64, "bf16")
    q = workloads.draw(rng, (3, 4, 64), "bf16")
    outs = []
    for bs in (8, 16, 32):
        kc, vc, t, sl = build_pool(Ks, Vs, bs, dtype="bf16", rng=rng)
        outs.append(orc.paged_decode(q, kc, vc, t, sl, q_dtype="bf16",
                                     cache_dtype="bf16", scale=0.125))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_prefix_equals_duplicated_copies(orc):
    """[P4] §2.1 / §4.2: sharing a block means pointing several tables at it;
    the result must equal every sequence owning its own copy."""
    rng = np.random.default_rng(13)
    bs, pre = 16, 64
    Kp = workloads.draw(rng, (pre, 2, 64), "f16")
    Vp = workloads.draw(rng, (pre, 2, 64), "f16")
    Ks, Vs = [], []
    for L in (20, 1, 45, 33):
        kt, vt = rand_logical(rng, [L], 2, 64, "f16")
        Ks.append(np.concatenate([Kp, kt[0]]))
        Vs.append(np.concatenate([Vp, vt[0]]))
    q = workloads.draw(rng, (4, 8, 64), "f16")
    shared = build_pool(Ks, Vs, bs, dtype="f16", rng=rng, shared_prefix_blocks=pre // bs)
    dup = build_pool(Ks, Vs, bs, dtype="f16", rng=rng)
    # the shared pool really shares: one physical copy of each prefix block
    assert np.all(shared[2][:, :pre // bs] == shared[2][0, :pre // bs])
    assert len(set(dup[2][:, 0].tolist())) == 4
    o1 = orc.paged_decode(q, *shared, q_dtype="f16", cache_dtype="f16", scale=0.125)
    o2 = orc.paged_decode(q, *dup, q_dtype="f16", cache_dtype="f16", scale=0.125)
    assert np.array_equal(o1, o2)


def test_gqa_equals_mha_with_repeated_kv_heads(orc):
    rng = np.random.default_rng(14)
    G, Hkv = 4, 2
    lens = [30, 70]
    Ks, Vs = rand_logical(rng, lens, Hkv, 64, "bf16")
    q = workloads.draw(rng, (2, Hkv * G, 64), "bf16")
    kc, vc, t, sl = build_pool(Ks, Vs, 16, dtype="bf16", rng=np.random.default_rng(1))
    gqa = orc.paged_decode(q, kc, vc, t, sl, q_dtype="bf16", cache_dtype="bf16", scale=0.1)
    Kr = [np.repeat(k, G, axis=1) for k in Ks]
    Vr = [np.repeat(v, G, axis=1) for v in Vs]
    kc2, vc2, t2, sl2 = build_pool(Kr, Vr, 16, dtype="bf16", rng=np.random.default_rng(2))
    mha = orc.paged_decode(q, kc2, vc2, t2, sl2, q_dtype="bf16", cache_dtype="bf16", scale=0.1)
    assert np.array_equal(gqa, mha)


def test_masked_tokens_never_contribute(orc):
    """Tokens at or past L hold NaN in every workload pool (tail of the last
    block, padding block); a finite output shows the oracle reads none."""
    for c in (workloads.tiny_f32(), workloads.make_case(
            "t", 5, [1, 8, 9, 31, 32, 33], 4, 2, 64, 8, q_dtype="bf16", cache_dtype="bf16")):
        assert np.isnan(workloads.bf16_values(c.k_cache) if c.cache_dtype == "bf16"
                        else c.k_cache).any()
        out = orc.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables,
                               c.seq_lens, q_dtype=c.q_dtype,
                               cache_dtype=c.cache_dtype, scale=c.scale)
        assert np.isfinite(out).all()


# --- worked examples printed on the pages ---------------------------------

def test_p4_worked_block_table(orc):
    """[P4] §2.2 worked example: bs 4, table [7, 2], lengths 8 and 7."""
    g = json.load(open(os.path.join(GOLDEN, "p4_block_table_example.json")))
    bs = g["block_size"]
    NB, D = 8, 4
    kc = np.full((NB, bs, 1, D), np.nan, np.float32)
    vc = np.full((NB, bs, 1, D), np.nan, np.float32)
    for b in range(NB):
        for o in range(bs):
            kc[b, o, 0, :] = 100 * b + o          # tag: which slot a value came from
            vc[b, o, 0, :] = -(100 * b + o)
    for case in g["cases"]:
        L = case["seq_len"]
        tables = np.array([g["block_table"]], np.int32)
        sl = np.array([L], np.int32)
        if L < 8:      # the unfilled slot of logical block 1 holds poison
            kc[2, 3] = np.nan
            vc[2, 3] = np.nan
        K, V = orc.gather_sequence(kc, vc, tables, sl, 0, 0, cache_dtype="f32")
        expect = [100 * b + o for b, o in case["token_to_physical"]]
        assert K[:, 0].tolist() == expect
        assert V[:, 0].tolist() == [-e for e in expect]
        q = np.zeros((1, 1, D), np.float32)
        out = orc.paged_decode(q, kc, vc, tables, sl, q_dtype="f32",
                               cache_dtype="f32", scale=1.0)
        assert np.isfinite(out).all()
        assert out[0, 0, 0] == pytest.approx(-np.mean(expect), abs=1e-12)


def test_p2_block_counts_are_ceilings(orc):
    """[P2] §1.2: 48 tokens occupy 3 blocks and 200 tokens 13 blocks at bs 16.
    The oracle must read exactly that many table entries: with an invalid id
    right after them it succeeds, with one of them invalid it refuses."""
    g = json.load(open(os.path.join(GOLDEN, "p2_block_counts.json")))
    bs = g["block_size"]
    NB = 32
    kc = np.zeros((NB, bs, 1, 8), np.float32)
    vc = np.zeros((NB, bs, 1, 8), np.float32)
    q = np.zeros((1, 1, 8), np.float32)
    for case in g["cases"]:
        n = case["blocks"]
        assert n == math.ceil(case["seq_len"] / bs)
        t = np.full((1, n + 3), -1, np.int32)
        t[0, :n] = np.arange(case["first_block"], case["first_block"] + n)
        sl = np.array([case["seq_len"]], np.int32)
        orc.paged_decode(q, kc, vc, t, sl, q_dtype="f32", cache_dtype="f32", scale=1.0)
        t[0, n - 1] = -1
        with pytest.raises(RuntimeError):
            orc.paged_decode(q, kc, vc, t, sl, q_dtype="f32", cache_dtype="f32", scale=1.0)


# --- split-K partials and their merge --------------------------------------

@pytest.mark.parametrize("P", [16, 32, 64, 512])
def test_partials_merge_to_single_pass(orc, P):
    """Splitting the softmax sums over disjoint token ranges is exact algebra,
    so partials + merge must equal the one-pass definition to rounding."""
    c = workloads.make_case("p", 21, [1, 15, 16, 17, 64, 100, 129, 600], 8, 2,
                            64, 16, q_dtype="bf16", cache_dtype="bf16")
    kw = dict(q_dtype="bf16", cache_dtype="bf16", scale=c.scale)
    ref = orc.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, **kw)
    P_max = -(-int(c.seq_lens.max()) // P)
    m, l, o = orc.paged_partials(c.query, c.k_cache, c.v_cache, c.block_tables,
                                 c.seq_lens, partition_size=P, P_max=P_max, **kw)
    out = orc.partition_reduce(m, l, o, c.seq_lens, partition_size=P)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    # one partition covering the sequence: o/l is the output, l >= 1
    one = c.seq_lens <= P
    np.testing.assert_allclose(o[one, :, 0] / l[one, :, 0, None], ref[one], rtol=0, atol=1e-13)
    assert np.all(l[one, :, 0] >= 1.0)


def test_partition_ranges_by_brute_force(orc):
    """m_p, l_p, o_p of each partition against numpy on the gathered tokens."""
    c = workloads.make_case("p", 22, [70, 33], 2, 1, 64, 8, q_dtype="f32", cache_dtype="f32")
    P = 32
    m, l, o = orc.paged_partials(c.query, c.k_cache, c.v_cache, c.block_tables,
                                 c.seq_lens, q_dtype="f32", cache_dtype="f32",
                                 scale=c.scale, partition_size=P, P_max=3)
    for s in range(2):
        L = int(c.seq_lens[s])
        nb = -(-L // c.bs)
        K = np.concatenate([c.k_cache[c.block_tables[s, j]] for j in range(nb)])[:L, 0]
        V = np.concatenate([c.v_cache[c.block_tables[s, j]] for j in range(nb)])[:L, 0]
        for hq in range(2):
            z = (K.astype(np.float64) @ c.query[s, hq].astype(np.float64)) * c.scale
            for p in range(-(-L // P)):
                zz = z[p * P:(p + 1) * P]
                mm = zz.max()
                assert m[s, hq, p] == pytest.approx(mm, abs=1e-13)
                w = np.exp(zz - mm)
                assert l[s, hq, p] == pytest.approx(w.sum(), abs=1e-12)
                np.testing.assert_allclose(o[s, hq, p], w @ V[p * P:(p + 1) * P], atol=1e-12)
            assert np.isnan(m[s, hq, -(-L // P):]).all()   # untouched beyond ceil(L/P)


# --- several query tokens per sequence (chunked prefill, verification) -----
# [P4] §6.3 (chunked prefill) and §6.5 (speculative verification): the new
# tokens of a sequence are its last Qn cached tokens; token i attends to
# every token up to its own position.

def _multi_case(rng, lens, qlens, Hkv, G, D, bs, dtype):
    Ks, Vs = rand_logical(rng, lens, Hkv, D, dtype)
    kc, vc, tables, sl = build_pool(Ks, Vs, bs, dtype=dtype, rng=rng)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = workloads.draw(rng, (int(qs[-1]), Hkv * G, D), dtype)
    return Ks, Vs, kc, vc, tables, sl, qs, q


@pytest.mark.parametrize("seed", range(4))
def test_multi_matches_dense_causal_softmax(orc, seed):
    """Library brute force: for query token i of sequence s at position
    p = L - Qn + i, softmax(scale * K[:p+1] q) V[:p+1] in float64."""
    rng = np.random.default_rng(400 + seed)
    dtype = ["f32", "bf16", "f16", "bf16"][seed]
    bs, Hkv, G, D = [16, 8, 32, 16][seed], [1, 2, 4, 2][seed], [4, 2, 1, 8][seed], [64, 128][seed % 2]
    S = 3
    lens = rng.integers(5, 70, size=S)
    qlens = np.minimum(lens, rng.integers(1, 9, size=S))
    Ks, Vs, kc, vc, tables, sl, qs, q = _multi_case(rng, lens, qlens, Hkv, G, D, bs, dtype)
    scale = 1.0 / math.sqrt(D)
    out = orc.paged_multi(q, kc, vc, tables, sl, qs, q_dtype=dtype, cache_dtype=dtype,
                          scale=scale)
    assert np.isfinite(out).all()
    for s in range(S):
        for i in range(int(qlens[s])):
            pos = int(lens[s]) - int(qlens[s]) + i
            for hq in range(Hkv * G):
                h = hq // G
                ref = dense_attention_fp64(widen(q[qs[s] + i, hq], dtype, orc),
                                           widen(Ks[s][:pos + 1, h], dtype, orc),
                                           widen(Vs[s][:pos + 1, h], dtype, orc), scale)
                np.testing.assert_allclose(out[qs[s] + i, hq], ref, rtol=0, atol=1e-12)


def test_multi_single_token_equals_decode(orc):
    """Qn = 1 for every sequence is decode: bit-identical rows."""
    rng = np.random.default_rng(410)
    lens = rng.integers(1, 120, size=5)
    Ks, Vs, kc, vc, tables, sl, qs, q = _multi_case(rng, lens, np.ones(5, int), 2, 4, 64, 16,
                                                     "bf16")
    a = orc.paged_multi(q, kc, vc, tables, sl, qs, q_dtype="bf16", cache_dtype="bf16",
                        scale=0.125)
    b = orc.paged_decode(q, kc, vc, tables, sl, q_dtype="bf16", cache_dtype="bf16",
                         scale=0.125)
    assert np.array_equal(a, b)


def test_multi_token_equals_decode_of_its_prefix(orc):
    """Query token i of a sequence equals decode of the same query against
    the sequence cut after position L - Qn + i: bit-identical."""
    rng = np.random.default_rng(411)
    lens = np.array([40, 17, 64])
    qlens = np.array([6, 17, 3])
    Ks, Vs, kc, vc, tables, sl, qs, q = _multi_case(rng, lens, qlens, 2, 2, 64, 8, "f16")
    out = orc.paged_multi(q, kc, vc, tables, sl, qs, q_dtype="f16", cache_dtype="f16",
                          scale=0.2)
    for s in range(3):
        for i in range(int(qlens[s])):
            cut = sl.copy()
            cut[s] = lens[s] - qlens[s] + i + 1
            qd = np.zeros((3, 4, 64), np.float16)
            qd[s] = q[qs[s] + i]
            ref = orc.paged_decode(qd, kc, vc, tables, cut, q_dtype="f16", cache_dtype="f16",
                                   scale=0.2, rows=[s * 4 + hq for hq in range(4)])
            assert np.array_equal(out[qs[s] + i], ref[s])


def test_multi_queries_before_the_sequence_are_zero(orc):
    """Qn > L: query tokens whose position is negative see nothing."""
    rng = np.random.default_rng(412)
    Ks, Vs, kc, vc, tables, sl, qs, q = _multi_case(rng, np.array([3]), np.array([5]), 1, 1,
                                                     64, 16, "f32")
    out = orc.paged_multi(q, kc, vc, tables, sl, qs, q_dtype="f32", cache_dtype="f32",
                          scale=0.125)
    assert np.all(out[:2] == 0.0)
    assert np.isfinite(out[2:]).all() and np.any(out[2:] != 0.0)


# --- mixed block sizes ([P1] "vLLM 0.5 ..." §1.3) ------------------------------

from pool_util import build_mixed_pool  # noqa: E402


@pytest.mark.parametrize("seed,page", [(0, 8), (1, 8), (2, 16)])
def test_mixed_matches_dense_softmax(orc, seed, page):
    """Sequences with 8-, 16- and 32-token blocks over one pool of pages,
    against the library brute force on the logical K/V."""
    rng = np.random.default_rng(700 + seed)
    dtype = ["bf16", "f16", "f32"][seed]
    Hkv, G, D = 2, 4, 64
    sizes = [b for b in (8, 16, 32) if b >= page]
    S = 6
    lens = rng.integers(1, 140, size=S)
    seq_bs = np.array([sizes[i % len(sizes)] for i in range(S)], np.int32)
    Ks, Vs = rand_logical(rng, lens, Hkv, D, dtype)
    kc, vc, tables, sl = build_mixed_pool(Ks, Vs, seq_bs, page, dtype=dtype, rng=rng)
    q = workloads.draw(rng, (S, Hkv * G, D), dtype)
    scale = 1.0 / math.sqrt(D)
    out = orc.paged_decode_mixed(q, kc, vc, tables, sl, seq_bs, q_dtype=dtype,
                                 cache_dtype=dtype, scale=scale)
    for s in range(S):
        for hq in range(Hkv * G):
            ref = dense_attention_fp64(widen(q[s, hq], dtype, orc),
                                       widen(Ks[s][:, hq // G], dtype, orc),
                                       widen(Vs[s][:, hq // G], dtype, orc), scale)
            np.testing.assert_allclose(out[s, hq], ref, rtol=0, atol=1e-12)


def test_mixed_equals_page_tables(orc):
    """A block of k pages is the same as k one-page blocks: expanding every
    table entry e of a bs_s-token block into e, e+1, .., e + bs_s/page - 1
    gives a uniform page-sized table with bit-identical output."""
    rng = np.random.default_rng(710)
    page, Hkv, G, D = 8, 2, 2, 64
    lens = rng.integers(1, 200, size=5)
    seq_bs = np.array([8, 16, 32, 16, 32], np.int32)
    Ks, Vs = rand_logical(rng, lens, Hkv, D, "bf16")
    kc, vc, tables, sl = build_mixed_pool(Ks, Vs, seq_bs, page, dtype="bf16", rng=rng)
    q = workloads.draw(rng, (5, Hkv * G, D), "bf16")
    kw = dict(q_dtype="bf16", cache_dtype="bf16", scale=0.125)
    mixed = orc.paged_decode_mixed(q, kc, vc, tables, sl, seq_bs, **kw)
    rows = []
    for s in range(5):
        k = int(seq_bs[s]) // page
        nblk = -(-int(lens[s]) // int(seq_bs[s]))
        rows.append([int(tables[s, j]) + i for j in range(nblk) for i in range(k)])
    wide = np.zeros((5, max(len(r) for r in rows)), np.int32)
    for s, r in enumerate(rows):
        wide[s, :len(r)] = r
    uniform = orc.paged_decode(q, kc, vc, wide, sl, **kw)
    assert np.array_equal(mixed, uniform)


def test_mixed_with_page_sized_blocks_is_plain_decode(orc):
    rng = np.random.default_rng(720)
    Ks, Vs = rand_logical(rng, [5, 40, 77], 2, 64, "f16")
    kc, vc, tables, sl = build_pool(Ks, Vs, 16, dtype="f16", rng=rng)
    q = workloads.draw(rng, (3, 4, 64), "f16")
    kw = dict(q_dtype="f16", cache_dtype="f16", scale=0.125)
    assert np.array_equal(
        orc.paged_decode_mixed(q, kc, vc, tables, sl, np.full(3, 16, np.int32), **kw),
        orc.paged_decode(q, kc, vc, tables, sl, **kw))


def test_mixed_block_size_rule():
    """[P1] §1.3: short requests (< 128 tokens) 8 per block, medium (< 2048)
    16, long 32."""
    assert [workloads.block_size_for_length(L) for L in (1, 127, 128, 2047, 2048, 9000)] == \
        [8, 8, 16, 16, 32, 32]
