"""paged_attention_decode (+ reduce) on the GPU against the oracle.

Every workload configuration at full size, both kernels, split-K, the
invariants of the method (bit-exact under block relabelling and prefix
sharing), closed forms, masking under NaN poison, zero and one-token
sequences, every E4M3 code, and a seeded fuzz over shapes and types.
Tolerances: max abs error 5e-3 for f16/bf16 caches and 3e-2 for fp8 (the
bounds this library is held to), 1e-5 for fp32, flat on the five workload
configurations; the fuzz and small-batch cases add half an output ulp only
where |ref| >= 1 (the rounding of the stored result itself)."""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_361_amd as pkv
import workloads
from gpu_case import (TOL, DevCase, assert_within, bound, from_dev, gpu_run, max_err,
                      oracle_caches, oracle_run, to_dev)

pytestmark = pytest.mark.gpu

ALGOS = ["valu", "mfma"]


@functools.lru_cache(maxsize=None)
def workload(name, *args):
    return workloads.WORKLOADS[name](*args)


@functools.lru_cache(maxsize=None)
def workload_ref(name, *args):
    """The oracle's output for every row of a workload, computed once per
    session and shared by the tests of the different split modes."""
    return oracle_run(workload(name, *args))


def _skip_unsupported(fn):
    @functools.wraps(fn)
    def wrap(*a, **kw):
        try:
            return fn(*a, **kw)
        except pkv.PagedKVError as e:
            if e.status == -4:
                pytest.skip("kernel does not support this combination")
            raise
    return wrap


def check(c, out, ref, rows=None, tol=None):
    """Flat tolerance at every magnitude (the bound the workloads are held to)."""
    tol = TOL[c.cache_dtype] if tol is None else tol
    err = max_err(out, ref, rows)
    print("%s: max abs err %.3g (tol %.3g)" % (c.name, err, tol), flush=True)
    if rows is not None:
        S, Hq, D = ref.shape
        out, ref = out.reshape(S * Hq, D)[rows], ref.reshape(S * Hq, D)[rows]
    assert_within(out, ref, tol)


# --- the five workload configurations ------------------------------------

@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_tiny_fp32(algo):
    c = workload("tiny-f32")
    check(c, gpu_run(c, algo), oracle_run(c))


@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_llama2_13b_mha_fp16_full(algo):
    c = workload("llama2-13b-mha")
    check(c, gpu_run(c, algo), oracle_run(c))


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("P", [0, 512])
@_skip_unsupported
def test_llama3_8b_gqa_bf16_full(algo, P):
    c = workload("llama3-8b-gqa")
    check(c, gpu_run(c, algo, P), oracle_run(c))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_long_context_splitk_full(algo):
    """Full 32K-128K lengths, partitions of 512, reduced by the second kernel;
    all 512 rows (8 sequences x 64 query heads, every KV head) against the
    oracle."""
    c = workload("long-context-gqa")
    check(c, gpu_run(c, algo), workload_ref("long-context-gqa"))


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("bs", [8, 16, 32])
@_skip_unsupported
def test_shared_prefix_fp8(algo, bs):
    c = workload("shared-prefix-fp8", bs)
    check(c, gpu_run(c, algo), oracle_run(c))


# --- split-K ---------------------------------------------------------------

def small_gqa(seed=3, S=24, dtype="bf16", **kw):
    return workloads.make_case("small-gqa", seed, lambda r: workloads.llama3_8b_gqa_lens(r, S),
                               32, 8, 128, kw.pop("bs", 16), q_dtype=dtype,
                               cache_dtype=dtype, max_seq_len=4096, **kw)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("P", [16, 64, 256, 1024])
@_skip_unsupported
def test_split_k_partition_sizes(algo, P):
    c = small_gqa(seed=40 + P)
    ref = oracle_run(c)
    check(c, gpu_run(c, algo, P), ref)


@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_split_k_one_partition_is_single_pass_bit_exact(algo):
    c = small_gqa(seed=41)
    a = gpu_run(c, algo, 0)
    b = gpu_run(c, algo, 4096)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_reduce_on_oracle_partials(dtype):
    """The second kernel alone: partials from the oracle (rounded to fp32, the
    workspace format) merged on the GPU and by the oracle merge."""
    c = workloads.make_case("red", 42, [1, 100, 513, 1024, 1025, 3000, 4096], 8, 2, 128,
                            16, q_dtype="bf16", cache_dtype="bf16", max_seq_len=4096)
    P = 256
    P_max = -(-c.max_seq_len // P)
    m, l, o = oracle.paged_partials(c.query, c.k_cache, c.v_cache, c.block_tables,
                                    c.seq_lens, q_dtype="bf16", cache_dtype="bf16",
                                    scale=c.scale, partition_size=P, P_max=P_max)
    m32 = np.nan_to_num(m).astype(np.float32)
    l32 = np.nan_to_num(l).astype(np.float32)
    o32 = np.nan_to_num(o).astype(np.float32)
    ref = oracle.partition_reduce(m32.astype(np.float64), l32.astype(np.float64),
                                  o32.astype(np.float64), c.seq_lens, partition_size=P)
    nbytes = pkv.decode_workspace_bytes(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
    n = c.S * c.Hq * P_max
    a = -(-4 * n // 256) * 256
    ws = np.zeros(nbytes, np.uint8)
    ws[:4 * n] = m32.reshape(-1).view(np.uint8)
    ws[a:a + 4 * n] = l32.reshape(-1).view(np.uint8)
    ws[2 * a:] = o32.reshape(-1).view(np.uint8)
    out = torch.full((c.S, c.Hq, c.D), 7.0, dtype=gpu_torch(dtype), device="cuda")
    pkv.paged_attention_reduce(out, torch.from_numpy(ws).cuda(), torch.from_numpy(c.seq_lens).cuda(),
                               num_kv_heads=c.Hkv, max_seq_len=c.max_seq_len, partition_size=P)
    got = from_dev(out)
    multi = c.seq_lens > P
    tol = {"f32": 1e-6, "f16": 1e-3, "bf16": 4e-3}[dtype]
    assert np.max(np.abs(got[multi] - ref[multi])) <= tol
    assert np.all(got[~multi] == 7.0)          # single-partition rows untouched


def gpu_torch(dtype):
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


# --- invariants -------------------------------------------------------------

@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_block_relabelling_is_bit_exact(algo):
    c = small_gqa(seed=50)
    a = gpu_run(c, algo)
    rng = np.random.default_rng(51)
    c2 = c.copy()
    pi = rng.permutation(c.NB).astype(np.int32)
    c2.k_cache = np.empty_like(c.k_cache)
    c2.v_cache = np.empty_like(c.v_cache)
    c2.k_cache[pi] = c.k_cache
    c2.v_cache[pi] = c.v_cache
    c2.block_tables = pi[c.block_tables]
    c2.slot_mapping = (pi[c.slot_mapping // c.bs].astype(np.int64) * c.bs
                       + c.slot_mapping % c.bs)
    b = gpu_run(c2, algo)
    assert np.array_equal(a, b)


def duplicate_prefix(c):
    """Twin of a shared-prefix case in which every sequence owns a copy of
    the prefix blocks (written through the cache writer like the original)."""
    pre = c.notes["prefix_len"]
    npre = pre // c.bs
    t = c.copy()
    extra = c.S * npre
    t.NB = c.NB + extra
    shape = (t.NB,) + c.k_cache.shape[1:]
    t.k_cache = np.full(shape, workloads.POISON[c.cache_dtype], c.k_cache.dtype)
    t.v_cache = np.full(shape, workloads.POISON[c.cache_dtype], c.v_cache.dtype)
    for s in range(c.S):
        t.block_tables[s, :npre] = c.NB + s * npre + np.arange(npre)
    pk, pv = c.new_key[:pre], c.new_value[:pre]
    pslots = c.slot_mapping[:pre]
    keys, vals, slots = [], [], []
    for s in range(c.S):
        keys.append(pk)
        vals.append(pv)
        blk = (pslots // c.bs) - 0
        # the prefix tokens were written to the shared blocks in table order
        order = {int(b): j for j, b in enumerate(c.block_tables[0, :npre])}
        newb = np.array([c.NB + s * npre + order[int(b)] for b in blk], np.int64)
        slots.append(newb * c.bs + pslots % c.bs)
    t.new_key = np.concatenate(keys + [c.new_key[pre:]])
    t.new_value = np.concatenate(vals + [c.new_value[pre:]])
    t.slot_mapping = np.concatenate(slots + [c.slot_mapping[pre:]])
    return t


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("bs", [8, 32])
@_skip_unsupported
def test_shared_prefix_equals_duplicated_bit_exact(algo, bs):
    c = workloads.shared_prefix_fp8(bs=bs, S=12)
    t = duplicate_prefix(c)
    a = gpu_run(c, algo)
    b = gpu_run(t, algo)
    assert np.array_equal(a, b)
    check(c, a, oracle_run(c))


@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_identical_keys_give_mean_of_values(algo):
    c = small_gqa(seed=60, S=8, dtype="bf16")
    for s in range(c.S):                       # every live key row equal to one row
        L = int(c.seq_lens[s])
        k0 = c.k_cache[c.block_tables[s, 0], 0].copy()
        for j in range(-(-L // c.bs)):
            c.k_cache[c.block_tables[s, j]] = k0
    out = gpu_run(c, algo)
    kc, vc = oracle_caches(c)
    for s in range(c.S):
        L = int(c.seq_lens[s])
        V = np.concatenate([vc[c.block_tables[s, j]] for j in range(-(-L // c.bs))])[:L]
        V = workloads.bf16_values(V).astype(np.float64)   # [L, Hkv, D]
        mean = V.mean(axis=0)
        for hq in range(c.Hq):
            assert np.max(np.abs(out[s, hq] - mean[hq // c.G])) <= 5e-3


@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_gqa_equals_mha_with_repeated_heads(algo):
    c = small_gqa(seed=61, S=6)
    a = gpu_run(c, algo)
    m = c.copy()
    m.Hkv = c.Hq
    m.k_cache = np.ascontiguousarray(np.repeat(c.k_cache, c.G, axis=2))
    m.v_cache = np.ascontiguousarray(np.repeat(c.v_cache, c.G, axis=2))
    m.new_key = np.ascontiguousarray(np.repeat(c.new_key, c.G, axis=1))
    m.new_value = np.ascontiguousarray(np.repeat(c.new_value, c.G, axis=1))
    b = gpu_run(m, algo)
    assert np.max(np.abs(a - b)) <= 2e-3


# --- edge cases ----------------------------------------------------------------

@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_zero_and_one_token_sequences(algo):
    c = workloads.make_case("edge", 70, [1, 5, 1, 40, 1], 8, 2, 128, 16,
                            q_dtype="bf16", cache_dtype="bf16")
    c.seq_lens[1] = 0
    out = gpu_run(c, algo)
    assert np.all(out[1] == 0.0)
    for s in (0, 2, 4):                       # L = 1: exactly the value row
        v = workloads.bf16_values(c.v_cache[c.block_tables[s, 0], 0]).astype(np.float64)
        for hq in range(c.Hq):
            assert np.array_equal(out[s, hq], v[hq // c.G])
    ref = oracle_run(c)
    check(c, out, ref)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("P", [0, 64, 512])
@_skip_unsupported
def test_all_zero_length_batch(algo, P):
    """No sequence holds a token, so the batch has no tiles at all: every row
    of the output (filled with NaN first) is written as zeros, unsplit and
    split."""
    c = workloads.make_case("all-empty", 91, [1, 1, 1, 1], 16, 4, 128, 16,
                            q_dtype="bf16", cache_dtype="bf16")
    c.seq_lens[:] = 0
    d = DevCase(c)
    d.write()
    d.out.fill_(float("nan"))
    d.decode(algo, P)
    torch.cuda.synchronize()
    assert np.all(from_dev(d.out) == 0.0)


@pytest.mark.parametrize("algo", ALGOS)
@_skip_unsupported
def test_every_e4m3_code_decodes_exactly(algo):
    """L = 1 returns v_scale * decode(code) of the value row: with scale 1 and
    a bf16 output (which holds every E4M3 value exactly) each of the 256
    codes must come back exactly, NaN codes as NaN."""
    S, Hkv, D, bs = 2, 1, 128, 16
    kc = np.full((4, bs, Hkv, D), 0x7F, np.uint8)
    vc = np.full((4, bs, Hkv, D), 0x7F, np.uint8)
    kc[1, 0, 0] = 0x38                          # keys: 1.0
    kc[2, 0, 0] = 0x38
    vc[1, 0, 0] = np.arange(128, dtype=np.uint8)
    vc[2, 0, 0] = np.arange(128, 256, dtype=np.uint8)
    tables = np.array([[1], [2]], np.int32)
    lens = np.array([1, 1], np.int32)
    q = workloads.draw(np.random.default_rng(1), (S, 1, D), "bf16")
    out = torch.empty(S, 1, D, dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_decode(out, to_dev(q, "bf16"), torch.from_numpy(kc).cuda(),
                               torch.from_numpy(vc).cuda(), torch.from_numpy(tables).cuda(),
                               torch.from_numpy(lens).cuda(), scale=0.1, max_seq_len=16,
                               k_scale=1.0, v_scale=1.0, algo=algo)
    got = from_dev(out).reshape(256)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(ref[~nan], oracle.e4m3_decode(np.arange(256, dtype=np.uint8))[~nan])


def fuzz_cases(n=24):
    rng = np.random.default_rng(2024)
    types = [("bf16", "bf16"), ("f16", "f16"), ("bf16", "fp8"), ("f16", "fp8"), ("f32", "f32")]
    for i in range(n):
        qd, cd = types[i % len(types)]
        G = [1, 2, 4, 8][rng.integers(4)]
        Hkv = [1, 2, 3][rng.integers(3)]
        D = [64, 128][rng.integers(2)]
        bs = [8, 16, 32][rng.integers(3)]
        S = int(rng.integers(1, 7))
        lens = rng.integers(1, 1400, size=S)
        lens[0] = [1, bs, 512, 16 * bs][i % 4]
        P = [0, 0, 512, 16 * max(1, bs // 16) * 4][i % 4]
        yield i, qd, cd, G, Hkv, D, bs, lens, P


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("case", list(fuzz_cases()), ids=lambda t: "fuzz%d" % t[0])
@_skip_unsupported
def test_fuzz(algo, case):
    i, qd, cd, G, Hkv, D, bs, lens, P = case
    c = workloads.make_case("fuzz%d" % i, 3000 + i, lens, Hkv * G, Hkv, D, bs,
                            q_dtype=qd, cache_dtype=cd, src_dtype=qd if cd == "fp8" else None,
                            max_seq_len=int(max(lens)) + 37, partition_size=P,
                            append_last=(cd != "fp8" and i % 2 == 0))
    out = gpu_run(c, algo)
    ref = oracle_run(c)
    assert_within(out, ref, bound(ref, cd, qd))


# --- balanced split (persistent grid, whole-batch work cut evenly) ----------

BAL = pkv.PARTITION_BALANCED


@pytest.mark.parametrize("cfg", ["llama2-13b-mha", "llama3-8b-gqa"])
def test_balanced_batch_workloads_full(cfg):
    c = workload(cfg)
    check(c, gpu_run(c, "mfma", BAL), oracle_run(c))


@pytest.mark.timeout(600)
def test_balanced_long_context_full():
    """All 512 rows; the balanced split cuts each (sequence, KV head) stream
    across chunks, so every KV head's merge is checked."""
    c = workload("long-context-gqa")
    check(c, gpu_run(c, "mfma", BAL), workload_ref("long-context-gqa"))


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_balanced_shared_prefix_fp8(bs):
    c = workload("shared-prefix-fp8", bs)
    check(c, gpu_run(c, "auto", BAL), oracle_run(c))


def test_balanced_f32_is_unsupported():
    c = workload("tiny-f32")
    with pytest.raises(pkv.PagedKVError) as e:
        gpu_run(c, "auto", BAL)
    assert e.value.status == -4


@pytest.mark.parametrize("lens", [[1], [3, 0, 17], [1, 1, 1, 0, 2], [16, 32, 48], [5000],
                                  [0, 0, 700], [0, 0, 0]])
def test_balanced_small_batches(lens):
    """Far fewer tiles than waves (most waves idle), zero-length rows written by
    the reduce, one-token and tile-multiple lengths."""
    c = workloads.make_case("bal-small", 80 + len(lens), [max(1, L) for L in lens], 16, 4, 128,
                            16, q_dtype="bf16", cache_dtype="bf16",
                            max_seq_len=max(max(lens), 1) + 5)
    c.seq_lens = np.asarray(lens, np.int32)
    out = gpu_run(c, "mfma", BAL)
    ref = oracle_run(c)
    for s, L in enumerate(lens):
        if L == 0:
            assert np.all(out[s] == 0.0)
    # few tokens: |out| can exceed 1, where the bf16 output's own rounding
    # is allowed on top of the tolerance
    assert_within(out, ref, bound(ref, "bf16", "bf16"))


@pytest.mark.parametrize("case", list(fuzz_cases()), ids=lambda t: "fuzz%d" % t[0])
@_skip_unsupported
def test_balanced_fuzz(case):
    i, qd, cd, G, Hkv, D, bs, lens, _ = case
    c = workloads.make_case("bfuzz%d" % i, 5000 + i, lens, Hkv * G, Hkv, D, bs,
                            q_dtype=qd, cache_dtype=cd, src_dtype=qd if cd == "fp8" else None,
                            max_seq_len=int(max(lens)) + 37,
                            append_last=(cd != "fp8" and i % 2 == 0))
    out = gpu_run(c, "mfma", BAL)
    ref = oracle_run(c)
    assert_within(out, ref, bound(ref, cd, qd))


def test_balanced_block_relabelling_is_bit_exact():
    c = small_gqa(seed=90)
    a = gpu_run(c, "mfma", BAL)
    rng = np.random.default_rng(91)
    c2 = c.copy()
    pi = rng.permutation(c.NB).astype(np.int32)
    c2.k_cache = np.empty_like(c.k_cache)
    c2.v_cache = np.empty_like(c.v_cache)
    c2.k_cache[pi] = c.k_cache
    c2.v_cache[pi] = c.v_cache
    c2.block_tables = pi[c.block_tables]
    c2.slot_mapping = (pi[c.slot_mapping // c.bs].astype(np.int64) * c.bs
                       + c.slot_mapping % c.bs)
    assert np.array_equal(a, gpu_run(c2, "mfma", BAL))


@pytest.mark.parametrize("bs", [8, 32])
def test_balanced_shared_prefix_equals_duplicated_bit_exact(bs):
    c = workloads.shared_prefix_fp8(bs=bs, S=12)
    a = gpu_run(c, "mfma", BAL)
    assert np.array_equal(a, gpu_run(duplicate_prefix(c), "mfma", BAL))
    check(c, a, oracle_run(c))


def test_balanced_workspace_shared_with_fixed_partitions():
    """A fixed-partition call that writes over the balanced header (its
    partials start at byte 0) must leave the next balanced call correct: it
    finds the counter state broken, assigns chunks statically and readies the
    counter; the call after it uses the counter again.  All balanced calls
    agree bit for bit."""
    c = small_gqa(seed=93, S=40)
    d = DevCase(c)
    d.write()
    nb = max(pkv.decode_workspace_bytes(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
             for P in (BAL, 256))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    outs = []
    for P in (BAL, BAL, 256, BAL, BAL, 256, BAL):
        d.out.fill_(float("nan"))
        d.decode("mfma", P, workspace=ws)
        torch.cuda.synchronize()
        outs.append((P, d.out.clone()))
    bal = [o for P, o in outs if P == BAL]
    for o in bal[1:]:
        assert torch.equal(o.view(torch.uint8), bal[0].view(torch.uint8))
    ref = oracle_run(c)
    check(c, from_dev(bal[0]), ref)
    check(c, from_dev(outs[2][1]), ref)


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x5A])
def test_balanced_workspace_contents_do_not_matter(fill):
    """The chunk counter in a fresh workspace holds whatever the memory held:
    zeros (below any call's range), all ones (above it) or another pattern.
    Each must give the right result, on the first call and the next ones."""
    c = small_gqa(seed=94, S=64)
    d = DevCase(c)
    d.write()
    ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, BAL)
    ws.fill_(fill)
    outs = []
    for _ in range(3):
        d.out.fill_(float("nan"))
        d.decode("mfma", BAL, workspace=ws)
        torch.cuda.synchronize()
        outs.append(d.out.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.uint8), outs[0].view(torch.uint8))
    check(c, from_dev(outs[0]), oracle_run(c))


@pytest.mark.parametrize("D", [64, 128])
def test_balanced_largest_batch(D):
    """8192 sequences, the most the balanced split takes (the lengths and the
    tile prefix fill 64 KiB of LDS; each thread scans 32 sequences), with
    short ragged lengths including zeros; every row is checked.  At head_dim
    64 the K tiles still go through LDS (a 64 KiB ring beside the prefix); at
    128 the 96 KiB ring no longer fits beside it and the kernel that loads K
    into registers runs."""
    rng = np.random.default_rng(95)
    lens = rng.integers(0, 40, size=8192)
    c = workloads.make_case("largest-batch", 95, lens, 8, 2, D, 16, q_dtype="bf16",
                            cache_dtype="bf16", max_seq_len=64)
    out = gpu_run(c, "mfma", BAL)
    ref = oracle_run(c)
    # short rows average few values, so |out| can exceed 1: there the
    # output's own bf16 rounding is allowed on top of the tolerance
    assert_within(out, ref, bound(ref, "bf16", "bf16"))


def test_balanced_agrees_with_fixed_partitions():
    c = small_gqa(seed=92, S=40)
    a = gpu_run(c, "mfma", BAL)
    b = gpu_run(c, "mfma", 256)
    assert np.max(np.abs(a - b)) <= 4e-3


@pytest.mark.parametrize("P", [BAL, 512])
def test_split_decode_replays_in_a_graph(P):
    """The split decode call (decode + reduce) holds no memset and its
    balanced chunk counter needs no reset between calls, so it can be
    captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit."""
    c = small_gqa(seed=96, S=48)
    d = DevCase(c)
    d.write()
    ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
    d.decode("mfma", P, workspace=ws)
    torch.cuda.synchronize()
    eager = d.out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.out.fill_(float("nan"))
        with torch.cuda.graph(g, stream=s):
            pkv.paged_attention_decode(d.out, d.query, d.k_cache, d.v_cache, d.tables, d.lens,
                                       scale=c.scale, max_seq_len=c.max_seq_len,
                                       partition_size=P, workspace=ws, algo="mfma", stream=s)
            pkv.paged_attention_reduce(d.out, ws, d.lens, num_kv_heads=c.Hkv,
                                       max_seq_len=c.max_seq_len, partition_size=P, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for _ in range(4):
        d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.uint8), eager.view(torch.uint8))
        d.decode("mfma", P, workspace=ws)      # eager calls between replays
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.uint8), eager.view(torch.uint8))


def test_balanced_graph_replays_track_changing_inputs():
    """Replays of a captured balanced decode + reduce, back to back with no
    eager call between them and new queries before each, equal eager calls
    on the same inputs bit for bit (the reduce hands the chunk counter back,
    so a replay's frozen call number still takes it over)."""
    c = small_gqa(seed=97, S=48)
    d = DevCase(c)
    d.write()
    P = BAL
    ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
    ws_eager = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
    out_eager = torch.empty_like(d.out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pkv.paged_attention_decode(d.out, d.query, d.k_cache, d.v_cache, d.tables, d.lens,
                                       scale=c.scale, max_seq_len=c.max_seq_len,
                                       partition_size=P, workspace=ws, algo="mfma", stream=s)
            pkv.paged_attention_reduce(d.out, ws, d.lens, num_kv_heads=c.Hkv,
                                       max_seq_len=c.max_seq_len, partition_size=P, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(98)
    for step in range(5):
        d.query.copy_(torch.randn(d.query.shape, generator=gen, device="cuda").to(d.query.dtype))
        d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        pkv.paged_attention_decode(out_eager, d.query, d.k_cache, d.v_cache, d.tables, d.lens,
                                   scale=c.scale, max_seq_len=c.max_seq_len, partition_size=P,
                                   workspace=ws_eager, algo="mfma")
        pkv.paged_attention_reduce(out_eager, ws_eager, d.lens, num_kv_heads=c.Hkv,
                                   max_seq_len=c.max_seq_len, partition_size=P)
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.uint8), out_eager.view(torch.uint8)), step
