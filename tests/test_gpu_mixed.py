"""Mixed block sizes on the GPU against the oracle: sequences with 8-, 16-
and 32-token blocks over one pool of pages ("vLLM 0.5 深度拆解" §1.3
picks the block size per request; a block is consecutive pages, this
library's layout for them).  Everything goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_361_amd as pkv
import workloads
from gpu_case import TOL, DevCase, assert_within, bound, from_dev, oracle_caches

pytestmark = pytest.mark.gpu


def run_mixed(mc: workloads.MixedCase, P: int = 0, d: DevCase = None):
    c = mc.case
    if d is None:
        d = DevCase(c)
        d.write()                      # slots are pool rows: block_size = page
    sbs = torch.from_numpy(mc.seq_bs).cuda()
    ws = None
    if P:
        ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
        ws.fill_(0xFF)
    d.out.fill_(float("nan"))
    print("mixed %s S=%d page=%d P=%d" % (c.name, c.S, c.bs, P), flush=True)
    pkv.paged_attention_decode_mixed(d.out, d.query, d.k_cache, d.v_cache, d.tables, d.lens,
                                     sbs, scale=c.scale, max_seq_len=c.max_seq_len,
                                     k_scale=c.k_scale, v_scale=c.v_scale,
                                     partition_size=P, workspace=ws)
    if P:
        pkv.paged_attention_reduce(d.out, ws, d.lens, num_kv_heads=c.Hkv,
                                   max_seq_len=c.max_seq_len, partition_size=P)
    torch.cuda.synchronize()
    return from_dev(d.out), d


def oracle_mixed(mc: workloads.MixedCase, rows=None):
    c = mc.case
    kc, vc = oracle_caches(c)
    return oracle.paged_decode_mixed(c.query, kc, vc, c.block_tables, c.seq_lens, mc.seq_bs,
                                     q_dtype=c.q_dtype, cache_dtype=c.cache_dtype,
                                     scale=c.scale, k_scale=c.k_scale, v_scale=c.v_scale,
                                     rows=rows)


def check(mc, out, ref, rows=None):
    c = mc.case
    if rows is not None:
        S, Hq, D = ref.shape
        out = out.reshape(S * Hq, D)[rows]
        ref = ref.reshape(S * Hq, D)[rows]
    ratio = assert_within(out, ref, bound(ref, c.cache_dtype, c.q_dtype))
    print("%s: worst err/bound %.3g" % (c.name, ratio), flush=True)


def random_sizes(choices):
    return lambda r, lens: r.choice(np.asarray(choices), size=lens.size)


def case(seed, S=24, page=8, dtype="bf16", cache="bf16", Hq=32, Hkv=8, D=128, lmax=600,
         sizes=(8, 16, 32), **kw):
    return workloads.make_mixed_case(
        "mixed-%d" % seed, seed, lambda r: r.integers(1, lmax, size=S), Hq, Hkv, D, page,
        q_dtype=dtype, cache_dtype=cache, block_sizes=random_sizes(sizes), max_seq_len=lmax,
        src_dtype=dtype if cache == "fp8" else None, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mixed_ragged(dtype):
    mc = case(800, dtype=dtype, cache=dtype, append_last=True)
    out, _ = run_mixed(mc)
    check(mc, out, oracle_mixed(mc))


def test_mixed_fp8_cache():
    mc = case(801, cache="fp8", S=16, lmax=500)
    out, _ = run_mixed(mc)
    check(mc, out, oracle_mixed(mc))


@pytest.mark.parametrize("G,Hkv,D", [(1, 8, 128), (16, 1, 128), (8, 2, 64)])
def test_mixed_group_sizes(G, Hkv, D):
    mc = case(810 + G, S=12, Hq=G * Hkv, Hkv=Hkv, D=D, lmax=700)
    out, _ = run_mixed(mc)
    check(mc, out, oracle_mixed(mc))


def test_mixed_page_16():
    mc = case(820, page=16, sizes=(16, 32), dtype="f16", cache="f16", D=64, Hq=16, Hkv=4)
    out, _ = run_mixed(mc)
    check(mc, out, oracle_mixed(mc))


@pytest.mark.parametrize("P", [32, 64, 512])
def test_mixed_split(P):
    """Fixed partitions (multiples of every block size) merged by the reduce."""
    mc = case(830 + P, S=20, lmax=1500)
    out, _ = run_mixed(mc, P)
    check(mc, out, oracle_mixed(mc))


def test_page_sized_blocks_equal_the_decode_kernel():
    """Every block one page of 16 tokens: bit for bit the one-pass decode
    kernel on the same pool."""
    mc = case(840, page=16, sizes=(16,))
    out, d = run_mixed(mc)
    d.decode("mfma", 0)
    torch.cuda.synchronize()
    assert np.array_equal(out, from_dev(d.out))


def test_blocks_equal_their_pages_as_8_token_blocks():
    """A 16- or 32-token block is the same as its 8-token pages: the mixed
    kernel (larger-block loop) against the 8-token decode kernel over tables
    expanded page by page, bit for bit."""
    mc = case(850, page=8, sizes=(16, 32), lmax=900)
    out, d = run_mixed(mc)
    c = mc.case
    rows = []
    for s in range(c.S):
        k = int(mc.seq_bs[s]) // 8
        nblk = -(-int(c.seq_lens[s]) // int(mc.seq_bs[s]))
        rows.append([int(c.block_tables[s, j]) + i for j in range(nblk) for i in range(k)])
    wide = np.full((c.S, max(len(r) for r in rows)), c.pad_block, np.int32)
    for s, r in enumerate(rows):
        wide[s, :len(r)] = r
    d.tables = torch.from_numpy(wide).cuda()
    d.decode("mfma", 0)
    torch.cuda.synchronize()
    assert np.array_equal(out, from_dev(d.out))


def test_mixed_block_sizes_workload_sampled_rows():
    """The Llama-3-8B decode shape with block sizes by length, split at 512
    as the bench runs it: the oracle on a sample of rows."""
    mc = workloads.mixed_block_sizes()
    c = mc.case
    rng = np.random.default_rng(860)
    seqs = set(rng.choice(c.S, size=24, replace=False).tolist())
    for b in (8, 16, 32):                       # every block size in the sample
        seqs.update(np.nonzero(mc.seq_bs == b)[0][:3].tolist())
    rows = sorted(s * c.Hq + hq for s in seqs for hq in (0, 5, 18, 31))
    out, _ = run_mixed(mc, 512)
    check(mc, out, oracle_mixed(mc, rows), rows)


# ---- the balanced split over mixed block sizes ------------------------------
BAL = pkv.PARTITION_BALANCED


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mixed_balanced_ragged(dtype):
    """The balanced split walking each sequence's own block size: 8-token
    blocks in 8-token tiles, 16 and 32 in 16-token tiles."""
    mc = case(870, S=40, dtype=dtype, cache=dtype, lmax=1200)
    out, _ = run_mixed(mc, BAL)
    check(mc, out, oracle_mixed(mc))


def test_mixed_balanced_fp8_and_page_16():
    mc = case(871, S=30, cache="fp8", lmax=900)
    out, _ = run_mixed(mc, BAL)
    check(mc, out, oracle_mixed(mc))
    mc = case(872, S=30, page=16, sizes=(16, 32), lmax=900)
    out, _ = run_mixed(mc, BAL)
    check(mc, out, oracle_mixed(mc))


def test_mixed_balanced_small_blocks_and_empty_rows():
    """Only 8-token blocks (every tile an 8-token one), and a batch with
    zero-length sequences, whose rows the reduce writes as zeros."""
    mc = case(873, S=20, sizes=(8,), lmax=400)
    out, _ = run_mixed(mc, BAL)
    check(mc, out, oracle_mixed(mc))
    mc = case(874, S=12, lmax=300)
    mc.case.seq_lens[[1, 4, 5]] = 0
    out, _ = run_mixed(mc, BAL)
    assert np.all(out[[1, 4, 5]] == 0.0)
    check(mc, out, oracle_mixed(mc))


def test_mixed_balanced_equals_the_balanced_decode_on_page_sized_blocks():
    """Every block one page of 16 tokens: the mixed balanced walk is the
    uniform pool's, tile for tile and chunk for chunk, so the rows agree bit
    for bit with the balanced decode on the same pool."""
    mc = case(875, S=48, page=16, sizes=(16,), lmax=2000)
    out, d = run_mixed(mc, BAL)
    c = mc.case
    ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, BAL)
    d.out.fill_(float("nan"))
    pkv.paged_attention_decode(d.out, d.query, d.k_cache, d.v_cache, d.tables, d.lens,
                               scale=c.scale, max_seq_len=c.max_seq_len, k_scale=c.k_scale,
                               v_scale=c.v_scale, partition_size=BAL, workspace=ws)
    pkv.paged_attention_reduce(d.out, ws, d.lens, num_kv_heads=c.Hkv,
                               max_seq_len=c.max_seq_len, partition_size=BAL)
    torch.cuda.synchronize()
    assert np.array_equal(out, from_dev(d.out))


def test_mixed_block_sizes_workload_balanced():
    """The bench's workload (Llama-3-8B decode shape, block size by length)
    on the balanced split: the oracle on a sample of rows covering every
    block size, and every row within twice the tolerance of the fixed split
    at 512."""
    mc = workloads.mixed_block_sizes()
    c = mc.case
    rng = np.random.default_rng(876)
    seqs = set(rng.choice(c.S, size=24, replace=False).tolist())
    for b in (8, 16, 32):
        seqs.update(np.nonzero(mc.seq_bs == b)[0][:3].tolist())
    rows = sorted(s * c.Hq + hq for s in seqs for hq in (0, 7, 18, 31))
    out, d = run_mixed(mc, BAL)
    check(mc, out, oracle_mixed(mc, rows), rows)
    fixed, _ = run_mixed(mc, 512, d)
    assert np.all(np.abs(out - fixed) <= 2 * bound(fixed, c.cache_dtype, c.q_dtype))
