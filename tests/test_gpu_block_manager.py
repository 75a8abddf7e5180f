"""The block manager's tables, slots and copy-on-write pairs driving the GPU
path: copy_blocks bit for bit against a plain copy, and a batch built with a
shared system prompt (prefix caching), a fork (shared blocks) and appends
(copy on write) decoded on the GPU against the oracle on a CPU mirror of the
same pool ("vLLM 推理引擎源码级拆解" §2.1-2.2, §4.2)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_361_amd as pkv
import workloads
from gpu_case import assert_within, bound, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "fp8"])
def test_copy_blocks_bit_exact(dtype):
    rng = np.random.default_rng(600)
    NB, bs, Hkv, D = 40, 16, 2, 64
    npdt = workloads.NP_DTYPE[dtype]
    kc = rng.integers(0, 255, size=(NB, bs, Hkv, D * np.dtype(npdt).itemsize), dtype=np.uint8)
    vc = rng.integers(0, 255, size=kc.shape, dtype=np.uint8)
    kc, vc = kc.view(npdt), vc.view(npdt)
    pairs = np.array([[3, 7], [0, 39], [12, 12], [5, 50], [-1, 2], [20, 1]], np.int32)
    dk = torch.from_numpy(kc.view(np.uint8).copy()).cuda()
    dv = torch.from_numpy(vc.view(np.uint8).copy()).cuda()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
           "fp8": torch.uint8}[dtype]
    shape = (NB, bs, Hkv, D)
    dk = dk.view(tdt).view(shape) if dtype != "fp8" else dk.view(shape)
    dv = dv.view(tdt).view(shape) if dtype != "fp8" else dv.view(shape)
    # the fp8 pool is passed as bytes with its dtype code
    if dtype == "fp8":
        rc = pkv._load().pkv_copy_blocks(pkv._ptr(dk), pkv._ptr(dv), pkv._ptr(dk), pkv._ptr(dv),
                                         3, pkv._ptr(torch.from_numpy(pairs).cuda()),
                                         len(pairs), NB, NB, bs, Hkv, D, pkv._stream(None))
        assert rc == 0
    else:
        pkv.copy_blocks(dk, dv, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    ek, ev = kc.copy(), vc.copy()
    for s, d in pairs:
        if 0 <= s < NB and 0 <= d < NB and s != d:
            ek[d] = ek[s]
            ev[d] = ev[s]
    assert np.array_equal(dk.view(torch.uint8).cpu().numpy().reshape(-1), ek.view(np.uint8).reshape(-1))
    assert np.array_equal(dv.view(torch.uint8).cpu().numpy().reshape(-1), ev.view(np.uint8).reshape(-1))


def token_rows(tokens, t0, t1, Hkv, D, dtype):
    """K and V rows of positions t0..t1-1: a function of the token prefix up to
    each position, so equal prefixes hold equal K/V (what sharing relies on)."""
    if t1 <= t0:
        e = np.zeros((0, Hkv, D), workloads.NP_DTYPE[dtype])
        return e, e.copy()
    ks, vs = [], []
    for t in range(t0, t1):
        seed = zlib.crc32(np.asarray(tokens[:t + 1], np.int32).tobytes())
        r = np.random.default_rng(seed)
        ks.append(workloads.draw(r, (Hkv, D), dtype))
        vs.append(workloads.draw(r, (Hkv, D), dtype))
    return np.stack(ks), np.stack(vs)


class Mirror:
    """The same pool on the GPU and on the host, written the same way."""

    def __init__(self, NB, bs, Hkv, D, dtype):
        self.shape, self.dtype = (NB, bs, Hkv, D), dtype
        pz = workloads.POISON[dtype]
        self.kc = np.full(self.shape, pz, workloads.NP_DTYPE[dtype])
        self.vc = self.kc.copy()
        self.dk, self.dv = to_dev(self.kc, dtype), to_dev(self.vc, dtype)

    def write(self, kv, slots):
        k, v = kv
        if len(slots) == 0:
            return
        sl = np.asarray(slots, np.int64)
        pkv.reshape_and_cache(to_dev(k, self.dtype), to_dev(v, self.dtype), self.dk, self.dv,
                              torch.from_numpy(sl).cuda())
        oracle.reshape_and_cache(k, v, self.kc, self.vc, sl, src_dtype=self.dtype,
                                 cache_dtype=self.dtype)

    def copy(self, pair):
        pkv.copy_blocks(self.dk, self.dv, torch.tensor([pair], dtype=torch.int32).cuda())
        self.kc[pair[1]] = self.kc[pair[0]]
        self.vc[pair[1]] = self.vc[pair[0]]


def test_block_manager_drives_decode():
    NB, bs, Hkv, G, D, dtype = 48, 16, 2, 4, 64, "bf16"
    bm = pkv.BlockManager(NB, bs, prefix_cache=True)
    pool = Mirror(NB, bs, Hkv, D, dtype)
    rng = np.random.default_rng(610)
    system = rng.integers(0, 1000, size=32).tolist()          # two full blocks
    toks = {}

    def add(seq, prompt):
        slots, cached = bm.add_sequence(seq, prompt)
        toks[seq] = list(prompt)
        pool.write(token_rows(prompt, cached, len(prompt), Hkv, D, dtype), slots[cached:])
        return cached

    def append(seq, tok):
        slot, copy = bm.append(seq, tok)
        if copy is not None:
            pool.copy(copy)
        toks[seq].append(tok)
        n = len(toks[seq])
        pool.write(token_rows(toks[seq], n - 1, n, Hkv, D, dtype), [slot])
        return copy

    assert add(0, system + rng.integers(0, 1000, size=9).tolist()) == 0
    assert add(1, system + rng.integers(0, 1000, size=21).tolist()) == 32     # prefix reused
    bm.fork(0, 2)
    toks[2] = list(toks[0])
    copies = [append(s, int(rng.integers(0, 1000))) for s in (2, 0, 2, 1)]
    assert copies[0] is not None and copies[1] is None        # the first writer copies
    for _ in range(20):
        for s in (0, 1, 2):
            append(s, int(rng.integers(0, 1000)))
    bm.free(1)
    assert add(3, system + [7, 7, 7]) == 32                   # still cached, held by 0 and 2
    for _ in range(5):
        append(3, int(rng.integers(0, 1000)))
    torch.cuda.synchronize()
    # the GPU pool equals the host pool byte for byte
    for dev_pool, host_pool in ((pool.dk, pool.kc), (pool.dv, pool.vc)):
        got = dev_pool.view(torch.int16 if dtype != "f32" else torch.int32).cpu().numpy()
        assert np.array_equal(got.view(host_pool.dtype), host_pool)

    seqs = [0, 2, 3]
    S = len(seqs)
    max_blocks = max(len(bm.block_table(s)) for s in seqs)
    tables = np.zeros((S, max_blocks), np.int32)
    lens = np.zeros(S, np.int32)
    for i, s in enumerate(seqs):
        t = bm.block_table(s)
        tables[i, :len(t)] = t
        lens[i] = bm.seq_len(s)
        assert lens[i] == len(toks[s])
    q = workloads.draw(rng, (S, Hkv * G, D), dtype)
    ref = oracle.paged_decode(q, pool.kc, pool.vc, tables, lens, q_dtype=dtype,
                              cache_dtype=dtype, scale=0.125)
    dq, dt, dl = to_dev(q, dtype), torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    for P in (0, pkv.PARTITION_BALANCED):
        out = torch.empty(S, Hkv * G, D, dtype=torch.bfloat16, device="cuda")
        ws = pkv.allocate_workspace(S, Hkv * G, Hkv, D, int(lens.max()), P)
        pkv.paged_attention_decode(out, dq, pool.dk, pool.dv, dt, dl, scale=0.125,
                                   max_seq_len=int(lens.max()), partition_size=P, workspace=ws,
                                   algo="mfma")
        if P != 0:
            pkv.paged_attention_reduce(out, ws, dl, num_kv_heads=Hkv,
                                       max_seq_len=int(lens.max()), partition_size=P)
        torch.cuda.synchronize()
        o = from_dev(out)
        assert_within(o, ref, bound(ref, dtype, dtype))


def test_swap_round_trip_bit_exact():
    """Device blocks out to a pinned host pool and back into other device
    blocks ("vLLM 推理引擎源码级拆解" §3.2 swapping), byte for byte."""
    rng = np.random.default_rng(620)
    NB, NBh, bs, Hkv, D = 64, 16, 16, 2, 128
    k = torch.from_numpy(workloads.draw(rng, (NB, bs, Hkv, D), "bf16").view(np.int16)).cuda()
    v = torch.from_numpy(workloads.draw(rng, (NB, bs, Hkv, D), "bf16").view(np.int16)).cuda()
    k, v = k.view(torch.bfloat16), v.view(torch.bfloat16)
    hk = torch.zeros((NBh, bs, Hkv, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    src = [5, 9, 20, 33, 63]
    out_pairs = torch.tensor([[b, i] for i, b in enumerate(src)], dtype=torch.int32).cuda()
    orig_k, orig_v = k[src].cpu().clone(), v[src].cpu().clone()
    pkv.swap_blocks(hk, hv, k, v, out_pairs)
    torch.cuda.synchronize()
    assert torch.equal(hk[:5].view(torch.int16), orig_k.view(torch.int16))
    assert torch.equal(hv[:5].view(torch.int16), orig_v.view(torch.int16))
    # the device blocks are reused for other data, then the swapped-out ones return
    pkv.copy_blocks(k, v, torch.tensor([[1, b] for b in src], dtype=torch.int32).cuda())
    dst = [40, 41, 42, 43, 0]
    in_pairs = torch.tensor([[i, b] for i, b in enumerate(dst)], dtype=torch.int32).cuda()
    pkv.swap_blocks(k, v, hk, hv, in_pairs)
    torch.cuda.synchronize()
    assert torch.equal(k[dst].cpu().view(torch.int16), orig_k.view(torch.int16))
    assert torch.equal(v[dst].cpu().view(torch.int16), orig_v.view(torch.int16))


def test_preempt_by_swap_and_resume():
    """A sequence is swapped out (its blocks copied to the host pool and
    freed), its device blocks are taken and overwritten by another sequence,
    and it is swapped back into fresh blocks: its decode is unchanged, bit for
    bit."""
    NB, NBh, bs, Hkv, G, D, dtype = 24, 16, 16, 2, 4, 64, "bf16"
    gpu = pkv.BlockManager(NB, bs, prefix_cache=False)
    host = pkv.BlockManager(NBh, bs, prefix_cache=False)
    pool = Mirror(NB, bs, Hkv, D, dtype)
    hk = torch.zeros((NBh, bs, Hkv, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    rng = np.random.default_rng(630)
    toks = rng.integers(0, 1000, size=150).tolist()
    slots, _ = gpu.add_sequence(0, toks)
    pool.write(token_rows(toks, 0, len(toks), Hkv, D, dtype), slots)
    q = to_dev(workloads.draw(rng, (1, Hkv * G, D), dtype), dtype)

    def decode(table):
        out = torch.empty(1, Hkv * G, D, dtype=torch.bfloat16, device="cuda")
        pkv.paged_attention_decode(out, q, pool.dk, pool.dv,
                                   torch.from_numpy(table[None].astype(np.int32)).cuda(),
                                   torch.tensor([len(toks)], dtype=torch.int32).cuda(),
                                   scale=0.125, max_seq_len=len(toks), algo="mfma")
        torch.cuda.synchronize()
        return out.cpu().clone()

    before = decode(gpu.block_table(0))
    # swap out: host blocks for the sequence, copy, free on the device
    host.add_sequence(0, toks)
    pairs = np.stack([gpu.block_table(0), host.block_table(0)], 1).astype(np.int32)
    pkv.swap_blocks(hk, hv, pool.dk, pool.dv, torch.from_numpy(pairs).cuda())
    gpu.free(0)
    # another sequence takes (and overwrites) the freed blocks
    other = rng.integers(0, 1000, size=200).tolist()
    slots, _ = gpu.add_sequence(1, other)
    pool.write(token_rows(other, 0, len(other), Hkv, D, dtype), slots)
    # swap in: fresh device blocks, copy back, release the host blocks
    gpu.add_sequence(2, toks)
    pairs = np.stack([host.block_table(0), gpu.block_table(2)], 1).astype(np.int32)
    pkv.swap_blocks(pool.dk, pool.dv, hk, hv, torch.from_numpy(pairs).cuda())
    host.free(0)
    after = decode(gpu.block_table(2))
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))
