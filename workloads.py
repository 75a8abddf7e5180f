"""Seeded synthetic inputs for paged decode attention.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic and imports neither the oracle nor the HIP package, so
both sides can be fed the same bytes.

Layout produced (the pool layout of "vLLM 推理引擎源码级拆解" §2.3, with the
head axis read as KV heads):
  k_cache, v_cache  [NB, bs, Hkv, D]   shared physical block pool
  block_tables      [S, max_blocks]    int32, logical -> physical block
  seq_lens          [S]                int32, tokens each query attends to
  query             [S, Hq, D]
  new_key/new_value [T, Hkv, D]        tokens the cache writer stores first
  slot_mapping      [T]                int64, destination slot of each

Blocks are handed out by a seeded random permutation of the pool, so a
sequence's blocks are scattered the way the block table of §2.2 allows.  Pool
memory not holding a live token is poisoned (NaN, or the E4M3 NaN code 0x7F):
unused blocks, the unfilled tail of each last block, the slot the writer is
about to fill, and table padding points at an unused block.

Storage conventions: 'f32' float32, 'f16' float16, 'bf16' uint16 bit patterns
(round-to-nearest-even from float32), 'fp8' uint8 E4M3 codes.

Configurations (sizes from the workload list this library is measured on):
  1 tiny fp32      4 seqs, L {7,16,33,100}, 4/4 heads, D 64, bs 16, 64 blocks
  2 13B-MHA fp16   64 seqs, L ~ U{512..2048}, 40/40 heads, D 128, bs 16
  3 8B-GQA bf16    256 seqs, L = clip(round(LogNormal(ln 1024, 1)), 1, 4096),
                   32/8 heads, D 128, bs 16
  4 long split-K   8 seqs, L {32,48,64,64,96,96,128,128}*1024, 64/8 heads,
                   D 128, bs 32, partitions of 512 tokens
  5 prefix + fp8   128 seqs sharing a 1024-token prefix plus tails U{16..512},
                   32/8 heads, D 128, bs 8/16/32, E4M3 cache, bf16 query
Configs 2 and 3 hold L-1 tokens in the pool and append token L-1 of every
sequence through the cache writer; config 5 writes every token through it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NP_DTYPE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
POISON = {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
          "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}


@dataclass
class Case:
    name: str
    seed: int
    S: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    q_dtype: str
    cache_dtype: str
    src_dtype: str
    scale: float
    max_seq_len: int
    partition_size: int
    seq_lens: np.ndarray
    block_tables: np.ndarray
    query: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    new_key: np.ndarray
    new_value: np.ndarray
    slot_mapping: np.ndarray
    k_scale: float = 1.0
    v_scale: float = 1.0
    pad_block: int = -1
    notes: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]

    def copy(self) -> "Case":
        c = Case(**{k: (v.copy() if isinstance(v, np.ndarray) else v)
                    for k, v in self.__dict__.items()})
        c.notes = dict(self.notes)
        return c


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def draw(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) values stored as `dtype` (drawn as float32, then rounded)."""
    n = int(np.prod(shape))
    out = np.empty(n, NP_DTYPE[dtype])
    for i in range(0, n, chunk):
        x = rng.standard_normal(min(chunk, n - i), dtype=np.float32)
        if dtype == "f32":
            out[i:i + x.size] = x
        elif dtype == "f16":
            out[i:i + x.size] = x.astype(np.float16)
        elif dtype == "bf16":
            out[i:i + x.size] = bf16_bits(x)
        else:
            raise ValueError("cannot draw values directly as " + dtype)
    return out.reshape(shape)


def _as_float32(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_values(x)
    return x.astype(np.float32)


def amax_scale(x: np.ndarray, dtype: str) -> float:
    """Per-tensor E4M3 scale: amax(|x|) / 448, in float32."""
    a = np.float32(np.max(np.abs(_as_float32(x, dtype))))
    return float(np.float32(a / np.float32(448.0)))


def make_case(name: str, seed: int, lens, Hq: int, Hkv: int, D: int, bs: int, *,
              q_dtype: str, cache_dtype: str, src_dtype: Optional[str] = None,
              pool_factor: float = 1.1, NB: Optional[int] = None,
              max_seq_len: Optional[int] = None, partition_size: int = 0,
              append_last: bool = False, prefix_len: int = 0,
              write_all: bool = False, rng: Optional[np.random.Generator] = None,
              scale: Optional[float] = None) -> Case:
    """Generic seeded case.

    lens          sequence lengths (or a callable rng -> lengths).
    append_last   pool holds L-1 tokens; token L-1 of each sequence arrives in
                  new_key/new_value with its slot in slot_mapping.
    prefix_len    every sequence starts with the same prefix_len tokens stored
                  once, in blocks all tables share (prefix_len % bs == 0).
    write_all     the pool starts fully poisoned; every live token arrives
                  through new_key/new_value (used for the fp8 cache).
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    if callable(lens):
        lens = lens(rng)
    seq_lens = np.asarray(lens, dtype=np.int64)
    S = seq_lens.size
    src_dtype = src_dtype or cache_dtype
    if cache_dtype == "fp8":
        write_all = True
    if prefix_len:
        assert prefix_len % bs == 0 and np.all(seq_lens >= prefix_len)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max())
    max_blocks = max(1, -(-max_seq_len // bs))

    # --- block assignment: seeded permutation of the pool -------------------
    nblk = -(-seq_lens // bs)
    npre = prefix_len // bs
    need = int(nblk.sum() - (S - 1) * npre) if prefix_len else int(nblk.sum())
    if NB is None:
        NB = int(math.ceil(pool_factor * need - 1e-9))
    assert NB > need, "the pool needs at least one spare block for table padding"
    perm = rng.permutation(NB).astype(np.int32)
    pad_block = int(perm[-1])
    tables = np.full((S, max_blocks), pad_block, np.int32)
    pos = npre
    for s in range(S):
        tables[s, :npre] = perm[:npre]
        k = int(nblk[s]) - npre
        tables[s, npre:npre + k] = perm[pos:pos + k]
        pos += k
    assert pos == need

    # --- pool contents -------------------------------------------------------
    shape = (NB, bs, Hkv, D)
    if write_all:
        k_cache = np.full(shape, POISON[cache_dtype], NP_DTYPE[cache_dtype])
        v_cache = np.full(shape, POISON[cache_dtype], NP_DTYPE[cache_dtype])
    else:
        k_cache = draw(rng, shape, cache_dtype)
        v_cache = draw(rng, shape, cache_dtype)
    query = draw(rng, (S, Hq, D), q_dtype)

    # Poison what holds no live token.
    used = np.zeros(NB, bool)
    for s in range(S):
        used[tables[s, :nblk[s]]] = True
    if not write_all:
        k_cache[~used] = POISON[cache_dtype]
        v_cache[~used] = POISON[cache_dtype]
        cached = seq_lens - 1 if append_last else seq_lens
        for s in range(S):
            last = int(tables[s, nblk[s] - 1])
            first_dead = int(cached[s] - (nblk[s] - 1) * bs)
            if first_dead < bs:
                k_cache[last, first_dead:] = POISON[cache_dtype]
                v_cache[last, first_dead:] = POISON[cache_dtype]

    # --- tokens that reach the pool through the cache writer ---------------
    def slot_of(s, t):
        return int(tables[s, t // bs]) * bs + t % bs

    slots: List[int] = []
    if write_all:
        if prefix_len:
            slots += [slot_of(0, t) for t in range(prefix_len)]
        for s in range(S):
            slots += [slot_of(s, t) for t in range(prefix_len, int(seq_lens[s]))]
    elif append_last:
        slots = [slot_of(s, int(seq_lens[s]) - 1) for s in range(S)]
    T = len(slots)
    if T:
        new_key = draw(rng, (T, Hkv, D), src_dtype)
        new_value = draw(rng, (T, Hkv, D), src_dtype)
    else:
        new_key = np.zeros((0, Hkv, D), NP_DTYPE[src_dtype])
        new_value = np.zeros((0, Hkv, D), NP_DTYPE[src_dtype])
    k_scale = v_scale = 1.0
    if cache_dtype == "fp8":
        k_scale = amax_scale(new_key, src_dtype)
        v_scale = amax_scale(new_value, src_dtype)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return Case(name=name, seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB,
                q_dtype=q_dtype, cache_dtype=cache_dtype, src_dtype=src_dtype,
                scale=scale, max_seq_len=int(max_seq_len),
                partition_size=int(partition_size),
                seq_lens=seq_lens.astype(np.int32), block_tables=tables,
                query=query, k_cache=k_cache, v_cache=v_cache, new_key=new_key,
                new_value=new_value,
                slot_mapping=np.asarray(slots, np.int64).reshape(T),
                k_scale=k_scale, v_scale=v_scale, pad_block=pad_block,
                notes={"prefix_len": prefix_len, "append_last": append_last})


# --- mixed block sizes ---------------------------------------------------

def block_size_for_length(L: int) -> int:
    """Tokens per block by expected length, the thresholds of "vLLM 0.5 深度拆解"
    §1.3 (short < 128: 8; medium < 2048: 16; long: 32); here the length
    itself stands in for the estimate."""
    return 8 if L < 128 else (16 if L < 2048 else 32)


@dataclass
class MixedCase:
    """A pool of pages (case.bs = page tokens, case.NB = pages) whose
    sequences have blocks of seq_bs[s] tokens: seq_bs[s] / page consecutive
    pages from the page the table names."""
    case: Case
    seq_bs: np.ndarray


def make_mixed_case(name: str, seed: int, lens, Hq: int, Hkv: int, D: int, page: int, *,
                    q_dtype: str, cache_dtype: str, block_sizes=None,
                    src_dtype: Optional[str] = None, pool_factor: float = 1.1,
                    max_seq_len: Optional[int] = None, append_last: bool = False,
                    rng: Optional[np.random.Generator] = None) -> MixedCase:
    """Seeded case with a block size per sequence (default: by length, as
    block_size_for_length).  Pages are handed out in aligned groups of 32
    tokens (32 / page pages), shuffled: a 32-token block takes a group, a
    16-token block half of one, an 8-token block a quarter, so every block's
    pages are consecutive.  Unused pages and the dead rows of each last
    block are poisoned.  fp8: every live token arrives through the writer,
    as in make_case."""
    if rng is None:
        rng = np.random.default_rng(seed)
    if callable(lens):
        lens = lens(rng)
    seq_lens = np.asarray(lens, dtype=np.int64)
    S = seq_lens.size
    if block_sizes is None:
        seq_bs = np.array([block_size_for_length(int(L)) for L in seq_lens], np.int64)
    else:
        seq_bs = np.asarray(block_sizes(rng, seq_lens) if callable(block_sizes)
                            else block_sizes, np.int64)
    assert np.all(seq_bs >= page) and np.all(seq_bs % page == 0) and np.all(seq_bs <= 32)
    src_dtype = src_dtype or cache_dtype
    write_all = cache_dtype == "fp8"
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max())
    max_blocks = max(1, -(-max_seq_len // page))       # enough for the smallest block
    gp = 32 // page                                    # pages per 32-token group
    nblk = -(-seq_lens // seq_bs)
    need_groups = int(math.ceil(float((nblk * seq_bs).sum()) / 32))
    n_groups = int(math.ceil(pool_factor * need_groups - 1e-9)) + 1
    NP = n_groups * gp
    groups = rng.permutation(n_groups).astype(np.int64)
    pad_page = int(groups[-1]) * gp
    tables = np.full((S, max_blocks), pad_page, np.int32)
    gi = 0
    for size in (32, 16, 8):                           # largest blocks first
        owners = [(s, j) for s in range(S) if seq_bs[s] == size for j in range(nblk[s])]
        per = 32 // size
        pieces = []
        while len(pieces) < len(owners):
            g = int(groups[gi])
            gi += 1
            pieces += [g * gp + k * (size // page) for k in range(per)]
        pieces = rng.permutation(np.asarray(pieces, np.int64))[:len(owners)]
        for (s, j), first in zip(owners, pieces):
            tables[s, j] = first
    assert gi < n_groups

    shape = (NP, page, Hkv, D)
    if write_all:
        k_cache = np.full(shape, POISON[cache_dtype], NP_DTYPE[cache_dtype])
        v_cache = np.full(shape, POISON[cache_dtype], NP_DTYPE[cache_dtype])
    else:
        k_cache = draw(rng, shape, cache_dtype)
        v_cache = draw(rng, shape, cache_dtype)
    query = draw(rng, (S, Hq, D), q_dtype)

    def rows_of(s, t):                                 # pool rows of tokens t of sequence s
        b = int(seq_bs[s])
        return tables[s, t // b].astype(np.int64) * page + t % b

    def row_of(s, t):
        return int(rows_of(s, np.array([t]))[0])

    if not write_all:
        live = np.zeros(NP * page, bool)
        cached = seq_lens - 1 if append_last else seq_lens
        for s in range(S):
            live[rows_of(s, np.arange(int(cached[s])))] = True
        kf = k_cache.reshape(NP * page, Hkv, D)
        vf = v_cache.reshape(NP * page, Hkv, D)
        kf[~live] = POISON[cache_dtype]
        vf[~live] = POISON[cache_dtype]
    if write_all:
        slots = np.concatenate([rows_of(s, np.arange(int(seq_lens[s]))) for s in range(S)])
    elif append_last:
        slots = [row_of(s, int(seq_lens[s]) - 1) for s in range(S)]
    else:
        slots = []
    T = len(slots)
    new_key = draw(rng, (T, Hkv, D), src_dtype)
    new_value = draw(rng, (T, Hkv, D), src_dtype)
    k_scale = v_scale = 1.0
    if cache_dtype == "fp8":
        k_scale = amax_scale(new_key, src_dtype)
        v_scale = amax_scale(new_value, src_dtype)
    c = Case(name=name, seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=page, NB=NP,
             q_dtype=q_dtype, cache_dtype=cache_dtype, src_dtype=src_dtype,
             scale=float(np.float32(1.0 / math.sqrt(D))), max_seq_len=int(max_seq_len),
             partition_size=0, seq_lens=seq_lens.astype(np.int32), block_tables=tables,
             query=query, k_cache=k_cache, v_cache=v_cache, new_key=new_key,
             new_value=new_value, slot_mapping=np.asarray(slots, np.int64).reshape(T),
             k_scale=k_scale, v_scale=v_scale, pad_block=pad_page,
             notes={"append_last": append_last, "mixed": True})
    return MixedCase(c, seq_bs.astype(np.int32))


def mixed_block_sizes(S: int = 256) -> MixedCase:
    """The Llama-3-8B GQA decode shape with each sequence's block size picked
    by its length (8 / 16 / 32 tokens), over a pool of 8-token pages."""
    return make_mixed_case("mixed-bs-llama3-8b", 8, lambda r: llama3_8b_gqa_lens(r, S),
                           32, 8, 128, 8, q_dtype="bf16", cache_dtype="bf16",
                           max_seq_len=4096, append_last=True)


# --- the five workloads ------------------------------------------------

def tiny_f32() -> Case:
    return make_case("tiny-fp32", 1, [7, 16, 33, 100], 4, 4, 64, 16,
                     q_dtype="f32", cache_dtype="f32", NB=64)


def llama2_13b_mha_lens(rng):
    return rng.integers(512, 2048, size=64, endpoint=True)


def llama2_13b_mha() -> Case:
    return make_case("llama2-13b-mha-fp16", 2, llama2_13b_mha_lens, 40, 40, 128, 16,
                     q_dtype="f16", cache_dtype="f16", max_seq_len=2048,
                     append_last=True)


def llama3_8b_gqa_lens(rng, S: int = 256):
    x = rng.lognormal(mean=math.log(1024.0), sigma=1.0, size=S)
    return np.clip(np.rint(x), 1, 4096).astype(np.int64)


def llama3_8b_gqa() -> Case:
    return make_case("llama3-8b-gqa-bf16", 3, llama3_8b_gqa_lens, 32, 8, 128, 16,
                     q_dtype="bf16", cache_dtype="bf16", max_seq_len=4096,
                     append_last=True)


LONG_CONTEXT_KTOKENS = [32, 48, 64, 64, 96, 96, 128, 128]


def long_context_gqa(scale_down: int = 1) -> Case:
    """Long-context split-K.  scale_down > 1 divides every length (for tests
    that keep the shape family but need the oracle to finish quickly)."""
    lens = [k * 1024 // scale_down for k in LONG_CONTEXT_KTOKENS]
    return make_case("long-gqa-bf16-splitk", 4, lens, 64, 8, 128, 32,
                     q_dtype="bf16", cache_dtype="bf16",
                     max_seq_len=max(lens), partition_size=512)


def shared_prefix_lens(rng, S: int = 128, prefix: int = 1024):
    return prefix + rng.integers(16, 512, size=S, endpoint=True)


def shared_prefix_fp8(bs: int = 16, S: int = 128) -> Case:
    return make_case("shared-prefix-fp8-bs%d" % bs, 5, lambda r: shared_prefix_lens(r, S),
                     32, 8, 128, bs, q_dtype="bf16", cache_dtype="fp8",
                     src_dtype="bf16", max_seq_len=1536, prefix_len=1024)


WORKLOADS = {"tiny-f32": tiny_f32, "llama2-13b-mha": llama2_13b_mha,
             "llama3-8b-gqa": llama3_8b_gqa, "long-context-gqa": long_context_gqa,
             "shared-prefix-fp8": shared_prefix_fp8}


# --- several new query tokens per sequence ---------------------------------

@dataclass
class MultiCase:
    """A paged pool and tables (`case`, whose seq_lens count the new tokens)
    with Qn new query tokens per sequence: query [total_q, Hq, D], the
    exclusive prefix query_start [S + 1] and the bound max_query_len."""
    case: Case
    query: np.ndarray
    query_start: np.ndarray
    max_query_len: int


def make_multi_case(name: str, seed: int, lens, qlens, Hq: int, Hkv: int, D: int, bs: int, *,
                    q_dtype: str, cache_dtype: str, **kw) -> MultiCase:
    """Seeded multi-query case: the pool as make_case builds it (the Qn new
    tokens of a sequence are its last Qn cached tokens), then the query
    tokens drawn N(0,1) in the query dtype."""
    rng = np.random.default_rng(seed)
    if callable(lens):
        lens = lens(rng)
    if callable(qlens):
        qlens = qlens(rng, np.asarray(lens))
    c = make_case(name, seed, lens, Hq, Hkv, D, bs, q_dtype=q_dtype, cache_dtype=cache_dtype,
                  rng=rng, **kw)
    qlens = np.asarray(qlens, np.int64)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    query = draw(rng, (int(qs[-1]), Hq, D), q_dtype)
    return MultiCase(c, query, qs, max(1, int(qlens.max()) if qlens.size else 1))


def spec_verify(S: int = 256, draft: int = 4) -> MultiCase:
    """Speculative verification on the Llama-3-8B GQA decode shape: every
    sequence checks `draft` drafted tokens (its last `draft` cached tokens),
    lengths as the Llama-3-8B decode workload."""
    return make_multi_case("spec-verify-llama3-8b", 6, lambda r: np.maximum(
        llama3_8b_gqa_lens(r, S), draft), np.full(S, draft), 32, 8, 128, 16,
        q_dtype="bf16", cache_dtype="bf16", max_seq_len=4096)


def chunked_prefill(S: int = 8, chunk: int = 512) -> MultiCase:
    """Chunked prefill on the Llama-3-8B GQA shape: each sequence has 512 to
    3072 tokens already cached and brings a chunk of `chunk` new prompt
    tokens (the last `chunk` of its cached tokens)."""
    return make_multi_case("chunked-prefill-llama3-8b", 7,
                           lambda r: r.integers(512, 3072, size=S, endpoint=True) + chunk,
                           np.full(S, chunk), 32, 8, 128, 16, q_dtype="bf16",
                           cache_dtype="bf16", max_seq_len=3072 + chunk)
