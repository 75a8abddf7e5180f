"""Test-side pool construction from logical K/V (independent of the oracle).

Builds a paged pool by slicing each sequence's logical K/V into block-sized
chunks and copying chunk j into the physical block its table names, the
block table of "vLLM 推理引擎源码级拆解" §2.2.  Written with numpy slices so
that it shares nothing with the oracle's per-element address arithmetic.
"""
from __future__ import annotations

import numpy as np

import workloads


def build_pool(Ks, Vs, bs, *, dtype, NB=None, rng=None, max_blocks=None,
               shared_prefix_blocks=0):
    """Ks, Vs: lists of [L_s, Hkv, D] arrays in storage dtype `dtype`.

    Returns (k_cache, v_cache, block_tables, seq_lens).  Unused pool memory
    and block tails are poisoned; table padding points at a poisoned block.
    With shared_prefix_blocks = n, the first n blocks of every sequence are
    stored once (taken from sequence 0) and all tables point at them."""
    rng = rng or np.random.default_rng(0)
    S = len(Ks)
    Hkv, D = Ks[0].shape[1], Ks[0].shape[2]
    lens = np.array([k.shape[0] for k in Ks], np.int32)
    nblk = [(-(-int(L) // bs)) for L in lens]
    need = sum(nblk) - (S - 1) * shared_prefix_blocks
    if NB is None:
        NB = need + 1 + need // 4
    assert NB > need
    if max_blocks is None:
        max_blocks = max(nblk)
    perm = rng.permutation(NB).astype(np.int32)
    poison = workloads.POISON[dtype]
    npdt = workloads.NP_DTYPE[dtype]
    kc = np.full((NB, bs, Hkv, D), poison, npdt)
    vc = np.full((NB, bs, Hkv, D), poison, npdt)
    tables = np.full((S, max_blocks), perm[-1], np.int32)
    nxt = shared_prefix_blocks
    for s in range(S):
        for j in range(nblk[s]):
            if j < shared_prefix_blocks:
                phys = perm[j]
            else:
                phys = perm[nxt]
                nxt += 1
            tables[s, j] = phys
            lo, hi = j * bs, min((j + 1) * bs, int(lens[s]))
            if j < shared_prefix_blocks and s > 0:
                continue
            kc[phys, :hi - lo] = Ks[s][lo:hi]
            vc[phys, :hi - lo] = Vs[s][lo:hi]
    return kc, vc, tables, lens


def relabel(k_cache, v_cache, tables, rng):
    """Moves every physical block b to pi[b] and rewrites the tables."""
    NB = k_cache.shape[0]
    pi = rng.permutation(NB).astype(np.int32)
    k2 = np.empty_like(k_cache)
    v2 = np.empty_like(v_cache)
    k2[pi] = k_cache
    v2[pi] = v_cache
    return k2, v2, pi[tables]


def build_mixed_pool(Ks, Vs, seq_bs, page, *, dtype, rng=None, spare_groups=2):
    """A pool of `page`-token pages where sequence s has blocks of seq_bs[s]
    tokens, each seq_bs[s] / page consecutive pages ("vLLM 0.5 深度拆解"
    §1.3 block sizes per request; pages are this library's layout for them).
    Each block is placed in its own piece of a shuffled 32-token group of
    pages, and its tokens are copied with one slice into the pool seen as
    rows: block j of sequence s starts at row table[s][j] * page.

    Returns (k_cache, v_cache, block_tables, seq_lens)."""
    rng = rng or np.random.default_rng(0)
    S = len(Ks)
    Hkv, D = Ks[0].shape[1], Ks[0].shape[2]
    lens = np.array([k.shape[0] for k in Ks], np.int32)
    gp = 32 // page
    nblk = [-(-int(L) // int(b)) for L, b in zip(lens, seq_bs)]
    groups_needed = sum(-(-n * int(b) // 32) for n, b in zip(nblk, seq_bs))
    n_groups = groups_needed + spare_groups
    order = list(rng.permutation(n_groups))
    poison = workloads.POISON[dtype]
    npdt = workloads.NP_DTYPE[dtype]
    NP = n_groups * gp
    kc = np.full((NP, page, Hkv, D), poison, npdt)
    vc = np.full((NP, page, Hkv, D), poison, npdt)
    krows = kc.reshape(NP * page, Hkv, D)
    vrows = vc.reshape(NP * page, Hkv, D)
    max_blocks = max(nblk)
    tables = np.full((S, max_blocks), order[-1] * gp, np.int32)
    for s in range(S):
        b = int(seq_bs[s])
        free = []
        for j in range(nblk[s]):
            if not free:                   # a fresh group, cut into 32 / b blocks
                g = order.pop(0)
                free = [g * gp + k * (b // page) for k in range(32 // b)]
            first = free.pop(0)
            tables[s, j] = first
            lo, hi = j * b, min((j + 1) * b, int(lens[s]))
            krows[first * page:first * page + hi - lo] = Ks[s][lo:hi]
            vrows[first * page:first * page + hi - lo] = Vs[s][lo:hi]
    return kc, vc, tables, lens
