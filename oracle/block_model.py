"""Plain model of the paged pool's books: the expected behaviour of the
library's block manager, written from the pages' description.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the library never imports
it, and it shares nothing with the C++ manager.

"vLLM 推理引擎源码级拆解" §2.1-2.2: blocks of a fixed number of tokens come from
one pool on demand; each sequence has a table from logical to physical
blocks; a new token goes into the free slot of the last block or into a
fresh block; tables may share a physical block, kept alive by a reference
count, and writing into a shared block first copies it (copy on write).
§3.3: the manager only keeps these books.  §4.2: with prefix caching each
full block is identified by its tokens and by everything before it; a new
sequence reuses the blocks of its longest cached prefix of full blocks;
cached blocks nobody references are reclaimed least recently used first.

Orders the pages leave open, as the library documents them: the lowest free
block is taken first; with none free, the cached unreferenced block released
longest ago is taken (and forgotten); a sequence releases its blocks last
block first; partial blocks are never cached.  A cached block is identified
here by the full token prefix up to its end, which is what the library's
chained hash plus stored tokens stands for.
"""
from __future__ import annotations

from collections import OrderedDict


class NoBlocks(Exception):
    """The pool cannot give the blocks a request needs (nothing changed)."""


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, prefix_cache: bool = True):
        self.NB = num_blocks
        self.bs = block_size
        self.prefix_cache = prefix_cache
        self.ref = [0] * num_blocks
        self.free = set(range(num_blocks))          # unreferenced, not cached
        self.lru = OrderedDict()                    # unreferenced, cached: oldest first
        self.key_of = {}                            # block -> full token prefix it ends
        self.block_of = {}                          # full token prefix -> block
        self.tables = {}                            # seq -> [blocks]
        self.tokens = {}                            # seq -> [token ids]

    # ---- pool ------------------------------------------------------------
    def available(self) -> int:
        return len(self.free) + len(self.lru)

    def _take(self) -> int:
        if self.free:
            b = min(self.free)
            self.free.remove(b)
        else:
            b, _ = self.lru.popitem(last=False)
            del self.block_of[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _retain(self, b: int) -> None:
        if self.ref[b] == 0:
            self.lru.pop(b, None)
        self.ref[b] += 1

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.lru[b] = True
            else:
                self.free.add(b)

    def _cache_full_block(self, seq, j: int) -> None:
        if not self.prefix_cache:
            return
        key = tuple(self.tokens[seq][:(j + 1) * self.bs])
        b = self.tables[seq][j]
        if b in self.key_of or key in self.block_of:
            return
        self.key_of[b] = key
        self.block_of[key] = b

    # ---- operations --------------------------------------------------------
    def add_sequence(self, seq, token_ids):
        if seq in self.tables:
            raise KeyError(seq)
        toks = [int(t) for t in token_ids]
        n, bs = len(toks), self.bs
        nblk = -(-n // bs)
        hits = []
        if self.prefix_cache:
            for j in range(n // bs):
                b = self.block_of.get(tuple(toks[:(j + 1) * bs]))
                if b is None:
                    break
                hits.append(b)
        if nblk - len(hits) > self.available() - sum(1 for b in hits if self.ref[b] == 0):
            raise NoBlocks()
        for b in hits:
            self._retain(b)
        self.tables[seq] = list(hits)
        self.tokens[seq] = toks
        for j in range(len(hits), nblk):
            self.tables[seq].append(self._take())
            if (j + 1) * bs <= n:
                self._cache_full_block(seq, j)
        slots = [self.tables[seq][t // bs] * bs + t % bs for t in range(n)]
        return slots, len(hits) * bs

    def append(self, seq, token_id):
        table, toks, bs = self.tables[seq], self.tokens[seq], self.bs
        n = len(toks)
        copy = None
        if n % bs == 0:
            if self.available() < 1:
                raise NoBlocks()
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            if self.available() < 1:
                raise NoBlocks()
            new = self._take()
            self._release(table[-1])
            copy = (table[-1], new)
            table[-1] = new
        toks.append(int(token_id))
        slot = table[-1] * bs + n % bs
        if (n + 1) % bs == 0:
            self._cache_full_block(seq, (n + 1) // bs - 1)
        return slot, copy

    def fork(self, parent, child):
        if child in self.tables:
            raise KeyError(child)
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = list(self.tokens[parent])
        for b in self.tables[child]:
            self._retain(b)

    def free_sequence(self, seq):
        for b in reversed(self.tables.pop(seq)):
            self._release(b)
        del self.tokens[seq]
