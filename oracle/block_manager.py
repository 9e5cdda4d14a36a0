"""Plain reference model of the block manager (host bookkeeping of the paged pool).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (cited by page title and section):

* [C13-L2] "C13 推理 · 第2课 服务端:连续批处理与 PagedAttention"
  (geekvape-learning), section "改进二:PagedAttention": a request wastes at most
  b - 1 slots of its last block; any free block can serve any request, so
  there is no external fragmentation; several sequences may point at the same
  blocks (parallel sampling keeps one copy of the prompt's KV) and a shared
  block is copied only when one of them writes into it (copy-on-write).
* [Engine-core] "第2章:推理引擎核心技术" (aiinfra.vidrealm.tech): §1.2 (a
  sequence's block table maps logical block j, tokens 16j..16j+15, to a
  physical page), §1.5 (beams share prefix pages and copy only where they
  diverge), §3.2 (prefix cache: cut the prompt into pages, hash each page's
  tokens, look the hash up, share a hit page by raising its reference count,
  and prefill only the misses).

Readings where the pages are silent (each is listed in the design notes):

* free blocks form a FIFO queue: allocation takes the front, a block whose
  reference count drops to zero goes to the back;
* the hash of full block j is 64-bit FNV-1a (Fowler-Noll-Vo) over the 8
  little-endian bytes of block j-1's hash (0 for j = 0) followed by the 16
  token ids of the block as 4 little-endian bytes each; a result of 0 becomes 1;
* a prompt's full blocks are registered under their hash when allocated; a
  freed block keeps its registration while it waits in the queue and loses it
  when handed out for new content; a lookup stops at the first miss;
* only a partly filled last block can be shared and written, so an append
  copies at most one block.

Each operation validates everything before changing any state, like the
library; on failure it raises and the model is unchanged.
"""
from __future__ import annotations

from collections import OrderedDict

BLOCK = 16
FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK64 = (1 << 64) - 1


class NoSpace(Exception):
    pass


class BadArgument(Exception):
    pass


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the prime (mod 2^64)."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(prev: int, tokens) -> int:
    """Chained hash of one full block ([Engine-core] §3.2: hash each page's tokens; chaining with
    the previous page's hash makes a hit imply the whole prefix matches)."""
    data = prev.to_bytes(8, "little") + b"".join((int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    h = fnv1a64(data)
    return h if h != 0 else 1


class BlockManagerModel:
    def __init__(self, num_blocks: int, free_order=None):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise BadArgument("free_order must be a permutation")
        self.n = num_blocks
        self.ref = [0] * num_blocks
        self.queue = OrderedDict((b, None) for b in order)  # front = next to allocate
        self.hash = [0] * num_blocks
        self.table = {}  # block hash -> block

    # -- helpers ------------------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.queue)

    def _fresh(self) -> int:
        b, _ = self.queue.popitem(last=False)
        if self.hash[b] and self.table.get(self.hash[b]) == b:
            del self.table[self.hash[b]]
        self.hash[b] = 0
        self.ref[b] = 1
        return b

    def _share(self, b: int) -> None:
        if self.ref[b] == 0:
            del self.queue[b]
        self.ref[b] += 1

    def _check_row(self, row, nb: int) -> None:
        for j in range(nb):
            b = int(row[j])
            if not (0 <= b < self.n) or self.ref[b] <= 0:
                raise BadArgument("table row names a block not in use")

    # -- operations ---------------------------------------------------------------------------
    def add_sequence(self, tokens, row, max_blocks: int) -> int:
        """New prompt: share the blocks of its longest cached prefix of full blocks, allocate the
        rest; returns the number of cached tokens ([Engine-core] §3.2 steps 1-5)."""
        tokens = [int(t) for t in tokens]
        nb = -(-len(tokens) // BLOCK)
        nfull = len(tokens) // BLOCK
        if nb > max_blocks:
            raise BadArgument("table row too short")
        hashes, hits, h = [], 0, 0
        for j in range(nfull):
            h = block_hash(h, tokens[j * BLOCK:(j + 1) * BLOCK])
            hashes.append(h)
        for j in range(nfull):
            if hashes[j] not in self.table:
                break
            hits += 1
        waiting = sum(1 for j in range(hits) if self.ref[self.table[hashes[j]]] == 0)
        if self.num_free() - waiting < nb - hits:
            raise NoSpace()
        for j in range(hits):
            b = self.table[hashes[j]]
            self._share(b)
            row[j] = b
        for j in range(hits, nb):
            b = self._fresh()
            row[j] = b
            if j < nfull:
                self.hash[b] = hashes[j]
                self.table.setdefault(hashes[j], b)
        return hits * BLOCK

    def append(self, row, max_blocks: int, ctx: int, num_new: int):
        """Grow a sequence by num_new tokens; returns (slots, copy pairs).  A shared, partly filled
        last block is first replaced by a private copy ([C13-L2] copy-on-write; [Engine-core] §1.5)."""
        nb_old = -(-ctx // BLOCK)
        if nb_old > max_blocks:
            raise BadArgument("table row too short")
        self._check_row(row, nb_old)
        if num_new == 0:
            return [], []
        nb_new = -(-(ctx + num_new) // BLOCK)
        if nb_new > max_blocks:
            raise BadArgument("table row too short")
        cow = ctx % BLOCK != 0 and self.ref[int(row[nb_old - 1])] > 1
        if self.num_free() < (nb_new - nb_old) + (1 if cow else 0):
            raise NoSpace()
        pairs = []
        if cow:
            old = int(row[nb_old - 1])
            new = self._fresh()
            self.ref[old] -= 1
            row[nb_old - 1] = new
            pairs.append((old, new))
        for j in range(nb_old, nb_new):
            row[j] = self._fresh()
        slots = [int(row[p // BLOCK]) * BLOCK + p % BLOCK for p in range(ctx, ctx + num_new)]
        return slots, pairs

    def fork(self, parent_row, ctx: int, child_row, max_blocks: int) -> None:
        """The child points at every block of the parent ([C13-L2]: parallel samples share the
        prompt's blocks)."""
        nb = -(-ctx // BLOCK)
        if nb > max_blocks:
            raise BadArgument("table row too short")
        self._check_row(parent_row, nb)
        for j in range(nb):
            child_row[j] = parent_row[j]
            self.ref[int(parent_row[j])] += 1

    def free_sequence(self, row, ctx: int) -> None:
        nb = -(-ctx // BLOCK)
        self._check_row(row, nb)
        if len({int(row[j]) for j in range(nb)}) != nb:
            raise BadArgument("a row repeats a block")
        for j in range(nb):
            b = int(row[j])
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.queue[b] = None  # to the back
