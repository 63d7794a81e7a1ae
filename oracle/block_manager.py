"""Plain reference model of the paged KV-cache block manager.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the tests call it;
the library never imports it and it imports nothing from the library.

What it follows:
  * "Idea 1: PagedAttention" on the day-9 post (skandtandon.pages.dev): the
    cache is cut into fixed-size blocks (16 tokens) and a block table maps a
    request's logical blocks to physical blocks; blocks can sit anywhere; two
    requests with a common prefix can share the same physical blocks; when a
    shared block must diverge, only that block is copied (copy-on-write).
  * "The idea vLLM started from: pages" and "Code" on "What vLLM Is and Why It
    Exists": blocks are handed out on demand, a request holds memory only for
    the tokens it produced (rounded up to a block), and "preemption" is one
    request's blocks being taken away to feed another.

Readings (the pages leave these open):
  * Free blocks form a stack. It starts as [NB-1, ..., 1, 0] with block 0 on
    top, so a fresh pool hands out 0, 1, 2, ...; a released block goes on top
    and is handed out next.
  * A block's reference count is the number of block tables that hold it. A
    block returns to the free stack when its count reaches 0; releasing a
    table walks it from its first entry to its last.
  * Adding a sequence of n tokens takes ceil(n / B) blocks at once, or none
    when fewer are free (the pool is left as it was).
  * Appending a token writes position L (the current length). When L is a
    multiple of B a new block is taken; otherwise the token goes into the
    table's last block, and if that block is shared (count > 1) it is first
    replaced by a fresh copy: the pair (old, new) is reported for the caller to
    copy, the old block's count drops by one. With no free block the append
    fails and nothing changes.
  * Forking gives the child the parent's whole table (every count + 1) and
    length.
  * Preempting a sequence is releasing its table (its tokens must be
    recomputed later); which sequence to preempt is the caller's choice.
  * slot of position t = table[t // B] * B + t % B.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class NoSpace(Exception):
    """No free block for the request; the pool is unchanged."""


class OracleBlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("bad pool")
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))   # top of stack = end
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- helpers -------------------------------------------------------------
    def _take(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def _slot(self, seq: int, t: int) -> int:
        B = self.block_size
        return self.tables[seq][t // B] * B + t % B

    # -- operations ----------------------------------------------------------
    def add_sequence(self, seq: int, num_tokens: int) -> List[int]:
        """Blocks for a new sequence's num_tokens tokens; returns their slots."""
        if seq in self.tables or num_tokens < 0:
            raise ValueError("sequence exists or negative length")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise NoSpace()
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = num_tokens
        return [self._slot(seq, t) for t in range(num_tokens)]

    def append_token(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Room for one more token; returns (its slot, copy-on-write pair or None)."""
        table = self.tables[seq]
        t = self.lens[seq]
        cow = None
        if t % self.block_size == 0:
            if not self.free:
                raise NoSpace()
            table.append(self._take())
        else:
            last = table[-1]
            if self.ref[last] > 1:
                if not self.free:
                    raise NoSpace()
                new = self._take()
                self.ref[last] -= 1
                table[-1] = new
                cow = (last, new)
        self.lens[seq] = t + 1
        return self._slot(seq, t), cow

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise ValueError("child exists")
        self.tables[child] = list(self.tables[parent])
        for b in self.tables[child]:
            self.ref[b] += 1
        self.lens[child] = self.lens[parent]

    def free_sequence(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    preempt = free_sequence

    def num_free(self) -> int:
        return len(self.free)

    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lens[seq]
