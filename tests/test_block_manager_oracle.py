"""Pins of the block-manager reference model (oracle/block_manager.py), on the CPU.

None retypes the model: a scenario worked by hand from the rules, invariants over
random operation sequences, a content model (every sequence must read back exactly
its own token history through its table, shared prefixes and copy-on-write included),
the capacity figures printed by the pages' program, and planted mistakes that a pin
must catch."""
import json
import os

import numpy as np
import pytest

from oracle.block_manager import NoSpace, OracleBlockManager

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capacity_program.json")


def test_hand_worked_scenario():
    """Four blocks of 16 tokens, worked by hand from the rules."""
    bm = OracleBlockManager(4)
    assert bm.add_sequence(1, 20) == list(range(0, 20))        # blocks 0, 1 (block 0 on top)
    assert bm.table(1) == [0, 1] and bm.num_free() == 2
    bm.fork(1, 2)                                                # both tables hold 0, 1
    slot, cow = bm.append_token(2)                               # position 20 of a shared block
    assert (slot, cow) == (2 * 16 + 4, (1, 2))                   # copied to fresh block 2
    assert bm.table(2) == [0, 2] and bm.table(1) == [0, 1]
    slot, cow = bm.append_token(1)                               # block 1 is no longer shared
    assert (slot, cow) == (1 * 16 + 4, None)
    bm.free_sequence(2)                                          # block 2 back on top; 0 still held
    assert bm.num_free() == 2 and bm.free == [3, 2]
    for _ in range(11):
        bm.append_token(1)                                       # positions 21 .. 31
    slot, cow = bm.append_token(1)                               # position 32: a new block
    assert (slot, cow) == (2 * 16, None) and bm.table(1) == [0, 1, 2]
    with pytest.raises(NoSpace):
        bm.add_sequence(3, 17)                                   # needs 2 blocks, 1 free
    assert bm.num_free() == 1
    assert bm.add_sequence(3, 16) == list(range(48, 64))         # exactly one block
    with pytest.raises(NoSpace):
        bm.append_token(3)                                       # position 16: no block left
    assert bm.length(3) == 16 and bm.num_free() == 0
    bm.preempt(1)
    assert sorted(bm.free) == [0, 1, 2] and bm.free[-1] == 2     # released first to last


def random_ops(bm, rng, steps, content=None, max_seqs=12):
    """Random adds, appends, forks and frees; `content` (slot -> token tag) tracks the KV
    data: appends write their tag, copy-on-write pairs copy the whole block. Returns the
    per-sequence token histories."""
    B = bm.block_size
    hist = {}
    next_id = 0
    for _ in range(steps):
        op = rng.integers(0, 10)
        live = sorted(hist)
        if op <= 2 or not live:
            n = int(rng.integers(0, 3 * B))
            try:
                slots = bm.add_sequence(next_id, n)
            except NoSpace:
                continue
            tags = [(next_id, t) for t in range(n)]
            if content is not None:
                for s, tag in zip(slots, tags):
                    content[s] = tag
            hist[next_id] = tags
            next_id += 1
        elif op <= 6:
            s = live[rng.integers(0, len(live))]
            try:
                slot, cow = bm.append_token(s)
            except NoSpace:
                continue
            if content is not None:
                if cow is not None:
                    for r in range(B):
                        if cow[0] * B + r in content:
                            content[cow[1] * B + r] = content[cow[0] * B + r]
                content[slot] = (s, len(hist[s]))
            hist[s] = hist[s] + [(s, len(hist[s]))]
        elif op <= 7 and len(live) < max_seqs:
            s = live[rng.integers(0, len(live))]
            bm.fork(s, next_id)
            hist[next_id] = list(hist[s])
            next_id += 1
        else:
            s = live[rng.integers(0, len(live))]
            bm.free_sequence(s)
            del hist[s]
    return hist


def check_invariants(bm, hist, content=None):
    B = bm.block_size
    held = {}
    for s in hist:
        tab = bm.table(s)
        assert len(tab) == -(-bm.length(s) // B) and bm.length(s) == len(hist[s])
        for b in tab:
            held[b] = held.get(b, 0) + 1
    for b in range(bm.num_blocks):
        assert bm.ref[b] == held.get(b, 0)
    assert sorted(bm.free) == sorted(b for b in range(bm.num_blocks) if b not in held)
    assert len(set(bm.free)) == len(bm.free)
    if content is not None:
        for s, h in hist.items():
            tab = bm.table(s)
            got = [content[tab[t // B] * B + t % B] for t in range(len(h))]
            assert got == h, f"sequence {s} reads back a wrong history"


@pytest.mark.parametrize("seed", range(6))
def test_random_ops_invariants_and_content(seed):
    rng = np.random.default_rng(seed)
    bm = OracleBlockManager(int(rng.integers(4, 40)))
    content = {}
    hist = random_ops(bm, rng, 400, content)
    check_invariants(bm, hist, content)
    for s in list(hist):
        bm.free_sequence(s)
    assert bm.num_free() == bm.num_blocks and not any(bm.ref)


def test_capacity_program_figures():
    """The pages' program: requests of 100 + Exp(400) tokens (capped at 4096) admitted
    until the 1M-token pool is full: about 8x the reserve-the-maximum count, about 1.5%
    lost to rounding, at most 15 tokens per request."""
    g = json.load(open(GOLDEN))
    B, cap, maxtok = g["block_size"], g["capacity_tokens"], g["max_tokens"]
    for seed in range(3):
        rng = np.random.default_rng(seed)
        L = np.minimum(maxtok, 100 + np.floor(rng.exponential(400.0, g["requests"])).astype(np.int64))
        bm = OracleBlockManager(cap // B, B)
        admitted = 0
        for i, n in enumerate(L):
            try:
                bm.add_sequence(i, int(n))
            except NoSpace:
                break
            admitted += 1
        used = (bm.num_blocks - bm.num_free()) * B
        waste = 100.0 * (used - L[:admitted].sum()) / used
        assert abs(admitted / (cap // maxtok) - g["printed"]["improvement_value"]) <= 0.5
        assert abs(waste - g["printed"]["rounding_waste_pct"]) <= 0.3
        assert all(len(bm.table(i)) * B - bm.length(i) <= 15 for i in range(admitted))


class _NoCopyOnWrite(OracleBlockManager):
    def append_token(self, seq):
        t = self.lens[seq]
        if t % self.block_size == 0:
            if not self.free:
                raise NoSpace()
            self.tables[seq].append(self._take())
        self.lens[seq] = t + 1
        return self._slot(seq, t), None


class _ForkWithoutRefs(OracleBlockManager):
    def fork(self, parent, child):
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]


@pytest.mark.parametrize("cls", [_NoCopyOnWrite, _ForkWithoutRefs])
def test_planted_mistakes_are_caught(cls):
    caught = False
    for seed in range(6):
        rng = np.random.default_rng(seed)
        bm = cls(int(rng.integers(4, 40)))
        content = {}
        try:
            hist = random_ops(bm, rng, 400, content)
            check_invariants(bm, hist, content)
        except (AssertionError, KeyError, IndexError, ValueError):
            caught = True
            break
    assert caught, f"{cls.__name__} passed every pin"
