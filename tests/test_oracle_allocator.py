"""Pins for the allocator's reference model (oracle/allocator.py), CPU only.

Each check holds for the allocator's definition whatever the operation mix:
the published FNV-1a vectors; blocks taken exactly when a sequence crosses a
block boundary and slot ids inside its own blocks; every block back in the
pool once its sequences end; no block in two live tables unless it is a
prefix hit; reference counts equal table memberships; a hit only ever lands
on a block whose writer had exactly the requester's whole prefix (checked
from an outside record of which token went to which slot, not from the
model's own hash table); identical prompts hit, prompts that differ before
or inside a block do not, partial blocks never hit, the last token is always
computed; a failed call changes nothing.
"""

from __future__ import annotations

import copy
import json
import os

import numpy as np
import pytest

from oracle import allocator as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fnv1a64_vectors.json")
BS = 16


def test_fnv1a64_published_vectors():
    fx = json.load(open(GOLDEN))
    for v in fx["vectors"]:
        assert A.fnv1a64(v["ascii"].encode()) == int(v["fnv1a64"], 16), v


def test_on_demand_blocks_and_slots():
    al = A.RefAllocator(40, BS, prefix_cache=False)
    al.add(7)
    seen = []
    for pos in range(100):
        slots, cached = al.append(7, 1)
        assert cached == 0
        blocks = al.blocks(7)
        assert len(blocks) == pos // BS + 1                      # a block exactly at each boundary
        assert slots == [blocks[pos // BS] * BS + pos % BS]
        seen.append(slots[0])
    assert len(set(seen)) == 100
    assert al.num_free() == 40 - 7
    al.release(7)
    assert al.num_free() == 40 and sorted(al.free) == list(range(40))


def _state(al):
    return copy.deepcopy((al.free, al.ref, al.hash_of, al.cached,
                          {k: vars(s) for k, s in al.seqs.items()}, al.queried, al.hits))


def test_out_of_blocks_changes_nothing():
    al = A.RefAllocator(5, BS)
    al.add(1)
    al.append(1, 70, list(range(70)))                            # 5 blocks
    al.add(2)
    before = _state(al)
    with pytest.raises(A.AllocError):
        al.append(2, 1, [3])
    with pytest.raises(A.AllocError):
        al.append(1, 11, list(range(11)))                        # 70 + 11 > 80 slots
    assert _state(al) == before
    al.append(1, 10, list(range(10)))                            # exactly fills the pool
    assert al.num_free() == 0


def _check_invariants(al, live_written):
    member = [0] * al.num_blocks
    for s in al.seqs.values():
        assert len(s.blocks) == -(-s.length // BS)
        for b in s.blocks:
            member[b] += 1
    assert member == al.ref
    assert sorted(al.free) == [b for b in range(al.num_blocks) if al.ref[b] == 0]
    for h, b in al.cached.items():
        assert al.hash_of[b] == h
    # Positions written by live sequences: a (block, slot) is written by one of them only.
    owners = {}
    for sid, slots in live_written.items():
        for sl in slots:
            assert owners.setdefault(sl, sid) == sid


def _random_ops(al, rng, steps, vocab, track):
    """Random adds / prompt appends / decode appends / releases; checks hits from the outside."""
    writer_prefix = {}     # slot id -> the full token prefix (through that slot) of its writer
    history = {}           # seq -> its tokens
    written = {}           # seq -> slot ids it wrote
    next_id = 0
    for _ in range(steps):
        op = rng.random()
        if op < 0.25 or not al.seqs:
            sid = next_id
            next_id += 1
            al.add(sid)
            history[sid], written[sid] = [], []
            # A prompt from a few shared stems so that prefixes repeat.
            stem = [int(t) for t in np.random.default_rng(int(rng.integers(3))).integers(0, vocab, 64)]
            n = int(rng.integers(1, 70))
            toks = stem[:min(n, int(rng.integers(0, 65)))]
            toks += [int(t) for t in rng.integers(0, vocab, n - len(toks))]
        elif op < 0.85:
            sid = int(rng.choice(list(al.seqs)))
            n = int(rng.integers(1, 4))
            toks = [int(t) for t in rng.integers(0, vocab, n)]
        else:
            sid = int(rng.choice(list(al.seqs)))
            al.release(sid)
            written.pop(sid)
            history.pop(sid)
            if track:
                _check_invariants(al, written)
            continue
        try:
            slots, cached = al.append(sid, len(toks), toks)
        except A.AllocError:
            continue
        base = len(history[sid])
        assert slots[:cached] == [-1] * cached and all(s >= 0 for s in slots[cached:])
        assert cached % BS == 0 and cached < len(toks) + (1 if A.MUTANT == 2 else 0)
        blocks = al.blocks(sid)
        for j in range(cached):                   # a hit block holds what this prefix would write
            pos = base + j
            sl = blocks[pos // BS] * BS + pos % BS
            assert writer_prefix.get(sl) == tuple(history[sid] + toks[:j + 1]), "false prefix hit"
        for j in range(cached, len(toks)):
            writer_prefix[slots[j]] = tuple(history[sid] + toks[:j + 1])
            written[sid].append(slots[j])
        history[sid] += toks
        if track:
            _check_invariants(al, written)
    return al


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_operations_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    al = _random_ops(A.RefAllocator(48, BS), rng, 400, vocab=3, track=True)
    assert al.hits > 0                     # the stems make prefixes repeat


def test_random_operations_without_prefix_cache():
    rng = np.random.default_rng(9)
    al = _random_ops(A.RefAllocator(40, BS, prefix_cache=False), rng, 300, vocab=3, track=True)
    assert al.hits == 0 and al.queried == 0


def _prompt(al, sid, toks):
    al.add(sid)
    return al.append(sid, len(toks), toks)


def test_identical_prompts_share_full_blocks():
    al = A.RefAllocator(32, BS)
    p = list(range(100, 149))                  # 49 tokens: 3 full blocks + 1
    s1, c1 = _prompt(al, 1, p)
    s2, c2 = _prompt(al, 2, p)
    assert c1 == 0 and c2 == 48
    assert s2[:48] == [-1] * 48 and s2[48] >= 0
    assert al.blocks(2)[:3] == al.blocks(1)[:3] and al.blocks(2)[3] != al.blocks(1)[3]
    assert (al.queried, al.hits) == (1 + 3, 3)   # the first prompt looked up one block and missed


def test_last_token_is_always_computed():
    al = A.RefAllocator(32, BS)
    p = list(range(48))                        # exactly 3 blocks
    _prompt(al, 1, p)
    _, c = _prompt(al, 2, p)
    assert c == 32                             # the third block holds the last token


def test_chained_hash_needs_the_same_prefix():
    al = A.RefAllocator(32, BS)
    a = list(range(40))
    b = list(range(40))
    b[3] = 999                                 # differs in block 0, block 1 identical
    c = list(range(40))
    c[20] = 999                                # differs inside block 1
    _prompt(al, 1, a)
    assert _prompt(al, 2, b)[1] == 0
    assert _prompt(al, 3, c)[1] == 16
    # b's block 1 holds the same tokens as a's but after another block 0: a prompt equal to b
    # must find b's blocks, never a's.
    assert _prompt(al, 4, b)[1] == 32
    assert al.blocks(4)[:2] == al.blocks(2)[:2]


def test_partial_blocks_are_not_cached_until_full():
    a = list(range(40))                        # blocks 0, 1 full, block 2 holds 8 tokens
    ext = a + list(range(40, 49))
    al = A.RefAllocator(32, BS)
    _prompt(al, 1, a)
    assert _prompt(al, 2, ext)[1] == 32
    al = A.RefAllocator(32, BS)
    _prompt(al, 1, a)
    al.append(1, 8, list(range(40, 48)))       # sequence 1 fills its block 2 by decoding
    assert _prompt(al, 3, ext)[1] == 48


def test_released_prefix_stays_findable_and_plain_blocks_go_first():
    al = A.RefAllocator(6, BS)
    p = list(range(40))                        # 3 blocks: two registered, one partial
    _prompt(al, 1, p)
    b1 = al.blocks(1)
    al.release(1)
    assert al.free[0] == b1[2]                 # the partial block went to the front
    assert al.free[-2:] == [b1[1], b1[0]]      # registered blocks at the back, last block first
    al.add(2)
    al.append(2, 16, [7] * 16)                 # one fresh block: the plain one is reused
    assert al.blocks(2) == [b1[2]]
    _, c = _prompt(al, 3, p)
    assert c == 32 and al.blocks(3)[:2] == b1[:2]


def test_fresh_block_drops_its_old_registration():
    al = A.RefAllocator(3, BS)
    p = list(range(33))
    _prompt(al, 1, p[:32])                     # blocks 0, 1 registered
    al.release(1)
    al.add(2)
    al.append(2, 48, [5] * 48)                 # takes all three blocks
    al.release(2)
    _, c = _prompt(al, 3, p)
    assert c == 0                              # the old prefix was overwritten


def test_tokens_without_ids_are_never_registered():
    al = A.RefAllocator(8, BS)
    al.add(1)
    al.append(1, 32)                           # no ids
    assert not al.cached
    _, c = _prompt(al, 2, list(range(33)))
    assert c == 0


MUTANT_NAMES = {1: "hash without the parent", 2: "the last token's block may hit",
                3: "partial blocks registered", 4: "freed blocks all join the back"}


@pytest.mark.parametrize("mutant", sorted(MUTANT_NAMES))
def test_each_mutant_fails_a_pin(mutant):
    pins = [f for name, f in sorted(globals().items())
            if name.startswith("test_") and name != "test_each_mutant_fails_a_pin" and callable(f)]
    failed = []
    A.MUTANT = mutant
    try:
        for f in pins:
            args = {"seed": 0} if "seed" in f.__code__.co_varnames[:f.__code__.co_argcount] else {}
            try:
                f(**args)
            except (AssertionError, A.AllocError):
                failed.append(f.__name__)
    finally:
        A.MUTANT = 0
    assert failed, f"mutant {mutant} ({MUTANT_NAMES[mutant]}) passed every pin"


def test_ring_sequence_wraps_at_its_block_count():
    al = A.RefAllocator(10, BS)
    al.add(1, ring_blocks=3)
    slots, _ = al.append(1, 100, list(range(100)))
    blocks = al.blocks(1)
    assert len(blocks) == 3 and al.num_free() == 7                # never more than its ring
    for t in range(100):                                          # slot t mod 48; -1 if overwritten later
        want = blocks[(t // BS) % 3] * BS + t % BS if t >= 100 - 48 else -1
        assert slots[t] == want
    assert len(set(slots[-48:])) == 48                            # one write per slot and call
    assert not al.cached and al.queried == 0                       # rings never touch the prefix cache
    more, _ = al.append(1, 5, [1] * 5)
    assert more == [blocks[(t // BS) % 3] * BS + t % BS for t in range(100, 105)]
    table, lens = al.block_table([1], 3)
    assert table == [blocks] and lens == [105]
    al.release(1)
    assert al.num_free() == 10
