"""Reference model of the paged KV block allocator (test infrastructure).

Only the test suite may import this module. It is the plain, slow statement
of what the library's allocator must do, in Python lists and dicts, and it
shares no code with the library.

What it follows (tiniestgpt notes):

* "PagedAttention: why it is needed": the cache is a pool of fixed-size
  physical blocks; a sequence's block table maps its logical blocks to
  physical ones; blocks are taken on demand and go back to the pool when the
  sequence ends.
* "Prefix Caching": only complete blocks are cached, under the chained hash
  h_i = H(h_{i-1}, tokens of block i); a request whose leading blocks hit
  needs no forward pass over them, only over the tokens after them.

Readings where the notes leave a choice open (the library makes the same ones):

* H is 64-bit FNV-1a over the parent hash (8 bytes, little-endian) followed
  by the block's token ids (4 bytes each, little-endian, two's complement);
  the first block's parent is 0.
* Matching runs only while a sequence consists of hit blocks (from its
  start), stops at the first miss, and never covers the block that holds the
  call's last token: that token is computed so that the step has its logits.
* A block that fills is registered under its hash unless another block
  already holds that hash.
* Free blocks wait in one queue. A sequence's blocks are released last
  logical block first; a released block with a registered hash joins the
  back of the queue (it stays findable until it is reused), one without
  joins the front. A fresh block is taken from the front, and its old
  registration, if any, is dropped. A hit on a free block takes it out of
  the queue.
* A call either succeeds whole or changes nothing.
* Positions whose keys and values are already cached get slot id -1, so the
  KV append skips them.
* A ring sequence (Lab 5, "Ring KV Cache", for window layers) takes blocks
  until it holds R of them; position t then lives in its block
  (t / block_size) mod R, i.e. slot t mod (R * block_size), overwriting the
  token R * block_size positions earlier. Its blocks are rewritten, so it
  never registers or matches a prefix. A position that a later token of the
  same call overwrites gets slot id -1 (one write per slot and call).
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1

# Planted mistakes for the mutant tests (0: none). 1: hash without the parent;
# 2: the block holding the last token may hit; 3: partial blocks registered;
# 4: freed blocks all join the back of the queue.
MUTANT = 0


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    """64-bit FNV-1a: per byte, xor it in, then multiply by the FNV prime mod 2^64."""
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & _MASK64
    return h


def block_hash(parent: int, tokens: Sequence[int]) -> int:
    if MUTANT == 1:
        parent = 0
    data = parent.to_bytes(8, "little") + b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


class AllocError(RuntimeError):
    pass


class _Seq:
    def __init__(self):
        self.blocks: List[int] = []
        self.length = 0
        self.parent = 0            # hash of the last complete block (0 before the first)
        self.tail: List[int] = []  # token ids of the incomplete last block
        self.hashable = True       # every token so far came with its id
        self.matching = True       # every block so far was a prefix hit
        self.ring = 0              # > 0: a ring of this many blocks


class RefAllocator:
    def __init__(self, num_blocks: int, block_size: int = 16, prefix_cache: bool = True):
        if num_blocks < 1 or block_size < 1:
            raise AllocError("bad sizes")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.prefix_cache = prefix_cache
        self.free: List[int] = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.hash_of: List[Optional[int]] = [None] * num_blocks
        self.cached: Dict[int, int] = {}
        self.seqs: Dict[int, _Seq] = {}
        self.queried = 0
        self.hits = 0

    # -- queries -------------------------------------------------------------------------------

    def num_free(self) -> int:
        return len(self.free)

    def seq_len(self, sid: int) -> int:
        return self.seqs[sid].length

    def blocks(self, sid: int) -> List[int]:
        return list(self.seqs[sid].blocks)

    def block_table(self, sids: Sequence[int], max_blocks: int) -> Tuple[List[List[int]], List[int]]:
        table, lens = [], []
        for sid in sids:
            s = self.seqs[sid]
            if len(s.blocks) > max_blocks:
                raise AllocError("max_blocks too small")
            table.append(s.blocks + [0] * (max_blocks - len(s.blocks)))
            lens.append(s.length)
        return table, lens

    # -- updates -------------------------------------------------------------------------------

    def add(self, sid: int, ring_blocks: int = 0) -> None:
        if sid in self.seqs:
            raise AllocError("sequence exists")
        if ring_blocks < 0:
            raise AllocError("bad ring size")
        s = _Seq()
        if ring_blocks:
            s.ring = ring_blocks
            s.hashable = False
            s.matching = False
        self.seqs[sid] = s

    def append(self, sid: int, n: int, tokens: Optional[Sequence[int]] = None) -> Tuple[List[int], int]:
        """Grow sequence `sid` by n tokens. Returns (slot id per token, -1 if cached; cached count)."""
        if sid not in self.seqs:
            raise AllocError("no such sequence")
        if n < 0 or (tokens is not None and len(tokens) != n):
            raise AllocError("bad token count")
        s = self.seqs[sid]
        bs = self.bs

        # Plan: leading full blocks that hit the cache.
        hits: List[Tuple[int, int]] = []
        queried = 0
        if (self.prefix_cache and tokens is not None and s.hashable and s.matching and s.length % bs == 0 and n > 0):
            may_hit = n // bs if MUTANT == 2 else (n - 1) // bs
            parent = s.parent
            for i in range(may_hit):
                h = block_hash(parent, tokens[i * bs:(i + 1) * bs])
                queried += 1
                if h not in self.cached:
                    break
                hits.append((self.cached[h], h))
                parent = h
        cached_tokens = len(hits) * bs
        total_blocks = -(-(s.length + n) // bs)
        if s.ring:
            total_blocks = min(total_blocks, s.ring)
        fresh = total_blocks - len(s.blocks) - len(hits)
        from_queue = fresh + sum(1 for b, _ in hits if self.ref[b] == 0)
        if from_queue > len(self.free):
            raise AllocError("out of blocks")

        # Commit.
        self.queried += queried
        self.hits += len(hits)
        slots: List[int] = []
        for b, h in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            s.blocks.append(b)
            s.parent = h
            s.length += bs
            slots.extend([-1] * bs)
        if tokens is None and n > 0:
            s.hashable = False
        if n > cached_tokens:
            s.matching = False
        final = s.length + (n - cached_tokens)
        for i in range(cached_tokens, n):
            pos = s.length
            entry = (pos // bs) % s.ring if s.ring else pos // bs
            if entry == len(s.blocks):
                b = self.free.pop(0)
                if self.hash_of[b] is not None:
                    del self.cached[self.hash_of[b]]
                    self.hash_of[b] = None
                self.ref[b] = 1
                s.blocks.append(b)
            overwritten = s.ring and pos < final - s.ring * bs
            slots.append(-1 if overwritten else s.blocks[entry] * bs + pos % bs)
            s.length += 1
            if s.hashable:
                s.tail.append(int(tokens[i]))
            full = s.length % bs == 0
            if self.prefix_cache and s.hashable and (full or (MUTANT == 3 and i == n - 1)):
                h = block_hash(s.parent, s.tail)
                b = s.blocks[-1]
                if h not in self.cached and self.hash_of[b] is None:
                    self.cached[h] = b
                    self.hash_of[b] = h
                if full:
                    s.parent = h
            if full:
                s.tail = []
        return slots, cached_tokens

    def release(self, sid: int) -> None:
        """The sequence ends: its blocks go back (last logical block first)."""
        if sid not in self.seqs:
            raise AllocError("no such sequence")
        s = self.seqs.pop(sid)
        for b in reversed(s.blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.hash_of[b] is not None or MUTANT == 4:
                    self.free.append(b)
                else:
                    self.free.insert(0, b)
