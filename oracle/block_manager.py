"""Plain-Python model of the host block manager -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module.  The product's block manager is the
C++ one in libpa (``include/pa_block_manager.h``); the two share no code and
are compared operation by operation on seeded random workloads.

What it models (the pages' description of the allocator around the kernel):

* "What problem does PagedAttention solve, and what is continuous
  batching?" (datarekha), section "How PagedAttention works": KV lives in
  fixed-size blocks; a per-request block table maps logical block to
  physical block; the allocator can take any free block; the last, partly
  filled block wastes at most the rest of one block; candidates with an
  identical prefix reference the same blocks, and copy-on-write gives a
  diverging candidate a private block; prefix caching uses the same idea.
* same page, "A concrete memory example": when a request finishes, its
  blocks return to the pool immediately.
* same page, "A failure mode you can diagnose": the free KV-block count is
  what decides whether another request fits.
* "Continuous Batching & Paged Attention" (topicspectrum), section "Paged
  attention borrows a trick from operating systems": a growing request
  attaches another block; a finished one returns its blocks for reuse.
* "PagedAttention & Continuous Batching" (ai-ml-animation-academy), section
  "If you remember three things": shared prefixes are shared blocks, which
  is prefix caching.

The pages fix no allocation order, so the model fixes one (the C++ manager
follows the same rules, which is what makes the comparison exact):

* free blocks form a FIFO queue, initially in the order given at creation;
  a freed block joins the back;
* a full block is registered in the prefix cache under its content key,
  (key of the previous block, the block's token ids); a registered block
  whose last user goes away stays cached and joins a least-recently-freed
  list instead of the queue; allocation takes the queue first, then evicts
  the least recently freed cached block;
* a sequence created from a prompt reuses the cached block of every full
  prompt block whose key is registered, stopping at the first miss; its
  other tokens get fresh slots;
* appending a token to a block shared with another sequence first gives the
  appending sequence a private copy (one (src, dst) pair for the copy
  kernel);
* an operation that cannot get the blocks it needs changes nothing.
"""
import copy
from collections import OrderedDict, deque


class NoBlocks(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, free_order=None):
        self.nb, self.bs = int(num_blocks), int(block_size)
        order = list(range(self.nb)) if free_order is None else [int(x) for x in free_order]
        assert sorted(order) == list(range(self.nb))
        self.free = deque(order)
        self.ref = [0] * self.nb
        self.key_of = [None] * self.nb        # registered content key of a block
        self.cache = {}                        # content key -> block
        self.evictable = OrderedDict()         # cached blocks nobody uses, oldest first
        self.seqs = {}                         # id -> dict(blocks, len, tokens, last_key)

    # ---- pool
    def num_free(self):
        return len(self.free) + len(self.evictable)

    def _take(self):
        if self.free:
            b = self.free.popleft()
        elif self.evictable:
            b, _ = self.evictable.popitem(last=False)
            del self.cache[self.key_of[b]]
            self.key_of[b] = None
        else:
            raise NoBlocks()
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            if self.key_of[b] is not None:
                self.evictable[b] = True
            else:
                self.free.append(b)

    def _use_cached(self, b):
        if self.ref[b] == 0:
            del self.evictable[b]
        self.ref[b] += 1

    # ---- sequences
    def _register_if_full(self, seq):
        """After a token lands: a block that just filled joins the cache."""
        if seq["len"] % self.bs != 0:
            return
        blk = seq["blocks"][-1]
        key = (seq["last_key"], tuple(seq["tokens"]))
        seq["last_key"] = key
        seq["tokens"] = []
        if key not in self.cache and self.key_of[blk] is None:
            self.cache[key] = blk
            self.key_of[blk] = key

    def add_sequence(self, sid, prompt):
        """Returns (number of prompt tokens found cached, slots of the others)."""
        assert sid not in self.seqs
        prompt = [int(t) for t in prompt]
        bs = self.bs
        # cached prefix: whole blocks, stopping at the first miss
        hits, key = [], None
        for j in range(len(prompt) // bs):
            k = (key, tuple(prompt[j * bs:(j + 1) * bs]))
            if k not in self.cache:
                break
            hits.append(self.cache[k])
            key = k
        n_cached = len(hits) * bs
        need = -(-len(prompt) // bs) - len(hits)
        revive = sum(1 for b in hits if self.ref[b] == 0)
        if need > self.num_free() - revive:
            raise NoBlocks()
        for b in hits:
            self._use_cached(b)
        seq = {"blocks": list(hits), "len": n_cached, "tokens": [], "last_key": key}
        self.seqs[sid] = seq
        slots = [-1] * n_cached
        for t in prompt[n_cached:]:
            if seq["len"] % bs == 0:
                seq["blocks"].append(self._take())
            slots.append(seq["blocks"][-1] * bs + seq["len"] % bs)
            seq["tokens"].append(t)
            seq["len"] += 1
            self._register_if_full(seq)
        return n_cached, slots

    def append(self, sid, tokens):
        """Returns (slots of the new tokens, copy-on-write pairs)."""
        seq = self.seqs[sid]
        bs = self.bs
        tokens = [int(t) for t in tokens]
        # blocks needed: a private copy of a shared partial block, plus new ones
        need = 0
        if tokens and seq["len"] % bs != 0 and self.ref[seq["blocks"][-1]] > 1:
            need += 1
        need += -(-(seq["len"] + len(tokens)) // bs) - (-(-seq["len"] // bs))
        if need > self.num_free():
            raise NoBlocks()
        slots, cow = [], []
        for t in tokens:
            if seq["len"] % bs == 0:
                seq["blocks"].append(self._take())
            elif self.ref[seq["blocks"][-1]] > 1:
                src = seq["blocks"][-1]
                dst = self._take()
                self._release(src)
                seq["blocks"][-1] = dst
                cow.append((src, dst))
            slots.append(seq["blocks"][-1] * bs + seq["len"] % bs)
            seq["tokens"].append(t)
            seq["len"] += 1
            self._register_if_full(seq)
        return slots, cow

    def append_batch(self, sids, tokens):
        """One token for each sequence, in order, as single appends would do
        it; if any of them runs out of blocks, the state before the step is
        restored and NoBlocks raised.  Returns (slots, copy-on-write pairs)."""
        sids = [int(s) for s in sids]
        assert len(set(sids)) == len(sids) and all(s in self.seqs for s in sids)
        saved = copy.deepcopy(self.__dict__)
        slots, cow = [], []
        try:
            for sid, t in zip(sids, tokens):
                s, c = self.append(sid, [t])
                slots += s
                cow += c
        except NoBlocks:
            self.__dict__.clear()
            self.__dict__.update(saved)
            raise
        return slots, cow

    def fork(self, parent, child):
        assert child not in self.seqs
        p = self.seqs[parent]
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs[child] = {"blocks": list(p["blocks"]), "len": p["len"],
                            "tokens": list(p["tokens"]), "last_key": p["last_key"]}

    def free_sequence(self, sid):
        seq = self.seqs.pop(sid)
        for b in seq["blocks"]:
            self._release(b)

    def table(self, sid):
        return list(self.seqs[sid]["blocks"])

    def length(self, sid):
        return self.seqs[sid]["len"]
