"""Plain model of the paged-KV block manager (the allocator in front of the pool).

TEST INFRASTRUCTURE.  Only the tests may import this module; the library never
does.  It shares no code with the C++ block manager: it is the specification,
written as directly as the pages state it, with Python lists and dicts and no
attention to speed.

What it follows (cited by title and section):

* [P3] "LLM 推理优化：KV Cache、PagedAttention 与量化" (blog.tanteng.space),
  §2.2: the cache is cut into fixed 16-token blocks and a per-sequence block
  table maps logical to physical blocks.
  §2.3 (1) block scheduling: a sequence takes a block from the fixed-capacity
  physical pool when it writes into it (on demand); when a sequence ends its
  blocks go back to the pool at once; the pool keeps counts of unreferenced
  blocks and an LRU order; a full pool is an error the scheduler must handle
  (it preempts).
  §2.3 (2) copy-on-write: a fork copies the block table only, the physical
  blocks are shared; a block is copied, and only that sequence's table entry
  changed, when a sequence writes into a block it shares.
  §2.3 (3) prefix sharing: identical prefixes are found by hashing block
  contents and several tables then point at the same physical blocks.
* [P4] "大模型推理加速与显存黑科技 (Inference Acceleration & KV Cache)"
  (ialgorithm.me), §3.2: memory is taken on demand, as much as is used.

Policy (the pages leave the choice of block open; these readings make every
result unique, so the C++ manager can be compared with this model exactly):

* Free blocks form a stack.  A fresh pool hands out 0, 1, 2, ...; a released
  block is pushed and is the next one handed out.
* A full block whose content is registered (see below) is not pushed when its
  last reference goes: it becomes *cached* -- unreferenced, still valid, at the
  most-recent end of an LRU list.  When the stack is empty the least-recently
  released cached block is evicted (its registration dropped) and handed out.
* Releasing a sequence walks its table from the last block to the first, so
  the first blocks of a prefix end up most recent and are evicted last.
* Content identity of a full block is the whole token prefix up to its end (the
  K/V of a token depend on every token before it).  Here the key *is* that
  prefix; the library keys a chained hash of it.
* Blocks hold 16 tokens (the pages' default) or 8 (the variant of §2.2); the
  model takes either.
* A lookup never covers the last prompt token: at most (n - 1) // bs full
  blocks are matched, so at least one prompt token is computed by the model
  (its logits are needed).
* The first token of an append may land in a partially filled block that other
  tables share: that block is copied (one copy per append at most) -- later
  tokens of the same append land in blocks the sequence owns.
* An append that needs more blocks than are free plus cached fails and changes
  nothing (pool exhausted).
"""
from __future__ import annotations

from collections import OrderedDict

BLOCK_SIZE = 16


class PoolExhausted(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        assert num_blocks > 0 and block_size in (8, 16)
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = list(range(num_blocks - 1, -1, -1))  # stack: pop() gives 0 first
        self.ref = [0] * num_blocks
        self.key_of = {}          # block -> token prefix tuple it holds (registered blocks)
        self.block_of = {}        # token prefix tuple -> block
        self.cached = OrderedDict()  # unreferenced registered blocks, oldest first
        self.tables = {}          # seq -> [physical ids]
        self.lens = {}            # seq -> context length
        self.tokens = {}          # seq -> list of token ids, or None when not hashing
        self.swapped = {}         # seq -> (length, tokens) while swapped out

    # ----------------------------------------------------------------- helpers
    def available(self) -> int:
        return len(self.free) + len(self.cached)

    def _take(self) -> int:
        if self.free:
            return self.free.pop()
        if self.cached:
            b, _ = self.cached.popitem(last=False)   # least recently released
            del self.block_of[self.key_of.pop(b)]
            return b
        raise PoolExhausted()

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            if b in self.key_of:
                self.cached[b] = True           # most recent end
            else:
                self.free.append(b)

    # --------------------------------------------------------------- sequences
    def add_seq(self, seq: int, hashing: bool = True) -> None:
        assert seq not in self.tables and seq not in self.swapped
        self.tables[seq] = []
        self.lens[seq] = 0
        self.tokens[seq] = [] if hashing else None

    def match_prefix(self, seq: int, prompt) -> int:
        """Share the registered full blocks that begin ``prompt``; returns the number
        of tokens now cached for ``seq`` (a multiple of 16)."""
        assert self.lens[seq] == 0 and self.tokens[seq] is not None
        prompt = list(prompt)
        n_blocks = max(len(prompt) - 1, 0) // self.bs
        for i in range(n_blocks):
            key = tuple(prompt[: (i + 1) * self.bs])
            b = self.block_of.get(key)
            if b is None:
                break
            if self.ref[b] == 0:
                del self.cached[b]
            self.ref[b] += 1
            self.tables[seq].append(b)
            self.lens[seq] += self.bs
            self.tokens[seq].extend(prompt[i * self.bs:(i + 1) * self.bs])
        return self.lens[seq]

    def blocks_needed(self, seq: int, n: int) -> int:
        L = self.lens[seq]
        new = -(-(L + n) // self.bs) - (-(-L // self.bs))
        cow = 1 if (n > 0 and L % self.bs != 0 and self.ref[self.tables[seq][-1]] > 1) else 0
        return new + cow

    def append(self, seq: int, n: int, token_ids=None):
        """Slots for ``n`` new tokens of ``seq``; returns (slots, copy) with copy =
        (src, dst) of a copy-on-write or None.  Raises PoolExhausted (no change)."""
        if self.blocks_needed(seq, n) > self.available():
            raise PoolExhausted()
        table = self.tables[seq]
        toks = self.tokens[seq]
        if token_ids is None and toks is not None:
            self.tokens[seq] = toks = None      # content unknown from here on: stop hashing
        slots, copy = [], None
        for i in range(n):
            t = self.lens[seq]
            if t % self.bs == 0:
                b = self._take()
                self.ref[b] = 1
                table.append(b)
            elif i == 0 and self.ref[table[-1]] > 1:
                src = table[-1]
                dst = self._take()
                self.ref[dst] = 1
                self.ref[src] -= 1              # still referenced by another table
                table[-1] = dst
                copy = (src, dst)
            slots.append(table[t // self.bs] * self.bs + t % self.bs)
            self.lens[seq] = t + 1
            if toks is not None:
                toks.append(int(token_ids[i]))
                if (t + 1) % self.bs == 0:
                    key = tuple(toks)
                    b = table[t // self.bs]
                    if key not in self.block_of and b not in self.key_of:
                        self.block_of[key] = b
                        self.key_of[b] = key
        return slots, copy

    def fork(self, parent: int, child: int) -> None:
        assert child not in self.tables and child not in self.swapped
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        toks = self.tokens[parent]
        self.tokens[child] = None if toks is None else list(toks)
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        if seq in self.swapped:          # holds no blocks: just forget it
            del self.swapped[seq]
            return
        for b in reversed(self.tables.pop(seq)):
            self._release(b)
        del self.lens[seq]
        del self.tokens[seq]

    # -------------------------------------------------------------- preemption
    def swap_out(self, seq: int):
        """Preemption ([P3] §2.3 (1): a full pool swaps a request's blocks out to the
        host): the sequence gives back its blocks as ``free_seq`` does and keeps its
        length and token history.  Returns its table before release -- the blocks
        whose contents the caller copies out, in logical order."""
        table = list(self.tables[seq])
        L, toks = self.lens[seq], self.tokens[seq]
        self.free_seq(seq)
        self.swapped[seq] = (L, toks)
        return table, L

    def swap_in(self, seq: int):
        """Bring a swapped-out sequence back: ceil(L / 16) fresh blocks, all or
        nothing; returns its new table (where the caller copies the contents back).
        The fresh blocks are not registered for prefix sharing."""
        L, toks = self.swapped[seq]
        need = -(-L // self.bs)
        if need > self.available():
            raise PoolExhausted()
        del self.swapped[seq]
        table = []
        for _ in range(need):
            b = self._take()
            self.ref[b] = 1
            table.append(b)
        self.tables[seq] = table
        self.lens[seq] = L
        self.tokens[seq] = toks
        return list(table)

    # ------------------------------------------------------------------ views
    def table(self, seq: int):
        return list(self.tables[seq])

    def stats(self):
        used = sum(1 for r in self.ref if r > 0)
        return {"free": len(self.free), "cached": len(self.cached), "used": used,
                "seqs": len(self.tables)}


def append_step(model: BlockManagerModel, seqs, token_ids=None):
    """One decode step: one new token for each of ``seqs`` (distinct ids), all or
    nothing.  The blocks the step needs are counted before anything changes (a
    copy-on-write that a later sequence of the same step would make unnecessary
    still counts); then the sequences are appended in order.  Returns (slots,
    copies)."""
    seqs = list(seqs)
    assert len(set(seqs)) == len(seqs)
    need = sum(model.blocks_needed(s, 1) for s in seqs)
    if need > model.available():
        raise PoolExhausted()
    slots, copies = [], []
    for i, s in enumerate(seqs):
        sl, cp = model.append(s, 1, None if token_ids is None else [token_ids[i]])
        slots.extend(sl)
        if cp is not None:
            copies.append(cp)
    return slots, copies


def sort_longest_first(model: BlockManagerModel, seqs):
    """The batch ordered by context length, longest first; equal lengths keep
    their order."""
    return sorted(seqs, key=lambda s: -model.lens[s])


def common_prefix(model: BlockManagerModel, seqs):
    """Leading table entries every sequence of the batch shares (the same
    physical blocks), capped at the full blocks every context covers."""
    seqs = list(seqs)
    if not seqs:
        return 0
    tables = [model.tables[s] for s in seqs]
    k = min(len(tables[0]), min(model.lens[s] for s in seqs) // model.bs)
    for t in tables[1:]:
        j = 0
        while j < k and j < len(t) and t[j] == tables[0][j]:
            j += 1
        k = j
    return k
