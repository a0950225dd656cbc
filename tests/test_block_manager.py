"""Block manager: the plain model (``oracle/block_manager.py``) pinned against the
pages and against an independent content simulation, then the C++ manager of
``libpa.so`` compared with the model operation by operation (bit-exact: every
slot, copy, table, reference count and error).  Host-only: no GPU is used.

Pins of the model:
* the copy-on-write figure of §2.3 (2) of the blog.tanteng.space page (block #7
  shared by two beams, the writer's copy lands in #15) -- tests/golden/page3_cow.json;
* the beam-search saving of the same section (4 beams of a 1024-token sequence
  hold 1024 tokens plus a few new ones, not 4 x 1024);
* the over-reservation example of §3.1 of the ialgorithm.me page (500 and 800
  tokens used of 4K reservations) and its waste figures;
* prefix sharing (§2.3 (3)): requests with one system prompt share its blocks;
* random traces checked by a slot-content simulation written here: every live
  sequence must read back, through its table, exactly the tokens it wrote.
"""
import json
import os
import random

import numpy as np
import pytest

from oracle.block_manager import (BLOCK_SIZE, BlockManagerModel, PoolExhausted, append_step,
                                  common_prefix,
                                  sort_longest_first)
from paged_kv_cache_365_amd import pa
from paged_kv_cache_365_amd.block_manager import EXPORTS, BlockManager

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# an adapter giving the library the model's interface
# --------------------------------------------------------------------------
class Lib:
    def __init__(self, num_blocks, block_size=BLOCK_SIZE):
        self.bm = BlockManager(num_blocks, block_size)
        self.num_blocks = num_blocks

    def _call(self, fn, *a):
        try:
            return fn(*a)
        except pa.PAError as e:
            if e.status == pa.PA_ERR_NO_SPACE:
                raise PoolExhausted() from None
            raise

    def add_seq(self, seq, hashing=True):
        self.bm.add_seq(seq, hashing)

    def match_prefix(self, seq, prompt):
        return self.bm.match_prefix(seq, prompt)

    def append(self, seq, n, token_ids=None):
        slots, cp = self._call(self.bm.append, seq, n, token_ids)
        return [int(s) for s in slots], cp

    def append_step(self, seqs, token_ids=None):
        slots, copies = self._call(self.bm.append_step, seqs, token_ids)
        return [int(s) for s in slots], [tuple(int(x) for x in c) for c in copies]

    def fork(self, parent, child):
        self.bm.fork(parent, child)

    def free_seq(self, seq):
        self.bm.free_seq(seq)

    def swap_out(self, seq):
        t, L = self._call(self.bm.swap_out, seq)
        return [int(b) for b in t], L

    def swap_in(self, seq):
        return [int(b) for b in self._call(self.bm.swap_in, seq)]

    def table(self, seq):
        return [int(b) for b in self.bm.table(seq)[0]]

    def length(self, seq):
        return self.bm.table(seq)[1]

    def refs(self):
        return [self.bm.refcount(b) for b in range(self.num_blocks)]

    def stats(self):
        s = self.bm.stats()
        return {"free": s["free_blocks"], "cached": s["cached_blocks"], "used": s["used_blocks"],
                "seqs": s["num_seqs"]}


def model_append_step(m, seqs, token_ids=None):
    return append_step(m, seqs, token_ids)


# --------------------------------------------------------------------------
# slot-content simulation (independent of both managers)
# --------------------------------------------------------------------------
class Contents:
    """What each slot holds: the token prefix of the token written there."""

    def __init__(self, bs=BLOCK_SIZE):
        self.bs = bs
        self.slot = {}
        self.history = {}   # seq -> token ids it has written or shared

    def write(self, seq, slots, toks):
        h = self.history.setdefault(seq, [])
        for s, t in zip(slots, toks):
            h.append(t)
            self.slot[s] = tuple(h)

    def copy_block(self, src, dst):
        bs = self.bs
        for o in range(bs):
            if src * bs + o in self.slot:
                self.slot[dst * bs + o] = self.slot[src * bs + o]
            else:
                self.slot.pop(dst * bs + o, None)

    def check(self, seq, table, length):
        h = self.history[seq]
        assert len(h) == length
        bs = self.bs
        for t in range(length):
            s = table[t // bs] * bs + t % bs
            assert self.slot.get(s) == tuple(h[: t + 1]), (seq, t, s)


# --------------------------------------------------------------------------
# pins of the model against the pages
# --------------------------------------------------------------------------
def _run_setup(m, steps):
    ids = {}
    for op in steps:
        if op[0] == "append":
            name, n = op[1], op[2]
            if name not in ids:
                ids[name] = len(ids)
                m.add_seq(ids[name], hashing=False)
            last = m.append(ids[name], n)
        elif op[0] == "free":
            m.free_seq(ids[op[1]])
        elif op[0] == "fork":
            ids[op[2]] = len(ids)
            m.fork(ids[op[1]], ids[op[2]])
    return ids, last


@pytest.mark.parametrize("impl", ["model", "lib"])
def test_cow_figure_golden(impl):
    g = json.load(open(os.path.join(GOLDEN, "page3_cow.json")))
    m = BlockManagerModel(g["num_blocks"]) if impl == "model" else Lib(g["num_blocks"])
    ids, (slots, copy) = _run_setup(m, g["setup"])
    exp = g["expected"]
    assert m.table(ids["P"]) == exp["table_P"]
    assert m.table(ids["B"]) == exp["table_B"]
    assert list(copy) == exp["copy"]
    refs = m.ref if impl == "model" else m.refs()
    assert refs[7] == exp["refcount_7"] and refs[15] == exp["refcount_15"]
    # the new token of beam B lands in its own copy, at offset 10
    assert slots == [15 * BLOCK_SIZE + 10]


@pytest.mark.parametrize("impl", ["model", "lib"])
@pytest.mark.parametrize("L", [1024, 1000])
def test_beam_search_sharing(impl, L):
    """Four beams forked from one L-token sequence, one new token each.  The pool
    holds the shared context once plus the beams' new blocks: ceil(L/16) + 4 when
    the context ends on a block boundary, ceil(L/16) + 3 otherwise (three beams
    copy the shared partial block; the last writer owns it by then)."""
    m = BlockManagerModel(400) if impl == "model" else Lib(400)
    m.add_seq(0, hashing=False)
    m.append(0, L)
    for c in (1, 2, 3):
        m.fork(0, c)
    copies = 0
    for s in (0, 1, 2, 3):
        _, cp = m.append(s, 1)
        copies += cp is not None
    nb = -(-L // 16)
    used = m.stats()["used"]
    if L % 16 == 0:
        assert used == nb + 4 and copies == 0
    else:
        assert used == nb + 3 and copies == 3
    # without sharing every beam would hold its own ceil((L+1)/16) blocks
    assert used < 4 * (-(-(L + 1) // 16)) * 0.3


@pytest.mark.parametrize("impl", ["model", "lib"])
def test_on_demand_waste_example(impl):
    """§3.1 of the ialgorithm.me page: requests using 500 and 800 tokens of 4K
    reservations waste 3500 and 3200 slots (the "60-80 %" of its text); taken on
    demand in 16-token blocks they hold 32 and 50 blocks and waste 12 slots."""
    m = BlockManagerModel(200) if impl == "model" else Lib(200)
    for s, n in ((0, 500), (1, 800)):
        m.add_seq(s, hashing=False)
        m.append(s, n)
    assert len(m.table(0)) == 32 and len(m.table(1)) == 50
    reserved_waste = ((4096 - 500) + (4096 - 800)) / (2 * 4096)
    paged_waste = (32 * 16 + 50 * 16 - 1300) / (82 * 16)
    assert 0.6 <= reserved_waste <= 0.85
    assert paged_waste < 0.04


def test_utilisation_of_the_7b_length_mix():
    """§2.2 of the blog.tanteng.space page: utilisation above 95 % with blocks; the
    7B-style length mix U[512, 4096] of 32 sequences."""
    rng = np.random.default_rng(1001)
    lens = rng.integers(512, 4097, size=32)
    m = BlockManagerModel(int(sum(-(-lens // 16))))
    for s, L in enumerate(lens):
        m.add_seq(s, hashing=False)
        m.append(s, int(L))
    used = m.stats()["used"]
    assert used == int(sum(-(-lens // 16)))
    assert lens.sum() / (used * 16) > 0.95
    assert lens.sum() / (32 * 4096) < 0.7     # a max-length reservation per request


@pytest.mark.parametrize("impl", ["model", "lib"])
def test_prefix_sharing_system_prompt(impl):
    """§2.3 (3): three requests with one 48-token system prompt point at the same
    three physical blocks and then append private blocks."""
    m = BlockManagerModel(64) if impl == "model" else Lib(64)
    sys_prompt = list(range(100, 148))
    tables = []
    for r in range(3):
        prompt = sys_prompt + [1000 + 10 * r + i for i in range(20)]
        m.add_seq(r)
        cached = m.match_prefix(r, prompt)
        assert cached == (0 if r == 0 else 48)
        m.append(r, len(prompt) - cached, prompt[cached:])
        tables.append(m.table(r))
    assert tables[0][:3] == tables[1][:3] == tables[2][:3]
    private = [b for t in tables for b in t[3:]]
    assert len(set(private)) == len(private) == 3 * 2
    assert set(private).isdisjoint(tables[0][:3])
    assert m.stats()["used"] == 3 + 6
    # a prompt of exactly 48 tokens shares only two blocks: its last token stays uncached
    m.add_seq(9)
    assert m.match_prefix(9, sys_prompt) == 32


@pytest.mark.parametrize("impl", ["model", "lib"])
def test_prefix_key_covers_the_whole_prefix(impl):
    """A block's K/V depend on every token before it, so equal block tokens after
    different prefixes must not be shared: prompts A+B+.. and C+B+.. share nothing,
    and a later C+B+.. prompt shares the blocks of the first C+B one."""
    m = BlockManagerModel(32) if impl == "model" else Lib(32)
    A, B, C = [7] * 16, list(range(16)), [9] * 16
    tables = []
    for s, prompt in enumerate([A + B + [1], C + B + [1], C + B + [2]]):
        m.add_seq(s)
        cached = m.match_prefix(s, prompt)
        assert cached == (32 if s == 2 else 0)
        m.append(s, len(prompt) - cached, prompt[cached:])
        tables.append(m.table(s))
    assert tables[2][:2] == tables[1][:2]
    assert not set(tables[1]) & set(tables[0])


def test_cached_blocks_survive_release_and_are_evicted_lru():
    m = BlockManagerModel(6)
    p = list(range(33))
    m.add_seq(0)
    m.append(0, 33, p)               # blocks 0, 1 (full, registered), 2 (partial)
    m.free_seq(0)                    # 2 -> free stack; 1, 0 -> cached (0 most recent)
    assert m.stats() == {"free": 4, "cached": 2, "used": 0, "seqs": 0}
    assert list(m.cached) == [1, 0]
    m.add_seq(1)
    assert m.match_prefix(1, p) == 32 and m.table(1) == [0, 1]
    m.free_seq(1)
    # exhaust the stack: the next take evicts the least recently released (1)
    m.add_seq(2, hashing=False)
    m.append(2, 4 * 16)
    assert m.table(2) == [2, 3, 4, 5]
    m.append(2, 1)
    assert m.table(2)[-1] == 1 and 1 not in m.key_of
    m.add_seq(3)
    assert m.match_prefix(3, p) == 16   # block 0 still cached, block 1 gone


@pytest.mark.parametrize("impl", ["model", "lib"])
def test_exhaustion_changes_nothing(impl):
    m = BlockManagerModel(4) if impl == "model" else Lib(4)
    m.add_seq(0, hashing=False)
    m.append(0, 40)                   # 3 blocks
    before = (m.table(0), m.stats())
    with pytest.raises(PoolExhausted):
        m.append(0, 40)               # needs 2 more, 1 left
    assert (m.table(0), m.stats()) == before
    m.fork(0, 1)
    m.add_seq(2, hashing=False)
    m.append(2, 16)                   # the last block
    with pytest.raises(PoolExhausted):   # copy-on-write of the shared partial block
        m.append(1, 1)
    step = model_append_step if impl == "model" else (lambda mm, s, t=None: mm.append_step(s, t))
    with pytest.raises(PoolExhausted):
        step(m, [0, 1])
    assert m.stats()["used"] == 4


# --------------------------------------------------------------------------
# random traces: the model against the content simulation, the library
# against the model
# --------------------------------------------------------------------------
def run_trace(seed, num_blocks, n_ops, impls, vocab=3, bs=BLOCK_SIZE):
    rnd = random.Random(seed)
    sims = [Contents(bs) for _ in impls]
    live, swapped, saved = [], [], {}
    next_id = 0
    sys_prompts = [[rnd.randrange(vocab) for _ in range(rnd.choice([16, 32, 40, 64]))]
                   for _ in range(3)]

    def both(fn):
        """Apply fn to every impl; all must return the same value or all raise
        PoolExhausted."""
        outs = []
        for impl in impls:
            try:
                outs.append(("ok", fn(impl)))
            except PoolExhausted:
                outs.append(("full", None))
        assert all(o == outs[0] for o in outs), outs
        return outs[0]

    for _ in range(n_ops):
        r = rnd.random()
        if r < 0.25 or not live:
            seq = next_id
            next_id += 1
            hashing = rnd.random() < 0.8
            prompt = (rnd.choice(sys_prompts) if rnd.random() < 0.7 else []) + \
                [rnd.randrange(vocab) for _ in range(rnd.randrange(1, 40))]
            for impl in impls:
                impl.add_seq(seq, hashing)
            cached = 0
            if hashing:
                _, cached = both(lambda m: m.match_prefix(seq, prompt))
            for sim in sims:
                sim.history[seq] = list(prompt[:cached])
            st, res = both(lambda m: m.append(seq, len(prompt) - cached,
                                              prompt[cached:] if hashing else None))
            if st == "full":
                for impl in impls:
                    impl.free_seq(seq)
                continue
            slots, cp = res
            assert cp is None
            for sim in sims:
                sim.write(seq, slots, prompt[cached:])
            live.append(seq)
        elif r < 0.55:
            seqs = rnd.sample(live, rnd.randint(1, len(live)))
            toks = [rnd.randrange(vocab) for _ in seqs]
            use_toks = rnd.random() < 0.9

            def step(m):
                t = toks if use_toks else None
                if isinstance(m, BlockManagerModel):
                    return model_append_step(m, seqs, t)
                return m.append_step(seqs, t)
            st, res = both(step)
            if st == "ok":
                slots, copies = res
                for sim in sims:
                    for src, dst in copies:
                        sim.copy_block(src, dst)
                    for s, slot, t in zip(seqs, slots, toks):
                        sim.write(s, [slot], [t])
        elif r < 0.65:
            parent = rnd.choice(live)
            child = next_id
            next_id += 1
            for impl in impls:
                impl.fork(parent, child)
            for sim in sims:
                sim.history[child] = list(sim.history[parent])
            live.append(child)
        elif r < 0.8:
            seq = live.pop(rnd.randrange(len(live)))
            for impl in impls:
                impl.free_seq(seq)
        elif r < 0.9:
            seq = live.pop(rnd.randrange(len(live)))
            _, (table, L) = both(lambda m: m.swap_out(seq))
            saved[seq] = [[sim.slot.get(b * bs + o) for b in table for o in range(bs)]
                          for sim in sims]
            swapped.append(seq)
        elif swapped:
            seq = swapped[0]
            st, table = both(lambda m: m.swap_in(seq))
            if st == "ok":
                swapped.pop(0)
                for sim, vals in zip(sims, saved.pop(seq)):
                    for i, v in enumerate(vals):
                        s = table[i // bs] * bs + i % bs
                        if v is None:
                            sim.slot.pop(s, None)
                        else:
                            sim.slot[s] = v
                live.append(seq)
        # invariants after every operation
        for impl, sim in zip(impls, sims):
            refs = impl.ref if isinstance(impl, BlockManagerModel) else impl.refs()
            count = [0] * num_blocks
            for s in live:
                t = impl.table(s)
                for b in t:
                    count[b] += 1
                L = impl.lens[s] if isinstance(impl, BlockManagerModel) else impl.length(s)
                sim.check(s, t, L)
            assert count == list(refs)
            st = impl.stats()
            assert st["free"] + st["cached"] + st["used"] == num_blocks
            assert st["seqs"] == len(live)
        if len(impls) == 2:
            a, b = impls
            assert a.ref == b.refs()
            assert a.stats() == b.stats()
            if live:
                batch = rnd.sample(live, len(live))
                assert sort_longest_first(a, batch) == b.bm.sort_longest_first(batch).tolist()
    return next_id


@pytest.mark.parametrize("seed", range(6))
def test_model_random_trace_contents(seed):
    """The model alone: every live sequence reads back what it wrote."""
    run_trace(seed, num_blocks=48, n_ops=300, impls=[BlockManagerModel(48)])


@pytest.mark.parametrize("seed", range(8))
def test_library_matches_model(seed):
    nb = [24, 48, 96, 200][seed % 4]
    run_trace(100 + seed, num_blocks=nb, n_ops=400, impls=[BlockManagerModel(nb), Lib(nb)])


@pytest.mark.parametrize("seed", range(4))
def test_eight_token_blocks_library_matches_model(seed):
    """The 8-token block variant: the same operation-by-operation equality and
    slot-content invariants, with blocks (and registered prefixes) of 8 tokens."""
    nb = [16, 40, 96, 150][seed]
    run_trace(300 + seed, num_blocks=nb, n_ops=400,
              impls=[BlockManagerModel(nb, 8), Lib(nb, 8)], bs=8)


def _eight_token_basics(impl):
    impl.add_seq(0)
    assert impl.append(0, 20, list(range(20)))[0][:9] == list(range(9))   # blocks 0, 1, 2
    impl.add_seq(1)
    assert impl.match_prefix(1, list(range(20))) == 16                    # two full blocks
    assert impl.table(1) == [0, 1]


def test_eight_token_blocks_basics():
    _eight_token_basics(BlockManagerModel(20, 8))


def test_eight_token_blocks_library():
    _eight_token_basics(Lib(20, 8))
    with pytest.raises(pa.PAError) as e:
        BlockManager(8, 12)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED


def test_library_errors():
    bm = BlockManager(8)
    bm.add_seq(1)
    for fn, args in [(bm.add_seq, (1,)), (bm.free_seq, (5,)), (bm.fork, (5, 6)), (bm.fork, (1, 1)),
                     (bm.append, (5, 1)), (bm.swap_in, (1,)), (bm.table, (7,))]:
        with pytest.raises(pa.PAError) as e:
            fn(*args)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
    with pytest.raises(pa.PAError):
        bm.append_step([1, 1])                      # duplicate ids
    bm.append(1, 20, list(range(20)))
    with pytest.raises(pa.PAError):
        bm.match_prefix(1, list(range(40)))         # not empty
    bm.add_seq(2, hashing=False)
    with pytest.raises(pa.PAError):
        bm.match_prefix(2, list(range(40)))         # not hashing
    with pytest.raises(pa.PAError):
        bm.fill_tables([1], 1)                      # two blocks do not fit in one
    tables, lens = bm.fill_tables([1, 2], 4)
    assert tables.tolist() == [[0, 1, -1, -1], [-1, -1, -1, -1]] and lens.tolist() == [20, 0]
    assert bm.refcount(-1) == -1 and bm.refcount(8) == -1
    assert bm.blocks_needed(1, 12) == 0 and bm.blocks_needed(1, 13) == 1
    assert bm.blocks_needed(99, 1) == -1
    with pytest.raises(pa.PAError):
        BlockManager(0)


def test_block_manager_exports():
    lib = pa.load()
    import re
    text = open(os.path.join(os.path.dirname(GOLDEN), "..", "include", "pa_block_manager.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(pa_bm_[a-z_]+)\s*\(", text))
    assert names == set(EXPORTS)
    for n in names:
        assert hasattr(lib, n)


def test_sort_longest_first():
    m = BlockManagerModel(64)
    for s, n in enumerate([5, 40, 17, 40, 1, 33]):
        m.add_seq(s, False)
        m.append(s, n)
    batch = [4, 3, 0, 1, 5, 2]
    assert sort_longest_first(m, batch) == [3, 1, 5, 2, 0, 4]   # 40, 40, 33, 17, 5, 1; ties keep order


def test_sort_longest_first_library():
    bm = BlockManager(64)
    for s, n in enumerate([5, 40, 17, 40, 1, 33]):
        bm.add_seq(s, False)
        bm.append(s, n)
    assert bm.sort_longest_first([4, 3, 0, 1, 5, 2]).tolist() == [3, 1, 5, 2, 0, 4]
    with pytest.raises(pa.PAError):
        bm.sort_longest_first([0, 99])


def _prefix_batch(impl, bs=16):
    """Four sequences behind one 83-token system prompt (5 full blocks + 3
    tokens) with 0, 40, 7 and 100 private tokens, each matched against the
    cached prompt blocks first; then a fork of sequence 0 (10) and an unrelated
    40-token sequence (11)."""
    prompt = list(range(1000, 1000 + 5 * bs + 3))
    for s, extra in enumerate([0, 40, 7, 100]):
        toks = prompt + [s] * extra
        impl.add_seq(s, True)
        impl.match_prefix(s, toks)
        t = impl.table(s)
        done = len(t[0] if isinstance(t, tuple) else t) * bs
        impl.append(s, len(toks) - done, toks[done:])
    impl.fork(0, 10)
    impl.add_seq(11, True)
    impl.append(11, 40, list(range(40)))


COMMON_PREFIX_CASES = [([0, 1, 2, 3], 5), ([1, 3], 5), ([2], 5), ([], 0), ([0, 10], 5), ([0, 1, 11], 0),
                       ([0, 11], 0), ([11], 2)]


def test_common_prefix_of_a_batch():
    """System-prompt sharing (§2.3 of the blog.tanteng.space page): sequences that
    matched the same prompt share its leading blocks; the batch's common prefix
    is those blocks, capped at the full blocks every context covers (a fork
    shares the partial sixth block too, but no context fills it); a sequence
    that shares nothing makes it 0."""
    m = BlockManagerModel(256)
    _prefix_batch(m)
    for batch, want in COMMON_PREFIX_CASES:
        assert common_prefix(m, batch) == want, batch
    assert m.tables[10] == m.tables[0] and len(m.tables[0]) == 6


def test_common_prefix_library_matches_model():
    bm = BlockManager(256)
    _prefix_batch(bm)
    for batch, want in COMMON_PREFIX_CASES:
        assert bm.common_prefix(batch) == want, batch
    # the tables pa_decode reads agree: the first 5 entries are equal
    tables, lens = bm.fill_tables([0, 1, 2, 3], 16)
    assert (tables[:, :5] == tables[0, :5]).all() and not (tables[:, 5] == tables[0, 5]).all()
    assert lens.min() >= 5 * 16
    with pytest.raises(pa.PAError):
        bm.common_prefix([0, 99])
