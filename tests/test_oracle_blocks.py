"""Pins of the block-allocator oracle (oracle/block_manager.py): the serving
lesson's exercise 3 (21 -> 7 -> 9 blocks), the serving lesson's paging trace
(323,568 paged slots for 322,055 live tokens), the waste bound, conservation
invariants of the reference counts on random traces, the free-list order of
the brunomaga post's PagedKVCache, out-of-blocks, and copy-on-write contents.
A last test plants mistakes and checks that a pin catches each."""

import json
import os

import numpy as np
import pytest

import oracle.block_manager as bm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_exercise3():
    g = _golden("serving_lesson_cow.json")
    n, T, bs = g["samples"], g["prompt_tokens"], g["block_size"]
    m = bm.BlockManager(64, bs)                       # unshared: every sample prefills
    for s in range(n):
        m.add(s)
        m.append_slots(s, T)
    ok = m.used_blocks() == g["blocks_unshared"]
    ok &= len(m.tables[0]) == g["blocks_per_prompt"] and T - (len(m.tables[0]) - 1) * bs == g["last_block_tokens"]
    m = bm.BlockManager(64, bs)                       # shared: one prefill, n - 1 forks
    m.add(0)
    m.append_slots(0, T)
    for s in range(1, n):
        m.fork(0, s)
    ok &= m.used_blocks() == g["blocks_shared"]
    ok &= all(m.ref[b] == g["shared_refcount"] for b in m.tables[0])
    last = m.tables[0][-1]
    for s in range(n):                                # each sample writes its first new token
        copies = m.append_slots(s, 1)
        ok &= len(copies) == g["copies_per_writer"][s]
        ok &= all(src == last for src, _ in copies)
        ok &= m.ref[last] == g["last_block_refcount_after_each_write"][s]
    ok &= m.used_blocks() == g["blocks_after_first_new_token"]
    return bool(ok)


def pin_paging_trace():
    p = _golden("serving_lesson_numbers.json")["paging"]
    live = np.random.default_rng(p["seed"]).integers(p["low"], p["high"], size=p["n"])
    m = bm.BlockManager(p["reserved"] // p["block"], p["block"])
    for i, n in enumerate(live.tolist()):
        m.add(i)
        m.append_slots(i, n)
    return (m.used_blocks() * p["block"] == p["paged"] and int(live.sum()) == p["live_sum"]
            and round(100 * live.sum() / (m.used_blocks() * p["block"]), 1) == p["used_share_paged_pct"])


def _random_trace(m, rng, steps=300, max_seqs=12):
    """Adds, forks, appends (one token or a chunk) and frees at random."""
    nxt = 0
    for _ in range(steps):
        live = list(m.tables)
        r = rng.random()
        try:
            if not live or (r < 0.15 and len(live) < max_seqs):
                m.add(nxt)
                nxt += 1
                m.append_slots(nxt - 1, int(rng.integers(1, 40)))
            elif r < 0.3 and len(live) < max_seqs:
                m.fork(int(rng.choice(live)), nxt)
                nxt += 1
            elif r < 0.4:
                m.free_seq(int(rng.choice(live)))
            else:
                m.append_slots(int(rng.choice(live)), int(rng.choice([1, 1, 1, 3, 17])))
        except bm.OutOfBlocks:
            m.free_seq(int(rng.choice(list(m.tables))))
        yield


def pin_invariants(seed=0, num_blocks=48, bs=4):
    rng = np.random.default_rng(seed)
    m = bm.BlockManager(num_blocks, bs)
    for _ in _random_trace(m, rng):
        held = {}
        for s, t in m.tables.items():
            if len(t) != -(-m.lengths[s] // bs):      # waste bound: ceil(len / bs) blocks
                return False
            for b in t:
                held[b] = held.get(b, 0) + 1
        if any(m.ref[b] != c for b, c in held.items()):
            return False
        if any(m.ref[b] != 0 for b in m.free) or len(set(m.free)) != len(m.free):
            return False
        if len(m.free) + len(held) != num_blocks:
            return False
    return True


def pin_free_list_order():
    """PagedKVCache: free_blocks = list(range(n)); append pops the last entry;
    free appends the table.  10 blocks of 4: A takes 9, 8, 7 for 9 tokens; B
    takes 6, 5 for 6 tokens; after A is freed the list ends 9, 8, 7, so C's
    first two blocks are 7 and 8."""
    m = bm.BlockManager(10, 4)
    m.add("A"); m.append_slots("A", 9)
    m.add("B"); m.append_slots("B", 6)
    ok = m.tables["A"] == [9, 8, 7] and m.tables["B"] == [6, 5]
    m.free_seq("A")
    ok &= m.free == [0, 1, 2, 3, 4, 9, 8, 7]
    m.add("C"); m.append_slots("C", 5)
    return bool(ok and m.tables["C"] == [7, 8])


def pin_out_of_blocks():
    m = bm.BlockManager(3, 4)
    m.add(0)
    m.append_slots(0, 10)                             # 3 blocks
    m.fork(0, 1)
    before = (list(m.free), list(m.ref), {k: list(v) for k, v in m.tables.items()}, dict(m.lengths))
    try:
        m.append_slots(1, 1)                          # needs a copy of the shared last block
        return False
    except bm.OutOfBlocks:
        pass
    after = (list(m.free), list(m.ref), {k: list(v) for k, v in m.tables.items()}, dict(m.lengths))
    return before == after


def pin_copy_contents(seed=1):
    """Data written through the tables after copy-on-write: every sequence
    reads back exactly its own tokens (a shadow copy per sequence)."""
    rng = np.random.default_rng(seed)
    bs, NB = 4, 40
    m = bm.BlockManager(NB, bs)
    pool = np.full((NB, bs), -1, np.int64)
    shadow = {}

    def write(seq, n):
        nonlocal pool
        start = m.lengths[seq]
        copies = m.append_slots(seq, n)
        pool = bm.copy_blocks([pool], copies)[0]
        for pos in range(start, start + n):
            tok = int(rng.integers(1 << 30))
            pool[m.tables[seq][pos // bs], pos % bs] = tok
            shadow[seq].append(tok)

    m.add(0); shadow[0] = []
    write(0, 10)
    for c in (1, 2, 3):
        m.fork(0, c)
        shadow[c] = list(shadow[0])
    for _ in range(30):
        s = int(rng.integers(4))
        write(s, int(rng.choice([1, 2, 5])))
    for s, toks in shadow.items():
        got = [int(pool[m.tables[s][p // bs], p % bs]) for p in range(m.lengths[s])]
        if got != toks:
            return False
    return True


def test_exercise3_golden():
    assert pin_exercise3()


def test_paging_trace_golden():
    assert pin_paging_trace()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants_on_random_traces(seed):
    assert pin_invariants(seed)


def test_free_list_order():
    assert pin_free_list_order()


def test_out_of_blocks_changes_nothing():
    assert pin_out_of_blocks()


def test_copy_on_write_contents():
    assert pin_copy_contents()


def test_block_tables_view():
    m = bm.BlockManager(8, 4)
    m.add(5); m.append_slots(5, 6)
    m.add(6)
    t, lens = m.block_tables([6, 5], 3)
    assert t.tolist() == [[-1, -1, -1], [7, 6, -1]] and lens.tolist() == [0, 6]
    with pytest.raises(ValueError):
        m.block_tables([5], 1)


# --- planted mistakes ------------------------------------------------------------

def _mut_no_cow(mp):
    orig = bm.BlockManager.append_slots

    def app(self, seq, n):
        saved = list(self.ref)
        for b in self.tables[seq]:
            self.ref[b] = 1                            # pretend nothing is shared
        out = orig(self, seq, n)
        for b, r in enumerate(saved):
            if self.ref[b] == 1 and r > 1:
                self.ref[b] = r
        return out
    mp.setattr(bm.BlockManager, "append_slots", app)


def _mut_cow_keeps_count(mp):
    orig = bm.BlockManager.append_slots

    def app(self, seq, n):
        copies = orig(self, seq, n)
        for src, _ in copies:
            self.ref[src] += 1
        return copies
    mp.setattr(bm.BlockManager, "append_slots", app)


def _mut_fork_no_ref(mp):
    def fork(self, parent, child):
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
    mp.setattr(bm.BlockManager, "fork", fork)


def _mut_fifo(mp):
    orig = bm.BlockManager.append_slots

    def app(self, seq, n):
        self.free.reverse()
        try:
            return orig(self, seq, n)
        finally:
            self.free.reverse()
    mp.setattr(bm.BlockManager, "append_slots", app)


def _mut_eager_block(mp):
    orig = bm.BlockManager._blocks_needed
    mp.setattr(bm.BlockManager, "_blocks_needed", lambda self, s, n: orig(self, s, n))
    orig_app = bm.BlockManager.append_slots

    def app(self, seq, n):
        out = orig_app(self, seq, n)
        if self.lengths[seq] % self.block_size == 0 and self.free:   # a block too early
            b = self.free.pop()
            self.ref[b] = 1
            self.tables[seq].append(b)
        return out
    mp.setattr(bm.BlockManager, "append_slots", app)


def _mut_free_drops_shared(mp):
    def free_seq(self, seq):
        for b in self.tables.pop(seq):
            self.ref[b] = 0
            if b not in self.free:
                self.free.append(b)
        del self.lengths[seq]
    mp.setattr(bm.BlockManager, "free_seq", free_seq)


def _mut_copy_wrong_direction(mp):
    orig = bm.copy_blocks
    mp.setattr(bm, "copy_blocks", lambda pools, pairs: orig(pools, [(d, s) for s, d in pairs]))


def _mut_no_precheck(mp):
    mp.setattr(bm.BlockManager, "_blocks_needed", lambda self, s, n: 0)


PINS = {"exercise3": pin_exercise3, "paging": pin_paging_trace, "invariants": pin_invariants,
        "order": pin_free_list_order, "oob": pin_out_of_blocks, "contents": pin_copy_contents}


@pytest.mark.parametrize("mutant", [_mut_no_cow, _mut_cow_keeps_count, _mut_fork_no_ref, _mut_fifo,
                                    _mut_eager_block, _mut_free_drops_shared,
                                    _mut_copy_wrong_direction, _mut_no_precheck])
def test_planted_allocator_mistake_is_caught(monkeypatch, mutant):
    mutant(monkeypatch)
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"{mutant.__name__} slipped past every pin"
