"""Pins of the block-manager oracle (``oracle.blocks``), shared by its pin tests and by the tests
that plant mistakes in copies of it. Each pin takes the oracle module (or a mutated copy).

What pins it: the pages' worked examples (fixtures under tests/golden/), eviction order checks,
and a brute force over random operation sequences in which (a) every sequence reads its own
prefix back from the simulated cache after every step, (b) reference counts equal the table
entries that name each block, and (c) every prefix hit equals a count computed from the
simulated cache contents alone.
"""
from __future__ import annotations

import numpy as np


class Sim:
    """An oracle manager driven step by step, with the brute-force checks after each step."""

    def __init__(self, ob, num_blocks, block_size):
        self.ob = ob
        self.m = ob.BlockManagerOracle(num_blocks, block_size)
        self.bs = block_size
        self.closed = {}   # sequence -> positions computed in closed steps
        self.conf_closed = {}   # sequence -> positions confirmed when the last step closed
        self.real = {}     # sequence -> its real tokens (placeholders included, by value)
        self.outs, self.ins = [], []   # the open step's swap gathers and scatters

    def add(self, sid, tokens):
        expect = self.expected_hit(tokens)
        got = self.m.add_sequence(sid, tokens)
        assert got == expect, f"prefix hit {got} != brute force {expect}"
        self.closed[sid] = got
        self.conf_closed[sid] = len(tokens)
        self.real[sid] = [int(t) for t in tokens]
        return got

    def append(self, sid, tokens):
        self.m.append_tokens(sid, tokens)
        self.real[sid] += [int(t) for t in tokens]

    def append_batch(self, ids, counts, tokens):
        off = 0
        done = 0
        try:
            for sid, n in zip(ids, counts):
                self.m.append_tokens(sid, list(tokens[off:off + n]))
                self.real[sid] += [int(t) for t in tokens[off:off + n]]
                off += n
                done += 1
        except self.ob.BlockError as e:
            e.num_done = done
            raise
        return len(ids)

    def append_placeholders(self, sid, values):
        self.m.append_placeholders(sid, len(values))
        self.real[sid] += [int(t) for t in values]

    def confirm(self, sid, values):
        self.m.confirm_tokens(sid, values)

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.closed[child] = self.closed[parent]
        self.conf_closed[child] = self.conf_closed[parent]
        self.real[child] = list(self.real[parent])

    def free(self, sid):
        self.m.free_sequence(sid)
        del self.closed[sid]

    def swap_out(self, sid):
        pairs = self.m.swap_out(sid)
        self.outs += pairs
        return pairs

    def swap_in(self, sid):
        pairs = self.m.swap_in(sid)
        self.ins += pairs
        self.closed[sid] = 0      # its new blocks are written by this step's scatter
        return pairs

    def step(self, ids, qs, max_blocks=4096):
        cu, kv, bt, slots, toks = self.m.build_batch(ids, qs, max_blocks, int(sum(qs)))
        copies = self.m.take_copies()
        srcs = [s for s, _ in copies]
        dsts = [d for _, d in copies]
        assert len(set(dsts)) == len(dsts), "two copies write one block"
        assert not set(dsts) & set(srcs), "a copy writes another copy's source"
        gathered = [b for b, _ in self.outs]
        out_slots = [sl for _, sl in self.outs]
        scattered = [b for _, b in self.ins]
        assert len(set(out_slots)) == len(out_slots), "two gathers write one slot"
        assert len(set(scattered)) == len(scattered), "two scatters write one block"
        assert not set(scattered) & (set(gathered) | set(dsts) | set(srcs)), \
            "a scatter writes a block another transfer of the step uses"
        self.m.apply_step(copies, (list(ids), cu, slots), self.outs, self.ins, real=self.real)
        self.outs, self.ins = [], []
        for sid in self.m.seqs:
            self.closed[sid] = self.m.seqs[sid]["computed"]
            self.conf_closed[sid] = self.m.seqs[sid]["confirmed"]
        self.check()
        return cu, kv, bt, slots, toks, copies

    def check(self):
        err = self.m.check_views(real=self.real) or self.m.check_counts()
        assert err is None, err

    def expected_hit(self, tokens):
        """Brute force from cache contents: the longest run of leading full blocks (short of the
        block holding the last token) each of which some block holds in full, where "holds"
        means its simulated KV equals that prefix's and it sits in the cached pool, is held
        (released, read by a transfer of the open step) with a key, or sits at that index of a
        live sequence that computed it in a closed step."""
        m, bs = self.m, self.bs
        n = len(tokens)
        j = 0
        while j < (n - 1) // bs:
            want = [tuple(tokens[:j * bs + o + 1]) for o in range(bs)]
            cands = set(m.cached) | {b for b in range(m.nb)
                                     if m.state[b] == self.ob.HELD and m.key[b] is not None}
            for sid, s in m.seqs.items():
                if len(s["table"]) > j and min(self.closed.get(sid, 0),
                                               self.conf_closed.get(sid, 0)) >= (j + 1) * bs:
                    cands.add(s["table"][j])
            if not any(m.kv[b] == want for b in cands):
                break
            j += 1
        return j * bs


def _fixture(rows):
    return {r[0]: [int(x) if x.lstrip("-").isdigit() else x for x in r[1:]] for r in rows}


def pin_fork_cow_example(ob, rows):
    """The page's allocator simulation: a 6-token prompt forked twice, each sample writing one
    token, then the parent freed."""
    fx = {k: v[0] for k, v in _fixture(rows).items()}
    sim = Sim(ob, fx["num_blocks"], fx["block_size"])
    m = sim.m
    prompt = list(range(100, 100 + fx["prompt"]))
    sim.add(0, prompt)
    sim.step([0], [fx["prompt"]])                 # the prompt's KV is computed
    kids = list(range(1, fx["forks"] + 1))
    for c in kids:
        sim.fork(0, c)
    for c in kids:
        sim.append(c, [200 + c])
    t0 = m.block_table(0)
    tabs = [m.block_table(c) for c in kids]
    assert all(t[0] == t0[0] for t in tabs), "the first block must stay shared"
    lasts = [t[-1] for t in tabs] + [t0[-1]]
    assert fx["private_last_block"] == 1 and len(set(lasts)) == len(lasts), \
        "every sample needs a private copy of the last prompt block"
    assert m.copies == [(t0[-1], t[-1]) for t in tabs]
    assert m.stats()[0] == fx["free_after_appends"]
    sim.free(0)
    assert m.ref[t0[0]] == fx["first_block_ref_after_parent_freed"]
    assert all(m.ref[t[-1]] == 1 for t in tabs)
    assert sum(m.ref) == fx["first_block_ref_after_parent_freed"] + len(kids)
    sim.step(kids, [1] * len(kids))               # copies, then each sample's token
    assert m.stats()[0] == fx["free_after_parent_freed"]
    # the same calls in one step: the prompt has no KV yet, so a fork is refused
    m2 = ob.BlockManagerOracle(fx["num_blocks"], fx["block_size"])
    m2.add_sequence(0, prompt)
    try:
        m2.fork(0, 1)
        raise AssertionError("fork of a parent with uncomputed tokens must be refused")
    except ob.BlockError as e:
        assert e.status == ob.INVALID


def pin_block_table_example(ob, rows):
    """The page's block-size-4 example: A has 10 tokens (3 blocks), B has 6 (2 blocks); A's token
    9 is in A's logical block 2 at offset 1; 2 slots are unused in each last block; a block is
    added only when the last one is full."""
    bs = int(rows[0][1])
    seqs = {r[1]: (int(r[2]), [int(x) for x in r[4:]]) for r in rows if r[0] == "seq"}
    look = next(r for r in rows if r[0] == "lookup")
    waste = {r[1]: int(r[2]) for r in rows if r[0] == "waste"}
    m = ob.BlockManagerOracle(8, bs)
    ids = {name: i for i, name in enumerate(sorted(seqs))}
    for name, (n, table) in sorted(seqs.items()):
        m.add_sequence(ids[name], list(range(1000 * ids[name], 1000 * ids[name] + n)))
        assert len(m.block_table(ids[name])) == len(table)
        assert len(table) * bs - n == waste[name]
    names = sorted(seqs)
    cu, kv, bt, slots, _ = m.build_batch([ids[x] for x in names], [seqs[x][0] for x in names], 8,
                                         100)
    s, p = names.index(look[1]), int(look[2])
    logical = seqs[look[1]][1].index(int(look[4]))
    assert p // bs == logical and p % bs == int(look[6])
    assert slots[cu[s] + p] == bt[s][logical] * bs + int(look[6])
    m.take_copies()
    a = ids["A"]
    free0 = m.stats()[0]
    m.append_tokens(a, [1, 2])            # 10 -> 12 tokens: the last block fills, none taken
    assert m.stats()[0] == free0
    m.append_tokens(a, [3])               # the 13th token needs a new block
    assert m.stats()[0] == free0 - 1 and len(m.block_table(a)) == 4


def pin_prefix_worked_example(ob, rows):
    fx = {r[0]: dict(zip(r[1::2], [int(x) for x in r[2::2]])) for r in rows}
    w = fx["worked"]
    bs, shared, own = w["block_size"], w["shared"], w["own"]
    k = 5
    sim = Sim(ob, 50 + k * 20, bs)
    system = list(range(1, shared + 1))
    hits = []
    for r in range(k):
        prompt = system + [10_000 * (r + 1) + i for i in range(own)]
        hits.append(sim.add(r, prompt))
        sim.step([r], [len(prompt) - hits[-1]])
    assert hits[0] == 0 and all(h == shared for h in hits[1:])
    assert len(system + [0] * own) - hits[1] == w["prefill"]
    assert round(100 * hits[1] / (shared + own)) == w["drop_percent"]
    used = {b for s in sim.m.seqs.values() for b in s["table"]}
    assert shared // bs == w["shared_blocks"]
    assert len(used) == w["shared_blocks"] + k * -(-own // bs), "the shared prefix is stored once"

    t = fx["three"]
    bs = t["block_size"]
    sim = Sim(ob, 256, bs)
    S = list(range(1, t["shared"] + 1))
    common = [90001 + i for i in range(t["r2_common"])]
    r1 = S + common + [91001 + i for i in range(t["r1_own"] - t["r2_common"])]
    r2 = S + common + [92001 + i for i in range(t["r2_own"] - t["r2_common"])]
    r3 = S + [93001 + i for i in range(t["r3_own"])]
    for i, (prompt, want) in enumerate([(r1, t["r1_cached"]), (r2, t["r2_cached"]),
                                        (r3, t["r3_cached"])]):
        got = sim.add(i, prompt)
        assert got == want, (i, got, want)
        sim.step([i], [len(prompt) - got])


def pin_last_token_block_not_reused(ob):
    """A prompt identical to a cached one whose length is a multiple of the block size reuses all
    but its last block: the last token's KV (and output) is computed."""
    sim = Sim(ob, 16, 4)
    p = list(range(1, 17))
    sim.add(0, p)
    sim.step([0], [16])
    assert sim.add(1, p) == 12
    sim.step([1], [4])
    assert sim.add(2, p[:13]) == 12


def pin_eviction_order(ob):
    """Cached blocks count as free but go only after the never-used ones, least recently freed
    first; a sequence's last block is freed first."""
    bs = 4
    sim = Sim(ob, 16, bs)
    m = sim.m
    A = list(range(1, 9)) + [50]                     # 2 full blocks + 1 partial
    B = list(range(101, 109)) + [60]
    sim.add(0, A)
    sim.add(1, B)
    sim.step([0, 1], [9, 9])
    sim.free(0)
    sim.free(1)                                      # cached: A1, A0, B1, B0 (freed order)
    assert m.stats()[:2] == (16 - 4, 4)
    filler = [1000 + i for i in range(4 * 10)]       # all never-used blocks but two
    sim.add(2, filler)
    assert m.stats()[:2] == (2, 4), "never-used blocks go before cached ones"
    sim.step([2], [len(filler)])
    assert sim.add(3, A) == 8 and sim.add(4, B) == 8, "no cached block was evicted"
    assert m.stats()[:2] == (0, 0)
    sim.step([3, 4], [1, 1])
    sim.free(3)
    sim.free(4)                                      # cached: A1, A0, B1, B0 again
    sim.free(2)                                      # then the filler's blocks, last first
    cached = list(m.cached)
    assert [m.key[b] for b in cached[:4]] == [tuple(A[:8]), tuple(A[:4]), tuple(B[:8]),
                                              tuple(B[:4])]
    assert [m.key[b] for b in cached[4:]] == [tuple(filler[:4 * j]) for j in range(10, 0, -1)]
    # two never-used blocks are left: a 3-block prompt takes them and evicts the least
    # recently freed cached block (A's second block), and nothing else
    sim.add(5, [7000 + i for i in range(12)])
    assert m.key[cached[0]] is None
    assert all(m.key[b] is not None for b in cached[1:])
    sim.step([5], [12])
    assert sim.add(6, A) == 4


def pin_protocol_rules(ob):
    """The step rules that keep copies and lookups from reading KV that is not written yet."""
    bs = 4
    P = [1, 2, 3, 4, 5, 6]

    def refused(fn, *a):
        try:
            fn(*a)
        except ob.BlockError as e:
            return e.status == ob.INVALID
        return False

    # a copy-on-write of a block written in the open step is refused until the step closes
    m = ob.BlockManagerOracle(16, bs)
    m.add_sequence(0, P)
    cu, _, _, slots, _ = m.build_batch([0], [6], 8, 6)
    m.fork(0, 1)                       # the parent's tokens are all in a built batch
    assert refused(m.append_tokens, 1, [7])
    m.apply_step(m.take_copies(), ([0], cu, slots))
    m.append_tokens(1, [7])
    cu, _, _, slots, _ = m.build_batch([1], [1], 8, 1)
    m.apply_step(m.take_copies(), ([1], cu, slots))
    assert m.check_views() is None and m.check_counts() is None

    # a sequence in the open step's batch cannot be freed
    m = ob.BlockManagerOracle(16, bs)
    m.add_sequence(0, P)
    m.build_batch([0], [6], 8, 6)
    assert refused(m.free_sequence, 0)
    m.take_copies()
    m.free_sequence(0)

    # blocks computed in the open step are found only after it closes
    m = ob.BlockManagerOracle(16, bs)
    A = list(range(1, 9))
    m.add_sequence(0, A + [9])
    m.build_batch([0], [9], 8, 9)
    assert m.add_sequence(1, A + [10]) == 0
    m.take_copies()
    assert m.add_sequence(2, A + [11]) == 8

    # a copy's source that loses its last holder stays out of the pools until the copies are
    # taken, so it cannot become the destination of another copy of the same step
    sim = Sim(ob, 16, bs)
    m = sim.m
    sim.add(0, P)
    sim.add(1, [11, 12, 13, 14, 15, 16])
    sim.step([0, 1], [6, 6])
    sim.fork(0, 2)
    sim.fork(1, 3)
    sim.append(2, [7])                 # copy of sequence 0's last block
    sim.free(0)                        # its only other holder leaves
    assert m.stats()[2] == 1
    sim.append(3, [8])                 # this copy's destination must be a different block
    sim.step([2, 3], [1, 1])
    assert m.stats()[2] == 0

    # a copy's destination whose sequence is freed in the same step is held as well, so it
    # cannot become the destination of a second copy of that step
    sim.fork(2, 4)
    sim.fork(2, 5)
    sim.append(4, [1])                 # copy into a new block D
    sim.free(4)                        # D's only holder leaves before the copy has run
    sim.append(5, [2])                 # its copy must not write D too
    sim.step([5], [1])


def pin_swap(ob):
    """The offload tier: victims' blocks go to pool slots in one batched transfer, their device
    blocks serve others meanwhile, and a swap-in resumes the request with nothing recomputed; a
    request that does not fit the pool is refused (the caller soft-resets it)."""
    bs = 4
    sim = Sim(ob, 20, bs)
    m = sim.m
    m.set_swap_slots(6)

    def refused(fn, *a, status=None):
        try:
            fn(*a)
        except ob.BlockError as e:
            return status is None or e.status == status
        return False

    A, B, C = [1, 2, 3, 4, 5, 6, 7], [9, 8, 7, 6, 5], [3, 3, 3, 3, 3, 3, 3, 3, 3]
    E = [4, 4, 2, 2, 1]
    for i, t in enumerate((A, B, C)):
        sim.add(i, t)
    sim.add(5, E)
    sim.step([0, 1, 2, 5], [7, 5, 9, 5])
    assert refused(m.swap_in, 0)                          # not swapped out
    outs = sim.swap_out(0) + sim.swap_out(1)              # one batched transfer: 2 + 2 blocks
    assert len(outs) == 4 and len({sl for _, sl in outs}) == 4
    assert refused(m.swap_out, 2, status=ob.OUT_OF_BLOCKS)  # 3 blocks, 2 slots left
    for fn, a in ((m.append_tokens, (0, [1])), (m.fork, (0, 7)), (m.build_batch, ([0], [1], 8, 1))):
        assert refused(fn, *a, status=ob.INVALID)
    assert m.sequence_info(0) == (7, 7, 0)
    sim.step([], [])
    free_after = m.stats()[0] + m.stats()[1]
    assert free_after == 20 - 5                           # only C and E hold device blocks
    # the victims' blocks serve a new request
    D = [50 + i for i in range(16)]
    sim.add(3, D)
    sim.step([3], [16])
    # swap A back in: nothing recomputed, its view is intact after the step's scatter
    ins = sim.swap_in(0)
    assert [sl for sl, _ in ins] == [sl for _, sl in outs[:2]]
    assert m.sequence_info(0) == (7, 7, 2)
    # A's slots are held until the step's scatter has read them: E's swap-out takes others
    outs_e = sim.swap_out(5)
    assert not {sl for _, sl in outs_e} & {sl for sl, _ in ins}
    assert refused(m.swap_out, 0, status=ob.INVALID)      # its blocks are written this step
    sim.step([], [])
    sim.append(0, [8])
    sim.step([0], [1])
    assert m.swap_stats() == (2, 4, 0)                    # B and E hold 2 slots each
    # a swapped-in sequence freed in the same step: its new blocks stay held, so another swap-in
    # of that step scatters elsewhere
    sim.swap_in(1)                     # B comes back ...
    sim.free(1)                        # ... and leaves again before the scatter has run
    sim.swap_in(5)                     # E's scatter must not target B's blocks
    sim.step([], [])
    # soft reset of C (freed, re-added with its tokens): its cached full blocks are reused
    sim.free(2)
    assert sim.add(4, C) == 8
    sim.step([4], [1])


def pin_placeholders(ob):
    """Async steps append a token before its value is known: the block it completes is keyed only
    once the value is confirmed, so no request reuses KV computed from a token it does not have."""
    bs = 4
    sim = Sim(ob, 16, bs)
    m = sim.m

    def refused(fn, *a):
        try:
            fn(*a)
        except ob.BlockError as e:
            return e.status == ob.INVALID
        return False

    sim.add(0, [1, 2, 3])
    sim.step([0], [3])
    sim.append_placeholders(0, [4])          # the GPU will see token 4; the manager holds 0
    sim.step([0], [1])                       # block 0 is full and computed, but unconfirmed
    assert refused(m.fork, 0, 9)             # a fork needs confirmed tokens
    assert sim.add(1, [1, 2, 3, 0, 9]) == 0  # the placeholder value must not match
    sim.step([1], [5])
    assert refused(m.confirm_tokens, 0, [4, 5])
    sim.confirm(0, [4])                      # now block 0 is keyed as (1, 2, 3, 4)
    sim.step([], [])
    assert sim.add(2, [1, 2, 3, 4, 5]) == 4
    sim.step([2], [1])
    sim.fork(0, 3)


def random_ops(rng, n_ops, vocab=3, bs=4, shared=(), max_prompt=14):
    """A random operation stream (host only): prompts from a few shared prefixes plus random
    suffixes over a tiny vocabulary, so prefixes collide often."""
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.25:
            base = list(shared[rng.integers(len(shared))]) if shared and rng.random() < 0.7 else []
            extra = rng.integers(1, max_prompt)
            ops.append(("add", base + [int(x) for x in rng.integers(0, vocab, extra)]))
        elif r < 0.35:
            ops.append(("append", [int(x) for x in rng.integers(0, vocab, rng.integers(1, 4))]))
        elif r < 0.38:
            ops.append(("placeholders", [int(x) for x in rng.integers(0, vocab, rng.integers(1, 3))]))
        elif r < 0.4:
            ops.append(("confirm", None))
        elif r < 0.45:
            ops.append(("append_batch", int(rng.integers(1, 1 << 30))))
        elif r < 0.5:
            ops.append(("fork", None))
        elif r < 0.53:
            ops.append(("swap_out", None))
        elif r < 0.56:
            ops.append(("swap_in", None))
        elif r < 0.7:
            ops.append(("free", None))
        else:
            ops.append(("step", int(rng.integers(1, 1 << 30))))
    return ops


def drive(sim_like, ops, rng_seed):
    """Runs an operation stream against a manager-like object exposing add/append/fork/free/step
    (each raising an exception with .status on refusal); returns the log of outcomes."""
    rng = np.random.default_rng(rng_seed)
    live, next_id, log = [], 0, []
    swapped = set()
    unconfirmed = {}   # sequence -> real values of its placeholders not yet confirmed
    for kind, arg in ops:
        try:
            if kind == "add":
                out = sim_like.add(next_id, arg)
                live.append(next_id)
                next_id += 1
            elif kind == "append" and live:
                sid = live[rng.integers(len(live))]
                out = sim_like.append(sid, arg)
            elif kind == "placeholders" and live:
                sid = live[rng.integers(len(live))]
                out = sim_like.append_placeholders(sid, arg)
                unconfirmed.setdefault(sid, []).extend(arg)
            elif kind == "confirm" and unconfirmed:
                sid = sorted(unconfirmed)[rng.integers(len(unconfirmed))]
                vals = unconfirmed.pop(sid)
                out = sim_like.confirm(sid, vals)
            elif kind == "append_batch" and live:
                r2 = np.random.default_rng(arg)
                ids = [s for s in live if r2.random() < 0.5]
                counts = [int(r2.integers(0, 3)) for _ in ids]
                toks = [int(x) for x in r2.integers(0, 3, sum(counts))]
                out = sim_like.append_batch(ids, counts, toks)
            elif kind == "fork" and live:
                sid = live[rng.integers(len(live))]
                out = sim_like.fork(sid, next_id)
                live.append(next_id)
                next_id += 1
            elif kind in ("swap_out", "swap_in") and live:
                pool = sorted(swapped) if kind == "swap_in" and swapped and rng.random() < 0.8 else live
                sid = pool[rng.integers(len(pool))]
                out = getattr(sim_like, kind)(sid)
                (swapped.add if kind == "swap_out" else swapped.discard)(sid)
            elif kind == "free" and live:
                sid = live[rng.integers(len(live))]
                out = sim_like.free(sid)
                live.remove(sid)
                swapped.discard(sid)
                unconfirmed.pop(sid, None)
            elif kind == "step":
                pend = sim_like.pending([s for s in live if s not in swapped])
                r2 = np.random.default_rng(arg)
                ids = [s for s in live if s not in swapped and pend[s] > 0 and r2.random() < 0.8]
                qs = [int(r2.integers(1, pend[s] + 1)) for s in ids]
                out = sim_like.step(ids, qs)
            else:
                out = None
            log.append((kind, "ok", out))
        except Exception as e:  # noqa: BLE001 -- refusals are part of the compared behaviour
            if not hasattr(e, "status"):
                raise
            log.append((kind, e.status, getattr(e, "num_done", None)))
            if kind == "add":
                next_id += 1
            if kind == "fork":
                next_id += 1
    return log


class OracleDriver:
    """drive() adapter for the oracle with the brute-force checks."""

    def __init__(self, ob, nb, bs):
        self.sim = Sim(ob, nb, bs)

    def add(self, sid, toks):
        return self.sim.add(sid, toks)

    def append(self, sid, toks):
        return self.sim.append(sid, toks)

    def append_batch(self, ids, counts, toks):
        return self.sim.append_batch(ids, counts, toks)

    def append_placeholders(self, sid, vals):
        return self.sim.append_placeholders(sid, vals)

    def confirm(self, sid, vals):
        return self.sim.confirm(sid, vals)

    def swap_out(self, sid):
        return [tuple(p) for p in self.sim.swap_out(sid)]

    def swap_in(self, sid):
        return [tuple(p) for p in self.sim.swap_in(sid)]

    def fork(self, p, c):
        return self.sim.fork(p, c)

    def free(self, sid):
        return self.sim.free(sid)

    def pending(self, live):
        return {s: len(self.sim.m.seqs[s]["tokens"]) - self.sim.m.seqs[s]["computed"] for s in live}

    def step(self, ids, qs):
        cu, kv, bt, slots, toks, copies = self.sim.step(ids, qs)
        return (cu.tolist(), kv.tolist(), slots.tolist(), toks.tolist(), copies,
                self.sim.m.stats(), list(self.sim.m.ref))


def pin_random_bruteforce(ob, seeds=range(12), n_ops=160):
    for seed in seeds:
        rng = np.random.default_rng(seed)
        shared = [list(rng.integers(0, 3, int(rng.integers(4, 12)))) for _ in range(3)]
        ops = random_ops(rng, n_ops, shared=shared)
        d = OracleDriver(ob, 40, 4)
        d.sim.m.set_swap_slots(24)
        drive(d, ops, seed + 1000)
