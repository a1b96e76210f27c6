"""The C++ block manager (through the C ABI) against the oracle: identical outcomes, block ids,
copies, batch metadata, pool counts and reference counts on random operation streams and the
pages' examples; the C ABI's argument checks (CPU only: the manager is host code)."""
import ctypes

import numpy as np
import pytest

import oracle.blocks as ob
from pins_blocks import OracleDriver, drive, random_ops

cb = pytest.importorskip("ragged_paged_kv_amd")


class LibDriver:
    """drive() adapter for the library's manager."""

    def __init__(self, nb, bs):
        self.m = cb.BlockManager(nb, bs)
        self.nb = nb

    def add(self, sid, toks):
        return self.m.add_sequence(sid, toks)

    def append(self, sid, toks):
        return self.m.append_tokens(sid, toks)

    def append_batch(self, ids, counts, toks):
        return self.m.append_batch(ids, counts, toks)

    def append_placeholders(self, sid, vals):
        return self.m.append_placeholders(sid, len(vals))

    def confirm(self, sid, vals):
        return self.m.confirm_tokens(sid, vals)

    def swap_out(self, sid):
        a, b = self.m.swap_out(sid)
        return list(zip(a.tolist(), b.tolist()))

    def swap_in(self, sid):
        a, b = self.m.swap_in(sid)
        return list(zip(a.tolist(), b.tolist()))

    def fork(self, p, c):
        return self.m.fork(p, c)

    def free(self, sid):
        return self.m.free_sequence(sid)

    def pending(self, live):
        out = {}
        for s in live:
            n, c, _ = self.m.sequence_info(s)
            out[s] = n - c
        return out

    def step(self, ids, qs):
        cu, kv, bt, slots, toks = self.m.build_batch(ids, qs, 4096)
        src, dst = self.m.take_copies()
        return (cu.tolist(), kv.tolist(), slots.tolist(), toks.tolist(),
                list(zip(src.tolist(), dst.tolist())), self.m.stats(), self.m.ref_counts().tolist())


def compare(seed, nb, bs, n_ops, vocab=3, max_prompt=14, n_shared=3):
    rng = np.random.default_rng(seed)
    shared = [list(rng.integers(0, vocab, int(rng.integers(bs, 3 * bs)))) for _ in range(n_shared)]
    ops = random_ops(rng, n_ops, vocab=vocab, bs=bs, shared=shared, max_prompt=max_prompt)
    o, c = OracleDriver(ob, nb, bs), LibDriver(nb, bs)
    o.sim.m.set_swap_slots(nb // 2)
    c.m.set_swap_slots(nb // 2)
    lo = drive(o, ops, seed + 7)
    lc = drive(c, ops, seed + 7)
    assert len(lo) == len(lc)
    for i, (a, b) in enumerate(zip(lo, lc)):
        assert a == b, f"seed {seed} op {i}: oracle {a} vs library {b}"
    for sid in o.sim.m.seqs:
        assert o.sim.m.block_table(sid) == c.m.block_table(sid).tolist()
        assert o.sim.m.sequence_info(sid) == c.m.sequence_info(sid)
    assert o.sim.m.stats() == c.m.stats()
    assert o.sim.m.swap_stats() == c.m.swap_stats()
    return lo


@pytest.mark.parametrize("seed", range(16))
def test_matches_oracle_small_pool(seed):
    compare(seed, nb=40, bs=4, n_ops=200)


@pytest.mark.parametrize("seed", range(4))
def test_matches_oracle_block16(seed):
    compare(100 + seed, nb=96, bs=16, n_ops=300, vocab=2, max_prompt=40)


def test_fork_cow_example_through_library():
    m = cb.BlockManager(8, 4)
    assert m.add_sequence(0, [100, 101, 102, 103, 104, 105]) == 0
    m.build_batch([0], [6], 4)
    assert m.take_copies()[0].size == 0
    m.fork(0, 1)
    m.fork(0, 2)
    m.append_tokens(1, [201])
    m.append_tokens(2, [202])
    t0, t1, t2 = m.block_table(0), m.block_table(1), m.block_table(2)
    assert t1[0] == t2[0] == t0[0] and len({t0[1], t1[1], t2[1]}) == 3
    assert m.stats()[0] == 4
    m.free_sequence(0)
    refs = m.ref_counts()
    assert refs[t0[0]] == 2 and refs.sum() == 4
    src, dst = m.take_copies()
    assert list(zip(src, dst)) == [(t0[1], t1[1]), (t0[1], t2[1])]
    assert m.stats()[0] == 5


def status_of(fn, *a):
    try:
        fn(*a)
    except cb.CBError as e:
        return e.status
    return 0


def test_rules_and_refusals():
    m = cb.BlockManager(6, 4)
    assert status_of(m.add_sequence, 0, []) == -1
    m.add_sequence(0, [1, 2, 3, 4, 5, 6])
    assert status_of(m.add_sequence, 0, [1]) == -1                 # id in use
    assert status_of(m.append_tokens, 9, [1]) == -1                # unknown id
    assert status_of(m.fork, 0, 1) == -1                           # parent not computed
    m.build_batch([0], [6], 4)
    assert status_of(m.free_sequence, 0) == -1                     # in the open step's batch
    m.fork(0, 1)
    assert status_of(m.append_tokens, 1, [7]) == -1                # copy of a dirty block
    assert status_of(m.build_batch, [1, 1], [1, 1], 4) == -1       # no pending tokens / twice
    m.take_copies()
    m.append_tokens(1, [7])
    assert status_of(m.build_batch, [1], [2], 4) == -1             # q beyond pending tokens
    assert status_of(m.build_batch, [1], [1], 1) == -1             # table longer than the row
    assert status_of(m.add_sequence, 2, list(range(100, 117))) == cb.CB_ERR_OUT_OF_BLOCKS
    before = (m.stats(), m.ref_counts().tolist())
    assert status_of(m.append_tokens, 1, list(range(50))) == cb.CB_ERR_OUT_OF_BLOCKS
    assert (m.stats(), m.ref_counts().tolist()) == before          # a failing call changes nothing


def test_take_copies_reports_count_when_too_small():
    m = cb.BlockManager(16, 4)
    m.add_sequence(0, [1, 2, 3, 4, 5])
    m.build_batch([0], [5], 8)
    m.take_copies()
    for c in (1, 2, 3):
        m.fork(0, c)
    for c in (1, 2, 3):
        m.append_tokens(c, [9])
    n = ctypes.c_int32()
    src = np.zeros(2, np.int32)
    st = cb.lib.cb_bm_take_copies(m._h, src.ctypes.data_as(ctypes.c_void_p),
                                  src.ctypes.data_as(ctypes.c_void_p), 2, ctypes.byref(n))
    assert st == -1 and n.value == 3
    s, d = m.take_copies()
    assert s.size == 3 and len(set(d.tolist())) == 3


def test_c_abi_argument_checks():
    h = ctypes.c_void_p()
    assert cb.lib.cb_bm_create(0, 16, ctypes.byref(h)) == -1
    assert cb.lib.cb_bm_create(16, 0, ctypes.byref(h)) == -1
    assert cb.lib.cb_bm_create(1 << 28, 16, ctypes.byref(h)) == -1   # slots past 2^31
    assert cb.lib.cb_bm_create(16, 16, None) == -1
    assert cb.lib.cb_bm_add_sequence(None, 0, None, 1, None) == -1
    assert cb.lib.cb_bm_stats(None, None, None, None, None) == -1
    m = cb.BlockManager(4, 16)
    out = np.zeros(2, np.int32)
    assert cb.lib.cb_bm_ref_counts(m._h, out.ctypes.data_as(ctypes.c_void_p), 2) == -1
    assert cb.lib.cb_bm_add_sequence(m._h, 0, None, 3, None) == -1
    assert cb.lib.cb_bm_take_copies(m._h, None, None, 0, None) == -1
    cb.lib.cb_bm_destroy(None)


def test_copy_blocks_host_checks():
    fake = ctypes.c_void_p(0x10000)
    f = cb.lib.cb_copy_blocks
    assert f(fake, fake, fake, fake, -1, 4096, 8, 1, 0, None) == -1
    assert f(fake, fake, fake, fake, 1, 4008, 8, 1, 0, None) == -1            # not 16-multiple
    assert f(fake, fake, fake, fake, 1, 4096, 0, 1, 0, None) == -1
    assert f(fake, fake, fake, fake, 1, 4096, 8, 2, 4096 * 7, None) == -1     # stride too small
    assert f(None, fake, fake, fake, 1, 4096, 8, 1, 0, None) == -1
    assert f(ctypes.c_void_p(0x10008), fake, fake, fake, 1, 4096, 8, 1, 0, None) == -1
    assert f(None, None, None, None, 0, 4096, 8, 1, 0, None) == 0              # nothing to do


@pytest.mark.parametrize("hq,hkv,d,bs,nb,seed", [(4, 2, 64, 16, 96, 0), (2, 2, 64, 32, 40, 1)])
def test_serving_steps_cpu_data_path(hq, hkv, d, bs, nb, seed):
    """The library's manager driving the oracle's copy, cache write and attention: reading
    through shared, copied and reused blocks gives the attention of private contiguous KV."""
    from serving_helpers import CpuBackend, serving_run
    stats = serving_run(cb, CpuBackend, hq, hkv, d, bs, nb, n_steps=24, seed=seed,
                        log=lambda *a: None)
    assert stats["hits"] > 0 and stats["copies"] > 0 and stats["forks"] > 0
    assert stats["swap_outs"] > 0 and stats["swap_ins"] > 0


def test_copy_blocks_rejects_oversized_dispatch():
    fake = ctypes.c_void_p(0x10000)
    # 2^21 copies x 32 layers x 2 tensors x 16 workgroups of 128 lanes > 2^32 work-items
    assert cb.lib.cb_copy_blocks(fake, fake, fake, fake, 1 << 21, 32768, 1 << 22, 32,
                                 32768 << 22, None) == -2


def test_build_batch_into_caller_buffers():
    m = cb.BlockManager(64, 4)
    for s in range(3):
        m.add_sequence(s, list(range(10 * s, 10 * s + 5 + s)))
    a = m.build_batch([0, 1, 2], [5, 6, 7], 8)
    m2 = cb.BlockManager(64, 4)
    for s in range(3):
        m2.add_sequence(s, list(range(10 * s, 10 * s + 5 + s)))
    bufs = (np.zeros(4, np.int32), np.zeros(3, np.int32), np.full((3, 8), -1, np.int32),
            np.zeros(18, np.int32), np.zeros(18, np.int32))
    b = m2.build_batch([0, 1, 2], [5, 6, 7], 8, out=bufs)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    with pytest.raises(ValueError):
        m2.build_batch([0], [1], 8, out=(bufs[0].astype(np.int64),) + bufs[1:])


def test_append_batch_stops_at_first_refusal():
    m = cb.BlockManager(4, 4)
    m.add_sequence(0, [1, 2, 3, 4])
    m.add_sequence(1, [5, 6, 7, 8])
    m.build_batch([0, 1], [4, 4], 4)
    m.take_copies()
    # seq 0 takes a block, seq 1 takes the last, the third append (seq 0 again) needs one more
    with pytest.raises(cb.CBError) as e:
        m.append_batch([0, 1, 0], [1, 1, 4], list(range(6)))
    assert e.value.status == cb.CB_ERR_OUT_OF_BLOCKS and e.value.num_done == 2
    assert m.sequence_info(0)[0] == 5 and m.sequence_info(1)[0] == 5


def test_batched_placeholders_and_confirmation_match_single_calls():
    a, b = cb.BlockManager(64, 4), cb.BlockManager(64, 4)
    for m in (a, b):
        for s_ in range(3):
            m.add_sequence(s_, [5 + s_] * 6)
        m.build_batch([0, 1, 2], [6, 6, 6], 8)
        m.take_copies()
    a.append_batch([0, 1, 2], [1, 2, 1], None)
    for s_, n in ((0, 1), (1, 2), (2, 1)):
        b.append_placeholders(s_, n)
    a.confirm_batch([0, 1, 2], [1, 2, 1], [7, 8, 9, 10])
    b.confirm_tokens(0, [7])
    b.confirm_tokens(1, [8, 9])
    b.confirm_tokens(2, [10])
    for s_ in range(3):
        assert a.sequence_info(s_) == b.sequence_info(s_)
        assert a.block_table(s_).tolist() == b.block_table(s_).tolist()
    with pytest.raises(cb.CBError) as e:
        a.confirm_batch([0, 1], [0, 1], [3])   # sequence 1 has no unconfirmed token left
    assert e.value.num_done == 1
