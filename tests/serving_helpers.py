"""Serving steps driven by the library's host block manager: admissions with a shared system
prompt (prefix reuse), forks (parallel sampling, copy-on-write), chunked prefill, decode, frees
and eviction. Each step's attention, read through the manager's shared block tables, is checked
against the oracle's attention over each sequence's own contiguous KV.

The data path of a step (block copies, cache write, attention) runs on a backend: the library's
kernels on the GPU, or the oracle's functions on numpy caches (CPU)."""
from __future__ import annotations

import numpy as np

import oracle
import oracle.blocks as ob
import synth

P61 = (1 << 61) - 1


def rand_bf16(rng, shape):
    # finite bf16 patterns (no NaN/Inf), so equality of bits is equality of values
    return synth.bf16_from_f32(rng.standard_normal(shape).astype(np.float32))


class KVSource:
    """The K/V of a position depends on the whole prefix through it: rows are drawn from a
    generator seeded by a rolling hash of the prefix, so equal prefixes give equal rows."""

    def __init__(self, seed, hkv, d):
        self.seed, self.hkv, self.d = seed, hkv, d
        self.memo = {}

    def rows(self, tokens, p0, p1):
        h, hs = 0, []
        for p, t in enumerate(tokens[:p1]):
            h = (h * 1000003 + int(t) + 1) % P61
            if p >= p0:
                hs.append(h)
        k = np.empty((p1 - p0, self.hkv, self.d), np.uint16)
        v = np.empty_like(k)
        for i, hv in enumerate(hs):
            if hv not in self.memo:
                g = np.random.default_rng([self.seed, hv])
                self.memo[hv] = synth.bf16_from_f32(
                    g.standard_normal((2, self.hkv, self.d)).astype(np.float32))
            k[i], v[i] = self.memo[hv]
        return k, v


def contiguous_reference(seqs, ids, q_lens, kv_lens, q, src: KVSource, bs, scale):
    """Oracle attention with every sequence reading its own contiguous KV (private blocks)."""
    nblk = [-(-int(L) // bs) for L in kv_lens]
    base = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)
    kc = np.zeros((int(base[-1]) + 1, bs, src.hkv, src.d), np.uint16)
    vc = np.zeros_like(kc)
    kf, vf = kc.reshape(-1, src.hkv, src.d), vc.reshape(-1, src.hkv, src.d)
    tables = np.full((len(ids), max(nblk)), -1, np.int32)
    for i, (sid, L) in enumerate(zip(ids, kv_lens)):
        k, v = src.rows(seqs[sid], 0, int(L))
        kf[base[i] * bs: base[i] * bs + int(L)] = k
        vf[base[i] * bs: base[i] * bs + int(L)] = v
        tables[i, :nblk[i]] = np.arange(base[i], base[i + 1])
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return oracle.paged_attention(q, cu, kv_lens, tables, kc, vc, scale)[0]


class CpuBackend:
    """The step's data path with the oracle's functions on numpy caches and a numpy pool."""

    def __init__(self, kc, vc, num_slots):
        self.kc, self.vc = kc, vc
        self.pool = np.zeros((num_slots, 2, 1) + kc.shape[1:], np.uint16)

    def step(self, src, dst, outs, ins, knew, vnew, slots, q, cu, kv_lens, tables, scale, max_q,
             max_kv):
        self.kc, self.vc = ob.copy_blocks(self.kc, self.vc, src, dst)
        if len(outs[0]):
            self.pool = ob.swap_out_blocks(self.kc, self.vc, outs[0], outs[1], self.pool)
        if len(ins[0]):
            self.kc, self.vc = ob.swap_in_blocks(self.pool, ins[0], ins[1], self.kc, self.vc)
        self.kc, self.vc = oracle.cache_write(self.kc, self.vc, knew, vnew, slots)
        if q is None:
            return None
        return oracle.paged_attention(q, cu, kv_lens, tables, self.kc, self.vc, scale)[0]


def serving_run(cb, backend_factory, hq, hkv, d, bs, nb, n_steps=28, seed=0, log=print):
    """Runs the steps; returns counters. backend_factory(kc, vc, num_slots) takes the initial
    caches (stale random data everywhere) and the swap pool size, and returns an object with
    step(...) -> float64 output."""
    rng = np.random.default_rng(seed)
    kvsrc = KVSource(seed + 7, hkv, d)
    scale = 1.0 / np.sqrt(d)
    m = cb.BlockManager(nb, bs)
    num_slots = nb // 2
    m.set_swap_slots(num_slots)
    backend = backend_factory(rand_bf16(rng, (nb, bs, hkv, d)), rand_bf16(rng, (nb, bs, hkv, d)),
                              num_slots)
    system = [int(x) for x in rng.integers(0, 50, 5 * bs + 3)]
    seqs, live, swapped = {}, [], []
    next_id = 0
    stats = dict(hits=0, copies=0, steps=0, rows=0, refusals=0, forks=0, swap_outs=0, swap_ins=0)

    for step in range(n_steps):
        outs, ins = ([], []), ([], [])
        just_in = set()
        if step % 5 == 4 and len(live) > 3:
            sid = live[int(rng.integers(len(live)))]
            m.free_sequence(sid)
            live.remove(sid)
        if step % 6 == 2 and len(live) > 2:       # offload one request
            sid = live[int(rng.integers(len(live)))]
            try:
                b, sl = m.swap_out(sid)
                outs = (outs[0] + b.tolist(), outs[1] + sl.tolist())
                live.remove(sid)
                swapped.append(sid)
                stats["swap_outs"] += 1
            except cb.CBError as e:
                assert e.status == cb.CB_ERR_OUT_OF_BLOCKS
                stats["refusals"] += 1
        if step % 6 == 5 and swapped:             # and bring one back
            sid = swapped[0]
            try:
                sl, b = m.swap_in(sid)
                ins = (ins[0] + sl.tolist(), ins[1] + b.tolist())
                swapped.remove(sid)
                live.append(sid)
                just_in.add(sid)
                stats["swap_ins"] += 1
            except cb.CBError as e:
                assert e.status == cb.CB_ERR_OUT_OF_BLOCKS
                stats["refusals"] += 1
        if step < n_steps - 8 and (step % 2 == 0 or len(live) < 2):
            own = [int(x) for x in rng.integers(0, 50, int(rng.integers(1, 3 * bs)))]
            tokens = (system if rng.random() < 0.8 else []) + own
            try:
                stats["hits"] += m.add_sequence(next_id, tokens) > 0
                seqs[next_id] = tokens
                live.append(next_id)
            except cb.CBError as e:
                assert e.status == cb.CB_ERR_OUT_OF_BLOCKS
                stats["refusals"] += 1
            next_id += 1
        for sid in list(live):
            n, c, _ = m.sequence_info(sid)
            # parallel sampling (not of a sequence whose blocks this step's scatter writes)
            if n == c and sid not in just_in and rng.random() < 0.2 and len(live) < 12:
                m.fork(sid, next_id)
                seqs[next_id] = list(seqs[sid])
                live.append(next_id)
                next_id += 1
                stats["forks"] += 1
        for sid in live:
            n, c, _ = m.sequence_info(sid)
            if n == c:                                              # decode: the next token
                t = int(rng.integers(0, 50))
                try:
                    m.append_tokens(sid, [t])
                    seqs[sid].append(t)
                except cb.CBError as e:
                    assert e.status == cb.CB_ERR_OUT_OF_BLOCKS
                    stats["refusals"] += 1
        ids, qs = [], []
        for sid in live:                      # prefill chunks of two to three blocks
            n, c, _ = m.sequence_info(sid)
            if n > c:
                ids.append(sid)
                qs.append(min(n - c, 2 * bs + int(rng.integers(0, bs))))
        if not ids:
            src, dst = m.take_copies()
            if src.size or outs[0] or ins[0]:
                backend.step(src, dst, outs, ins, np.zeros((0, hkv, d), np.uint16),
                             np.zeros((0, hkv, d), np.uint16), np.zeros(0, np.int32), None, None,
                             None, None, scale, 0, 0)
            continue
        mb = max(m.sequence_info(s)[2] for s in ids)
        cu, kv_lens, tables, slots, toks = m.build_batch(ids, qs, mb)
        src, dst = m.take_copies()
        T = int(cu[-1])
        log(f"step {step}: seqs={len(ids)} tokens={T} copies={src.size} "
            f"max_kv={int(kv_lens.max())}")
        knew = np.empty((T, hkv, d), np.uint16)
        vnew = np.empty_like(knew)
        for i, sid in enumerate(ids):
            L, q = int(kv_lens[i]), qs[i]
            knew[cu[i]:cu[i + 1]], vnew[cu[i]:cu[i + 1]] = kvsrc.rows(seqs[sid], L - q, L)
            assert toks[cu[i]:cu[i + 1]].tolist() == seqs[sid][L - q:L]
        qh = rand_bf16(np.random.default_rng(seed * 1000 + step), (T, hq, d))
        cb.cb_validate_batch(cu, kv_lens, tables, slots, bs, nb, max(qs), int(kv_lens.max()))
        got = backend.step(src, dst, outs, ins, knew, vnew, slots, qh, cu, kv_lens, tables, scale,
                           max(qs), int(kv_lens.max()))
        ref = contiguous_reference(seqs, ids, qs, kv_lens, qh, kvsrc, bs, scale)
        ok, rep = oracle.within_tolerance(got, ref)
        assert ok, f"step {step}: {rep}"
        stats["copies"] += int(src.size)
        stats["steps"] += 1
        stats["rows"] += T
    log(f"serving steps: {stats}")
    return stats
