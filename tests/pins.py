"""Checks that tie the oracle to something other than itself.

Each ``pin_*`` function takes an oracle-like namespace (``orc``) and raises AssertionError
when the oracle disagrees with what the pages print, a closed form, a library routine, a
brute-force formulation written independently here, or an invariant. ``test_oracle_*.py``
runs them on the real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle
with a planted mistake and requires that at least one pin fails for each mistake.
"""
from __future__ import annotations

import math

import numpy as np

import synth


# ----------------------------------------------------------------------------------------------
# helpers written independently of the oracle


def table_slots(table_row, L, bs):
    """Slots of a sequence's first L positions, by walking its blocks in logical order and each
    block's offsets in order (no // or % on positions)."""
    out = []
    for b in table_row:
        if len(out) >= L:
            break
        for o in range(bs):
            out.append(int(b) * bs + o)
    return out[:L]


def apply_step_write(batch):
    """(k_cache, v_cache) after writing the new tokens, using table_slots for placement."""
    kc = batch.k_cache.copy()
    vc = batch.v_cache.copy()
    nb, bs, hkv, d = kc.shape
    kf = kc.reshape(nb * bs, hkv, d)
    vf = vc.reshape(nb * bs, hkv, d)
    cu = batch.cu_seqlens_q
    for s in range(batch.num_seqs):
        q = int(cu[s + 1] - cu[s])
        L = int(batch.kv_lens[s])
        slots = table_slots(batch.block_tables[s], L, bs)
        for i in range(q):
            kf[slots[L - q + i]] = batch.k[cu[s] + i]
            vf[slots[L - q + i]] = batch.v[cu[s] + i]
    return kc, vc


def widen(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tiny_batch(specs, Hq, Hkv, D, bs, seed, scale=None, shared_prefix_tokens=0, num_blocks=None):
    rng = np.random.default_rng(seed)
    return synth.build_batch(f"tiny-{seed}", seed, rng, specs, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=D, block_size=bs, scale=scale,
                             shared_prefix_tokens=shared_prefix_tokens, num_blocks=num_blocks)


def raw_batch(q_rows, k_rows, v_rows, qlen, Hq=1, Hkv=1, bs=4, scale=1.0, seed=0):
    """One sequence whose whole KV (L rows) and last ``qlen`` queries are given explicitly as
    float arrays exactly representable in bf16. Returns (batch with the cache already written)."""
    k_rows = np.asarray(k_rows, dtype=np.float64).reshape(len(k_rows), Hkv, -1)
    v_rows = np.asarray(v_rows, dtype=np.float64).reshape(len(v_rows), Hkv, -1)
    q_rows = np.asarray(q_rows, dtype=np.float64).reshape(qlen, Hq, -1)
    L, _, D = k_rows.shape
    b = tiny_batch([synth.SeqSpec(qlen, L)], Hq, Hkv, D, bs, seed, scale=scale)
    kb = synth.bf16_from_f32(k_rows.astype(np.float32))
    vb = synth.bf16_from_f32(v_rows.astype(np.float32))
    assert np.array_equal(widen(kb), k_rows) and np.array_equal(widen(vb), v_rows)
    slots = table_slots(b.block_tables[0], L, bs)
    kf = b.k_cache.reshape(-1, Hkv, D)
    vf = b.v_cache.reshape(-1, Hkv, D)
    for p in range(L):
        kf[slots[p]] = kb[p]
        vf[slots[p]] = vb[p]
    b.k = kb[L - qlen:].copy()
    b.v = vb[L - qlen:].copy()
    b.q = synth.bf16_from_f32(q_rows.astype(np.float32))
    return b


def run_oracle(orc, batch, tokens=None):
    sl = orc.slot_mapping(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables, batch.block_size)
    kc, vc = orc.cache_write(batch.k_cache, batch.v_cache, batch.k, batch.v, sl)
    return orc.paged_attention(batch.q, batch.cu_seqlens_q, batch.kv_lens, batch.block_tables,
                               kc, vc, batch.scale, tokens=tokens)


# ----------------------------------------------------------------------------------------------
# packing and block arithmetic


def pin_padding_waste(orc, rows):
    """The page's printed example (one 100-token prompt among 7 one-token decodes) and the three
    printed ratios of waste when B, n or both double."""
    g = {r[0]: r[1] for r in rows}
    B, n = int(g["B"]), int(g["n"])
    c = orc.prompt_among_decodes(B, n)
    assert (c["wasted"], c["padded"], c["ragged"]) == (int(g["waste"]), int(g["padded"]),
                                                       int(g["real"]))
    for key, (b2, n2) in {"ratio_double_B": (2 * B, n), "ratio_double_n": (B, 2 * n),
                          "ratio_double_both": (2 * B, 2 * n)}.items():
        r = orc.prompt_among_decodes(b2, n2)["wasted"] / c["wasted"]
        assert f"{r:.3f}" == g[key], (key, r)
    # The page also prints zero second differences in B and n and a unit mixed difference: the
    # signature of the bilinear form (n - 1)(B - 1), which pin_padding_closed_form checks the
    # oracle against cell by cell.
    assert (int(g["second_difference_B"]), int(g["second_difference_n"]),
            int(g["mixed_difference"])) == (0, 0, 1)


def pin_padding_closed_form(orc):
    # the occupancy count against the closed form (n - 1)(B - 1), including the degenerate
    # cases B = 1 and n = 1
    for B in range(1, 30):
        for n in range(1, 30):
            c = orc.prompt_among_decodes(B, n)
            assert c["wasted"] == (n - 1) * (B - 1)
            assert c["padded"] == B * n and c["ragged"] == n + B - 1
    # arbitrary rows: padded = rows x longest, ragged = sum, brute-forced cell by cell
    rng = np.random.default_rng(4)
    for _ in range(50):
        lens = rng.integers(1, 40, size=int(rng.integers(1, 9)))
        c = orc.rectangle_count(lens)
        cells = sum(1 for r in lens for j in range(int(lens.max())) if j < r)
        assert c["ragged"] == cells == int(lens.sum())
        assert c["padded"] == len(lens) * int(lens.max())
    # the tiny workload: decodes at 1 token each and a 24-token prompt -> 27 rows vs 4 x 24
    c = orc.rectangle_count([1, 1, 1, 24])
    assert c["ragged"] == 27 and c["padded"] == 96 and c["wasted"] == (24 - 1) * (4 - 1)
    packed, cu = orc.pack_ragged([np.zeros((r, 2)) for r in (1, 1, 1, 24)])
    assert packed.shape[0] == 27 and list(cu) == [0, 1, 2, 3, 27]


def pin_block_arithmetic(orc, rows):
    """The page's table (block-table rows for an 8192-token sequence, worst tail waste per block
    size) and the chapter's two counts (1000 and 1300 tokens at block size 16)."""
    for r in rows:
        if r[0] == "table":
            bs, table_rows, worst = int(r[1]), int(r[2]), int(r[3])
            assert orc.block_layout(8192, bs)["blocks"] == table_rows
            assert max(orc.block_layout(L, bs)["unused_tail"] for L in range(1, 2 * bs + 1)) == worst
        elif r[0] == "blocks":
            L, bs, nb, waste = (int(x) for x in r[1:])
            assert orc.block_layout(L, bs) == {"blocks": nb, "unused_tail": waste}
    # ceil(L / bs) blocks and bs * blocks - L unused slots, for every L up to a few blocks
    for bs in (4, 16, 32, 48, 256):
        for L in range(0, 5 * bs):
            assert orc.block_layout(L, bs) == {"blocks": -(-L // bs), "unused_tail": -(-L // bs) * bs - L}


# ----------------------------------------------------------------------------------------------
# slot mapping and cache write


def pin_slot_mapping_p3(orc, rows):
    bs = None
    seqs, pool, lookups, waste = {}, [], [], {}
    for r in rows:
        if r[0] == "block_size":
            bs = int(r[1])
        elif r[0] == "seq":
            seqs[r[1]] = (int(r[2]), [int(x) for x in r[4:]])
        elif r[0] == "block":
            pool.append((int(r[1]), r[2], int(r[3]), int(r[4])))
        elif r[0] == "lookup":
            lookups.append((r[1], int(r[2]), int(r[4]), int(r[6])))
        elif r[0] == "waste":
            waste[r[1]] = int(r[2])
    names = sorted(seqs)
    width = max(len(t) for _, t in seqs.values())
    tables = np.full((len(names), width), -1, dtype=np.int32)
    for i, nm in enumerate(names):
        tables[i, :len(seqs[nm][1])] = seqs[nm][1]
    kv = np.array([seqs[nm][0] for nm in names], dtype=np.int32)
    # whole sequences as one prefill each: every token's slot
    cu = np.concatenate([[0], np.cumsum(kv)]).astype(np.int32)
    sl = orc.slot_mapping(cu, kv, tables, bs)
    for blk, nm, t0, t1 in pool:
        i = names.index(nm)
        for t in range(t0, t1 + 1):
            assert sl[cu[i] + t] // bs == blk, (nm, t, sl[cu[i] + t])
    for nm, t, blk, off in lookups:
        i = names.index(nm)
        assert sl[cu[i] + t] == blk * bs + off
    # one decode token per sequence at its last position
    cu1 = np.arange(len(names) + 1, dtype=np.int32)
    sl1 = orc.slot_mapping(cu1, kv, tables, bs)
    for i, nm in enumerate(names):
        assert sl1[i] == sl[cu[i] + kv[i] - 1]
    for nm, w in waste.items():
        assert orc.block_layout(seqs[nm][0], bs)["unused_tail"] == w


def pin_slot_mapping_bruteforce(orc, seed=0):
    rng = np.random.default_rng(seed)
    for bs in (4, 8, 16, 32):
        for _ in range(20):
            S = int(rng.integers(1, 6))
            L = rng.integers(1, 70, size=S)
            q = np.array([int(rng.integers(1, l + 1)) for l in L])
            nb = [-(-int(l) // bs) for l in L]
            pool = rng.permutation(sum(nb) + 5)
            tables = np.full((S, max(nb) + 2), -1, dtype=np.int32)
            c = 0
            for s in range(S):
                tables[s, :nb[s]] = pool[c:c + nb[s]]
                c += nb[s]
            cu = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
            got = orc.slot_mapping(cu, L.astype(np.int32), tables, bs)
            want = []
            for s in range(S):
                slots = table_slots(tables[s], int(L[s]), bs)
                want += slots[int(L[s] - q[s]):int(L[s])]
            assert got.dtype == np.int32 and list(got) == want


def pin_cache_write(orc, seed=0):
    b = tiny_batch([synth.SeqSpec(1, 9), synth.SeqSpec(5, 12), synth.SeqSpec(3, 3)], 4, 2, 8, 4, seed)
    sl = orc.slot_mapping(b.cu_seqlens_q, b.kv_lens, b.block_tables, b.block_size)
    sl = sl.copy()
    sl[2] = -1  # one token that must not be written
    kc, vc = orc.cache_write(b.k_cache, b.v_cache, b.k, b.v, sl)
    kw, vw = b.k_cache.copy(), b.v_cache.copy()
    flat_k = kw.reshape(-1, 2, 8)
    flat_v = vw.reshape(-1, 2, 8)
    for t, s in enumerate(sl):
        if s >= 0:
            flat_k[s] = b.k[t]
            flat_v[s] = b.v[t]
    assert kc.dtype == np.uint16 and np.array_equal(kc, kw) and np.array_equal(vc, vw)
    # the input is untouched, and exactly the written rows changed
    changed = np.nonzero(np.any(kc.reshape(-1, 16) != b.k_cache.reshape(-1, 16), axis=1))[0]
    assert sorted(changed.tolist()) == sorted(int(s) for s in sl if s >= 0)
    # reading positions [L - q, L) back through the block table gives the new rows
    cu = b.cu_seqlens_q
    for s in range(b.num_seqs):
        q = int(cu[s + 1] - cu[s])
        L = int(b.kv_lens[s])
        slots = table_slots(b.block_tables[s], L, b.block_size)
        for i in range(q):
            t = int(cu[s] + i)
            if sl[t] >= 0:
                assert np.array_equal(kc.reshape(-1, 2, 8)[slots[L - q + i]], b.k[t])
                assert np.array_equal(vc.reshape(-1, 2, 8)[slots[L - q + i]], b.v[t])


# ----------------------------------------------------------------------------------------------
# attention: closed forms, hand cases, library case, brute force, invariants


def pin_single_key(orc):
    # one key: the softmax weight is 1 and the output is that key's value, exactly
    b = tiny_batch([synth.SeqSpec(1, 1), synth.SeqSpec(1, 1)], 4, 2, 16, 4, 7)
    out, lse = run_oracle(orc, b)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(out[s, h], widen(b.v[s, h // 2]))


def pin_uniform_prefix_means(orc):
    # zero queries: every visible key has the same score, so row i is the mean of the values it
    # sees, keys 0 .. L - q + i, and lse = log(L - q + i + 1). Chunk of q = 3 at offset 5.
    L, q, D = 8, 3, 4
    rng = np.random.default_rng(3)
    V = rng.integers(-4, 5, size=(L, D)).astype(np.float64)
    K = rng.integers(-4, 5, size=(L, D)).astype(np.float64)
    b = raw_batch(np.zeros((q, D)), K, V, q)
    out, lse = run_oracle(orc, b)
    for i in range(q):
        last = L - q + i
        np.testing.assert_allclose(out[i, 0], V[:last + 1].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i, 0] - math.log(last + 1)) < 1e-14


def pin_hand_cases(orc):
    ln2 = float(np.float32(math.log(2.0)))
    tol = 1e-8  # the fp32 rounding of ln 2 moves e^score by ~4e-9 relative
    # scores 0 and ln2 -> weights 1 : 2
    b = raw_batch([[1, 0]], [[0, 0], [1, 0]], [[1, 0], [0, 1]], 1, scale=ln2)
    out, lse = run_oracle(orc, b)
    np.testing.assert_allclose(out[0, 0], [1 / 3, 2 / 3], atol=tol)
    assert abs(lse[0, 0] - math.log(3.0)) < tol
    # scores ln2 and -ln2 -> weights 2 : 1/2 -> 0.8, 0.2
    b = raw_batch([[1, 0]], [[1, 0], [-1, 0]], [[1, 1], [-1, 0]], 1, scale=ln2)
    out, lse = run_oracle(orc, b)
    np.testing.assert_allclose(out[0, 0], [0.6, 0.8], atol=tol)
    assert abs(lse[0, 0] - math.log(2.5)) < tol
    # two-token chunk over three keys with equal scores: rows see keys 0..1 and 0..2
    b = raw_batch([[0, 0], [0, 0]], [[1, 0], [0, 1], [1, 1]], [[1, 0], [0, 1], [1, 1]], 2)
    out, _ = run_oracle(orc, b)
    np.testing.assert_allclose(out[0, 0], [0.5, 0.5], atol=1e-15)
    np.testing.assert_allclose(out[1, 0], [2 / 3, 2 / 3], atol=1e-15)
    # three keys, a decode at the last position; scores 0, ln2, 2 ln2 -> weights 1 : 2 : 4
    b = raw_batch([[1, 0]], [[0, 0], [1, 0], [2, 0]], [[7, 0], [0, 7], [0, 0]], 1, scale=ln2)
    out, lse = run_oracle(orc, b)
    np.testing.assert_allclose(out[0, 0], [1.0, 2.0], atol=tol)
    assert abs(lse[0, 0] - math.log(7.0)) < tol


def pin_gqa_mapping(orc):
    # 8 query heads over 2 KV heads: heads 0-3 read KV head 0, heads 4-7 read KV head 1
    Hq, Hkv, D, L = 8, 2, 4, 5
    V = np.zeros((L, Hkv, D))
    V[:, 0, :] = 1.0
    V[:, 1, :] = -2.0
    rng = np.random.default_rng(5)
    K = rng.integers(-2, 3, size=(L, Hkv, D)).astype(np.float64)
    Q = rng.integers(-2, 3, size=(1, Hq, D)).astype(np.float64)
    b = raw_batch(Q, K, V, 1, Hq=Hq, Hkv=Hkv, scale=0.5)
    out, _ = run_oracle(orc, b)
    for h in range(Hq):
        want = 1.0 if h < 4 else -2.0
        np.testing.assert_allclose(out[0, h], want, atol=1e-14)


def _sdpa(Q, K, V, scale):
    """torch CPU float64 causal SDPA; Q [L, Hq, D], K/V [L, Hkv, D] with GQA by repetition."""
    import torch
    G = Q.shape[1] // K.shape[1]
    q = torch.from_numpy(Q).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(),
                                                         is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def pin_sdpa(orc, seed=11):
    # one sequence with q = L is ordinary causal attention; a chunk (q < L) must equal the last q
    # rows of causal attention over the whole sequence
    rng = np.random.default_rng(seed)
    for (Hq, Hkv, D, bs, L) in [(4, 2, 16, 4, 23), (8, 1, 32, 16, 40), (6, 3, 8, 8, 17)]:
        b = tiny_batch([synth.SeqSpec(L, L)], Hq, Hkv, D, bs, int(rng.integers(1 << 30)),
                       scale=float(rng.uniform(0.1, 0.5)))
        out, _ = run_oracle(orc, b)
        Q = widen(b.q)
        K = widen(b.k)
        V = widen(b.v)
        sc = float(np.float32(b.scale))
        ref = _sdpa(Q, K, V, sc)
        assert np.max(np.abs(out - ref)) < 1e-12
        for qn in (1, 5, L - 1):
            c = raw_batch(Q[L - qn:], K, V, qn, Hq=Hq, Hkv=Hkv, bs=bs, scale=b.scale)
            oc, _ = run_oracle(orc, c)
            assert np.max(np.abs(oc - ref[L - qn:])) < 1e-12


def bruteforce_ragged(batch):
    """Attention of the whole packed batch as ONE dense masked softmax per head over the
    concatenation of every sequence's keys, with the block-diagonal causal mask
    M[t, j] = (seq_t == seq_j) and (pos_j <= pos_t)."""
    kc, vc = apply_step_write(batch)
    nb, bs, Hkv, D = kc.shape
    kf = kc.reshape(-1, Hkv, D)
    vf = vc.reshape(-1, Hkv, D)
    Ks, Vs, kseq, kpos = [], [], [], []
    for s in range(batch.num_seqs):
        L = int(batch.kv_lens[s])
        sl = table_slots(batch.block_tables[s], L, bs)
        Ks.append(kf[sl])
        Vs.append(vf[sl])
        kseq += [s] * L
        kpos += list(range(L))
    K = widen(np.concatenate(Ks))
    V = widen(np.concatenate(Vs))
    kseq = np.array(kseq)
    kpos = np.array(kpos)
    qseq, qpos = [], []
    cu = batch.cu_seqlens_q
    for s in range(batch.num_seqs):
        q = int(cu[s + 1] - cu[s])
        L = int(batch.kv_lens[s])
        qseq += [s] * q
        qpos += list(range(L - q, L))
    qseq = np.array(qseq)
    qpos = np.array(qpos)
    M = (qseq[:, None] == kseq[None, :]) & (kpos[None, :] <= qpos[:, None])
    Q = widen(batch.q)
    Hq = Q.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(batch.scale))
    out = np.empty_like(Q)
    for h in range(Hq):
        z = sc * Q[:, h] @ K[:, h // G].T
        z = np.where(M, z, -np.inf)
        w = np.exp(z - z.max(axis=1, keepdims=True))
        out[:, h] = (w @ V[:, h // G]) / w.sum(axis=1, keepdims=True)
    return out


def pin_bruteforce(orc, batch):
    out, _ = run_oracle(orc, batch)
    ref = bruteforce_ragged(batch)
    assert np.max(np.abs(out - ref)) <= 1e-12, np.max(np.abs(out - ref))


def permute_blocks(batch, seed):
    """Same logical batch with physical blocks renumbered by a random permutation."""
    import copy
    rng = np.random.default_rng(seed)
    pi = rng.permutation(batch.num_blocks)
    b = copy.copy(batch)
    kc = np.empty_like(batch.k_cache)
    vc = np.empty_like(batch.v_cache)
    kc[pi] = batch.k_cache
    vc[pi] = batch.v_cache
    b.k_cache, b.v_cache = kc, vc
    t = batch.block_tables
    b.block_tables = np.where(t >= 0, pi[np.maximum(t, 0)], -1).astype(np.int32)
    return b


def pin_permutation_invariance(orc, batch, seed=3):
    out, lse = run_oracle(orc, batch)
    out2, lse2 = run_oracle(orc, permute_blocks(batch, seed))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def pin_split_merge(orc, batch, seed=9):
    out, lse = run_oracle(orc, batch)
    sl = orc.slot_mapping(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables, batch.block_size)
    kc, vc = orc.cache_write(batch.k_cache, batch.v_cache, batch.k, batch.v, sl)
    rng = np.random.default_rng(seed)
    for mode in ("one", "random", "singletons"):
        bounds = []
        for L in batch.kv_lens.tolist():
            if mode == "one":
                bounds.append([0, L])
            elif mode == "singletons":
                bounds.append(list(range(0, L + 1)))
            else:
                cuts = sorted(set(rng.integers(1, L, size=min(L - 1, 4)).tolist())) if L > 1 else []
                bounds.append([0] + cuts + [L])
        o, l_, n = orc.split_partials(batch.q, batch.cu_seqlens_q, batch.kv_lens, batch.block_tables,
                                      kc, vc, batch.scale, bounds)
        merged = orc.merge_partials(o, l_, n)
        if mode == "one":
            assert np.array_equal(merged, out)
        assert np.max(np.abs(merged - out)) < 1e-12, (mode, np.max(np.abs(merged - out)))
        # the log-sum-exp of the range lse values is the whole-range lse
        m = l_.max(axis=2)
        tot = m + np.log(np.exp(l_ - m[..., None]).sum(axis=2))
        assert np.max(np.abs(tot - lse)) < 1e-12
    # a range with lse = -inf carries no weight whatever its o holds (NaN, as 0/0 would give)
    o2 = np.concatenate([o, np.full(o.shape[:2] + (1,) + o.shape[3:], np.nan)], axis=2)
    l2 = np.concatenate([l_, np.full(l_.shape[:2] + (1,), -np.inf)], axis=2)
    merged2 = orc.merge_partials(o2, l2, n + 1)
    assert np.max(np.abs(merged2 - out)) < 1e-12


def pin_tolerance(orc):
    ok, _ = orc.within_tolerance(np.array([1.0, 0.0]), np.array([1.0 + 0.029, 0.0199]))
    assert ok  # 0.029 <= 0.02 + 0.01 * 1.029
    ok, _ = orc.within_tolerance(np.array([1.0, 0.0]), np.array([1.0 + 0.031, 0.0]))
    assert not ok
    ok, _ = orc.within_tolerance(np.array([np.nan]), np.array([0.0]))
    assert not ok
