"""Oracle for the paged KV-cache write and ragged paged attention (test infrastructure only).

What is computed, and where the pages say so:
  * Ragged batch: the step's tokens of all sequences are concatenated with no batch axis
    and sequences are kept apart by a block-diagonal mask ("Continuous batching from first
    principles", Summary and Takeaways; "3.3 Batching & Memory Management", section
    "Continuous (iteration-level) batching": kernels take per-sequence lengths and KV
    locations). Here ``cu_seqlens_q[s]`` is where sequence s starts in the packed batch.
  * Paged cache: a page is one token's K (or V) in one layer, a block is block_size pages
    ("Continuous batching in transformers", section "The paged cache, its two reserved
    blocks, and the block-size trade"); entry j of a sequence's block table is the physical
    block holding its positions [j*bs, (j+1)*bs), so position p lives in block table[p // bs]
    at offset p % bs ("3.3 Batching & Memory Management", section "PagedAttention: block
    tables", worked example with block size 4).
  * Chunked prefill: a chunk's queries attend to a cache that already holds the earlier
    chunks (same page, section "Chunked prefill"); a decode is one new token.
  * Attention itself is not written out on the pages. The reading used here is scaled
    dot-product softmax attention per query head, with query head h reading KV head
    h // (Hq / Hkv), and with the i-th of a sequence's q new tokens sitting at position
    L - q + i, where L counts the sequence's KV tokens after this step's write; it sees
    keys 0 .. L - q + i of its own sequence only.

All floating point is float64. bf16 inputs are widened exactly. The caller's fp32 scale is
used as float64(float32(scale)).
"""
from __future__ import annotations

import numpy as np

ATOL = 2e-2
RTOL = 1e-2


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def slot_mapping(cu_seqlens_q, kv_lens, block_tables, block_size: int) -> np.ndarray:
    """Cache slot of every packed token: the i-th new token of sequence s sits at position
    p = L_s - q_s + i and goes to slot table[s][p // bs] * bs + p % bs.
    """
    cu = [int(x) for x in cu_seqlens_q]
    out = np.empty(cu[-1], dtype=np.int64)
    bs = int(block_size)
    for s in range(len(cu) - 1):
        q = cu[s + 1] - cu[s]
        L = int(kv_lens[s])
        for i in range(q):
            p = L - q + i
            blk = int(block_tables[s][p // bs])
            out[cu[s] + i] = blk * bs + p % bs
    return out.astype(np.int32)


def cache_write(k_cache, v_cache, k, v, slots):
    """Copy of the caches after writing token t's K/V rows (all KV heads) into slot slots[t].
    A negative slot means "do not write". Bit copy: arrays are uint16 bf16 patterns.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb, bs, hkv, d = kc.shape
    kflat = kc.reshape(nb * bs, hkv, d)
    vflat = vc.reshape(nb * bs, hkv, d)
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if slot >= 0:
            kflat[slot] = k[t]
            vflat[slot] = v[t]
    return kc, vc


def unpage(cache, table_row, L: int, kv_head: int) -> np.ndarray:
    """Contiguous float64 [L, D] of one sequence's keys (or values) for one KV head,
    read position by position through the block table."""
    bs = cache.shape[1]
    p = np.arange(int(L))
    table_row = np.asarray(table_row, dtype=np.int64)
    rows = cache[table_row[p // bs], p % bs, kv_head]  # position p -> (block, offset)
    return bf16_to_f64(rows)


def _attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, last_key: np.ndarray, scale: float):
    """Dense masked softmax attention for query rows [R, D] over keys K/V [L, D]; row r may see
    keys 0..last_key[r]. Returns (out [R, D], lse [R]). Fully masked rows give (0, -inf)."""
    z = scale * (qrows @ K.T)
    j = np.arange(K.shape[0])[None, :]
    visible = j <= last_key[:, None]
    z = np.where(visible, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(z - m)
    ssum = w.sum(axis=1)
    out = (w @ V) / np.where(empty, 1.0, ssum)[:, None]
    lse = np.where(empty, -np.inf, m[:, 0] + np.log(np.where(empty, 1.0, ssum)))
    out[empty] = 0.0
    return out, lse


def paged_attention(q, cu_seqlens_q, kv_lens, block_tables, k_cache, v_cache, scale,
                    tokens=None, row_chunk: int = 512):
    """out [T, Hq, D] and lse [T, Hq] (float64) for the packed batch.

    ``q`` is uint16 bf16 [T, Hq, D]; caches are uint16 [num_blocks, bs, Hkv, D] and must
    already hold this step's K/V. ``tokens`` restricts the work to a subset of packed rows
    (others are left NaN). Rows are processed ``row_chunk`` tokens at a time only to bound
    memory; every row's softmax runs over its full key range.
    """
    cu = [int(x) for x in cu_seqlens_q]
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    want = np.ones(T, dtype=bool) if tokens is None else np.zeros(T, dtype=bool)
    if tokens is not None:
        want[np.asarray(tokens, dtype=np.int64)] = True
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    for s in range(len(cu) - 1):
        rows = np.nonzero(want[cu[s]:cu[s + 1]])[0]
        if rows.size == 0:
            continue
        qn = cu[s + 1] - cu[s]
        L = int(kv_lens[s])
        for g in range(Hkv):
            K = unpage(k_cache, block_tables[s], L, g)
            V = unpage(v_cache, block_tables[s], L, g)
            for c0 in range(0, rows.size, row_chunk):
                ii = rows[c0:c0 + row_chunk]
                t = cu[s] + ii
                Q = bf16_to_f64(q[t, g * G:(g + 1) * G]).reshape(-1, D)  # [len(ii) * G, D]
                last = np.repeat(L - qn + ii, G)
                o, l_ = _attend(Q, K, V, last, sc)
                out[t, g * G:(g + 1) * G] = o.reshape(len(ii), G, D)
                lse[t, g * G:(g + 1) * G] = l_.reshape(len(ii), G)
    return out, lse


def split_partials(q, cu_seqlens_q, kv_lens, block_tables, k_cache, v_cache, scale, bounds):
    """Per-range attention of every packed token over a partition of its sequence's keys.

    ``bounds[s]`` is a list of cut points 0 = b0 < b1 < ... < bn = L_s; range k is keys
    [b_k, b_{k+1}). Returns o [T, Hq, n_max, D], lse [T, Hq, n_max], nsplit [T]; unused
    ranges and fully masked ranges have lse = -inf and o = 0.
    """
    cu = [int(x) for x in cu_seqlens_q]
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    nmax = max(len(b) - 1 for b in bounds)
    o = np.zeros((T, Hq, nmax, D))
    lse = np.full((T, Hq, nmax), -np.inf)
    nsplit = np.zeros(T, dtype=np.int32)
    for s in range(len(cu) - 1):
        qn = cu[s + 1] - cu[s]
        L = int(kv_lens[s])
        b = [int(x) for x in bounds[s]]
        assert b[0] == 0 and b[-1] == L and all(x < y for x, y in zip(b, b[1:]))
        ii = np.arange(qn)
        t = cu[s] + ii
        nsplit[t] = len(b) - 1
        for g in range(Hkv):
            K = unpage(k_cache, block_tables[s], L, g)
            V = unpage(v_cache, block_tables[s], L, g)
            Q = bf16_to_f64(q[t, g * G:(g + 1) * G]).reshape(-1, D)
            last = np.repeat(L - qn + ii, G)
            for k in range(len(b) - 1):
                lo, hi = b[k], b[k + 1]
                # keys [lo, hi) only: shift the visibility limit into the range's own indices
                ok, ol = _attend(Q, K[lo:hi], V[lo:hi], last - lo, sc)
                o[t, g * G:(g + 1) * G, k] = ok.reshape(qn, G, D)
                lse[t, g * G:(g + 1) * G, k] = ol.reshape(qn, G)
    return o, lse, nsplit


def merge_partials(o_part, lse_part, num_splits):
    """Log-sum-exp merge: out = sum_k exp(lse_k - M) o_k / sum_k exp(lse_k - M), M = max_k lse_k,
    over the non-empty ranges among the first num_splits[t] of token t. A range with
    lse = -inf saw no key: it has no weight and its o (0/0, undefined) is never used. Rows with
    num_splits 0 are NaN."""
    T, Hq, nmax, D = o_part.shape
    out = np.full((T, Hq, D), np.nan)
    for t in range(T):
        n = int(num_splits[t])
        if n <= 0:
            continue
        l_ = lse_part[t, :, :n]
        nonempty = l_ > -np.inf
        M = np.where(nonempty, l_, -np.inf).max(axis=1, keepdims=True)
        M = np.where(np.isfinite(M), M, 0.0)
        w = np.where(nonempty, np.exp(np.where(nonempty, l_, 0.0) - M), 0.0)
        den = w.sum(axis=1)
        o = np.where(nonempty[:, :, None], o_part[t, :, :n], 0.0)
        num = (w[:, :, None] * o).sum(axis=1)
        out[t] = num / np.where(den > 0, den, 1.0)[:, None]
    return out


def within_tolerance(got, ref, atol: float = ATOL, rtol: float = RTOL):
    """Elementwise |got - ref| <= atol + rtol * |ref|; returns (ok, report dict)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    bad = ~(diff <= atol + rtol * np.abs(ref))  # NaN counts as bad
    big = np.abs(ref) > atol
    rel = np.where(big, diff / np.where(big, np.abs(ref), 1.0), 0.0)
    finite = np.isfinite(diff)
    report = {
        "max_abs": float(diff[finite].max()) if finite.any() else float("nan"),
        "max_rel": float(rel[finite].max()) if finite.any() else float("nan"),
        "n_bad": int(bad.sum()),
        "n_nan": int((~finite).sum()),
        "worst": (tuple(int(x) for x in np.unravel_index(np.argmax(np.where(finite, diff, -1.0)),
                                                         diff.shape))
                  if finite.any() else None),
    }
    return (not bad.any()), report
