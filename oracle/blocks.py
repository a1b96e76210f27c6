"""Oracle of the host block manager of the paged KV cache (test infrastructure only).

Plain Python, one step at a time, written from these passages:
  * "3.3 Batching & Memory Management", section "PagedAttention: block tables": the pool is
    split into physical blocks of bs tokens; a sequence's table maps its logical block j to the
    physical block holding positions [j*bs, (j+1)*bs); a new block is taken only when the last
    one is full.
  * same page, section "Sharing and copy-on-write": every block carries a reference count; a
    forked sequence shares all of its parent's blocks; before a sequence writes into a block
    whose count is above 1 it copies the block, points its table at the copy and decrements the
    original's count.
  * same page, section "Prefix caching and RadixAttention" (hash-based blocks): a full block is
    identified by its tokens together with everything before it; a new request reuses every
    leading block found; free cached blocks are evicted least recently used first.
  * "Continuous batching architecture", sections "Prefix caching" and "Eviction": freed blocks
    keep their content and key and count as free; cached blocks are given up only when the
    never-used blocks run out.
  * same page, section "Offloading" (and "Continuous batching in transformers", the offload
    paragraph): an offloaded request's KV blocks are copied to a pre-allocated pinned host pool,
    all requests that fit in one batched transfer, and copied back when space frees up, so the
    request resumes without recomputing its tokens; a request that does not fit is soft-reset.

Where the pages leave a choice open, the reading taken (the library follows the same one):
  * never-used blocks go out lowest id first; the cached pool is evicted least recently freed
    first (the chapter's LRU, not the transformers docs' most-recent-first demotion); a sequence
    frees its blocks last block first;
  * the block holding a prompt's last token is never reused (its KV is computed so that the
    step yields that token's output);
  * a block's key here is the exact token prefix it completes (the library hashes it and checks
    the hit), every block that completes a prefix is keyed, and a lookup takes the lowest id;
  * every block a transfer of the open step reads or writes (a copy's source and destination, a
    gather's source, a scatter's destination) stays out of the free pools until the step closes,
    even if its sequence lets it go, so no two transfers of one launch touch one block;
  * swap: every block of the victim is copied (shared ones too) into pool slots taken lowest id
    first; its blocks are released (held until the step closes, since the step's gather reads
    them); swap-in takes new blocks, releases the slots (held until the step
    closes), keys the full computed blocks again and counts them as written in the open step; a
    swapped sequence cannot be appended to, forked or batched until it is swapped in;
  * placeholder tokens (for async steps, "Continuous batching in transformers", Async batching:
    a step's input is built before the previous step's token is known): a sequence may hold
    placeholder tokens whose values are confirmed later, in order; a full block is keyed only
    once all its tokens are confirmed (and its KV computed), and a fork needs a fully confirmed
    parent;
  * the step protocol of the library header: KV is written by the GPU after the step closes,
    so keys become findable, copy sources leave the pools, and written blocks may be copied
    only after that; a copy whose source was written in the open step is refused; a sequence
    in the open step's batch cannot be freed; a fork needs a parent with no pending tokens.

``apply_step`` plays the GPU's part of a step on a simulated cache in which a slot holds the
tuple of tokens its KV depends on (the whole prefix through its position), so that
``check_views`` can verify by brute force that every sequence reads its own prefix back.
"""
from __future__ import annotations

import numpy as np

OK = 0
INVALID = -1
OUT_OF_BLOCKS = -5

FRESH, CACHED, USED, HELD = range(4)


class BlockError(Exception):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class BlockManagerOracle:
    def __init__(self, num_blocks: int, block_size: int):
        if block_size < 1 or num_blocks < 1:
            raise BlockError(INVALID, "sizes")
        self.nb, self.bs = num_blocks, block_size
        self.ref = [0] * num_blocks
        self.pending = [0] * num_blocks
        self.state = [FRESH] * num_blocks
        self.cached: list[int] = []            # least recently freed first
        self.key: list[tuple | None] = [None] * num_blocks
        self.visible = [False] * num_blocks
        self.dirty = [False] * num_blocks
        self.seqs: dict[int, dict] = {}
        self.copies: list[tuple[int, int]] = []
        self.step_blocks: list[int] = []
        self.step_seqs: list[int] = []
        self.kv = [[None] * block_size for _ in range(num_blocks)]  # simulated cache
        self.num_slots = 0
        self.slot_state: list[int] = []        # 0 free, 1 used, 2 held until the step closes
        self.swap_src: list[int] = []          # blocks the open step's gathers read
        self.pool: list[list] = []             # simulated host pool

    # -- pools ------------------------------------------------------------------------------
    def _available(self) -> int:
        return self.state.count(FRESH) + len(self.cached)

    def _take(self) -> int:
        fresh = [b for b in range(self.nb) if self.state[b] == FRESH]
        if fresh:
            b = min(fresh)
        else:
            b = self.cached.pop(0)
            self.key[b] = None
            self.visible[b] = False
        self.state[b] = USED
        self.ref[b] = 1
        return b

    def _add_ref(self, b: int):
        if self.state[b] == CACHED:
            self.cached.remove(b)
        self.state[b] = USED          # a held block found by a lookup is in use again
        self.ref[b] += 1

    def _to_pool(self, b: int):
        if self.pending[b] > 0:
            self.state[b] = HELD
        elif self.key[b] is not None:
            self.state[b] = CACHED
            self.cached.append(b)
        else:
            self.state[b] = FRESH

    def _release(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self._to_pool(b)

    def _lookup(self, prefix: tuple) -> int | None:
        hits = [b for b in range(self.nb) if self.visible[b] and self.key[b] == prefix]
        return min(hits) if hits else None

    def _seq(self, sid, swapped_ok: bool = False) -> dict:
        if sid not in self.seqs:
            raise BlockError(INVALID, "unknown sequence id")
        if self.seqs[sid].get("swapped") and not swapped_ok:
            raise BlockError(INVALID, "sequence is swapped out")
        return self.seqs[sid]

    # -- operations -------------------------------------------------------------------------
    def add_sequence(self, sid: int, tokens) -> int:
        tokens = [int(t) for t in tokens]
        n, bs = len(tokens), self.bs
        if n < 1:
            raise BlockError(INVALID, "empty prompt")
        if sid in self.seqs:
            raise BlockError(INVALID, "id in use")
        hits = []
        for j in range((n - 1) // bs):
            b = self._lookup(tuple(tokens[:(j + 1) * bs]))
            if b is None:
                break
            hits.append(b)
        nblocks = -(-n // bs)
        cached_hits = sum(1 for b in hits if self.state[b] == CACHED)
        if nblocks - len(hits) > self._available() - cached_hits:
            raise BlockError(OUT_OF_BLOCKS, "pool exhausted")
        table = []
        for b in hits:
            self._add_ref(b)
            table.append(b)
        while len(table) < nblocks:
            table.append(self._take())
        self.seqs[sid] = dict(tokens=tokens, table=table, computed=len(hits) * bs,
                              nkeys=len(hits), in_batch=False, confirmed=n)
        return len(hits) * bs

    def _key_blocks(self, s):
        """Keys the sequence's full blocks whose KV is computed and whose tokens are confirmed
        (found by lookups once the step closes)."""
        bs = self.bs
        for j in range(s["nkeys"], min(s["computed"], s["confirmed"]) // bs):
            b = s["table"][j]
            if self.key[b] is None:
                self.key[b] = tuple(s["tokens"][:(j + 1) * bs])
                self.visible[b] = False
                self.step_blocks.append(b)
        s["nkeys"] = max(s["nkeys"], min(s["computed"], s["confirmed"]) // bs)

    def append_tokens(self, sid: int, tokens, placeholders: bool = False):
        s = self._seq(sid)
        tokens = [int(t) for t in tokens]
        if not tokens:
            return
        bs, n = self.bs, len(s["tokens"])
        last = s["table"][-1]
        cow = n % bs != 0 and self.ref[last] > 1
        if cow and self.dirty[last]:
            raise BlockError(INVALID, "copy of a block written in the open step")
        nblocks = -(-(n + len(tokens)) // bs)
        if nblocks - len(s["table"]) + int(cow) > self._available():
            raise BlockError(OUT_OF_BLOCKS, "pool exhausted")
        if cow:
            dst = self._take()
            self.pending[last] += 1
            self.pending[dst] += 1      # a copy's destination is held until the step closes too
            self.ref[last] -= 1
            self.copies.append((last, dst))
            s["table"][-1] = dst
        if placeholders:
            tokens = [0] * len(tokens)
        elif s["confirmed"] == len(s["tokens"]):
            s["confirmed"] += len(tokens)
        s["tokens"].extend(tokens)
        while len(s["table"]) < nblocks:
            s["table"].append(self._take())

    def append_placeholders(self, sid: int, n: int):
        """n tokens whose values are not known yet (entered as 0)."""
        self.append_tokens(sid, [0] * int(n), placeholders=True)

    def confirm_tokens(self, sid: int, tokens):
        """The values of the next len(tokens) unconfirmed tokens, in order."""
        s = self._seq(sid, swapped_ok=True)
        tokens = [int(t) for t in tokens]
        c = s["confirmed"]
        if c + len(tokens) > len(s["tokens"]):
            raise BlockError(INVALID, "more values than unconfirmed tokens")
        s["tokens"][c:c + len(tokens)] = tokens
        s["confirmed"] = c + len(tokens)
        if not s.get("swapped"):
            self._key_blocks(s)

    def append_batch(self, seq_ids, counts, tokens):
        """append_tokens for each sequence in order until one is refused; returns how many were
        appended, or raises with .num_done set."""
        off = 0
        for i, (sid, n) in enumerate(zip(seq_ids, counts)):
            try:
                self.append_tokens(int(sid), list(tokens[off:off + int(n)]))
            except BlockError as e:
                e.num_done = i
                raise
            off += int(n)
        return len(seq_ids)

    def fork(self, parent: int, child: int):
        p = self._seq(parent)
        if child in self.seqs:
            raise BlockError(INVALID, "child id in use")
        if p["computed"] != len(p["tokens"]) or p["confirmed"] != len(p["tokens"]):
            raise BlockError(INVALID, "parent has tokens not yet computed or confirmed")
        c = dict(tokens=list(p["tokens"]), table=list(p["table"]), computed=p["computed"],
                 nkeys=p["nkeys"], in_batch=False, confirmed=p["confirmed"])
        for b in c["table"]:
            self._add_ref(b)
        self.seqs[child] = c

    def free_sequence(self, sid: int):
        s = self._seq(sid, swapped_ok=True)
        if s["in_batch"]:
            raise BlockError(INVALID, "sequence in the open step's batch")
        for b in reversed(s["table"]):
            self._release(b)
        for slot in s.get("slots", []):
            self.slot_state[slot] = 2
        del self.seqs[sid]

    # -- swap tier ----------------------------------------------------------------------------
    def set_swap_slots(self, n: int):
        if any(s.get("swapped") for s in self.seqs.values()) or n < 0:
            raise BlockError(INVALID, "cannot resize the pool now")
        self.num_slots = n
        self.slot_state = [0] * n
        self.pool = [[None] * self.bs for _ in range(n)]

    def swap_out(self, sid: int):
        """Copies every block of the sequence to pool slots; returns [(block, slot)]."""
        s = self._seq(sid)
        if s["in_batch"] or any(self.dirty[b] for b in s["table"]):
            raise BlockError(INVALID, "sequence has blocks written in the open step")
        free = [i for i in range(self.num_slots) if self.slot_state[i] == 0]
        if len(free) < len(s["table"]):
            raise BlockError(OUT_OF_BLOCKS, "swap pool full")
        pairs = list(zip(s["table"], free[:len(s["table"])]))
        for b, slot in pairs:
            self.slot_state[slot] = 1
            self.pending[b] += 1
            self.swap_src.append(b)
        for b in reversed(s["table"]):
            self._release(b)
        s["slots"] = [slot for _, slot in pairs]
        s["table"] = []
        s["swapped"] = True
        return pairs

    def swap_in(self, sid: int):
        """New blocks for a swapped sequence; returns [(slot, block)]."""
        s = self._seq(sid, swapped_ok=True)
        if not s.get("swapped"):
            raise BlockError(INVALID, "sequence is not swapped out")
        if len(s["slots"]) > self._available():
            raise BlockError(OUT_OF_BLOCKS, "pool exhausted")
        table = [self._take() for _ in s["slots"]]
        pairs = list(zip(s["slots"], table))
        for b in table:                  # the scatter's destinations are held like the gathers'
            self.pending[b] += 1
            self.swap_src.append(b)
        for slot in s["slots"]:
            self.slot_state[slot] = 2
        for b in table:
            self.dirty[b] = True
            self.step_blocks.append(b)
        s["table"], s["slots"], s["swapped"] = table, [], False
        s["nkeys"] = 0
        self._key_blocks(s)              # the computed, confirmed full blocks are keyed again
        return pairs

    def swap_stats(self):
        return (self.slot_state.count(0), self.slot_state.count(1), self.slot_state.count(2))

    def build_batch(self, seq_ids, q_lens, max_blocks_per_seq: int, token_capacity: int):
        """Returns (cu_seqlens_q, kv_lens, block_tables, slot_mapping, token_ids) as int32 arrays.
        The i-th batch row computes positions [computed, computed + q) of its sequence; position p
        is stored at slot table[p // bs] * bs + p % bs."""
        bs = self.bs
        seq_ids, q_lens = [int(x) for x in seq_ids], [int(x) for x in q_lens]
        seen = set()
        for sid, q in zip(seq_ids, q_lens):
            s = self._seq(sid)
            if sid in seen:
                raise BlockError(INVALID, "sequence twice in one batch")
            seen.add(sid)
            if not 1 <= q <= len(s["tokens"]) - s["computed"]:
                raise BlockError(INVALID, "bad q_len")
            if len(s["table"]) > max_blocks_per_seq:
                raise BlockError(INVALID, "table longer than max_blocks_per_seq")
            for j in range(s["computed"] // bs, (s["computed"] + q - 1) // bs + 1):
                if self.ref[s["table"][j]] != 1:
                    raise BlockError(INVALID, "a written block is shared")
        if sum(q_lens) > token_capacity:
            raise BlockError(INVALID, "token_capacity too small")
        S = len(seq_ids)
        cu = np.zeros(S + 1, np.int32)
        kv_lens = np.zeros(S, np.int32)
        tables = np.full((S, max_blocks_per_seq), -1, np.int32)
        slots, toks = [], []
        for i, (sid, q) in enumerate(zip(seq_ids, q_lens)):
            s = self.seqs[sid]
            p0 = s["computed"]
            for p in range(p0, p0 + q):
                b = s["table"][p // bs]
                slots.append(b * bs + p % bs)
                toks.append(s["tokens"][p])
                if not self.dirty[b]:
                    self.dirty[b] = True
                    self.step_blocks.append(b)
            cu[i + 1] = len(slots)
            kv_lens[i] = p0 + q
            tables[i, :len(s["table"])] = s["table"]
            s["computed"] = p0 + q
            self._key_blocks(s)
            if not s["in_batch"]:
                s["in_batch"] = True
                self.step_seqs.append(sid)
        return cu, kv_lens, tables, np.array(slots, np.int32), np.array(toks, np.int32)

    def take_copies(self, capacity: int | None = None):
        """Closes the step; returns the pending (src, dst) copies in the order they were made."""
        if capacity is not None and len(self.copies) > capacity:
            raise BlockError(INVALID, "capacity too small")
        out = list(self.copies)
        for src in [b for pair in out for b in pair] + self.swap_src:
            self.pending[src] -= 1
            if self.pending[src] == 0 and self.state[src] == HELD:
                self._to_pool(src)
        self.swap_src = []
        self.slot_state = [0 if st == 2 else st for st in self.slot_state]
        for b in self.step_blocks:
            self.dirty[b] = False
            if self.key[b] is not None:
                self.visible[b] = True
        for sid in self.step_seqs:
            if sid in self.seqs:
                self.seqs[sid]["in_batch"] = False
        self.copies, self.step_blocks, self.step_seqs = [], [], []
        return out

    # -- views ------------------------------------------------------------------------------
    def stats(self):
        held = sum(1 for b in range(self.nb) if self.state[b] == HELD)
        return self.state.count(FRESH), len(self.cached), held, len(self.seqs)

    def block_table(self, sid) -> list[int]:
        return list(self._seq(sid, swapped_ok=True)["table"])

    def sequence_info(self, sid):
        s = self._seq(sid, swapped_ok=True)
        return len(s["tokens"]), s["computed"], len(s["table"])

    # -- the GPU's part of a step, simulated -------------------------------------------------
    def apply_step(self, copies, batch, swap_outs=(), swap_ins=(), real=None):
        """Copies first (whole blocks), then the swap gathers (block -> pool slot) and scatters
        (pool slot -> block), then the batch's new KV at its slots: the KV of the token at
        position p of a sequence is the tuple of that sequence's tokens 0..p."""
        for src, dst in copies:
            self.kv[dst] = list(self.kv[src])
        for b, slot in swap_outs:
            self.pool[slot] = list(self.kv[b])
        for slot, b in swap_ins:
            self.kv[b] = list(self.pool[slot])
        seq_ids, cu, slots = batch
        bs = self.bs
        for i, sid in enumerate(seq_ids):
            s = self.seqs[sid]
            toks = real[sid] if real is not None else s["tokens"]   # the GPU sees real tokens
            q = int(cu[i + 1] - cu[i])
            p0 = s["computed"] - q
            for k in range(q):
                p = p0 + k
                sl = int(slots[cu[i] + k])
                self.kv[sl // bs][sl % bs] = tuple(toks[:p + 1])

    def check_views(self, real=None):
        """Brute force: every computed position of every live sequence reads its own prefix
        (real token values where the manager holds placeholders)."""
        bs = self.bs
        for sid, s in self.seqs.items():
            if s.get("swapped"):
                continue
            toks = real[sid] if real is not None else s["tokens"]
            for p in range(s["computed"]):
                b = s["table"][p // bs]
                if self.kv[b][p % bs] != tuple(toks[:p + 1]):
                    return f"sequence {sid} position {p} reads the wrong KV (block {b})"
        return None

    def check_counts(self):
        """Reference counts equal the table entries that name each block; pool states agree."""
        count = [0] * self.nb
        for s in self.seqs.values():
            for b in s["table"]:
                count[b] += 1
        if count != self.ref:
            return "reference counts differ from table entries"
        for b in range(self.nb):
            st = self.state[b]
            if (st == USED) != (self.ref[b] > 0):
                return f"block {b}: state {st} with ref {self.ref[b]}"
            if st == HELD and self.pending[b] == 0:
                return f"block {b} held without a pending copy"
            if st == CACHED and (self.key[b] is None or b not in self.cached):
                return f"block {b} cached without a key"
        if len(set(self.cached)) != len(self.cached):
            return "a block is cached twice"
        return None


def copy_blocks(k_cache, v_cache, src, dst):
    """Copies of the caches after the copy-on-write copies: block dst[i] of K and of V becomes
    block src[i] ("Sharing and copy-on-write": the engine copies the shared block before the
    write). Arrays [..., num_blocks, bs, Hkv, D] (a leading layer axis is allowed); pairs with an
    id outside [0, num_blocks) or src == dst are skipped, as the library does. Pairs are applied
    from the originals, so the result does not depend on their order when no dst is a src."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    nb = kc.shape[-4]
    for s, d in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        if 0 <= s < nb and 0 <= d < nb and s != d:
            kc[..., d, :, :, :] = k_cache[..., s, :, :, :]
            vc[..., d, :, :, :] = v_cache[..., s, :, :, :]
    return kc, vc


def swap_out_blocks(k_cache, v_cache, blocks, slots, pool):
    """Pool after the swap-out gather ("Continuous batching architecture", Offloading: the
    request's blocks are copied to the pinned host pool): slot slots[i] takes block blocks[i] of
    K and of V in every layer. Caches [..., num_blocks, bs, Hkv, D] (leading layer axis allowed),
    pool [num_slots, 2, layers, bs, Hkv, D]; pairs with an id out of range are skipped."""
    out = np.array(pool, copy=True)
    kc, vc = np.asarray(k_cache), np.asarray(v_cache)
    if kc.ndim == 4:
        kc, vc = kc[None], vc[None]
    nb, ns = kc.shape[1], out.shape[0]
    for b, sl in zip(np.asarray(blocks).tolist(), np.asarray(slots).tolist()):
        if 0 <= b < nb and 0 <= sl < ns:
            out[sl, 0] = kc[:, b]
            out[sl, 1] = vc[:, b]
    return out


def swap_in_blocks(pool, slots, blocks, k_cache, v_cache):
    """Caches after the swap-in scatter (the blocks are copied back to the GPU): block blocks[i]
    takes slot slots[i] of K and of V in every layer; out-of-range pairs are skipped."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    kv, vv = (kc[None], vc[None]) if kc.ndim == 4 else (kc, vc)
    p = np.asarray(pool)
    nb, ns = kv.shape[1], p.shape[0]
    for sl, b in zip(np.asarray(slots).tolist(), np.asarray(blocks).tolist()):
        if 0 <= b < nb and 0 <= sl < ns:
            kv[:, b] = p[sl, 0]
            vv[:, b] = p[sl, 1]
    return kc, vc
