// Host block manager: the paged KV pool's allocator with reference counts, copy-on-write of a
// shared partial block, reuse of content-keyed full blocks across requests, and the step's
// batch metadata (cu_seqlens_q, kv_lens, block tables, slot mapping) for the attention kernels.
//
// Pages: "3.3 Batching & Memory Management" (PagedAttention: block tables; Sharing and
// copy-on-write; Prefix caching and RadixAttention, the hash-based variant) and "Continuous
// batching architecture" (Prefix caching; Eviction). Policies the pages leave open, fixed here
// so that the result is deterministic:
//   - never-used blocks are handed out lowest id first;
//   - a freed block that holds a keyed full block stays cached; when no never-used block is
//     left, the least recently freed cached block is evicted and loses its key (the chapter's
//     LRU; the transformers docs demote the most recent instead);
//   - a sequence frees its blocks last block first, so its prefix is evicted last;
//   - admission reuses the leading full blocks whose prefix is cached, short of the block that
//     holds the prompt's last token (that token is always computed);
//   - a full block is keyed once its KV is computed (blocks holding the same prefix are all
//     keyed; a lookup takes the lowest id) and is found by lookups only after the step that
//     computes it has closed;
//   - every block a transfer of the open step reads or writes (a copy's source and destination,
//     a gather's source, a scatter's destination) stays out of the free pools until the step
//     closes, even if its sequence lets it go, so no two transfers of one launch touch one block;
//   - swap tier ("Continuous batching architecture", Offloading): a swap-out copies every block
//     of the sequence to host pool slots (lowest free id first) and releases the blocks, held
//     until the step closes because the step's gather reads them; a swap-in takes new blocks,
//     releases the slots (held until the step closes), keys the computed full blocks again and
//     counts the blocks as written in the open step.
// A full block's key is a chained 64-bit FNV-1a hash of its parent's key and its own tokens; a
// hit is verified against the block's tokens and its parent's key.

#include <algorithm>
#include <cstring>
#include <list>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "cb_internal.h"
#include "cbblocks.h"

struct cb_block_manager {
  struct Seq {
    std::vector<int32_t> tokens;
    std::vector<int32_t> table;
    std::vector<uint64_t> keys;  // chained key of each leading full block whose KV is computed
    int64_t computed = 0;        // leading positions whose KV is computed or in a built batch
    bool in_batch = false;       // part of a batch built since the step last closed
    uint64_t stamp = 0;          // the last cb_bm_build_batch call that named this sequence
    int64_t confirmed = 0;       // leading tokens whose values are known (not placeholders)
    bool swapped = false;        // its blocks live in host pool slots
    std::vector<int32_t> slots;  // those slots, in table order
  };

  int64_t num_blocks = 0;
  int32_t bs = 0;
  std::vector<int32_t> ref;       // table entries referencing each block
  std::vector<int32_t> pending;   // pending copies reading each block
  std::vector<uint8_t> state;     // kFresh, kCached, kUsed, kHeld
  std::set<int32_t> fresh;        // free blocks without a key, lowest id first
  std::list<int32_t> lru;         // free keyed blocks, least recently freed first
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::unordered_multimap<uint64_t, int32_t> by_key;
  std::vector<uint8_t> keyed, visible, dirty;
  std::vector<uint64_t> key, parent_key;
  std::vector<int32_t> key_tokens;  // bs tokens per keyed block
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int32_t> copy_src, copy_dst;  // pending copy-on-write block copies
  std::vector<int32_t> step_blocks;         // blocks keyed or written in the open step
  std::vector<int64_t> step_seqs;           // sequences in batches of the open step
  int64_t held = 0;                         // blocks in state kHeld
  uint64_t build_calls = 0;                 // cb_bm_build_batch calls so far
  std::vector<Seq*> batch;                  // scratch of cb_bm_build_batch
  // swap pool
  std::vector<uint8_t> slot_state;          // 0 free, 1 used, 2 held until the step closes
  std::set<int32_t> free_slots;
  std::vector<int32_t> held_slots;          // released in the open step
  std::vector<int32_t> swap_src;            // blocks the open step's gathers and scatters use
  int64_t swapped_seqs = 0;
};

namespace {

using Mgr = cb_block_manager;
enum : uint8_t { kFresh = 0, kCached = 1, kUsed = 2, kHeld = 3 };
constexpr int E = CB_ERR_INVALID_ARG;
constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull, kFnvPrime = 0x100000001b3ull;

// FNV-1a over the parent key's 8 bytes and the block's tokens as 4-byte little-endian words
uint64_t block_key(uint64_t parent, const int32_t* tok, int32_t bs) {
  uint64_t h = kFnvOffset;
  for (int i = 0; i < 8; ++i) {
    h ^= (parent >> (8 * i)) & 0xff;
    h *= kFnvPrime;
  }
  for (int32_t t = 0; t < bs; ++t) {
    const uint32_t w = static_cast<uint32_t>(tok[t]);
    for (int i = 0; i < 4; ++i) {
      h ^= (w >> (8 * i)) & 0xff;
      h *= kFnvPrime;
    }
  }
  return h;
}

int64_t available(const Mgr* m) { return (int64_t)m->fresh.size() + (int64_t)m->lru.size(); }

void drop_key(Mgr* m, int32_t b) {
  if (!m->keyed[b]) return;
  auto range = m->by_key.equal_range(m->key[b]);
  for (auto it = range.first; it != range.second; ++it)
    if (it->second == b) {
      m->by_key.erase(it);
      break;
    }
  m->keyed[b] = m->visible[b] = 0;
}

// A never-used block if any is left, else the least recently freed cached one (its key is
// dropped). The caller has checked that one is available.
int32_t take_block(Mgr* m) {
  int32_t b;
  if (!m->fresh.empty()) {
    b = *m->fresh.begin();
    m->fresh.erase(m->fresh.begin());
  } else {
    b = m->lru.front();
    m->lru.pop_front();
    drop_key(m, b);
  }
  m->state[b] = kUsed;
  m->ref[b] = 1;
  return b;
}

void add_ref(Mgr* m, int32_t b) {
  if (m->state[b] == kCached) m->lru.erase(m->lru_pos[b]);
  if (m->state[b] == kHeld) --m->held;  // a held block found by a lookup is in use again
  m->state[b] = kUsed;
  ++m->ref[b];
}

// A block no table references goes back to a pool, or is held while a pending copy reads it.
void to_pool(Mgr* m, int32_t b) {
  if (m->pending[b] > 0) {
    m->state[b] = kHeld;
    ++m->held;
  } else if (m->keyed[b]) {
    m->state[b] = kCached;
    m->lru_pos[b] = m->lru.insert(m->lru.end(), b);
  } else {
    m->state[b] = kFresh;
    m->fresh.insert(b);
  }
}

void release(Mgr* m, int32_t b) {
  if (--m->ref[b] == 0) to_pool(m, b);
}

// The lowest-id keyed block holding the block (parent, tokens), or -1; `visible_only` skips
// blocks keyed in the open step, whose KV is not written yet.
int32_t find_block(const Mgr* m, uint64_t k, uint64_t parent, const int32_t* tok, bool visible_only) {
  int32_t best = -1;
  auto range = m->by_key.equal_range(k);
  for (auto it = range.first; it != range.second; ++it) {
    const int32_t b = it->second;
    if ((visible_only && !m->visible[b]) || (best >= 0 && b > best)) continue;
    if (m->parent_key[b] == parent &&
        std::memcmp(&m->key_tokens[(size_t)b * m->bs], tok, sizeof(int32_t) * m->bs) == 0)
      best = b;
  }
  return best;
}

Mgr::Seq* find_seq(Mgr* m, int64_t id) {
  auto it = m->seqs.find(id);
  return it == m->seqs.end() ? nullptr : &it->second;
}

// Extends the keys of the sequence's full blocks whose KV is computed and whose tokens are all
// confirmed, and keys each such block (visible to lookups once the step closes). Blocks holding
// the same prefix are all keyed, so evicting one leaves the others findable.
void key_computed_blocks(Mgr* m, Mgr::Seq& s) {
  const int32_t bs = m->bs;
  const int64_t full = std::min(s.computed, s.confirmed) / bs;
  for (int64_t j = (int64_t)s.keys.size(); j < full; ++j) {
    const uint64_t parent = j ? s.keys[j - 1] : 0;
    const int32_t* tok = s.tokens.data() + j * bs;
    const uint64_t k = block_key(parent, tok, bs);
    s.keys.push_back(k);
    const int32_t b = s.table[j];
    if (m->keyed[b]) continue;
    m->keyed[b] = 1;
    m->visible[b] = 0;
    m->key[b] = k;
    m->parent_key[b] = parent;
    std::memcpy(&m->key_tokens[(size_t)b * bs], tok, sizeof(int32_t) * bs);
    m->by_key.emplace(k, b);
    m->step_blocks.push_back(b);
  }
}

}  // namespace

extern "C" int cb_bm_create(int64_t num_blocks, int32_t block_size, cb_block_manager** out) {
  if (!out) return cb::fail(E, "out is NULL");
  *out = nullptr;
  if (block_size < 1) return cb::fail(E, "block_size must be >= 1");
  if (num_blocks < 1 || num_blocks * (int64_t)block_size > INT32_MAX)
    return cb::fail(E, "num_blocks must be >= 1 with num_blocks * block_size < 2^31");
  Mgr* m = new (std::nothrow) Mgr;
  if (!m) return cb::fail(E, "out of host memory");
  try {
    m->num_blocks = num_blocks;
    m->bs = block_size;
    m->ref.assign(num_blocks, 0);
    m->pending.assign(num_blocks, 0);
    m->state.assign(num_blocks, kFresh);
    m->lru_pos.resize(num_blocks);
    m->keyed.assign(num_blocks, 0);
    m->visible.assign(num_blocks, 0);
    m->dirty.assign(num_blocks, 0);
    m->key.assign(num_blocks, 0);
    m->parent_key.assign(num_blocks, 0);
    m->key_tokens.assign((size_t)num_blocks * block_size, 0);
    for (int64_t b = 0; b < num_blocks; ++b) m->fresh.insert(m->fresh.end(), (int32_t)b);
  } catch (const std::bad_alloc&) {
    delete m;
    return cb::fail(E, "out of host memory");
  }
  *out = m;
  return cb::ok();
}

extern "C" void cb_bm_destroy(cb_block_manager* m) { delete m; }

extern "C" int cb_bm_add_sequence(cb_block_manager* m, int64_t seq_id, const int32_t* tokens,
                                  int32_t num_tokens, int32_t* num_cached) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (num_tokens < 1) return cb::fail(E, "a prompt needs at least one token");
  if (!tokens) return cb::fail(E, "tokens is NULL");
  if (m->seqs.count(seq_id)) return cb::fail(E, "sequence id already in use");
  const int32_t bs = m->bs;
  const int64_t nblocks = cb::ceil_div(num_tokens, bs);
  std::vector<int32_t> hit;
  std::vector<uint64_t> keys;
  uint64_t parent = 0;
  for (int64_t j = 0; j < (int64_t)(num_tokens - 1) / bs; ++j) {
    const int32_t* tok = tokens + j * bs;
    const uint64_t k = block_key(parent, tok, bs);
    const int32_t b = find_block(m, k, parent, tok, true);
    if (b < 0) break;
    hit.push_back(b);
    keys.push_back(k);
    parent = k;
  }
  int64_t cached_hits = 0;  // hits that sit in the cached pool leave it
  for (int32_t b : hit) cached_hits += m->state[b] == kCached;
  if (nblocks - (int64_t)hit.size() > available(m) - cached_hits)
    return cb::fail(CB_ERR_OUT_OF_BLOCKS, "not enough free KV blocks for the prompt");
  Mgr::Seq s;
  s.tokens.assign(tokens, tokens + num_tokens);
  s.table.reserve(nblocks);
  for (int32_t b : hit) {
    add_ref(m, b);
    s.table.push_back(b);
  }
  while ((int64_t)s.table.size() < nblocks) s.table.push_back(take_block(m));
  s.keys = std::move(keys);
  s.computed = (int64_t)hit.size() * bs;
  s.confirmed = num_tokens;
  m->seqs.emplace(seq_id, std::move(s));
  if (num_cached) *num_cached = (int32_t)(hit.size() * bs);
  return cb::ok();
}

namespace {

// Appends num_tokens tokens (values from `tokens`, or placeholders 0 whose values come later).
int append_impl(Mgr* m, int64_t seq_id, const int32_t* tokens, int32_t num_tokens, bool placeholders) {
  if (num_tokens < 0) return cb::fail(E, "num_tokens must be >= 0");
  if (num_tokens > 0 && !tokens && !placeholders) return cb::fail(E, "tokens is NULL");
  Mgr::Seq* s = find_seq(m, seq_id);
  if (!s) return cb::fail(E, "unknown sequence id");
  if (s->swapped) return cb::fail(E, "sequence is swapped out");
  if (num_tokens == 0) return cb::ok();
  const int32_t bs = m->bs;
  const int64_t len = (int64_t)s->tokens.size();
  if (len + num_tokens > INT32_MAX) return cb::fail(E, "sequence longer than 2^31 - 1 tokens");
  const bool cow = len % bs != 0 && m->ref[s->table.back()] > 1;
  if (cow && m->dirty[s->table.back()])
    return cb::fail(E, "copy-on-write of a block written in the open step: close the step "
                       "(cb_bm_take_copies) before appending to this sequence");
  const int64_t nblocks = cb::ceil_div(len + num_tokens, bs);
  const int64_t need = nblocks - (int64_t)s->table.size() + (cow ? 1 : 0);
  if (need > available(m)) return cb::fail(CB_ERR_OUT_OF_BLOCKS, "not enough free KV blocks to append");
  if (cow) {  // the shared partial block: copy it and point this table at the copy
    const int32_t src = s->table.back();
    const int32_t dst = take_block(m);
    ++m->pending[src];
    ++m->pending[dst];  // the destination too is held until the step closes
    --m->ref[src];  // others still hold it: it stays in use
    m->copy_src.push_back(src);
    m->copy_dst.push_back(dst);
    s->table.back() = dst;
  }
  if (placeholders) {
    s->tokens.insert(s->tokens.end(), num_tokens, 0);
  } else {
    if (s->confirmed == len) s->confirmed += num_tokens;
    s->tokens.insert(s->tokens.end(), tokens, tokens + num_tokens);
  }
  while ((int64_t)s->table.size() < nblocks) s->table.push_back(take_block(m));
  return cb::ok();
}

}  // namespace

extern "C" int cb_bm_append_tokens(cb_block_manager* m, int64_t seq_id, const int32_t* tokens,
                                   int32_t num_tokens) {
  if (!m) return cb::fail(E, "manager is NULL");
  return append_impl(m, seq_id, tokens, num_tokens, false);
}

extern "C" int cb_bm_append_placeholders(cb_block_manager* m, int64_t seq_id, int32_t num_tokens) {
  if (!m) return cb::fail(E, "manager is NULL");
  return append_impl(m, seq_id, nullptr, num_tokens, true);
}

extern "C" int cb_bm_confirm_tokens(cb_block_manager* m, int64_t seq_id, const int32_t* tokens,
                                    int32_t num_tokens) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) return cb::fail(E, "bad tokens");
  Mgr::Seq* s = find_seq(m, seq_id);
  if (!s) return cb::fail(E, "unknown sequence id");
  if (s->confirmed + num_tokens > (int64_t)s->tokens.size())
    return cb::fail(E, "more values than unconfirmed tokens");
  std::copy(tokens, tokens + num_tokens, s->tokens.begin() + s->confirmed);
  s->confirmed += num_tokens;
  if (!s->swapped) key_computed_blocks(m, *s);
  return cb::ok();
}

extern "C" int cb_bm_append_batch(cb_block_manager* m, const int64_t* seq_ids,
                                  const int32_t* counts, const int32_t* tokens, int32_t num_seqs,
                                  int32_t* num_done) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (!num_done) return cb::fail(E, "num_done is NULL");
  *num_done = 0;
  if (num_seqs < 0) return cb::fail(E, "num_seqs must be >= 0");
  if (num_seqs > 0 && (!seq_ids || !counts)) return cb::fail(E, "NULL array");
  int64_t off = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    // tokens NULL: every appended token is a placeholder
    const int st = append_impl(m, seq_ids[i], tokens ? tokens + off : nullptr, counts[i], !tokens);
    if (st != CB_OK) return st;
    off += counts[i];
    *num_done = i + 1;
  }
  return cb::ok();
}

extern "C" int cb_bm_confirm_batch(cb_block_manager* m, const int64_t* seq_ids,
                                   const int32_t* counts, const int32_t* tokens, int32_t num_seqs,
                                   int32_t* num_done) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (!num_done) return cb::fail(E, "num_done is NULL");
  *num_done = 0;
  if (num_seqs < 0) return cb::fail(E, "num_seqs must be >= 0");
  if (num_seqs > 0 && (!seq_ids || !counts || !tokens)) return cb::fail(E, "NULL array");
  int64_t off = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int st = cb_bm_confirm_tokens(m, seq_ids[i], tokens + off, counts[i]);
    if (st != CB_OK) return st;
    off += counts[i];
    *num_done = i + 1;
  }
  return cb::ok();
}

extern "C" int cb_bm_fork(cb_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return cb::fail(E, "manager is NULL");
  Mgr::Seq* p = find_seq(m, parent);
  if (!p) return cb::fail(E, "unknown parent sequence id");
  if (p->swapped) return cb::fail(E, "parent sequence is swapped out");
  if (m->seqs.count(child)) return cb::fail(E, "child sequence id already in use");
  if (p->computed != (int64_t)p->tokens.size() || p->confirmed != (int64_t)p->tokens.size())
    return cb::fail(E, "fork needs a parent whose every token is confirmed and computed or in a built batch");
  Mgr::Seq c = *p;
  c.in_batch = false;
  for (int32_t b : c.table) add_ref(m, b);
  m->seqs.emplace(child, std::move(c));
  return cb::ok();
}

extern "C" int cb_bm_free_sequence(cb_block_manager* m, int64_t seq_id) {
  if (!m) return cb::fail(E, "manager is NULL");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return cb::fail(E, "unknown sequence id");
  if (it->second.in_batch)
    return cb::fail(E, "sequence is in a batch of the open step: close the step first");
  const auto& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) release(m, *b);
  for (int32_t slot : it->second.slots) {
    m->slot_state[slot] = 2;
    m->held_slots.push_back(slot);
  }
  if (it->second.swapped) --m->swapped_seqs;
  m->seqs.erase(it);
  return cb::ok();
}

extern "C" int cb_bm_set_swap_slots(cb_block_manager* m, int64_t num_slots) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (num_slots < 0 || num_slots > INT32_MAX) return cb::fail(E, "num_slots must be in [0, 2^31 - 1]");
  if (m->swapped_seqs > 0 || !m->held_slots.empty())
    return cb::fail(E, "the swap pool cannot be resized while it holds data");
  m->slot_state.assign(num_slots, 0);
  m->free_slots.clear();
  for (int64_t i = 0; i < num_slots; ++i) m->free_slots.insert(m->free_slots.end(), (int32_t)i);
  return cb::ok();
}

extern "C" int cb_bm_swap_out(cb_block_manager* m, int64_t seq_id, int32_t* blocks, int32_t* slots,
                              int32_t capacity, int32_t* num_pairs) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (!num_pairs) return cb::fail(E, "num_pairs is NULL");
  *num_pairs = 0;
  Mgr::Seq* s = find_seq(m, seq_id);
  if (!s) return cb::fail(E, "unknown sequence id");
  if (s->swapped) return cb::fail(E, "sequence is swapped out");
  bool dirty = s->in_batch;
  for (int32_t b : s->table) dirty = dirty || m->dirty[b];
  if (dirty) return cb::fail(E, "sequence has blocks written in the open step: close the step first");
  const int32_t n = (int32_t)s->table.size();
  if (n > capacity || (n > 0 && (!blocks || !slots)))
    return cb::fail(E, "the output arrays hold fewer entries than the sequence's blocks");
  if ((int64_t)m->free_slots.size() < n) return cb::fail(CB_ERR_OUT_OF_BLOCKS, "swap pool full");
  s->slots.resize(n);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t slot = *m->free_slots.begin();
    m->free_slots.erase(m->free_slots.begin());
    m->slot_state[slot] = 1;
    const int32_t b = s->table[j];
    ++m->pending[b];
    m->swap_src.push_back(b);
    blocks[j] = b;
    slots[j] = slot;
    s->slots[j] = slot;
  }
  for (auto b = s->table.rbegin(); b != s->table.rend(); ++b) release(m, *b);
  s->table.clear();
  s->swapped = true;
  ++m->swapped_seqs;
  *num_pairs = n;
  return cb::ok();
}

extern "C" int cb_bm_swap_in(cb_block_manager* m, int64_t seq_id, int32_t* slots, int32_t* blocks,
                             int32_t capacity, int32_t* num_pairs) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (!num_pairs) return cb::fail(E, "num_pairs is NULL");
  *num_pairs = 0;
  Mgr::Seq* s = find_seq(m, seq_id);
  if (!s) return cb::fail(E, "unknown sequence id");
  if (!s->swapped) return cb::fail(E, "sequence is not swapped out");
  const int32_t n = (int32_t)s->slots.size();
  if (n > available(m)) return cb::fail(CB_ERR_OUT_OF_BLOCKS, "not enough free KV blocks to swap in");
  if (n > capacity || (n > 0 && (!blocks || !slots)))
    return cb::fail(E, "the output arrays hold fewer entries than the sequence's slots");
  s->table.resize(n);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t b = take_block(m);
    s->table[j] = b;
    slots[j] = s->slots[j];
    blocks[j] = b;
    ++m->pending[b];  // the scatter's destination is held until the step closes
    m->swap_src.push_back(b);
    m->slot_state[s->slots[j]] = 2;
    m->held_slots.push_back(s->slots[j]);
    if (!m->dirty[b]) {
      m->dirty[b] = 1;
      m->step_blocks.push_back(b);
    }
  }
  s->slots.clear();
  s->swapped = false;
  --m->swapped_seqs;
  s->keys.clear();  // the computed full blocks are keyed again (found once the step closes)
  key_computed_blocks(m, *s);
  *num_pairs = n;
  return cb::ok();
}

extern "C" int cb_bm_swap_stats(const cb_block_manager* m, int64_t* free_slots, int64_t* used_slots,
                                int64_t* held_slots) {
  if (!m) return cb::fail(E, "manager is NULL");
  int64_t used = 0, held = 0;
  for (uint8_t st : m->slot_state) {
    used += st == 1;
    held += st == 2;
  }
  if (free_slots) *free_slots = (int64_t)m->free_slots.size();
  if (used_slots) *used_slots = used;
  if (held_slots) *held_slots = held;
  return cb::ok();
}

extern "C" int cb_bm_build_batch(cb_block_manager* m, const int64_t* seq_ids, const int32_t* q_lens,
                                 int32_t num_seqs, int32_t max_blocks_per_seq, int32_t token_capacity,
                                 int32_t* cu_seqlens_q, int32_t* kv_lens, int32_t* block_tables,
                                 int32_t* slot_mapping, int32_t* token_ids) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (num_seqs < 0 || max_blocks_per_seq < 1 || token_capacity < 0)
    return cb::fail(E, "num_seqs and token_capacity must be >= 0, max_blocks_per_seq >= 1");
  if (!cu_seqlens_q) return cb::fail(E, "cu_seqlens_q is NULL");
  if (num_seqs > 0 && (!seq_ids || !q_lens || !kv_lens || !block_tables || !slot_mapping))
    return cb::fail(E, "NULL array");
  auto& ss = m->batch;
  ss.resize(num_seqs);
  const uint64_t stamp = ++m->build_calls;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Mgr::Seq* s = ss[i] = find_seq(m, seq_ids[i]);
    if (!s) return cb::fail(E, "unknown sequence id");
    if (s->swapped) return cb::fail(E, "sequence is swapped out");
    if (s->stamp == stamp) return cb::fail(E, "a sequence appears twice in the batch");
    s->stamp = stamp;
    const int64_t left = (int64_t)s->tokens.size() - s->computed;
    if (q_lens[i] < 1 || q_lens[i] > left)
      return cb::fail(E, "q_len must be in [1, tokens not yet computed]");
    if ((int64_t)s->table.size() > max_blocks_per_seq)
      return cb::fail(E, "a block table is longer than max_blocks_per_seq");
    for (int64_t j = s->computed / m->bs; j <= (s->computed + q_lens[i] - 1) / m->bs; ++j)
      if (m->ref[s->table[j]] != 1) return cb::fail(E, "internal: a written block is shared");
    total += q_lens[i];
  }
  if (total > token_capacity) return cb::fail(E, "token_capacity is below the batch's token count");
  int64_t t = 0;
  cu_seqlens_q[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Mgr::Seq& s = *ss[i];
    const int64_t p0 = s.computed, p1 = s.computed + q_lens[i];
    for (int64_t p = p0; p < p1; ++p, ++t) {
      const int32_t b = s.table[p / m->bs];
      slot_mapping[t] = (int32_t)((int64_t)b * m->bs + p % m->bs);
      if (token_ids) token_ids[t] = s.tokens[p];
      if (!m->dirty[b]) {
        m->dirty[b] = 1;
        m->step_blocks.push_back(b);
      }
    }
    cu_seqlens_q[i + 1] = (int32_t)t;
    kv_lens[i] = (int32_t)p1;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    std::memcpy(row, s.table.data(), sizeof(int32_t) * s.table.size());  // the rest is not read
    s.computed = p1;
    key_computed_blocks(m, s);
    if (!s.in_batch) {
      s.in_batch = true;
      m->step_seqs.push_back(seq_ids[i]);
    }
  }
  return cb::ok();
}

extern "C" int cb_bm_take_copies(cb_block_manager* m, int32_t* src, int32_t* dst, int32_t capacity,
                                 int32_t* num_copies) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (!num_copies) return cb::fail(E, "num_copies is NULL");
  const int64_t n = (int64_t)m->copy_src.size();
  *num_copies = (int32_t)n;
  if (n > capacity || (n > 0 && (!src || !dst)))
    return cb::fail(E, "the copy arrays hold fewer entries than the pending copies");
  for (int64_t i = 0; i < n; ++i) {
    src[i] = m->copy_src[i];
    dst[i] = m->copy_dst[i];
  }
  for (int64_t i = 0; i < 2 * n + (int64_t)m->swap_src.size(); ++i) {
    const int32_t b = i < n ? m->copy_src[i] : i < 2 * n ? m->copy_dst[i - n] : m->swap_src[i - 2 * n];
    if (--m->pending[b] == 0 && m->state[b] == kHeld) {
      --m->held;
      to_pool(m, b);
    }
  }
  m->swap_src.clear();
  for (int32_t slot : m->held_slots) {
    m->slot_state[slot] = 0;
    m->free_slots.insert(slot);
  }
  m->held_slots.clear();
  for (int32_t b : m->step_blocks) {
    m->dirty[b] = 0;
    if (m->keyed[b]) m->visible[b] = 1;
  }
  for (int64_t id : m->step_seqs) {
    Mgr::Seq* s = find_seq(m, id);
    if (s) s->in_batch = false;
  }
  m->copy_src.clear();
  m->copy_dst.clear();
  m->step_blocks.clear();
  m->step_seqs.clear();
  return cb::ok();
}

extern "C" int cb_bm_sequence_info(const cb_block_manager* m, int64_t seq_id, int64_t* num_tokens,
                                   int64_t* num_computed, int32_t* num_blocks) {
  if (!m) return cb::fail(E, "manager is NULL");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return cb::fail(E, "unknown sequence id");
  if (num_tokens) *num_tokens = (int64_t)it->second.tokens.size();
  if (num_computed) *num_computed = it->second.computed;
  if (num_blocks) *num_blocks = (int32_t)it->second.table.size();
  return cb::ok();
}

extern "C" int cb_bm_block_table(const cb_block_manager* m, int64_t seq_id, int32_t* out,
                                 int32_t capacity) {
  if (!m) return cb::fail(E, "manager is NULL");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return cb::fail(E, "unknown sequence id");
  const auto& t = it->second.table;
  if (!out || capacity < (int64_t)t.size()) return cb::fail(E, "out holds fewer entries than the table");
  std::memcpy(out, t.data(), sizeof(int32_t) * t.size());
  return cb::ok();
}

extern "C" int cb_bm_stats(const cb_block_manager* m, int64_t* free_blocks, int64_t* cached_blocks,
                           int64_t* held_blocks, int64_t* num_sequences) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (free_blocks) *free_blocks = (int64_t)m->fresh.size();
  if (cached_blocks) *cached_blocks = (int64_t)m->lru.size();
  if (held_blocks) *held_blocks = m->held;
  if (num_sequences) *num_sequences = (int64_t)m->seqs.size();
  return cb::ok();
}

extern "C" int cb_bm_ref_counts(const cb_block_manager* m, int32_t* out, int64_t capacity) {
  if (!m) return cb::fail(E, "manager is NULL");
  if (!out || capacity < m->num_blocks) return cb::fail(E, "out must hold num_blocks entries");
  std::memcpy(out, m->ref.data(), sizeof(int32_t) * m->num_blocks);
  return cb::ok();
}
