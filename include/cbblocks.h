/*
 * cbblocks — the host block manager of the paged KV cache, and the GPU block copy that carries
 * out its copy-on-write decisions.
 *
 * Sources: "3.3 Batching & Memory Management", sections "PagedAttention: block tables" (a pool
 * of fixed-size physical blocks; a per-sequence table maps logical block j to the block holding
 * positions [j*bs, (j+1)*bs); a new block only when the last is full), "Sharing and
 * copy-on-write" (per-block reference counts; fork shares every block; a write into a block
 * whose count exceeds 1 first copies it) and "Prefix caching and RadixAttention" (hash-based
 * variant: a full block is identified by its tokens and the hash of all blocks before it; a new
 * request reuses its leading cached blocks; free cached blocks are evicted LRU); "Continuous
 * batching architecture", sections "Prefix caching" and "Eviction" (freed blocks keep their
 * content and key until the allocator needs them).
 *
 * The manager is HOST code: every pointer passed to a cb_bm_* function is a host pointer, and
 * none of them touches a GPU. It is not thread-safe: one caller at a time per manager.
 *
 * Policies (deterministic, so that two runs of the same calls give the same block ids):
 *  - Never-used blocks are handed out lowest id first. When none is left, the least recently
 *    freed cached block is evicted (its key is dropped) and reused.
 *  - A sequence's blocks are freed last block first, so its prefix stays cached longest.
 *  - cb_bm_add_sequence reuses the leading full blocks of the prompt whose prefix is cached, but
 *    never the block holding the prompt's last token (that token's KV is always computed).
 *  - A full block is keyed when a built batch completes its KV (several blocks may hold one
 *    prefix; a lookup takes the lowest id); it is found by lookups only after the step closes.
 *
 * The step protocol. One forward step of the engine is:
 *   1. cb_bm_free_sequence / cb_bm_add_sequence / cb_bm_fork / cb_bm_append_tokens, in any order;
 *   2. cb_bm_build_batch (the batch's metadata for the kernels);
 *   3. cb_bm_take_copies, which returns the pending copy-on-write copies and CLOSES the step;
 *   4. on one stream, in this order: cb_copy_blocks (those copies), cb_cache_write (the batch's
 *      new K/V at its slot mapping), cb_paged_attention.
 * Rules the manager enforces so that the data the copies and lookups read exists:
 *  - a copy-on-write whose source block is written by a batch built in the open step is refused
 *    (its KV would be written after the copy runs): close the step first;
 *  - every block a transfer of the open step reads or writes (a copy's source or destination,
 *    a swap gather's source, a swap scatter's destination) stays out of the free pools until the
 *    step closes, even if its sequence is freed, so no two transfers of one launch touch one
 *    block; no copy's destination is a source;
 *  - a sequence in a batch of the open step cannot be freed;
 *  - a fork needs a parent whose every token is computed or in a built batch;
 *  - swap (below): a sequence with blocks written in the open step cannot be swapped out; blocks
 *    released by a swap-out and slots released by a swap-in or a free are held until the step
 *    closes; swapped-in blocks count as written in the open step; a swapped sequence cannot be
 *    appended to, forked or batched.
 *
 * The swap tier ("Continuous batching architecture", section "Offloading": an offloaded
 * request's KV blocks are copied to a pre-allocated pinned host pool, every request that fits
 * in one batched transfer, and copied back when device blocks free up, so the request resumes
 * without recomputing its tokens; one that does not fit is soft-reset by the caller). A step's
 * GPU work runs in this order: cb_copy_blocks, cb_swap_out_blocks (the step's swap-out pairs),
 * cb_swap_in_blocks (its swap-in pairs), cb_cache_write, cb_paged_attention.
 *
 * Return values: CB_OK, CB_ERR_INVALID_ARG (null pointer, unknown or duplicate id, a rule above
 * broken, an output array too small) or CB_ERR_OUT_OF_BLOCKS (the pool cannot supply the blocks;
 * the scheduler must preempt). A failing call changes nothing; cb_last_error() has the detail.
 */
#ifndef CBBLOCKS_H
#define CBBLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "cbattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cb_block_manager cb_block_manager;

/* A manager of num_blocks blocks of block_size tokens (num_blocks * block_size < 2^31), all
 * never-used. *out receives the handle (NULL on failure); the caller owns it and releases it with
 * cb_bm_destroy. */
int cb_bm_create(int64_t num_blocks, int32_t block_size, cb_block_manager** out);

/* Releases the manager and everything it holds. NULL is a no-op. */
void cb_bm_destroy(cb_block_manager* m);

/*
 * Admits a sequence with its prompt tokens[0 .. num_tokens) (host array, copied; num_tokens >= 1).
 * Reuses cached leading full blocks (prefix caching) and allocates the rest. *num_cached (may be
 * NULL) receives the number of leading positions whose KV is already in the cache: they are
 * computed, and the sequence's batches start at that position.
 */
int cb_bm_add_sequence(cb_block_manager* m, int64_t seq_id, const int32_t* tokens,
                       int32_t num_tokens, int32_t* num_cached);

/* Appends num_tokens >= 0 tokens (host array) to a sequence: a new block at each block boundary;
 * a copy-on-write of the last block if it is partial and shared. */
int cb_bm_append_tokens(cb_block_manager* m, int64_t seq_id, const int32_t* tokens,
                        int32_t num_tokens);

/* cb_bm_append_tokens for seq_ids[i] with counts[i] tokens taken in order from the packed host
 * array tokens (sum of counts entries), for i = 0, 1, ... until one fails: that failure's status is
 * returned, earlier appends stay done and *num_done receives how many succeeded (a decode step's
 * appends in one call; the scheduler preempts from the first refused sequence on). tokens NULL:
 * every appended token is a placeholder (cb_bm_append_placeholders). */
int cb_bm_append_batch(cb_block_manager* m, const int64_t* seq_ids, const int32_t* counts,
                       const int32_t* tokens, int32_t num_seqs, int32_t* num_done);

/*
 * Placeholder tokens for async steps ("Continuous batching in transformers", Async batching: a
 * step's inputs are built before the previous step's tokens exist). cb_bm_append_placeholders
 * appends num_tokens tokens whose values are not known yet (as cb_bm_append_tokens otherwise:
 * blocks, copy-on-write); cb_bm_confirm_tokens gives the values of the next num_tokens
 * unconfirmed tokens, in order. A full block is keyed for prefix reuse only once all its tokens
 * are confirmed (and its KV computed), so no request reuses KV computed from a token it does not
 * have. Tokens appended with values after an unconfirmed one stay unconfirmed until confirmed.
 */
int cb_bm_append_placeholders(cb_block_manager* m, int64_t seq_id, int32_t num_tokens);
int cb_bm_confirm_tokens(cb_block_manager* m, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens);
/* cb_bm_confirm_tokens for seq_ids[i] with counts[i] values taken in order from tokens, until one
 * fails (as cb_bm_append_batch). */
int cb_bm_confirm_batch(cb_block_manager* m, const int64_t* seq_ids, const int32_t* counts,
                        const int32_t* tokens, int32_t num_seqs, int32_t* num_done);

/* New sequence `child` sharing every block of `parent` (parallel sampling, beam search); the
 * parent's tokens must all be confirmed. */
int cb_bm_fork(cb_block_manager* m, int64_t parent, int64_t child);

/* Ends a sequence: drops its references; a block nobody references returns to a pool (cached if
 * keyed, never-used otherwise). */
int cb_bm_free_sequence(cb_block_manager* m, int64_t seq_id);

/*
 * The step's batch: sequence seq_ids[i] computes its next q_lens[i] positions
 * (1 <= q_lens[i] <= tokens not yet computed; no sequence twice). Outputs (host arrays the caller
 * allocates), in the layouts cb_paged_attention reads (include/cbattn.h):
 *   cu_seqlens_q [num_seqs + 1], kv_lens [num_seqs] (positions computed after this step),
 *   block_tables [num_seqs, max_blocks_per_seq] (row i gets sequence i's table; entries past it
 *   are left as they are: cb_paged_attention never reads them),
 *   slot_mapping [T] and token_ids [T] (may be NULL) with T = sum q_lens <= token_capacity.
 * Those positions count as computed from here on.
 */
int cb_bm_build_batch(cb_block_manager* m, const int64_t* seq_ids, const int32_t* q_lens,
                      int32_t num_seqs, int32_t max_blocks_per_seq, int32_t token_capacity,
                      int32_t* cu_seqlens_q, int32_t* kv_lens, int32_t* block_tables,
                      int32_t* slot_mapping, int32_t* token_ids);

/*
 * Closes the step and returns its pending copy-on-write copies in call order: copy block src[i]
 * to block dst[i] (host arrays of `capacity` entries; one sequence makes at most one copy per
 * step, so capacity = live sequences suffices). *num_copies receives the count even when
 * capacity is too small (then CB_ERR_INVALID_ARG and the step stays open).
 */
int cb_bm_take_copies(cb_block_manager* m, int32_t* src, int32_t* dst, int32_t capacity,
                      int32_t* num_copies);

/* Sets the swap pool to num_slots host slots of one block each (K and V, every layer), all free.
 * Refused while any slot holds data. */
int cb_bm_set_swap_slots(cb_block_manager* m, int64_t num_slots);

/* Swaps a sequence out: every block of its table, in order, goes to a free slot (lowest id
 * first): blocks[i] -> slots[i] (host arrays of `capacity` entries), *num_pairs of them; its
 * blocks are released. CB_ERR_OUT_OF_BLOCKS when the pool lacks free slots. */
int cb_bm_swap_out(cb_block_manager* m, int64_t seq_id, int32_t* blocks, int32_t* slots,
                   int32_t capacity, int32_t* num_pairs);

/* Swaps a sequence back in: new blocks for its slots, slots[i] -> blocks[i] (host arrays of
 * `capacity` entries) in table order; its computed positions stay computed. CB_ERR_OUT_OF_BLOCKS
 * when the device pool cannot supply the blocks. */
int cb_bm_swap_in(cb_block_manager* m, int64_t seq_id, int32_t* slots, int32_t* blocks,
                  int32_t capacity, int32_t* num_pairs);

/* Swap pool occupancy: free, used and held slots (each output may be NULL). */
int cb_bm_swap_stats(const cb_block_manager* m, int64_t* free_slots, int64_t* used_slots,
                     int64_t* held_slots);

/* Tokens, computed positions and table length of a sequence (each output may be NULL; a swapped
 * sequence has table length 0). */
int cb_bm_sequence_info(const cb_block_manager* m, int64_t seq_id, int64_t* num_tokens,
                        int64_t* num_computed, int32_t* num_blocks);

/* A sequence's block table into out[0 .. table length) (host, capacity entries). */
int cb_bm_block_table(const cb_block_manager* m, int64_t seq_id, int32_t* out, int32_t capacity);

/* Pool occupancy: never-used free blocks, cached (free, keyed) blocks, blocks held for a pending
 * copy, live sequences (each output may be NULL). */
int cb_bm_stats(const cb_block_manager* m, int64_t* free_blocks, int64_t* cached_blocks,
                int64_t* held_blocks, int64_t* num_sequences);

/* Reference count of every block into out[0 .. num_blocks) (host, capacity entries). */
int cb_bm_ref_counts(const cb_block_manager* m, int32_t* out, int64_t capacity);

/*
 * cb_copy_blocks — GPU copy of whole blocks, K and V, in every layer ("Sharing and copy-on-write":
 * the copy of a shared block before a write into it).
 * k_cache, v_cache: device, layer l of each at byte offset l * layer_stride_bytes, each layer
 * [num_blocks, block_bytes] (for cb_paged_attention's layout, block_bytes =
 * block_size * Hkv * D * 2); 16-byte aligned; block_bytes a multiple of 16; layer_stride_bytes
 * (read only when num_layers > 1) a multiple of 16, >= num_blocks * block_bytes.
 * src_blocks, dst_blocks: device int32 [num_copies]. For every i and layer: block dst[i] of K and
 * of V becomes a bit copy of block src[i]. Pairs with an id outside [0, num_blocks) or with
 * src == dst are skipped. The pairs must not overlap (no dst repeated, no dst that is another
 * pair's src): cb_bm_take_copies never returns such pairs. Enqueued on `stream`; no allocation,
 * no synchronization.
 */
int cb_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                   const int32_t* dst_blocks, int32_t num_copies, int64_t block_bytes,
                   int64_t num_blocks, int32_t num_layers, int64_t layer_stride_bytes,
                   void* stream);

/*
 * cb_swap_out_blocks / cb_swap_in_blocks — the swap tier's transfers ("Continuous batching
 * architecture", Offloading: a batched copy of offloaded requests' blocks to a pinned host pool,
 * and back). host_pool: pinned host memory the GPU can address (hipHostMalloc; checked: anything
 * else returns CB_ERR_INVALID_ARG), 16-byte aligned, laid out [num_slots][2 (K, V)][num_layers]
 * [block_bytes]. Caches and layers as in cb_copy_blocks. blocks, slots: device int32
 * [num_pairs]. Swap-out: for every pair and layer, slot slots[i] receives a bit copy of block
 * blocks[i] of K and of V; swap-in: block blocks[i] receives slot slots[i]. Pairs with an id
 * out of range are skipped; no slot (swap-out) or block (swap-in) may appear twice. The data
 * crosses PCIe inside the kernel (device stores to, or loads from, host memory). Enqueued on
 * `stream`; no allocation, no synchronization.
 */
int cb_swap_out_blocks(const void* k_cache, const void* v_cache, const int32_t* blocks,
                       const int32_t* slots, int32_t num_pairs, void* host_pool, int64_t num_slots,
                       int64_t block_bytes, int64_t num_blocks, int32_t num_layers,
                       int64_t layer_stride_bytes, void* stream);
int cb_swap_in_blocks(const void* host_pool, const int32_t* slots, const int32_t* blocks,
                      int32_t num_pairs, void* k_cache, void* v_cache, int64_t num_slots,
                      int64_t block_bytes, int64_t num_blocks, int32_t num_layers,
                      int64_t layer_stride_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CBBLOCKS_H */
