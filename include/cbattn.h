/*
 * cbattn — ragged paged attention and the paged KV-cache write for one forward pass of a
 * continuous-batching engine, on AMD Instinct MI355X (gfx950).
 *
 * The step's tokens of all sequences are packed with no batch axis: sequence s owns packed rows
 * [cu_seqlens_q[s], cu_seqlens_q[s+1]) ("Continuous batching from first principles", Summary
 * and Takeaways: ragged batching concatenates the sequences and keeps them apart with a
 * block-diagonal mask). Each sequence's K/V lives in fixed-size physical blocks reached through
 * its block table: entry j holds its token positions [j*block_size, (j+1)*block_size)
 * ("3.3 Batching & Memory Management", section "PagedAttention: block tables").
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says host. bf16 tensors are passed as
 *    void* and hold IEEE bfloat16 values. Every tensor is dense row-major.
 *  - Shapes (T = num_tokens, S = num_seqs, Hq, Hkv, D = head_dim, bs = block_size,
 *    NB = num_blocks, MB = max_blocks_per_seq):
 *        q_packed      [T, Hq, D]        bf16
 *        k, v (new)    [T, Hkv, D]       bf16
 *        k_cache/v_cache [NB, bs, Hkv, D] bf16   (slot = block * bs + offset)
 *        cu_seqlens_q  [S + 1]           int32
 *        kv_lens       [S]               int32   KV tokens of each sequence AFTER this step's
 *                                                write, including its new tokens
 *        block_tables  [S, MB]           int32
 *        slot_mapping  [T]               int32   slot of each new token, or -1 = do not write
 *        out           [T, Hq, D]        bf16
 *  - The caller owns every buffer. The library allocates no device memory (its one device
 *    array, the scratch of cb_paged_attention_write_noalloc, is placed by the HIP runtime when
 *    the library's code is loaded on a device), does not synchronize, and keeps no pointer to
 *    caller buffers after it returns. Work is enqueued on
 *    `stream` (a hipStream_t; NULL means the default stream) in call order. For a batch with
 *    both decode and prefill rows, cb_paged_attention runs its decode kernel on an internal
 *    second stream (created on first use per device and caller stream, default priority, kept
 *    until the process ends; at most 64 caller streams per device get one, calls on further
 *    streams run that kernel after the prefill kernel on `stream`, with the same results) that
 *    it forks from and joins back into `stream` with events, so the call still completes in
 *    `stream` order.
 *  - Return value: CB_OK (0) or a negative cb_status. Only host-checkable facts are checked
 *    (null pointers, shape limits, alignment, workspace size); on error nothing is enqueued
 *    and cb_last_error() describes the failure. Data-dependent preconditions (below, and
 *    cb_validate_batch) are the caller's contract and are NOT checked on the GPU path.
 *  - Data-dependent preconditions: cu_seqlens_q[0] = 0, non-decreasing, cu_seqlens_q[S] = T;
 *    1 <= q_s <= kv_lens[s] for every sequence (q_s = cu[s+1] - cu[s]);
 *    kv_lens[s] <= MB * bs; table entries for logical blocks < ceil(kv_lens[s] / bs) lie in
 *    [0, NB) (entries past that are never read and may hold -1); slots are -1 or in
 *    [0, NB * bs) with no slot repeated; kv_lens and q lengths do not exceed max_kv_len and
 *    max_q_len. In cb_paged_attention, a sequence whose q or kv length breaks these bounds
 *    (q = 0, kv_len < q, kv_len > max_kv_len or > MB * bs, a decode-type q > max_q_len) gets no
 *    work: nothing is read for it and its output rows are left unwritten.
 */
#ifndef CBATTN_H
#define CBATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CB_OK = 0,
  CB_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad shape relation, misalignment */
  CB_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, block_size or head ratio */
  CB_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required */
  CB_ERR_HIP = -4,         /* a HIP launch failed; see cb_last_error() */
  CB_ERR_OUT_OF_BLOCKS = -5 /* the block manager's pool cannot supply the blocks (cbblocks.h) */
} cb_status;

/* Static text naming a status code. Never NULL. */
const char* cb_status_string(int status);

/* Detail of the last failing call made by this thread ("" if none). Valid until this thread's
 * next call into the library. */
const char* cb_last_error(void);

/*
 * cb_slot_mapping — cache slot of every new token.
 * Source: "3.3 Batching & Memory Management", section "PagedAttention: block tables" (position p
 * of a sequence lives in block table[p / bs] at offset p % bs; the worked example with block
 * size 4). The i-th new token of sequence s is at position p = kv_lens[s] - q_s + i, so
 *     slot_mapping[cu[s] + i] = block_tables[s][p / bs] * bs + p % bs.
 * Output: slot_mapping [T] int32 (device, caller-allocated). Requires block_size >= 4
 * (CB_ERR_INVALID_ARG below that, as "Continuous batching in transformers" rejects blocks
 * smaller than 4 in its paged-cache section) and NB * bs < 2^31 is the caller's contract.
 */
int cb_slot_mapping(const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                    const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t* slot_mapping,
                    void* stream);

/*
 * cb_cache_write — write the step's new K/V rows into the paged cache.
 * Source: "Continuous batching in transformers", section "The paged cache, its two reserved
 * blocks, and the block-size trade" (a page is one token's K or V in one layer; the cache
 * tensor is the physical store), and "Continuous batching architecture", section "Memory
 * management" (each request holds block ids the attention kernel reads from and writes to).
 * For every token t with 0 <= slot = slot_mapping[t] < num_blocks * block_size:
 *     k_cache[slot] = k[t]; v_cache[slot] = v[t]   (all Hkv heads, bit copy)
 * Tokens with slot -1 are skipped, and so are slots past the pool (nothing is written outside it). k, v, k_cache, v_cache must be 16-byte aligned and
 * Hkv * D must be a multiple of 8. Slots must be distinct (two tokens writing one slot race).
 */
int cb_cache_write(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                   void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, void* stream);

/*
 * Bytes of device workspace cb_paged_attention needs for these host-side bounds (same meaning
 * as its arguments). Returns 0 only when nothing would be launched.
 */
size_t cb_paged_attention_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_q_len, int32_t max_kv_len,
                                         int32_t kv_split_tokens);

/*
 * KV partition size (tokens) cb_paged_attention uses for decode-type sequences with these
 * bounds (the same arguments as cb_paged_attention_workspace_size); kv_split_tokens > 0 requests
 * a size (rounded up to a multiple of 32, at most 2048). Automatic: about
 * max_kv_len * num_seqs * num_kv_heads / 5461 in steps of 256, within [256, 2048]; when that
 * gives 256 and no prefill-type sequence is possible (max_q_len * num_q_heads / num_kv_heads <=
 * 16): with K = max_kv_len * num_seqs * num_kv_heads, the larger of K / 640 and max_kv_len / 24,
 * at most the larger of 768 and max_kv_len / 8, rounded up to a multiple of 64 within
 * [128, 2048]; and max_kv_len rounded up to a multiple of 32 (one partition per sequence) when
 * twice that size reaches max_kv_len.
 */
int32_t cb_paged_attention_split_tokens(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t max_q_len,
                                        int32_t max_kv_len, int32_t kv_split_tokens);

/*
 * cb_paged_attention — attention of the packed batch over the paged cache.
 * Sources: ragged batching with a block-diagonal mask ("Continuous batching from first
 * principles", Takeaways); chunked prefill, where a chunk's queries attend to a cache that
 * already holds the earlier chunks ("3.3 Batching & Memory Management", section "Chunked
 * prefill"); block-table gather ("PagedAttention: block tables"). The pages give no formula;
 * this computes scaled dot-product softmax attention: for token t = cu[s] + i of sequence s,
 * query head h, KV head g = h / (Hq / Hkv), position p = kv_lens[s] - q_s + i,
 *     out[t][h] = sum_{j <= p} softmax_j(scale * <q[t][h], K_s,g[j]>) V_s,g[j]
 * with K_s,g[j] the key of position j of sequence s read through its block table. The cache must
 * already hold this step's K/V (call cb_cache_write first). bf16 inputs, fp32 accumulation and
 * softmax, bf16 output (round to nearest even).
 *
 * Host scalars: max_q_len >= every q_s and max_kv_len >= every kv_lens[s] (upper bounds: they
 * size grids and the workspace); kv_split_tokens = 0 lets the library choose the KV partition
 * of decode-type sequences (q_s * Hq/Hkv <= 16), > 0 requests one (see
 * cb_paged_attention_split_tokens). Sequences with more than one partition are merged by the
 * log-sum-exp reduction of cb_split_kv_reduce inside this call.
 * Supported: head_dim 64 or 128; Hq / Hkv in {1, 2, 4, 8, 16}; block_size a multiple of 16
 * (4..15 and other values: CB_ERR_UNSUPPORTED; below 4: CB_ERR_INVALID_ARG); scale finite, > 0.
 * q_packed, caches and out must be 16-byte aligned. workspace: device memory of at least
 * cb_paged_attention_workspace_size(...) bytes, 256-byte aligned, used in stream order; its
 * contents on entry do not matter. out is fully overwritten.
 */
int cb_paged_attention(const void* q_packed, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                       const int32_t* block_tables, const void* k_cache, const void* v_cache,
                       void* out, float scale, int32_t num_seqs, int32_t num_tokens,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                       int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * cb_paged_attention_write — cb_slot_mapping + cb_cache_write + cb_paged_attention in one call:
 * the step's new K/V rows k_new, v_new [T, Hkv, D] (bf16, 16-byte aligned) are written at the
 * slots the slot mapping would give ("3.3 Batching & Memory Management", PagedAttention: block
 * tables), then attention runs as in cb_paged_attention. The write's slots are computed in place
 * (no slot array), and it runs in the first launch beside the planning workgroup, which reads
 * no cache, instead of in two launches before it. A decode-only batch of at most 64 sequences
 * with fewer (partition, KV head) items than decode waves has no planning launch: the decode
 * kernel plans itself, its spare waves write the step's rows and each item's wave writes the
 * new rows of its own partition before reading them. Results are those of the three calls, bit
 * for bit; rows whose position or slot the slot mapping would mark -1 (and slots past the pool)
 * are not written. Arguments, preconditions and errors as cb_paged_attention's, plus
 * num_blocks * block_size < 2^31 and: no sequence reads, at a position below its kv_len, a slot
 * that this call writes for another sequence (blocks shared between sequences are copied
 * before they are written, as copy-on-write does).
 */
int cb_paged_attention_write(const void* q_packed, const void* k_new, const void* v_new,
                             const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                             const int32_t* block_tables, void* k_cache, void* v_cache, void* out,
                             float scale, int32_t num_seqs, int32_t num_tokens,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * cb_paged_attention_write_noalloc — cb_paged_attention_write with no workspace argument and no
 * allocation, for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 * The scratch it needs (work lists, counters, split-KV partials) lives in a device array of
 * CB_NOALLOC_SCRATCH_BYTES that the library holds, one per device, from the first call on that
 * device until the process ends; the call allocates nothing (no hipMalloc, hipFree, stream or
 * event creation). The caller still passes inputs and outputs, as to cb_paged_attention_write.
 * Differences from cb_paged_attention_write:
 *  - A batch whose work needs more scratch than CB_NOALLOC_SCRATCH_BYTES returns
 *    CB_ERR_WORKSPACE (cb_last_error() gives both sizes) and enqueues nothing. Prefill tiles are
 *    split along the keys only while their partials fit a quarter of the scratch, so results of
 *    mixed batches may differ from cb_paged_attention_write's by rounding (both are within the
 *    same tolerance of the exact result); decode-only batches give the same bits.
 *  - Every kernel runs on `stream` (no internal second stream): with prefill rows the decode
 *    kernel follows the prefill kernel instead of running beside it.
 *  - All calls on one device share its scratch, and each call leaves its contents behind: calls
 *    that may overlap on one device (different streams, or host threads) race and must be
 *    ordered by the caller. The kernels clear what must start at zero themselves (no memset).
 * Arguments, preconditions and other errors as cb_paged_attention_write's.
 */
#define CB_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int cb_paged_attention_write_noalloc(const void* q_packed, const void* k_new, const void* v_new,
                                     const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                     const int32_t* block_tables, void* k_cache, void* v_cache,
                                     void* out, float scale, int32_t num_seqs, int32_t num_tokens,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t max_blocks_per_seq,
                                     int64_t num_blocks, int32_t max_q_len, int32_t max_kv_len,
                                     int32_t kv_split_tokens, void* stream);

/*
 * cb_split_kv_reduce — merge per-partition attention results (log-sum-exp merge).
 * For each token t with n = num_splits[t] >= 1 and each head h:
 *     M = max_k lse[t][h][k];  w_k = exp(lse[t][h][k] - M)
 *     out[t][h] = sum_k w_k o_part[t][h][k] / sum_k w_k          (k < n)
 * where o_part[t][h][k] is the softmax-normalised attention of the query over partition k and
 * lse its natural-log sum-exp of scaled scores; lse = -inf marks an empty partition (weight 0).
 * Tokens with num_splits[t] <= 0 are not written. Layouts (fp32): o_part [T, Hq, max_splits, D],
 * lse_part [T, Hq, max_splits]; num_splits [T] int32; out [T, Hq, D] bf16, 16-byte aligned.
 * head_dim 64 or 128. The pages describe no partitioned attention; the merge is the exact
 * identity of softmax over a union of disjoint key ranges.
 */
int cb_split_kv_reduce(const float* o_part, const float* lse_part, const int32_t* num_splits,
                       void* out, int32_t num_tokens, int32_t num_q_heads, int32_t head_dim,
                       int32_t max_splits, void* stream);

/*
 * cb_validate_batch — HOST-ONLY check of the data-dependent preconditions listed at the top of
 * this file (host pointers; slot_mapping may be NULL). Not on the hot path: for tests and
 * debugging callers. Returns CB_OK or CB_ERR_INVALID_ARG with the first violation in
 * cb_last_error(). Beyond the listed rules it rejects a slot that lands in a block referenced
 * by more than one table row (a write into a shared block needs a copy first: "3.3 Batching &
 * Memory Management", section "Sharing and copy-on-write"), and block_size < 4 ("Continuous
 * batching in transformers", paged-cache section).
 */
int cb_validate_batch(const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                      const int32_t* block_tables, const int32_t* slot_mapping, int32_t num_seqs,
                      int32_t num_tokens, int32_t max_blocks_per_seq, int32_t block_size,
                      int64_t num_blocks, int32_t max_q_len, int32_t max_kv_len);

/*
 * cb_time_next_kernel — measurement hook: time one kernel of the next attention call.
 * Not an operation of the method: it serves throughput measurement against a kernel's roofline.
 * The next cb_paged_attention call made by this thread records `start_event` on its stream right
 * before it launches kernel `which` and `stop_event` right after (one-shot: that call clears the
 * request, whether it launches the kernel or not).
 *   which: CB_KERNEL_DECODE (the decode / split-KV kernel) or CB_KERNEL_PREFILL (the
 *          prefill-chunk kernel, launched only when the batch holds prefill rows); 0 clears a
 *          pending request.
 *   start_event, stop_event: hipEvent_t handles created by the caller (with timing enabled),
 *          owned by the caller; they must outlive the call they are recorded in.
 * Errors: CB_ERR_INVALID_ARG for an unknown `which` or a NULL event with which != 0. A failing
 * hipEventRecord inside the attention call makes that call return CB_ERR_HIP.
 */
enum { CB_KERNEL_DECODE = 1, CB_KERNEL_PREFILL = 2 };
int cb_time_next_kernel(int32_t which, void* start_event, void* stop_event);

/*
 * cb_stream_read — measurement aid: read `bytes` of device memory at `buf` once, with 16-byte
 * non-temporal loads, as fast as the GPU streams HBM. Not an operation of the method: its rate
 * is the measured streaming-read ceiling that the bandwidth-bound kernels are reported against
 * beside the 8 TB/s specification.
 *   buf: device memory, 16-byte aligned; bytes a multiple of 16 (0: nothing is launched).
 *   sink: device memory of sink_words >= 256 uint32 words, caller-owned; each thread of the
 *         launch (at most 1024 workgroups of 256, and at most sink_words threads, rounded down
 *         to 256) writes one word.
 * Errors: CB_ERR_INVALID_ARG for NULL pointers, misalignment or a sink under 256 words;
 * CB_ERR_HIP if the launch fails. Enqueued on `stream`; nothing else is read or written.
 */
int cb_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CBATTN_H */
