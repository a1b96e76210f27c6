/*
 * cbgraphs — one step of the hot path (slot mapping, cache write, paged attention: one
 * cb_paged_attention_write) recorded as a HIP graph per padded batch shape and replayed, or
 * launched directly.
 *
 * Source: "Continuous batching architecture", section "CUDA graphs": a step's GPU work is
 * recorded once and replayed for batches of the same shape, which removes the CPU cost of
 * launching each kernel; because the shape changes every step, query lengths are padded to a
 * multiple of one interval and KV lengths to a multiple of another, and recorded graphs are kept
 * in a cache. Padding tokens ("Continuous batching in transformers", The paged cache section,
 * reserves blocks for them to read and write) here belong to a padding sequence with KV length 0,
 * which the kernels give no work and whose slots are -1: padding reads and writes nothing.
 *
 * The padded shape of a step with S sequences, T tokens, longest q max_q and longest KV max_kv:
 *   tokens  Tb = min(round_up(T, token_interval), max_tokens)
 *   seqs    Sb = min(round_up(S + (Tb > T), seq_interval), max_seqs)    (one padding sequence
 *                takes the Tb - T padding tokens; the others have none)
 *   max q   min(next power of two >= max_q, Tb)   (the kernels' decode threshold 16 / (Hq / Hkv)
 *           is a power of two, so a decode-only batch stays one)
 *   max kv  min(round_up(max_kv, kv_interval), max_kv_len)
 * With use_graphs, the first step of a padded shape runs eagerly; its next step records the
 * graph; later steps replay it. At most max_graphs graphs are kept (least recently used evicted).
 * Without, every step launches the step's kernels directly on the padded shape. Measured on
 * MI355X (ROCm 7.2, a 16-sequence decode step of the Llama-3-8B shape, from native code): direct
 * launches 46 us per step back to back and 59 us waited for, replays 53 and 65 us: replay adds
 * GPU time per step and the launches it saves are cheap. Either mode is one call per step.
 *
 * Buffers: the caller's q [max_tokens, Hq, D], k and v [max_tokens, Hkv, D], out
 * [max_tokens, Hq, D] and the caches [num_blocks, bs, Hkv, D] (bf16, device, 16-byte aligned)
 * are fixed at creation: a step's rows go in rows [0, T) of q, k, v before cb_graphs_run, and its
 * output is rows [0, T) of out once the stream reaches it. The executor allocates (at creation
 * and, for the attention workspace, when a shape first needs more) device memory for the
 * metadata and the workspace, and pinned host memory for staging the metadata; it frees them in
 * cb_graphs_destroy.
 *
 * Streams: every cb_graphs_run of one executor must be on the same stream (a real stream, not
 * NULL: the NULL stream cannot be recorded), and the caller must not change q, k, v before the
 * stream has run the step that reads them. Not thread-safe: one caller at a time per executor.
 *
 * Return values as in cbattn.h; a failing run enqueues nothing that reads the failing step's
 * metadata (it may already have uploaded it).
 */
#ifndef CBGRAPHS_H
#define CBGRAPHS_H

#include <stddef.h>
#include <stdint.h>

#include "cbattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cb_step_graphs cb_step_graphs;

typedef struct {
  int32_t num_q_heads, num_kv_heads, head_dim, block_size; /* as in cb_paged_attention */
  int64_t num_blocks;
  int32_t max_blocks_per_seq;   /* block-table row length of every step */
  int32_t max_tokens;           /* rows of q, k, v, out: the largest padded step */
  int32_t max_seqs;             /* the most sequences of a padded step, the padding one included (>= 2) */
  int32_t max_kv_len;           /* the longest KV length of any step (<= max_blocks_per_seq * block_size) */
  int32_t token_interval;       /* padding interval of the token count */
  int32_t kv_interval;          /* padding interval of max kv */
  int32_t seq_interval;         /* padding interval of the sequence count */
  int32_t max_graphs;           /* recorded graphs kept */
  int32_t use_graphs;           /* 1: record and replay HIP graphs; 0: launch the kernels directly */
  float scale;                  /* softmax scale */
  void* q;
  void* k;
  void* v;
  void* out;
  void* k_cache;
  void* v_cache;
} cb_step_graphs_config;

/* An executor for the configuration (checked; device and pinned allocations). */
int cb_graphs_create(const cb_step_graphs_config* cfg, cb_step_graphs** out);

/* Waits for the executor's outstanding work, then frees it. NULL is a no-op. */
void cb_graphs_destroy(cb_step_graphs* g);

/*
 * One step: host metadata of S = num_seqs sequences (cu_seqlens_q [S + 1], kv_lens [S],
 * block_tables [S, max_blocks_per_seq], with cb_paged_attention's meaning and preconditions;
 * T = cu_seqlens_q[S] <= max_tokens; every kv_lens <= max_kv_len). Pads them to the step's
 * padded shape, uploads them with one copy on `stream` and runs the step there (eagerly, by
 * recording, or by replay). padded_shape (may be NULL) receives {Sb, Tb, max q, max kv}.
 */
int cb_graphs_run(cb_step_graphs* g, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                  const int32_t* block_tables, int32_t num_seqs, void* stream,
                  int32_t* padded_shape);

/* Counters: graphs recorded, replays, eager first runs, graphs cached (outputs may be NULL). */
int cb_graphs_stats(const cb_step_graphs* g, int64_t* captures, int64_t* replays,
                    int64_t* eager_runs, int32_t* cached);

#ifdef __cplusplus
}
#endif

#endif /* CBGRAPHS_H */
