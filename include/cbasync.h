/*
 * cbasync — async steps: the CPU prepares step N + 1 while the GPU computes step N.
 *
 * Source: "Continuous batching in transformers", section "Async batching": three streams (upload,
 * compute, download) and three events; two sets of input/output buffers used alternately, since
 * the CPU must not write step N + 1's inputs while the GPU still reads step N's; one recorded
 * graph per buffer set (a graph records fixed addresses); and the carry-over: step N + 1's inputs
 * are built before step N has produced its tokens, so those tokens enter as placeholders 0 and a
 * carry-over mask (for each output of step N, the index of its destination among step N + 1's
 * inputs, or -1) adds them in before the forward pass.
 *
 * A step, with slot = (steps ended so far) % 2:
 *   1. cb_async_slot: waits until the slot's host input buffers are free (their previous upload
 *      has run); the caller then writes in_ids_host[slot][0, T) (placeholders 0 where a token of
 *      the previous step goes) and carry_dest_host[slot][0, num_carried) (for each output of the
 *      previous step: its destination index in this step's inputs, or -1);
 *   2. cb_async_begin: uploads the step's metadata (through the slot's step executor), input ids
 *      and carry mask on the upload stream, once the slot's previous compute is done; on the
 *      compute stream, after the upload, runs the carry-over from the previous slot's out_ids;
 *      returns the compute stream;
 *   3. the caller enqueues its forward pass up to attention on the compute stream (writing q, k,
 *      v rows [0, T) from in_ids[slot]);
 *   4. cb_async_attention: the step's slot mapping, cache write and paged attention on the
 *      compute stream (direct launches or graphs, per the step configuration);
 *   5. the caller enqueues the rest of its forward pass and its sampler, writing out_ids[slot];
 *   6. cb_async_end: records compute over, and copies out_ids[slot][0, num_outputs) to
 *      out_ids_host[slot] on the download stream;
 *   7. cb_async_wait(slot) blocks until that copy has run. The caller reads step N's outputs
 *      after beginning step N + 1, so its CPU work overlaps the GPU's; it must have read a
 *      slot's outputs before ending the next step that uses that slot.
 * Buffers (caller-owned, fixed at creation): the step configuration's (cbgraphs.h); device int32
 * in_ids, out_ids, carry_dest [2][max_tokens]; pinned host int32 in_ids_host, carry_dest_host,
 * out_ids_host [2][max_tokens] (checked: pageable memory is refused). Streams are created at
 * default priority and kept until cb_async_destroy.
 */
#ifndef CBASYNC_H
#define CBASYNC_H

#include <stdint.h>

#include "cbgraphs.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * cb_carry_over — for every i < num_prev with 0 <= dest[i] < num_next:
 *     next_inputs[dest[i]] += prev_outputs[i]
 * (device int32 arrays; destinations must be distinct). Source: the carry-over of "Async
 * batching" above: placeholders are 0, so the add enters the token.
 */
int cb_carry_over(const int32_t* prev_outputs, const int32_t* dest, int32_t num_prev,
                  int32_t* next_inputs, int32_t num_next, void* stream);

typedef struct cb_async_steps cb_async_steps;

typedef struct {
  cb_step_graphs_config step; /* shared by both slots' step executors */
  int32_t* in_ids[2];
  int32_t* out_ids[2];
  int32_t* carry_dest[2];
  int32_t* in_ids_host[2];
  int32_t* carry_dest_host[2];
  int32_t* out_ids_host[2];
} cb_async_config;

int cb_async_create(const cb_async_config* cfg, cb_async_steps** out);
/* Waits for the streams, then frees streams, events and the two step executors. */
void cb_async_destroy(cb_async_steps* a);
int cb_async_slot(cb_async_steps* a, int32_t* slot);
int cb_async_begin(cb_async_steps* a, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                   const int32_t* block_tables, int32_t num_seqs, int32_t num_carried,
                   void** compute_stream);
int cb_async_attention(cb_async_steps* a);
int cb_async_end(cb_async_steps* a, int32_t num_outputs);
int cb_async_wait(cb_async_steps* a, int32_t slot);

#ifdef __cplusplus
}
#endif

#endif /* CBASYNC_H */
