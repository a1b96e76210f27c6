// Step graphs: the hot path of one step (slot mapping, cache write, paged attention) as one
// native call per step on a padded batch shape, either recorded once per shape as a HIP graph
// and replayed (one metadata upload and one graph launch per step) or launched directly (one
// upload and the step's kernels); measured on MI355X, direct launches cost less GPU time per step
// than replaying the same kernels as a graph, so both are offered.
//
// "Continuous batching architecture", section "CUDA graphs": the step's GPU work is recorded
// once and replayed for batches of matching shape; since the shape changes every step, query
// lengths and KV lengths are padded to multiples of fixed intervals and the recorded graphs are
// kept in a cache; a padded shape with no graph is recorded anew. "Continuous batching in
// transformers", The paged cache section: padding tokens must read and write somewhere
// harmless. Here a padding token belongs to a padding sequence whose KV length is 0: the
// kernels give such a sequence no work and its slots are -1, so padding reads and writes
// nothing (no reserved trash blocks are needed).
//
// Graphs record fixed addresses: the executor owns the device metadata buffers (cu_seqlens_q,
// kv_lens, block tables, slots) and the attention workspace, and takes fixed caller buffers for
// q, k, v, out and the caches at creation. The workspace a shape needs is not monotone in the
// shape (fewer tokens allow more prefill splits, fewer sequences smaller KV partitions), so it
// grows on demand: a shape that needs more waits for the stream, replaces the workspace and drops
// the recorded graphs (they name the old address); they are recorded again on their next use.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <list>
#include <map>
#include <new>
#include <tuple>

#include "cb_internal.h"
#include "cbgraphs.h"

namespace {

using Key = std::tuple<int32_t, int32_t, int32_t, int32_t>;  // seqs, tokens, max q, max kv

struct Entry {
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;  // recorded after the latest launch (eviction waits for it)
  std::list<Key>::iterator lru;
};

constexpr int kStagingSlots = 2;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

struct cb_step_graphs {
  cb_step_graphs_config cfg{};
  // device metadata: cu [max_seqs + 1] | kv_lens [max_seqs] | tables [max_seqs * MB], then slots
  int32_t* meta = nullptr;
  int32_t* slots = nullptr;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  // pinned host staging of the metadata, double-buffered: a slot is reused only after the copy
  // that read it has run (its event)
  int32_t* staging[kStagingSlots] = {nullptr, nullptr};
  hipEvent_t staged[kStagingSlots] = {nullptr, nullptr};
  int next_slot = 0;
  std::map<Key, Entry> graphs;
  std::list<Key> lru;  // least recently used first
  std::map<Key, bool> seen;  // shapes run once eagerly (recorded on their next use)
  int64_t captures = 0, replays = 0, eager = 0;

  size_t meta_ints() const {
    return (size_t)cfg.max_seqs + 1 + cfg.max_seqs + (size_t)cfg.max_seqs * cfg.max_blocks_per_seq;
  }
};

namespace {

using G = cb_step_graphs;
constexpr int E = CB_ERR_INVALID_ARG;

void drop_graphs(G* g) {
  for (auto& kv : g->graphs) {
    if (kv.second.done) {
      (void)hipEventSynchronize(kv.second.done);
      (void)hipEventDestroy(kv.second.done);
    }
    if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
  }
  g->graphs.clear();
  g->lru.clear();
}

void release(G* g) {
  drop_graphs(g);
  for (int i = 0; i < kStagingSlots; ++i) {
    if (g->staged[i]) {
      (void)hipEventSynchronize(g->staged[i]);
      (void)hipEventDestroy(g->staged[i]);
    }
    if (g->staging[i]) (void)hipHostFree(g->staging[i]);
  }
  if (g->meta) (void)hipFree(g->meta);
  if (g->workspace) (void)hipFree(g->workspace);
}

// The step on `st` with the device metadata of a padded shape: slot mapping, cache write and
// paged attention in one call (the write runs beside the planning workgroup).
int enqueue_step(G* g, const Key& k, hipStream_t st) {
  const auto& c = g->cfg;
  const int32_t S = std::get<0>(k), T = std::get<1>(k), mq = std::get<2>(k), mkv = std::get<3>(k);
  const int32_t* cu = g->meta;
  const int32_t* kv = cu + c.max_seqs + 1;
  const int32_t* tables = kv + c.max_seqs;
  return cb_paged_attention_write(c.q, c.k, c.v, cu, kv, tables, c.k_cache, c.v_cache, c.out,
                                  c.scale, S, T, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                  c.block_size, c.max_blocks_per_seq, c.num_blocks, mq, mkv, 0,
                                  g->workspace, g->workspace_bytes, st);
}

// A workspace of at least `need` bytes; a replacement drops every recorded graph.
int ensure_workspace(G* g, size_t need, hipStream_t st) {
  if (need <= g->workspace_bytes && g->workspace) return CB_OK;
  if (g->workspace) {
    if (hipStreamSynchronize(st) != hipSuccess) return cb::fail(CB_ERR_HIP, "stream wait failed");
    drop_graphs(g);
    (void)hipFree(g->workspace);
    g->workspace = nullptr;
    g->workspace_bytes = 0;
  }
  const size_t bytes = (std::max<size_t>(need, 256) * 5 / 4 + (1u << 20) - 1) & ~size_t((1u << 20) - 1);
  if (hipMalloc(&g->workspace, bytes) != hipSuccess) {
    g->workspace = nullptr;
    return cb::fail(CB_ERR_HIP, "workspace allocation failed");
  }
  g->workspace_bytes = bytes;
  return CB_OK;
}

int capture(G* g, const Key& k, hipStream_t st, hipGraphExec_t* out) {
  if (hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed) != hipSuccess)
    return cb::fail(CB_ERR_HIP, "hipStreamBeginCapture failed (a NULL stream cannot be captured)");
  const int r = enqueue_step(g, k, st);
  hipGraph_t graph = nullptr;
  const hipError_t e = hipStreamEndCapture(st, &graph);
  if (r != CB_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return r;
  }
  if (e != hipSuccess || !graph) return cb::fail(CB_ERR_HIP, "hipStreamEndCapture failed");
  const hipError_t ie = hipGraphInstantiate(out, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ie != hipSuccess) return cb::fail(CB_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(ie));
  return CB_OK;
}

}  // namespace

extern "C" int cb_graphs_create(const cb_step_graphs_config* cfg, cb_step_graphs** out) {
  if (!out) return cb::fail(E, "out is NULL");
  *out = nullptr;
  if (!cfg) return cb::fail(E, "cfg is NULL");
  const auto& c = *cfg;
  if (c.num_q_heads < 1 || c.num_kv_heads < 1 || c.head_dim < 1 || c.block_size < 4 ||
      c.num_blocks < 1 || c.max_blocks_per_seq < 1 || c.max_tokens < 1 || c.max_seqs < 2 ||
      c.max_kv_len < 1 || c.token_interval < 1 || c.kv_interval < 1 || c.seq_interval < 1 ||
      c.max_graphs < 1)
    return cb::fail(E, "cb_graphs_create: a size is out of range (max_seqs >= 2: one is for padding)");
  if ((int64_t)c.max_kv_len > (int64_t)c.max_blocks_per_seq * c.block_size)
    return cb::fail(E, "cb_graphs_create: max_kv_len exceeds max_blocks_per_seq * block_size");
  if (!c.q || !c.k || !c.v || !c.out || !c.k_cache || !c.v_cache)
    return cb::fail(E, "cb_graphs_create: NULL buffer");
  if (!std::isfinite(c.scale) || !(c.scale > 0.f)) return cb::fail(E, "scale must be finite and positive");
  G* g = new (std::nothrow) G;
  if (!g) return cb::fail(E, "out of host memory");
  g->cfg = c;
  const size_t mi = g->meta_ints();
  if (hipMalloc(&g->meta, sizeof(int32_t) * (mi + (size_t)c.max_tokens)) != hipSuccess) {
    release(g);
    delete g;
    return cb::fail(CB_ERR_HIP, "cb_graphs_create: device allocation failed");
  }
  g->slots = g->meta + mi;
  for (int i = 0; i < kStagingSlots; ++i) {
    if (hipHostMalloc(reinterpret_cast<void**>(&g->staging[i]), sizeof(int32_t) * mi, hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&g->staged[i], hipEventDisableTiming) != hipSuccess) {
      release(g);
      delete g;
      return cb::fail(CB_ERR_HIP, "cb_graphs_create: pinned staging allocation failed");
    }
  }
  *out = g;
  return cb::ok();
}

extern "C" void cb_graphs_destroy(cb_step_graphs* g) {
  if (!g) return;
  release(g);
  delete g;
}

namespace {

// Checks and pads a step's host metadata and uploads it on `upload` (the executor's metadata
// buffers); *key receives the padded shape.
int prepare(G* g, const int32_t* cu_seqlens_q, const int32_t* kv_lens, const int32_t* block_tables,
            int32_t num_seqs, hipStream_t upload, Key* key) {
  const auto& c = g->cfg;
  const int32_t T = cu_seqlens_q[num_seqs];
  if (cu_seqlens_q[0] != 0 || T < 1 || T > c.max_tokens)
    return cb::fail(E, "cu_seqlens_q must start at 0 and end in [1, max_tokens]");
  int32_t max_q = 1, max_kv = 1;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    if (q < 0) return cb::fail(E, "cu_seqlens_q decreases");
    max_q = std::max(max_q, q);
    max_kv = std::max(max_kv, kv_lens[s]);
  }
  if (max_kv > c.max_kv_len) return cb::fail(E, "a kv length exceeds the executor's max_kv_len");
  // the padded shape
  const int32_t Tb = (int32_t)std::min<int64_t>(round_up(T, c.token_interval), c.max_tokens);
  const int32_t seqs = num_seqs + (Tb > T ? 1 : 0);
  if (seqs > c.max_seqs) return cb::fail(E, "more sequences (with the padding one) than max_seqs");
  const int32_t Sb = (int32_t)std::min<int64_t>(round_up(seqs, c.seq_interval), c.max_seqs);
  // max q to a power of two: the kernels' decode threshold (16 / (Hq / Hkv)) is one, so padding
  // never turns a decode-only batch into one with prefill work
  int32_t mq2 = 1;
  while (mq2 < max_q) mq2 *= 2;
  const int32_t mqb = std::min(mq2, Tb);
  const int32_t mkvb = (int32_t)std::min<int64_t>(round_up(max_kv, c.kv_interval), c.max_kv_len);
  *key = Key{Sb, Tb, mqb, mkvb};

  // metadata of the padded batch into a staging slot whose previous copy has run
  const int slot = g->next_slot;
  g->next_slot = (slot + 1) % kStagingSlots;
  if (hipEventSynchronize(g->staged[slot]) != hipSuccess) return cb::fail(CB_ERR_HIP, "staging wait failed");
  int32_t* hcu = g->staging[slot];
  int32_t* hkv = hcu + c.max_seqs + 1;
  int32_t* htab = hkv + c.max_seqs;
  const int32_t MB = c.max_blocks_per_seq;
  std::memcpy(hcu, cu_seqlens_q, sizeof(int32_t) * (num_seqs + 1));
  std::memcpy(hkv, kv_lens, sizeof(int32_t) * num_seqs);
  std::memcpy(htab, block_tables, sizeof(int32_t) * (size_t)num_seqs * MB);
  // padding sequences: the first takes the padding tokens, all have KV length 0 (no work)
  for (int32_t s = num_seqs; s < Sb; ++s) {
    hcu[s + 1] = Tb;
    hkv[s] = 0;
  }
  std::fill(htab + (size_t)num_seqs * MB, htab + (size_t)Sb * MB, -1);
  // the device copy: cu and kv_lens whole-capacity prefixes, tables for Sb rows
  const size_t head = (size_t)c.max_seqs + 1 + c.max_seqs;
  if (hipMemcpyAsync(g->meta, hcu, sizeof(int32_t) * (head + (size_t)Sb * MB), hipMemcpyHostToDevice, upload) != hipSuccess ||
      hipEventRecord(g->staged[slot], upload) != hipSuccess)
    return cb::fail(CB_ERR_HIP, "metadata upload failed");
  return CB_OK;
}

// Runs the padded step `key` on `st` (after its metadata upload): eagerly, by recording or by
// replay.
int launch(G* g, const Key& key, hipStream_t st) {
  const auto& c = g->cfg;
  const size_t need = cb_paged_attention_workspace_size(std::get<0>(key), std::get<1>(key), c.num_q_heads,
                                                       c.num_kv_heads, c.head_dim, c.block_size,
                                                       std::get<2>(key), std::get<3>(key), 0);
  int r = ensure_workspace(g, need, st);
  if (r != CB_OK) return r;
  if (!c.use_graphs) {  // direct launches: the same padded step, no recording
    ++g->eager;
    r = enqueue_step(g, key, st);
    return r == CB_OK ? cb::ok() : r;
  }
  auto it = g->graphs.find(key);
  if (it == g->graphs.end() && !g->seen.count(key)) {
    // first use of a shape: run eagerly (creates any stream the step needs), record next time
    g->seen[key] = true;
    ++g->eager;
    r = enqueue_step(g, key, st);
    return r == CB_OK ? cb::ok() : r;
  }
  if (it == g->graphs.end()) {
    if ((int32_t)g->graphs.size() >= c.max_graphs) {  // evict the least recently used graph
      const Key old = g->lru.front();
      Entry& e = g->graphs[old];
      (void)hipEventSynchronize(e.done);
      (void)hipEventDestroy(e.done);
      (void)hipGraphExecDestroy(e.exec);
      g->lru.pop_front();
      g->graphs.erase(old);
    }
    Entry e;
    r = capture(g, key, st, &e.exec);
    if (r != CB_OK) return r;
    if (hipEventCreateWithFlags(&e.done, hipEventDisableTiming) != hipSuccess) {
      (void)hipGraphExecDestroy(e.exec);
      return cb::fail(CB_ERR_HIP, "event creation failed");
    }
    e.lru = g->lru.insert(g->lru.end(), key);
    it = g->graphs.emplace(key, e).first;
    ++g->captures;
  } else {
    g->lru.splice(g->lru.end(), g->lru, it->second.lru);
    ++g->replays;
  }
  if (hipGraphLaunch(it->second.exec, st) != hipSuccess || hipEventRecord(it->second.done, st) != hipSuccess)
    return cb::fail(CB_ERR_HIP, "hipGraphLaunch failed");
  return cb::ok();
}

}  // namespace

extern "C" int cb_graphs_run(cb_step_graphs* g, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                             const int32_t* block_tables, int32_t num_seqs, void* stream,
                             int32_t* padded_shape) {
  if (!g) return cb::fail(E, "executor is NULL");
  if (num_seqs < 0) return cb::fail(E, "num_seqs must be >= 0");
  if (num_seqs > 0 && (!cu_seqlens_q || !kv_lens || !block_tables)) return cb::fail(E, "NULL array");
  hipStream_t st = (hipStream_t)stream;
  if (!st) return cb::fail(E, "cb_graphs_run needs a stream other than NULL (NULL cannot be recorded)");
  if (num_seqs == 0) return cb::ok();
  Key key;
  int r = prepare(g, cu_seqlens_q, kv_lens, block_tables, num_seqs, st, &key);
  if (r != CB_OK) return r;
  if (padded_shape) {
    padded_shape[0] = std::get<0>(key);
    padded_shape[1] = std::get<1>(key);
    padded_shape[2] = std::get<2>(key);
    padded_shape[3] = std::get<3>(key);
  }
  return launch(g, key, st);
}

extern "C" int cb_graphs_stats(const cb_step_graphs* g, int64_t* captures, int64_t* replays,
                               int64_t* eager_runs, int32_t* cached) {
  if (!g) return cb::fail(E, "executor is NULL");
  if (captures) *captures = g->captures;
  if (replays) *replays = g->replays;
  if (eager_runs) *eager_runs = g->eager;
  if (cached) *cached = (int32_t)g->graphs.size();
  return cb::ok();
}

// ---------------------------------------------------------------------------------------------
// Async steps ("Continuous batching in transformers", Async batching): the CPU prepares step
// N + 1 while the GPU computes step N. Three streams (upload, compute, download) and, per I/O
// slot, three events (upload over, compute over, download over); two I/O slots used alternately
// (A/B), each with its own step executor (metadata buffers and recorded graphs: a graph records
// one slot's addresses); the carry-over adds the tokens step N produces into step N + 1's inputs
// on the compute stream, before the caller's forward pass.

#include "cbasync.h"

struct cb_async_steps {
  cb_async_config cfg{};
  cb_step_graphs* ex[2] = {nullptr, nullptr};
  hipStream_t up = nullptr, compute = nullptr, down = nullptr;
  hipEvent_t up_over[2] = {nullptr, nullptr}, compute_over[2] = {nullptr, nullptr},
             down_over[2] = {nullptr, nullptr};
  int64_t steps = 0;  // steps ended
  int open = -1;      // slot of the step begun and not yet ended
  bool attended = false;
  Key key{};
  int32_t tokens = 0;
};

namespace {

using A = cb_async_steps;

void async_release(A* a) {
  for (hipStream_t s : {a->up, a->compute, a->down})
    if (s) (void)hipStreamSynchronize(s);
  for (int i = 0; i < 2; ++i) {
    cb_graphs_destroy(a->ex[i]);
    for (hipEvent_t e : {a->up_over[i], a->compute_over[i], a->down_over[i]})
      if (e) (void)hipEventDestroy(e);
  }
  for (hipStream_t s : {a->up, a->compute, a->down})
    if (s) (void)hipStreamDestroy(s);
}

bool pinned_host(const void* p) {
  hipPointerAttribute_t attr{};
  const bool ok = hipPointerGetAttributes(&attr, p) == hipSuccess && attr.type == hipMemoryTypeHost;
  if (!ok) (void)hipGetLastError();
  return ok;
}

}  // namespace

extern "C" int cb_async_create(const cb_async_config* cfg, cb_async_steps** out) {
  if (!out) return cb::fail(E, "out is NULL");
  *out = nullptr;
  if (!cfg) return cb::fail(E, "cfg is NULL");
  for (int i = 0; i < 2; ++i) {
    if (!cfg->in_ids[i] || !cfg->out_ids[i] || !cfg->carry_dest[i] || !cfg->in_ids_host[i] ||
        !cfg->carry_dest_host[i] || !cfg->out_ids_host[i])
      return cb::fail(E, "cb_async_create: NULL buffer");
  }
  A* a = new (std::nothrow) A;
  if (!a) return cb::fail(E, "out of host memory");
  a->cfg = *cfg;
  for (int i = 0; i < 2; ++i) {
    const int r = cb_graphs_create(&cfg->step, &a->ex[i]);
    if (r != CB_OK) {
      async_release(a);
      delete a;
      return r;
    }
  }
  for (int i = 0; i < 2; ++i)
    if (!pinned_host(cfg->in_ids_host[i]) || !pinned_host(cfg->carry_dest_host[i]) ||
        !pinned_host(cfg->out_ids_host[i])) {
      async_release(a);
      delete a;
      return cb::fail(E, "cb_async_create: host buffers must be pinned (hipHostMalloc)");
    }
  bool ok = true;
  for (hipStream_t* s : {&a->up, &a->compute, &a->down})
    ok = ok && hipStreamCreateWithFlags(s, hipStreamNonBlocking) == hipSuccess;
  for (int i = 0; i < 2; ++i)
    for (hipEvent_t* e : {&a->up_over[i], &a->compute_over[i], &a->down_over[i]})
      ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    async_release(a);
    delete a;
    return cb::fail(CB_ERR_HIP, "cb_async_create: stream or event creation failed");
  }
  *out = a;
  return cb::ok();
}

extern "C" void cb_async_destroy(cb_async_steps* a) {
  if (!a) return;
  async_release(a);
  delete a;
}

extern "C" int cb_async_slot(cb_async_steps* a, int32_t* slot) {
  if (!a || !slot) return cb::fail(E, "NULL argument");
  const int s = (int)(a->steps % 2);
  // the slot's host inputs were read by its previous upload: wait for that copy
  if (hipEventSynchronize(a->up_over[s]) != hipSuccess) return cb::fail(CB_ERR_HIP, "upload wait failed");
  *slot = s;
  return cb::ok();
}

extern "C" int cb_async_begin(cb_async_steps* a, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                              const int32_t* block_tables, int32_t num_seqs, int32_t num_carried,
                              void** compute_stream) {
  if (!a) return cb::fail(E, "NULL handle");
  if (a->open >= 0) return cb::fail(E, "the previous step has not ended (cb_async_end)");
  if (num_seqs < 1 || !cu_seqlens_q || !kv_lens || !block_tables)
    return cb::fail(E, "a step needs at least one sequence and its metadata");
  const int32_t max_t = a->cfg.step.max_tokens;
  if (num_carried < 0 || num_carried > max_t || (a->steps == 0 && num_carried > 0))
    return cb::fail(E, "num_carried must be in [0, max_tokens] (0 for the first step)");
  const int s = (int)(a->steps % 2), prev = 1 - s;
  // the slot's device inputs are free once its previous step's compute has read them
  if (hipStreamWaitEvent(a->up, a->compute_over[s], 0) != hipSuccess)
    return cb::fail(CB_ERR_HIP, "upload stream wait failed");
  Key key;
  int r = prepare(a->ex[s], cu_seqlens_q, kv_lens, block_tables, num_seqs, a->up, &key);
  if (r != CB_OK) return r;
  const int32_t T = cu_seqlens_q[num_seqs];
  if (hipMemcpyAsync(a->cfg.in_ids[s], a->cfg.in_ids_host[s], sizeof(int32_t) * T,
                     hipMemcpyHostToDevice, a->up) != hipSuccess ||
      (num_carried > 0 && hipMemcpyAsync(a->cfg.carry_dest[s], a->cfg.carry_dest_host[s],
                                         sizeof(int32_t) * num_carried, hipMemcpyHostToDevice, a->up) != hipSuccess) ||
      hipEventRecord(a->up_over[s], a->up) != hipSuccess ||
      hipStreamWaitEvent(a->compute, a->up_over[s], 0) != hipSuccess)
    return cb::fail(CB_ERR_HIP, "input upload failed");
  // carry-over: the previous step's output tokens into this step's placeholders
  r = cb_carry_over(a->cfg.out_ids[prev], a->cfg.carry_dest[s], num_carried, a->cfg.in_ids[s], T,
                    a->compute);
  if (r != CB_OK) return r;
  a->open = s;
  a->attended = false;
  a->key = key;
  a->tokens = T;
  if (compute_stream) *compute_stream = a->compute;
  return cb::ok();
}

extern "C" int cb_async_attention(cb_async_steps* a) {
  if (!a) return cb::fail(E, "NULL handle");
  if (a->open < 0 || a->attended) return cb::fail(E, "no begun step awaits its attention");
  const int r = launch(a->ex[a->open], a->key, a->compute);
  if (r != CB_OK) return r;
  a->attended = true;
  return cb::ok();
}

extern "C" int cb_async_end(cb_async_steps* a, int32_t num_outputs) {
  if (!a) return cb::fail(E, "NULL handle");
  if (a->open < 0 || !a->attended) return cb::fail(E, "no step with its attention enqueued is open");
  if (num_outputs < 0 || num_outputs > a->cfg.step.max_tokens)
    return cb::fail(E, "num_outputs must be in [0, max_tokens]");
  const int s = a->open;
  if (hipEventRecord(a->compute_over[s], a->compute) != hipSuccess ||
      hipStreamWaitEvent(a->down, a->compute_over[s], 0) != hipSuccess ||
      (num_outputs > 0 && hipMemcpyAsync(a->cfg.out_ids_host[s], a->cfg.out_ids[s], sizeof(int32_t) * num_outputs,
                                         hipMemcpyDeviceToHost, a->down) != hipSuccess) ||
      hipEventRecord(a->down_over[s], a->down) != hipSuccess)
    return cb::fail(CB_ERR_HIP, "output download failed");
  a->open = -1;
  ++a->steps;
  return cb::ok();
}

extern "C" int cb_async_wait(cb_async_steps* a, int32_t slot) {
  if (!a || slot < 0 || slot > 1) return cb::fail(E, "bad handle or slot");
  if (hipEventSynchronize(a->down_over[slot]) != hipSuccess) return cb::fail(CB_ERR_HIP, "download wait failed");
  return cb::ok();
}
