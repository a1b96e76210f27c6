// Slot mapping and the paged KV-cache write (integer and copy work, no floating point).
//
// Slot of a new token: "3.3 Batching & Memory Management", section "PagedAttention: block
// tables" — position p of a sequence lives in physical block table[p / bs] at offset p % bs.
// Cache write: "Continuous batching in transformers", paged-cache section — the cache tensor is
// the physical store of pages, one page per token per layer for K and for V.
#include <hip/hip_runtime.h>

#include "cb_internal.h"

namespace {

constexpr int kSlotThreads = 256;

// One wave per sequence; lanes stride over the sequence's new tokens.
__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
    int32_t block_size, int32_t* __restrict__ slot_mapping) {
  const int s = blockIdx.x * (kSlotThreads / 64) + (threadIdx.x >> 6);
  if (s >= num_seqs) return;
  const int lane = threadIdx.x & 63;
  const int t0 = cu[s];
  const int q = cu[s + 1] - t0;
  const int first_pos = kv_lens[s] - q;  // position of the sequence's first new token
  const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
  for (int i = lane; i < q; i += 64) {
    const int p = first_pos + i;
    const int j = p / block_size;
    // positions a valid batch cannot have (kv_len < q, or past the table row) get slot -1
    const bool ok = p >= 0 && j < max_blocks_per_seq;
    slot_mapping[t0 + i] = ok ? row[j] * block_size + (p % block_size) : -1;
  }
}

// One thread per 16-byte chunk of a token's K row or V row; rows of all Hkv heads are one
// contiguous [Hkv * D] run in both the new-token tensors and a cache slot. Slots outside
// [0, num_slots) are skipped (-1 marks a token with no slot; larger ones are not in the pool).
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int32_t* __restrict__ slots,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int32_t num_tokens,
    int32_t chunks_per_row, int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tensor = (int64_t)num_tokens * chunks_per_row;
  if (idx >= 2 * per_tensor) return;
  const bool is_v = idx >= per_tensor;
  const int64_t r = is_v ? idx - per_tensor : idx;
  const int64_t t = r / chunks_per_row;
  const int64_t c = r - t * chunks_per_row;
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const uint4* src = is_v ? v : k;
  uint4* dst = is_v ? v_cache : k_cache;
  dst[(int64_t)slot * chunks_per_row + c] = src[t * chunks_per_row + c];
}

// One thread per output of the previous step (see cb_carry_over).
__global__ __launch_bounds__(256) void carry_over_kernel(const int32_t* __restrict__ prev_out,
                                                         const int32_t* __restrict__ dest,
                                                         int32_t n, int32_t* __restrict__ next_in,
                                                         int32_t n_next) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t d = dest[i];
  if (d >= 0 && d < n_next) next_in[d] += prev_out[i];
}

}  // namespace

extern "C" int cb_carry_over(const int32_t* prev_outputs, const int32_t* dest, int32_t num_prev,
                             int32_t* next_inputs, int32_t num_next, void* stream) {
  using cb::fail;
  if (num_prev < 0 || num_next < 0) return fail(CB_ERR_INVALID_ARG, "cb_carry_over: negative size");
  if (num_prev == 0 || num_next == 0) return cb::ok();
  if (!prev_outputs || !dest || !next_inputs) return fail(CB_ERR_INVALID_ARG, "cb_carry_over: NULL pointer");
  carry_over_kernel<<<(num_prev + 255) / 256, 256, 0, (hipStream_t)stream>>>(prev_outputs, dest, num_prev,
                                                                           next_inputs, num_next);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CB_ERR_HIP, std::string("carry_over launch: ") + hipGetErrorString(e));
  return cb::ok();
}

extern "C" int cb_slot_mapping(const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                               const int32_t* block_tables, int32_t num_seqs, int32_t num_tokens,
                               int32_t max_blocks_per_seq, int32_t block_size,
                               int32_t* slot_mapping, void* stream) {
  using cb::fail;
  if (block_size < 4)
    return fail(CB_ERR_INVALID_ARG, "block_size must be at least 4, got " + std::to_string(block_size));
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 0)
    return fail(CB_ERR_INVALID_ARG, "negative size argument");
  if (num_seqs == 0 || num_tokens == 0) return cb::ok();
  if (!cu_seqlens_q || !kv_lens || !block_tables || !slot_mapping)
    return fail(CB_ERR_INVALID_ARG, "cb_slot_mapping: NULL pointer argument");
  if (max_blocks_per_seq < 1) return fail(CB_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  const int waves = kSlotThreads / 64;
  const int grid = (num_seqs + waves - 1) / waves;
  slot_mapping_kernel<<<grid, kSlotThreads, 0, (hipStream_t)stream>>>(
      cu_seqlens_q, kv_lens, block_tables, num_seqs, max_blocks_per_seq, block_size, slot_mapping);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(CB_ERR_HIP, std::string("slot_mapping launch: ") + hipGetErrorString(e));
  return cb::ok();
}

extern "C" int cb_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                              void* k_cache, void* v_cache, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, void* stream) {
  using cb::fail;
  if (block_size < 4)
    return fail(CB_ERR_INVALID_ARG, "block_size must be at least 4, got " + std::to_string(block_size));
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || num_blocks < 1)
    return fail(CB_ERR_INVALID_ARG, "cb_cache_write: bad size argument");
  if (((int64_t)num_kv_heads * head_dim) % 8 != 0)
    return fail(CB_ERR_UNSUPPORTED, "num_kv_heads * head_dim must be a multiple of 8");
  if (num_tokens == 0) return cb::ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(CB_ERR_INVALID_ARG, "cb_cache_write: NULL pointer argument");
  if (!cb::aligned16(k) || !cb::aligned16(v) || !cb::aligned16(k_cache) || !cb::aligned16(v_cache))
    return fail(CB_ERR_INVALID_ARG, "cb_cache_write: bf16 tensors must be 16-byte aligned");
  const int32_t chunks = (int32_t)((int64_t)num_kv_heads * head_dim * 2 / 16);
  const int64_t total = 2 * (int64_t)num_tokens * chunks;
  const int64_t grid = (total + 255) / 256;
  // a dispatch holds fewer than 2^32 work-items
  if (grid * 256 > (int64_t)UINT32_MAX) return fail(CB_ERR_UNSUPPORTED, "cb_cache_write: batch too large");
  cache_write_kernel<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(
      (const uint4*)k, (const uint4*)v, slot_mapping, (uint4*)k_cache, (uint4*)v_cache,
      num_tokens, chunks, num_blocks * block_size);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(CB_ERR_HIP, std::string("cache_write launch: ") + hipGetErrorString(e));
  return cb::ok();
}
