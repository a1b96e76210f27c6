// Block data movement: copy-on-write copies of whole physical KV blocks, K and V, in every
// layer; and the swap tier's gather to and scatter from a pinned host pool.
//
// "3.3 Batching & Memory Management", section "Sharing and copy-on-write": before a sequence
// writes into a block other sequences still reference, the engine copies the block and points
// this sequence's table at the copy. The host block manager decides the (src, dst) pairs; this
// kernel moves the bytes. Pure copy work, bound by HBM bandwidth: each pair moves
// 2 (K and V) x num_layers x block_bytes in and out.
#include <hip/hip_runtime.h>

#include "cb_internal.h"
#include "cbblocks.h"

namespace {

// Measured on MI355X over 256 copies of 32 KiB blocks in 32 layers: one 16-byte chunk per lane,
// 128-lane workgroups, and nontemporal loads and stores (the copied blocks are not read again by
// this kernel, so they should not displace cache lines) gave the highest rate.
constexpr int kCopyThreads = 128;
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * 16;  // bytes per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per kCopyChunk bytes of one block copy of one tensor (K or V) of one layer.
// Workgroups are ordered chunk-fastest, so consecutive workgroups stream one block's run.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, int32_t num_layers, int64_t block_bytes,
    int64_t num_blocks, int64_t layer_stride, int32_t chunks_per_block) {
  const int64_t wg = blockIdx.x;
  const int32_t chunk = (int32_t)(wg % chunks_per_block);
  const int64_t rest = wg / chunks_per_block;
  const int32_t is_v = (int32_t)(rest & 1);
  const int64_t lp = rest >> 1;
  const int32_t layer = (int32_t)(lp % num_layers);
  const int64_t pair = lp / num_layers;
  const int32_t s = src[pair], d = dst[pair];
  // pairs a valid manager never produces (out of range, or a block onto itself) are skipped
  if (s < 0 || d < 0 || s >= num_blocks || d >= num_blocks || s == d) return;
  uint8_t* base = (is_v ? v_cache : k_cache) + (int64_t)layer * layer_stride;
  const u32x4* from = reinterpret_cast<const u32x4*>(base + (int64_t)s * block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(base + (int64_t)d * block_bytes);
  const int64_t c = (int64_t)chunk * kCopyThreads + threadIdx.x;
  if (c < block_bytes / 16) __builtin_nontemporal_store(__builtin_nontemporal_load(from + c), to + c);
}

// Swap tier: one workgroup per kCopyChunk bytes of one block of K or V of one layer, moving it
// between the caches and a pinned host pool laid out [slot][K, V][layer][block_bytes]. TO_HOST
// gathers cache blocks into pool slots (stores over PCIe), otherwise pool slots are scattered
// into cache blocks (loads over PCIe).
template <bool TO_HOST>
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, uint8_t* __restrict__ pool,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ slots, int32_t num_layers,
    int64_t block_bytes, int64_t num_blocks, int64_t num_slots, int64_t layer_stride,
    int32_t chunks_per_block) {
  const int64_t wg = blockIdx.x;
  const int32_t chunk = (int32_t)(wg % chunks_per_block);
  const int64_t rest = wg / chunks_per_block;
  const int32_t is_v = (int32_t)(rest & 1);
  const int64_t lp = rest >> 1;
  const int32_t layer = (int32_t)(lp % num_layers);
  const int64_t pair = lp / num_layers;
  const int32_t b = blocks[pair], sl = slots[pair];
  if (b < 0 || b >= num_blocks || sl < 0 || sl >= num_slots) return;  // skipped pair
  u32x4* dev = reinterpret_cast<u32x4*>((is_v ? v_cache : k_cache) + (int64_t)layer * layer_stride +
                                        (int64_t)b * block_bytes);
  u32x4* host = reinterpret_cast<u32x4*>(pool + (((int64_t)sl * 2 + is_v) * num_layers + layer) * block_bytes);
  const int64_t c = (int64_t)chunk * kCopyThreads + threadIdx.x;
  if (c >= block_bytes / 16) return;
  if (TO_HOST)
    __builtin_nontemporal_store(__builtin_nontemporal_load(dev + c), host + c);
  else
    __builtin_nontemporal_store(__builtin_nontemporal_load(host + c), dev + c);
}

// Checks a swap call and returns the device address of the pinned pool (0 on error).
int swap_args(const void* k_cache, const void* v_cache, const void* pool, const int32_t* blocks,
              const int32_t* slots, int32_t n, int64_t num_slots, int64_t block_bytes,
              int64_t num_blocks, int32_t num_layers, int64_t layer_stride, void** pool_dev,
              int64_t* grid, int64_t* chunks) {
  using cb::fail;
  const int E = CB_ERR_INVALID_ARG;
  if (n < 0 || num_slots < 1) return fail(E, "swap: n must be >= 0 and num_slots >= 1");
  if (block_bytes < 16 || block_bytes % 16 != 0)
    return fail(E, "swap: block_bytes must be a positive multiple of 16");
  if (num_blocks < 1 || num_layers < 1) return fail(E, "swap: num_blocks and num_layers must be >= 1");
  if (num_layers > 1 && (layer_stride < num_blocks * block_bytes || layer_stride % 16 != 0))
    return fail(E, "swap: layer_stride_bytes must be a multiple of 16 and hold num_blocks blocks");
  if (n == 0) return CB_OK;
  if (!k_cache || !v_cache || !pool || !blocks || !slots) return fail(E, "swap: NULL pointer argument");
  if (!cb::aligned16(k_cache) || !cb::aligned16(v_cache) || !cb::aligned16(pool))
    return fail(E, "swap: caches and pool must be 16-byte aligned");
  // the pool must be pinned host memory the GPU can address (pageable memory would fault it)
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, pool) != hipSuccess || attr.type != hipMemoryTypeHost ||
      !attr.devicePointer) {
    (void)hipGetLastError();  // the query's own error is not the caller's
    return fail(E, "swap: the pool is not pinned host memory (allocate it with hipHostMalloc)");
  }
  *pool_dev = attr.devicePointer;
  *chunks = cb::ceil_div(block_bytes, kCopyChunk);
  *grid = (int64_t)n * num_layers * 2 * *chunks;
  if (*grid * kCopyThreads > (int64_t)UINT32_MAX) return fail(CB_ERR_UNSUPPORTED, "swap: too many blocks in one call");
  return CB_OK;
}

}  // namespace

extern "C" int cb_swap_out_blocks(const void* k_cache, const void* v_cache, const int32_t* blocks,
                                  const int32_t* slots, int32_t num_pairs, void* host_pool,
                                  int64_t num_slots, int64_t block_bytes, int64_t num_blocks,
                                  int32_t num_layers, int64_t layer_stride_bytes, void* stream) {
  void* pool = nullptr;
  int64_t grid = 0, chunks = 0;
  const int r = swap_args(k_cache, v_cache, host_pool, blocks, slots, num_pairs, num_slots, block_bytes,
                          num_blocks, num_layers, layer_stride_bytes, &pool, &grid, &chunks);
  if (r != CB_OK || num_pairs == 0) return r == CB_OK ? cb::ok() : r;
  swap_blocks_kernel<true><<<(unsigned)grid, kCopyThreads, 0, (hipStream_t)stream>>>(
      (uint8_t*)k_cache, (uint8_t*)v_cache, (uint8_t*)pool, blocks, slots, num_layers, block_bytes,
      num_blocks, num_slots, num_layers > 1 ? layer_stride_bytes : 0, (int32_t)chunks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return cb::fail(CB_ERR_HIP, std::string("swap_out launch: ") + hipGetErrorString(e));
  return cb::ok();
}

extern "C" int cb_swap_in_blocks(const void* host_pool, const int32_t* slots, const int32_t* blocks,
                                 int32_t num_pairs, void* k_cache, void* v_cache, int64_t num_slots,
                                 int64_t block_bytes, int64_t num_blocks, int32_t num_layers,
                                 int64_t layer_stride_bytes, void* stream) {
  void* pool = nullptr;
  int64_t grid = 0, chunks = 0;
  const int r = swap_args(k_cache, v_cache, host_pool, blocks, slots, num_pairs, num_slots, block_bytes,
                          num_blocks, num_layers, layer_stride_bytes, &pool, &grid, &chunks);
  if (r != CB_OK || num_pairs == 0) return r == CB_OK ? cb::ok() : r;
  swap_blocks_kernel<false><<<(unsigned)grid, kCopyThreads, 0, (hipStream_t)stream>>>(
      (uint8_t*)k_cache, (uint8_t*)v_cache, (uint8_t*)pool, blocks, slots, num_layers, block_bytes,
      num_blocks, num_slots, num_layers > 1 ? layer_stride_bytes : 0, (int32_t)chunks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return cb::fail(CB_ERR_HIP, std::string("swap_in launch: ") + hipGetErrorString(e));
  return cb::ok();
}

extern "C" int cb_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                              const int32_t* dst_blocks, int32_t num_copies, int64_t block_bytes,
                              int64_t num_blocks, int32_t num_layers, int64_t layer_stride_bytes,
                              void* stream) {
  using cb::fail;
  const int E = CB_ERR_INVALID_ARG;
  if (num_copies < 0) return fail(E, "cb_copy_blocks: num_copies must be >= 0");
  if (block_bytes < 16 || block_bytes % 16 != 0)
    return fail(E, "cb_copy_blocks: block_bytes must be a positive multiple of 16");
  if (num_blocks < 1 || num_layers < 1) return fail(E, "cb_copy_blocks: num_blocks and num_layers must be >= 1");
  if (num_layers > 1 && (layer_stride_bytes < num_blocks * block_bytes || layer_stride_bytes % 16 != 0))
    return fail(E, "cb_copy_blocks: layer_stride_bytes must be a multiple of 16 and hold num_blocks blocks");
  if (num_copies == 0) return cb::ok();
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks)
    return fail(E, "cb_copy_blocks: NULL pointer argument");
  if (!cb::aligned16(k_cache) || !cb::aligned16(v_cache))
    return fail(E, "cb_copy_blocks: caches must be 16-byte aligned");
  const int64_t chunks = cb::ceil_div(block_bytes, kCopyChunk);
  if (chunks > INT32_MAX) return fail(CB_ERR_UNSUPPORTED, "cb_copy_blocks: block too large");
  const int64_t grid = (int64_t)num_copies * num_layers * 2 * chunks;
  // a dispatch holds fewer than 2^32 work-items
  if (grid * kCopyThreads > (int64_t)UINT32_MAX)
    return fail(CB_ERR_UNSUPPORTED, "cb_copy_blocks: too many copies in one call");
  copy_blocks_kernel<<<(unsigned)grid, kCopyThreads, 0, (hipStream_t)stream>>>(
      (uint8_t*)k_cache, (uint8_t*)v_cache, src_blocks, dst_blocks, num_layers, block_bytes,
      num_blocks, num_layers > 1 ? layer_stride_bytes : 0, (int32_t)chunks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CB_ERR_HIP, std::string("copy_blocks launch: ") + hipGetErrorString(e));
  return cb::ok();
}
