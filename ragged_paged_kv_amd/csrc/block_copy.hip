// Copy-on-write data movement: copy whole physical KV blocks, K and V, in every layer.
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

}  // namespace

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
