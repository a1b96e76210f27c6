// Measurement aid, not an operation of the method: a plain streaming read of a device buffer,
// the HBM read rate that the bandwidth-bound kernels are reported against beside the 8 TB/s
// specification.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "cb_internal.h"

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;     // 16-byte loads in flight per lane
constexpr int kReadGroups = 1024;  // workgroups (four per compute unit)

__device__ inline uint4 ld_nt16(const uint4* p) {
  uint4 v;
  v.x = __builtin_nontemporal_load(&p->x);
  v.y = __builtin_nontemporal_load(&p->y);
  v.z = __builtin_nontemporal_load(&p->z);
  v.w = __builtin_nontemporal_load(&p->w);
  return v;
}

// The buffer is read in chunks of 64 * kReadUnroll 16-byte elements (4 KB), one chunk per wave
// at a time, chunks dealt to the waves in turn; every load instruction of a wave reads 1 KB of
// contiguous memory. A sweep on MI355X (2 GiB): 6.96 TB/s this way with 1024 workgroups, 5.9-6.0
// TB/s with each lane striding over the whole grid. Each thread folds what it read into one
// word, written to sink[thread], so that no load is dead.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kReadThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * (kReadThreads / 64);
  constexpr int64_t CH = 64 * kReadUnroll;
  uint32_t acc = 0;
  const int64_t full = n16 / CH;
  for (int64_t c = wave; c < full; c += nwaves) {
    const uint4* q = buf + c * CH + lane;
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = ld_nt16(q + 64 * u);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (wave == full % nwaves)  // the last, partial chunk
    for (int64_t i = full * CH + lane; i < n16; i += 64) {
      const uint4 v = ld_nt16(buf + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  sink[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int cb_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_words,
                              void* stream) {
  using cb::fail;
  if (bytes == 0) return cb::ok();
  if (!buf || !sink) return fail(CB_ERR_INVALID_ARG, "cb_stream_read: NULL pointer argument");
  if (!cb::aligned16(buf) || bytes % 16 != 0)
    return fail(CB_ERR_INVALID_ARG, "cb_stream_read: buffer must be 16-byte aligned, a multiple of 16 bytes");
  if (sink_words < kReadThreads)
    return fail(CB_ERR_INVALID_ARG, "cb_stream_read: sink must hold at least 256 words");
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = std::min<int64_t>({(int64_t)kReadGroups, sink_words / kReadThreads,
                                            std::max<int64_t>(1, n16 / (64 * kReadUnroll))});
  stream_read_kernel<<<(unsigned)blocks, kReadThreads, 0, (hipStream_t)stream>>>(
      static_cast<const uint4*>(buf), n16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CB_ERR_HIP, std::string("stream read launch: ") + hipGetErrorString(e));
  return cb::ok();
}
