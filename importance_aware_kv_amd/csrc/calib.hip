// calib.hip -- measurement aids for the decode step's roofline (see
// include/hikv_calib.h): a streaming read of the live KV rows in the cache's
// layout, and an empty kernel.  Nothing of the method is computed here.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "hikv_calib.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads per lane in flight

__global__ __launch_bounds__(kThreads) void k_stream(const char *k, const char *v, int64_t cap, int64_t rb,
                                                     const int32_t *tiles, uint32_t *sink) {
  const int tile = blockIdx.x, tid = threadIdx.x;
  const int u = tiles[3 * tile], t0 = tiles[3 * tile + 1], t1 = tiles[3 * tile + 2];
  const int64_t base = (int64_t)u * cap * rb + (int64_t)t0 * rb;
  const int64_t n16 = ((int64_t)(t1 - t0) * rb) / 16;  // 16-byte pieces of the tile in each array
  const uint4 *kp = reinterpret_cast<const uint4 *>(k + base);
  const uint4 *vp = reinterpret_cast<const uint4 *>(v + base);
  uint32_t acc = 0;
  for (int64_t i0 = tid; i0 < n16; i0 += (int64_t)kThreads * kUnroll) {
    uint4 a[kUnroll], b[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t i = i0 + (int64_t)j * kThreads;
      const int64_t ic = i < n16 ? i : n16 - 1;
      a[j] = kp[ic];
      b[j] = vp[ic];
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= a[j].x ^ a[j].y ^ a[j].z ^ a[j].w ^ b[j].x ^ b[j].y ^ b[j].z ^ b[j].w;
  }
  // one word per tile: the lanes' values folded (keeps every load live)
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t w[kThreads / 64];
  if ((tid & 63) == 0) w[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) sink[tile] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

__global__ void k_empty() {}

}  // namespace

extern "C" int hikv_calib_stream(const void *k, const void *v, int64_t cap, int64_t row_bytes, const int32_t *tiles,
                                 int32_t n_tiles, uint32_t *sink, void *ev_start, void *ev_stop, void *stream) {
  if (!k || !v || !tiles || !sink || n_tiles < 0 || cap <= 0 || row_bytes <= 0 || row_bytes % 16) return -1;
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u) return -1;
  if ((ev_start == nullptr) != (ev_stop == nullptr)) return -1;
  if (n_tiles == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ev_start) {
    hipExtLaunchKernelGGL(k_stream, dim3((unsigned)n_tiles), dim3(kThreads), 0, s, static_cast<hipEvent_t>(ev_start),
                          static_cast<hipEvent_t>(ev_stop), 0, static_cast<const char *>(k),
                          static_cast<const char *>(v), cap, row_bytes, tiles, sink);
  } else {
    hipLaunchKernelGGL(k_stream, dim3((unsigned)n_tiles), dim3(kThreads), 0, s, static_cast<const char *>(k),
                       static_cast<const char *>(v), cap, row_bytes, tiles, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hikv_calib_empty(int32_t n, void *stream) {
  if (n < 0) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
