// Read-stream reference for measurements: reads a buffer the way the decode
// kernels read their pages (16-byte loads, 1 KB per wave instruction, every
// load of a workgroup issued before the first is used) and keeps nothing but
// one XOR word per 16 KB chunk, so that its time is the read rate this GPU
// reaches for that many bytes, the figure a decode's fraction of the HBM
// peak is read against. Not part of the method.
#include "kvq_internal.h"

namespace kvq {

constexpr int STREAM_CHUNK = 16384;   // bytes per workgroup: 16 wave loads of 1 KB
typedef uint32_t stream_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void read_stream_kernel(const uint8_t* src, size_t bytes, uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * STREAM_CHUNK;
  const int lane = threadIdx.x;
  stream_u32x4 v[STREAM_CHUNK / 1024];
#pragma unroll
  for (int i = 0; i < STREAM_CHUNK / 1024; ++i) {
    const size_t off = base + 1024 * i + 16 * lane;
    v[i] = off < bytes ? *reinterpret_cast<const stream_u32x4*>(src + off) : (stream_u32x4){0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < STREAM_CHUNK / 1024; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  if (lane == 0) sink[blockIdx.x] = x;
}

}  // namespace kvq

extern "C" kvq_status kvq_read_stream(const void* src, size_t bytes, uint32_t* sink, size_t sink_bytes,
                                      void* stream) {
  if (bytes == 0) return KVQ_OK;
  if (!src || !sink || ((uintptr_t)src & 15u) || ((uintptr_t)sink & 3u) || (bytes & 15u)) return KVQ_INVALID_ARG;
  const size_t chunks = (bytes + kvq::STREAM_CHUNK - 1) / kvq::STREAM_CHUNK;
  if (sink_bytes < 4 * chunks) return KVQ_WORKSPACE_TOO_SMALL;
  if (chunks > 0x7fffffffu) return KVQ_INVALID_ARG;
  hipLaunchKernelGGL(kvq::read_stream_kernel, dim3((unsigned)chunks), dim3(64), 0, (hipStream_t)stream,
                     (const uint8_t*)src, bytes, sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}
