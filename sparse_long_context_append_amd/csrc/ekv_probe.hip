// Read-bandwidth probe: a plain streaming read of a device buffer, the
// ceiling the decode step's kernels are compared with at their own
// working-set sizes.  Measurement helper only; not part of the decode path.
//
// Every thread reads 16-byte words at a grid stride with eight loads in
// flight, and folds them with XOR; the result decides a store to `sink`
// (made only for one fixed pattern), so no load can be dropped.
#include "ekv_kernels.h"

namespace ekv {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                                    uint32_t* sink) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= (v[u].x ^ v[u].y) ^ (v[u].z ^ v[u].w);
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= (v.x ^ v.y) ^ (v.z ^ v.w);
  }
  if (acc == 0x9E3779B9u) atomicOr(sink, 1u);
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace ekv
