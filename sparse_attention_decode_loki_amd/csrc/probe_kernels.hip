// Streaming-read probe: the measured HBM read ceiling the decode kernels are
// compared with.  A grid-stride loop of nontemporal 16-byte loads over a
// buffer; each thread writes its sum so that no load can be dropped.
#include "launch.hpp"

namespace loki {

namespace {

constexpr int kProbeBlock = 256;

__global__ void __launch_bounds__(kProbeBlock) stream_read_kernel(const float4* __restrict__ p,
                                                                  size_t n, float* __restrict__ sink) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4* q = reinterpret_cast<const f4*>(p);
  const size_t stride = static_cast<size_t>(gridDim.x) * kProbeBlock;
  float acc = 0.f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kProbeBlock + threadIdx.x; i < n; i += stride) {
    const f4 v = __builtin_nontemporal_load(q + i);
    acc += (v.x + v.y) + (v.z + v.w);
  }
  sink[static_cast<size_t>(blockIdx.x) * kProbeBlock + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, float* sink, int workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeBlock), 0, stream,
                     static_cast<const float4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace loki
