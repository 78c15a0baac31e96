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

// Each workgroup reads its own contiguous share of `share` 16-byte chunks,
// U loads in flight per lane: the read pattern of a kernel that gives every
// workgroup one row (as the decode kernels do), at a chosen occupancy.
template <int NT, int U>
__global__ void __launch_bounds__(NT) share_read_kernel(const float4* __restrict__ p, size_t share,
                                                        float* __restrict__ sink) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4* base = reinterpret_cast<const f4*>(p) + static_cast<size_t>(blockIdx.x) * share;
  float acc = 0.f;
  for (size_t i = threadIdx.x; i < share; i += static_cast<size_t>(NT) * U) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + static_cast<size_t>(u) * NT;
      v[u] = j < share ? __builtin_nontemporal_load(base + j) : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  sink[static_cast<size_t>(blockIdx.x) * NT + threadIdx.x] = acc;
}

template <int NT>
hipError_t share_read_t(const float4* p, size_t share, float* sink, int workgroups, int loads,
                        hipStream_t stream) {
  switch (loads) {
    case 1: hipLaunchKernelGGL((share_read_kernel<NT, 1>), dim3(workgroups), dim3(NT), 0, stream, p, share, sink); break;
    case 2: hipLaunchKernelGGL((share_read_kernel<NT, 2>), dim3(workgroups), dim3(NT), 0, stream, p, share, sink); break;
    case 4: hipLaunchKernelGGL((share_read_kernel<NT, 4>), dim3(workgroups), dim3(NT), 0, stream, p, share, sink); break;
    case 8: hipLaunchKernelGGL((share_read_kernel<NT, 8>), dim3(workgroups), dim3(NT), 0, stream, p, share, sink); break;
    case 16: hipLaunchKernelGGL((share_read_kernel<NT, 16>), dim3(workgroups), dim3(NT), 0, stream, p, share, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_share_read(const void* buf, size_t bytes, float* sink, int workgroups,
                             int threads, int loads, hipStream_t stream) {
  const auto* p = static_cast<const float4*>(buf);
  const size_t share = bytes / 16 / static_cast<size_t>(workgroups);
  switch (threads) {
    case 256: return share_read_t<256>(p, share, sink, workgroups, loads, stream);
    case 512: return share_read_t<512>(p, share, sink, workgroups, loads, stream);
    case 1024: return share_read_t<1024>(p, share, sink, workgroups, loads, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_read(const void* buf, size_t bytes, float* sink, int workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeBlock), 0, stream,
                     static_cast<const float4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace loki
