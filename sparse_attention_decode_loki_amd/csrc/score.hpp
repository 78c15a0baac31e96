// Streaming pass of the ranking scores over the d-wide key slab, and the
// XCD-aware workgroup order shared by the decode kernels.
#pragma once

#include "device.hpp"

namespace loki {

// ----------------------------------------------------------------- helpers --

// Workgroup id -> logical id such that consecutive logical ids land on the
// same XCD (workgroups are dealt round-robin over the 8 XCDs), so the
// sequences of one head share that head's basis in one L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
  if ((n & 7) != 0) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

// Scores of tokens [j0, j1) for NH heads.  LPS lanes share one token's slab
// row (d*bytes/16 lanes rounded up to a power of two; lanes past the row
// idle); a wave covers 64/LPS consecutive tokens per load, so the slab is
// streamed with fully coalesced 16-byte loads.  score_first issues the first
// batch of loads, which do not depend on the query, so a caller can start
// them before the query is rotated.
template <class E, int LPS, int U, int NT = kBlock>
__device__ __forceinline__ void score_first(const typename E::T* __restrict__ slab, int d, int j0,
                                            int j1, Chunk (&c)[U]) {
  constexpr int VEC = E::VEC;
  constexpr int TPI = NT / LPS;
  const int part = threadIdx.x % LPS;
  const int tk = threadIdx.x / LPS;
  const bool active = part * VEC < d;
  const Region gs = make_region(slab, 0x7fffffffu);
  const uint32_t row = static_cast<uint32_t>(d) * E::BYTES;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = j0 + tk + TPI * u;
    c[u] = (active && j < j1) ? ld16_region(gs, static_cast<uint32_t>(j) * row + part * 16u)
                              : zero_chunk();
  }
}

// c holds the first batch (from score_first).
template <class E, int LPS, int NH, int U, int NT = kBlock, class Write>
__device__ __forceinline__ void score_loop(const typename E::T* __restrict__ slab, int d, int j0,
                                           int j1, const float (&qf)[NH][E::VEC], Write write,
                                           Chunk (&c)[U]) {
  constexpr int VEC = E::VEC;
  constexpr int TPI = NT / LPS;
  const int part = threadIdx.x % LPS;
  const int tk = threadIdx.x / LPS;
  const bool active = part * VEC < d;
  const Region gs = make_region(slab, 0x7fffffffu);
  const uint32_t row = static_cast<uint32_t>(d) * E::BYTES;
  for (int jb = j0 + tk; jb < j1; jb += TPI * U) {
    if (jb != j0 + tk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jb + TPI * u;
        c[u] = (active && j < j1) ? ld16_region(gs, static_cast<uint32_t>(j) * row + part * 16u)
                                  : zero_chunk();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[VEC];
      unpack<E>(c[u], x);
      const int j = jb + TPI * u;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot = fmaf(qf[h][v], x[v], dot);
        dot = group_sum<LPS>(dot);
        if (part == 0 && j < j1) write(h, j, dot);
      }
    }
  }
}

}  // namespace loki
