// Device helpers shared by the gfx950 kernels: 16-byte element loads,
// wave64 reductions and scans, and the order-preserving float key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loki {

constexpr int kBlock = 256;  // threads per workgroup of the decode kernels
constexpr float kLog2e = 1.4426950408889634f;

// Element formats.  VEC = elements per 16-byte load.
struct F32 {
  using T = float;
  static constexpr int VEC = 4;
  static constexpr int BYTES = 4;
};
struct BF16 {
  using T = uint16_t;
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
};

// bf16 bit pattern -> float32 (exact: bf16 is the upper half of a float32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw 16-byte chunk; converted to floats separately so that loads can be
// issued ahead of their use.
struct Chunk {
  uint4 u;
};

__device__ __forceinline__ Chunk ld16(const void* p) {
  Chunk c;
  c.u = *reinterpret_cast<const uint4*>(p);
  return c;
}

__device__ __forceinline__ Chunk zero_chunk() {
  Chunk c;
  c.u = make_uint4(0u, 0u, 0u, 0u);
  return c;
}

template <class E>
__device__ __forceinline__ void unpack(const Chunk& c, float (&x)[E::VEC]);

template <>
__device__ __forceinline__ void unpack<F32>(const Chunk& c, float (&x)[4]) {
  x[0] = __uint_as_float(c.u.x);
  x[1] = __uint_as_float(c.u.y);
  x[2] = __uint_as_float(c.u.z);
  x[3] = __uint_as_float(c.u.w);
}

template <>
__device__ __forceinline__ void unpack<BF16>(const Chunk& c, float (&x)[8]) {
  x[0] = bf16_lo(c.u.x);
  x[1] = bf16_hi(c.u.x);
  x[2] = bf16_lo(c.u.y);
  x[3] = bf16_hi(c.u.y);
  x[4] = bf16_lo(c.u.z);
  x[5] = bf16_hi(c.u.z);
  x[6] = bf16_lo(c.u.w);
  x[7] = bf16_hi(c.u.w);
}

// Scalar element load (used for queries, which are read once).
template <class E>
__device__ __forceinline__ float ld_elem(const typename E::T* p, int64_t i);

template <>
__device__ __forceinline__ float ld_elem<F32>(const float* p, int64_t i) { return p[i]; }

template <>
__device__ __forceinline__ float ld_elem<BF16>(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of the group receives the group total.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    unsigned y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Order-preserving map float32 -> uint32: a > b (as floats) iff key(a) >
// key(b); -0.0 is first made +0.0 so the two rank equal.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = (x == 0.0f) ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace loki
