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

// 16-byte load of data read once per launch (key slab stream, gathered key
// and value rows): marked nontemporal, so it does not displace reused lines
// from the caches.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Chunk ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  Chunk c;
  c.u = make_uint4(v.x, v.y, v.z, v.w);
  return c;
}

// Buffer resource over one (sequence, KV head) region of a cache tensor:
// loads take 32-bit byte offsets from the region base (wave-uniform in
// SGPRs), and an offset past `bytes` reads zeros.
struct Region {
  __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ Region make_region(const void* base, uint32_t bytes) {
  Region g;
  g.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                          static_cast<int>(bytes), 0x00020000);
  return g;
}

// Cache policy of the streamed and gathered loads (read once per launch):
// nontemporal.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ Chunk ld16_region(const Region& g, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(g.r, static_cast<int>(off), 0,
                                                          kStreamPolicy);
  Chunk c;
  c.u = make_uint4(v.x, v.y, v.z, v.w);
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

// Element m of the D-vector x (storage type) after the rotary position
// embedding at position pos, in float64: dims i and i + D/2 turn together by
// the angle pos * base^(-2i/D) (the embedding of the Llama-family models the
// pages evaluate; they name RoPE without its form).  base == 0 means no
// embedding: the element itself.
// Cosine and sine of the angle of pair i (every caller forms them with this
// one expression, so every kernel embeds identically).
__device__ __forceinline__ void rope_cs(int i, int D, double base, int pos, double& cs,
                                        double& sn) {
  sincos(static_cast<double>(pos) * pow(base, -2.0 * i / D), &sn, &cs);
}

// a = x_m, b = its partner (x_{m+D/2} for m < D/2, else x_{m-D/2}):
// first half x_i cos - x_{i+h} sin, second half x_{i+h} cos + x_i sin.
__device__ __forceinline__ double rope_apply(double a, double b, double cs, double sn, bool first) {
  const double t = b * sn;  // explicit fused forms: the same rounding wherever it is inlined
  return first ? fma(a, cs, -t) : fma(a, cs, t);
}

template <class E>
__device__ __forceinline__ double rope_elem(const typename E::T* x, int m, int D, double base,
                                            int pos) {
  const double a = static_cast<double>(ld_elem<E>(x, m));
  if (base == 0.0) return a;
  const int h = D >> 1;
  const bool first = m < h;
  const double b = static_cast<double>(ld_elem<E>(x, first ? m + h : m - h));
  double cs, sn;
  rope_cs(first ? m : m - h, D, base, pos, cs, sn);
  return rope_apply(a, b, cs, sn, first);
}

// Data-parallel-primitive (DPP) lane moves.  dpp<CTRL, ROW_MASK, BANK_MASK>
// returns, per lane, the value of the lane selected by CTRL within its row of
// 16 lanes; lanes whose source is out of range, or that the masks disable,
// get 0.  Controls used: quad_perm [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E),
// row_shr:n (0x110 + n), row_mirror (0x140), row_half_mirror (0x141),
// row_bcast:15 (0x142), row_bcast:31 (0x143).
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ unsigned dpp_u(unsigned v) {
  return static_cast<unsigned>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, BANK_MASK, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of the group receives the group total.  Within a row of 16 the
// butterfly uses DPP (quad swaps, then half-row and row mirrors, which pair
// each lane with one holding the complementary partial sum); wider groups
// cross rows with lane shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  if (W >= 2) x += dpp_f<0xB1>(x);
  if (W >= 4) x += dpp_f<0x4E>(x);
  if (W >= 8) x += dpp_f<0x141>(x);
  if (W >= 16) x += dpp_f<0x140>(x);
  if (W >= 32) x += __shfl_xor(x, 16, 64);
  if (W >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: prefix within rows of 16
// from shifted copies (shifts 1-3 of the input, then 4 and 8 of the partial
// result on the upper banks), then row totals broadcast to the later rows.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x, int /*lane*/) {
  unsigned v = x;
  v += dpp_u<0x111>(x);
  v += dpp_u<0x112>(x);
  v += dpp_u<0x113>(x);
  v += dpp_u<0x114, 0xf, 0xe>(v);
  v += dpp_u<0x118, 0xf, 0xc>(v);
  v += dpp_u<0x142, 0xa, 0xf>(v);
  v += dpp_u<0x143, 0xc, 0xf>(v);
  return v;
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

// ---- handing data from one workgroup to another within a launch ----------
//
// The XCDs have their own L2 caches, which are not kept coherent with each
// other for ordinary stores and loads.  Data that one workgroup leaves for
// another of the same launch is therefore stored and loaded with device
// scope (the store is written through its L2, the load is served
// coherently), and the hand-over is a device-scope flag set after the
// producer's stores have completed.  No release fence is used: on this chip
// it writes back the whole of the producing XCD's L2.
constexpr int kDevScope = 16;  // cache-policy bits of device-scope buffer accesses

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st16_dev(const Region& g, uint32_t off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, g.r, static_cast<int>(off),
                                         0, kDevScope);
}
__device__ __forceinline__ uint4 ld16_dev(const Region& g, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(g.r, static_cast<int>(off), 0, kDevScope);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Called by every thread of a workgroup after its device-scope stores: once
// they have all completed, sets *flag = value (device scope).
__device__ __forceinline__ void publish(unsigned long long* flag, unsigned long long value) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have been acknowledged
  __syncthreads();                // ... and every other thread's
  if (threadIdx.x == 0)
    __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Longest wait for other workgroups' flags, in polls of about 0.1 us: far
// beyond any launch of this library, so only a workgroup that never ran
// could exhaust it; the waiter then gives up rather than hang.
constexpr int kSpinMax = 1 << 19;

// Called by every thread of a workgroup: waits until flags[0 .. n) (n <= 64)
// all equal `value`.  Returns false in every thread if the wait gave up.
__device__ __forceinline__ bool wait_flags(const unsigned long long* flags, int n,
                                           unsigned long long value) {
  __shared__ int ok;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    bool done = false;
    for (int spins = 0; !done && spins < kSpinMax; ++spins) {
      const unsigned long long f = lane < n ? ld_dev(flags + lane) : value;
      done = __all(f == value);
      if (!done) __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) ok = done ? 1 : 0;
  }
  __syncthreads();
  return ok != 0;
}

// float64 -> bf16 bits, round to nearest, ties to even, done on the bit
// pattern so that there is a single rounding.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 63) << 15;
  const int e = static_cast<int>((u >> 52) & 0x7ffu);
  const uint64_t m = u & ((1ull << 52) - 1);
  if (e == 0x7ff) return static_cast<uint16_t>(sign | 0x7f80u | (m ? 0x40u : 0u));
  if (e == 0) return static_cast<uint16_t>(sign);  // |x| < 2^-1022 rounds to zero
  int E = e - 1023 + 127;                          // bf16 biased exponent
  const uint64_t sig = (1ull << 52) | m;           // 53-bit significand
  int shift = 45;                                  // keep 8 significant bits
  if (E < 1) {                                     // bf16 subnormal range
    shift += 1 - E;
    E = 0;
    if (shift > 54) return static_cast<uint16_t>(sign);
  }
  uint64_t keep = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1ull))) ++keep;
  uint32_t bits = (E == 0) ? static_cast<uint32_t>(keep)
                           : (static_cast<uint32_t>(E) << 7) + static_cast<uint32_t>(keep - 128);
  if (bits >= 0x7f80u) bits = 0x7f80u;  // overflow -> infinity
  return static_cast<uint16_t>(sign | bits);
}

template <class E>
__device__ __forceinline__ typename E::T round_store(double x);

template <>
__device__ __forceinline__ float round_store<F32>(double x) {
  return static_cast<float>(x);  // round to nearest even
}

template <>
__device__ __forceinline__ uint16_t round_store<BF16>(double x) {
  return f64_to_bf16_rne(x);
}

}  // namespace loki
