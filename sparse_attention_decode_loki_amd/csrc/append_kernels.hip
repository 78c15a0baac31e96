// Cache append: rotate new keys into the PCA basis and store them split into
// the leading-d slab and the rest; copy values unchanged.  Keys and queries
// are both PCA-projected and no cache entry is ever deleted (pages titled
// "Loki: Low-rank Keys for Efficient Sparse Attention", summary page,
// "Approach").
//
// The rotation is accumulated in float64 (128 FMAs per output element) and
// rounded once to the cache type, so the stored key is the correctly rounded
// value of x . P; append is off the decode path and float64 FMA throughput is
// ample for it.
#include "device.hpp"
#include "launch.hpp"

namespace loki {

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

constexpr int kAppendTok = 32;  // tokens per append workgroup

// Grid (B * Hkv, ceil(T / kAppendTok)).  Each thread keeps one column of
// P[g] in registers; the workgroup's new keys are staged in LDS as float32
// [kAppendTok][D] (exact for both types) and read as broadcasts.
template <class E, int D>
__global__ void __launch_bounds__(kBlock) append_kernel(
    const typename E::T* __restrict__ k_new, const typename E::T* __restrict__ v_new,
    const float* __restrict__ P, typename E::T* __restrict__ slab, typename E::T* __restrict__ rest,
    typename E::T* __restrict__ val, int Hkv, int d, int S_max, int pos, int T) {
  __shared__ float ks[kAppendTok * D];
  const int bg = blockIdx.x;
  const int g = bg % Hkv;
  const int t0 = blockIdx.y * kAppendTok;
  const int nt = min(kAppendTok, T - t0);
  constexpr int NP = kBlock / D;  // tokens rotated at once
  const int col = threadIdx.x % D;
  const int sub = threadIdx.x / D;
  const int dr = D - d;

  float pc[D];  // column `col` of P[g]
  const float* Pg = P + static_cast<int64_t>(g) * D * D;
#pragma unroll
  for (int m = 0; m < D; ++m) pc[m] = Pg[m * D + col];
  const int64_t in0 = (static_cast<int64_t>(bg) * T + t0) * D;
  for (int i = threadIdx.x; i < nt * D; i += kBlock) ks[i] = ld_elem<E>(k_new, in0 + i);
  __syncthreads();

  for (int tt = sub; tt < nt; tt += NP) {
    double acc = 0.0;
#pragma unroll
    for (int m = 0; m < D; ++m)
      acc = fma(static_cast<double>(ks[tt * D + m]), static_cast<double>(pc[m]), acc);
    const int64_t slot = static_cast<int64_t>(bg) * S_max + pos + t0 + tt;
    if (col < d)
      slab[slot * d + col] = round_store<E>(acc);
    else
      rest[slot * dr + (col - d)] = round_store<E>(acc);
  }
  for (int i = threadIdx.x; i < nt * D; i += kBlock) {
    const int tt = i / D, c = i % D;
    const int64_t slot = static_cast<int64_t>(bg) * S_max + pos + t0 + tt;
    val[slot * D + c] = v_new[in0 + i];
  }
}

namespace {
template <class E, int D>
hipError_t append_t(const void* k_new, const void* v_new, const float* P, void* k_slab,
                    void* k_rest, void* v, int B, int Hkv, int d, int S_max, int pos, int T,
                    hipStream_t stream) {
  using T_ = typename E::T;
  dim3 grid(B * Hkv, (T + kAppendTok - 1) / kAppendTok);
  hipLaunchKernelGGL((append_kernel<E, D>), grid, dim3(kBlock), 0, stream,
                     static_cast<const T_*>(k_new), static_cast<const T_*>(v_new), P,
                     static_cast<T_*>(k_slab), static_cast<T_*>(k_rest), static_cast<T_*>(v), Hkv,
                     d, S_max, pos, T);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_append(const void* k_new, const void* v_new, const float* P, void* k_slab,
                         void* k_rest, void* v, int B, int Hkv, int D, int d, int S_max, int pos,
                         int T, int dtype, hipStream_t stream) {
  if (dtype == kF32)
    return D == 64 ? append_t<F32, 64>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos, T, stream)
                   : append_t<F32, 128>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos, T, stream);
  return D == 64 ? append_t<BF16, 64>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos, T, stream)
                 : append_t<BF16, 128>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos, T, stream);
}

}  // namespace loki
