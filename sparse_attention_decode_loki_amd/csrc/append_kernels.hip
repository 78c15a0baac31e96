// Cache append: rotate new keys into the PCA basis and store them split into
// the leading-d slab and the rest; copy values unchanged.  Keys and queries
// are both PCA-projected and no cache entry is ever deleted (pages titled
// "Loki: Low-rank Keys for Efficient Sparse Attention", summary page,
// "Approach").
//
// The rotation is accumulated in float64 (128 FMAs per output element) and
// rounded once to the cache type, so the stored key is the correctly rounded
// value of x . P; append is off the decode path and float64 FMA throughput is
// ample for it.  The RoPE variant first embeds each key at its slot's
// position, also in float64.
#include "device.hpp"
#include "launch.hpp"

namespace loki {

constexpr int kAppendTok = 8;  // tokens rotated per pass of a workgroup

// Grid (nblk, Hkv).  Workgroup (x, g) rotates the tokens of KV head g of every
// sequence, flattened as n = b * T + t, in chunks of kAppendTok: chunk x,
// x + nblk, ...  Thread (col, part) keeps rows [part*D/NP, (part+1)*D/NP) of
// column `col` of P[g] in registers (loaded once per workgroup) and
// accumulates one float64 partial per token of the chunk (independent
// chains); the NP partials of each output are then added in a fixed order.
template <class E, int D>
__global__ void __launch_bounds__(kBlock) append_kernel(
    const typename E::T* __restrict__ k_new, const typename E::T* __restrict__ v_new,
    const float* __restrict__ P, typename E::T* __restrict__ slab, typename E::T* __restrict__ rest,
    typename E::T* __restrict__ val, int B, int Hkv, int d, int S_max, int pos, int T,
    double rope_base) {
  constexpr int NP = kBlock / D;  // partial sums per output
  constexpr int R = D / NP;       // rows of P per partial
  __shared__ double ks[kAppendTok][D];  // the chunk's keys (embedded when rope_base > 0)
  __shared__ double red[NP][kAppendTok][D];
  const int g = blockIdx.y;
  const int col = threadIdx.x % D;
  const int part = threadIdx.x / D;
  const int dr = D - d;
  const int ntok = B * T;

  float pc[R];
  const float* Pg = P + static_cast<int64_t>(g) * D * D;
#pragma unroll
  for (int r = 0; r < R; ++r) pc[r] = Pg[(part * R + r) * D + col];

  for (int n0 = blockIdx.x * kAppendTok; n0 < ntok; n0 += gridDim.x * kAppendTok) {
    const int nt = min(kAppendTok, ntok - n0);
    for (int i = threadIdx.x; i < kAppendTok * D; i += kBlock) {
      const int tt = i / D, c = i % D;
      double x = 0.0;
      if (tt < nt) {
        const int n = n0 + tt, b = n / T, t = n % T;
        x = rope_elem<E>(k_new + ((static_cast<int64_t>(b) * Hkv + g) * T + t) * D, c, D,
                         rope_base, pos + t);
      }
      ks[tt][c] = x;
    }
    __syncthreads();
    double acc[kAppendTok];
#pragma unroll
    for (int tt = 0; tt < kAppendTok; ++tt) acc[tt] = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const double pv = static_cast<double>(pc[r]);
#pragma unroll
      for (int tt = 0; tt < kAppendTok; ++tt)
        acc[tt] = fma(ks[tt][part * R + r], pv, acc[tt]);
    }
#pragma unroll
    for (int tt = 0; tt < kAppendTok; ++tt) red[part][tt][col] = acc[tt];
    __syncthreads();
    for (int i = threadIdx.x; i < nt * D; i += kBlock) {
      const int tt = i / D, c = i % D;
      double x = 0.0;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) x += red[pp][tt][c];
      const int n = n0 + tt, b = n / T, t = n % T;
      const int64_t slot = (static_cast<int64_t>(b) * Hkv + g) * S_max + pos + t;
      if (c < d)
        slab[slot * d + c] = round_store<E>(x);
      else
        rest[slot * dr + (c - d)] = round_store<E>(x);
      val[slot * D + c] = v_new[((static_cast<int64_t>(b) * Hkv + g) * T + t) * D + c];
    }
    __syncthreads();  // ks and red are rewritten by the next chunk
  }
}

namespace {
template <class E, int D>
hipError_t append_t(const void* k_new, const void* v_new, const float* P, void* k_slab,
                    void* k_rest, void* v, int B, int Hkv, int d, int S_max, int pos, int T,
                    hipStream_t stream, double rope_base) {
  using T_ = typename E::T;
  const int64_t chunks = (static_cast<int64_t>(B) * T + kAppendTok - 1) / kAppendTok;
  // enough workgroups to fill the chip, each reusing its basis column over
  // several chunks
  const int64_t want = (1024 + Hkv - 1) / Hkv;
  const int nblk = static_cast<int>(chunks < want ? chunks : want);
  dim3 grid(nblk, Hkv);
  hipLaunchKernelGGL((append_kernel<E, D>), grid, dim3(kBlock), 0, stream,
                     static_cast<const T_*>(k_new), static_cast<const T_*>(v_new), P,
                     static_cast<T_*>(k_slab), static_cast<T_*>(k_rest), static_cast<T_*>(v), B,
                     Hkv, d, S_max, pos, T, rope_base);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_append(const void* k_new, const void* v_new, const float* P, void* k_slab,
                         void* k_rest, void* v, int B, int Hkv, int D, int d, int S_max, int pos,
                         int T, int dtype, hipStream_t stream, double rope_base) {
  if (dtype == kF32)
    return D == 64 ? append_t<F32, 64>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos,
                                       T, stream, rope_base)
                   : append_t<F32, 128>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos,
                                        T, stream, rope_base);
  return D == 64 ? append_t<BF16, 64>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos, T,
                                      stream, rope_base)
                 : append_t<BF16, 128>(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, d, S_max, pos,
                                       T, stream, rope_base);
}

}  // namespace loki
