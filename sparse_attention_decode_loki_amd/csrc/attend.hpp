// Gather + exact attention with an online softmax, shared by the split and
// fused decode kernels and by the dense baseline.
//
// Exact attention runs over the kept tokens only (Loki summary page,
// summary line and "Approach").  Layout of the work: a token row of D
// elements is D*bytes/16 lanes wide (16 lanes for D = 128 bf16), so every
// lane issues one 16-byte load of the key row and one of the value row and a
// 64-wide wave carries 64*VEC/D tokens at a time.  Rows are read straight
// into registers: no row is used twice, so staging through LDS would only
// add latency.  Each lane group keeps its own running max m, running sum l
// and value accumulator (base-2 exponent domain); groups are merged through
// LDS at the end.
#pragma once

#include "device.hpp"

namespace loki {

template <class E, int D, int NT = kBlock>
struct Geo {
  static constexpr int VEC = E::VEC;
  static constexpr int LPV = D / VEC;   // lanes per token row
  static constexpr int NG = NT / LPV;   // token groups of an NT-thread workgroup
  static_assert(LPV >= 1 && LPV <= 64 && (LPV & (LPV - 1)) == 0, "row must map to 2^n lanes");
};

template <int VEC>
struct Acc {
  float m, l;
  float a[VEC];
};

template <int VEC>
__device__ __forceinline__ void acc_init(Acc<VEC>& s) {
  s.m = -INFINITY;
  s.l = 0.f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) s.a[v] = 0.f;
}

// Attend over list positions t in [t0, t1) for NH query heads sharing the
// same tokens.  Group `grp` takes t = t0 + grp + NG*u.
//   get_j(t)      token id at list position t
//   get_s(h, t, j) score over K' dims [0, d) (SPARSE only)
// SPARSE: dims [0, d) of q'.k' come from get_s and only lanes whose dims lie
//   in [d, D) load the key (from k_rest).  DENSE: every lane loads its key
//   chunk from k_slab or k_rest.
// qf[h][v] = q'_h[lane_dim0 + v] (zero where the lane's dims come from get_s).
// Token jo (if >= 0) is not read from the cache: its rotated key row
// [slab | rest] and value row are taken from ko / vo (LDS, storage format).
// NoMask: every head takes every token.  A union list (GQA) passes get_mask(t),
// a bitmask of the heads that kept token t; the other heads skip it.
struct NoMask {
  __device__ __forceinline__ unsigned operator()(int) const { return 0xffffffffu; }
};

template <class E, int D, int NH, bool SPARSE, int U, int NT = kBlock, class GetJ, class GetS,
          class GetMask = NoMask>
__device__ __forceinline__ void attend_loop(GetJ get_j, GetS get_s, int t0, int t1,
                                            const typename E::T* __restrict__ slab,
                                            const typename E::T* __restrict__ rest,
                                            const typename E::T* __restrict__ val, int d,
                                            const float (&qf)[NH][E::VEC], float scale_log2,
                                            Acc<E::VEC> (&st)[NH], int jo = -1,
                                            const typename E::T* ko = nullptr,
                                            const typename E::T* vo = nullptr,
                                            GetMask get_mask = GetMask()) {
  using G = Geo<E, D, NT>;
  constexpr int VEC = G::VEC;
  constexpr int LPV = G::LPV;
  constexpr int NG = G::NG;
  const int r = threadIdx.x % LPV;
  const int grp = threadIdx.x / LPV;
  const int kd0 = r * VEC;
  const int dr = D - d;
  const bool in_rest = kd0 >= d;
  const bool kload = SPARSE ? in_rest : true;
  constexpr uint32_t EB = E::BYTES;
  // regions of this (sequence, KV head): slab, rest and value rows
  const Region gs = make_region(slab, 0x7fffffffu);
  const Region gr = make_region(rest ? rest : slab, 0x7fffffffu);
  const Region gv = make_region(val, 0x7fffffffu);
  const uint32_t srow = static_cast<uint32_t>(d) * EB, rrow = static_cast<uint32_t>(dr) * EB;
  const uint32_t scol = static_cast<uint32_t>(kd0) * EB;
  const uint32_t rcol = static_cast<uint32_t>(in_rest ? kd0 - d : 0) * EB;

  for (int tb = t0 + grp; tb < t1; tb += NG * U) {
    int j[U];
    bool ok[U];
    unsigned hm[U];
    Chunk kc[U], vc[U];
    float sv[NH][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + NG * u;
      ok[u] = t < t1;
      j[u] = ok[u] ? get_j(t) : 0;
      hm[u] = ok[u] ? get_mask(t) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t jj = static_cast<uint32_t>(j[u]);
      kc[u] = zero_chunk();
      vc[u] = zero_chunk();
      if (ok[u]) {
        if (j[u] != jo) {  // separate branches keep each load's address space known
          if (kload) {  // each branch keeps its buffer resource wave-uniform
            if (in_rest)
              kc[u] = ld16_region(gr, jj * rrow + rcol);
            else
              kc[u] = ld16_region(gs, jj * srow + scol);
          }
          vc[u] = ld16_region(gv, jj * static_cast<uint32_t>(D) * EB + kd0 * EB);
        } else {
          if (kload) kc[u] = ld16(ko + kd0);
          vc[u] = ld16(vo + kd0);
        }
      }
    }
    if (SPARSE) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u)
          sv[h][u] = (((hm[u] >> h) & 1u) && r == 0) ? get_s(h, tb + NG * u, j[u]) : 0.f;
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float x[U];
      float mx = st[h].m;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kf[VEC];
        unpack<E>(kc[u], kf);
        float dot = SPARSE ? sv[h][u] : 0.f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot = fmaf(qf[h][v], kf[v], dot);
        dot = group_sum<LPV>(dot);
        x[u] = ((hm[u] >> h) & 1u) ? dot * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[u]);
      }
      const float c = (st[h].m == mx) ? 1.f : fast_exp2(st[h].m - mx);
      st[h].l *= c;
#pragma unroll
      for (int v = 0; v < VEC; ++v) st[h].a[v] *= c;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = ((hm[u] >> h) & 1u) ? fast_exp2(x[u] - mx) : 0.f;
        float vf[VEC];
        unpack<E>(vc[u], vf);
        st[h].l += p;
#pragma unroll
        for (int v = 0; v < VEC; ++v) st[h].a[v] = fmaf(p, vf[v], st[h].a[v]);
      }
      st[h].m = mx;
    }
  }
}

// LDS for merging the NG group states of NH heads.
template <int D, int NH, int NG>
struct MergeSmem {
  float m[NH][NG];
  float l[NH][NG];
  float a[NH][NG][D];
};

// Merge the group states.  Afterwards thread t handles outputs o = t,
// t + NT, ... < NH*D (head o / D, dim o % D) and `fin(h, dim, M, L, A)`
// is called with the merged max M, sum L and accumulator A.
template <class E, int D, int NH, int NT = kBlock, class Fin>
__device__ __forceinline__ void merge_groups(const Acc<E::VEC> (&st)[NH],
                                             MergeSmem<D, NH, Geo<E, D, NT>::NG>& sm, Fin fin) {
  using G = Geo<E, D, NT>;
  constexpr int VEC = G::VEC;
  constexpr int LPV = G::LPV;
  constexpr int NG = G::NG;
  const int r = threadIdx.x % LPV;
  const int grp = threadIdx.x / LPV;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (r == 0) {
      sm.m[h][grp] = st[h].m;
      sm.l[h][grp] = st[h].l;
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) sm.a[h][grp][r * VEC + v] = st[h].a[v];
  }
  __syncthreads();
  // PT threads share one output (groups split PT ways, partial sums added
  // across neighbouring lanes) when the workgroup has that many threads per
  // output; otherwise each output is one thread's loop over all groups.
  constexpr int PT = (NT >= 4 * NH * D && NG % 4 == 0)   ? 4
                     : (NT >= 2 * NH * D && NG % 2 == 0) ? 2
                                                         : 1;
  if constexpr (PT > 1) {
    constexpr int GP = NG / PT;
    const int o = threadIdx.x / PT, part = threadIdx.x % PT;
    if (o < NH * D) {  // NT is a multiple of PT: whole lane quads take part
      const int h = o / D, dim = o % D;
      float M = -INFINITY;
#pragma unroll
      for (int g = 0; g < NG; ++g) M = fmaxf(M, sm.m[h][g]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int i = 0; i < GP; ++i) {
        const int g = part * GP + i;
        const float mg = sm.m[h][g];
        const float w = (mg == -INFINITY) ? 0.f : fast_exp2(mg - M);
        L = fmaf(sm.l[h][g], w, L);
        A = fmaf(sm.a[h][g][dim], w, A);
      }
      L += dpp_f<0xB1>(L);  // lanes 0<->1, 2<->3
      A += dpp_f<0xB1>(A);
      if constexpr (PT == 4) {
        L += dpp_f<0x4E>(L);  // lanes 0<->2, 1<->3
        A += dpp_f<0x4E>(A);
      }
      if (part == 0) fin(h, dim, M, L, A);
    }
  } else {
    for (int o = threadIdx.x; o < NH * D; o += NT) {
      const int h = o / D, dim = o % D;
      float M = -INFINITY;
#pragma unroll
      for (int g = 0; g < NG; ++g) M = fmaxf(M, sm.m[h][g]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float mg = sm.m[h][g];
        const float w = (mg == -INFINITY) ? 0.f : fast_exp2(mg - M);
        L = fmaf(sm.l[h][g], w, L);
        A = fmaf(sm.a[h][g][dim], w, A);
      }
      fin(h, dim, M, L, A);
    }
  }
}

}  // namespace loki
