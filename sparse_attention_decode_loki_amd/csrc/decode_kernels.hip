// gfx950 kernels of the Loki decode step and the dense baseline.
//
// Method (pages titled "Loki: Low-rank Keys for Efficient Sparse Attention":
// AI-extracted summary, summary line and "Approach"; arXiv "Abstract"):
// project the query onto the calibrated PCA basis, score every cached token
// with the leading d rotated dimensions, keep the top k, and run exact
// softmax attention over the kept tokens.  Every stage is bound by HBM
// bandwidth (about 1 flop per byte), so the kernels use the vector ALU with
// wide coalesced loads and no matrix cores.
//
// Kernels:
//   rotate_kernel   q' = q . P[g] for all query heads of one KV head
//   score_kernel    s_j over a chunk of the key slab for up to 4 query heads
//   topk_kernel     exact top-k of one score row, ascending indices
//   attend_kernel   gather + online softmax over a slice of the kept tokens
//                   (also the dense baseline, with all tokens)
//   combine_kernel  log-sum-exp merge of the slices
//   fused_kernel    one workgroup per (sequence, query head) doing all of
//                   the above with the scores and indices held in LDS
#include "launch.hpp"
#include "attend.hpp"
#include "select.hpp"

namespace loki {

// ----------------------------------------------------------------- helpers --

// Workgroup id -> logical id such that consecutive logical ids land on the
// same XCD (workgroups are dealt round-robin over the 8 XCDs), so the
// sequences of one head share that head's basis in one L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
  if ((n & 7) != 0) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

// ------------------------------------------------------------------ rotate --

constexpr int kRotQ = 4;  // queries per rotate workgroup

// Grid (ceil(B*G / kRotQ), Hkv).  Thread t covers columns 4*(t % (D/4)) .. +3
// of P[g] over a block of rows, loaded as 16-byte chunks (each row of P is
// read by D/4 consecutive threads, fully coalesced); partial sums over the
// row blocks are added through LDS.
template <class E, int D>
__global__ void __launch_bounds__(kBlock) rotate_kernel(const typename E::T* __restrict__ q,
                                                        const float* __restrict__ P,
                                                        float* __restrict__ qrot, int B, int Hq,
                                                        int Hkv) {
  constexpr int CQ = D / 4;        // column quads
  constexpr int NRB = kBlock / CQ; // row blocks
  constexpr int RB = D / NRB;      // rows per block
  __shared__ float qsh[kRotQ][D];
  __shared__ float red[NRB][kRotQ][D];
  const int g = blockIdx.y;
  const int G = Hq / Hkv;
  const int n0 = blockIdx.x * kRotQ;
  const int nq = min(kRotQ, B * G - n0);
  const int cq = threadIdx.x % CQ;
  const int rb = threadIdx.x / CQ;

  float4 p[RB];
  const float* Pg = P + static_cast<int64_t>(g) * D * D;
#pragma unroll
  for (int rr = 0; rr < RB; ++rr)
    p[rr] = *reinterpret_cast<const float4*>(Pg + (rb * RB + rr) * D + 4 * cq);

  for (int e = threadIdx.x; e < nq * D; e += kBlock) {
    const int r = e / D, m = e % D;
    const int n = n0 + r, b = n / G, h = g * G + n % G;
    qsh[r][m] = ld_elem<E>(q, (static_cast<int64_t>(b) * Hq + h) * D + m);
  }
  __syncthreads();
  for (int r = 0; r < nq; ++r) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float x = qsh[r][rb * RB + rr];
      acc.x = fmaf(x, p[rr].x, acc.x);
      acc.y = fmaf(x, p[rr].y, acc.y);
      acc.z = fmaf(x, p[rr].z, acc.z);
      acc.w = fmaf(x, p[rr].w, acc.w);
    }
    *reinterpret_cast<float4*>(&red[rb][r][4 * cq]) = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nq * D; e += kBlock) {
    const int r = e / D, c = e % D;
    const int n = n0 + r, b = n / G, h = g * G + n % G;
    float s = 0.f;
#pragma unroll
    for (int pp = 0; pp < NRB; ++pp) s += red[pp][r][c];
    qrot[(static_cast<int64_t>(b) * Hq + h) * D + c] = s;
  }
}

// ------------------------------------------------------------------- score --

// Scores of tokens [j0, j1) for NH heads.  LPS lanes share one token's slab
// row (d*bytes/16 lanes rounded up to a power of two; lanes past the row
// idle); a wave covers 64/LPS consecutive tokens per load, so the slab is
// streamed with fully coalesced 16-byte loads.  score_first issues the first
// batch of loads, which do not depend on the query, so a caller can start
// them before the query is rotated.
template <class E, int LPS, int U>
__device__ __forceinline__ void score_first(const typename E::T* __restrict__ slab, int d, int j0,
                                            int j1, Chunk (&c)[U]) {
  constexpr int VEC = E::VEC;
  constexpr int TPI = kBlock / LPS;
  const int part = threadIdx.x % LPS;
  const int tk = threadIdx.x / LPS;
  const bool active = part * VEC < d;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = j0 + tk + TPI * u;
    c[u] = (active && j < j1) ? ld16(slab + static_cast<int64_t>(j) * d + part * VEC) : zero_chunk();
  }
}

// c holds the first batch (from score_first).
template <class E, int LPS, int NH, int U, class Write>
__device__ __forceinline__ void score_loop(const typename E::T* __restrict__ slab, int d, int j0,
                                           int j1, const float (&qf)[NH][E::VEC], Write write,
                                           Chunk (&c)[U]) {
  constexpr int VEC = E::VEC;
  constexpr int TPI = kBlock / LPS;
  const int part = threadIdx.x % LPS;
  const int tk = threadIdx.x / LPS;
  const bool active = part * VEC < d;
  for (int jb = j0 + tk; jb < j1; jb += TPI * U) {
    if (jb != j0 + tk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jb + TPI * u;
        c[u] = (active && j < j1) ? ld16(slab + static_cast<int64_t>(j) * d + part * VEC)
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

constexpr int kScoreChunk = 1024;  // tokens per score workgroup

template <class E, int LPS, int NH>
__global__ void __launch_bounds__(kBlock) score_kernel(const typename E::T* __restrict__ slab,
                                                       const float* __restrict__ qrot,
                                                       float* __restrict__ scores, int Hq, int Hkv,
                                                       int D, int d, int S, int S_max, int nhb) {
  constexpr int VEC = E::VEC;
  const int G = Hq / Hkv;
  const int bg = blockIdx.x / nhb;
  const int hb = blockIdx.x % nhb;
  const int b = bg / Hkv, g = bg % Hkv;
  const int h0 = g * G + hb * NH;
  const int nh = min(NH, G - hb * NH);
  const int part = threadIdx.x % LPS;
  float qf[NH][VEC];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      qf[h][v] = (h < nh && part * VEC < d)
                     ? qrot[(static_cast<int64_t>(b) * Hq + h0 + h) * D + part * VEC + v]
                     : 0.f;
  const int j0 = blockIdx.y * kScoreChunk;
  const int j1 = min(S, j0 + kScoreChunk);
  const typename E::T* sl = slab + static_cast<int64_t>(bg) * S_max * d;
  float* srow = scores + (static_cast<int64_t>(b) * Hq + h0) * S;
  Chunk c[4];
  score_first<E, LPS, 4>(sl, d, j0, j1, c);
  score_loop<E, LPS, NH, 4>(sl, d, j0, j1, qf, [&](int h, int j, float s) {
    if (h < nh) srow[static_cast<int64_t>(h) * S + j] = s;
  }, c);
}

// -------------------------------------------------------------------- topk --

template <int BLOCK>
__global__ void __launch_bounds__(BLOCK) topk_kernel(const float* __restrict__ scores, int S,
                                                     int64_t ld, int k, int* __restrict__ idx,
                                                     int use_lds) {
  __shared__ SelectSmemAny<BLOCK> sm;
  extern __shared__ float sbuf[];
  const int row = blockIdx.x;
  const float* s = scores + static_cast<int64_t>(row) * ld;
  int* out = idx + static_cast<int64_t>(row) * k;
  auto emit = [&](int p, int j) { out[p] = j; };
  if (use_lds) {
    const int n4 = S >> 2;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    for (int i = threadIdx.x; i < n4; i += BLOCK) reinterpret_cast<float4*>(sbuf)[i] = s4[i];
    for (int i = (n4 << 2) + threadIdx.x; i < S; i += BLOCK) sbuf[i] = s[i];
    __syncthreads();
    block_select_topk_any<BLOCK>([&](int j) { return sbuf[j]; }, S, k, emit, sm);
  } else {
    block_select_topk_any<BLOCK>([&](int j) { return s[j]; }, S, k, emit, sm);
  }
}

// ------------------------------------------------------------------ attend --

constexpr int kAttendStage = 2048;  // max kept tokens per attend workgroup

// Grid (rows, nsplit).  SPARSE: rows = B*Hq, one head per workgroup, tokens
// are slice `split` of the kept list; the slice's ids and scores are staged
// in LDS first.  DENSE: rows = B*Hkv*nhb, NH heads of one KV head per
// workgroup, tokens are slice `split` of 0..S-1.
template <class E, int D, int NH, bool SPARSE>
__global__ void __launch_bounds__(kBlock) attend_kernel(
    const typename E::T* __restrict__ slab, const typename E::T* __restrict__ rest,
    const typename E::T* __restrict__ val, const float* __restrict__ qrot,
    const float* __restrict__ scores, const int* __restrict__ idx, float* __restrict__ part,
    float* __restrict__ out, int Hq, int Hkv, int d, int S, int S_max, int kk, int nsplit,
    int nhb, float scale_log2) {
  using Gm = Geo<E, D>;
  constexpr int VEC = Gm::VEC;
  constexpr int LPV = Gm::LPV;
  __shared__ MergeSmem<D, NH, Gm::NG> msm;
  __shared__ int jst[SPARSE ? kAttendStage : 1];
  __shared__ float sst[SPARSE ? kAttendStage : 1];

  const int G = Hq / Hkv;
  const int split = blockIdx.y;
  int b, g, h0, nh;
  if (SPARSE) {
    const int row = blockIdx.x;  // b*Hq + h
    b = row / Hq;
    h0 = row % Hq;
    g = h0 / G;
    nh = 1;
  } else {
    const int bg = blockIdx.x / nhb;
    const int hb = blockIdx.x % nhb;
    b = bg / Hkv;
    g = bg % Hkv;
    h0 = g * G + hb * NH;
    nh = min(NH, G - hb * NH);
  }
  const int total = SPARSE ? kk : S;
  const int per = (total + nsplit - 1) / nsplit;
  const int t0 = split * per;
  const int t1 = min(total, t0 + per);

  const int64_t bgo = static_cast<int64_t>(b) * Hkv + g;
  const typename E::T* sl = slab + bgo * S_max * d;
  const typename E::T* rs = rest ? rest + bgo * S_max * (D - d) : nullptr;
  const typename E::T* vv = val + bgo * S_max * D;

  const int r = threadIdx.x % LPV;
  const int kd0 = r * VEC;
  float qf[NH][VEC];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const bool use = (h < nh) && (!SPARSE || kd0 >= d);
      qf[h][v] = use ? qrot[(static_cast<int64_t>(b) * Hq + h0 + h) * D + kd0 + v] : 0.f;
    }

  Acc<VEC> st[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) acc_init(st[h]);

  if (SPARSE) {
    const int* irow = idx + (static_cast<int64_t>(b) * Hq + h0) * kk;
    const float* srow = scores + (static_cast<int64_t>(b) * Hq + h0) * S;
    for (int t = t0 + threadIdx.x; t < t1; t += kBlock) {
      // ids may come from the caller: keep every read inside the cache
      const int j = min(max(irow[t], 0), S - 1);
      jst[t - t0] = j;
      sst[t - t0] = srow[j];
    }
    __syncthreads();
    attend_loop<E, D, NH, true, 4>([&](int t) { return jst[t - t0]; },
                                   [&](int, int t, int) { return sst[t - t0]; }, t0, t1, sl, rs,
                                   vv, d, qf, scale_log2, st);
  } else {
    attend_loop<E, D, NH, false, 4>([&](int t) { return t; }, [&](int, int, int) { return 0.f; },
                                    t0, t1, sl, rs, vv, d, qf, scale_log2, st);
  }

  merge_groups<E, D, NH>(st, msm, [&](int h, int dim, float M, float L, float A) {
    if (h >= nh) return;
    const int64_t row = static_cast<int64_t>(b) * Hq + h0 + h;
    if (nsplit == 1) {
      out[row * D + dim] = A / L;
    } else {
      float* pp = part + (row * nsplit + split) * (D + 2);
      pp[dim] = A;
      if (dim == 0) {
        pp[D] = M;
        pp[D + 1] = L;
      }
    }
  });
}

template <int D>
__global__ void __launch_bounds__(128) combine_kernel(const float* __restrict__ part,
                                                     float* __restrict__ out, int nsplit) {
  const int64_t row = blockIdx.x;
  const float* pr = part + row * nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pr[s * (D + 2) + D]);
  for (int dim = threadIdx.x; dim < D; dim += 128) {
    float L = 0.f, A = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = pr[s * (D + 2) + D];
      const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
      L = fmaf(pr[s * (D + 2) + D + 1], w, L);
      A = fmaf(pr[s * (D + 2) + dim], w, A);
    }
    out[row * D + dim] = A / L;
  }
}

// ------------------------------------------------------------------- fused --

// One workgroup per (sequence, query head): rotate the query, score the
// whole slab into LDS, select the top k in LDS, then gather and attend.
// Dynamic LDS: q' [D] | scores [S] | kept ids [kk].
// SMALL: S <= 16 * kBlock, so the selection keeps 16 keys per thread.
template <class E, int D, int LPS, bool SMALL>
__global__ void __launch_bounds__(kBlock) fused_kernel(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ slab,
    const typename E::T* __restrict__ rest, const typename E::T* __restrict__ val,
    const float* __restrict__ P, float* __restrict__ out, int* __restrict__ idx, int B, int Hq,
    int Hkv, int d, int S, int S_max, int kk, float scale_log2) {
  using Gm = Geo<E, D>;
  constexpr int VEC = E::VEC;
  constexpr int CQ = D / 4;          // column quads of P
  constexpr int NRB = kBlock / CQ;   // row blocks of P
  constexpr int RB = D / NRB;        // rows per block
  constexpr int US = 8;              // slab loads in flight per lane
  union Scratch {
    SelectSmemAny<kBlock> sel;
    MergeSmem<D, 1, Gm::NG> mrg;
    float rot[NRB][D];
  };
  __shared__ Scratch sc;
  extern __shared__ float dyn[];
  float* qs = dyn;
  float* sb = dyn + D;
  int* ib = reinterpret_cast<int*>(dyn + D + S);

  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int h = L / B, b = L % B;
  const int G = Hq / Hkv;
  const int g = h / G;
  const int64_t row = static_cast<int64_t>(b) * Hq + h;
  const int64_t bgo = static_cast<int64_t>(b) * Hkv + g;
  const typename E::T* sl = slab + bgo * S_max * d;

  // 0. the first slab loads do not depend on q': start them now
  Chunk c[US];
  score_first<E, LPS, US>(sl, d, 0, S, c);

  // 1. q' = q . P[g]: thread (cq, rb) adds rows [rb*RB, rb*RB + RB) for
  //    columns 4*cq .. 4*cq + 3, read as 16-byte chunks
  {
    const int cq = threadIdx.x % CQ, rb = threadIdx.x / CQ;
    const float* Pg = P + static_cast<int64_t>(g) * D * D;
    const typename E::T* qr = q + row * D;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int m = rb * RB + rr;
      const float x = ld_elem<E>(qr, m);
      const float4 p = *reinterpret_cast<const float4*>(Pg + m * D + 4 * cq);
      acc.x = fmaf(x, p.x, acc.x);
      acc.y = fmaf(x, p.y, acc.y);
      acc.z = fmaf(x, p.z, acc.z);
      acc.w = fmaf(x, p.w, acc.w);
    }
    *reinterpret_cast<float4*>(&sc.rot[rb][4 * cq]) = acc;
    __syncthreads();
    if (threadIdx.x < D) {
      float s = 0.f;
#pragma unroll
      for (int pp = 0; pp < NRB; ++pp) s += sc.rot[pp][threadIdx.x];
      qs[threadIdx.x] = s;
    }
    __syncthreads();
  }

  // 2. ranking scores of all S tokens -> LDS
  {
    const int part = threadIdx.x % LPS;
    float qf[1][VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) qf[0][v] = (part * VEC < d) ? qs[part * VEC + v] : 0.f;
    score_loop<E, LPS, 1, US>(sl, d, 0, S, qf, [&](int, int j, float s) { sb[j] = s; }, c);
  }
  __syncthreads();

  // 3. top-k -> LDS and the idx output
  {
    int* irow = idx + row * kk;
    auto emit = [&](int p, int j) {
      ib[p] = j;
      irow[p] = j;
    };
    if (SMALL)
      block_select_topk_reg<kBlock, 16>([&](int j) { return sb[j]; }, S, kk, emit, sc.sel.reg);
    else
      block_select_topk_any<kBlock>([&](int j) { return sb[j]; }, S, kk, emit, sc.sel);
  }
  __syncthreads();

  // 4. gather + exact attention over the kept tokens
  const int r = threadIdx.x % Gm::LPV;
  const int kd0 = r * VEC;
  float qf[1][VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) qf[0][v] = (kd0 >= d) ? qs[kd0 + v] : 0.f;
  Acc<VEC> st[1];
  acc_init(st[0]);
  const typename E::T* rs = rest ? rest + bgo * S_max * (D - d) : nullptr;
  attend_loop<E, D, 1, true, 4>([&](int t) { return ib[t]; },
                                [&](int, int, int j) { return sb[j]; }, 0, kk, sl, rs,
                                val + bgo * S_max * D, d, qf, scale_log2, st);
  __syncthreads();  // the merge scratch aliases the selection scratch
  merge_groups<E, D, 1>(st, sc.mrg, [&](int, int dim, float, float Ls, float A) {
    out[row * D + dim] = A / Ls;
  });
}

// --------------------------------------------------------------- launchers --

namespace {

template <class E>
const typename E::T* cptr(const void* p) {
  return static_cast<const typename E::T*>(p);
}

int lps_for(int d, int vec) {
  int n = (d + vec - 1) / vec, p = 1;
  while (p < n) p <<= 1;
  return p;
}

template <class E, int D>
hipError_t rotate_t(const DecodeArgs& a, float* qrot) {
  const int G = a.Hq / a.Hkv;
  dim3 grid((a.B * G + kRotQ - 1) / kRotQ, a.Hkv);
  hipLaunchKernelGGL((rotate_kernel<E, D>), grid, dim3(kBlock), 0, a.stream, cptr<E>(a.q), a.P,
                     qrot, a.B, a.Hq, a.Hkv);
  return hipGetLastError();
}

template <class E, int LPS>
hipError_t score_t(const DecodeArgs& a, const float* qrot, float* scores) {
  const int G = a.Hq / a.Hkv;
  const int nh = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
  const int nhb = (G + nh - 1) / nh;
  dim3 grid(a.B * a.Hkv * nhb, (a.S + kScoreChunk - 1) / kScoreChunk);
  const auto* sl = cptr<E>(a.k_slab);
  if (nh == 4)
    hipLaunchKernelGGL((score_kernel<E, LPS, 4>), grid, dim3(kBlock), 0, a.stream, sl, qrot, scores,
                       a.Hq, a.Hkv, a.D, a.d, a.S, a.S_max, nhb);
  else if (nh == 2)
    hipLaunchKernelGGL((score_kernel<E, LPS, 2>), grid, dim3(kBlock), 0, a.stream, sl, qrot, scores,
                       a.Hq, a.Hkv, a.D, a.d, a.S, a.S_max, nhb);
  else
    hipLaunchKernelGGL((score_kernel<E, LPS, 1>), grid, dim3(kBlock), 0, a.stream, sl, qrot, scores,
                       a.Hq, a.Hkv, a.D, a.d, a.S, a.S_max, nhb);
  return hipGetLastError();
}

template <class E>
hipError_t score_lps(const DecodeArgs& a, const float* qrot, float* scores) {
  switch (lps_for(a.d, E::VEC)) {
    case 1: return score_t<E, 1>(a, qrot, scores);
    case 2: return score_t<E, 2>(a, qrot, scores);
    case 4: return score_t<E, 4>(a, qrot, scores);
    case 8: return score_t<E, 8>(a, qrot, scores);
    case 16: return score_t<E, 16>(a, qrot, scores);
    default: return score_t<E, 32>(a, qrot, scores);
  }
}

template <class E, int D, bool SPARSE>
hipError_t attend_t(const DecodeArgs& a, const float* qrot, const float* scores, const int* idx,
                    int kk, float* part, int nsplit) {
  const float scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
  const auto* sl = cptr<E>(a.k_slab);
  const auto* rs = cptr<E>(a.k_rest);
  const auto* vv = cptr<E>(a.v);
  if (SPARSE) {
    dim3 grid(a.B * a.Hq, nsplit);
    hipLaunchKernelGGL((attend_kernel<E, D, 1, true>), grid, dim3(kBlock), 0, a.stream, sl, rs, vv,
                       qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk, nsplit,
                       1, scale_log2);
  } else {
    const int G = a.Hq / a.Hkv;
    const int nh = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
    const int nhb = (G + nh - 1) / nh;
    dim3 grid(a.B * a.Hkv * nhb, nsplit);
    if (nh == 4)
      hipLaunchKernelGGL((attend_kernel<E, D, 4, false>), grid, dim3(kBlock), 0, a.stream, sl, rs,
                         vv, qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk,
                         nsplit, nhb, scale_log2);
    else if (nh == 2)
      hipLaunchKernelGGL((attend_kernel<E, D, 2, false>), grid, dim3(kBlock), 0, a.stream, sl, rs,
                         vv, qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk,
                         nsplit, nhb, scale_log2);
    else
      hipLaunchKernelGGL((attend_kernel<E, D, 1, false>), grid, dim3(kBlock), 0, a.stream, sl, rs,
                         vv, qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk,
                         nsplit, nhb, scale_log2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(a.B * a.Hq), dim3(128), 0, a.stream, part, a.out,
                     nsplit);
  return hipGetLastError();
}

template <class E, int D, int LPS>
hipError_t fused_t(const DecodeArgs& a, int kk, size_t lds) {
  const float scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
  if (a.S <= 16 * kBlock)
    hipLaunchKernelGGL((fused_kernel<E, D, LPS, true>), dim3(a.B * a.Hq), dim3(kBlock), lds,
                       a.stream, cptr<E>(a.q), cptr<E>(a.k_slab), cptr<E>(a.k_rest), cptr<E>(a.v),
                       a.P, a.out, a.idx, a.B, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk, scale_log2);
  else
    hipLaunchKernelGGL((fused_kernel<E, D, LPS, false>), dim3(a.B * a.Hq), dim3(kBlock), lds,
                       a.stream, cptr<E>(a.q), cptr<E>(a.k_slab), cptr<E>(a.k_rest), cptr<E>(a.v),
                       a.P, a.out, a.idx, a.B, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk, scale_log2);
  return hipGetLastError();
}

template <class E, int D>
hipError_t fused_lps(const DecodeArgs& a, int kk, size_t lds) {
  switch (lps_for(a.d, E::VEC)) {
    case 1: return fused_t<E, D, 1>(a, kk, lds);
    case 2: return fused_t<E, D, 2>(a, kk, lds);
    case 4: return fused_t<E, D, 4>(a, kk, lds);
    case 8: return fused_t<E, D, 8>(a, kk, lds);
    case 16: return fused_t<E, D, 16>(a, kk, lds);
    default: return fused_t<E, D, 32>(a, kk, lds);
  }
}

}  // namespace

hipError_t launch_rotate(const DecodeArgs& a, float* qrot) {
  if (a.dtype == kF32) return a.D == 64 ? rotate_t<F32, 64>(a, qrot) : rotate_t<F32, 128>(a, qrot);
  return a.D == 64 ? rotate_t<BF16, 64>(a, qrot) : rotate_t<BF16, 128>(a, qrot);
}

hipError_t launch_scores(const DecodeArgs& a, const float* qrot, float* scores) {
  return a.dtype == kF32 ? score_lps<F32>(a, qrot, scores) : score_lps<BF16>(a, qrot, scores);
}

int topk_block_for(int S) { return S <= 4096 ? 256 : (S <= 8192 ? 512 : 1024); }

hipError_t launch_topk(const float* scores, int rows, int S, int64_t ld, int k, int* idx,
                       hipStream_t stream) {
  const int blk = topk_block_for(S);
  const size_t lds_bytes = static_cast<size_t>(S) * sizeof(float);
  const int use_lds = (lds_bytes <= kTopkLdsMax) && (ld % 4 == 0) ? 1 : 0;
  const size_t dyn = use_lds ? lds_bytes : 0;
  if (blk == 256)
    hipLaunchKernelGGL((topk_kernel<256>), dim3(rows), dim3(256), dyn, stream, scores, S, ld, k, idx,
                       use_lds);
  else if (blk == 512)
    hipLaunchKernelGGL((topk_kernel<512>), dim3(rows), dim3(512), dyn, stream, scores, S, ld, k, idx,
                       use_lds);
  else
    hipLaunchKernelGGL((topk_kernel<1024>), dim3(rows), dim3(1024), dyn, stream, scores, S, ld, k,
                       idx, use_lds);
  return hipGetLastError();
}

hipError_t launch_attend(const DecodeArgs& a, const float* qrot, const float* scores,
                         const int* idx, int kk, float* part, int nsplit, bool sparse) {
  if (a.dtype == kF32) {
    if (a.D == 64)
      return sparse ? attend_t<F32, 64, true>(a, qrot, scores, idx, kk, part, nsplit)
                    : attend_t<F32, 64, false>(a, qrot, scores, idx, kk, part, nsplit);
    return sparse ? attend_t<F32, 128, true>(a, qrot, scores, idx, kk, part, nsplit)
                  : attend_t<F32, 128, false>(a, qrot, scores, idx, kk, part, nsplit);
  }
  if (a.D == 64)
    return sparse ? attend_t<BF16, 64, true>(a, qrot, scores, idx, kk, part, nsplit)
                  : attend_t<BF16, 64, false>(a, qrot, scores, idx, kk, part, nsplit);
  return sparse ? attend_t<BF16, 128, true>(a, qrot, scores, idx, kk, part, nsplit)
                : attend_t<BF16, 128, false>(a, qrot, scores, idx, kk, part, nsplit);
}

size_t fused_lds_bytes(int D, int S, int kk) {
  return (static_cast<size_t>(D) + S + kk) * sizeof(float);
}

hipError_t launch_fused(const DecodeArgs& a, int kk) {
  const size_t lds = fused_lds_bytes(a.D, a.S, kk);
  if (a.dtype == kF32) return a.D == 64 ? fused_lps<F32, 64>(a, kk, lds) : fused_lps<F32, 128>(a, kk, lds);
  return a.D == 64 ? fused_lps<BF16, 64>(a, kk, lds) : fused_lps<BF16, 128>(a, kk, lds);
}

}  // namespace loki
