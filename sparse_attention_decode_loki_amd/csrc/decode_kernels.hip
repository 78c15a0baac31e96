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
// The single-kernel path (fused_kernel) is in fused_kernels.hip.
#include "launch.hpp"
#include "attend.hpp"
#include "score.hpp"
#include "select.hpp"

namespace loki {

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

}  // namespace loki
