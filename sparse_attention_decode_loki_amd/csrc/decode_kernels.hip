// gfx950 kernels of the Loki decode step and the dense baseline.
//
// Method (pages titled "Loki: Low-rank Keys for Efficient Sparse Attention":
// AI-extracted summary, summary line and "Approach"; arXiv "Abstract"):
// project the query onto the calibrated PCA basis, score every cached token
// with the leading d rotated dimensions, keep the top k, and run exact
// softmax attention over the kept tokens.  Every stage is bound by HBM
// bandwidth (about 1 flop per byte), so the kernels use wide coalesced loads
// and the vector ALU; only where G query heads share each loaded row (the
// grouped-query union gather and dense baseline) would the G heads' products
// saturate the vector ALU, and there they run as small MFMA tiles.
//
// Kernels:
//   rotate_kernel   q' = q . P[g] for all query heads of one KV head (dense
//                   baseline)
//   score_kernel    q' and s_j over a chunk of the key slab for up to 4 query
//                   heads; chunk 0 also stores q' for the attention kernels
//   topk_kernel     exact top-k of one score row, ascending indices (and the
//                   kept-position bitmap for the union gather)
//   attend_kernel   gather + online softmax over a slice of the kept tokens
//                   (also the dense baseline, with all tokens)
//   attend_union_kernel  the grouped-query variant: the union of the G query
//                   heads' kept tokens is gathered once per KV head (VALU)
//   attend_union_mfma_kernel  the same on the matrix cores for bf16 caches;
//                   also the grouped-query dense baseline
//   combine_kernel  log-sum-exp merge of the slices
// The single-kernel path (fused_kernel) is in fused_kernels.hip.
#include <type_traits>

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
                                                        int Hkv, Rope rope) {
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
    qsh[r][m] = static_cast<float>(
        rope_elem<E>(q + (static_cast<int64_t>(b) * Hq + h) * D, m, D, rope.base, rope.pos));
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

// Tokens per score workgroup: the largest of 1024, 512, 256 that still gives
// about four workgroups per CU (the rotation at the start of each workgroup
// is amortised over its chunk).
constexpr int kScoreChunkMax = 1024;

int score_chunk(int units, int S) {
  for (int c = kScoreChunkMax; c > 256; c >>= 1)
    if (static_cast<int64_t>(units) * ((S + c - 1) / c) >= 1024) return c;
  return 256;
}

// Grid (B*Hkv*nhb, ceil(S / chunk)).  Workgroup (bg*nhb + hb, i) scores
// tokens [i*chunk, i*chunk + chunk) for the NH query heads
// hb*NH.. of KV head g.  The queries are rotated here: the slab loads are
// issued first, then q' = q . P[g] is formed exactly as rotate_kernel and the
// fused kernel form it (thread (cq, rb) adds rows [rb*RB, rb*RB + RB) of
// columns 4*cq .. +3 in order, then the NRB partials are added in order), so
// every path ranks with the same float32 q'.  Chunk-0 workgroups form all D
// columns and store q' for the attention kernel; the others form only the d
// columns that ranking needs.
template <int D, int NH>
struct ScoreSmem {
  static constexpr int NRB = kBlock / (D / 4);  // row blocks of P
  float qin[NH][D];
  float red[NRB][NH][D];
  float qr[NH][D];
  // this chunk's scores; the pad puts the heads of one token in different banks
  __align__(16) float ssc[NH][kScoreChunkMax + 16];
};

// Unit `unit` (= (b*Hkv + g)*nhb + hb) and chunk `ci` of the ranking pass.
// With `flag` the chunk's scores are published to top-k workgroups of the
// same launch: stored with device scope, then, once they have completed,
// `flag` is set to `fval`.
template <class E, int D, int LPS, int NH>
__device__ __forceinline__ void score_role(const typename E::T* __restrict__ slab,
                                           const typename E::T* __restrict__ q,
                                           const float* __restrict__ P, float* __restrict__ qrot,
                                           float* __restrict__ scores, int Hq, int Hkv, int d,
                                           int S, int S_max, int nhb, int chunk, Rope rope,
                                           int unit, int ci, ScoreSmem<D, NH>& sm,
                                           unsigned long long* flag, unsigned long long fval) {
  constexpr int VEC = E::VEC;
  constexpr int CQ = D / 4;         // column quads of P
  constexpr int NRB = kBlock / CQ;  // row blocks of P
  constexpr int RB = D / NRB;       // rows per block
  auto& qin = sm.qin;
  auto& red = sm.red;
  auto& qr = sm.qr;
  auto& ssc = sm.ssc;
  const int G = Hq / Hkv;
  const int bg = unit / nhb;
  const int hb = unit % nhb;
  const int b = bg / Hkv, g = bg % Hkv;
  const int h0 = g * G + hb * NH;
  const int nh = min(NH, G - hb * NH);
  const int j0 = ci * chunk;
  const int j1 = min(S, j0 + chunk);
  const typename E::T* sl = slab + static_cast<int64_t>(bg) * S_max * d;

  // Loads are issued in the order they are needed: the query elements, (with
  // one head per workgroup) this thread's rows of P, then the first slab
  // batch.  One in-order counter covers every load, so waiting for the query
  // or the basis then does not also wait for the slab (the 7B shape's ranking
  // pass: 5.0 -> 4.6 us).  With 2-4 heads the basis rows are read in the
  // rotation loop: held across the slab loads they would cost the registers
  // of the fourth workgroup per CU.
  constexpr bool kEarly = NH == 1;
  constexpr int QPT = (NH * D + kBlock - 1) / kBlock;  // query elements per thread
  constexpr int H2 = D / 2;
  const int ncols = ci == 0 ? D : d;
  const int cq = threadIdx.x % CQ, rb = threadIdx.x / CQ;
  const bool rot = 4 * cq < ncols;
  const float* Pg = P + static_cast<int64_t>(g) * D * D;
  float qa[QPT], qb[QPT];  // element m and its rotary partner m +- D/2
  auto load_q = [&]() {
#pragma unroll
    for (int t = 0; t < QPT; ++t) {
      const int e = threadIdx.x + t * kBlock;
      const int h = e / D, m = e % D;
      qa[t] = qb[t] = 0.f;
      if (e < NH * D && h < nh) {
        const typename E::T* qv = q + (static_cast<int64_t>(b) * Hq + h0 + h) * D;
        qa[t] = ld_elem<E>(qv, m);
        if (rope.base != 0.0) qb[t] = ld_elem<E>(qv, m < H2 ? m + H2 : m - H2);
      }
    }
  };
  float4 pv[kEarly ? RB : 1];
  Chunk c[4];
  load_q();
  if constexpr (kEarly) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
      pv[rr] = rot ? *reinterpret_cast<const float4*>(Pg + (rb * RB + rr) * D + 4 * cq)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  score_first<E, LPS, 4>(sl, d, j0, j1, c);
#pragma unroll
  for (int t = 0; t < QPT; ++t) {
    const int e = threadIdx.x + t * kBlock;
    if (e < NH * D) {
      const int h = e / D, m = e % D;
      float x = qa[t];
      if (rope.base != 0.0 && h < nh) {
        double cs, sn;
        rope_cs(m < H2 ? m : m - H2, D, rope.base, rope.pos, cs, sn);
        x = static_cast<float>(rope_apply(qa[t], qb[t], cs, sn, m < H2));
      }
      qin[h][m] = x;
    }
  }
  __syncthreads();
  if (rot) {
    float4 acc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int m = rb * RB + rr;
      float4 p;
      if constexpr (kEarly)
        p = pv[rr];
      else
        p = *reinterpret_cast<const float4*>(Pg + m * D + 4 * cq);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float x = qin[h][m];
        acc[h].x = fmaf(x, p.x, acc[h].x);
        acc[h].y = fmaf(x, p.y, acc[h].y);
        acc[h].z = fmaf(x, p.z, acc[h].z);
        acc[h].w = fmaf(x, p.w, acc[h].w);
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) *reinterpret_cast<float4*>(&red[rb][h][4 * cq]) = acc[h];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NH * ncols; e += kBlock) {
    const int h = e / ncols, col = e % ncols;
    float x = 0.f;
#pragma unroll
    for (int pp = 0; pp < NRB; ++pp) x += red[pp][h][col];
    qr[h][col] = x;
    if (ci == 0 && h < nh) qrot[(static_cast<int64_t>(b) * Hq + h0 + h) * D + col] = x;
  }
  __syncthreads();

  const int part = threadIdx.x % LPS;
  float qf[NH][VEC];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      qf[h][v] = (part * VEC < d) ? qr[h][part * VEC + v] : 0.f;

  // The stream: the loads and dot products of the fused kernel's ranking
  // pass (same lanes, same order), but every lane of a token's lane group
  // ends with the group's sums, so lane `part` keeps heads part, part + LPS,
  // ...  The scores collect in LDS and are stored row by row afterwards: the
  // loop issues no global stores, which on this chip would share the loads'
  // completion counter and stall each wait for the next batch.
  {
    constexpr int TPI = kBlock / LPS;
    constexpr int U = 4;
    constexpr int RND = (NH + LPS - 1) / LPS;
    const int tk = threadIdx.x / LPS;
    const bool active = part * VEC < d;
    const Region gs = make_region(sl, 0x7fffffffu);
    const uint32_t rowb = static_cast<uint32_t>(d) * E::BYTES;
    for (int jb = j0 + tk; jb < j1; jb += TPI * U) {
      if (jb != j0 + tk) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = jb + TPI * u;
          c[u] = (active && j < j1) ? ld16_region(gs, static_cast<uint32_t>(j) * rowb + part * 16u)
                                    : zero_chunk();
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[VEC];
        unpack<E>(c[u], x);
        const int j = jb + TPI * u;
        float dots[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          float dot = 0.f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) dot = fmaf(qf[h][v], x[v], dot);
          dots[h] = group_sum<LPS>(dot);
        }
#pragma unroll
        for (int r = 0; r < RND; ++r) {
          const int hh = r * LPS + part;
          float val = dots[0];
#pragma unroll
          for (int h = 1; h < NH; ++h) val = (h == hh) ? dots[h] : val;
          if (hh < NH && j < j1) ssc[hh][j - j0] = val;
        }
      }
    }
  }
  __syncthreads();
  const int n = j1 - j0;
  float* srow = scores + (static_cast<int64_t>(b) * Hq + h0) * S + j0;
  if (flag) {
    // device-scope stores (written through this XCD's L2), then the flag
    const bool vec = (S & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    if (vec) {
      const Region rr = make_region(srow, 0x7fffffffu);
      for (int h = 0; h < nh; ++h)
        for (int i = threadIdx.x; 4 * i < n; i += kBlock)
          st16_dev(rr, static_cast<uint32_t>((h * S + 4 * i) * 4),
                   *reinterpret_cast<const uint4*>(&ssc[h][4 * i]));
    } else {
      for (int h = 0; h < nh; ++h)
        for (int i = threadIdx.x; i < n; i += kBlock)
          st_dev(srow + static_cast<int64_t>(h) * S + i, ssc[h][i]);
    }
    publish(flag, fval);
    return;
  }
  if ((S & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) {
    // rows start 16-byte aligned (chunks are multiples of 256 tokens)
    for (int h = 0; h < nh; ++h)
      for (int i = threadIdx.x; 4 * i < n; i += kBlock)
        *reinterpret_cast<float4*>(srow + static_cast<int64_t>(h) * S + 4 * i) =
            *reinterpret_cast<const float4*>(&ssc[h][4 * i]);
  } else {
    for (int h = 0; h < nh; ++h)
      for (int i = threadIdx.x; i < n; i += kBlock) srow[static_cast<int64_t>(h) * S + i] = ssc[h][i];
  }
}

// The ranking pass alone.  Grid (B*Hkv*nhb, ceil(S / chunk)).
template <class E, int D, int LPS, int NH>
__global__ void __launch_bounds__(kBlock) score_kernel(const typename E::T* __restrict__ slab,
                                                       const typename E::T* __restrict__ q,
                                                       const float* __restrict__ P,
                                                       float* __restrict__ qrot,
                                                       float* __restrict__ scores, int Hq, int Hkv,
                                                       int d, int S, int S_max, int nhb,
                                                       int chunk, Rope rope) {
  __shared__ ScoreSmem<D, NH> sm;
  score_role<E, D, LPS, NH>(slab, q, P, qrot, scores, Hq, Hkv, d, S, S_max, nhb, chunk, rope,
                            blockIdx.x, blockIdx.y, sm, nullptr, 0ull);
}

// -------------------------------------------------------------------- topk --

// Dynamic LDS: the score row (when use_lds) followed by the kept-position
// bitmap (when `bits` is given: ceil(S/32) words per row, written out for
// the union gather).  The row is staged with coalesced loads, one pad word
// after every 32 scores, so that the register-resident select, where each
// thread takes a contiguous run of up to 32 scores, reads it without bank
// conflicts.  Once the keys are in registers the row's LDS is dead and
// collects the kept ids, which are written out coalesced at the end.
__host__ __device__ constexpr int topk_padded(int S) { return S + (S >> 5) + 1; }

template <int BLOCK>
__global__ void __launch_bounds__(BLOCK) topk_kernel(const float* __restrict__ scores, int S,
                                                     int64_t ld, int k, int* __restrict__ idx,
                                                     int use_lds, unsigned* __restrict__ bits) {
  __shared__ SelectSmemAny<BLOCK> sm;
  extern __shared__ float sbuf[];
  const int row = blockIdx.x;
  const int nw = (S + 31) >> 5;
  unsigned* lbits = reinterpret_cast<unsigned*>(sbuf + (use_lds ? topk_padded(S) : 0));
  if (bits)
    for (int i = threadIdx.x; i < nw; i += BLOCK) lbits[i] = 0u;
  const float* s = scores + static_cast<int64_t>(row) * ld;
  int* out = idx + static_cast<int64_t>(row) * k;
  // the register-resident select reads the row only before its first barrier
  const bool stage_out = use_lds && S <= BLOCK * 32;
  int* lidx = reinterpret_cast<int*>(sbuf);
  auto emit = [&](int p, int j) {
    if (stage_out)
      lidx[p] = j;
    else
      out[p] = j;
    if (bits) atomicOr(&lbits[j >> 5], 1u << (j & 31));
  };
  if (use_lds) {
    const int n4 = S >> 2;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    for (int i = threadIdx.x; i < n4; i += BLOCK) {
      const float4 x = s4[i];
      float* dst = sbuf + 4 * i + (i >> 3);  // 4 scores never straddle a pad word
      dst[0] = x.x;
      dst[1] = x.y;
      dst[2] = x.z;
      dst[3] = x.w;
    }
    for (int i = (n4 << 2) + threadIdx.x; i < S; i += BLOCK) sbuf[i + (i >> 5)] = s[i];
    __syncthreads();
    block_select_topk_any<BLOCK, true>([&](int j) { return sbuf[j + (j >> 5)]; }, S, k, emit, sm);
  } else {
    __syncthreads();
    block_select_topk_any<BLOCK, true>([&](int j) { return s[j]; }, S, k, emit, sm);
  }
  if (stage_out) {
    __syncthreads();
    const int kk = min(k, S);
    for (int p = threadIdx.x; p < kk; p += BLOCK) out[p] = lidx[p];
  }
  if (bits) {
    __syncthreads();
    unsigned* brow = bits + static_cast<int64_t>(row) * nw;
    for (int i = threadIdx.x; i < nw; i += BLOCK) brow[i] = lbits[i];
  }
}

// ------------------------------------------------------- ranking + top-k --

// The ranking pass and the top-k in one launch, for rows of at most
// kSelectMaxS scores.  Workgroups [0, nscore) are the ranking pass's chunks
// (unit id % nunits, chunk id / nunits); workgroup nscore + r selects the
// top k of row r once every chunk of its unit has published its scores.  A
// selecting workgroup waits only on workgroups of lower index, which are
// dispatched before it, so the wait needs no co-residency.  The flags of a
// launch carry its epoch + 1; the epoch, a workspace word, is advanced by the
// gather launch that follows, so flags left by earlier launches never read
// as set, nor do the contents of a fresh workspace (short of a 64-bit
// match), also when a captured graph replays the launches.
// 16 register keys per thread: the 32-key select would raise the whole
// kernel's registers past four waves per SIMD, which the ranking pass needs
constexpr int kSelectMaxS = 16 * kBlock;
static_assert(kSelectMaxS == kScoreSelectMaxS, "the host's limit of the combined launch");
// ranking chunks are at least 256 tokens: at most this many per unit (one
// lane of the waiting wave each)
constexpr int kSelectMaxChunks = kSelectMaxS / 256;
static_assert(kSelectMaxChunks <= 64, "one wave polls a unit's flags");

struct SelSmem {
  SelectSmemR<kBlock> r;
  unsigned bits[kSelectMaxS / 32];
};

// Top-k of one score row (srow, published by other workgroups of this
// launch) into out (kk ascending ids) and, when brow is given, the row's
// kept-position bitmap.  Gives up after kSpinMax polls: then the ids are -1
// and err counts it, so a failure shows in every check of the output.
template <int EMAX, bool LIN>
__device__ __forceinline__ void select_role(const float* __restrict__ srow, int S, int kk, int* __restrict__ out,
                            unsigned* __restrict__ brow, const unsigned long long* flags, int nch,
                            unsigned long long fval, unsigned* err, SelSmem& sm) {
  const int nw = (S + 31) >> 5;
  if (brow)
    for (int i = threadIdx.x; i < nw; i += kBlock) sm.bits[i] = 0u;
  if (!wait_flags(flags, nch, fval)) {
    if (threadIdx.x == 0) atomicAdd(err, 1u);
    for (int p = threadIdx.x; p < kk; p += kBlock) out[p] = -1;
    if (brow)
      for (int i = threadIdx.x; i < nw; i += kBlock) brow[i] = 0u;
    return;
  }
  // this thread's E consecutive scores, loaded with device scope
  const int E = (S + kBlock - 1) / kBlock;
  const int j0 = threadIdx.x * E;
  int nvalid = S - j0;
  nvalid = nvalid < 0 ? 0 : (nvalid > E ? E : nvalid);
  uint32_t key[EMAX];
  if ((E & 3) == 0 && (reinterpret_cast<uintptr_t>(srow) & 15) == 0) {
    const Region rg = make_region(srow, static_cast<uint32_t>(S) * 4u);
#pragma unroll
    for (int c = 0; c < EMAX / 4; ++c) {
      const uint4 v = 4 * c < nvalid ? ld16_dev(rg, static_cast<uint32_t>(j0 + 4 * c) * 4u)
                                     : make_uint4(0u, 0u, 0u, 0u);
      key[4 * c] = order_key(__uint_as_float(v.x));
      key[4 * c + 1] = order_key(__uint_as_float(v.y));
      key[4 * c + 2] = order_key(__uint_as_float(v.z));
      key[4 * c + 3] = order_key(__uint_as_float(v.w));
    }
  } else {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) key[e] = e < nvalid ? order_key(ld_dev(srow + j0 + e)) : 0u;
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e >= nvalid) key[e] = 0u;
  auto emit = [&](int p, int j) {
    out[p] = j;
    if (brow) atomicOr(&sm.bits[j >> 5], 1u << (j & 31));
  };
  block_select_topk_keys<kBlock, EMAX, LIN>(key, nvalid, j0, S, kk, emit, sm.r);
  if (brow) {
    __syncthreads();
    for (int i = threadIdx.x; i < nw; i += kBlock) brow[i] = sm.bits[i];
  }
}

// sync: [0] the epoch, [1] (low word) the count of given-up waits, [2 ..)
// the flags, nch per unit.
template <class E, int D, int LPS, int NH>
__global__ void __launch_bounds__(kBlock) score_select_kernel(
    const typename E::T* __restrict__ slab, const typename E::T* __restrict__ q,
    const float* __restrict__ P, float* __restrict__ qrot, float* __restrict__ scores, int Hq,
    int Hkv, int d, int S, int S_max, int nhb, int chunk, int nch, int nunits, Rope rope, int kk,
    int* __restrict__ idx, unsigned* __restrict__ bits, unsigned long long* __restrict__ sync) {
  __shared__ union {
    ScoreSmem<D, NH> sc;
    SelSmem sel;
  } sm;
  const unsigned long long fval = ld_dev(sync) + 1ull;
  unsigned long long* flags = sync + 2;
  const int nscore = nunits * nch;
  const int id = blockIdx.x;
  if (id < nscore) {
    const int unit = id % nunits, ci = id / nunits;
    score_role<E, D, LPS, NH>(slab, q, P, qrot, scores, Hq, Hkv, d, S, S_max, nhb, chunk, rope,
                              unit, ci, sm.sc, flags + static_cast<int64_t>(unit) * nch + ci, fval);
    return;
  }
  const int row = id - nscore;
  const int G = Hq / Hkv;
  const int b = row / Hq, h = row % Hq;
  const int unit = (b * Hkv + h / G) * nhb + (h % G) / NH;
  const int nw = (S + 31) >> 5;
  const float* srow = scores + static_cast<int64_t>(row) * S;
  int* out = idx + static_cast<int64_t>(row) * kk;
  unsigned* brow = bits ? bits + static_cast<int64_t>(row) * nw : nullptr;
  const unsigned long long* fl = flags + static_cast<int64_t>(unit) * nch;
  unsigned* err = reinterpret_cast<unsigned*>(sync + 1);
  select_role<16, true>(srow, S, kk, out, brow, fl, nch, fval, err, sm.sel);
}

// ------------------------------------------------------------------ attend --

constexpr int kAttendStage = 2048;  // max kept tokens per attend workgroup

// The gather launch after a combined ranking + top-k launch advances the
// epoch of the flags (one thread; the launches on either side are ordered
// by the stream).
__device__ __forceinline__ void advance_epoch(unsigned long long* epoch) {
  if (epoch && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *epoch += 1ull;
}

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
    int nhb, float scale_log2, unsigned long long* __restrict__ epoch) {
  using Gm = Geo<E, D>;
  advance_epoch(epoch);
  constexpr int VEC = Gm::VEC;
  constexpr int LPV = Gm::LPV;
  __shared__ MergeSmem<D, NH, Gm::NG> msm;
  __shared__ int jst[SPARSE ? kAttendStage : 1];
  __shared__ float sst[SPARSE ? kAttendStage : 1];

  const int G = Hq / Hkv;
  int split = blockIdx.y;
  int b, g, h0, nh;
  if (SPARSE) {
    int row = blockIdx.x;  // b*Hq + h
    if (G > 1) {
      // the G query heads of one KV head with the same split index read
      // overlapping position ranges: give them consecutive logical ids on one
      // XCD, so rows that several heads kept come from HBM once and then
      // from that XCD's L2
      const int n = gridDim.x * gridDim.y;
      const int L = xcd_logical(blockIdx.x + blockIdx.y * gridDim.x, n);
      const int rest = L / G;
      split = rest % nsplit;
      row = (rest / nsplit) * G + L % G;
    }
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

constexpr int kUnionMax = kUnionMaxTok;  // token positions per union-gather workgroup
static_assert(kUnionMax % 32 == 0 && kUnionMax / 8 <= kBlock, "one byte of positions per thread");
static_assert(kUnionMaxS <= (1 << 24), "token id and head mask share one word");

template <int NH>
struct UnionList {
  unsigned bw[NH][kUnionMax / 32];  // the G heads' bitmap words of the range
  unsigned ulist[kUnionMax];        // token id | head mask << 24
  unsigned wsum[kBlock / 64];
};

template <int D, int NH, int NG>
union UnionSmem {
  UnionList<NH> g;
  MergeSmem<D, NH, NG> m;  // after the gather
};

// The union of the NH heads' kept tokens in positions [j0, j0 + n) (j0 a
// multiple of 32, n <= kUnionMax), in ascending order with each token's head
// mask: the heads' bitmap words of the range (brow: head h's row at
// brow + h * nw) are read once into LDS; thread t takes 8 positions (one
// byte of each head's bitmap) and the positions that any head kept are
// compacted with a block scan.  Returns the count; ends with a barrier.
template <int NH>
__device__ int union_compact(const unsigned* __restrict__ brow, int nw, int j0, int n,
                             UnionList<NH>& L) {
  constexpr int NW = kBlock / 64;
  const int tid = threadIdx.x;
  const int nwr = (n + 31) >> 5;
  for (int i = tid; i < NH * nwr; i += kBlock) {
    const int h = i / nwr, w = i - h * nwr;
    L.bw[h][w] = brow[static_cast<int64_t>(h) * nw + w];
  }
  __syncthreads();
  unsigned hb[NH];
  unsigned any = 0u;
  {
    const int p0 = tid * 8;
    const unsigned valid = p0 < n ? (n - p0 >= 8 ? 0xffu : (1u << (n - p0)) - 1u) : 0u;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      hb[h] = valid ? (L.bw[h][p0 >> 5] >> (p0 & 31)) & valid : 0u;
      any |= hb[h];
    }
  }
  const unsigned mine = __popc(any);
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned incl = wave_incl_scan(mine, lane);
  if (lane == 63) L.wsum[wave] = incl;
  __syncthreads();
  unsigned before = 0u, ucnt = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += (w < wave) ? L.wsum[w] : 0u;
    ucnt += L.wsum[w];
  }
  unsigned at = before + incl - mine;
  while (any) {
    const int e = __ffs(any) - 1;
    any &= any - 1u;
    unsigned m = 0u;
#pragma unroll
    for (int h = 0; h < NH; ++h) m |= ((hb[h] >> e) & 1u) << h;
    L.ulist[at++] = static_cast<unsigned>(j0 + tid * 8 + e) | (m << 24);
  }
  __syncthreads();
  return static_cast<int>(ucnt);
}

// Union gather for grouped-query attention.  Grid (B*Hkv, nsplit); workgroup
// (bg, split) covers positions [split*R, split*R + R), R a multiple of 32 and
// at most kUnionMax, whose union tokens come from union_compact.  Each union
// token's key and value rows are loaded once for all G = NH heads; a head that
// did not keep a token skips it.
template <class E, int D, int NH>
__global__ void __launch_bounds__(kBlock, 4) attend_union_kernel(
    const typename E::T* __restrict__ slab, const typename E::T* __restrict__ rest,
    const typename E::T* __restrict__ val, const float* __restrict__ qrot,
    const float* __restrict__ scores, const unsigned* __restrict__ bits, float* __restrict__ part,
    float* __restrict__ out, int Hq, int Hkv, int d, int S, int S_max, int R, int nsplit,
    float scale_log2, unsigned long long* __restrict__ epoch) {
  using Gm = Geo<E, D>;
  advance_epoch(epoch);
  constexpr int VEC = Gm::VEC;
  constexpr int LPV = Gm::LPV;
  __shared__ UnionSmem<D, NH, Gm::NG> sm;

  const int bg = blockIdx.x, split = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int h0 = g * NH;
  const int j0 = split * R;
  const int n = max(0, min(S, j0 + R) - j0);
  const int tid = threadIdx.x;

  // this lane's q' dims of the G heads, issued first so that their latency
  // overlaps the bitmap reads
  const int r = tid % LPV;
  const int kd0 = r * VEC;
  float qf[NH][VEC];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const float* qr = qrot + (static_cast<int64_t>(b) * Hq + h0 + h) * D + kd0;
#pragma unroll
    for (int v = 0; v < VEC; v += 4) {
      const float4 x = (kd0 >= d) ? *reinterpret_cast<const float4*>(qr + v)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
      qf[h][v] = x.x;
      qf[h][v + 1] = x.y;
      qf[h][v + 2] = x.z;
      qf[h][v + 3] = x.w;
    }
  }
  const int nw = (S + 31) >> 5;
  const int ucnt = union_compact<NH>(
      bits + (static_cast<int64_t>(b) * Hq + h0) * nw + (j0 >> 5), nw, j0, n, sm.g);

  Acc<VEC> st[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) acc_init(st[h]);
  const int64_t bgo = static_cast<int64_t>(b) * Hkv + g;
  const typename E::T* sl = slab + bgo * S_max * d;
  const typename E::T* rs = rest ? rest + bgo * S_max * (D - d) : nullptr;
  const typename E::T* vv = val + bgo * S_max * D;
  const float* srow = scores + (static_cast<int64_t>(b) * Hq + h0) * S;
  // two tokens in flight per lane group at NH = 4 keeps the kernel within 128
  // VGPRs (four waves per SIMD)
  attend_loop<E, D, NH, true, (NH >= 4 ? 2 : 4)>(
      [&](int t) { return static_cast<int>(sm.g.ulist[t] & 0xffffffu); },
      [&](int h, int, int j) { return srow[static_cast<int64_t>(h) * S + j]; }, 0, ucnt, sl, rs,
      vv, d, qf, scale_log2, st, -1, nullptr, nullptr,
      [&](int t) { return sm.g.ulist[t] >> 24; });
  __syncthreads();  // the merge buffer aliases the token list

  merge_groups<E, D, NH>(st, sm.m, [&](int h, int dim, float M, float L, float A) {
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

// Union gather on the matrix cores (bf16 caches).  Each wave takes the union
// tokens 16 at a time (a tile) and runs both products of all G = NH heads as
// 16x16x16 bf16 MFMAs:
//   logits  S[h][t] = q'_rest[h] . rest[t]: A = q' (heads x dims, rows past G
//           zero), B = the tile's rest rows (dims x tokens; each lane loads 16
//           bytes of one token's row), so lane t < 16 receives token t's G
//           logits;
//   values  O[h][:] += P[h][t] V[t][:]: A = the softmax weights (heads x
//           tokens), B = the tile's value rows (tokens x dims), read from LDS
//           transposed (the rows are staged there as loaded, with a pad of 16
//           bytes per row so the four lane groups read different banks).
// q' and the weights are split into bf16 high and low parts (two MFMAs per
// step), which keeps about 16 bits beyond bf16 with float32 accumulation.
// Softmax statistics are kept per wave (a DPP max and sum over the 16 logit
// lanes per tile); the waves' states are merged in LDS at the end.  NT =
// ceil((D - d) / 32) 32-dim steps of the rest row.
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned short f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even (finite x)
  return static_cast<unsigned short>(u >> 16);
}

// x = hi + lo with hi, lo bf16, for four values (high and low parts of an
// MFMA operand)
__device__ __forceinline__ void split_bf16(const float4& x, bf16x4& hi, bf16x4& lo) {
  const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned short h = f32_to_bf16_bits(xs[i]);
    hi[i] = static_cast<short>(h);
    lo[i] = static_cast<short>(
        f32_to_bf16_bits(xs[i] - __uint_as_float(static_cast<uint32_t>(h) << 16)));
  }
}

template <int D, int NH>
union UnionMfmaSmem {
  struct {
    UnionList<NH> list;
    alignas(16) uint16_t vt[kBlock / 64][16][D + 8];  // per wave: the tile's value rows
    alignas(16) float pt[kBlock / 64][16][20];  // per wave: weights by head row (rows >= NH zero)
  } g;
  struct {
    float m[NH][kBlock / 64], l[NH][kBlock / 64];
    float a[NH][kBlock / 64][D];
  } mrg;
};

// DENSE: the same kernel as the grouped-query dense baseline: every position
// of the range, every head, and the logits over all D dims (NTS 32-dim steps
// of the slab row, then NT of the rest row), with no ranking scores.
template <int D, int NH, int NT, int NTS, bool DENSE>
__global__ void __launch_bounds__(kBlock, 4) attend_union_mfma_kernel(
    const uint16_t* __restrict__ slab, const uint16_t* __restrict__ rest,
    const uint16_t* __restrict__ val, const float* __restrict__ qrot,
    const float* __restrict__ scores, const unsigned* __restrict__ bits,
    float* __restrict__ part, float* __restrict__ out, int Hq, int Hkv, int d, int S, int S_max,
    int R, int nsplit, float scale_log2, unsigned long long* __restrict__ epoch) {
  constexpr int VEC = 8;
  advance_epoch(epoch);
  constexpr int LPV = D / VEC;     // lanes per value row
  constexpr int GPW = 64 / LPV;    // value rows per wave load
  constexpr int TILE = 16;         // union tokens per wave step
  constexpr int US = TILE / GPW;   // value-row loads per lane per tile
  constexpr int NDB = D / 16;      // 16-dim output blocks
  constexpr int NW = kBlock / 64;
  constexpr int NTS1 = NTS > 0 ? NTS : 1;
  static_assert(NH <= 4, "the heads occupy rows 0..3 of the MFMA outputs");
  static_assert(DENSE || NTS == 0, "slab steps only for the dense kernel");
  __shared__ UnionMfmaSmem<D, NH> sm;

  const int bg = blockIdx.x, split = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int h0 = g * NH;
  const int j0 = split * R;
  const int n = max(0, min(S, j0 + R) - j0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int mc = lane >> 4;   // MFMA lane group
  const int mn = lane & 15;   // MFMA row / column index of this lane
  const int Dr = D - d;

  // logits A operand: q' rest dims 32t + 8mc + 4hf + i of head mn
  bf16x4 ahi[NT][2], alo[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int dim = 32 * t + 8 * mc + 4 * hf;  // 4 dims, 16-byte aligned (d % 8 == 0)
      const float4 x4 =
          (mn < NH && dim < Dr)
              ? *reinterpret_cast<const float4*>(
                    qrot + (static_cast<int64_t>(b) * Hq + h0 + mn) * D + d + dim)
              : make_float4(0.f, 0.f, 0.f, 0.f);
      split_bf16(x4, ahi[t][hf], alo[t][hf]);
    }
  // DENSE: the slab dims 32t + 8mc + 4hf + i as well
  bf16x4 shi[NTS1][2], slo[NTS1][2];
  if constexpr (DENSE) {
#pragma unroll
    for (int t = 0; t < NTS; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int dim = 32 * t + 8 * mc + 4 * hf;
        const float4 x4 =
            (mn < NH && dim < d)
                ? *reinterpret_cast<const float4*>(
                      qrot + (static_cast<int64_t>(b) * Hq + h0 + mn) * D + dim)
                : make_float4(0.f, 0.f, 0.f, 0.f);
        split_bf16(x4, shi[t][hf], slo[t][hf]);
      }
  }
  // weight rows past the heads stay zero
  for (int i = lane; i < 16 * 20; i += 64)
    if (i / 20 >= NH) sm.g.pt[wave][i / 20][i % 20] = 0.f;

  int ucnt;
  if constexpr (DENSE) {
    ucnt = n;
    __syncthreads();
  } else {
    const int nw = (S + 31) >> 5;
    ucnt = union_compact<NH>(bits + (static_cast<int64_t>(b) * Hq + h0) * nw + (j0 >> 5), nw,
                             j0, n, sm.g.list);
  }

  const int64_t bgo = static_cast<int64_t>(b) * Hkv + g;
  const Region gs = make_region(DENSE ? slab + bgo * S_max * d : val, 0x7fffffffu);
  const Region gr = make_region(rest ? rest + bgo * S_max * Dr : val, 0x7fffffffu);
  const Region gv = make_region(val + bgo * S_max * D, 0x7fffffffu);
  const float* srow = DENSE ? nullptr : scores + (static_cast<int64_t>(b) * Hq + h0) * S;
  const int r = lane % LPV, gw = lane / LPV;
  const uint32_t vcol = static_cast<uint32_t>(r * VEC) * 2u;

  float m[NH], l[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = wave * TILE; t0 < ucnt; t0 += NW * TILE) {  // wave-uniform
    const int tn = t0 + mn;
    const unsigned en = tn >= ucnt ? 0u
                        : DENSE    ? static_cast<unsigned>(j0 + tn) | (0xfu << 24)
                                   : sm.g.list.ulist[tn];
    const int jn = tn < ucnt ? static_cast<int>(en & 0xffffffu) : -1;
    Chunk sc[NTS1];
    if constexpr (DENSE) {
#pragma unroll
      for (int t = 0; t < NTS; ++t) {
        const int dim = 32 * t + 8 * mc;
        sc[t] = (jn >= 0 && dim < d)
                    ? ld16_region(gs, static_cast<uint32_t>(jn) * d * 2u + dim * 2u)
                    : zero_chunk();
      }
    }
    Chunk rc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int dim = 32 * t + 8 * mc;
      rc[t] = (jn >= 0 && dim < Dr)
                  ? ld16_region(gr, static_cast<uint32_t>(jn) * Dr * 2u + dim * 2u)
                  : zero_chunk();
    }
    Chunk vc[US];
#pragma unroll
    for (int u = 0; u < US; ++u) {
      const int tv = t0 + u * GPW + gw;
      const uint32_t jv = DENSE ? static_cast<uint32_t>(j0 + tv) : (sm.g.list.ulist[tv] & 0xffffffu);
      vc[u] = tv < ucnt ? ld16_region(gv, jv * (D * 2u) + vcol) : zero_chunk();
    }
    float sv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h)
      sv[h] = (!DENSE && mc == 0 && jn >= 0 && ((en >> (24 + h)) & 1u))
                  ? srow[static_cast<int64_t>(h) * S + jn]
                  : 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DENSE) {
#pragma unroll
      for (int t = 0; t < NTS; ++t)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x2 w = hf == 0 ? u32x2{sc[t].u.x, sc[t].u.y} : u32x2{sc[t].u.z, sc[t].u.w};
          const bf16x4 bop = __builtin_bit_cast(bf16x4, w);
          acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(shi[t][hf], bop, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(slo[t][hf], bop, acc, 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x2 w = hf == 0 ? u32x2{rc[t].u.x, rc[t].u.y} : u32x2{rc[t].u.z, rc[t].u.w};
        const bf16x4 bop = __builtin_bit_cast(bf16x4, w);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi[t][hf], bop, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo[t][hf], bop, acc, 0, 0, 0);
      }
    // logits of token mn in lanes 0..15.  The wave's reference maximum m[h]
    // only moves when a logit exceeds it by more than kSlack (weights stay
    // below 2^kSlack), so most tiles need no reduction; l[h] is kept per lane
    // (lanes 0..15, their own tokens) and summed at the end.
    constexpr float kSlack = 8.f;
    float e[NH];
    bool above = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      e[h] = (mc == 0 && jn >= 0 && ((en >> (24 + h)) & 1u)) ? (acc[h] + sv[h]) * scale_log2
                                                              : -INFINITY;
      above |= e[h] > m[h] + kSlack;
    }
    if (__ballot(above)) {  // wave-uniform: move the reference maxima
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float mx = e[h];
        mx = fmaxf(mx, dpp_f<0xB1>(mx));
        mx = fmaxf(mx, dpp_f<0x4E>(mx));
        mx = fmaxf(mx, dpp_f<0x141>(mx));
        mx = fmaxf(mx, dpp_f<0x140>(mx));
        mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
        const float mnew = fmaxf(m[h], mx);
        const float c = (m[h] == mnew) ? 1.f : fast_exp2(m[h] - mnew);
        m[h] = mnew;
        l[h] *= c;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][h] *= c;
      }
    }
    float p[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      p[h] = (e[h] == -INFINITY) ? 0.f : fast_exp2(e[h] - m[h]);
      l[h] += p[h];
    }
    // stage the weights (head rows) and the value rows of the tile
    if (mc == 0) {
#pragma unroll
      for (int h = 0; h < NH; ++h) sm.g.pt[wave][h][mn] = p[h];
    }
#pragma unroll
    for (int u = 0; u < US; ++u)
      *reinterpret_cast<uint4*>(&sm.g.vt[wave][u * GPW + gw][r * VEC]) = vc[u].u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // values A operand: weights of head mn for tokens 4mc .. 4mc+3
    const float4 pw = *reinterpret_cast<const float4*>(&sm.g.pt[wave][mn][4 * mc]);
    bf16x4 phi, plo;
    split_bf16(pw, phi, plo);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 bv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bv[i] = static_cast<short>(sm.g.vt[wave][4 * mc + i][16 * db + mn]);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, o[db], 0, 0, 0);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, o[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the stages are rewritten by the next tile
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // the wave's weight sums: lanes 0..15 hold their own tokens' partial sums
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float sum = l[h];
    sum += dpp_f<0xB1>(sum);
    sum += dpp_f<0x4E>(sum);
    sum += dpp_f<0x141>(sum);
    sum += dpp_f<0x140>(sum);
    l[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), 0));
  }
  __syncthreads();  // the merge buffer aliases the token list and the stages

  // lanes 0..15 hold O[h][16 db + lane]; merge the waves' states
  if (mc == 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int h = 0; h < NH; ++h) sm.mrg.a[h][wave][16 * db + mn] = o[db][h];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      sm.mrg.m[h][wave] = m[h];
      sm.mrg.l[h][wave] = l[h];
    }
  }
  __syncthreads();
  for (int oi = tid; oi < NH * D; oi += kBlock) {
    const int h = oi / D, dim = oi % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.mrg.m[h][w]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm.mrg.m[h][w];
      const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      L = fmaf(sm.mrg.l[h][w], wt, L);
      A = fmaf(sm.mrg.a[h][w][dim], wt, A);
    }
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
  }
}

// Log-sum-exp merge of the nsplit slices of each row (a separate launch:
// a device-wide fence in every attention workgroup would cost more on a
// multi-XCD part, where each XCD's L2 must be written back).  The slice
// weights exp(m_s - M) are computed once per row into LDS (dynamic, nsplit
// floats); each thread then sums its output dims over the slices.
constexpr int kCombineBlock = 128;
constexpr int kCombineMaxSplit = 8192;

template <int D>
__global__ void __launch_bounds__(kCombineBlock) combine_kernel(const float* __restrict__ part,
                                                               float* __restrict__ out,
                                                               int nsplit) {
  extern __shared__ float cw[];
  __shared__ float red[kCombineBlock / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pr = part + row * nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += kCombineBlock) {
    const float m = pr[s * (D + 2) + D];
    cw[s] = m;
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kCombineBlock / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  float L = 0.f;
  for (int s = tid; s < nsplit; s += kCombineBlock) {
    const float m = cw[s];
    const float w = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
    cw[s] = w;
    L = fmaf(pr[s * (D + 2) + D + 1], w, L);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineBlock / 64; ++w) L += red[w];
  for (int dim = tid; dim < D; dim += kCombineBlock) {
    float A = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) A = fmaf(pr[s * (D + 2) + dim], cw[s], A);
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
                     qrot, a.B, a.Hq, a.Hkv, a.rope);
  return hipGetLastError();
}

template <class E, int D, int LPS>
hipError_t score_t(const DecodeArgs& a, float* qrot, float* scores) {
  const int G = a.Hq / a.Hkv;
  const int nh = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
  const int nhb = (G + nh - 1) / nh;
  const int chunk = score_chunk(a.B * a.Hkv * nhb, a.S);
  dim3 grid(a.B * a.Hkv * nhb, (a.S + chunk - 1) / chunk);
  const auto* sl = cptr<E>(a.k_slab);
  const auto* qq = cptr<E>(a.q);
  if (nh == 4)
    hipLaunchKernelGGL((score_kernel<E, D, LPS, 4>), grid, dim3(kBlock), 0, a.stream, sl, qq, a.P,
                       qrot, scores, a.Hq, a.Hkv, a.d, a.S, a.S_max, nhb, chunk, a.rope);
  else if (nh == 2)
    hipLaunchKernelGGL((score_kernel<E, D, LPS, 2>), grid, dim3(kBlock), 0, a.stream, sl, qq, a.P,
                       qrot, scores, a.Hq, a.Hkv, a.d, a.S, a.S_max, nhb, chunk, a.rope);
  else
    hipLaunchKernelGGL((score_kernel<E, D, LPS, 1>), grid, dim3(kBlock), 0, a.stream, sl, qq, a.P,
                       qrot, scores, a.Hq, a.Hkv, a.d, a.S, a.S_max, nhb, chunk, a.rope);
  return hipGetLastError();
}

template <class E, int D, int LPS>
hipError_t score_select_t(const DecodeArgs& a, float* qrot, float* scores, int kk,
                          unsigned* bits) {
  const int G = a.Hq / a.Hkv;
  const int nh = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
  const int nhb = (G + nh - 1) / nh;
  const int nunits = a.B * a.Hkv * nhb;
  const int chunk = score_chunk(nunits, a.S);
  const int nch = (a.S + chunk - 1) / chunk;
  if (nch > kSelectMaxChunks) return hipErrorInvalidValue;
  dim3 grid(nunits * nch + a.B * a.Hq);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, a.stream, cptr<E>(a.k_slab), cptr<E>(a.q), a.P,
                       qrot, scores, a.Hq, a.Hkv, a.d, a.S, a.S_max, nhb, chunk, nch, nunits,
                       a.rope, kk, a.idx, bits, a.sync);
  };
  if (nh == 4)
    go(score_select_kernel<E, D, LPS, 4>);
  else if (nh == 2)
    go(score_select_kernel<E, D, LPS, 2>);
  else
    go(score_select_kernel<E, D, LPS, 1>);
  return hipGetLastError();
}

template <class E, int D>
hipError_t score_select_lps(const DecodeArgs& a, float* qrot, float* scores, int kk,
                            unsigned* bits) {
  constexpr int MAXL = D / E::VEC;
  switch (lps_for(a.d, E::VEC)) {
    case 1: return score_select_t<E, D, 1>(a, qrot, scores, kk, bits);
    case 2: return score_select_t<E, D, 2>(a, qrot, scores, kk, bits);
    case 4: return score_select_t<E, D, 4>(a, qrot, scores, kk, bits);
    case 8: return score_select_t<E, D, 8>(a, qrot, scores, kk, bits);
    case 16:
      if constexpr (MAXL >= 16) return score_select_t<E, D, 16>(a, qrot, scores, kk, bits);
      break;
    case 32:
      if constexpr (MAXL >= 32) return score_select_t<E, D, 32>(a, qrot, scores, kk, bits);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <class E, int D>
hipError_t score_lps(const DecodeArgs& a, float* qrot, float* scores) {
  constexpr int MAXL = D / E::VEC;
  switch (lps_for(a.d, E::VEC)) {
    case 1: return score_t<E, D, 1>(a, qrot, scores);
    case 2: return score_t<E, D, 2>(a, qrot, scores);
    case 4: return score_t<E, D, 4>(a, qrot, scores);
    case 8: return score_t<E, D, 8>(a, qrot, scores);
    case 16:
      if constexpr (MAXL >= 16) return score_t<E, D, 16>(a, qrot, scores);
      break;
    case 32:
      if constexpr (MAXL >= 32) return score_t<E, D, 32>(a, qrot, scores);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t combine(const DecodeArgs& a, const float* part, int nsplit) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  return launch_combine(part, a.out, a.B * a.Hq, a.D, nsplit, a.stream);
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
                       qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, kk,
                       nsplit, 1, scale_log2, a.sync);
  } else {
    const int G = a.Hq / a.Hkv;
    if constexpr (std::is_same_v<E, BF16>) {
      // grouped-query dense attention on the matrix cores: the union
      // kernel over every position of its range
      const int nts = (a.d + 31) / 32, nt = (D - a.d + 31) / 32;
      if ((G == 2 || G == 4) && a.d < D && nts + nt <= 4) {
        const int R = (a.S + nsplit - 1) / nsplit;
        dim3 grid(a.B * a.Hkv, nsplit);
        auto go = [&](auto kern) {
          hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, a.stream, sl, rs, vv, qrot, nullptr,
                             nullptr, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, R, nsplit,
                             scale_log2, nullptr);
        };
        if constexpr (D == 128) {
          if (G == 4)
            nts == 1 ? go(attend_union_mfma_kernel<D, 4, 3, 1, true>)
            : nts == 2 ? go(attend_union_mfma_kernel<D, 4, 2, 2, true>)
                       : go(attend_union_mfma_kernel<D, 4, 1, 3, true>);
          else
            nts == 1 ? go(attend_union_mfma_kernel<D, 2, 3, 1, true>)
            : nts == 2 ? go(attend_union_mfma_kernel<D, 2, 2, 2, true>)
                       : go(attend_union_mfma_kernel<D, 2, 1, 3, true>);
        } else {
          if (G == 4)
            nts == 2 ? go(attend_union_mfma_kernel<D, 4, 1, 2, true>)
            : nt == 2 ? go(attend_union_mfma_kernel<D, 4, 2, 1, true>)
                      : go(attend_union_mfma_kernel<D, 4, 1, 1, true>);
          else
            nts == 2 ? go(attend_union_mfma_kernel<D, 2, 1, 2, true>)
            : nt == 2 ? go(attend_union_mfma_kernel<D, 2, 2, 1, true>)
                      : go(attend_union_mfma_kernel<D, 2, 1, 1, true>);
        }
        return combine(a, part, nsplit);
      }
    }
    const int nh = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
    const int nhb = (G + nh - 1) / nh;
    dim3 grid(a.B * a.Hkv * nhb, nsplit);
    if (nh == 4)
      hipLaunchKernelGGL((attend_kernel<E, D, 4, false>), grid, dim3(kBlock), 0, a.stream, sl, rs,
                         vv, qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max,
                         kk, nsplit, nhb, scale_log2, nullptr);
    else if (nh == 2)
      hipLaunchKernelGGL((attend_kernel<E, D, 2, false>), grid, dim3(kBlock), 0, a.stream, sl, rs,
                         vv, qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max,
                         kk, nsplit, nhb, scale_log2, nullptr);
    else
      hipLaunchKernelGGL((attend_kernel<E, D, 1, false>), grid, dim3(kBlock), 0, a.stream, sl, rs,
                         vv, qrot, scores, idx, part, a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max,
                         kk, nsplit, nhb, scale_log2, nullptr);
  }
  return combine(a, part, nsplit);
}

template <class E, int D>
hipError_t union_t(const DecodeArgs& a, const float* qrot, const float* scores,
                   const unsigned* bits, float* part, int nsplit) {
  const float scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
  const int R = ((a.S + nsplit - 1) / nsplit + 31) / 32 * 32;
  if (R > kUnionMax) return hipErrorInvalidValue;
  dim3 grid(a.B * a.Hkv, nsplit);
  const int G = a.Hq / a.Hkv;
  const int Dr = D - a.d;
  if constexpr (std::is_same_v<E, BF16>) {
    const int nt = (Dr + 31) / 32;
    if (Dr > 0 && nt <= 3) {  // key products on the matrix cores
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, a.stream, cptr<E>(a.k_slab),
                           cptr<E>(a.k_rest), cptr<E>(a.v), qrot, scores, bits, part, a.out, a.Hq,
                           a.Hkv, a.d, a.S, a.S_max, R, nsplit, scale_log2, a.sync);
      };
      if (G == 4) {
        if (nt == 1) go(attend_union_mfma_kernel<D, 4, 1, 0, false>);
        else if (nt == 2) go(attend_union_mfma_kernel<D, 4, 2, 0, false>);
        else if constexpr (D > 64) go(attend_union_mfma_kernel<D, 4, 3, 0, false>);
      } else {
        if (nt == 1) go(attend_union_mfma_kernel<D, 2, 1, 0, false>);
        else if (nt == 2) go(attend_union_mfma_kernel<D, 2, 2, 0, false>);
        else if constexpr (D > 64) go(attend_union_mfma_kernel<D, 2, 3, 0, false>);
      }
      return combine(a, part, nsplit);
    }
  }
  if (G == 4)
    hipLaunchKernelGGL((attend_union_kernel<E, D, 4>), grid, dim3(kBlock), 0, a.stream,
                       cptr<E>(a.k_slab), cptr<E>(a.k_rest), cptr<E>(a.v), qrot, scores, bits, part,
                       a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, R, nsplit, scale_log2, a.sync);
  else
    hipLaunchKernelGGL((attend_union_kernel<E, D, 2>), grid, dim3(kBlock), 0, a.stream,
                       cptr<E>(a.k_slab), cptr<E>(a.k_rest), cptr<E>(a.v), qrot, scores, bits, part,
                       a.out, a.Hq, a.Hkv, a.d, a.S, a.S_max, R, nsplit, scale_log2, a.sync);
  return combine(a, part, nsplit);
}

}  // namespace

hipError_t launch_combine(const float* part, float* out, int rows, int D, int nsplit,
                          hipStream_t stream) {
  if (nsplit > kCombineMaxSplit) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(nsplit) * sizeof(float);
  if (D == 64)
    hipLaunchKernelGGL((combine_kernel<64>), dim3(rows), dim3(kCombineBlock), lds, stream, part,
                       out, nsplit);
  else
    hipLaunchKernelGGL((combine_kernel<128>), dim3(rows), dim3(kCombineBlock), lds, stream, part,
                       out, nsplit);
  return hipGetLastError();
}

hipError_t launch_rotate(const DecodeArgs& a, float* qrot) {
  if (a.dtype == kF32) return a.D == 64 ? rotate_t<F32, 64>(a, qrot) : rotate_t<F32, 128>(a, qrot);
  return a.D == 64 ? rotate_t<BF16, 64>(a, qrot) : rotate_t<BF16, 128>(a, qrot);
}

hipError_t launch_score_select(const DecodeArgs& a, float* qrot, float* scores, int kk,
                               unsigned* bits) {
  if (a.dtype == kF32)
    return a.D == 64 ? score_select_lps<F32, 64>(a, qrot, scores, kk, bits)
                     : score_select_lps<F32, 128>(a, qrot, scores, kk, bits);
  return a.D == 64 ? score_select_lps<BF16, 64>(a, qrot, scores, kk, bits)
                   : score_select_lps<BF16, 128>(a, qrot, scores, kk, bits);
}

hipError_t launch_scores(const DecodeArgs& a, float* qrot, float* scores) {
  if (a.dtype == kF32)
    return a.D == 64 ? score_lps<F32, 64>(a, qrot, scores) : score_lps<F32, 128>(a, qrot, scores);
  return a.D == 64 ? score_lps<BF16, 64>(a, qrot, scores) : score_lps<BF16, 128>(a, qrot, scores);
}

int topk_block_for(int S) { return S <= 4096 ? 256 : (S <= 8192 ? 512 : 1024); }

hipError_t launch_topk(const float* scores, int rows, int S, int64_t ld, int k, int* idx,
                       hipStream_t stream, unsigned* bits) {
  const int blk = topk_block_for(S);
  const size_t lds_bytes = static_cast<size_t>(topk_padded(S)) * sizeof(float);
  const int use_lds = (lds_bytes <= kTopkLdsMax) && (ld % 4 == 0) ? 1 : 0;
  const size_t dyn = (use_lds ? lds_bytes : 0) +
                     (bits ? static_cast<size_t>((S + 31) >> 5) * sizeof(unsigned) : 0);
  if (blk == 256)
    hipLaunchKernelGGL((topk_kernel<256>), dim3(rows), dim3(256), dyn, stream, scores, S, ld, k, idx,
                       use_lds, bits);
  else if (blk == 512)
    hipLaunchKernelGGL((topk_kernel<512>), dim3(rows), dim3(512), dyn, stream, scores, S, ld, k, idx,
                       use_lds, bits);
  else
    hipLaunchKernelGGL((topk_kernel<1024>), dim3(rows), dim3(1024), dyn, stream, scores, S, ld, k,
                       idx, use_lds, bits);
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

hipError_t launch_attend_union(const DecodeArgs& a, const float* qrot, const float* scores,
                               const unsigned* bits, float* part, int nsplit) {
  if (a.dtype == kF32)
    return a.D == 64 ? union_t<F32, 64>(a, qrot, scores, bits, part, nsplit)
                     : union_t<F32, 128>(a, qrot, scores, bits, part, nsplit);
  return a.D == 64 ? union_t<BF16, 64>(a, qrot, scores, bits, part, nsplit)
                   : union_t<BF16, 128>(a, qrot, scores, bits, part, nsplit);
}

}  // namespace loki
