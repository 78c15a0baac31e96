// Single-kernel Loki decode: one workgroup per (sequence, query head) rotates
// the query, streams the whole key slab into LDS scores, selects the top k in
// LDS and gathers + attends over the kept rows (pages titled "Loki: Low-rank
// Keys for Efficient Sparse Attention": summary page, summary line and
// "Approach"; arXiv "Abstract").  Nothing goes through global memory between
// the stages.
//
// The STEP variant is one step of a generation loop: it also appends the
// step's new key/value at position pos (the key rotated into the PCA basis in
// float64 and rounded once, as loki_kv_append does) and decodes over the
// pos + 1 tokens.  No workgroup uses the new token's row from the cache: the
// stream's load of that slot is discarded, and the token's score and rows come
// from LDS, so it does not matter when the writing workgroup's stores land.
// Only the workgroup of the first query head of each KV head writes the slot,
// after its gather.
#include "attend.hpp"
#include "launch.hpp"
#include "score.hpp"
#include "select.hpp"

namespace loki {

struct FusedArgs {
  const void* q;
  const void* k_new;  // STEP: [B, Hkv, D]
  const void* v_new;  // STEP: [B, Hkv, D]
  const float* P;
  void* slab;
  void* rest;
  void* val;
  float* out;
  int* idx;
  int B, Hq, Hkv, d, S, S_max, kk, pos;
  float scale_log2;
  Rope rope;  // the query's embedding; STEP embeds the new key at pos
};

// Eight waves per row: the slab stream and the gather each keep twice the
// bytes in flight of a four-wave workgroup, which is what bounds both.
constexpr int kFusedBlock = 512;
constexpr int kFusedKeys = 8;  // keys per thread of the SMALL selection

// SMALL: S <= kFusedKeys * kFusedBlock, so the selection keeps the scores as
// register keys with a first-digit histogram counted during the stream.
// At least six waves per SIMD (at most 80 VGPRs): three workgroups of eight
// waves share a CU when the rows outnumber the CUs.
template <class E, int D, int LPS, bool SMALL, bool STEP>
__global__ void __launch_bounds__(kFusedBlock, 6) fused_kernel(FusedArgs a) {
  using T = typename E::T;
  constexpr int NT = kFusedBlock;
  using Gm = Geo<E, D, NT>;
  constexpr int VEC = E::VEC;
  // the rotation is formed by kBlock threads with the partition of
  // rotate_kernel and score_kernel, so every path ranks with the same q'
  constexpr int CQ = D / 4;         // column quads of P
  constexpr int NRB = kBlock / CQ;  // row blocks of P
  constexpr int RB = D / NRB;       // rows per block
  struct Rot {
    float q[NRB][D];
    double k[STEP ? NRB : 1][D];
  };
  constexpr int CAP = 64;  // crossing bins up to this size are ranked directly
  struct Sel {
    SelectSmemAny<NT> s;
    uint32_t cand[CAP];
  };
  union Scratch {
    Sel sel;
    MergeSmem<D, 1, Gm::NG> mrg;
    Rot rot;
  };
  __shared__ Scratch sc;
  __shared__ unsigned hist0[SMALL ? kSelBins : 1];  // first-digit histogram of the scores
  __shared__ float rin[D];                     // q as float (embedded)
  __shared__ double kin[STEP ? D : 1];         // STEP: the new key, float64 (embedded)
  __shared__ __align__(16) T kslot[STEP ? D : VEC];  // new key row [slab | rest], stored values
  __shared__ __align__(16) T vslot[STEP ? D : VEC];  // new value row
  extern __shared__ float dyn[];
  float* qs = dyn;
  float* sb = dyn + D;
  int* ib = reinterpret_cast<int*>(dyn + D + a.S);

  const int S = a.S, d = a.d, kk = a.kk;
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int h = L / a.B, b = L % a.B;
  const int G = a.Hq / a.Hkv;
  const int g = h / G;
  const int64_t row = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bgo = static_cast<int64_t>(b) * a.Hkv + g;
  const T* sl = static_cast<const T*>(a.slab) + bgo * a.S_max * d;
  const T* rs = d < D ? static_cast<const T*>(a.rest) + bgo * a.S_max * (D - d) : nullptr;
  const T* vv = static_cast<const T*>(a.val) + bgo * a.S_max * D;

  if (SMALL)
    for (int i = threadIdx.x; i < kSelBins; i += NT) hist0[i] = 0u;

  // 1. q' = q . P[g] (and, for STEP, k' = k_new . P[g] in float64): thread
  //    (cq, rb) adds rows [rb*RB, rb*RB + RB) for columns 4*cq .. 4*cq + 3,
  //    read as 16-byte chunks; the NRB partials are added through LDS.  The
  //    new value row is loaded together with the query.
  T vn{};
  if (STEP && threadIdx.x < D) vn = static_cast<const T*>(a.v_new)[bgo * D + threadIdx.x];
  if (a.rope.base == 0.0) {
    if (threadIdx.x < D) {
      rin[threadIdx.x] = ld_elem<E>(static_cast<const T*>(a.q), row * D + threadIdx.x);
      if (STEP)
        kin[threadIdx.x] = ld_elem<E>(static_cast<const T*>(a.k_new), bgo * D + threadIdx.x);
    }
  } else {
    // RoPE: each pair's cosine and sine once, then the elements (a step
    // places the query and the new key both at pos: a.rope.pos == a.pos)
    __shared__ double rcs[2][D / 2];
    if (threadIdx.x < D / 2)
      rope_cs(threadIdx.x, D, a.rope.base, a.rope.pos, rcs[0][threadIdx.x], rcs[1][threadIdx.x]);
    __syncthreads();
    if (threadIdx.x < D) {
      const int m = threadIdx.x, h = D / 2;
      const bool first = m < h;
      const int i = first ? m : m - h, mp = first ? m + h : m - h;
      const T* qv = static_cast<const T*>(a.q) + row * D;
      rin[m] = static_cast<float>(rope_apply(ld_elem<E>(qv, m), ld_elem<E>(qv, mp), rcs[0][i],
                                             rcs[1][i], first));
      if (STEP) {
        const T* kv = static_cast<const T*>(a.k_new) + bgo * D;
        kin[m] = rope_apply(ld_elem<E>(kv, m), ld_elem<E>(kv, mp), rcs[0][i], rcs[1][i], first);
      }
    }
  }
  if (STEP && threadIdx.x < D) vslot[threadIdx.x] = vn;
  __syncthreads();
  if (threadIdx.x < kBlock) {
    const int cq = threadIdx.x % CQ, rb = threadIdx.x / CQ;
    const float* Pg = a.P + static_cast<int64_t>(g) * D * D;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    double kacc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int m = rb * RB + rr;
      const float4 p = *reinterpret_cast<const float4*>(Pg + m * D + 4 * cq);
      const float x = rin[m];
      acc.x = fmaf(x, p.x, acc.x);
      acc.y = fmaf(x, p.y, acc.y);
      acc.z = fmaf(x, p.z, acc.z);
      acc.w = fmaf(x, p.w, acc.w);
      if (STEP) {
        const double xk = kin[STEP ? m : 0];
        kacc[0] = fma(xk, static_cast<double>(p.x), kacc[0]);
        kacc[1] = fma(xk, static_cast<double>(p.y), kacc[1]);
        kacc[2] = fma(xk, static_cast<double>(p.z), kacc[2]);
        kacc[3] = fma(xk, static_cast<double>(p.w), kacc[3]);
      }
    }
    *reinterpret_cast<float4*>(&sc.rot.q[rb][4 * cq]) = acc;
    if (STEP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc.rot.k[STEP ? rb : 0][4 * cq + i] = kacc[i];
    }
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int col = threadIdx.x;
    float s = 0.f;
#pragma unroll
    for (int pp = 0; pp < NRB; ++pp) s += sc.rot.q[pp][col];
    qs[col] = s;
    if (STEP) {
      double x = 0.0;
#pragma unroll
      for (int pp = 0; pp < NRB; ++pp) x += sc.rot.k[STEP ? pp : 0][col];
      kslot[col] = round_store<E>(x);
    }
  }
  __syncthreads();

  // 2. ranking scores of all S tokens -> LDS
  {
    const int part = threadIdx.x % LPS;
    float qf[1][VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) qf[0][v] = (part * VEC < d) ? qs[part * VEC + v] : 0.f;
    // STEP: the new token's score from its LDS row, with the streaming
    // pass's arithmetic, formed by every wave (each lane group ends with the
    // same sum), so the stream's value for that slot, read from the cache row
    // the launch has not written yet, is replaced without a barrier
    float snew = 0.f;
    if (STEP) {
      float x[VEC];
      Chunk ch = (part * VEC < d) ? ld16(kslot + part * VEC) : zero_chunk();
      unpack<E>(ch, x);
#pragma unroll
      for (int v = 0; v < VEC; ++v) snew = fmaf(qf[0][v], x[v], snew);
      snew = group_sum<LPS>(snew);
    }
    constexpr int US = 3;  // 16-byte slab loads in flight per lane (8 waves)
    Chunk c[US];
    score_first<E, LPS, US, NT>(sl, d, 0, S, c);
    // the selection's first radix digit is counted here, under the stream
    score_loop<E, LPS, 1, US, NT>(sl, d, 0, S, qf, [&](int, int j, float s) {
      if (STEP && j == a.pos) s = snew;
      sb[j] = s;
      if (SMALL) atomicAdd(&hist0[first_digit(order_key(s))], 1u);
    }, c);
  }
  __syncthreads();

  // 3. top-k -> LDS (the idx output is written at the end: one in-order
  //    counter tracks loads and stores alike, so stores issued here would
  //    delay the first wait of the gather by their own latency)
  {
    auto emit = [&](int p, int j) { ib[p] = j; };
    if (SMALL)
      block_select_topk_hist<NT, kFusedKeys, CAP>([&](int j) { return sb[j]; }, S, kk, hist0,
                                                  emit, sc.sel.s.reg, sc.sel.cand);
    else
      block_select_topk_any<NT>([&](int j) { return sb[j]; }, S, kk, emit, sc.sel.s);
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
  attend_loop<E, D, 1, true, 4, NT>([&](int t) { return ib[t]; },
                                [&](int, int, int j) { return sb[j]; }, 0, kk, sl, rs, vv, d,
                                qf, a.scale_log2, st, STEP ? a.pos : -1, kslot, vslot);
  __syncthreads();  // the merge scratch aliases the selection scratch
  merge_groups<E, D, 1, NT>(st, sc.mrg, [&](int, int dim, float, float Ls, float A) {
    a.out[row * D + dim] = A / Ls;
  });
  // The row's stores come last (see the selection above): the idx output and,
  // for STEP, the appended token's cache row (one writer per KV head; this
  // launch served that token from LDS).
  int* irow = a.idx + row * kk;
  for (int p = threadIdx.x; p < kk; p += NT) irow[p] = ib[p];
  if (STEP && h % G == 0 && threadIdx.x < D) {
    const int col = threadIdx.x;
    const int64_t slot = bgo * a.S_max + a.pos;
    if (col < d)
      static_cast<T*>(a.slab)[slot * d + col] = kslot[col];
    else
      static_cast<T*>(a.rest)[slot * (D - d) + (col - d)] = kslot[col];
    static_cast<T*>(a.val)[slot * D + col] = vslot[col];
  }
}

// --------------------------------------------------------------- launchers --

namespace {

template <class E, int D, int LPS, bool STEP>
hipError_t fused_t(const FusedArgs& fa, size_t lds, hipStream_t stream, int grid) {
  if (fa.S <= kFusedKeys * kFusedBlock)
    hipLaunchKernelGGL((fused_kernel<E, D, LPS, true, STEP>), dim3(grid), dim3(kFusedBlock), lds,
                       stream, fa);
  else
    hipLaunchKernelGGL((fused_kernel<E, D, LPS, false, STEP>), dim3(grid), dim3(kFusedBlock), lds,
                       stream, fa);
  return hipGetLastError();
}

// LPS = d*bytes/16 rounded up to a power of two, at most D*bytes/16.
template <class E, int D, bool STEP>
hipError_t fused_lps(const FusedArgs& fa, size_t lds, hipStream_t stream, int grid) {
  int n = (fa.d + E::VEC - 1) / E::VEC, lps = 1;
  while (lps < n) lps <<= 1;
  constexpr int MAXL = D / E::VEC;
  switch (lps) {
    case 1: return fused_t<E, D, 1, STEP>(fa, lds, stream, grid);
    case 2: return fused_t<E, D, 2, STEP>(fa, lds, stream, grid);
    case 4: return fused_t<E, D, 4, STEP>(fa, lds, stream, grid);
    case 8: return fused_t<E, D, 8, STEP>(fa, lds, stream, grid);
    case 16:
      if constexpr (MAXL >= 16) return fused_t<E, D, 16, STEP>(fa, lds, stream, grid);
      break;
    case 32:
      if constexpr (MAXL >= 32) return fused_t<E, D, 32, STEP>(fa, lds, stream, grid);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <bool STEP>
hipError_t fused_dispatch(const FusedArgs& fa, int dtype, int D, hipStream_t stream) {
  const size_t lds = fused_lds_bytes(D, fa.S, fa.kk);
  const int grid = fa.B * fa.Hq;
  if (dtype == kF32)
    return D == 64 ? fused_lps<F32, 64, STEP>(fa, lds, stream, grid)
                   : fused_lps<F32, 128, STEP>(fa, lds, stream, grid);
  return D == 64 ? fused_lps<BF16, 64, STEP>(fa, lds, stream, grid)
                 : fused_lps<BF16, 128, STEP>(fa, lds, stream, grid);
}

FusedArgs fused_args(const DecodeArgs& a, int kk) {
  FusedArgs fa;
  fa.q = a.q;
  fa.k_new = nullptr;
  fa.v_new = nullptr;
  fa.P = a.P;
  fa.slab = const_cast<void*>(a.k_slab);
  fa.rest = const_cast<void*>(a.k_rest);
  fa.val = const_cast<void*>(a.v);
  fa.out = a.out;
  fa.idx = a.idx;
  fa.B = a.B;
  fa.Hq = a.Hq;
  fa.Hkv = a.Hkv;
  fa.d = a.d;
  fa.S = a.S;
  fa.S_max = a.S_max;
  fa.kk = kk;
  fa.pos = -1;
  fa.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(a.D)));
  fa.rope = a.rope;
  return fa;
}

}  // namespace

size_t fused_lds_bytes(int D, int S, int kk) {
  return (static_cast<size_t>(D) + S + kk) * sizeof(float);
}

hipError_t launch_fused(const DecodeArgs& a, int kk) {
  return fused_dispatch<false>(fused_args(a, kk), a.dtype, a.D, a.stream);
}

hipError_t launch_fused_step(const DecodeArgs& a, const void* k_new, const void* v_new, int pos,
                             int kk) {
  FusedArgs fa = fused_args(a, kk);
  fa.k_new = k_new;
  fa.v_new = v_new;
  fa.pos = pos;
  return fused_dispatch<true>(fa, a.dtype, a.D, a.stream);
}

}  // namespace loki
