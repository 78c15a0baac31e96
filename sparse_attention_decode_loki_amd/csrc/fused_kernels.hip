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
#include <type_traits>

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
  // Rows in launch order (head-major: row r is head r / B of sequence
  // r % B).  The first nfull are taken whole by one workgroup each; each
  // later row by nsl workgroups ("slices", consecutive ids), which each
  // gather 1/nsl of the row's kept tokens.  With nfull > 0 (the grid, nfull
  // and the sliced rows all multiples of 8) each XCD takes an eighth of the
  // whole rows, then an eighth of the sliced rows, so every CU gets the same
  // mix.  Without coop every slice ranks and selects the whole row and
  // leaves its [accumulator, max, sum] partial in part [rows][nsl][D + 2]
  // for the combine launch.  With coop slice s ranks only its share of the
  // tokens and the slices exchange the scores through xsc [rows][S]; each
  // then selects the whole row and gathers its share, and the last slice
  // merges the others' partials (part [sliced rows][nsl][D + 2]) into out
  // itself.
  int nsl, nfull, coop;
  // grouped ranking (grp = Hq / Hkv > 1, one workgroup per row, rows in
  // (KV head, sequence, query head) order): the grp workgroups of one KV
  // head each score a 1/grp share of the tokens for all grp heads (one slab
  // read, grp products) and exchange the other heads' scores through xsc
  // and sync as the slices of a row do; each then selects and gathers its
  // own row.  Same ranking scores as the single-head pass, so the same result.
  int grp;
  float* part;
  float* xsc;
  // coop or grouped: [0] given-up waits, then kCoopStride words per sliced
  // row (per KV head unit when grouped): its epoch, then the flags of the
  // members' scores and (coop) of their partials
  unsigned long long* sync;
};

// Eight waves per row: the slab stream and the gather each keep twice the
// bytes in flight of a four-wave workgroup, which is what bounds both.
constexpr int kFusedBlock = 512;
constexpr int kFusedKeys = 8;  // keys per thread of the SMALL selection
static_assert(kCoopStride == 1 + 2 * kCoopMaxSlices, "epoch + two flags per slice");

// SMALL: S <= kFusedKeys * kFusedBlock, so the selection keeps the scores as
// register keys with a first-digit histogram counted during the stream.
// At least six waves per SIMD (at most 80 VGPRs): three workgroups of eight
// waves share a CU when the rows outnumber the CUs.
// GRP > 1: the grouped ranking for GRP query heads per KV head (four waves
// per SIMD: its ranking holds GRP products per token).
template <class E, int D, int LPS, bool SMALL, bool STEP, int GRP>
__global__ void __launch_bounds__(kFusedBlock, GRP > 1 ? 4 : 6) fused_kernel(FusedArgs a) {
  using T = typename E::T;
  constexpr int NT = kFusedBlock;
  constexpr bool GROUP = GRP > 1;
  constexpr int GD = GROUP ? kGrpMaxD : 1;
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
    float g[GROUP ? NRB : 1][GRP][GD];  // GROUP: the group's heads, ranking columns
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
  __shared__ float rin[GRP][D];                // q as float (embedded); GROUP: the group's heads
  __shared__ float qg[GRP][GD];                // GROUP: ranking q' of the group's heads
  __shared__ double kin[STEP ? D : 1];         // STEP: the new key, float64 (embedded)
  __shared__ __align__(16) T kslot[STEP ? D : VEC];  // new key row [slab | rest], stored values
  __shared__ __align__(16) T vslot[STEP ? D : VEC];  // new value row
  __shared__ float mown[D + 2];                 // coop: the merging slice's own partial
  extern __shared__ float dyn[];
  float* qs = dyn;
  float* sb = dyn + D;
  int* ib = reinterpret_cast<int*>(dyn + D + a.S);

  const int S = a.S, d = a.d, kk = a.kk;
  // the slices of a row have consecutive logical ids, so they run on one XCD
  // (and, without coop, all but the first find the row's slab in its L2)
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  int rl, slice, nsl;  // row in launch order, this workgroup's slice of it, its slices
  if (a.nfull == 0) {
    rl = L / a.nsl;
    slice = L % a.nsl;
    nsl = a.nsl;
  } else {
    const int m = gridDim.x >> 3, fpx = a.nfull >> 3;
    const int spx = (a.B * a.Hq - a.nfull) >> 3;
    const int x = L / m, i = L % m;
    const bool whole = i < fpx;
    rl = whole ? x * fpx + i : a.nfull + x * spx + (i - fpx) / a.nsl;
    slice = whole ? 0 : (i - fpx) % a.nsl;
    nsl = whole ? 1 : a.nsl;
  }
  const bool coop = a.coop && nsl > 1;
  const int G = a.Hq / a.Hkv;
  // GROUP: row rl is query head rl % GRP of unit rl / GRP = (KV head g,
  // sequence b), units KV-head-major (as rows are otherwise head-major), so
  // a unit's heads share its slab and an XCD's units share their basis in L2
  const int jg = GROUP ? rl % GRP : 0;
  const int h = GROUP ? (rl / GRP) / a.B * GRP + jg : rl / a.B;
  const int b = GROUP ? (rl / GRP) % a.B : rl % a.B;
  const int g = h / G;
  const int64_t row = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bgo = static_cast<int64_t>(b) * a.Hkv + g;
  const T* sl = static_cast<const T*>(a.slab) + bgo * a.S_max * d;
  const T* rs = d < D ? static_cast<const T*>(a.rest) + bgo * a.S_max * (D - d) : nullptr;
  const T* vv = static_cast<const T*>(a.val) + bgo * a.S_max * D;

  if (SMALL)
    for (int i = threadIdx.x; i < kSelBins; i += NT) hist0[i] = 0u;

  // GROUP: the ranking stream is ALU-bound (four products per token), so its
  // first batch of slab loads, four per lane, is issued here, ahead of the
  // rotation, for the share this workgroup ranks
  // (not for a step: its float64 key rotation needs those registers)
  constexpr bool GEARLY = GROUP && !STEP;
  constexpr int US = GEARLY ? 4 : 3;  // 16-byte slab loads in flight per lane
  Chunk cg[GEARLY ? US : 1];
  if constexpr (GEARLY) score_first<E, LPS, US, NT>(sl, d, jg * (S / GRP), (jg + 1) * (S / GRP), cg);

  // 1. q' = q . P[g] (and, for STEP, k' = k_new . P[g] in float64): thread
  //    (cq, rb) adds rows [rb*RB, rb*RB + RB) for columns 4*cq .. 4*cq + 3,
  //    read as 16-byte chunks; the NRB partials are added through LDS.  The
  //    new value row is loaded together with the query.
  // GROUP: the block's basis rows, loaded before the queries so that both
  // arrive in one round trip (the rotation waits for the queries behind a
  // barrier); the single-head kernel has no registers to hold them there
  constexpr bool PEARLY = GEARLY;
  float4 pre[PEARLY ? RB : 1];
  if constexpr (PEARLY) {
    if (threadIdx.x < kBlock) {
      const int cq = threadIdx.x % CQ, rb = threadIdx.x / CQ;
      const float* Pg = a.P + static_cast<int64_t>(g) * D * D;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
        pre[rr] = *reinterpret_cast<const float4*>(Pg + (rb * RB + rr) * D + 4 * cq);
    }
  }
  T vn{};
  if (STEP && threadIdx.x < D) vn = static_cast<const T*>(a.v_new)[bgo * D + threadIdx.x];
  // the queries: this row's, or (GROUP) those of the KV head's GRP heads
  const int64_t qrow0 = GROUP ? row - jg : row;
  if (a.rope.base == 0.0) {
    for (int e = threadIdx.x; e < GRP * D; e += NT)
      rin[e / D][e % D] = ld_elem<E>(static_cast<const T*>(a.q), qrow0 * D + e);
    if (STEP && threadIdx.x < D)
      kin[threadIdx.x] = ld_elem<E>(static_cast<const T*>(a.k_new), bgo * D + threadIdx.x);
  } else {
    // RoPE: each pair's cosine and sine once, then the elements (a step
    // places the query and the new key both at pos: a.rope.pos == a.pos)
    __shared__ double rcs[2][D / 2];
    if (threadIdx.x < D / 2)
      rope_cs(threadIdx.x, D, a.rope.base, a.rope.pos, rcs[0][threadIdx.x], rcs[1][threadIdx.x]);
    __syncthreads();
    for (int e = threadIdx.x; e < GRP * D; e += NT) {
      const int m = e % D, h = D / 2;
      const bool first = m < h;
      const int i = first ? m : m - h, mp = first ? m + h : m - h;
      const T* qv = static_cast<const T*>(a.q) + (qrow0 + e / D) * D;
      rin[e / D][m] = static_cast<float>(rope_apply(ld_elem<E>(qv, m), ld_elem<E>(qv, mp),
                                                    rcs[0][i], rcs[1][i], first));
    }
    if (threadIdx.x < D) {
      const int m = threadIdx.x, h = D / 2;
      const bool first = m < h;
      const int i = first ? m : m - h, mp = first ? m + h : m - h;
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
    float4 accg[GRP];  // GROUP: every head of the group, ranking columns only
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) accg[hh] = make_float4(0.f, 0.f, 0.f, 0.f);
    const bool gcol = GROUP && !STEP && 4 * cq < d;  // (a step: in a pass of its own)
    double kacc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int m = rb * RB + rr;
      const float4 p = PEARLY ? pre[PEARLY ? rr : 0]
                              : *reinterpret_cast<const float4*>(Pg + m * D + 4 * cq);
      const float x = rin[jg][m];
      acc.x = fmaf(x, p.x, acc.x);
      acc.y = fmaf(x, p.y, acc.y);
      acc.z = fmaf(x, p.z, acc.z);
      acc.w = fmaf(x, p.w, acc.w);
      if (gcol) {
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh) {
          const float xg = rin[hh][m];
          accg[hh].x = fmaf(xg, p.x, accg[hh].x);
          accg[hh].y = fmaf(xg, p.y, accg[hh].y);
          accg[hh].z = fmaf(xg, p.z, accg[hh].z);
          accg[hh].w = fmaf(xg, p.w, accg[hh].w);
        }
      }
      if (STEP) {
        const double xk = kin[STEP ? m : 0];
        kacc[0] = fma(xk, static_cast<double>(p.x), kacc[0]);
        kacc[1] = fma(xk, static_cast<double>(p.y), kacc[1]);
        kacc[2] = fma(xk, static_cast<double>(p.z), kacc[2]);
        kacc[3] = fma(xk, static_cast<double>(p.w), kacc[3]);
      }
    }
    *reinterpret_cast<float4*>(&sc.rot.q[rb][4 * cq]) = acc;
    if (gcol) {
#pragma unroll
      for (int hh = 0; hh < GRP; ++hh)
        *reinterpret_cast<float4*>(&sc.rot.g[GROUP ? rb : 0][hh][GROUP ? 4 * cq : 0]) = accg[hh];
    }
    if (STEP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc.rot.k[STEP ? rb : 0][4 * cq + i] = kacc[i];
    }
  }
  __syncthreads();
  if constexpr (GROUP && STEP) {
    // the group's ranking columns in a pass of their own, so that their sums
    // are not live beside the new key's float64 ones (the basis rows come
    // again from cache)
    if (threadIdx.x < kBlock) {
      const int cq = threadIdx.x % CQ, rb = threadIdx.x / CQ;
      if (4 * cq < d) {
        const float* Pg = a.P + static_cast<int64_t>(g) * D * D;
        float4 ag[GRP];
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh) ag[hh] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          const int m = rb * RB + rr;
          const float4 p = *reinterpret_cast<const float4*>(Pg + m * D + 4 * cq);
#pragma unroll
          for (int hh = 0; hh < GRP; ++hh) {
            const float xg = rin[hh][m];
            ag[hh].x = fmaf(xg, p.x, ag[hh].x);
            ag[hh].y = fmaf(xg, p.y, ag[hh].y);
            ag[hh].z = fmaf(xg, p.z, ag[hh].z);
            ag[hh].w = fmaf(xg, p.w, ag[hh].w);
          }
        }
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh)
          *reinterpret_cast<float4*>(&sc.rot.g[GROUP ? rb : 0][hh][GROUP ? 4 * cq : 0]) = ag[hh];
      }
    }
    __syncthreads();
  }
  if (GROUP && threadIdx.x >= NT - GRP * d) {
    // the group's ranking q', summed as the row's own columns are
    const int e = threadIdx.x - (NT - GRP * d), hh = e / d, col = e % d;
    float x = 0.f;
#pragma unroll
    for (int pp = 0; pp < NRB; ++pp) x += sc.rot.g[GROUP ? pp : 0][hh][GROUP ? col : 0];
    qg[hh][GROUP ? col : 0] = x;
  }
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

  // 2. ranking scores -> LDS: of all S tokens, or with coop of this slice's
  //    share [j0s, j1s) (shares of cs tokens, a multiple of 4), or (GROUP)
  //    of share jg (S / GRP tokens) for each head of the group: this row's
  //    into place, head hh's staged in share hh's slots of sb (free until
  //    the exchange below refills them)
  const int cs = coop ? ((S + nsl - 1) / nsl + 3) & ~3 : (GROUP ? S / GRP : S);
  const int j0s = coop ? min(S, slice * cs) : (GROUP ? jg * cs : 0);
  const int j1s = coop ? min(S, j0s + cs) : (GROUP ? j0s + cs : S);
  {
    constexpr int NH = GRP;
    const int part = threadIdx.x % LPS;
    float qf[NH][VEC];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        qf[hh][v] = (part * VEC < d) ? (GROUP ? qg[hh][GROUP ? part * VEC + v : 0]
                                              : qs[part * VEC + v])
                                     : 0.f;
    // STEP: the new token's score from its LDS row, with the streaming
    // pass's arithmetic, formed by every wave (each lane group ends with the
    // same sum), so the stream's value for that slot, read from the cache row
    // the launch has not written yet, is replaced without a barrier
    // (GROUP: after the stream instead, below; the registers are short)
    float snew[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) snew[hh] = 0.f;
    if (STEP && !GROUP) {
      float x[VEC];
      Chunk ch = (part * VEC < d) ? ld16(kslot + part * VEC) : zero_chunk();
      unpack<E>(ch, x);
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) snew[hh] = fmaf(qf[hh][v], x[v], snew[hh]);
        snew[hh] = group_sum<LPS>(snew[hh]);
      }
    }
    Chunk c[US];
    if constexpr (GEARLY) {
#pragma unroll
      for (int u = 0; u < US; ++u) c[u] = cg[GEARLY ? u : 0];
    } else {
      score_first<E, LPS, US, NT>(sl, d, j0s, j1s, c);
    }
    // the selection's first radix digit is counted here, under the stream
    score_loop<E, LPS, NH, US, NT>(sl, d, j0s, j1s, qf, [&](int hh, int j, float s) {
      if (STEP && !GROUP && j == a.pos) s = snew[hh];
      if (hh == jg) {
        sb[j] = s;
        if (SMALL) atomicAdd(&hist0[first_digit(order_key(s))], 1u);
      } else {
        sb[hh * cs + (j - j0s)] = s;
      }
    }, c);
  }
  __syncthreads();
  if constexpr (STEP && GROUP) {
    // the appended token's scores, if it lies in this share: formed from its
    // LDS row with the stream's arithmetic (one lane group per head) and put
    // in place of what the stream read from its slot, the first-digit count
    // moved with it
    const int part = threadIdx.x % LPS, hh = threadIdx.x / LPS;
    if (a.pos >= j0s && a.pos < j1s && hh < GRP) {
      float x[VEC];
      Chunk ch = (part * VEC < d) ? ld16(kslot + part * VEC) : zero_chunk();
      unpack<E>(ch, x);
      float sn = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        sn = fmaf((part * VEC < d) ? qg[hh][GROUP ? part * VEC + v : 0] : 0.f, x[v], sn);
      sn = group_sum<LPS>(sn);
      if (part == 0) {
        if (hh == jg) {
          if (SMALL) {
            atomicSub(&hist0[first_digit(order_key(sb[a.pos]))], 1u);
            atomicAdd(&hist0[first_digit(order_key(sn))], 1u);
          }
          sb[a.pos] = sn;
        } else {
          sb[hh * cs + (a.pos - j0s)] = sn;
        }
      }
    }
    __syncthreads();
  }

  // GROUP: hand the other heads' scores of share jg to their workgroups and
  // take this row's other shares (device scope; flags carry the KV head's
  // epoch + 1, advanced by its last head's workgroup once all have published)
  bool gave_up = false;
  if constexpr (GROUP) {
    unsigned long long* gsync = a.sync + 1 + static_cast<int64_t>(rl / GRP) * kCoopStride;
    const unsigned long long gev = ld_dev(gsync) + 1ull;
    const Region xg = make_region(a.xsc + qrow0 * S, static_cast<uint32_t>(GRP * S) * 4u);
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
      if (hh == jg) continue;
      for (int i = 4 * static_cast<int>(threadIdx.x); i < cs; i += 4 * NT)
        st16_dev(xg, static_cast<uint32_t>(hh * S + j0s + i) * 4u,
                 *reinterpret_cast<const uint4*>(&sb[hh * cs + i]));
    }
    publish(gsync + 1 + jg, gev);
    if (wait_flags(gsync + 1, GRP, gev)) {
      if (jg == GRP - 1 && threadIdx.x == 0) st_dev(gsync, gev);
      constexpr int XU = 4;
      for (int base = 4 * static_cast<int>(threadIdx.x); base < S; base += 4 * NT * XU) {
        uint4 v[XU];
#pragma unroll
        for (int u = 0; u < XU; ++u) {
          const int j = base + 4 * NT * u;
          v[u] = (j < S && (j < j0s || j >= j1s))
                     ? ld16_dev(xg, static_cast<uint32_t>(jg * S + j) * 4u)
                     : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < XU; ++u) {
          const int j = base + 4 * NT * u;
          if (j < S && (j < j0s || j >= j1s)) {
            const float f[4] = {__uint_as_float(v[u].x), __uint_as_float(v[u].y),
                                __uint_as_float(v[u].z), __uint_as_float(v[u].w)};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              sb[j + t] = f[t];
              if (SMALL) atomicAdd(&hist0[first_digit(order_key(f[t]))], 1u);
            }
          }
        }
      }
    } else {
      gave_up = true;
      if (threadIdx.x == 0) atomicAdd(reinterpret_cast<unsigned*>(a.sync), 1u);
    }
    __syncthreads();
  }

  // coop: hand this slice's scores to the row's other slices and take theirs
  // (device scope; each slice's flag carries the row's epoch + 1)
  unsigned long long* rsync = nullptr;
  unsigned long long ev = 0ull;
  if (coop) {
    rsync = a.sync + 1 + static_cast<int64_t>(rl - a.nfull) * kCoopStride;
    ev = ld_dev(rsync) + 1ull;
    float* xrow = a.xsc + row * S;
    const bool vec = (S & 3) == 0 && (reinterpret_cast<uintptr_t>(a.xsc) & 15) == 0;
    const Region xr = make_region(xrow, static_cast<uint32_t>(S) * 4u);
    if (vec) {
      for (int j = j0s + 4 * static_cast<int>(threadIdx.x); j < j1s; j += 4 * NT)
        st16_dev(xr, static_cast<uint32_t>(j) * 4u, *reinterpret_cast<const uint4*>(&sb[j]));
    } else {
      for (int j = j0s + static_cast<int>(threadIdx.x); j < j1s; j += NT) st_dev(xrow + j, sb[j]);
    }
    publish(rsync + 1 + slice, ev);
    if (wait_flags(rsync + 1, nsl, ev)) {
      // every slice has read the epoch: the merging slice advances it
      if (slice == nsl - 1 && threadIdx.x == 0) st_dev(rsync, ev);
      auto take = [&](int j, float s) {
        sb[j] = s;
        if (SMALL) atomicAdd(&hist0[first_digit(order_key(s))], 1u);
      };
      // every score outside this slice's share, XU loads in flight per thread
      constexpr int XU = 4;
      auto other = [&](int j) { return j < S && (j < j0s || j >= j1s); };
      if (vec) {
        for (int base = 4 * static_cast<int>(threadIdx.x); base < S; base += 4 * NT * XU) {
          uint4 v[XU];
#pragma unroll
          for (int u = 0; u < XU; ++u) {
            const int j = base + 4 * NT * u;
            v[u] = other(j) ? ld16_dev(xr, static_cast<uint32_t>(j) * 4u) : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int u = 0; u < XU; ++u) {
            const int j = base + 4 * NT * u;
            if (other(j)) {
              take(j, __uint_as_float(v[u].x));
              take(j + 1, __uint_as_float(v[u].y));
              take(j + 2, __uint_as_float(v[u].z));
              take(j + 3, __uint_as_float(v[u].w));
            }
          }
        }
      } else {
        for (int base = static_cast<int>(threadIdx.x); base < S; base += NT * XU) {
          float v[XU];
#pragma unroll
          for (int u = 0; u < XU; ++u) v[u] = other(base + NT * u) ? ld_dev(xrow + base + NT * u) : 0.f;
#pragma unroll
          for (int u = 0; u < XU; ++u)
            if (other(base + NT * u)) take(base + NT * u, v[u]);
        }
      }
    } else {
      gave_up = true;
      if (threadIdx.x == 0) atomicAdd(reinterpret_cast<unsigned*>(a.sync), 1u);
    }
    __syncthreads();
  }

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

  // 4. gather + exact attention over this slice of the kept tokens
  const int per = (kk + nsl - 1) / nsl;
  const int t0 = min(kk, slice * per), t1 = min(kk, t0 + per);
  const int r = threadIdx.x % Gm::LPV;
  const int kd0 = r * VEC;
  float qf[1][VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) qf[0][v] = (kd0 >= d) ? qs[kd0 + v] : 0.f;
  Acc<VEC> st[1];
  acc_init(st[0]);
  attend_loop<E, D, 1, true, 4, NT>([&](int t) { return ib[t]; },
                                [&](int, int, int j) { return sb[j]; }, t0, t1, sl, rs, vv, d,
                                qf, a.scale_log2, st, STEP ? a.pos : -1, kslot, vslot);
  __syncthreads();  // the merge scratch aliases the selection scratch
  const bool merger = coop && slice == nsl - 1;
  merge_groups<E, D, 1, NT>(st, sc.mrg, [&](int, int dim, float M, float Ls, float A) {
    if (nsl == 1) {
      a.out[row * D + dim] = gave_up ? __builtin_nanf("") : A / Ls;
    } else if (merger) {
      mown[dim] = A;
      if (dim == 0) {
        mown[D] = M;
        mown[D + 1] = Ls;
      }
    } else {
      // coop partials by sliced row, the combine launch's by output row
      const int64_t prow = coop ? rl - a.nfull : row;
      float* pp = a.part + (prow * nsl + slice) * (D + 2);
      if (coop) {
        st_dev(pp + dim, A);
        if (dim == 0) {
          st_dev(pp + D, M);
          st_dev(pp + D + 1, Ls);
        }
      } else {
        pp[dim] = A;
        if (dim == 0) {
          pp[D] = M;
          pp[D + 1] = Ls;
        }
      }
    }
  });
  if (coop && gave_up && merger && threadIdx.x < D)
    a.out[row * D + threadIdx.x] = __builtin_nanf("");
  if (coop && !gave_up) {
    if (!merger) {
      publish(rsync + 1 + kCoopMaxSlices + slice, ev);
    } else {
      // the log-sum-exp merge of the slices in order, as the combine launch
      // forms it, with this slice's own partial from LDS
      const bool ok = wait_flags(rsync + 1 + kCoopMaxSlices, nsl - 1, ev);
      if (!ok && threadIdx.x == 0) atomicAdd(reinterpret_cast<unsigned*>(a.sync), 1u);
      // every partial value loaded at once: the slices' max and sum by the
      // first threads, each output dim's accumulators by its own thread
      const float* pr = a.part + static_cast<int64_t>(rl - a.nfull) * nsl * (D + 2);
      __shared__ float mlx[2][kCoopMaxSlices];
      if (threadIdx.x < 2 * kCoopMaxSlices) {
        const int o = threadIdx.x % kCoopMaxSlices, w = threadIdx.x / kCoopMaxSlices;
        if (o + 1 < nsl) mlx[w][o] = ld_dev(pr + o * (D + 2) + D + w);
        else if (o + 1 == nsl) mlx[w][o] = mown[D + w];
      }
      float av[kCoopMaxSlices];
      const int dim = threadIdx.x;
#pragma unroll
      for (int o = 0; o < kCoopMaxSlices; ++o)
        av[o] = (dim < D && o + 1 < nsl) ? ld_dev(pr + o * (D + 2) + dim) : 0.f;
      __syncthreads();
      if (dim < D) {
        float M = -INFINITY;
        for (int o = 0; o < nsl; ++o) M = fmaxf(M, mlx[0][o]);
        float Ls = 0.f, A = 0.f;
#pragma unroll
        for (int o = 0; o < kCoopMaxSlices; ++o) {
          if (o < nsl) {
            const float m = mlx[0][o];
            const float w = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
            Ls = fmaf(mlx[1][o], w, Ls);
            A = fmaf(o + 1 == nsl ? mown[dim] : av[o], w, A);
          }
        }
        a.out[row * D + dim] = ok ? A / Ls : __builtin_nanf("");
      }
    }
  }
  // The row's stores come last (see the selection above): this slice's part
  // of the idx output and, for STEP, the appended token's cache row (one
  // writer per KV head; this launch served that token from LDS).
  int* irow = a.idx + row * kk;
  for (int p = t0 + threadIdx.x; p < t1; p += NT) irow[p] = gave_up ? -1 : ib[p];
  if (STEP && h % G == 0 && slice == 0 && threadIdx.x < D) {
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

template <class E, int D, int LPS, bool STEP, int GRP>
void fused_g(const FusedArgs& fa, size_t lds, hipStream_t stream, int grid) {
  if (fa.S <= kFusedKeys * kFusedBlock)
    hipLaunchKernelGGL((fused_kernel<E, D, LPS, true, STEP, GRP>), dim3(grid), dim3(kFusedBlock),
                       lds, stream, fa);
  else
    hipLaunchKernelGGL((fused_kernel<E, D, LPS, false, STEP, GRP>), dim3(grid),
                       dim3(kFusedBlock), lds, stream, fa);
}

// the grouped ranking is built for four query heads per KV head on bf16
// caches of D = 128 (the host takes it only there)
template <class E, int D, int LPS, bool STEP>
hipError_t fused_t(const FusedArgs& fa, size_t lds, hipStream_t stream, int grid) {
  if constexpr (std::is_same_v<E, BF16> && D == 128 && LPS * E::VEC <= kGrpMaxD) {
    if (fa.grp == kGrpHeads) {
      fused_g<E, D, LPS, STEP, kGrpHeads>(fa, lds, stream, grid);
      return hipGetLastError();
    }
  }
  if (fa.grp > 1) return hipErrorInvalidValue;
  fused_g<E, D, LPS, STEP, 1>(fa, lds, stream, grid);
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
  const int rows = fa.B * fa.Hq;
  const int grid = fa.nfull + (rows - fa.nfull) * fa.nsl;
  if (fa.nsl < 1 || fa.nfull < 0 || fa.nfull > rows) return hipErrorInvalidValue;
  if (fa.nfull > 0 && (!fa.coop || grid % 8 || fa.nfull % 8 || (rows - fa.nfull) % 8))
    return hipErrorInvalidValue;
  if (fa.coop && fa.nsl > 1 && (fa.nsl > kCoopMaxSlices || !fa.xsc || !fa.sync || !fa.part))
    return hipErrorInvalidValue;
  if (fa.grp > 1 && (fa.nsl != 1 || fa.grp != fa.Hq / fa.Hkv || fa.S % (4 * fa.grp) ||
                     fa.d > kGrpMaxD || !fa.xsc || !fa.sync))
    return hipErrorInvalidValue;
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
  fa.nsl = 1;
  fa.nfull = 0;
  fa.coop = 0;
  fa.grp = 1;
  fa.part = nullptr;
  fa.xsc = nullptr;
  fa.sync = nullptr;
  return fa;
}

void set_slices(FusedArgs& fa, const FusedSlices& fs) {
  fa.nsl = fs.nsl;
  fa.nfull = fs.nfull;
  fa.coop = fs.coop ? 1 : 0;
  fa.grp = fs.grp;
  fa.part = fs.part;
  fa.xsc = fs.xsc;
  fa.sync = fs.sync;
}

}  // namespace

size_t fused_lds_bytes(int D, int S, int kk) {
  return (static_cast<size_t>(D) + S + kk) * sizeof(float);
}

hipError_t launch_fused(const DecodeArgs& a, int kk, const FusedSlices& fs) {
  FusedArgs fa = fused_args(a, kk);
  set_slices(fa, fs);
  hipError_t e = fused_dispatch<false>(fa, a.dtype, a.D, a.stream);
  if (e == hipSuccess && fs.nsl > 1 && !fs.coop)
    e = launch_combine(fs.part, a.out, a.B * a.Hq, a.D, fs.nsl, a.stream);
  return e;
}

hipError_t launch_fused_step(const DecodeArgs& a, const void* k_new, const void* v_new, int pos,
                             int kk, const FusedSlices& fs) {
  FusedArgs fa = fused_args(a, kk);
  fa.k_new = k_new;
  fa.v_new = v_new;
  fa.pos = pos;
  set_slices(fa, fs);
  hipError_t e = fused_dispatch<true>(fa, a.dtype, a.D, a.stream);
  if (e == hipSuccess && fs.nsl > 1 && !fs.coop)
    e = launch_combine(fs.part, a.out, a.B * a.Hq, a.D, fs.nsl, a.stream);
  return e;
}

}  // namespace loki
