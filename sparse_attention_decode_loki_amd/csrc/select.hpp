// Block-wide exact top-k selection with lower-index tie-break and
// ascending output.
//
// The pages single out top-k selection as a bottleneck of the original
// implementation (Loki summary page, "Limitations").  Here the k-th largest
// score is found by a most-significant-digit radix select over the 32-bit
// order-preserving keys (four 8-bit digits; each pass histograms only the
// keys that still match the prefix found so far, into one private LDS
// histogram per wave), then the kept indices are compacted in index order
// with wave ballots, so the output is ascending without any sort.
#pragma once

#include "device.hpp"

namespace loki {

template <int BLOCK>
struct SelectSmem {
  static constexpr int NW = BLOCK / 64;
  unsigned hist[NW][256];
  unsigned wsum[NW];
  int wave_cnt[2][NW][2];
  unsigned bin, above, cnt;
};

// Selects the k (1 <= k <= S) largest of src(0..S-1).  Position p of the
// ascending result is delivered as emit(p, j).  All BLOCK threads must call
// it together (it contains barriers); BLOCK >= 256.
template <int BLOCK, class Src, class Emit>
__device__ void block_select_topk(Src src, int S, int k, Emit emit, SelectSmem<BLOCK>& sm) {
  static_assert(BLOCK >= 256 && BLOCK % 64 == 0, "select needs >= 256 threads");
  constexpr int NW = BLOCK / 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  uint32_t prefix = 0u, mask = 0u;
  int krem = k;  // how many of the keys matching `prefix` are still to keep
  if (k < S) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < NW * 256; i += BLOCK) (&sm.hist[0][0])[i] = 0u;
      __syncthreads();
      for (int j = tid; j < S; j += BLOCK) {
        const uint32_t key = order_key(src(j));
        if ((key & mask) == prefix) atomicAdd(&sm.hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // Thread t < 256 owns digit 255 - t, so an inclusive scan over t counts
      // keys from the largest digit down.
      unsigned c = 0u, incl = 0u;
      if (tid < 256) {
        const int bin = 255 - tid;
#pragma unroll
        for (int w = 0; w < NW; ++w) c += sm.hist[w][bin];
        incl = wave_incl_scan(c, lane);
        if (lane == 63) sm.wsum[wave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < wave; ++w) incl += sm.wsum[w];
        const unsigned above = incl - c;
        if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= incl) {
          sm.bin = 255u - tid;
          sm.above = above;
          sm.cnt = c;
        }
      }
      __syncthreads();
      prefix |= sm.bin << shift;
      mask |= 255u << shift;
      krem -= static_cast<int>(sm.above);
      // Every key of this digit is kept: no further digit can change the set.
      if (static_cast<int>(sm.cnt) == krem) break;
    }
  }

  // Compaction in index order.  Keep j when its masked key is above the
  // threshold, or equal to it and among the first `krem` such j.
  int run_sel = 0, run_eq = 0, it = 0;
  for (int base = 0; base < S; base += BLOCK, ++it) {
    const int j = base + tid;
    const bool valid = j < S;
    const uint32_t key = valid ? (order_key(src(j)) & mask) : 0u;
    const bool gt = valid && key > prefix;
    const bool eq = valid && key == prefix;
    const uint64_t bgt = __ballot(gt);
    const uint64_t beq = __ballot(eq);
    const int buf = it & 1;
    if (lane == 0) {
      sm.wave_cnt[buf][wave][0] = __popcll(bgt);
      sm.wave_cnt[buf][wave][1] = __popcll(beq);
    }
    __syncthreads();
    int eq_before = run_eq, sel_before = run_sel, tot_eq = 0, tot_sel = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int g = sm.wave_cnt[buf][w][0];
      const int e = sm.wave_cnt[buf][w][1];
      int take = krem - (run_eq + tot_eq);
      take = take < 0 ? 0 : (take > e ? e : take);
      if (w < wave) {
        eq_before += e;
        sel_before += g + take;
      }
      tot_eq += e;
      tot_sel += g + take;
    }
    const bool sel = gt || (eq && eq_before + lanes_below(beq) < krem);
    const uint64_t bsel = __ballot(sel);
    if (sel) emit(sel_before + lanes_below(bsel), j);
    run_eq += tot_eq;
    run_sel += tot_sel;
    if (run_sel >= k) break;
  }
}

}  // namespace loki
