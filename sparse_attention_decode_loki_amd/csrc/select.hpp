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

namespace loki {

// Register-resident variant: thread t owns the E = ceil(S / BLOCK)
// consecutive elements [t*E, t*E + E) and keeps their keys in registers; the
// radix select uses three digits (11, 11 and 10 bits) on one shared LDS
// histogram, and the compaction needs a single block-wide scan because each
// thread's elements are consecutive in index order.  Requires S <= BLOCK*EMAX.
//
// With LIN, a first pass bins the values linearly between the row's minimum
// and maximum.  The leading radix digit (sign, exponent, two mantissa bits)
// puts most of a bell-shaped row into a dozen bins, whose LDS atomics then
// serialise and whose crossing bin still holds a few percent of the row;
// linear bins spread the same row evenly, so the bin that holds the k-th
// value usually has only tens of scores, which are ranked against each other
// directly.  The bin of a value is a monotone function of it (a subtraction
// and a multiplication, each rounded, then a truncation clamped to the end
// bins), so every value in a higher bin is larger than every value in a
// lower one.  When the crossing bin holds more than kLinCap scores (heavy
// ties, or outliers spread over the row) the radix passes run as without
// LIN.
constexpr int kSelBins = 2048;
constexpr int kLinCap = 128;

template <int BLOCK>
struct SelectSmemR {
  static constexpr int NW = BLOCK / 64;
  unsigned hist[kSelBins];
  unsigned wsum[2][NW];
  unsigned bin, above, cnt;
  uint32_t wmin[NW], wmax[NW];
  __attribute__((aligned(16))) uint32_t cand[kLinCap];
};

// The value an order key stands for (+0.0 for the key of both zeros).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Minimum and maximum over the 64 lanes of a wave, returned to every lane:
// a DPP butterfly within each row of 16 lanes, then the four rows' results
// read as scalars.
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp_u<0xB1>(mn));
  mx = max(mx, dpp_u<0xB1>(mx));
  mn = min(mn, dpp_u<0x4E>(mn));
  mx = max(mx, dpp_u<0x4E>(mx));
  mn = min(mn, dpp_u<0x141>(mn));
  mx = max(mx, dpp_u<0x141>(mx));
  mn = min(mn, dpp_u<0x140>(mn));
  mx = max(mx, dpp_u<0x140>(mx));
  const auto rl = [](uint32_t v, int l) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  };
  mn = min(min(rl(mn, 0), rl(mn, 16)), min(rl(mn, 32), rl(mn, 48)));
  mx = max(max(rl(mx, 0), rl(mx, 16)), max(rl(mx, 32), rl(mx, 48)));
}

// Exclusive prefix over the block of one value per thread; returns it and
// the block total in `total`.  Contains one barrier; `buf` selects one of two
// LDS slots so back-to-back calls need no second barrier.
template <int BLOCK>
__device__ __forceinline__ unsigned block_excl_scan(unsigned x, unsigned& total,
                                                    SelectSmemR<BLOCK>& sm, int buf) {
  constexpr int NW = BLOCK / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned incl = wave_incl_scan(x, lane);
  if (lane == 63) sm.wsum[buf][wave] = incl;
  __syncthreads();
  unsigned before = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const unsigned s = sm.wsum[buf][w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  total = tot;
  return before + incl - x;
}

// Final compaction of the register-resident selects, in index order.  Key
// e of the calling thread (element j0 + e) is kept when its masked value is
// above `prefix`, or equal to it and among the first krem such keys in
// index order.  One scan of the above-threshold counts and one of the
// at-threshold counts give each thread its first output position; the
// thread then writes its kept elements by walking the set bits of a keep
// mask.
template <int BLOCK, int EMAX, class Emit>
__device__ __forceinline__ void emit_kept(const uint32_t (&key)[EMAX], int nvalid, uint32_t prefix,
                                          uint32_t mask, int krem, int j0, Emit emit,
                                          SelectSmemR<BLOCK>& sm, int buf) {
  static_assert(EMAX <= 32, "one keep mask bit per key");
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const uint32_t m = key[e] & mask;
    const uint32_t live = e < nvalid ? 1u : 0u;
    gtm |= (live & static_cast<uint32_t>(m > prefix)) << e;
    eqm |= (live & static_cast<uint32_t>(m == prefix)) << e;
  }
  const int ngt = __popc(gtm), neq = __popc(eqm);
  unsigned tot;
  const int gt_before = static_cast<int>(block_excl_scan<BLOCK>(ngt, tot, sm, buf));
  const int eq_before = static_cast<int>(block_excl_scan<BLOCK>(neq, tot, sm, buf ^ 1));
  // this thread keeps its first `take` equal keys
  const int take = max(0, min(neq, krem - eq_before));
  uint32_t keep = gtm;
  uint32_t rest = eqm;
  for (int i = 0; i < take; ++i) {
    keep |= rest & (0u - rest);  // lowest set bit
    rest &= rest - 1u;
  }
  int pos = gt_before + min(eq_before, krem);
  while (keep) {
    const int e = __ffs(keep) - 1;
    keep &= keep - 1u;
    emit(pos++, j0 + e);
  }
}

// Crossing bin of the kSelBins-bin histogram `hist` for the krem-th largest
// key, scanned top-down (thread t owns bins [kSelBins - PER*(t+1), kSelBins -
// PER*t)): sets sm.bin, sm.above (keys in higher bins), sm.cnt (keys in the
// bin); ends with a barrier.
template <int BLOCK>
__device__ __forceinline__ void crossing_bin(const unsigned* hist, int krem, SelectSmemR<BLOCK>& sm,
                                             int& buf) {
  constexpr int PER = kSelBins / BLOCK;
  const int hi = kSelBins - PER * static_cast<int>(threadIdx.x);
  unsigned c[PER];
  unsigned local = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = hist[hi - 1 - i];
    local += c[i];
  }
  unsigned total;
  unsigned above = block_excl_scan<BLOCK>(local, total, sm, buf);
  buf ^= 1;
  if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + local) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + c[i]) {
        sm.bin = static_cast<unsigned>(hi - 1 - i);
        sm.above = above;
        sm.cnt = c[i];
      }
      above += c[i];
    }
  }
  __syncthreads();
}

// The linear first pass of block_select_topk_reg<..., LIN>.  Returns true
// and sets prefix (the k-th largest key), mask (all ones) and krem (how many
// keys equal to it are kept) when the crossing bin holds at most kLinCap
// keys; returns false (nothing decided) otherwise.
template <int BLOCK, int EMAX>
__device__ __forceinline__ bool linear_select(const uint32_t (&key)[EMAX], int nvalid, int k,
                                              SelectSmemR<BLOCK>& sm, int& buf, uint32_t& prefix,
                                              uint32_t& mask, int& krem) {
  constexpr int NW = BLOCK / 64;
  static_assert(EMAX <= 32, "one member bit per key");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // row minimum and maximum (as keys: the order map is monotone)
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < nvalid) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  wave_minmax(kmin, kmax);
  if (lane == 0) {
    sm.wmin[wave] = kmin;
    sm.wmax[wave] = kmax;
  }
  for (int i = tid; i < kSelBins; i += BLOCK) sm.hist[i] = 0u;
  __syncthreads();
  // The bins span the second-smallest to the second-largest wave extreme,
  // values beyond them going to the end bins: a few outliers in one wave (the
  // attention sinks of a cache's first tokens) then do not squeeze the rest
  // of the row into a few bins.
  static_assert(NW >= 2, "two waves at least");
  uint32_t min1 = 0xffffffffu, min2 = 0xffffffffu, max1 = 0u, max2 = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t a = sm.wmin[w], b = sm.wmax[w];
    min2 = a < min1 ? min1 : min(min2, a);
    min1 = min(min1, a);
    max2 = b > max1 ? max1 : max(max2, b);
    max1 = max(max1, b);
  }
  kmin = min2;
  kmax = max2;
  const float lo = key_value(kmin);
  const float range = key_value(kmax) - lo;
  const float scale = static_cast<float>(kSelBins) / range;
  // a zero, overflowing or denormal range leaves the radix passes to decide
  if (!(range > 0.f && range < INFINITY && scale < INFINITY)) return false;
  auto bin_of = [&](uint32_t kk) -> int {
    const float f = (key_value(kk) - lo) * scale;
    return f >= static_cast<float>(kSelBins - 1) ? kSelBins - 1 : (f > 0.f ? static_cast<int>(f) : 0);
  };
  // each key's bin, kept in registers two to a word
  uint32_t bins[(EMAX + 1) / 2];
#pragma unroll
  for (int i = 0; i < (EMAX + 1) / 2; ++i) bins[i] = 0u;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < nvalid) {
      const int bn = bin_of(key[e]);
      bins[e >> 1] |= static_cast<uint32_t>(bn) << (16 * (e & 1));
      atomicAdd(&sm.hist[bn], 1u);
    }
  __syncthreads();
  crossing_bin<BLOCK>(sm.hist, k, sm, buf);
  const uint32_t bstar = sm.bin;
  const int above = static_cast<int>(sm.above);
  const int nbin = static_cast<int>(sm.cnt);
  if (nbin > kLinCap) return false;  // (uniform: every thread read the same values)
  // collect the crossing bin's keys (the scan's barrier also ends every
  // thread's reads of sm.bin / sm.above / sm.cnt above), then rank them
  uint32_t member = 0u;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    member |= static_cast<uint32_t>(e < nvalid && ((bins[e >> 1] >> (16 * (e & 1))) & 0xffffu) == bstar)
              << e;
  unsigned total;
  unsigned at = block_excl_scan<BLOCK>(static_cast<unsigned>(__popc(member)), total, sm, buf);
  buf ^= 1;
  if (member) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if ((member >> e) & 1u) sm.cand[at++] = key[e];
  }
  __syncthreads();
  const int kin = k - above;  // 1 <= kin <= nbin
  if (tid < nbin) {
    const uint32_t x = sm.cand[tid];
    int gt = 0, ge = 0;
    const int n4 = nbin & ~3;
    for (int m = 0; m < n4; m += 4) {
      const uint4 y = *reinterpret_cast<const uint4*>(&sm.cand[m]);
      gt += (y.x > x) + (y.y > x) + (y.z > x) + (y.w > x);
      ge += (y.x >= x) + (y.y >= x) + (y.z >= x) + (y.w >= x);
    }
    for (int m = n4; m < nbin; ++m) {
      const uint32_t y = sm.cand[m];
      gt += y > x;
      ge += y >= x;
    }
    // the k-th key: every thread holding its value writes the same result
    if (gt < kin && kin <= ge) {
      sm.bin = x;
      sm.above = static_cast<unsigned>(gt);
    }
  }
  __syncthreads();
  prefix = sm.bin;
  mask = 0xffffffffu;
  krem = kin - static_cast<int>(sm.above);
  return true;
}

// The selection of block_select_topk_reg once the keys are in registers:
// the calling thread's key[e] (e < nvalid) is element j0 + e, with j0 =
// threadIdx.x * ceil(S / BLOCK).
template <int BLOCK, int EMAX, bool LIN = false, class Emit>
__device__ __forceinline__ void block_select_topk_keys(const uint32_t (&key)[EMAX], int nvalid, int j0, int S,
                                       int k, Emit emit, SelectSmemR<BLOCK>& sm) {
  constexpr int PER = kSelBins / BLOCK;  // histogram bins owned per thread in the scan
  static_assert(kSelBins % BLOCK == 0, "bins must split evenly");
  static_assert(!LIN || BLOCK >= kLinCap, "one thread per ranked key");
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u;
  int krem = k;
  int buf = 0;
  if (k < S && !(LIN && linear_select<BLOCK, EMAX>(key, nvalid, k, sm, buf, prefix, mask, krem))) {
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = shifts[pass];
      const uint32_t dmask = (1u << widths[pass]) - 1u;
      for (int i = tid; i < kSelBins; i += BLOCK) sm.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < nvalid && (key[e] & mask) == prefix) atomicAdd(&sm.hist[(key[e] >> shift) & dmask], 1u);
      __syncthreads();
      // thread t scans bins (top-down) [kSelBins - PER*(t+1), kSelBins - PER*t)
      const int hi = kSelBins - PER * tid;
      unsigned c[PER];
      unsigned local = 0u;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        c[i] = sm.hist[hi - 1 - i];
        local += c[i];
      }
      unsigned total;
      unsigned above = block_excl_scan<BLOCK>(local, total, sm, buf);
      buf ^= 1;
      if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + local) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + c[i]) {
            sm.bin = static_cast<unsigned>(hi - 1 - i);
            sm.above = above;
            sm.cnt = c[i];
          }
          above += c[i];
        }
      }
      __syncthreads();
      prefix |= sm.bin << shift;
      mask |= dmask << shift;
      krem -= static_cast<int>(sm.above);
      if (static_cast<int>(sm.cnt) == krem) break;
    }
  }

  emit_kept<BLOCK, EMAX>(key, nvalid, prefix, mask, krem, j0, emit, sm, buf);
}

template <int BLOCK, int EMAX, bool LIN = false, class Src, class Emit>
__device__ void block_select_topk_reg(Src src, int S, int k, Emit emit, SelectSmemR<BLOCK>& sm) {
  const int E = (S + BLOCK - 1) / BLOCK;
  const int j0 = threadIdx.x * E;
  uint32_t key[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int j = j0 + e;
    key[e] = (e < E && j < S) ? order_key(src(j)) : 0u;
  }
  int nvalid = S - j0;
  nvalid = nvalid < 0 ? 0 : (nvalid > E ? E : nvalid);
  block_select_topk_keys<BLOCK, EMAX, LIN>(key, nvalid, j0, S, k, emit, sm);
}

}  // namespace loki

namespace loki {

// LDS for block_select_topk_any (either algorithm).
template <int BLOCK>
union SelectSmemAny {
  SelectSmem<BLOCK> lds;
  SelectSmemR<BLOCK> reg;
};

// Top-k with the register-resident select when each thread's share fits in
// 32 registers, else the LDS/global-resident one.  LIN asks for the linear
// first pass where each thread holds at most 16 keys (a 4096-score row: 8.3
// -> 7.7 us for 32 rows); at 32 keys per thread its extra per-key work costs
// more than the radix passes it saves.
template <int BLOCK, bool LIN = false, class Src, class Emit>
__device__ __forceinline__ void block_select_topk_any(Src src, int S, int k, Emit emit,
                                                      SelectSmemAny<BLOCK>& sm) {
  if (S <= BLOCK * 16)
    block_select_topk_reg<BLOCK, 16, LIN>(src, S, k, emit, sm.reg);
  else if (S <= BLOCK * 32)  // the linear pass does not pay at 32 keys per thread
    block_select_topk_reg<BLOCK, 32>(src, S, k, emit, sm.reg);
  else
    block_select_topk<BLOCK>(src, S, k, emit, sm.lds);
}

}  // namespace loki

namespace loki {

// First radix digit of a key: bits 31..21 (sign, exponent, 2 mantissa bits).
__device__ __forceinline__ uint32_t first_digit(uint32_t key) { return key >> 21; }

// Top-k from a histogram of the first digit that the producer of the scores
// has already accumulated (hist0, kSelBins counters in LDS, zeroed before the
// scores were written).  Thread t owns the E = ceil(S / BLOCK) consecutive
// elements [t*E, t*E + E) as register keys.  After the crossing bin of the
// first digit is known, its candidates (at most CAP; the usual case is about
// a percent of S) are gathered into `cand` (LDS) in index order and the exact
// threshold is found by ranking them against each other; when the bin holds
// more than CAP keys the remaining two digits are resolved by radix passes.
// Requires S <= BLOCK * EMAX.
template <int BLOCK, int EMAX, int CAP, class Src, class Emit>
__device__ void block_select_topk_hist(Src src, int S, int k, const unsigned* hist0, Emit emit,
                                       SelectSmemR<BLOCK>& sm, uint32_t* cand) {
  constexpr int PER = kSelBins / BLOCK;
  const int tid = threadIdx.x;
  const int E = (S + BLOCK - 1) / BLOCK;
  const int j0 = tid * E;
  uint32_t key[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int j = j0 + e;
    key[e] = (e < E && j < S) ? order_key(src(j)) : 0u;
  }
  int nvalid = S - j0;
  nvalid = nvalid < 0 ? 0 : (nvalid > E ? E : nvalid);

  uint32_t prefix = 0u, mask = 0u;
  int krem = k;
  int buf = 0;
  // crossing bin of digit `shift` in `hist`: sets prefix/mask/krem
  auto resolve_digit = [&](const unsigned* hist, int shift, uint32_t dmask) -> bool {
    const int hi = kSelBins - PER * tid;
    unsigned c[PER];
    unsigned local = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      c[i] = hist[hi - 1 - i];
      local += c[i];
    }
    unsigned total;
    unsigned above = block_excl_scan<BLOCK>(local, total, sm, buf);
    buf ^= 1;
    if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + local) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + c[i]) {
          sm.bin = static_cast<unsigned>(hi - 1 - i);
          sm.above = above;
          sm.cnt = c[i];
        }
        above += c[i];
      }
    }
    __syncthreads();
    prefix |= sm.bin << shift;
    mask |= dmask << shift;
    krem -= static_cast<int>(sm.above);
    return static_cast<int>(sm.cnt) == krem;  // the whole bin is kept
  };

  if (k < S && !resolve_digit(hist0, 21, 0x7ffu)) {
    const int nbin = static_cast<int>(sm.cnt);
    if (nbin <= CAP) {
      // gather the bin's keys in index order, then rank them exactly
      unsigned mine = 0u;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) mine += (e < nvalid && (key[e] & mask) == prefix);
      unsigned total;
      unsigned at = block_excl_scan<BLOCK>(mine, total, sm, buf);
      buf ^= 1;
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < nvalid && (key[e] & mask) == prefix) cand[at++] = key[e];
      __syncthreads();
      for (int i = tid; i < nbin; i += BLOCK) {
        const uint32_t x = cand[i];
        int gt = 0, ge = 0;
        for (int m = 0; m < nbin; ++m) {
          const uint32_t y = cand[m];
          gt += y > x;
          ge += y >= x;
        }
        if (gt < krem && krem <= ge) {  // every thread holding this key value agrees
          sm.bin = x;
          sm.above = static_cast<unsigned>(gt);
        }
      }
      __syncthreads();
      prefix = sm.bin;
      mask = 0xffffffffu;
      krem -= static_cast<int>(sm.above);
    } else {
      const int shifts[2] = {10, 0};
      const int widths[2] = {11, 10};
      for (int pass = 0; pass < 2; ++pass) {
        const int shift = shifts[pass];
        const uint32_t dmask = (1u << widths[pass]) - 1u;
        for (int i = tid; i < kSelBins; i += BLOCK) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (e < nvalid && (key[e] & mask) == prefix)
            atomicAdd(&sm.hist[(key[e] >> shift) & dmask], 1u);
        __syncthreads();
        if (resolve_digit(sm.hist, shift, dmask)) break;
      }
    }
  }

  // compaction in index order: one scan of the above-threshold counts and
  // one of the at-threshold counts
  emit_kept<BLOCK, EMAX>(key, nvalid, prefix, mask, krem, j0, emit, sm, buf);
}

}  // namespace loki
