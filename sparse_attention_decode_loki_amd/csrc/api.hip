// C ABI of libloki.so: argument checks on the host, workspace layout and
// path choice, then kernel launches on the caller's stream.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "loki.h"
#include "launch.hpp"

using loki::DecodeArgs;

// Device memory of the library itself for callers that cannot allocate
// (loki_decode_noalloc): one copy of this array per GPU, alive until the
// process ends.  In host code its name is only a stand-in, never a device
// address.
constexpr size_t kNoallocScratch = LOKI_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratch % 256 == 0, "the workspace layout is in 256-byte units");
static __device__ __align__(256) unsigned char scratch[kNoallocScratch];

namespace {

constexpr int kAbiVersion = LOKI_ABI_VERSION;
constexpr int kTargetWorkgroups = 1024;  // about four per compute unit
constexpr int kAttendStageTok = 2048;    // must match the attend kernel's LDS stage

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }
int esize(int dtype) { return dtype == LOKI_F32 ? 4 : 2; }

int sparse_nsplit(int rows, int kk) {
  int n = std::min(cdiv(kTargetWorkgroups, rows), cdiv(kk, 64));
  n = std::max(n, cdiv(kk, kAttendStageTok));
  return std::max(n, 1);
}

int heads_per_dense_block(int G) { return G >= 4 ? 4 : (G >= 2 ? 2 : 1); }

// Union gather (grouped-query heads): position ranges of at most
// kUnionMaxTok tokens, enough of them to give about four workgroups per CU.
bool union_ok(int Hq, int Hkv, int S) {
  const int G = Hq / Hkv;
  return (G == 2 || G == 4) && S <= loki::kUnionMaxS;
}

// Position ranges are whole bitmap words (R a multiple of 32).
int union_nsplit(int B, int Hkv, int S) {
  int n = std::min(cdiv(kTargetWorkgroups, static_cast<int64_t>(B) * Hkv), cdiv(S, 128));
  n = std::max({1, n, cdiv(S, loki::kUnionMaxTok)});
  const int R = cdiv(cdiv(S, n), 32) * 32;
  return cdiv(S, R);
}

int dense_nsplit(int B, int Hq, int Hkv, int S) {
  const int G = Hq / Hkv;
  const int rows = B * Hkv * cdiv(G, heads_per_dense_block(G));
  return std::max(1, std::min(cdiv(kTargetWorkgroups, rows), cdiv(S, 256)));
}

struct Layout {
  size_t sync, coop, qrot, scores, part, bits, total;
};

// sync (the combined ranking + top-k launch's epoch, given-up count and
// flags; first, so the epoch sits at the same offset for every shape) |
// coop (the sliced single-kernel path's given-up count, epochs and flags) |
// qrot [B*Hq, D] | scores [B*Hq, S_max] (also the sliced path's score
// exchange) | split partials | kept-position bitmaps [B*Hq, ceil(S_max/32)]
// (union gather)
Layout layout(int B, int Hq, int D, int S_max, int nsplit) {
  Layout L;
  const size_t rows = static_cast<size_t>(B) * Hq;
  L.sync = 0;
  L.coop = align256((2 + rows * loki::kScoreSelectFlags) * sizeof(unsigned long long));
  L.qrot = L.coop + align256((1 + rows * loki::kCoopStride) * sizeof(unsigned long long));
  L.scores = L.qrot + align256(rows * D * sizeof(float));
  L.part = L.scores + align256(rows * static_cast<size_t>(S_max) * sizeof(float));
  L.bits = L.part + align256(rows * static_cast<size_t>(nsplit) * (D + 2) * sizeof(float));
  L.total = L.bits + align256(rows * static_cast<size_t>(cdiv(S_max, 32)) * sizeof(unsigned));
  return L;
}

// Workspace layout of the split / union paths for these sizes.
Layout split_layout(int B, int Hq, int Hkv, int D, int S, int S_max, int kk, bool uni) {
  return layout(B, Hq, D, S_max, uni ? union_nsplit(B, Hkv, S) : sparse_nsplit(B * Hq, kk));
}

bool valid_path(int path) {
  return path == LOKI_PATH_AUTO || path == LOKI_PATH_FUSED || path == LOKI_PATH_SPLIT ||
         path == LOKI_PATH_UNION || path == LOKI_PATH_SLICED;
}

// The sliced single-kernel path's split of the rows over workgroups
// (slices of one row share its ranking, so slicing moves no extra bytes,
// but each slice repeats the row's selection).  Fewer rows than compute
// units: every row in nsl slices, the fewest that bring the busiest CU's
// share of rows, ceil(rows * nsl / CUs) / nsl, within 10% of the least
// any allowed count gives (32 rows: 8 slices, one workgroup per CU; 16
// slices, two per CU, measure slower), at least 64 kept tokens per slice.  More rows: whole rows for
// whole rounds of the compute units, and a remainder of at most
// kSlicedTail rows in slices that give every CU one more workgroup (a
// larger remainder measures slower sliced).  The partials fit the split
// path's workspace: rows * nsl <= rows * sparse_nsplit(rows, kk) for few
// rows, and (rows - nfull) * nsl <= kComputeUnits <= rows otherwise.
#ifndef LOKI_SLICED_TAIL
#define LOKI_SLICED_TAIL 64
#endif
constexpr int kSlicedTail = LOKI_SLICED_TAIL;
constexpr int kComputeUnits = 256;  // MI355X
loki::FusedSlices sliced_plan(int rows, int kk) {
  loki::FusedSlices fs;
  fs.coop = true;
  const int cap = std::min(loki::kCoopMaxSlices, cdiv(kk, 64));
  if (rows < kComputeUnits) {
    const int nmax = std::max(1, std::min(cap, sparse_nsplit(rows, kk)));
    // the busiest CU's share of rows with n slices, times 256 * 2^20 / rows
    auto load = [&](int n) {
      return (static_cast<int64_t>(cdiv(static_cast<int64_t>(rows) * n, kComputeUnits)) << 28) / n;
    };
    int64_t best = load(1);
    for (int n = 2; n <= nmax; ++n) best = std::min(best, load(n));
    int n = 1;
    while (10 * load(n) > 11 * best) ++n;
    fs.nsl = n;
    return fs;
  }
  const int rem = rows % kComputeUnits;
  if (rows % 8 != 0 || rem == 0 || rem > kSlicedTail) return fs;  // whole rows
  fs.nsl = std::max(1, std::min(kComputeUnits / rem, cap));
  fs.nfull = fs.nsl > 1 ? rows - rem : 0;
  return fs;
}

int max_nsplit(int B, int Hq, int S_max, int k_max) {
  const int kk = std::max(1, std::min(k_max, S_max));
  // dense_nsplit over any Hkv dividing Hq: its row count is at least B
  const int dense_max = std::max(1, std::min(cdiv(kTargetWorkgroups, B), cdiv(S_max, 256)));
  // union_nsplit never exceeds its range count before rounding, at Hkv = 1
  const int union_max = std::max(
      {1, std::min(cdiv(kTargetWorkgroups, B), cdiv(S_max, 128)), cdiv(S_max, loki::kUnionMaxTok)});
  return std::max({sparse_nsplit(B * Hq, kk), dense_max, union_max});
}

size_t workspace_bytes(int B, int Hq, int D, int S_max, int k_max) {
  return layout(B, Hq, D, S_max, max_nsplit(B, Hq, S_max, k_max)).total;
}

// Shape checks shared by the decode family.  Returns LOKI_OK or an error.
int check_shape(int B, int Hq, int Hkv, int D, int d, int S, int S_max, int dtype) {
  if (dtype != LOKI_F32 && dtype != LOKI_BF16) return LOKI_EINVAL;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return LOKI_EINVAL;
  if (D < 1 || d < 1 || d > D) return LOKI_EINVAL;
  if (S < 1 || S_max < S) return LOKI_EINVAL;
  if (D != 64 && D != 128) return LOKI_EUNSUPPORTED;
  if ((d * esize(dtype)) % 16 != 0) return LOKI_EUNSUPPORTED;
  if (static_cast<int64_t>(B) * Hq > (1 << 30) || Hkv > 65535) return LOKI_EUNSUPPORTED;
  if (S > 65535 * 1024) return LOKI_EUNSUPPORTED;  // score grid.y limit
  // loads address one (sequence, KV head) region with 31-bit byte offsets
  if (static_cast<int64_t>(S_max) * D * esize(dtype) >= (1LL << 31)) return LOKI_EUNSUPPORTED;
  return LOKI_OK;
}

int check_cache_ptrs(const void* k_slab, const void* k_rest, const void* v, const float* P, int D,
                     int d) {
  if (!k_slab || !v || !P) return LOKI_EINVAL;
  if (d < D && !k_rest) return LOKI_EINVAL;
  if (!aligned16(k_slab) || !aligned16(v) || !aligned16(P)) return LOKI_EINVAL;
  if (k_rest && !aligned16(k_rest)) return LOKI_EINVAL;
  return LOKI_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? LOKI_OK : LOKI_EDEVICE; }

bool rope_ok(double base) { return std::isfinite(base) && base > 0.0; }

DecodeArgs make_args(const void* q, const void* k_slab, const void* k_rest, const void* v,
                     const float* P, int B, int Hq, int Hkv, int D, int d, int S, int S_max,
                     int dtype, float* out, int32_t* idx, void* stream) {
  DecodeArgs a;
  a.q = q;
  a.k_slab = k_slab;
  a.k_rest = d < D ? k_rest : nullptr;
  a.v = v;
  a.P = P;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.d = d;
  a.S = S;
  a.S_max = S_max;
  a.dtype = dtype;
  a.out = out;
  a.idx = idx;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

bool fused_fits(int D, int S, int kk) {
  return loki::fused_lds_bytes(D, S, kk) <= loki::kFusedLdsMax;
}

// The fused kernel, when its LDS fits.  One workgroup streams a whole row:
// its time grows with S but hardly with the number of rows while they fit
// on the chip, about 8.7 + 0.0051 * S us; the split path costs about 20 us
// plus 2.7e-5 us per row and token.  Fused is faster when rows > 190 -
// 420000 / S (measured, bf16, D = 128, d = 32, k = S/4: split wins at 64
// rows of 4096 and 128 rows of 8192, fused at 96 and 192).  With grouped
// query heads it reads each KV head's slab once per query head, but the G
// workgroups of one KV head run on one XCD and share it in L2: at 256 and
// 512 rows of G = 4 it beats the union gather (Llama3-8B shape, 8 x 32
// heads of 8192: 58.6 against 63.3 us; 16 x 32 of 4096: 55.7 against 60.6).
bool auto_fused(int B, int Hq, int Hkv, int D, int S, int kk) {
  (void)Hkv;
  if (!fused_fits(D, S, kk)) return false;
  const int64_t rows = static_cast<int64_t>(B) * Hq;
  return rows * S + 420000 >= 190LL * S;
}

// The union gather is chosen (bf16 caches, where its products run on the
// matrix cores) when, even for query heads that select independently of
// each other, the union of their kept tokens, a fraction 1 - (1 - k/S)^G of
// the positions, is at most 3/4 of the G*k/S per-head reads: at k = S/4 and
// G = 4 (68% against 100%) it measures faster than the per-head gather, at
// k = S/8 (41% against 50%) slower.  Heads whose selections overlap only
// favour it more.
bool auto_union(int Hq, int Hkv, int D, int d, int S, int kk, int dtype) {
  if (!union_ok(Hq, Hkv, S) || dtype != LOKI_BF16 || d >= D || (D - d + 31) / 32 > 3) return false;
  const int G = Hq / Hkv;
  const double f = static_cast<double>(kk) / S;
  return 1.0 - std::pow(1.0 - f, G) <= 0.75 * G * f;
}

// The sliced single-kernel path wherever its plan slices rows (fewer rows
// than CUs, or a remainder of at most kSlicedTail rows past whole rounds)
// and rows hold at least 2048 tokens, when its LDS fits.  Measured (bf16,
// D = 128, d = 32, k = S/4, us): 32 rows of 4096 18.3 against split 22.2,
// fused 30.3 and dense 22.1; 64 rows 21.4 against split 27.8; 128 rows
// 28.2 against fused 33.9; 32 rows of 8192 24.0 against split 30.6; 288
// rows of 3584 37.9 against fused 44.8, 576 rows 67.3 against 72.0; 32
// query heads on 8 KV heads, 32 rows of 4096, 16.9 against split 23.6 and
// union 25.9.  Shorter rows give the slices too little to rank: 128 rows
// of 1024 16.8 against fused 15.4.
bool auto_sliced(int B, int Hq, int Hkv, int D, int S, int kk) {
  (void)Hkv;
  const int64_t rows = static_cast<int64_t>(B) * Hq;
  return fused_fits(D, S, kk) && S >= 2048 && rows <= (1 << 30) &&
         sliced_plan(static_cast<int>(rows), kk).nsl > 1;
}

// The path AUTO resolves to.
int auto_path(int B, int Hq, int Hkv, int D, int d, int S, int kk, int dtype) {
  if (auto_sliced(B, Hq, Hkv, D, S, kk)) return LOKI_PATH_SLICED;
  if (auto_fused(B, Hq, Hkv, D, S, kk)) return LOKI_PATH_FUSED;
  return auto_union(Hq, Hkv, D, d, S, kk, dtype) ? LOKI_PATH_UNION : LOKI_PATH_SPLIT;
}


int append_impl(const void* k_new, const void* v_new, const float* P, void* k_slab, void* k_rest,
                void* v, int32_t B, int32_t Hkv, int32_t D, int32_t d, int32_t S_max, int32_t pos,
                int32_t T, int32_t dtype, double rope_base, void* stream) {
  if (dtype != LOKI_F32 && dtype != LOKI_BF16) return LOKI_EINVAL;
  if (B < 0 || Hkv < 1 || D < 1 || d < 1 || d > D || S_max < 1 || pos < 0 || T < 0)
    return LOKI_EINVAL;
  if (static_cast<int64_t>(pos) + T > S_max) return LOKI_EINVAL;
  if (D != 64 && D != 128) return LOKI_EUNSUPPORTED;
  if ((d * esize(dtype)) % 16 != 0) return LOKI_EUNSUPPORTED;
  if (B == 0 || T == 0) return LOKI_OK;
  if (!k_new || !v_new) return LOKI_EINVAL;
  int st = check_cache_ptrs(k_slab, k_rest, v, P, D, d);
  if (st != LOKI_OK) return st;
  if (Hkv > 65535 || static_cast<int64_t>(B) * T > (1LL << 30)) return LOKI_EUNSUPPORTED;
  return status_of(loki::launch_append(k_new, v_new, P, k_slab, d < D ? k_rest : nullptr, v, B,
                                       Hkv, D, d, S_max, pos, T, dtype,
                                       static_cast<hipStream_t>(stream), rope_base));
}


// The sliced path's plan and its workspace regions (any slicing needs the
// workspace: partials, the score exchange and the hand-over flags).
int sliced_slices(int B, int Hq, int D, int S_max, int kk, void* workspace, size_t ws_bytes,
                  loki::FusedSlices& fs) {
  const int rows = B * Hq;
  fs = sliced_plan(rows, kk);
  if (fs.nsl == 1) return LOKI_OK;
  // partials of the sliced rows only, as many as nsplit per row would hold
  const Layout L = layout(B, Hq, D, S_max, cdiv(static_cast<int64_t>(rows - fs.nfull) * fs.nsl, rows));
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return LOKI_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  fs.part = reinterpret_cast<float*>(ws + L.part);
  fs.xsc = reinterpret_cast<float*>(ws + L.scores);
  fs.sync = reinterpret_cast<unsigned long long*>(ws + L.coop);
  return LOKI_OK;
}

// The grouped ranking of the single-kernel decode and step, where it is
// built (four query heads per KV head, bf16, D = 128, d <= 64, S a multiple
// of 16) and a large enough workspace is given; it changes no result (the
// same scores reach every selection), only where they are computed.
void grouped_ranking(int B, int Hq, int Hkv, int D, int d, int S, int S_max, int dtype,
                     void* workspace, size_t ws_bytes, loki::FusedSlices& fs) {
  if (fs.nsl != 1 || Hq != loki::kGrpHeads * Hkv || dtype != LOKI_BF16 || D != 128 ||
      d > loki::kGrpMaxD || S % (4 * loki::kGrpHeads) != 0)
    return;
  const Layout L = layout(B, Hq, D, S_max, 1);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return;
  char* ws = static_cast<char*>(workspace);
  fs.grp = loki::kGrpHeads;
  fs.xsc = reinterpret_cast<float*>(ws + L.scores);
  fs.sync = reinterpret_cast<unsigned long long*>(ws + L.coop);
}

int decode_impl(const void* q, const void* k_slab, const void* k_rest, const void* v,
                const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                int32_t S, int32_t S_max, int32_t k, int32_t dtype, float* out, int32_t* idx,
                void* workspace, size_t ws_bytes, int32_t path, loki::Rope rope, void* stream) {
  int st = check_shape(B, Hq, Hkv, D, d, S, S_max, dtype);
  if (st != LOKI_OK) return st;
  if (k < 1) return LOKI_EINVAL;
  if (!valid_path(path)) return LOKI_EINVAL;
  const int kk = std::min(k, S);
  if (path == LOKI_PATH_AUTO) path = auto_path(B, Hq, Hkv, D, d, S, kk, dtype);
  const bool uni = path == LOKI_PATH_UNION;
  if (uni && !union_ok(Hq, Hkv, S)) return LOKI_EUNSUPPORTED;
  if (B == 0) return LOKI_OK;
  if (!q || !out || !idx) return LOKI_EINVAL;
  st = check_cache_ptrs(k_slab, k_rest, v, P, D, d);
  if (st != LOKI_OK) return st;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(idx) & 3u)) return LOKI_EINVAL;
  DecodeArgs a = make_args(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, dtype, out, idx,
                           stream);
  a.rope = rope;
  const int rows = B * Hq;
  if (path == LOKI_PATH_FUSED || path == LOKI_PATH_SLICED) {
    if (!fused_fits(D, S, kk)) return LOKI_EUNSUPPORTED;
    loki::FusedSlices fs;
    if (path == LOKI_PATH_SLICED) {
      st = sliced_slices(B, Hq, D, S_max, kk, workspace, ws_bytes, fs);
      if (st != LOKI_OK) return st;
    }
    grouped_ranking(B, Hq, Hkv, D, d, S, S_max, dtype, workspace, ws_bytes, fs);
    return status_of(loki::launch_fused(a, kk, fs));
  }
  const int nsplit = uni ? union_nsplit(B, Hkv, S) : sparse_nsplit(rows, kk);
  const Layout L = split_layout(B, Hq, Hkv, D, S, S_max, kk, uni);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return LOKI_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* qrot = reinterpret_cast<float*>(ws + L.qrot);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  float* part = reinterpret_cast<float*>(ws + L.part);
  unsigned* bits = reinterpret_cast<unsigned*>(ws + L.bits);
  hipError_t e;
  if (S <= loki::kScoreSelectMaxS) {
    // ranking and top-k in one launch; the gather launch advances its epoch
    a.sync = reinterpret_cast<unsigned long long*>(ws + L.sync);
    e = loki::launch_score_select(a, qrot, scores, kk, uni ? bits : nullptr);
  } else {
    e = loki::launch_scores(a, qrot, scores);
    if (e == hipSuccess)
      e = loki::launch_topk(scores, rows, S, S, kk, idx, a.stream, uni ? bits : nullptr);
  }
  if (e == hipSuccess)
    e = uni ? loki::launch_attend_union(a, qrot, scores, bits, part, nsplit)
            : loki::launch_attend(a, qrot, scores, idx, kk, part, nsplit, true);
  return status_of(e);
}

int step_impl(const void* q, const void* k_new, const void* v_new, const float* P, void* k_slab,
              void* k_rest, void* v, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
              int32_t pos, int32_t S_max, int32_t k, int32_t dtype, float* out, int32_t* idx,
              void* workspace, size_t ws_bytes, int32_t path, double rope_base, void* stream) {
  if (pos < 0) return LOKI_EINVAL;
  const int S = pos + 1;
  int st = check_shape(B, Hq, Hkv, D, d, S, S_max, dtype);
  if (st != LOKI_OK) return st;
  if (k < 1) return LOKI_EINVAL;
  if (!valid_path(path)) return LOKI_EINVAL;
  const int kk = std::min(k, S);
  if (path == LOKI_PATH_AUTO) path = auto_path(B, Hq, Hkv, D, d, S, kk, dtype);
  const bool uni = path == LOKI_PATH_UNION;
  if (uni && !union_ok(Hq, Hkv, S)) return LOKI_EUNSUPPORTED;
  if (B == 0) return LOKI_OK;
  if (!q || !k_new || !v_new || !out || !idx) return LOKI_EINVAL;
  st = check_cache_ptrs(k_slab, k_rest, v, P, D, d);
  if (st != LOKI_OK) return st;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(idx) & 3u)) return LOKI_EINVAL;
  DecodeArgs a = make_args(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, dtype, out, idx,
                           stream);
  loki::Rope rope;  // the query and the new key sit at position pos
  rope.base = rope_base;
  rope.pos = pos;
  a.rope = rope;
  if (path == LOKI_PATH_FUSED || path == LOKI_PATH_SLICED) {
    if (!fused_fits(D, S, kk)) return LOKI_EUNSUPPORTED;
    loki::FusedSlices fs;
    if (path == LOKI_PATH_SLICED) {
      st = sliced_slices(B, Hq, D, S_max, kk, workspace, ws_bytes, fs);
      if (st != LOKI_OK) return st;
    }
    grouped_ranking(B, Hq, Hkv, D, d, S, S_max, dtype, workspace, ws_bytes, fs);
    return status_of(loki::launch_fused_step(a, k_new, v_new, pos, kk, fs));
  }
  const Layout L = split_layout(B, Hq, Hkv, D, S, S_max, kk, uni);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return LOKI_EWORKSPACE;
  hipError_t e = loki::launch_append(k_new, v_new, P, k_slab, d < D ? k_rest : nullptr, v, B, Hkv,
                                     D, d, S_max, pos, 1, dtype, a.stream, rope_base);
  if (e != hipSuccess) return LOKI_EDEVICE;
  return decode_impl(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, k, dtype, out, idx,
                     workspace, ws_bytes, uni ? LOKI_PATH_UNION : LOKI_PATH_SPLIT, rope, stream);
}

int dense_impl(const void* q, const void* k_slab, const void* k_rest, const void* v,
               const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d, int32_t S,
               int32_t S_max, int32_t dtype, float* out, void* workspace, size_t ws_bytes,
               loki::Rope rope, void* stream) {
  int st = check_shape(B, Hq, Hkv, D, d, S, S_max, dtype);
  if (st != LOKI_OK) return st;
  if (B == 0) return LOKI_OK;
  if (!q || !out) return LOKI_EINVAL;
  st = check_cache_ptrs(k_slab, k_rest, v, P, D, d);
  if (st != LOKI_OK) return st;
  if (!aligned16(out)) return LOKI_EINVAL;
  const int nsplit = dense_nsplit(B, Hq, Hkv, S);
  const Layout L = layout(B, Hq, D, S_max, nsplit);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return LOKI_EWORKSPACE;
  DecodeArgs a = make_args(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, dtype, out,
                           nullptr, stream);
  a.rope = rope;
  char* ws = static_cast<char*>(workspace);
  float* qrot = reinterpret_cast<float*>(ws + L.qrot);
  float* part = reinterpret_cast<float*>(ws + L.part);
  hipError_t e = loki::launch_rotate(a, qrot);
  if (e == hipSuccess)
    e = loki::launch_attend(a, qrot, nullptr, nullptr, S, part, nsplit, false);
  return status_of(e);
}

// ---- scratch of loki_decode_noalloc ----------------------------------------
//
// The array itself (`scratch`) is at file scope above; its device address is
// what hipGetSymbolAddress reports with a device current, looked up once per
// device and kept.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Address of the current device's scratch, or a status.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LOKI_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return LOKI_EUNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return LOKI_EDEVICE;
  *out = g_scratch_ptr[dev];
  return LOKI_OK;
}

}  // namespace

extern "C" {

const char* loki_status_string(int status) {
  switch (status) {
    case LOKI_OK: return "LOKI_OK";
    case LOKI_EINVAL: return "LOKI_EINVAL: invalid argument";
    case LOKI_EWORKSPACE: return "LOKI_EWORKSPACE: workspace missing or too small";
    case LOKI_EDEVICE: return "LOKI_EDEVICE: HIP launch failed";
    case LOKI_EUNSUPPORTED: return "LOKI_EUNSUPPORTED: unsupported shape or dtype";
    default: return "LOKI: unknown status";
  }
}

int loki_abi_version(void) { return kAbiVersion; }


int loki_kv_append(const void* k_new, const void* v_new, const float* P, void* k_slab,
                   void* k_rest, void* v, int32_t B, int32_t Hkv, int32_t D, int32_t d,
                   int32_t S_max, int32_t pos, int32_t T, int32_t dtype, void* stream) {
  return append_impl(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, D, d, S_max, pos, T, dtype, 0.0,
                     stream);
}

int loki_kv_append_rope(const void* k_new, const void* v_new, const float* P, void* k_slab,
                        void* k_rest, void* v, int32_t B, int32_t Hkv, int32_t D, int32_t d,
                        int32_t S_max, int32_t pos, int32_t T, int32_t dtype, double rope_base,
                        void* stream) {
  if (!rope_ok(rope_base)) return LOKI_EINVAL;
  return append_impl(k_new, v_new, P, k_slab, k_rest, v, B, Hkv, D, d, S_max, pos, T, dtype,
                     rope_base, stream);
}

size_t loki_decode_workspace_size(int32_t B, int32_t Hq, int32_t S_max, int32_t D, int32_t k_max) {
  if (B <= 0 || Hq <= 0 || D <= 0 || S_max <= 0) return 0;
  return workspace_bytes(B, Hq, D, S_max, k_max < 1 ? 1 : k_max);
}

int loki_decode_path(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d, int32_t S,
                     int32_t k, int32_t dtype, int32_t path) {
  int st = check_shape(B < 1 ? 1 : B, Hq, Hkv, D, d, S, S, dtype);
  if (st != LOKI_OK) return st;
  if (k < 1) return LOKI_EINVAL;
  const int kk = std::min(k, S);
  if (path == LOKI_PATH_SPLIT) return LOKI_PATH_SPLIT;
  if (path == LOKI_PATH_FUSED || path == LOKI_PATH_SLICED)
    return fused_fits(D, S, kk) ? path : LOKI_EUNSUPPORTED;
  if (path == LOKI_PATH_UNION) return union_ok(Hq, Hkv, S) ? LOKI_PATH_UNION : LOKI_EUNSUPPORTED;
  if (path != LOKI_PATH_AUTO) return LOKI_EINVAL;
  return auto_path(B, Hq, Hkv, D, d, S, kk, dtype);
}


int loki_decode_ex(const void* q, const void* k_slab, const void* k_rest, const void* v,
                   const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                   int32_t S, int32_t S_max, int32_t k, int32_t dtype, float* out, int32_t* idx,
                   void* workspace, size_t ws_bytes, int32_t path, void* stream) {
  return decode_impl(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, k, dtype, out, idx,
                     workspace, ws_bytes, path, loki::Rope(), stream);
}

int loki_decode_rope(const void* q, const void* k_slab, const void* k_rest, const void* v,
                     const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                     int32_t S, int32_t S_max, int32_t k, int32_t dtype, int32_t q_pos,
                     double rope_base, float* out, int32_t* idx, void* workspace,
                     size_t ws_bytes, int32_t path, void* stream) {
  if (!rope_ok(rope_base) || q_pos < 0) return LOKI_EINVAL;
  loki::Rope rope;
  rope.base = rope_base;
  rope.pos = q_pos;
  return decode_impl(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, k, dtype, out, idx,
                     workspace, ws_bytes, path, rope, stream);
}

int loki_decode_step(const void* q, const void* k_new, const void* v_new, const float* P,
                     void* k_slab, void* k_rest, void* v, int32_t B, int32_t Hq, int32_t Hkv,
                     int32_t D, int32_t d, int32_t pos, int32_t S_max, int32_t k, int32_t dtype,
                     float* out, int32_t* idx, void* workspace, size_t ws_bytes, int32_t path,
                     void* stream) {
  return step_impl(q, k_new, v_new, P, k_slab, k_rest, v, B, Hq, Hkv, D, d, pos, S_max, k, dtype,
                   out, idx, workspace, ws_bytes, path, 0.0, stream);
}

int loki_decode_step_rope(const void* q, const void* k_new, const void* v_new, const float* P,
                          void* k_slab, void* k_rest, void* v, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t d, int32_t pos, int32_t S_max, int32_t k,
                          int32_t dtype, double rope_base, float* out, int32_t* idx,
                          void* workspace, size_t ws_bytes, int32_t path, void* stream) {
  if (!rope_ok(rope_base)) return LOKI_EINVAL;
  return step_impl(q, k_new, v_new, P, k_slab, k_rest, v, B, Hq, Hkv, D, d, pos, S_max, k, dtype,
                   out, idx, workspace, ws_bytes, path, rope_base, stream);
}

int loki_decode(const void* q, const void* k_slab, const void* k_rest, const void* v,
                const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                int32_t S, int32_t S_max, int32_t k, int32_t dtype, float* out, int32_t* idx,
                void* workspace, size_t ws_bytes, void* stream) {
  return loki_decode_ex(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, k, dtype, out, idx,
                        workspace, ws_bytes, LOKI_PATH_AUTO, stream);
}

int loki_decode_noalloc(const void* q, const void* k_slab, const void* k_rest, const void* v,
                        const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                        int32_t S, int32_t S_max, int32_t k, int32_t dtype, float* out,
                        int32_t* idx, int32_t path, void* stream) {
  // argument checks first: a rejected call touches no device
  int st = check_shape(B, Hq, Hkv, D, d, S, S_max, dtype);
  if (st != LOKI_OK) return st;
  if (k < 1 || !valid_path(path)) return LOKI_EINVAL;
  const int kk = std::min(k, S);
  const int resolved = path == LOKI_PATH_AUTO ? auto_path(B, Hq, Hkv, D, d, S, kk, dtype) : path;
  if (resolved == LOKI_PATH_UNION && !union_ok(Hq, Hkv, S)) return LOKI_EUNSUPPORTED;
  if (B == 0) return LOKI_OK;
  if (resolved != LOKI_PATH_FUSED &&
      split_layout(B, Hq, Hkv, D, S, S_max, kk, resolved == LOKI_PATH_UNION).total > kNoallocScratch)
    return LOKI_EWORKSPACE;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != LOKI_OK) return st;
  return decode_impl(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, k, dtype, out, idx, ws,
                     kNoallocScratch, resolved, loki::Rope(), stream);
}

int loki_scores(const void* q, const void* k_slab, const float* P, int32_t B, int32_t Hq,
                int32_t Hkv, int32_t D, int32_t d, int32_t S, int32_t S_max, int32_t dtype,
                float* scores, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(B, Hq, Hkv, D, d, S, S_max, dtype);
  if (st != LOKI_OK) return st;
  if (B == 0) return LOKI_OK;
  if (!q || !k_slab || !P || !scores) return LOKI_EINVAL;
  if (!aligned16(k_slab) || !aligned16(P) || !aligned16(scores)) return LOKI_EINVAL;
  const Layout L = layout(B, Hq, D, S_max, 1);
  if (!workspace || ws_bytes < L.scores || !aligned16(workspace)) return LOKI_EWORKSPACE;
  DecodeArgs a = make_args(q, k_slab, nullptr, k_slab, P, B, Hq, Hkv, D, d, S, S_max, dtype,
                           nullptr, nullptr, stream);
  float* qrot = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.qrot);
  hipError_t e = loki::launch_scores(a, qrot, scores);
  return status_of(e);
}

int loki_topk(const float* scores, int32_t rows, int32_t S, int32_t ld, int32_t k, int32_t* idx,
              void* stream) {
  if (rows < 0 || S < 1 || ld < S || k < 1) return LOKI_EINVAL;
  if (rows == 0) return LOKI_OK;
  if (!scores || !idx || !aligned16(scores) || (ld % 4) != 0) return LOKI_EINVAL;
  if (reinterpret_cast<uintptr_t>(idx) & 3u) return LOKI_EINVAL;
  return status_of(loki::launch_topk(scores, rows, S, ld, std::min(k, S), idx,
                                     static_cast<hipStream_t>(stream)));
}

int loki_attend_indices(const void* q, const void* k_slab, const void* k_rest, const void* v,
                        const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                        int32_t S, int32_t S_max, const int32_t* idx, int32_t k, int32_t dtype,
                        float* out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(B, Hq, Hkv, D, d, S, S_max, dtype);
  if (st != LOKI_OK) return st;
  if (k < 1 || k > S) return LOKI_EINVAL;
  if (B == 0) return LOKI_OK;
  if (!q || !out || !idx) return LOKI_EINVAL;
  st = check_cache_ptrs(k_slab, k_rest, v, P, D, d);
  if (st != LOKI_OK) return st;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(idx) & 3u)) return LOKI_EINVAL;
  const int rows = B * Hq;
  const int nsplit = sparse_nsplit(rows, k);
  const Layout L = layout(B, Hq, D, S_max, nsplit);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return LOKI_EWORKSPACE;
  DecodeArgs a = make_args(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, dtype, out,
                           const_cast<int32_t*>(idx), stream);
  char* ws = static_cast<char*>(workspace);
  float* qrot = reinterpret_cast<float*>(ws + L.qrot);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  float* part = reinterpret_cast<float*>(ws + L.part);
  hipError_t e = loki::launch_scores(a, qrot, scores);
  if (e == hipSuccess) e = loki::launch_attend(a, qrot, scores, idx, k, part, nsplit, true);
  return status_of(e);
}

int loki_dense_decode(const void* q, const void* k_slab, const void* k_rest, const void* v,
                      const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                      int32_t S, int32_t S_max, int32_t dtype, float* out, void* workspace,
                      size_t ws_bytes, void* stream) {
  return dense_impl(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, dtype, out, workspace,
                    ws_bytes, loki::Rope(), stream);
}

int loki_dense_decode_rope(const void* q, const void* k_slab, const void* k_rest, const void* v,
                           const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t d, int32_t S, int32_t S_max, int32_t dtype, int32_t q_pos,
                           double rope_base, float* out, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (!rope_ok(rope_base) || q_pos < 0) return LOKI_EINVAL;
  loki::Rope rope;
  rope.base = rope_base;
  rope.pos = q_pos;
  return dense_impl(q, k_slab, k_rest, v, P, B, Hq, Hkv, D, d, S, S_max, dtype, out, workspace,
                    ws_bytes, rope, stream);
}

int loki_stream_read(const void* buf, size_t bytes, float* sink, int32_t workgroups,
                     void* stream) {
  if (workgroups < 1 || workgroups > 65536 || bytes % 16 != 0) return LOKI_EINVAL;
  if (bytes == 0) return LOKI_OK;
  if (!buf || !sink || !aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return LOKI_EINVAL;
  return status_of(loki::launch_stream_read(buf, bytes, sink, workgroups,
                                            static_cast<hipStream_t>(stream)));
}

int loki_stream_read_shares(const void* buf, size_t bytes, float* sink, int32_t workgroups,
                            int32_t threads, int32_t loads, void* stream) {
  if (workgroups < 1 || workgroups > 65536) return LOKI_EINVAL;
  if (threads != 256 && threads != 512 && threads != 1024) return LOKI_EINVAL;
  if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16) return LOKI_EINVAL;
  if (bytes % (16ull * static_cast<size_t>(workgroups)) != 0) return LOKI_EINVAL;
  if (bytes == 0) return LOKI_OK;
  if (!buf || !sink || !aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return LOKI_EINVAL;
  return status_of(loki::launch_share_read(buf, bytes, sink, workgroups, threads, loads,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"
