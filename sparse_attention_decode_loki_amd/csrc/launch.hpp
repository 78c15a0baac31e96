// Internal interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cmath>

namespace loki {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr size_t kTopkLdsMax = 136 * 1024;   // scores staged in LDS up to this size
constexpr size_t kFusedLdsMax = 56 * 1024;   // fused path: q' + scores + kept ids (dynamic LDS)

// Rotary position embedding of the query before its PCA rotation: base 0
// means none; pos is the query's position.
struct Rope {
  double base = 0.0;
  int pos = 0;
};

struct DecodeArgs {
  const void* q;
  const void* k_slab;
  const void* k_rest;
  const void* v;
  const float* P;
  int B, Hq, Hkv, D, d, S, S_max;
  int dtype;
  float* out;
  int* idx;
  hipStream_t stream;
  Rope rope;
  // workspace words of the combined ranking + top-k launch: [0] epoch, [1]
  // given-up waits, [2 ..) flags (kScoreSelectFlags per row); nullptr where
  // that launch is not used
  unsigned long long* sync = nullptr;
};

// The combined ranking + top-k launch takes rows of up to this many scores,
// with at most kScoreSelectFlags ranking chunks per row.
constexpr int kScoreSelectMaxS = 4096;
constexpr int kScoreSelectFlags = 16;

hipError_t launch_rotate(const DecodeArgs& a, float* qrot);
// rotates the queries itself (q' of every query head also stored to qrot)
hipError_t launch_scores(const DecodeArgs& a, float* qrot, float* scores);
// the ranking pass and the top-k in one launch (a.S <= kScoreSelectMaxS,
// a.sync set): scores, a.idx and, when bits is given, the kept-position
// bitmaps, as launch_scores followed by launch_topk would write them
hipError_t launch_score_select(const DecodeArgs& a, float* qrot, float* scores, int kk,
                               unsigned* bits);
// bits (optional): also write each row's kept-position bitmap, ceil(S/32)
// words per row, bit j%32 of word j/32 set when token j is kept
hipError_t launch_topk(const float* scores, int rows, int S, int64_t ld, int k, int* idx,
                       hipStream_t stream, unsigned* bits = nullptr);
// sparse: attention over idx (k_eff = kk per row, scores from `scores`);
// dense: over all S tokens.  nsplit > 1 writes `part` and combines into out.
hipError_t launch_attend(const DecodeArgs& a, const float* qrot, const float* scores,
                         const int* idx, int kk, float* part, int nsplit, bool sparse);
// grouped-query sparse attention over the union of the G = Hq/Hkv heads' kept
// tokens (G in {2, 4}), read from their kept-position bitmaps; nsplit position
// ranges of at most kUnionMaxTok tokens
constexpr int kUnionMaxTok = 1024;
// longest context the union gather takes (bitmap row in LDS: S/8 bytes)
constexpr int kUnionMaxS = 1 << 17;
hipError_t launch_attend_union(const DecodeArgs& a, const float* qrot, const float* scores,
                               const unsigned* bits, float* part, int nsplit);
size_t fused_lds_bytes(int D, int S, int kk);
// How the single-kernel path splits rows over workgroups.  Rows [0, nfull)
// (in the kernel's head-major launch order) take one workgroup each; every
// later row takes nsl (at most kCoopMaxSlices with coop), each gathering
// 1/nsl of its kept tokens.  Without coop (nfull must be 0) every slice
// ranks and selects the whole row, partials go to part [B*Hq][nsl][D + 2]
// and a combine launch merges them.  With coop the slices of a row rank a
// share of its tokens each and exchange the scores through xsc [B*Hq][S],
// and the row's last slice merges the partials (part [sliced rows][nsl]
// [D + 2]) itself; sync holds 1 + kCoopStride words per sliced row (any
// contents are valid).  With nfull > 0 the grid, nfull and the sliced rows
// are multiples of 8.
constexpr int kCoopMaxSlices = 16;
constexpr int kCoopStride = 1 + 2 * kCoopMaxSlices;
// Grouped ranking on the single-kernel decode and step (one workgroup per row): the
// kGrpHeads query heads of a KV head share the ranking of its slab, each
// scoring a quarter of the tokens for all four and exchanging the scores
// through xsc and sync (as coop slices do).  For bf16 caches with D = 128,
// d <= kGrpMaxD and S a multiple of 4 * kGrpHeads.
constexpr int kGrpHeads = 4;
constexpr int kGrpMaxD = 64;
struct FusedSlices {
  int nsl = 1;
  int nfull = 0;
  bool coop = false;
  int grp = 1;  // kGrpHeads: grouped ranking (nsl == 1, nfull == 0)
  float* part = nullptr;
  float* xsc = nullptr;
  unsigned long long* sync = nullptr;
};
hipError_t launch_fused(const DecodeArgs& a, int kk, const FusedSlices& fs = FusedSlices());
// append (k_new, v_new [B, Hkv, D]) at pos and decode over a.S = pos + 1;
// with a.rope.base > 0 the new key is embedded at pos (the query at
// a.rope.pos)
hipError_t launch_fused_step(const DecodeArgs& a, const void* k_new, const void* v_new, int pos,
                             int kk, const FusedSlices& fs = FusedSlices());
// log-sum-exp merge of nsplit slice partials [rows][nsplit][D + 2] into out
hipError_t launch_combine(const float* part, float* out, int rows, int D, int nsplit,
                          hipStream_t stream);

// rope_base > 0: new token t is embedded at position pos + t before rotating
hipError_t launch_append(const void* k_new, const void* v_new, const float* P, void* k_slab,
                         void* k_rest, void* v, int B, int Hkv, int D, int d, int S_max, int pos,
                         int T, int dtype, hipStream_t stream, double rope_base = 0.0);

// streaming read of bytes (multiple of 16) with nontemporal 16-byte loads;
// sink receives workgroups * 256 floats
hipError_t launch_stream_read(const void* buf, size_t bytes, float* sink, int workgroups,
                              hipStream_t stream);

// each of `workgroups` workgroups of `threads` threads (256, 512 or 1024)
// reads its own contiguous share, bytes / workgroups (a multiple of 16),
// with `loads` (1, 2, 4, 8 or 16) 16-byte loads in flight per lane; sink
// receives workgroups * threads floats
hipError_t launch_share_read(const void* buf, size_t bytes, float* sink, int workgroups,
                             int threads, int loads, hipStream_t stream);

}  // namespace loki
