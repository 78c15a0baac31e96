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
};

hipError_t launch_rotate(const DecodeArgs& a, float* qrot);
// rotates the queries itself (q' of every query head also stored to qrot)
hipError_t launch_scores(const DecodeArgs& a, float* qrot, float* scores);
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
hipError_t launch_fused(const DecodeArgs& a, int kk);
// append (k_new, v_new [B, Hkv, D]) at pos and decode over a.S = pos + 1;
// with a.rope.base > 0 the new key is embedded at pos (the query at
// a.rope.pos)
hipError_t launch_fused_step(const DecodeArgs& a, const void* k_new, const void* v_new, int pos,
                             int kk);

// rope_base > 0: new token t is embedded at position pos + t before rotating
hipError_t launch_append(const void* k_new, const void* v_new, const float* P, void* k_slab,
                         void* k_rest, void* v, int B, int Hkv, int D, int d, int S_max, int pos,
                         int T, int dtype, hipStream_t stream, double rope_base = 0.0);

// streaming read of bytes (multiple of 16) with nontemporal 16-byte loads;
// sink receives workgroups * 256 floats
hipError_t launch_stream_read(const void* buf, size_t bytes, float* sink, int workgroups,
                              hipStream_t stream);

}  // namespace loki
