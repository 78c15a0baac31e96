/*
 * loki.h -- C ABI of libloki.so: Loki decode-step sparse attention on AMD
 * MI355X (gfx950).
 *
 * The method (web pages titled "Loki: Low-rank Keys for Efficient Sparse
 * Attention": the AI-extracted summary, sections "Approach" and the summary
 * line, and the arXiv "Abstract"): keys live in the cache already projected
 * onto a PCA basis P calibrated offline; the decode query is projected by the
 * same P; every cached token is ranked by a score computed from only the
 * leading d principal dimensions; the k best tokens are kept and exact
 * softmax attention runs over them; nothing is ever evicted from the cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller allocates and owns every buffer.  The library keeps no
 *   state between calls, allocates no device memory and is thread-safe.
 * Streams: `stream` is a hipStream_t passed as void* (NULL: the default
 *   stream).  All device work is enqueued asynchronously on it; no entry point
 *   synchronises.  Device pointers must stay valid until that work finishes.
 * Errors: every call returns a loki_status.  Arguments are checked on the
 *   host before anything is launched; a rejected call has no side effects.
 *   LOKI_EDEVICE means a HIP launch reported an error (the outputs are then
 *   undefined).  Nothing is thrown across the ABI.
 * Element types: `dtype` is LOKI_F32 or LOKI_BF16 (bf16 = the upper 16 bits of
 *   an IEEE float32) and applies to q, k_new, v_new and the three cache
 *   tensors.  P, out and scores are always float32; idx is int32.
 * Shapes (all tensors dense, row-major, last index fastest):
 *   q        [B, Hq, D]              decode queries (unrotated)
 *   P        [Hkv, D, D]  float32    P[g][m][c]: component m of principal
 *                                    axis c of KV head g; columns orthonormal,
 *                                    variance descending.  The rotated
 *                                    vector is x' = x . P, i.e.
 *                                    x'[c] = sum_m x[m] * P[g][m][c].
 *   k_slab   [B, Hkv, S_max, d]      rotated keys, dimensions 0..d-1
 *   k_rest   [B, Hkv, S_max, D-d]    rotated keys, dimensions d..D-1
 *                                    (may be NULL when d == D)
 *   v        [B, Hkv, S_max, D]      values (not rotated)
 *   out      [B, Hq, D]   float32
 *   idx      [B, Hq, k_eff] int32    k_eff = min(k, S); ascending token ids
 * Query head h reads KV head h / (Hq / Hkv) (consecutive grouping).
 * Supported: D in {64, 128}; 1 <= d <= D with d * sizeof(element) a multiple
 *   of 16 bytes; Hq a multiple of Hkv; 1 <= S <= S_max; k >= 1 (k > S keeps
 *   all S tokens).  Device pointers must be 16-byte aligned (idx: 4-byte).
 *   B == 0 is a no-op that returns LOKI_OK.  Inputs must be finite.
 */
#ifndef LOKI_H
#define LOKI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOKI_OK = 0,
  LOKI_EINVAL = -1,       /* bad argument: null pointer, bad size, misalignment */
  LOKI_EWORKSPACE = -2,   /* workspace missing or smaller than required        */
  LOKI_EDEVICE = -3,      /* a HIP launch failed                               */
  LOKI_EUNSUPPORTED = -4  /* valid but unsupported shape / dtype               */
} loki_status;

typedef enum { LOKI_F32 = 0, LOKI_BF16 = 1 } loki_dtype;

/* Execution path of loki_decode_ex.  AUTO picks one by shape and dtype
 * (loki_decode_path reports which).  FUSED runs one kernel per (sequence,
 * query head) that scores, selects and attends with the scores held in LDS
 * (requires (D + S + min(k, S)) * 4 bytes <= 56 KiB).  It needs no
 * workspace; given one (at least loki_decode_workspace_size), with four
 * query heads per KV head on a bf16 cache of D = 128, d <= 64 and S a
 * multiple of 16, the four query heads' workgroups share the ranking of
 * their KV head's slab (each scores a quarter of the tokens for all four
 * and they exchange the scores through the workspace), with the same
 * result.  SLICED is FUSED with
 * some rows split over several workgroups ("slices"): the slices of a row
 * each rank a share of its tokens and exchange the scores through the
 * workspace, each selects the whole row and gathers a share of the kept
 * tokens, and the row's last slice merges the shares, all in one launch.
 * Rows are sliced when there are fewer rows (B * Hq) than the GPU's 256
 * compute units (enough slices to spread the rows evenly over them), and
 * past whole rounds of 256 rows a remainder of at most 64 rows (rows a
 * multiple of 8), sliced to give every compute unit one more workgroup;
 * otherwise SLICED runs as FUSED.  It needs the workspace whenever it
 * slices.  SPLIT runs separate score, selection and attention kernels
 * through the workspace; its attention reads each query head's kept rows,
 * with the query heads of one KV head scheduled together so that rows
 * several of them kept are served from cache.  UNION is SPLIT with a
 * grouped-query gather (Hq/Hkv of 2 or 4, S <= 131072, else
 * LOKI_EUNSUPPORTED): per KV head and position range, the union of its
 * query heads' kept tokens is loaded once and all heads' products are
 * formed over it (on the matrix cores for bf16 caches).  For rows of at
 * most 4096 tokens the SPLIT and UNION paths rank and select in one launch
 * (the selecting workgroups wait for the ranking workgroups of their row).
 * The workspace's first bytes hold the flags and epochs of these hand-overs
 * within a launch, which any contents of a fresh workspace leave valid.
 * AUTO, where FUSED's LDS fits: SLICED when it slices and S >= 2048, else
 * FUSED when rows * S + 420000 >= 190 * S.  Otherwise UNION for bf16 caches
 * with d >= D - 96 when, even for independently selecting heads, the
 * union, a fraction 1 - (1 - k/S)^G of the positions, is at most 3/4 of
 * the G*k/S per-head reads; else SPLIT.  All paths compute the same
 * function. */
typedef enum {
  LOKI_PATH_AUTO = 0,
  LOKI_PATH_FUSED = 1,
  LOKI_PATH_SPLIT = 2,
  LOKI_PATH_UNION = 3,
  LOKI_PATH_SLICED = 4
} loki_path;

/* Human-readable name of a status code.  Never NULL. */
const char* loki_status_string(int status);

/* ABI revision of this header, incremented on any signature change; a caller
 * compares it with loki_abi_version() of the library it loaded. */
#define LOKI_ABI_VERSION 4

/* ABI revision the library was built with (LOKI_ABI_VERSION of its header). */
int loki_abi_version(void);

/* Offline PCA of sample keys (host only, no device work).  The pages state
 * that the basis is calibrated offline (summary line; "Approach": keys and
 * queries are PCA-projected).
 *   keys        host [n, D] float32, n >= 2
 *   P_out       host [D, D] float32: eigenvectors of the centred sample
 *               covariance (divisor n-1) as columns, eigenvalues descending,
 *               each column's sign chosen so that its largest-magnitude entry
 *               (lowest index among equal magnitudes) is positive
 *   eigvals_out host [D] float64 or NULL
 * Accumulates in float64; cyclic Jacobi eigensolver.  Any D >= 1. */
int loki_calibrate(const float* keys, int64_t n, int32_t D, float* P_out, double* eigvals_out);

/* Append T tokens per (sequence, KV head) at cache positions pos..pos+T-1:
 * each key is rotated into the PCA basis (x' = x . P[g], accumulated in
 * float64, rounded once to the cache dtype, ties to even), its leading d
 * dimensions stored in k_slab and the rest in k_rest; values are copied
 * unchanged ("Approach": queries and keys are PCA-projected; cache entries
 * are never deleted).
 *   k_new, v_new  device [B, Hkv, T, D] dtype
 *   requires 0 <= pos, pos + T <= S_max; T == 0 is a no-op. */
int loki_kv_append(const void* k_new, const void* v_new, const float* P,
                   void* k_slab, void* k_rest, void* v,
                   int32_t B, int32_t Hkv, int32_t D, int32_t d, int32_t S_max,
                   int32_t pos, int32_t T, int32_t dtype, void* stream);

/* Bytes of device workspace that every decode-family entry point below needs
 * for these sizes (any S <= S_max, any k <= k_max, any Hkv dividing Hq).
 * Always a multiple of 256; 0 when B, Hq, S_max or D is not positive.
 * (ABI 4 put S_max before D; ABI 3 took D first.) */
size_t loki_decode_workspace_size(int32_t B, int32_t Hq, int32_t S_max, int32_t D, int32_t k_max);

/* One Loki decode step ("Approach"; "Abstract": ranking and selection by
 * attention scores computed in the low-dimensional space; summary line:
 * exact attention over the selected keys):
 *   q' = q . P[g]
 *   s_j = sum_{i<d} q'_i * k_slab[j, i]                 for j < S
 *   I   = the k_eff tokens with the largest s_j, equal scores to the lower j,
 *         written to idx in ascending order
 *   e_j = (q' . [k_slab[j] | k_rest[j]]) / sqrt(D)      for j in I
 *   out = sum_{j in I} softmax_I(e)_j * v[j]
 * Ranking scores are float32 sums of the stored keys times q' (float32);
 * accumulation is float32 throughout.  workspace: device, 16-byte aligned,
 * >= loki_decode_workspace_size(B, Hq, S_max, D, k) bytes; the fused path
 * does not touch it (loki_decode_ex with LOKI_PATH_FUSED accepts NULL). */
int loki_decode(const void* q, const void* k_slab, const void* k_rest, const void* v,
                const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                int32_t S, int32_t S_max, int32_t k, int32_t dtype,
                float* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                void* stream);

/* loki_decode with an explicit execution path (loki_path).  FUSED returns
 * LOKI_EUNSUPPORTED when its LDS limit is exceeded.  Both paths compute the
 * same function; AUTO never needs workspace beyond the size above. */
int loki_decode_ex(const void* q, const void* k_slab, const void* k_rest, const void* v,
                   const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                   int32_t S, int32_t S_max, int32_t k, int32_t dtype,
                   float* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                   int32_t path, void* stream);

/* One step of a generation loop, in one call: append each sequence's new
 * key/value at position pos exactly as loki_kv_append does with T = 1, then
 * decode exactly as loki_decode_ex does over S = pos + 1 tokens.  The pages
 * time decode with the append excluded ("Key results"); here the append is
 * folded into the decode launch on the fused path (each workgroup rotates the
 * new key with the basis it loads for the query, one workgroup per KV head
 * writes the slot, and the new token's score and rows are taken from LDS
 * rather than re-read).  The split path runs the append kernel first.
 *   k_new, v_new  device [B, Hkv, D] dtype (one token per sequence and KV head)
 *   requires 0 <= pos < S_max; other arguments as loki_decode_ex (the
 *   workspace rule is the same; the fused path ignores it). */
int loki_decode_step(const void* q, const void* k_new, const void* v_new, const float* P,
                     void* k_slab, void* k_rest, void* v, int32_t B, int32_t Hq, int32_t Hkv,
                     int32_t D, int32_t d, int32_t pos, int32_t S_max, int32_t k, int32_t dtype,
                     float* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                     int32_t path, void* stream);

/* The path loki_decode_ex would take for these sizes, cache dtype and
 * `path`: the resolved loki_path (FUSED, SPLIT or UNION), or a negative
 * status for invalid sizes or a FUSED / UNION request these sizes do not
 * allow.  Host only. */
int loki_decode_path(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d, int32_t S,
                     int32_t k, int32_t dtype, int32_t path);

/* The ranking pass alone: scores [B, Hq, S] float32 (device) receives s_j as
 * defined for loki_decode.  Same workspace rule. */
int loki_scores(const void* q, const void* k_slab, const float* P,
                int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                int32_t S, int32_t S_max, int32_t dtype, float* scores,
                void* workspace, size_t workspace_bytes, void* stream);

/* The selection alone: for each of `rows` score rows (device float32, row r
 * at scores + r * ld, S entries), writes the min(k, S) indices of the largest
 * scores, equal scores to the lower index, ascending, to idx + r * min(k, S).
 * -0.0 ranks equal to +0.0.  Requires ld >= S, 16-byte aligned scores and ld
 * a multiple of 4. */
int loki_topk(const float* scores, int32_t rows, int32_t S, int32_t ld, int32_t k,
              int32_t* idx, void* stream);

/* Exact attention over caller-chosen tokens: idx [B, Hq, k] int32 (device),
 * each row strictly ascending with entries in [0, S); out as loki_decode with
 * I = that row.  Same workspace rule (with k_max >= k). */
int loki_attend_indices(const void* q, const void* k_slab, const void* k_rest, const void* v,
                        const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                        int32_t d, int32_t S, int32_t S_max, const int32_t* idx, int32_t k,
                        int32_t dtype, float* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Dense ("vanilla") decode attention over all S tokens of the same rotated
 * cache, the baseline the pages compare Loki with ("Key results"):
 * out = softmax(q' . K'^T / sqrt(D)) . V with K' = [k_slab | k_rest].  Reads
 * each KV head's keys and values once for all its query heads.  Same
 * workspace rule. */
int loki_dense_decode(const void* q, const void* k_slab, const void* k_rest, const void* v,
                      const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                      int32_t S, int32_t S_max, int32_t dtype, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- Rotary position embedding (RoPE) variant ----------------------------
 *
 * The pages evaluate Loki on models whose attention uses rotary position
 * embeddings, and find a basis calibrated on keys before the embedding
 * ("pre-rotary") better than one calibrated after it, although attention
 * uses the embedded keys either way ("Measured effects", "Surprising
 * findings").  These entry points apply the embedding inside the library:
 * each key is embedded at its cache position before its PCA rotation, and
 * the query at q_pos before its own.  Pre- or post-rotary is only a choice of
 * the keys given to loki_calibrate.  The embedding turns dims i and i + D/2
 * together by the angle pos * rope_base^(-2i/D), computed in float64 (the
 * pages name RoPE but not its form; this is the Llama-family pairing).
 * rope_base must be finite and > 0 (10000 for Llama2, 500000 for Llama3) and
 * q_pos >= 0, else LOKI_EINVAL.  A cache must be filled with the _rope
 * append (same base) for these decodes to mean attention over embedded
 * keys; the library cannot tell. */

/* loki_kv_append, embedding new token t at position pos + t first. */
int loki_kv_append_rope(const void* k_new, const void* v_new, const float* P,
                        void* k_slab, void* k_rest, void* v,
                        int32_t B, int32_t Hkv, int32_t D, int32_t d, int32_t S_max,
                        int32_t pos, int32_t T, int32_t dtype, double rope_base, void* stream);

/* loki_decode_ex with the query embedded at position q_pos (usually S - 1,
 * the position of the token being generated). */
int loki_decode_rope(const void* q, const void* k_slab, const void* k_rest, const void* v,
                     const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                     int32_t S, int32_t S_max, int32_t k, int32_t dtype, int32_t q_pos,
                     double rope_base, float* out, int32_t* idx, void* workspace,
                     size_t workspace_bytes, int32_t path, void* stream);

/* loki_decode_step with the new key and the query both embedded at pos. */
int loki_decode_step_rope(const void* q, const void* k_new, const void* v_new, const float* P,
                          void* k_slab, void* k_rest, void* v, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t d, int32_t pos, int32_t S_max,
                          int32_t k, int32_t dtype, double rope_base, float* out, int32_t* idx,
                          void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/* loki_dense_decode with the query embedded at position q_pos. */
int loki_dense_decode_rope(const void* q, const void* k_slab, const void* k_rest, const void* v,
                           const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t d, int32_t S, int32_t S_max, int32_t dtype, int32_t q_pos,
                           double rope_base, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---- Decode without allocation ---------------------------------------------
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): this
 * variant of loki_decode_ex takes no workspace.  Its sliced, split and
 * union paths use instead a scratch array that the library holds in device
 * memory, one copy of LOKI_NOALLOC_SCRATCH_BYTES per GPU it runs on, from
 * the first call on that GPU (which looks up the array's address with that
 * GPU current; later calls allocate nothing and call no allocating routine)
 * until the process ends.  The GPU is the current device, which must be the
 * one `stream` belongs to.  No result depends on the scratch's contents at
 * entry.  Every call on a GPU shares that GPU's array, so calls whose work overlaps
 * on one GPU (different streams, different host threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe.
 * Arguments, path choice and results are those of loki_decode_ex; sizes
 * whose workspace (loki_decode_workspace_size for the resolved path) would
 * exceed LOKI_NOALLOC_SCRATCH_BYTES return LOKI_EWORKSPACE with nothing
 * launched (32 MiB covers every benchmark shape: e.g. 128 rows of 32768
 * tokens need about 18 MB).  The fused path uses no scratch. */
#define LOKI_NOALLOC_SCRATCH_BYTES (32u << 20)

int loki_decode_noalloc(const void* q, const void* k_slab, const void* k_rest, const void* v,
                        const float* P, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t d,
                        int32_t S, int32_t S_max, int32_t k, int32_t dtype, float* out,
                        int32_t* idx, int32_t path, void* stream);

/* Measurement helper, not part of the method: reads `bytes` of device memory
 * at buf (16-byte aligned, bytes a multiple of 16) with nontemporal 16-byte
 * loads in a grid-stride loop of `workgroups` workgroups of 256 threads, and
 * writes one float per thread (the sum of what it read) to sink (device,
 * workgroups * 256 floats).  Timing it gives the HBM read rate a plain
 * streaming kernel reaches on the device, the practical ceiling next to the
 * published peak.  1 <= workgroups <= 65536. */
int loki_stream_read(const void* buf, size_t bytes, float* sink, int32_t workgroups, void* stream);

/* Measurement helper, not part of the method: the read pattern of a kernel
 * that gives each workgroup one row.  Each of `workgroups` workgroups of
 * `threads` threads (256, 512 or 1024) reads its own contiguous share of
 * bytes / workgroups bytes at buf with nontemporal 16-byte loads, `loads`
 * (1, 2, 4, 8 or 16) in flight per lane, and writes one float per thread (the
 * sum of what it read) to sink (device, workgroups * threads floats).  Timing
 * it at a decode launch's grid and bytes gives the floor a plain stream of
 * that shape reaches.  buf 16-byte aligned; bytes a multiple of
 * 16 * workgroups; 1 <= workgroups <= 65536; otherwise LOKI_EINVAL. */
int loki_stream_read_shares(const void* buf, size_t bytes, float* sink, int32_t workgroups,
                            int32_t threads, int32_t loads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOKI_H */
