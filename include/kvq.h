/*
 * kvq.h — C ABI of the MI355X (gfx950) KV-cache vector codec.
 *
 * The codec works on one head_dim row ("vector") of a K or V cache at a time:
 *   norm      n = ||v||_2, stored as f32 inside the record
 *             [arc PR #98 "TurboQuant KV storage for DeepSeek-V4", section "What landed"];
 *   rotation  u = H_m (s (.) v), H_m the unnormalised Sylvester Hadamard matrix and s a seeded
 *             +-1 diagonal [kakeyaturbo PR #15 "v1.3 PPL on vLLM", commits "M4 Phase A" and
 *             "M4 Phase B"]; optionally v = B^T (x - mu) first, a rank-r PCA projection
 *             ["M4 Phase A", "M5"];
 *   scale     z = u / n, i.e. unit-variance units ["M4 Phase B"];
 *   quantize  code_i = #{k : z_i > t_k}, t_k the midpoints of a Gaussian Lloyd-Max table at b bits
 *             ["M4 Phase A"; larql PR #196, turbo-quant commit: one N(0,1) table per bit width];
 *   pack      b bit-planes of the codes + f32 norm = m*b/8 + 4 bytes per record (260 B at
 *             head_dim 512, 4 bits) [arc PR #98, "What landed" bytes table];
 *   outliers  optional sparse (coordinate, value) list for |z_i| > T, applied at decode before
 *             the inverse rotation [PR #15, calibrated Lloyd-Max + outlier commit and "M5"].
 * Its inverse, a rotated-domain score q.k over packed K, and a two-region cache (bf16 tail +
 * packed history) with chunked eviction [arc PR #98, "Eviction is chunked, on purpose"]
 * complete the library.
 *
 * Record format v1 (little-endian), for coded length m (m = head_dim, or proj_rank with PCA)
 * and b bits:
 *   plane position of coordinate i:  pi(i) = (i mod 8) * (m/8) + floor(i/8)
 *   word[g*b + p], g in [0, m/32), p in [0, b): bit j = bit p of the code of the coordinate
 *                                              whose plane position is 32*g + j
 *   then one f32: the norm n.  Record size = m*b/8 + 4 bytes, always a multiple of 4.
 * Records of n vectors are stored back to back (stride = kvq_record_bytes()).
 *
 * Conventions for every call below.
 *  - Pointers named *_dev are device memory (HIP), *_host host memory. The caller owns all of
 *    them; the library allocates nothing and keeps no device state, except the static scratch
 *    array of kvq_attend_packed_static (one per device).
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously;
 *    argument errors are detected on the host before anything is enqueued and nothing is then
 *    launched. A launch failure maps to KVQ_E_DEVICE.
 *  - All sizes and offsets are 64-bit.
 *  - On error, kvq_last_error() (thread-local) names the offending argument and value.
 *  - Rows of bf16 input must start 16-byte aligned: the base pointer 16-byte aligned and
 *    leading dimensions multiples of 8 elements. Records must be 4-byte aligned.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_E_NULL = 1,       /* a required pointer is NULL                                    */
  KVQ_E_DIM = 2,        /* head_dim / proj_rank not supported                            */
  KVQ_E_BITS = 3,       /* bits outside 1..4                                             */
  KVQ_E_CENTROIDS = 4,  /* custom table not strictly ascending or not finite             */
  KVQ_E_STRIDE = 5,     /* misaligned pointer or leading dimension                       */
  KVQ_E_OUTLIER = 6,    /* outlier request invalid (T < 0, projection codec, missing buffers) */
  KVQ_E_CAPACITY = 7,   /* a capacity is too small (outlier list, cache region, workspace) */
  KVQ_E_CACHE = 8,      /* cache struct not built by kvq_cache_init, or built for another codec */
  KVQ_E_DEVICE = 9,     /* HIP launch / runtime error                                    */
  KVQ_E_ARG = 10        /* any other invalid argument (negative size, unknown flags, ...) */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

/* The f32 scale a record stores, chosen by codec->flags & KVQ_SCALE_RULE_MASK. Decode computes
 * x^ = (scale/m) s (.) H z^ whatever the rule, so only encode changes [turboquant_plus log: the
 * EDEN scales and the matched-norm scale]:
 *   KVQ_SCALE_NORM     ||v||                          (the default)
 *   KVQ_SCALE_MATCHED  ||v|| sqrt(m) / ||z^||          ||x^|| = ||v||
 *   KVQ_SCALE_INNER    ||v|| m / <z, z^>               <x^, v> = ||v||^2 (inner-product preserving)
 *   KVQ_SCALE_LSQ      ||v|| <z, z^> / ||z^||^2        <v - x^, x^> = 0 (least-squares optimal)
 * with z = H (s (.) v) / ||v|| and z^ the chosen centroids. A rule whose denominator is not
 * positive stores ||v||. Rules other than KVQ_SCALE_NORM need a Hadamard codec (proj_rank 0)
 * without outlier list, and caches use KVQ_SCALE_NORM. */
#define KVQ_SCALE_NORM 0u
#define KVQ_SCALE_MATCHED 1u
#define KVQ_SCALE_INNER 2u
#define KVQ_SCALE_LSQ 3u
#define KVQ_SCALE_RULE_MASK 3u

/* Codec descriptor: caller-owned POD in host memory. */
typedef struct kvq_codec {
  uint32_t head_dim;          /* D in {64, 128, 256, 512}                                    */
  uint32_t bits;              /* b in 1..4                                                   */
  uint32_t proj_rank;         /* 0: rotate all D coordinates (m = D).
                                 r in {32, 64, 128}, r < D, D*r <= 32768, or r = D for D in
                                 {64, 128}: projection to r coordinates v = B^T (x - mu) (MFMA),
                                 then rotation over r (m = r). Projection codecs carry no
                                 outlier list.                                               */
  uint32_t flags;             /* bits 0..1: the stored scale (KVQ_SCALE_*); other bits 0     */
  uint64_t seed;              /* seed of the +-1 sign diagonal (SplitMix64 stream)           */
  float outlier_T;            /* 0: no side list. > 0: coordinates with |z| > T are listed.
                                 Units: rotated, normalised (z).                             */
  uint32_t reserved0;         /* must be 0                                                   */
  const float* centroids_host;   /* f32[2^b] strictly ascending, or NULL = Gaussian Lloyd-Max */
  const uint16_t* basis_dev;     /* PCA only: bf16 [basis_count][D][r] row-major; column j of
                                    basis k is its j-th basis vector                          */
  const float* mean_dev;         /* PCA only: f32 [basis_count][D] means mu, or NULL = zero   */
  uint32_t basis_count;          /* PCA only: number of bases (0 or 1 = one basis for all rows) */
  uint32_t basis_block_rows;     /* PCA with basis_count > 1: rows are grouped in blocks of this
                                    many rows (a multiple of 256); block k uses basis
                                    basis_index_dev[k]. For the packed score the row of record
                                    (b, kv, t) is b*rec_sb + kv*rec_sh + t.                     */
  const int32_t* basis_index_dev;   /* PCA with basis_count > 1: int32 per block, in
                                       [0, basis_count); the caller guarantees it covers every
                                       block touched. The host never reads it (reading would
                                       need a synchronisation), so the kernels clamp an entry
                                       outside the range into it: a negative entry selects basis
                                       0, an entry >= basis_count selects basis basis_count - 1. */
  const uint16_t* unbasis_dev;   /* projection codecs only: bf16 [basis_count][D][r], the decode
                                    basis C (same layout and indexing as basis_dev). Decode gives
                                    x^ = mu + C v^, the packed score and attention use C^T q. NULL:
                                    C = B (an orthonormal PCA basis). Q-preconditioning
                                    [kakeyaturbo PR #15: the artefacts commit (K_tilde = K @ L for
                                    Sigma_q = L L^T), the full-recipe commit (whiten K before the
                                    codec, unwhiten after it) and "M6 Phase B.2a"] is the pair
                                    B = L B_w, C = L^-T B_w, mu = L^-T mu_w, with (B_w, mu_w) a fit
                                    in the whitened domain (B_w = I, mu_w = 0 and r = D for
                                    whitening alone): the transform costs no extra pass.        */
} kvq_codec;

/* Outlier side list, CSR by vector. Entry e of vector v is at offsets[v] + e; within a vector
 * entries are in ascending coordinate order. idx = coordinate index i in [0, m) of the rotated
 * vector, val = bf16 bits of z_i (round to nearest even). */
typedef struct kvq_outliers {
  uint32_t* offsets_dev;   /* [n+1]: written by kvq_encode, read by kvq_decode. offsets[n] is
                              the total count, which may exceed capacity (entries past
                              capacity are not written; kvq_decode ignores them)             */
  void* idx_dev;           /* [capacity] coordinate indices: u8 while the coded length m <= 256,
                              u16 (little-endian) for m = 512 [kakeyaturbo PR #15, calibrated
                              Lloyd-Max + outlier commit: u16 index]                          */
  uint16_t* val_dev;       /* [capacity]                                                     */
  int64_t capacity;        /* entries                                                        */
  void* workspace_dev;     /* encode only: scratch of kvq_encode_workspace_bytes() bytes,
                              16-byte aligned; contents need not be initialised              */
  int64_t workspace_bytes;
} kvq_outliers;

/* Two-region cache of one (layer, kv-head) stream [arc PR #98, "What landed"]: a bf16 ring
 * `tail` of the newest rows and a region `packed` of records of older rows. Lengths live on
 * the host, so no eviction decision needs a device->host synchronisation. Fields are written
 * only by the library; callers read them. */
typedef struct kvq_cache {
  uint64_t magic;          /* set by kvq_cache_init                                          */
  uint64_t codec_key;      /* fingerprint of the codec the cache was built for               */
  void* packed_dev;        /* records [packed_cap]                                            */
  int64_t packed_len, packed_cap;   /* in records (= tokens)                                 */
  void* tail_dev;          /* bf16 ring [tail_cap][D]                                         */
  int64_t tail_head;       /* ring slot of the oldest dense row                               */
  int64_t tail_len, tail_cap;       /* in rows                                               */
  int32_t window, margin;  /* retention floor = window + max(t_new - 1, margin)               */
} kvq_cache;

/* Number of tokens moved from the dense tail to the packed region per eviction step
 * [arc PR #98, "Eviction is chunked, on purpose": EVICT_CHUNK = 128]. */
#define KVQ_EVICT_CHUNK 128

/* Bytes of one record for this codec: m*b/8 + 4 (b bit-planes of m codes, then the f32 norm:
 * 260 B at head_dim 512 and 4 bits, the packed row of arc PR #98's "What landed" bytes table,
 * against 1,026 B for bf16). Returns 0 for an invalid codec. */
size_t kvq_record_bytes(const kvq_codec* codec);

/* Workspace bytes kvq_encode needs for n vectors when codec->outlier_T > 0 (0 otherwise): the
 * block sums of the scan that turns per-vector outlier counts into CSR offsets and, at coded
 * length 128, per 16-vector tile a flag and room for 128 entries (3 bytes each) that the first
 * pass stages so that the rows are read once (about 24.3 bytes per vector). */
size_t kvq_encode_workspace_bytes(const kvq_codec* codec, int64_t n);

/* Host copies of the tables the kernels use, for inspection and tests: centroids f32[2^b],
 * decision thresholds f32[2^b - 1] (f32 of the midpoints of adjacent centroids), and the sign
 * diagonal int8[m] (+1 / -1). Any output pointer may be NULL. */
kvq_status kvq_codec_tables(const kvq_codec* codec, float* centroids_host, float* thresholds_host,
                            int8_t* signs_host);

/* Encode n vectors. x_dev: bf16 [n][ld_x] (row i at x_dev + i*ld_x elements, first D used).
 * records_dev: n records. ol: required iff codec->outlier_T > 0, else must be NULL.
 * ol_total_host: optional; when non-NULL the call synchronises the stream, stores the total
 * outlier count and returns KVQ_E_CAPACITY if it exceeds ol->capacity.
 * With an outlier list the work is three kernels on the stream: records + per-vector counts
 * (into offsets_dev), an exclusive scan of the counts in place, then the entries.
 * [kakeyaturbo PR #15, commits "M4 Phase A", "M4 Phase B"; arc PR #98, "What landed"] */
kvq_status kvq_encode(const kvq_codec* codec, const void* x_dev, int64_t n, int64_t ld_x,
                      void* records_dev, const kvq_outliers* ol, int64_t* ol_total_host,
                      void* stream);

/* Lloyd-Max table refitted to the codec's own rotated, normalised coordinates z = H (s (.) x) /
 * ||x|| of n calibration rows x_dev (bf16 [n][ld_x]) [kakeyaturbo PR #15, calibration-artefacts
 * commit: the table refitted to post-rotation residuals lowers the MSE below the Gaussian
 * table's; larql PR #196, turbo-quant commit: Lloyd's conditions]. Starting from the codec's
 * table (Gaussian or custom), each of `iters` passes puts every coordinate in its cell of the
 * current table (the quantiser's decision, the f32 thresholds of the table), sums z and counts
 * per cell on the GPU (one kernel; partial sums per block in the caller's workspace of
 * kvq_fit_workspace_bytes(codec, n) bytes), and moves each centroid to its cell's mean (f64 sum
 * on the host, rounded to f32); an empty cell keeps its centroid. Writes the 2^b f32 centroids to
 * centroids_host: a table for the codec's centroids_host. Hadamard codecs (proj_rank 0); the
 * codec's outlier threshold and scale rule play no part. Synchronises the stream once per pass.
 * Returns KVQ_E_CENTROIDS if the result is not strictly ascending. */
size_t kvq_fit_workspace_bytes(const kvq_codec* codec, int64_t n);
kvq_status kvq_fit_table(const kvq_codec* codec, const void* x_dev, int64_t n, int64_t ld_x,
                         int32_t iters, float* centroids_host, void* workspace_dev,
                         size_t workspace_bytes, void* stream);

/* Decode n records into y_dev [n][ld_y] of dtype y_dtype (bf16: round to nearest even).
 * x^ = mu + B (n/m) s (.) H_m z^, with z^_i = centroid[code_i] or the outlier value.
 * ol: NULL, or the side list kvq_encode wrote for these records.
 * [kakeyaturbo PR #15, commit "M5"] */
kvq_status kvq_decode(const kvq_codec* codec, const void* records_dev, int64_t n,
                      const kvq_outliers* ol, void* y_dev, kvq_dtype y_dtype, int64_t ld_y,
                      void* stream);

/* Raw attention logits over packed K without materialising dense K
 * [arc PR #98 / #94 kernel commit: paged attention over packed K]:
 *   scores[b][h][t] = q[b][h] . decode(records[b][h / (Hq/Hkv)][t])
 * computed in the rotated domain as (n_t/m) * sum_i q'_i z^_{t,i}, q' = H_m (s (.) q) (with PCA
 * q' = H_r (s (.) B^T q) plus the constant q.mu). No 1/sqrt(D), softcap or softmax.
 * q_dev: bf16, element q[b][h][d] at q_dev + b*q_sb + h*q_sh + d.
 * records_dev: record (b, kv, t) at index b*rec_sb + kv*rec_sh + t.
 * scores_dev: f32, score (b, h, t) at scores_dev + b*s_sb + h*s_sh + t.
 * Hq must be a multiple of Hkv (query heads h*Hkv/Hq share kv head). Outlier lists are not
 * consulted (score requires codec->outlier_T == 0).
 * Accuracy: the products are formed in f16 with the query held to ~2^-22 and each centroid to
 * 2^-11 (both scaled by powers of two into the f16 range), so |error| <= ~5e-4 *
 * (n_t/m) sum_i |q'_i z^_{t,i}|, under the 1e-3 normwise bar on scores. */
kvq_status kvq_score_packed(const kvq_codec* codec, const void* q_dev, int32_t B, int32_t Hq,
                            int64_t q_sb, int64_t q_sh, const void* records_dev, int32_t Hkv,
                            int64_t T, int64_t rec_sb, int64_t rec_sh, float* scores_dev,
                            int64_t s_sb, int64_t s_sh, void* stream);

/* Decode attention over packed K and V, for the query heads of each (batch, KV head):
 *   out[b][h] = sum_t w_t decode_V(vrec[b][kv][t]),  w = softmax_t(l_t),
 *   l_t = softmax_scale * (q[b][h] . decode_K(krec[b][kv][t])), kv = h / (Hq/Hkv),
 * and, when softcap > 0, l_t = softcap * tanh(l_t / softcap) after the scale multiply and before
 * the maximum [arc PR #98 / #94 kernel commit: attention reads the packed cache; arc PR #98,
 * "Also: two silently-ignored kernel parameters"]. Neither K nor V is materialised: logits are
 * formed in the K codec's rotated domain, values are accumulated in the V codec's rotated
 * domain and rotated back once per query head.
 * kcodec: any codec kvq_score_packed accepts with head_dim 64 or 128 (projection ranks 32, 64,
 * or r = D).
 * vcodec: Hadamard (proj_rank 0), same head_dim, bits 1..3. Neither may carry an outlier list.
 * q_dev: bf16, row (b, h) at q_dev + b*q_sb + h*q_sh elements (16-byte aligned).
 * krec_dev / vrec_dev: record (b, kv, t) at index b*rec_sb + kv*rec_sh + t of each array.
 * out_dev: f32 [D] per (b, h) at out_dev + b*o_sb + h*o_sh floats.
 * workspace_dev: kvq_attend_workspace_bytes(vcodec, B, Hkv, T) bytes, 16-byte aligned, caller
 * owned, contents need not be initialised (per-block partial maxima, sums and accumulators).
 * T must be >= 1. Two kernels on the stream; no synchronisation. */
size_t kvq_attend_workspace_bytes(const kvq_codec* vcodec, int32_t B, int32_t Hkv, int64_t T);
kvq_status kvq_attend_packed(const kvq_codec* kcodec, const kvq_codec* vcodec, const void* q_dev,
                             int32_t B, int32_t Hq, int64_t q_sb, int64_t q_sh,
                             const void* krec_dev, const void* vrec_dev, int32_t Hkv, int64_t T,
                             int64_t rec_sb, int64_t rec_sh, float softmax_scale, float softcap,
                             float* out_dev, int64_t o_sb, int64_t o_sh, void* workspace_dev,
                             size_t workspace_bytes, void* stream);

/* kvq_attend_packed without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The per-block partials go to a static device array of KVQ_STATIC_SCRATCH_BYTES (16 MiB), one
 * per device, held from the first call on that device until the process ends; the call itself
 * allocates nothing and frees nothing. A call whose partials need more
 * (kvq_attend_workspace_bytes(vcodec, B, Hkv, T) > KVQ_STATIC_SCRATCH_BYTES, e.g. B*Hkv > 992 at
 * head_dim 128) returns KVQ_E_CAPACITY before anything is launched. Every other argument, the
 * result and the errors are those of kvq_attend_packed. All calls on one device share that
 * device's array, and the array keeps the last call's contents (every partial a call reads is
 * written by the same call first): calls that overlap on one device, on different streams or
 * from different threads, race and give undefined results. */
#define KVQ_STATIC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_attend_packed_static(const kvq_codec* kcodec, const kvq_codec* vcodec,
                                    const void* q_dev, int32_t B, int32_t Hq, int64_t q_sb,
                                    int64_t q_sh, const void* krec_dev, const void* vrec_dev,
                                    int32_t Hkv, int64_t T, int64_t rec_sb, int64_t rec_sh,
                                    float softmax_scale, float softcap, float* out_dev,
                                    int64_t o_sb, int64_t o_sh, void* stream);

/* Build an empty cache over caller-owned buffers: packed_dev holds packed_cap records,
 * tail_dev holds tail_cap bf16 rows of head_dim. window >= 0, margin >= 0. Host only.
 * Outlier lists are not supported in caches (codec->outlier_T must be 0).
 * The cache is the two-region layout of arc PR #98, "What landed": a dense bf16 tail of the
 * newest rows in front of a packed region of records, sized by the caller. The struct records a
 * fingerprint of the codec, so a cache this library did not build, or built for another codec,
 * is refused by every later call (KVQ_E_CACHE) [arc PR #98, "Refuse what we can't serve"]. */
kvq_status kvq_cache_init(const kvq_codec* codec, kvq_cache* cache, void* packed_dev,
                          int64_t packed_cap, void* tail_dev, int64_t tail_cap, int32_t window,
                          int32_t margin);

/* Append t_new bf16 rows (new_rows_dev[c]: [t_new][D] contiguous) to each of n_caches caches,
 * then evict whole chunks of KVQ_EVICT_CHUNK oldest dense rows into the packed region while
 *   tail_len >= window + max(t_new - 1, margin) + KVQ_EVICT_CHUNK
 * [arc PR #98, "What landed" (dense-tail bound) and "Mutation runs" (retention floor)].
 * t_new = 0 flushes. All caches must be built for `codec`; each decides its own eviction count.
 * Updates the host-side lengths; evicted_host (optional, int64[n_caches]) receives the chunks evicted per cache.
 * No device->host synchronisation. Errors (capacity, foreign cache) leave every cache as it was. */
kvq_status kvq_append_evict_chunk(const kvq_codec* codec, kvq_cache* const* caches,
                                  int32_t n_caches, const void* const* new_rows_dev,
                                  int64_t t_new, void* stream, int64_t* evicted_host);

/* Roll a cache back to its first new_len tokens (0 <= new_len <= packed_len + tail_len), e.g.
 * after rejected speculative tokens. Truncation maps onto both regions [arc PR #98, "What
 * landed": the cache reports its length in tokens and maps truncation onto both time bases]:
 *  - new_len >= packed_len: the dense tail keeps its oldest new_len - packed_len rows;
 *  - new_len < packed_len: the packed region keeps its first new_len records and the tail
 *    empties (the rolled-back tokens are gone from both regions; rows a caller needs dense again
 *    come from kvq_decode of the kept records).
 * The retention floor keeps `margin` dense rows beyond the window after every append, so a
 * rollback of at most margin + 1 tokens never reaches the packed region [arc PR #98, "Mutation
 * runs": the rollback margin]. Host only: lengths change, no device memory is touched and
 * nothing is enqueued. A cache not built for `codec` is refused (KVQ_E_CACHE). */
kvq_status kvq_cache_truncate(const kvq_codec* codec, kvq_cache* cache, int64_t new_len);

/* Message for the last error on this thread ("" if none): the failing call's argument and
 * value, e.g. "ld_x=100 is not a multiple of 8 elements". Errors are typed statuses with a
 * named cause, never a silent fallback [kakeyaturbo PR #15, "M2" commit: validation at the
 * boundary with typed errors; arc PR #98, "Query strides": validate, name and refuse]. The
 * pointer stays valid until the next call on the same thread. */
const char* kvq_last_error(void);

/* Streaming copy of `bytes` (a multiple of 16; both pointers 16-byte aligned) from src_dev to
 * dst_dev on `stream`: the plain copy kernel a measurement times next to the codec kernels, so
 * that its bandwidth figures can be checked against what a trivial kernel reaches on the same
 * device in the same run. Not part of the codec. */
kvq_status kvq_stream_copy(void* dst_dev, const void* src_dev, int64_t bytes, void* stream);

/* Streaming read of `bytes` (a multiple of 16; src_dev 16-byte aligned) on `stream`, folded by
 * XOR into the one u32 at sink_dev (4-byte aligned): afterwards *sink_dev holds its old value
 * XOR the XOR of every 32-bit word of the source. The caller sets *sink_dev first. The
 * read-only bandwidth control of a measurement, beside kvq_stream_copy and kvq_stream_fill;
 * not part of the codec. */
kvq_status kvq_stream_read(const void* src_dev, int64_t bytes, uint32_t* sink_dev, void* stream);

/* Streaming fill of `bytes` (a multiple of 16; dst_dev 16-byte aligned) with the 32-bit `value`
 * on `stream`: the write-only bandwidth control of a measurement. Not part of the codec. */
kvq_status kvq_stream_fill(void* dst_dev, int64_t bytes, uint32_t value, void* stream);

/* ABI version of this header; record format version. */
#define KVQ_ABI_VERSION 1
#define KVQ_RECORD_FORMAT 1
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
