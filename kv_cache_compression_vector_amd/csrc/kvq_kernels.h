// kvq_kernels.h — argument blocks and launchers of the gfx950 kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"

namespace kvq {

struct EncodeArgs {
  Tables tab;
  const uint16_t* x;        // bf16 rows
  int64_t ld;               // elements between rows
  int64_t n;                // vectors
  uint8_t* rec;             // records
  // outlier side list (outlier kernels only)
  uint32_t* ol_off;
  void* ol_idx;             // u8 entries for m <= 256, u16 above
  uint16_t* ol_val;
  int64_t ol_cap;
  // staged outlier entries of the matrix-core encode at m = 128 (workspace): per 16-vector
  // tile a flag (0: its entries are staged, in order, at tile * kOutlierStage) and the entries
  uint32_t* stg_flag;
  uint8_t* stg_idx;
  uint16_t* stg_val;
  // PCA projection (PCA kernels only)
  Basis pca;                // PCA kernels only
  // stored scale: 0 the norm; 1 matched norm; 2 inner-product preserving; 3 least squares
  int32_t scale_rule, pad2;
};

struct DecodeArgs {
  Tables tab;
  const uint8_t* rec;
  int64_t n;
  const uint32_t* ol_off;   // nullptr = no side list
  const void* ol_idx;       // u8 entries for m <= 256, u16 above
  const uint16_t* ol_val;
  int64_t ol_cap;
  void* y;
  int64_t ld;
  Basis pca;                // PCA kernels only
};

struct ScoreArgs {
  Tables tab;
  const uint16_t* q;
  int64_t q_sb, q_sh;
  const uint8_t* rec;
  int64_t rec_sb, rec_sh;   // in records
  int64_t T;
  float* s;
  int64_t s_sb, s_sh;
  int32_t B, Hq, Hkv, pad;
  Basis pca;                // PCA kernels only
};

// Decode attention over packed K and V: the K side is a score launch (query, K records and
// their strides, K tables, projection); V records share the K records' (batch, KV head, token)
// indexing. Blocks write per-wave partials (running max, sum, rotated accumulator) to `part`;
// a second kernel merges them into `out`.
struct AttendArgs {
  ScoreArgs k;
  Tables tv;                // V codec tables (Hadamard, coded length = head_dim)
  const uint8_t* vrec;
  float* part;
  float* out;
  int64_t o_sb, o_sh;       // in floats
  float scale, softcap;     // logit multiplier; softcap > 0: softcap * tanh(logit / softcap)
  int64_t chunk, chunks;    // tokens per block (multiple of 256) and blocks per (batch, KV head)
};

// One cache of an append/evict launch: rows [0, rows) of the concatenation (tail ring, new rows)
// are encoded into dst.
struct EvictCache {
  const uint16_t* tail;     // ring base
  const uint16_t* fresh;    // new rows
  uint8_t* dst;             // first record to write
  int64_t tail_cap, tail_head, tail_len;
  int64_t rows;             // multiple of 128
  int64_t row_begin;        // prefix over caches
};

constexpr int kMaxEvictCaches = 32;

struct EvictArgs {
  Tables tab;
  int32_t n_caches, pad;
  int64_t total_rows;
  int64_t D;
  EvictCache c[kMaxEvictCaches];
};

struct TailCopyCache {
  const uint16_t* src;      // first new row to keep
  uint16_t* ring;
  int64_t cap, first_slot;  // ring slot of src row 0
  int64_t rows;
  int64_t row_begin;
};

struct TailCopyArgs {
  int32_t n_caches, pad;
  int64_t total_rows;
  int64_t D;
  TailCopyCache c[kMaxEvictCaches];
};

hipError_t launch_encode(int m, int bits, bool sym, const EncodeArgs& a, hipStream_t st);
// Rotation on the matrix cores (coded length 128, or 64 without a scale rule; no outlier list).
bool encode_mx_supported(int m, int scale_rule);
// Outlier lists in three passes (count + records, offsets scan, entries); `part` holds
// scan_partials(n) u32 of workspace.
int64_t scan_partials(int64_t n);
// Outlier entries staged per 16-vector tile by the first pass at m = 128 (a tile with more
// entries is recomputed by the second pass), and the workspace bytes that staging takes after
// the scan partials (0 for other coded lengths).
constexpr int kOutlierStage = 128;
int64_t outlier_stage_bytes(int m, int64_t n);
hipError_t launch_encode_outliers3(int m, int bits, bool sym, const EncodeArgs& a, uint32_t* part,
                                   hipStream_t st);
hipError_t launch_encode_mx(int m, int bits, bool sym, const EncodeArgs& a, hipStream_t st);
// Coded length 256 and 512: the rotation's 32-point blocks on the matrix cores (no outlier list),
// for plain encode and for eviction.
bool encode_kron_supported(int m);
hipError_t launch_encode_kron(int m, int bits, bool sym, const EncodeArgs& a, hipStream_t st);
hipError_t launch_evict_kron(int m, int bits, bool sym, const EvictArgs& a, hipStream_t st);
// The coded-length-128 outlier passes on the matrix-core encode: OL = 1 records + per-vector
// counts into ol_off, OL = 2 (after the scan) the entries.
template <int OL>
hipError_t launch_t128_outlier_pass(int bits, bool sym, const EncodeArgs& a, hipStream_t st);
// The entries the first pass staged, copied into the CSR (after the scan).
hipError_t launch_outlier_copy(const EncodeArgs& a, hipStream_t st);
bool pca_shape_supported(int D, int r);
hipError_t launch_encode_pca(int D, int r, int bits, bool sym, const EncodeArgs& a, hipStream_t st);
hipError_t launch_decode_pca(int D, int r, int bits, bool bf16_out, const DecodeArgs& a,
                             hipStream_t st);
// proj: a projection codec (a.pca holds the decode basis), also when m == D.
hipError_t launch_decode(int D, int m, bool proj, int bits, bool outliers, bool bf16_out,
                         const DecodeArgs& a, hipStream_t st);
// Hadamard decode with the 32-point blocks of the inverse rotation on the matrix cores.
bool decode_h_supported(int D, int m, bool outliers);
hipError_t launch_decode_h(int m, int bits, bool bf16_out, const DecodeArgs& a, hipStream_t st);
// Projection decode with the same split rotation feeding the unprojection from registers.
bool decode_pca_h_supported(int D, int r);
hipError_t launch_decode_pca_h(int D, int r, int bits, bool bf16_out, const DecodeArgs& a,
                               hipStream_t st);
hipError_t launch_score(int D, int m, bool proj, int bits, int group, const ScoreArgs& a, hipStream_t st);
// Attention: token chunk per block for (pairs, T), and the partial floats the launch writes.
int64_t attend_chunk(int64_t pairs, int64_t T);
int64_t attend_partial_floats(int64_t pairs, int64_t T, int D);
bool attend_supported(int D, int mk, bool proj, int bk, int bv);
hipError_t launch_attend(int D, int mk, bool proj, int bk, int bv, const AttendArgs& a, hipStream_t st);
hipError_t launch_evict(int m, int bits, bool sym, const EvictArgs& a, hipStream_t st);
hipError_t launch_tail_copy(const TailCopyArgs& a, hipStream_t st);
hipError_t launch_clear_u32(uint32_t* p, int64_t n_words, hipStream_t st);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t st);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_stream_fill(void* dst, int64_t bytes, uint32_t value, hipStream_t st);
// Lloyd-Max refit pass: per-block sums and counts of z in each cell of a.tab's table
// (fit_blocks(m, n) blocks, 2^bits floats and u32 each).
int64_t fit_blocks(int m, int64_t n);
hipError_t launch_fit_cells(int m, int bits, const EncodeArgs& a, float* part_sum, uint32_t* part_cnt,
                            hipStream_t st);

}  // namespace kvq
