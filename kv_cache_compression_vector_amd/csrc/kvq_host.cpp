// kvq_host.cpp — the C ABI: argument validation, codec tables, dispatch to the gfx950 kernels.
//
// The library keeps no device state and allocates no device memory: tables travel as kernel
// arguments, scratch comes from the caller. Every error is reported before anything is
// enqueued, as a typed status plus a thread-local message naming the argument and its value
// (refusal instead of silent fallback: arc PR #98, "Two refusals rather than fallbacks";
// kakeyaturbo PR #15, "M2" commit: validate at the boundary).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/kvq.h"
#include "kvq_kernels.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

kvq_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVQ_E_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------------------------
// Gaussian Lloyd-Max tables. Lloyd's optimality conditions for N(0,1): boundaries are midpoints
// of adjacent centroids and each centroid is the mean of N(0,1) over its cell,
// (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)); iterated to a fixed point (one table per bit width:
// larql PR #196 turbo-quant commit; kakeyaturbo PR #15 "M4 Phase A" centroids_gaussian).

double normal_pdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.3989422804014327; }

// Probability of (a, b) under N(0,1), taken from whichever tail keeps it accurate.
double normal_cell_mass(double a, double b) {
  const double r2 = 0.7071067811865476;
  if (a >= 0.0) return 0.5 * (std::erfc(a * r2) - std::erfc(b * r2));
  if (b <= 0.0) return 0.5 * (std::erfc(-b * r2) - std::erfc(-a * r2));
  return 1.0 - 0.5 * std::erfc(b * r2) - 0.5 * std::erfc(-a * r2);
}

struct GaussTable {
  bool ready = false;
  float c[16];
};

GaussTable g_gauss[5];
std::mutex g_gauss_mu;

const float* gaussian_centroids(int bits) {
  std::lock_guard<std::mutex> lk(g_gauss_mu);
  GaussTable& gt = g_gauss[bits];
  if (gt.ready) return gt.c;
  const int L = 1 << bits;
  double c[16], edge[17];
  for (int k = 0; k < L; ++k) c[k] = 6.0 * (k + 0.5) / L - 3.0;
  for (int iter = 0; iter < 200000; ++iter) {
    edge[0] = -INFINITY;
    edge[L] = INFINITY;
    for (int k = 1; k < L; ++k) edge[k] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      const double nc = (normal_pdf(edge[k]) - normal_pdf(edge[k + 1])) /
                        normal_cell_mass(edge[k], edge[k + 1]);
      delta = std::fmax(delta, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta < 1e-14) break;
  }
  for (int k = 0; k < L / 2; ++k) {  // exact antisymmetry
    const double h = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -h;
    c[L - 1 - k] = h;
  }
  for (int k = 0; k < L; ++k) gt.c[k] = (float)c[k];
  gt.ready = true;
  return gt.c;
}

// Sign diagonal: SplitMix64 (Steele, Lea & Flood 2014) — state += golden-ratio increment, the
// output mix applied to the state; s_i = -1 when the top bit of output i is set.
uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ---------------------------------------------------------------------------------------------
// Codec validation

struct Resolved {
  int D, m, bits, L, rule;
  bool pca, sym, outliers;
  kvq::Tables tab;
  kvq::Basis basis;    // encode side: v = B^T (x - mu)
  kvq::Basis unbasis;  // decode side (decode, score, attention): x^ = mu + C v^
};

bool is_pow2_in(uint32_t v, uint32_t lo, uint32_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

kvq_status resolve_codec(const kvq_codec* cd, Resolved& r) {
  if (!cd) return fail(KVQ_E_NULL, "codec is NULL");
  if (!is_pow2_in(cd->head_dim, 64, 512))
    return fail(KVQ_E_DIM, "head_dim=%u not supported (64, 128, 256, 512)", cd->head_dim);
  if (cd->bits < 1 || cd->bits > 4) return fail(KVQ_E_BITS, "bits=%u outside 1..4", cd->bits);
  if (cd->flags & ~KVQ_SCALE_RULE_MASK)
    return fail(KVQ_E_ARG, "flags=%u: only the scale-rule bits (0x%x) may be set", cd->flags,
                (unsigned)KVQ_SCALE_RULE_MASK);
  r.rule = (int)(cd->flags & KVQ_SCALE_RULE_MASK);
  if (cd->reserved0 != 0) return fail(KVQ_E_ARG, "reserved0=%u must be 0", cd->reserved0);
  r.D = (int)cd->head_dim;
  r.bits = (int)cd->bits;
  r.L = 1 << r.bits;
  r.pca = cd->proj_rank != 0;
  std::memset(&r.basis, 0, sizeof(r.basis));
  if (r.pca) {
    if (!kvq::pca_shape_supported((int)cd->head_dim, (int)cd->proj_rank))
      return fail(KVQ_E_DIM, "proj_rank=%u with head_dim=%u not supported (r in {32,64,128}, r < D, "
                  "D*r <= 32768, or r = D for D in {64,128})", cd->proj_rank, cd->head_dim);
    if (!cd->basis_dev) return fail(KVQ_E_NULL, "proj_rank=%u needs basis_dev", cd->proj_rank);
    if (cd->basis_count > 1) {
      if (!cd->basis_index_dev)
        return fail(KVQ_E_NULL, "basis_count=%u needs basis_index_dev", cd->basis_count);
      if (cd->basis_block_rows == 0 || cd->basis_block_rows % 256)
        return fail(KVQ_E_ARG, "basis_block_rows=%u must be a positive multiple of 256", cd->basis_block_rows);
    }
    r.basis.basis = cd->basis_dev;
    r.basis.mean = cd->mean_dev;
    r.basis.index = cd->basis_count > 1 ? cd->basis_index_dev : nullptr;
    r.basis.count = cd->basis_count > 1 ? (int32_t)cd->basis_count : 1;
    r.basis.block_rows = cd->basis_count > 1 ? (int32_t)cd->basis_block_rows : 0;
  } else if (cd->basis_count > 1) {
    return fail(KVQ_E_ARG, "basis_count=%u without proj_rank", cd->basis_count);
  } else if (cd->unbasis_dev) {
    return fail(KVQ_E_ARG, "unbasis_dev needs a projection codec (proj_rank > 0)");
  }
  r.unbasis = r.basis;
  if (r.pca && cd->unbasis_dev) r.unbasis.basis = cd->unbasis_dev;
  r.m = r.pca ? (int)cd->proj_rank : r.D;
  if (!(cd->outlier_T >= 0.0f) || std::isinf(cd->outlier_T))
    return fail(KVQ_E_OUTLIER, "outlier_T=%g must be finite and >= 0", (double)cd->outlier_T);
  r.outliers = cd->outlier_T > 0.0f;
  if (r.outliers && r.pca)
    return fail(KVQ_E_OUTLIER, "projection codecs carry no outlier list (proj_rank=%u, outlier_T=%g)",
                cd->proj_rank, (double)cd->outlier_T);
  if (r.rule != 0 && (r.pca || r.outliers))
    return fail(KVQ_E_ARG, "scale rule %d needs a Hadamard codec without outlier list "
                "(proj_rank=%u, outlier_T=%g)", r.rule, cd->proj_rank, (double)cd->outlier_T);
  std::memset(&r.tab, 0, sizeof(r.tab));
  const float* c = cd->centroids_host ? cd->centroids_host : gaussian_centroids(r.bits);
  for (int k = 0; k < r.L; ++k) {
    if (!std::isfinite(c[k]))
      return fail(KVQ_E_CENTROIDS, "centroids[%d]=%g is not finite", k, (double)c[k]);
    if (k > 0 && !(c[k] > c[k - 1]))
      return fail(KVQ_E_CENTROIDS, "centroids not strictly ascending at %d (%g <= %g)", k,
                  (double)c[k], (double)c[k - 1]);
    r.tab.c[k] = c[k];
  }
  for (int k = 0; k + 1 < r.L; ++k)
    r.tab.t[k] = (float)(0.5 * ((double)c[k] + (double)c[k + 1]));
  r.sym = true;
  for (int k = 0; k < r.L; ++k)
    if (c[r.L - 1 - k] != -c[k]) r.sym = false;
  uint64_t st = cd->seed;
  for (int i = 0; i < r.m; ++i)
    if (splitmix64_next(st) >> 63) {
      r.tab.sign_words[i >> 5] |= 1u << (i & 31);
      r.tab.sign_pairs[i >> 1] |= (i & 1) ? 0x80000000u : 0x8000u;
    }
  r.tab.T = cd->outlier_T;
  r.tab.inv_m = 1.0f / (float)r.m;
  return ok();
}

size_t record_bytes(const Resolved& r) { return (size_t)r.m * r.bits / 8 + 4; }

// Fingerprint of everything that changes the bytes a cache holds.
uint64_t codec_key(const kvq_codec* cd, const Resolved& r) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&](const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 0x100000001b3ull;
  };
  mix(&cd->head_dim, 4);
  mix(&cd->bits, 4);
  mix(&cd->proj_rank, 4);
  mix(&cd->seed, 8);
  mix(&cd->outlier_T, 4);
  mix(&cd->flags, 4);
  mix(r.tab.c, sizeof(float) * r.L);
  return h;
}

constexpr uint64_t kCacheMagic = 0x4b56514341434845ull;  // "KVQCACHE"

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device address of the static scratch array on the current device (see below), looked up once
// per device with that device current.
kvq_status static_scratch_address(void** out);

}  // namespace

// ---- Static scratch of the allocation-free attention entry point ----------------------------
// One array per device, held until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: every use goes through the address hipGetSymbolAddress returns
// for the current device.
static __device__ __align__(256) unsigned char scratch[KVQ_STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

kvq_status static_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KVQ_E_DEVICE, "device %d outside 0..63", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(KVQ_E_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_stream_copy(void* dst_dev, const void* src_dev, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(KVQ_E_ARG, "bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
  if (bytes == 0) return ok();
  if (!dst_dev || !src_dev) return fail(KVQ_E_NULL, "dst_dev or src_dev is NULL");
  if (!aligned(dst_dev, 16) || !aligned(src_dev, 16)) return fail(KVQ_E_STRIDE, "copy pointers must be 16-byte aligned");
  return from_hip(kvq::launch_stream_copy(dst_dev, src_dev, bytes, static_cast<hipStream_t>(stream)), "stream_copy");
}

kvq_status kvq_stream_read(const void* src_dev, int64_t bytes, uint32_t* sink_dev, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(KVQ_E_ARG, "bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
  if (bytes == 0) return ok();
  if (!src_dev || !sink_dev) return fail(KVQ_E_NULL, "src_dev or sink_dev is NULL");
  if (!aligned(src_dev, 16) || !aligned(sink_dev, 4)) return fail(KVQ_E_STRIDE, "src_dev must be 16-byte and sink_dev 4-byte aligned");
  return from_hip(kvq::launch_stream_read(src_dev, bytes, sink_dev, static_cast<hipStream_t>(stream)), "stream_read");
}

kvq_status kvq_stream_fill(void* dst_dev, int64_t bytes, uint32_t value, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(KVQ_E_ARG, "bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
  if (bytes == 0) return ok();
  if (!dst_dev) return fail(KVQ_E_NULL, "dst_dev is NULL");
  if (!aligned(dst_dev, 16)) return fail(KVQ_E_STRIDE, "dst_dev must be 16-byte aligned");
  return from_hip(kvq::launch_stream_fill(dst_dev, bytes, value, static_cast<hipStream_t>(stream)), "stream_fill");
}

size_t kvq_record_bytes(const kvq_codec* codec) {
  Resolved r;
  if (resolve_codec(codec, r) != KVQ_OK) return 0;
  return record_bytes(r);
}

size_t kvq_encode_workspace_bytes(const kvq_codec* codec, int64_t n) {
  Resolved r;
  if (resolve_codec(codec, r) != KVQ_OK || n < 0) return 0;
  if (!r.outliers) return 0;
  // the scan's block sums, then (coded length 128) the entries staged per 16-vector tile
  return (size_t)(16 + 4 * kvq::scan_partials(n) + 16 + kvq::outlier_stage_bytes(r.m, n));
}

kvq_status kvq_codec_tables(const kvq_codec* codec, float* centroids_host,
                            float* thresholds_host, int8_t* signs_host) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (centroids_host) std::memcpy(centroids_host, r.tab.c, sizeof(float) * r.L);
  if (thresholds_host) std::memcpy(thresholds_host, r.tab.t, sizeof(float) * (r.L - 1));
  if (signs_host)
    for (int i = 0; i < r.m; ++i)
      signs_host[i] = ((r.tab.sign_words[i >> 5] >> (i & 31)) & 1u) ? (int8_t)-1 : (int8_t)1;
  return ok();
}

kvq_status kvq_encode(const kvq_codec* codec, const void* x_dev, int64_t n, int64_t ld_x,
                      void* records_dev, const kvq_outliers* ol, int64_t* ol_total_host,
                      void* stream) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (n < 0) return fail(KVQ_E_ARG, "n=%lld is negative", (long long)n);
  if (ld_x < r.D) return fail(KVQ_E_STRIDE, "ld_x=%lld < head_dim=%d", (long long)ld_x, r.D);
  if (ld_x % 8) return fail(KVQ_E_STRIDE, "ld_x=%lld is not a multiple of 8 elements", (long long)ld_x);
  if (n > 0 && (!x_dev || !records_dev)) return fail(KVQ_E_NULL, "x_dev or records_dev is NULL");
  if (n > 0 && !aligned(x_dev, 16)) return fail(KVQ_E_STRIDE, "x_dev is not 16-byte aligned");
  if (n > 0 && !aligned(records_dev, 4)) return fail(KVQ_E_STRIDE, "records_dev is not 4-byte aligned");
  if (r.outliers) {
    if (!ol) return fail(KVQ_E_OUTLIER, "outlier_T=%g > 0 needs an outlier list", (double)codec->outlier_T);
    if (!ol->offsets_dev || (ol->capacity > 0 && (!ol->idx_dev || !ol->val_dev)))
      return fail(KVQ_E_NULL, "outlier list buffers are NULL");
    if (ol->capacity < 0) return fail(KVQ_E_OUTLIER, "outlier capacity=%lld < 0", (long long)ol->capacity);
    const size_t need = kvq_encode_workspace_bytes(codec, n);
    if (ol->workspace_bytes < (int64_t)need || !ol->workspace_dev)
      return fail(KVQ_E_CAPACITY, "outlier workspace %lld bytes < %zu needed",
                  (long long)ol->workspace_bytes, need);
    if (!aligned(ol->workspace_dev, 16)) return fail(KVQ_E_STRIDE, "workspace_dev is not 16-byte aligned");
  } else if (ol) {
    return fail(KVQ_E_OUTLIER, "outlier list given but outlier_T == 0");
  }
  if (ol_total_host && !r.outliers)
    return fail(KVQ_E_OUTLIER, "ol_total_host given but outlier_T == 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq::EncodeArgs a{};
  a.tab = r.tab;
  a.x = static_cast<const uint16_t*>(x_dev);
  a.ld = ld_x;
  a.n = n;
  a.rec = static_cast<uint8_t*>(records_dev);
  a.pca = r.basis;
  a.scale_rule = r.rule;
  if (!r.outliers) {
    if (n == 0) return ok();
    if (r.pca) return from_hip(kvq::launch_encode_pca(r.D, r.m, r.bits, r.sym, a, s), "encode_pca");
    return from_hip(kvq::launch_encode(r.m, r.bits, r.sym, a, s), "encode");
  }
  // outlier path: encode + counts, scan of the counts into offsets, entries
  uint32_t* ws = static_cast<uint32_t*>(ol->workspace_dev);
  a.ol_off = ol->offsets_dev;
  a.ol_idx = ol->idx_dev;
  a.ol_val = ol->val_dev;
  a.ol_cap = ol->capacity;
  hipError_t e;
  if (n == 0) {
    e = kvq::launch_clear_u32(ol->offsets_dev, 1, s);  // offsets[0] = 0
  } else {
    e = kvq::launch_encode_outliers3(r.m, r.bits, r.sym, a, ws + 4, s);
  }
  if (e != hipSuccess) return from_hip(e, "encode_outliers");
  if (ol_total_host) {
    uint32_t tot = 0;
    e = hipMemcpyAsync(&tot, ol->offsets_dev + n, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return from_hip(e, "encode outlier total");
    *ol_total_host = tot;
    if ((int64_t)tot > ol->capacity)
      return fail(KVQ_E_CAPACITY, "outlier count %u exceeds capacity %lld", tot, (long long)ol->capacity);
  }
  return ok();
}

size_t kvq_fit_workspace_bytes(const kvq_codec* codec, int64_t n) {
  Resolved r;
  if (resolve_codec(codec, r) != KVQ_OK || n <= 0 || r.pca) return 0;
  return (size_t)(kvq::fit_blocks(r.m, n) * r.L * 8);
}

kvq_status kvq_fit_table(const kvq_codec* codec, const void* x_dev, int64_t n, int64_t ld_x,
                         int32_t iters, float* centroids_host, void* workspace_dev,
                         size_t workspace_bytes, void* stream) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (r.pca) return fail(KVQ_E_ARG, "the refit needs a Hadamard codec (proj_rank=%u)", codec->proj_rank);
  if (n <= 0) return fail(KVQ_E_ARG, "n=%lld: the refit needs at least one row", (long long)n);
  if (iters < 0) return fail(KVQ_E_ARG, "iters=%d is negative", iters);
  if (!centroids_host) return fail(KVQ_E_NULL, "centroids_host is NULL");
  if (ld_x < r.D) return fail(KVQ_E_STRIDE, "ld_x=%lld < head_dim=%d", (long long)ld_x, r.D);
  if (ld_x % 8) return fail(KVQ_E_STRIDE, "ld_x=%lld is not a multiple of 8 elements", (long long)ld_x);
  if (!x_dev || !workspace_dev) return fail(KVQ_E_NULL, "x_dev or workspace_dev is NULL");
  if (!aligned(x_dev, 16)) return fail(KVQ_E_STRIDE, "x_dev is not 16-byte aligned");
  if (!aligned(workspace_dev, 16)) return fail(KVQ_E_STRIDE, "workspace_dev is not 16-byte aligned");
  const int64_t blocks = kvq::fit_blocks(r.m, n);
  if (workspace_bytes < (size_t)(blocks * r.L * 8))
    return fail(KVQ_E_CAPACITY, "workspace_bytes=%zu, need %lld", workspace_bytes, (long long)(blocks * r.L * 8));
  hipStream_t s = static_cast<hipStream_t>(stream);
  float table[16];
  std::memcpy(table, r.tab.c, sizeof(float) * r.L);
  float* part_sum = static_cast<float*>(workspace_dev);
  uint32_t* part_cnt = reinterpret_cast<uint32_t*>(part_sum + blocks * r.L);
  float* hs = new float[blocks * r.L];
  uint32_t* hc = new uint32_t[blocks * r.L];
  for (int it = 0; it < iters; ++it) {
    kvq_codec cur = *codec;
    cur.centroids_host = table;
    cur.outlier_T = 0.0f;
    Resolved rc;
    st = resolve_codec(&cur, rc);
    if (st != KVQ_OK) break;  // a pass that made the table non-ascending (cannot happen in exact
                              // arithmetic: Lloyd keeps the order) is reported, not used
    kvq::EncodeArgs a{};
    a.tab = rc.tab;
    a.x = static_cast<const uint16_t*>(x_dev);
    a.ld = ld_x;
    a.n = n;
    hipError_t e = kvq::launch_fit_cells(r.m, r.bits, a, part_sum, part_cnt, s);
    if (e == hipSuccess) e = hipMemcpyAsync(hs, part_sum, sizeof(float) * blocks * r.L, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(hc, part_cnt, sizeof(uint32_t) * blocks * r.L, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      st = from_hip(e, "fit_table");
      break;
    }
    for (int k = 0; k < r.L; ++k) {
      double sum = 0.0;
      uint64_t cnt = 0;
      for (int64_t b = 0; b < blocks; ++b) {
        sum += (double)hs[b * r.L + k];
        cnt += hc[b * r.L + k];
      }
      if (cnt > 0) table[k] = (float)(sum / (double)cnt);  // an empty cell keeps its centroid
    }
  }
  delete[] hs;
  delete[] hc;
  if (st != KVQ_OK) return st;
  for (int k = 1; k < r.L; ++k)
    if (!(table[k] > table[k - 1]))
      return fail(KVQ_E_CENTROIDS, "refitted table not strictly ascending at %d (%g <= %g)", k,
                  (double)table[k], (double)table[k - 1]);
  std::memcpy(centroids_host, table, sizeof(float) * r.L);
  return ok();
}

kvq_status kvq_decode(const kvq_codec* codec, const void* records_dev, int64_t n,
                      const kvq_outliers* ol, void* y_dev, kvq_dtype y_dtype, int64_t ld_y,
                      void* stream) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (n < 0) return fail(KVQ_E_ARG, "n=%lld is negative", (long long)n);
  if (y_dtype != KVQ_F32 && y_dtype != KVQ_BF16) return fail(KVQ_E_ARG, "y_dtype=%d unknown", (int)y_dtype);
  if (ld_y < r.D) return fail(KVQ_E_STRIDE, "ld_y=%lld < head_dim=%d", (long long)ld_y, r.D);
  if (ld_y % 8) return fail(KVQ_E_STRIDE, "ld_y=%lld is not a multiple of 8 elements", (long long)ld_y);
  if (n > 0 && (!records_dev || !y_dev)) return fail(KVQ_E_NULL, "records_dev or y_dev is NULL");
  if (n > 0 && !aligned(y_dev, 16)) return fail(KVQ_E_STRIDE, "y_dev is not 16-byte aligned");
  if (n > 0 && !aligned(records_dev, 4)) return fail(KVQ_E_STRIDE, "records_dev is not 4-byte aligned");
  if (ol && !r.outliers) return fail(KVQ_E_OUTLIER, "outlier list given but outlier_T == 0");
  if (ol && (!ol->offsets_dev || (ol->capacity > 0 && (!ol->idx_dev || !ol->val_dev))))
    return fail(KVQ_E_NULL, "outlier list buffers are NULL");
  if (n == 0) return ok();
  kvq::DecodeArgs a{};
  a.tab = r.tab;
  a.rec = static_cast<const uint8_t*>(records_dev);
  a.n = n;
  if (ol) {
    a.ol_off = ol->offsets_dev;
    a.ol_idx = ol->idx_dev;
    a.ol_val = ol->val_dev;
    a.ol_cap = ol->capacity;
  }
  a.y = y_dev;
  a.ld = ld_y;
  a.pca = r.unbasis;
  return from_hip(kvq::launch_decode(r.D, r.m, r.pca, r.bits, ol != nullptr, y_dtype == KVQ_BF16, a,
                                     static_cast<hipStream_t>(stream)),
                  "decode");
}

kvq_status kvq_score_packed(const kvq_codec* codec, const void* q_dev, int32_t B, int32_t Hq,
                            int64_t q_sb, int64_t q_sh, const void* records_dev, int32_t Hkv,
                            int64_t T, int64_t rec_sb, int64_t rec_sh, float* scores_dev,
                            int64_t s_sb, int64_t s_sh, void* stream) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (r.outliers) return fail(KVQ_E_OUTLIER, "score reads codes and norms only: outlier_T must be 0");
  if (B < 0 || Hq < 0 || Hkv < 0 || T < 0) return fail(KVQ_E_ARG, "negative size (B=%d Hq=%d Hkv=%d T=%lld)", B, Hq, Hkv, (long long)T);
  if (B == 0 || Hq == 0 || T == 0) return ok();
  if (Hkv == 0 || Hq % Hkv) return fail(KVQ_E_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int group = Hq / Hkv;
  if (group < 1 || group > 8) return fail(KVQ_E_ARG, "Hq/Hkv=%d not supported (1..8)", group);
  if (B * Hkv > 65535) return fail(KVQ_E_ARG, "B*Hkv=%d exceeds 65535", B * Hkv);
  if (!q_dev || !records_dev || !scores_dev) return fail(KVQ_E_NULL, "q_dev, records_dev or scores_dev is NULL");
  if (!aligned(q_dev, 16) || q_sb % 8 || q_sh % 8)
    return fail(KVQ_E_STRIDE, "q rows must be 16-byte aligned (q_sb=%lld, q_sh=%lld elements)", (long long)q_sb, (long long)q_sh);
  if (!aligned(records_dev, 4)) return fail(KVQ_E_STRIDE, "records_dev is not 4-byte aligned");
  if (!aligned(scores_dev, 4)) return fail(KVQ_E_STRIDE, "scores_dev is not 4-byte aligned");
  if (q_sb < 0 || q_sh < 0 || rec_sb < 0 || rec_sh < 0 || s_sb < 0 || s_sh < 0)
    return fail(KVQ_E_STRIDE, "negative stride");
  kvq::ScoreArgs a{};
  a.tab = r.tab;
  a.q = static_cast<const uint16_t*>(q_dev);
  a.q_sb = q_sb;
  a.q_sh = q_sh;
  a.rec = static_cast<const uint8_t*>(records_dev);
  a.rec_sb = rec_sb;
  a.rec_sh = rec_sh;
  a.T = T;
  a.s = scores_dev;
  a.s_sb = s_sb;
  a.s_sh = s_sh;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.pca = r.unbasis;
  if (r.pca && r.basis.count > 1 &&
      (r.basis.block_rows % 256 || rec_sb % 256 || rec_sh % 256))
    return fail(KVQ_E_STRIDE,
                "score with several bases needs basis_block_rows, rec_sb, rec_sh multiples of 256 "
                "(got %d, %lld, %lld)", r.basis.block_rows, (long long)rec_sb, (long long)rec_sh);
  return from_hip(kvq::launch_score(r.D, r.m, r.pca, r.bits, group, a, static_cast<hipStream_t>(stream)),
                  "score_packed");
}

size_t kvq_attend_workspace_bytes(const kvq_codec* vcodec, int32_t B, int32_t Hkv, int64_t T) {
  Resolved r;
  if (resolve_codec(vcodec, r) != KVQ_OK || B < 0 || Hkv < 0 || T < 0) return 0;
  if (B == 0 || Hkv == 0 || T == 0) return 0;
  return (size_t)(4 * kvq::attend_partial_floats((int64_t)B * Hkv, T, r.D));
}

kvq_status kvq_attend_packed(const kvq_codec* kcodec, const kvq_codec* vcodec, const void* q_dev,
                             int32_t B, int32_t Hq, int64_t q_sb, int64_t q_sh,
                             const void* krec_dev, const void* vrec_dev, int32_t Hkv, int64_t T,
                             int64_t rec_sb, int64_t rec_sh, float softmax_scale, float softcap,
                             float* out_dev, int64_t o_sb, int64_t o_sh, void* workspace_dev,
                             size_t workspace_bytes, void* stream) {
  Resolved rk, rv;
  kvq_status st = resolve_codec(kcodec, rk);
  if (st != KVQ_OK) return st;
  st = resolve_codec(vcodec, rv);
  if (st != KVQ_OK) return st;
  if (rk.outliers || rv.outliers)
    return fail(KVQ_E_OUTLIER, "attention reads codes and norms only: outlier_T must be 0 for K and V");
  if (rv.pca) return fail(KVQ_E_ARG, "the V codec must be Hadamard (proj_rank=0), got proj_rank=%u", vcodec->proj_rank);
  if (rk.D != rv.D) return fail(KVQ_E_DIM, "K head_dim=%d and V head_dim=%d differ", rk.D, rv.D);
  if (!kvq::attend_supported(rk.D, rk.m, rk.pca, rk.bits, rv.bits))
    return fail(KVQ_E_ARG, "attention supports head_dim 64/128, K coded length 32..D, K bits 1..4, V bits 1..3 "
                "(got D=%d, K m=%d b=%d, V b=%d)", rk.D, rk.m, rk.bits, rv.bits);
  if (B < 0 || Hq < 0 || Hkv < 0 || T < 0) return fail(KVQ_E_ARG, "negative size (B=%d Hq=%d Hkv=%d T=%lld)", B, Hq, Hkv, (long long)T);
  if (B == 0 || Hq == 0) return ok();
  if (T == 0) return fail(KVQ_E_ARG, "attention over T=0 tokens is undefined");
  if (Hkv == 0 || Hq % Hkv) return fail(KVQ_E_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int group = Hq / Hkv;
  if (group < 1 || group > 8) return fail(KVQ_E_ARG, "Hq/Hkv=%d not supported (1..8)", group);
  if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY || softmax_scale == -INFINITY)
    return fail(KVQ_E_ARG, "softmax_scale must be finite");
  if (!(softcap >= 0.0f) || softcap == INFINITY) return fail(KVQ_E_ARG, "softcap must be finite and >= 0 (0 = off)");
  if (!q_dev || !krec_dev || !vrec_dev || !out_dev || !workspace_dev)
    return fail(KVQ_E_NULL, "q_dev, krec_dev, vrec_dev, out_dev or workspace_dev is NULL");
  if (!aligned(q_dev, 16) || q_sb % 8 || q_sh % 8)
    return fail(KVQ_E_STRIDE, "q rows must be 16-byte aligned (q_sb=%lld, q_sh=%lld elements)", (long long)q_sb, (long long)q_sh);
  if (!aligned(krec_dev, 4) || !aligned(vrec_dev, 4)) return fail(KVQ_E_STRIDE, "records are not 4-byte aligned");
  if (!aligned(out_dev, 4)) return fail(KVQ_E_STRIDE, "out_dev is not 4-byte aligned");
  if (!aligned(workspace_dev, 16)) return fail(KVQ_E_STRIDE, "workspace_dev is not 16-byte aligned");
  if (q_sb < 0 || q_sh < 0 || rec_sb < 0 || rec_sh < 0 || o_sb < 0 || o_sh < 0)
    return fail(KVQ_E_STRIDE, "negative stride");
  const size_t need = kvq_attend_workspace_bytes(vcodec, B, Hkv, T);
  if (workspace_bytes < need)
    return fail(KVQ_E_ARG, "workspace_bytes=%zu, need %zu", workspace_bytes, need);
  if (rk.pca && rk.basis.count > 1 && (rk.basis.block_rows % 256 || rec_sb % 256 || rec_sh % 256))
    return fail(KVQ_E_STRIDE,
                "attention with several bases needs basis_block_rows, rec_sb, rec_sh multiples of 256 "
                "(got %d, %lld, %lld)", rk.basis.block_rows, (long long)rec_sb, (long long)rec_sh);
  kvq::AttendArgs a{};
  a.k.tab = rk.tab;
  a.k.q = static_cast<const uint16_t*>(q_dev);
  a.k.q_sb = q_sb;
  a.k.q_sh = q_sh;
  a.k.rec = static_cast<const uint8_t*>(krec_dev);
  a.k.rec_sb = rec_sb;
  a.k.rec_sh = rec_sh;
  a.k.T = T;
  a.k.B = B;
  a.k.Hq = Hq;
  a.k.Hkv = Hkv;
  a.k.pca = rk.unbasis;
  a.tv = rv.tab;
  a.vrec = static_cast<const uint8_t*>(vrec_dev);
  a.part = static_cast<float*>(workspace_dev);
  a.out = out_dev;
  a.o_sb = o_sb;
  a.o_sh = o_sh;
  a.scale = softmax_scale;
  a.softcap = softcap;
  return from_hip(kvq::launch_attend(rk.D, rk.m, rk.pca, rk.bits, rv.bits, a, static_cast<hipStream_t>(stream)),
                  "attend_packed");
}

kvq_status kvq_attend_packed_static(const kvq_codec* kcodec, const kvq_codec* vcodec,
                                    const void* q_dev, int32_t B, int32_t Hq, int64_t q_sb,
                                    int64_t q_sh, const void* krec_dev, const void* vrec_dev,
                                    int32_t Hkv, int64_t T, int64_t rec_sb, int64_t rec_sh,
                                    float softmax_scale, float softcap, float* out_dev,
                                    int64_t o_sb, int64_t o_sh, void* stream) {
  Resolved rv;
  kvq_status st = resolve_codec(vcodec, rv);
  if (st != KVQ_OK) return st;
  if (B > 0 && Hkv > 0 && T > 0) {
    const size_t need = kvq_attend_workspace_bytes(vcodec, B, Hkv, T);
    if (need > (size_t)KVQ_STATIC_SCRATCH_BYTES)
      return fail(KVQ_E_CAPACITY, "B=%d Hkv=%d T=%lld needs %zu bytes of partials; the static scratch "
                  "holds %zu (use kvq_attend_packed with a caller workspace)", B, Hkv, (long long)T,
                  need, (size_t)KVQ_STATIC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  st = static_scratch_address(&ws);
  if (st != KVQ_OK) return st;
  return kvq_attend_packed(kcodec, vcodec, q_dev, B, Hq, q_sb, q_sh, krec_dev, vrec_dev, Hkv, T,
                           rec_sb, rec_sh, softmax_scale, softcap, out_dev, o_sb, o_sh, ws,
                           (size_t)KVQ_STATIC_SCRATCH_BYTES, stream);
}

kvq_status kvq_cache_init(const kvq_codec* codec, kvq_cache* cache, void* packed_dev,
                          int64_t packed_cap, void* tail_dev, int64_t tail_cap, int32_t window,
                          int32_t margin) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (!cache) return fail(KVQ_E_NULL, "cache is NULL");
  if (r.outliers || r.pca || r.rule != 0)
    return fail(KVQ_E_ARG, "caches hold Hadamard records with the plain norm and no outlier list "
                "(proj_rank=%u, outlier_T=%g, flags=%u)", codec->proj_rank, (double)codec->outlier_T,
                codec->flags);
  if (packed_cap < 0 || tail_cap <= 0 || window < 0 || margin < 0)
    return fail(KVQ_E_ARG, "packed_cap=%lld tail_cap=%lld window=%d margin=%d", (long long)packed_cap,
                (long long)tail_cap, window, margin);
  if (!tail_dev || (packed_cap > 0 && !packed_dev)) return fail(KVQ_E_NULL, "cache buffers are NULL");
  if (!aligned(tail_dev, 16)) return fail(KVQ_E_STRIDE, "tail_dev is not 16-byte aligned");
  if (packed_dev && !aligned(packed_dev, 4)) return fail(KVQ_E_STRIDE, "packed_dev is not 4-byte aligned");
  std::memset(cache, 0, sizeof(*cache));
  cache->magic = kCacheMagic;
  cache->codec_key = codec_key(codec, r);
  cache->packed_dev = packed_dev;
  cache->packed_cap = packed_cap;
  cache->tail_dev = tail_dev;
  cache->tail_cap = tail_cap;
  cache->window = window;
  cache->margin = margin;
  return ok();
}

kvq_status kvq_cache_truncate(const kvq_codec* codec, kvq_cache* cache, int64_t new_len) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (!cache) return fail(KVQ_E_NULL, "cache is NULL");
  if (cache->magic != kCacheMagic) return fail(KVQ_E_CACHE, "cache was not built by kvq_cache_init");
  if (cache->codec_key != codec_key(codec, r)) return fail(KVQ_E_CACHE, "cache was built for another codec");
  const int64_t len = cache->packed_len + cache->tail_len;
  if (new_len < 0 || new_len > len)
    return fail(KVQ_E_ARG, "new_len=%lld outside [0, %lld] (packed %lld + dense %lld)", (long long)new_len,
                (long long)len, (long long)cache->packed_len, (long long)cache->tail_len);
  if (new_len >= cache->packed_len) {
    cache->tail_len = new_len - cache->packed_len;
  } else {
    cache->packed_len = new_len;
    cache->tail_len = 0;
  }
  return ok();
}

kvq_status kvq_append_evict_chunk(const kvq_codec* codec, kvq_cache* const* caches,
                                  int32_t n_caches, const void* const* new_rows_dev,
                                  int64_t t_new, void* stream, int64_t* evicted_host) {
  Resolved r;
  kvq_status st = resolve_codec(codec, r);
  if (st != KVQ_OK) return st;
  if (n_caches < 0 || t_new < 0) return fail(KVQ_E_ARG, "n_caches=%d t_new=%lld", n_caches, (long long)t_new);
  if (n_caches == 0) return ok();
  if (!caches) return fail(KVQ_E_NULL, "caches is NULL");
  if (t_new > 0 && !new_rows_dev) return fail(KVQ_E_NULL, "new_rows_dev is NULL with t_new=%lld", (long long)t_new);
  const uint64_t key = codec_key(codec, r);
  const int64_t rb = (int64_t)record_bytes(r);
  const int64_t C = KVQ_EVICT_CHUNK;
  // Plan every cache first; nothing is changed or launched unless all of them are valid.
  struct Plan { int64_t k, keep_from; };
  Plan* plan = new Plan[n_caches];
  for (int i = 0; i < n_caches; ++i) {
    const kvq_cache* c = caches[i];
    if (!c) { delete[] plan; return fail(KVQ_E_NULL, "caches[%d] is NULL", i); }
    if (c->magic != kCacheMagic) { delete[] plan; return fail(KVQ_E_CACHE, "caches[%d] was not built by kvq_cache_init", i); }
    if (c->codec_key != key) { delete[] plan; return fail(KVQ_E_CACHE, "caches[%d] was built for another codec", i); }
    if (t_new > 0 && !new_rows_dev[i]) { delete[] plan; return fail(KVQ_E_NULL, "new_rows_dev[%d] is NULL", i); }
    if (t_new > 0 && !aligned(new_rows_dev[i], 16)) { delete[] plan; return fail(KVQ_E_STRIDE, "new_rows_dev[%d] is not 16-byte aligned", i); }
    const int64_t floor = (int64_t)c->window + (t_new - 1 > c->margin ? t_new - 1 : (int64_t)c->margin);
    const int64_t total = c->tail_len + t_new;
    const int64_t k = total >= floor ? (total - floor) / C : 0;
    if (c->packed_len + k * C > c->packed_cap) {
      delete[] plan;
      return fail(KVQ_E_CAPACITY, "caches[%d]: packed region full (%lld + %lld > %lld records)", i,
                  (long long)c->packed_len, (long long)(k * C), (long long)c->packed_cap);
    }
    if (total - k * C > c->tail_cap) {
      delete[] plan;
      return fail(KVQ_E_CAPACITY, "caches[%d]: dense tail needs %lld rows > tail_cap %lld", i,
                  (long long)(total - k * C), (long long)c->tail_cap);
    }
    plan[i].k = k;
    plan[i].keep_from = k * C > c->tail_len ? k * C - c->tail_len : 0;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // 1) encode the evicted chunks (up to kMaxEvictCaches caches per launch)
  for (int i0 = 0; i0 < n_caches && e == hipSuccess; i0 += kvq::kMaxEvictCaches) {
    kvq::EvictArgs a{};
    a.tab = r.tab;
    a.D = r.D;
    int64_t rows = 0;
    int nc = 0;
    for (int i = i0; i < n_caches && i < i0 + kvq::kMaxEvictCaches; ++i) {
      if (plan[i].k == 0) continue;
      const kvq_cache* c = caches[i];
      kvq::EvictCache& ec = a.c[nc++];
      ec.tail = static_cast<const uint16_t*>(c->tail_dev);
      ec.fresh = t_new > 0 ? static_cast<const uint16_t*>(new_rows_dev[i]) : nullptr;
      ec.dst = static_cast<uint8_t*>(c->packed_dev) + c->packed_len * rb;
      ec.tail_cap = c->tail_cap;
      ec.tail_head = c->tail_head;
      ec.tail_len = c->tail_len;
      ec.rows = plan[i].k * C;
      ec.row_begin = rows;
      rows += ec.rows;
    }
    a.n_caches = nc;
    a.total_rows = rows;
    if (rows > 0) e = kvq::launch_evict(r.m, r.bits, r.sym, a, s);
  }
  // 2) append the surviving new rows to the tail rings
  for (int i0 = 0; i0 < n_caches && e == hipSuccess && t_new > 0; i0 += kvq::kMaxEvictCaches) {
    kvq::TailCopyArgs a{};
    a.D = r.D;
    int64_t rows = 0;
    int nc = 0;
    for (int i = i0; i < n_caches && i < i0 + kvq::kMaxEvictCaches; ++i) {
      const int64_t keep = t_new - plan[i].keep_from;
      if (keep <= 0) continue;
      const kvq_cache* c = caches[i];
      kvq::TailCopyCache& tc = a.c[nc++];
      tc.src = static_cast<const uint16_t*>(new_rows_dev[i]) + plan[i].keep_from * r.D;
      tc.ring = static_cast<uint16_t*>(c->tail_dev);
      tc.cap = c->tail_cap;
      tc.first_slot = (c->tail_head + c->tail_len + plan[i].keep_from) % c->tail_cap;
      tc.rows = keep;
      tc.row_begin = rows;
      rows += keep;
    }
    a.n_caches = nc;
    a.total_rows = rows;
    if (rows > 0) e = kvq::launch_tail_copy(a, s);
  }
  if (e != hipSuccess) {
    delete[] plan;
    return from_hip(e, "append_evict_chunk");
  }
  for (int i = 0; i < n_caches; ++i) {
    kvq_cache* c = caches[i];
    const int64_t ev = plan[i].k * C;
    c->packed_len += ev;
    c->tail_head = (c->tail_head + ev) % c->tail_cap;
    c->tail_len = c->tail_len + t_new - ev;
    if (evicted_host) evicted_host[i] = plan[i].k;
  }
  delete[] plan;
  return ok();
}

}  // extern "C"
