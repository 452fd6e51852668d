// kvq_encode.hip — encode kernels: bf16 rows -> packed records (+ optional outlier lists).
//
// Per vector [kakeyaturbo PR #15, commits "M4 Phase A" / "M4 Phase B"; arc PR #98 "What
// landed"]: n = ||v||, u = H_M (s (.) v), z = u/n, code_i = #{k : z_i > t_k}, b bit-planes + the
// f32 norm. These kernels hold a vector in the registers of one lane (two or four lanes for
// head_dim 256 / 512; kvq_lanevec.h); coded lengths 64 and 128 without an outlier list use the
// matrix-core rotation of kvq_encode_mx.hip.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_lanevec.h"

#include <type_traits>

namespace kvq {

template <int M, int BITS, bool SYM, bool RULE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LV<M>::WAVES)))
void k_encode(EncodeArgs a) {
  using L = LV<M>;
  using St = Stage<L::K>;
  constexpr int NWT = (M / 32) * BITS + 1;
  __shared__ __attribute__((aligned(16))) uint32_t s_sign[LV<M>::Q > 1 ? M / 2 : 4];
  __shared__ uint4 s_tile[4 * St::WORDS];
  build_sign_table<M>(a.tab, s_sign);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % L::Q, vw = lane / L::Q;
  uint4* tile = s_tile + wave * St::WORDS;
  const int64_t n_iter = (a.n + L::VPW - 1) / L::VPW;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < n_iter; it += (int64_t)gridDim.x * 4) {
    const int64_t vec = it * L::VPW + vw;
    const bool valid = vec < a.n;
    const int64_t vec0 = it * L::VPW;
    stage_rows_linear<M>(a.x, a.ld, vec0, a.n, tile);  // rows past the end repeat the last row
    float v[L::K];
    const float ss = load_part<L::K>(tile + lane * St::S, part_signs<M>(a.tab, s_sign, q), v);
    const float n = safe_norm_lv<L::K, L::Q>(part_sum<L::Q>(ss), tile + lane * St::S);
    fwht_regs<L::K, 8>(v);
    fwht_cross<L::Q, L::K>(v, q);
    float stored = n;
    if constexpr (RULE) {
      const Quant<BITS, SYM> qq(a.tab, n);
      float zu = 0.0f, zz = 0.0f;
#pragma unroll
      for (int i = 0; i < L::K; ++i) {
        const float zh = chosen_centroid<BITS, SYM>(v[i], qq, a.tab);
        zu = fmaf(v[i], zh, zu);
        zz = fmaf(zh, zh, zz);
      }
      stored = n > 0.0f ? rule_scale(a.scale_rule, n, part_sum<L::Q>(zu), part_sum<L::Q>(zz), M) : 0.0f;
    }
    quantize_store_lv<M, BITS, SYM>(v, n, stored, valid, q, a.tab,
                                    reinterpret_cast<uint32_t*>(a.rec) + vec * NWT);
  }
}

// ------------------------------------------------------------------------------------------
// Outlier side list [kakeyaturbo PR #15, calibrated Lloyd-Max + outlier commit: coordinates
// with |scaled residual| > T become sparse (index, value) overrides], in CSR order (vectors in
// input order, ascending coordinate inside a vector), built in three passes with no waiting
// between workgroups (on this chip device-scope
// flags cross the XCDs' separate L2s, so a chained prefix over tens of thousands of tiles is
// latency-bound): (1) encode + per-vector outlier count into offsets[v]; (2) an exclusive scan
// of the counts in place (block sums, one-block scan of the sums, local scans); (3) the same
// rotation again, writing each vector's entries at its offset in ascending coordinate order.
// Passes 1 and 3 run the same inlined load and rotation code and decide outliers with the same
// expression, so their counts agree; pass 3 still never writes outside [offsets[v],
// offsets[v+1]) or past the capacity.

__device__ __forceinline__ bool is_outlier(float u, float rn, float T) { return fabsf(u * rn) > T; }

// Rotated part of the vector owned by this lane (shared by the outlier passes).
template <int M>
__device__ __forceinline__ float rotate_owned(const EncodeArgs& a, const uint32_t* s_sign, int64_t it,
                                              uint4* tile, int q, float (&v)[LV<M>::K]) {
  using L = LV<M>;
  using St = Stage<L::K>;
  const int lane = threadIdx.x & 63;
  const int64_t vec0 = it * L::VPW;
  stage_rows_linear<M>(a.x, a.ld, vec0, a.n, tile);  // rows past the end repeat the last row
  const float ss = load_part<L::K>(tile + lane * St::S, part_signs<M>(a.tab, s_sign, q), v);
  const float n = safe_norm_lv<L::K, L::Q>(part_sum<L::Q>(ss), tile + lane * St::S);
  fwht_regs<L::K, 8>(v);
  fwht_cross<L::Q, L::K>(v, q);
  return n;
}

// Index type of an outlier entry: one byte while the coded length fits in it, two above.
template <int M>
using OutlierIdx = typename std::conditional<(M > 256), uint16_t, uint8_t>::type;

// Value of lane part k of this lane's quad (a DPP broadcast within the quad).
template <int K>
__device__ __forceinline__ uint32_t quad_lane_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, K | (K << 2) | (K << 4) | (K << 6), 0xF, 0xF, true);
}

// Sum over the Q lane parts of a vector, and the sum over the parts before this one (q).
template <int Q>
__device__ __forceinline__ void part_counts(uint32_t x, int q, uint32_t& total, uint32_t& before) {
  if constexpr (Q == 1) {
    total = x;
    before = 0u;
  } else if constexpr (Q == 2) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
    total = x + o;
    before = q == 1 ? o : 0u;
  } else {
    const uint32_t c0 = quad_lane_u32<0>(x), c1 = quad_lane_u32<1>(x), c2 = quad_lane_u32<2>(x),
                   c3 = quad_lane_u32<3>(x);
    total = c0 + c1 + c2 + c3;
    before = (q > 0 ? c0 : 0u) + (q > 1 ? c1 : 0u) + (q > 2 ? c2 : 0u);
  }
}

template <int M, int BITS, bool SYM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LV<M>::WAVES)))
void k_encode_count(EncodeArgs a) {
  using L = LV<M>;
  using St = Stage<L::K>;
  static_assert(L::Q <= 4, "outlier lists need m <= 512");
  constexpr int NWT = (M / 32) * BITS + 1;
  __shared__ __attribute__((aligned(16))) uint32_t s_sign[LV<M>::Q > 1 ? M / 2 : 4];
  __shared__ uint4 s_tile[4 * St::WORDS];
  build_sign_table<M>(a.tab, s_sign);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % L::Q, vw = lane / L::Q;
  uint4* tile = s_tile + wave * St::WORDS;
  const int64_t n_iter = (a.n + L::VPW - 1) / L::VPW;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < n_iter; it += (int64_t)gridDim.x * 4) {
    const int64_t vec = it * L::VPW + vw;
    const bool valid = vec < a.n;
    float v[L::K];
    const float n = rotate_owned<M>(a, s_sign, it, tile, q, v);
    const float rn = n > 0.0f ? 1.0f / n : 0.0f;
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < L::K; ++k) cnt += is_outlier(v[k], rn, a.tab.T) ? 1u : 0u;
    uint32_t total, before;
    part_counts<L::Q>(cnt, q, total, before);  // every lane takes part in the DPP moves
    if (valid && q == 0) a.ol_off[vec] = total;
    quantize_store_lv<M, BITS, SYM>(v, n, n, valid, q, a.tab,
                                    reinterpret_cast<uint32_t*>(a.rec) + vec * NWT);
  }
}

template <int M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LV<M>::WAVES)))
void k_encode_emit(EncodeArgs a) {
  using L = LV<M>;
  using St = Stage<L::K>;
  static_assert(L::Q <= 4, "outlier lists need m <= 512");
  __shared__ __attribute__((aligned(16))) uint32_t s_sign[LV<M>::Q > 1 ? M / 2 : 4];
  __shared__ uint4 s_tile[4 * St::WORDS];
  build_sign_table<M>(a.tab, s_sign);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % L::Q, vw = lane / L::Q;
  uint4* tile = s_tile + wave * St::WORDS;
  const int64_t n_iter = (a.n + L::VPW - 1) / L::VPW;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < n_iter; it += (int64_t)gridDim.x * 4) {
    const int64_t vec = it * L::VPW + vw;
    const bool valid = vec < a.n;
    float v[L::K];
    const float n = rotate_owned<M>(a, s_sign, it, tile, q, v);
    const float rn = n > 0.0f ? 1.0f / n : 0.0f;
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < L::K; ++k) cnt += is_outlier(v[k], rn, a.tab.T) ? 1u : 0u;
    uint32_t total, before;  // parts with lower coordinates come first
    part_counts<L::Q>(cnt, q, total, before);  // every lane takes part in the DPP moves
    if (!valid) continue;
    int64_t pos = (int64_t)a.ol_off[vec] + before;
    int64_t end = a.ol_off[vec + 1];
    if (end > a.ol_cap) end = a.ol_cap;
#pragma unroll
    for (int k = 0; k < L::K; ++k) {
      if (is_outlier(v[k], rn, a.tab.T)) {
        if (pos < end) {
          static_cast<OutlierIdx<M>*>(a.ol_idx)[pos] = (OutlierIdx<M>)(q * L::K + k);
          a.ol_val[pos] = (uint16_t)f32_to_bf16_rne(v[k] * rn);
        }
        ++pos;
      }
    }
  }
}

// Exclusive scan of n u32 counts in place, total at counts[n]. kScanItems per thread.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kScanSpan = kScanThreads * kScanItems;

// Block-wide exclusive scan (1024 threads) of one value per thread; returns the block total too.
__device__ __forceinline__ uint32_t scan_block_1024(uint32_t x, uint32_t* s_w, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wave) before += s_w[w];
    total += s_w[w];
  }
  __syncthreads();
  return before + incl - x;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_sums(const uint32_t* cnt, int64_t n, uint32_t* part) {
  __shared__ uint32_t s_w[kScanThreads / 64];
  const int64_t i0 = (int64_t)blockIdx.x * kScanSpan + threadIdx.x * kScanItems;
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) s += i0 + k < n ? cnt[i0 + k] : 0u;
  uint32_t total;
  scan_block_1024(s, s_w, total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_top(uint32_t* part, int64_t nb) {
  __shared__ uint32_t s_w[kScanThreads / 64];
  uint32_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += kScanThreads) {
    const int64_t i = b0 + threadIdx.x;
    const uint32_t x = i < nb ? part[i] : 0u;
    uint32_t total;
    const uint32_t ex = scan_block_1024(x, s_w, total);
    if (i < nb) part[i] = carry + ex;
    carry += total;
  }
}

__global__ __launch_bounds__(kScanThreads) void k_scan_apply(uint32_t* cnt, int64_t n, const uint32_t* part) {
  __shared__ uint32_t s_w[kScanThreads / 64];
  const int64_t i0 = (int64_t)blockIdx.x * kScanSpan + threadIdx.x * kScanItems;
  uint32_t x[kScanItems], s = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    x[k] = i0 + k < n ? cnt[i0 + k] : 0u;
    s += x[k];
  }
  uint32_t total;
  uint32_t run = part[blockIdx.x] + scan_block_1024(s, s_w, total);
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    if (i0 + k < n) cnt[i0 + k] = run;
    run += x[k];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) cnt[n] = part[blockIdx.x] + total;
}

int64_t scan_partials(int64_t n) { return (n + kScanSpan - 1) / kScanSpan; }

hipError_t launch_offsets_scan(uint32_t* cnt, int64_t n, uint32_t* part, hipStream_t st) {
  const int64_t nb = scan_partials(n);
  if (nb < 1) return hipSuccess;
  hipLaunchKernelGGL(k_scan_sums, dim3((unsigned)nb), dim3(kScanThreads), 0, st, cnt, n, part);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(kScanThreads), 0, st, part, nb);
  hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(kScanThreads), 0, st, cnt, n,
                     (const uint32_t*)part);
  return hipGetLastError();
}

template <int M, int BITS, bool SYM>
static hipError_t launch_count_t(const EncodeArgs& a, hipStream_t st) {
  const int64_t n_iter = (a.n + LV<M>::VPW - 1) / LV<M>::VPW;
  int64_t blocks = (n_iter + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((k_encode_count<M, BITS, SYM>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_emit_t(const EncodeArgs& a, hipStream_t st) {
  const int64_t n_iter = (a.n + LV<M>::VPW - 1) / LV<M>::VPW;
  int64_t blocks = (n_iter + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((k_encode_emit<M>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_outliers_m(int bits, bool sym, const EncodeArgs& a, uint32_t* part,
                                    hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: e = launch_count_t<M, 1, false>(a, st); break;
    case 3: e = launch_count_t<M, 1, true>(a, st); break;
    case 4: e = launch_count_t<M, 2, false>(a, st); break;
    case 5: e = launch_count_t<M, 2, true>(a, st); break;
    case 6: e = launch_count_t<M, 3, false>(a, st); break;
    case 7: e = launch_count_t<M, 3, true>(a, st); break;
    case 8: e = launch_count_t<M, 4, false>(a, st); break;
    case 9: e = launch_count_t<M, 4, true>(a, st); break;
  }
  if (e != hipSuccess) return e;
  e = launch_offsets_scan(a.ol_off, a.n, part, st);
  if (e != hipSuccess) return e;
  return launch_emit_t<M>(a, st);
}

static int64_t align16(int64_t b) { return (b + 15) & ~int64_t(15); }

int64_t outlier_stage_bytes(int m, int64_t n) {
  if (m != 128 || n <= 0) return 0;
  const int64_t tiles = (n + 15) / 16;
  return align16(4 * tiles) + align16(kOutlierStage * tiles) + align16(2 * kOutlierStage * tiles) + 16;
}

hipError_t launch_encode_outliers3(int m, int bits, bool sym, const EncodeArgs& a, uint32_t* part,
                                   hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (m == 128) {  // both passes on the matrix-core rotation, entries staged in between
    const int64_t tiles = (a.n + 15) / 16;
    uint8_t* w = reinterpret_cast<uint8_t*>(part) + align16(4 * scan_partials(a.n));
    w = reinterpret_cast<uint8_t*>(align16(reinterpret_cast<int64_t>(w)));
    EncodeArgs b = a;
    b.stg_flag = reinterpret_cast<uint32_t*>(w);
    b.stg_idx = w + align16(4 * tiles);
    b.stg_val = reinterpret_cast<uint16_t*>(b.stg_idx + align16(kOutlierStage * tiles));
    hipError_t e = launch_t128_outlier_pass<1>(bits, sym, b, st);
    if (e == hipSuccess) e = launch_offsets_scan(b.ol_off, b.n, part, st);
    if (e == hipSuccess) e = launch_outlier_copy(b, st);
    if (e == hipSuccess) e = launch_t128_outlier_pass<2>(bits, sym, b, st);
    return e;
  }
  switch (m) {
    case 64: return launch_outliers_m<64>(bits, sym, a, part, st);
    case 128: return launch_outliers_m<128>(bits, sym, a, part, st);
    case 256: return launch_outliers_m<256>(bits, sym, a, part, st);
    case 512: return launch_outliers_m<512>(bits, sym, a, part, st);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------
// Eviction: encode whole chunks of the oldest dense rows of several caches in one launch
// [arc PR #98, "Eviction is chunked, on purpose"]. Row r of cache k is row r of the
// concatenation (tail ring from its head, then the new rows). Chunks are 128 rows and a wave
// (64 / Q vectors) never straddles two caches.
template <int M, int BITS, bool SYM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LV<M>::WAVES)))
void k_evict(EvictArgs a) {
  using L = LV<M>;
  using St = Stage<L::K>;
  constexpr int NWT = (M / 32) * BITS + 1;
  __shared__ __attribute__((aligned(16))) uint32_t s_sign[LV<M>::Q > 1 ? M / 2 : 4];
  __shared__ uint4 s_tile[4 * St::WORDS];
  build_sign_table<M>(a.tab, s_sign);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % L::Q, vw = lane / L::Q;
  uint4* tile = s_tile + wave * St::WORDS;
  const int64_t n_iter = a.total_rows / L::VPW;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < n_iter; it += (int64_t)gridDim.x * 4) {
    const int64_t g0 = it * L::VPW;
    int k = 0;
    while (k + 1 < a.n_caches && g0 >= a.c[k + 1].row_begin) ++k;
    const EvictCache& ec = a.c[k];
    const int64_t r0 = g0 - ec.row_begin, r = r0 + vw;
    stage_rows_in<M>([&](int j) {
      // ring slot tail_head + rr < 2 tail_cap (both terms are below tail_cap): one conditional
      // subtract wraps it; caches hold Hadamard records, so rows are M = head_dim elements
      const int64_t rr = r0 + j;
      const int64_t slot = ec.tail_head + rr;
      return rr < ec.tail_len ? ec.tail + (slot >= ec.tail_cap ? slot - ec.tail_cap : slot) * M
                              : ec.fresh + (rr - ec.tail_len) * M;
    }, tile);
    float v[L::K];
    const float ss = load_part<L::K>(tile + lane * St::S, part_signs<M>(a.tab, s_sign, q), v);
    const float n = safe_norm_lv<L::K, L::Q>(part_sum<L::Q>(ss), tile + lane * St::S);
    fwht_regs<L::K, 8>(v);
    fwht_cross<L::Q, L::K>(v, q);
    quantize_store_lv<M, BITS, SYM>(v, n, n, true, q, a.tab,
                                    reinterpret_cast<uint32_t*>(ec.dst) + r * NWT);
  }
}

template <int M, int BITS, bool SYM>
static hipError_t launch_evict_t(const EvictArgs& a, hipStream_t st) {
  constexpr int VPW = LV<M>::VPW;
  const int64_t n_iter = a.total_rows / VPW;
  int64_t blocks = (n_iter + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((k_evict<M, BITS, SYM>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_evict_m(int bits, bool sym, const EvictArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_evict_t<M, 1, false>(a, st);
    case 3: return launch_evict_t<M, 1, true>(a, st);
    case 4: return launch_evict_t<M, 2, false>(a, st);
    case 5: return launch_evict_t<M, 2, true>(a, st);
    case 6: return launch_evict_t<M, 3, false>(a, st);
    case 7: return launch_evict_t<M, 3, true>(a, st);
    case 8: return launch_evict_t<M, 4, false>(a, st);
    case 9: return launch_evict_t<M, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_evict(int m, int bits, bool sym, const EvictArgs& a, hipStream_t st) {
  if (encode_kron_supported(m)) return launch_evict_kron(m, bits, sym, a, st);
  switch (m) {
    case 64: return launch_evict_m<64>(bits, sym, a, st);
    case 128: return launch_evict_m<128>(bits, sym, a, st);
    case 256: return launch_evict_m<256>(bits, sym, a, st);
    case 512: return launch_evict_m<512>(bits, sym, a, st);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------
// Lloyd-Max refit [kakeyaturbo PR #15, calibration-artefacts commit: the table refitted to the
// codec's own post-rotation coordinates]. One pass: per block, the sum and the count of the
// rotated, normalised coordinates z = u / n falling in each cell of the current table, the cell
// decided as the quantiser decides it (u > n t_k); the host sums the blocks' partials in f64 and
// moves each centroid to its cell's mean.

template <int M, int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LV<M>::WAVES)))
void k_fit_cells(EncodeArgs a, float* part_sum, uint32_t* part_cnt) {
  using L = LV<M>;
  using St = Stage<L::K>;
  constexpr int NL = 1 << BITS;
  __shared__ __attribute__((aligned(16))) uint32_t s_sign[LV<M>::Q > 1 ? M / 2 : 4];
  __shared__ uint4 s_tile[4 * St::WORDS];
  __shared__ float s_sum[4][NL];
  __shared__ uint32_t s_cnt[4][NL];
  build_sign_table<M>(a.tab, s_sign);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % L::Q, vw = lane / L::Q;
  uint4* tile = s_tile + wave * St::WORDS;
  float sum[NL];
  uint32_t cnt[NL];
#pragma unroll
  for (int c = 0; c < NL; ++c) {
    sum[c] = 0.0f;
    cnt[c] = 0u;
  }
  const int64_t n_iter = (a.n + L::VPW - 1) / L::VPW;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < n_iter; it += (int64_t)gridDim.x * 4) {
    const bool valid = it * L::VPW + vw < a.n;
    float v[L::K];
    const float n = rotate_owned<M>(a, s_sign, it, tile, q, v);
    const float rn = n > 0.0f ? 1.0f / n : 0.0f;
    // a zero vector has u = 0 and z = 0: its compares are 0 > t_k
    float thr[NL - 1];
#pragma unroll
    for (int k = 0; k < NL - 1; ++k) thr[k] = n > 0.0f ? n * a.tab.t[k] : (a.tab.t[k] < 0.0f ? -1.0f : 1.0f);
#pragma unroll
    for (int i = 0; i < L::K; ++i) {
      int code = 0;
#pragma unroll
      for (int k = 0; k < NL - 1; ++k) code += v[i] > thr[k] ? 1 : 0;
      const float z = v[i] * rn;
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        const bool hit = valid && code == c;
        sum[c] += hit ? z : 0.0f;
        cnt[c] += hit ? 1u : 0u;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NL; ++c) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      sum[c] += __shfl_xor(sum[c], m, 64);
      cnt[c] += (uint32_t)__shfl_xor((int)cnt[c], m, 64);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      s_sum[wave][c] = sum[c];
      s_cnt[wave][c] = cnt[c];
    }
  }
  __syncthreads();
  if (threadIdx.x < NL) {
    const int c = threadIdx.x;
    part_sum[(int64_t)blockIdx.x * NL + c] = s_sum[0][c] + s_sum[1][c] + s_sum[2][c] + s_sum[3][c];
    part_cnt[(int64_t)blockIdx.x * NL + c] = s_cnt[0][c] + s_cnt[1][c] + s_cnt[2][c] + s_cnt[3][c];
  }
}

int64_t fit_blocks(int m, int64_t n) {
  const int vpw = m > 128 ? 64 / (m / 128) : 64;  // vectors per wave (LV<m>::VPW)
  const int64_t n_iter = (n + vpw - 1) / vpw;
  int64_t blocks = (n_iter + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  return blocks < 1 ? 1 : blocks;
}

template <int M, int BITS>
static hipError_t launch_fit_t(const EncodeArgs& a, float* part_sum, uint32_t* part_cnt, hipStream_t st) {
  const int64_t blocks = fit_blocks(M, a.n);
  hipLaunchKernelGGL((k_fit_cells<M, BITS>), dim3((unsigned)blocks), dim3(256), 0, st, a, part_sum, part_cnt);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_fit_m(int bits, const EncodeArgs& a, float* ps, uint32_t* pc, hipStream_t st) {
  switch (bits) {
    case 1: return launch_fit_t<M, 1>(a, ps, pc, st);
    case 2: return launch_fit_t<M, 2>(a, ps, pc, st);
    case 3: return launch_fit_t<M, 3>(a, ps, pc, st);
    case 4: return launch_fit_t<M, 4>(a, ps, pc, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fit_cells(int m, int bits, const EncodeArgs& a, float* part_sum, uint32_t* part_cnt,
                            hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  switch (m) {
    case 64: return launch_fit_m<64>(bits, a, part_sum, part_cnt, st);
    case 128: return launch_fit_m<128>(bits, a, part_sum, part_cnt, st);
    case 256: return launch_fit_m<256>(bits, a, part_sum, part_cnt, st);
    case 512: return launch_fit_m<512>(bits, a, part_sum, part_cnt, st);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------
// Launchers

template <int M, int BITS, bool SYM>
static hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t st) {
  constexpr int VPW = LV<M>::VPW;
  const int64_t n_iter = (a.n + VPW - 1) / VPW;
  int64_t blocks = (n_iter + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return hipSuccess;
  if (a.scale_rule != 0)
    hipLaunchKernelGGL((k_encode<M, BITS, SYM, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_encode<M, BITS, SYM, false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_encode_m(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_encode_t<M, 1, false>(a, st);
    case 3: return launch_encode_t<M, 1, true>(a, st);
    case 4: return launch_encode_t<M, 2, false>(a, st);
    case 5: return launch_encode_t<M, 2, true>(a, st);
    case 6: return launch_encode_t<M, 3, false>(a, st);
    case 7: return launch_encode_t<M, 3, true>(a, st);
    case 8: return launch_encode_t<M, 4, false>(a, st);
    case 9: return launch_encode_t<M, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_encode(int m, int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  // the lane-per-vector kernel: coded length 32, and 64 with a scale rule
  if (encode_mx_supported(m, a.scale_rule)) return launch_encode_mx(m, bits, sym, a, st);
  if (encode_kron_supported(m)) return launch_encode_kron(m, bits, sym, a, st);
  switch (m) {
    case 32: return launch_encode_m<32>(bits, sym, a, st);
    case 64: return launch_encode_m<64>(bits, sym, a, st);
    case 128: return launch_encode_m<128>(bits, sym, a, st);
    case 256: return launch_encode_m<256>(bits, sym, a, st);
    case 512: return launch_encode_m<512>(bits, sym, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
