// kvq_encode.hip — encode kernels: bf16 rows -> packed records (+ optional outlier lists).
//
// Per vector [kakeyaturbo PR #15, commits "M4 Phase A" / "M4 Phase B"; arc PR #98 "What
// landed"]: n = ||v||, u = H_M (s (.) v), z = u/n, code_i = #{k : z_i > t_k}, b bit-planes + the
// f32 norm. The plain and eviction kernels hold a vector in the registers of one lane (two or
// four lanes for head_dim 256 / 512; kvq_lanevec.h). The outlier kernel keeps the wave-ballot
// layout of kvq_quant.h (8 coordinates per lane), where a vector's outliers are found by lane
// order.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_lanevec.h"
#include "kvq_quant.h"

namespace kvq {

template <int M, int BITS, bool SYM>
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
    stage_rows_in<M>([&](int j) {  // rows past the end repeat the last row (results unused)
      const int64_t r = vec0 + j < a.n ? vec0 + j : a.n - 1;
      return a.x + r * a.ld;
    }, tile);
    float v[L::K];
    const float ss = load_part<L::K>(tile + lane * St::S, part_signs<M>(a.tab, s_sign, q), v);
    const float n = sqrtf(part_sum<L::Q>(ss));
    fwht_regs<L::K, 8>(v);
    fwht_cross<L::Q, L::K>(v, q);
    quantize_store_lv<M, BITS, SYM>(v, n, valid, q, a.tab,
                                    reinterpret_cast<uint32_t*>(a.rec) + vec * NWT);
  }
}

// ------------------------------------------------------------------------------------------
// Outlier side list [kakeyaturbo PR #15, calibrated Lloyd-Max + outlier commit: coordinates
// with |scaled residual| > T become sparse (index, value) overrides]. CSR order (vectors in
// input order, ascending coordinate inside a vector) is produced in one pass: each workgroup
// takes a tile of consecutive vectors by ticket, scans its counts in LDS, and obtains the
// tile's global offset by a decoupled look-back over the status words of earlier tiles.

constexpr int kOutlierIters = 4;  // wave iterations per tile

template <int M>
constexpr int outlier_tile() { return 4 * (64 / (M / 8)) * kOutlierIters; }

constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagInclusive = 2ull << 62;
constexpr uint64_t kValueMask = (1ull << 62) - 1;
constexpr int kMaxSpin = 1 << 22;

// Exclusive prefix of the tiles before `tile`, publishing this tile's aggregate first and its
// inclusive prefix last. Every earlier tile holds an earlier ticket, so it is running or done
// and publishes without waiting on later tiles: the wait always ends. A bounded spin records
// an error instead of waiting forever.
__device__ uint64_t tile_lookback(uint64_t* status, uint32_t* err, int64_t tile, uint64_t agg) {
  if (tile == 0) {
    __hip_atomic_store(&status[0], kFlagInclusive | agg, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  __hip_atomic_store(&status[tile], kFlagAggregate | agg, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t prefix = 0;
  int64_t j = tile - 1;
  int spin = 0;
  while (j >= 0) {
    const uint64_t s = __hip_atomic_load(&status[j], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t flag = s & ~kValueMask;
    if (flag == 0) {
      if (++spin > kMaxSpin) {
        atomicOr(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    prefix += s & kValueMask;
    if (flag == kFlagInclusive) break;
    --j;
  }
  __hip_atomic_store(&status[tile], kFlagInclusive | (prefix + agg), __ATOMIC_RELEASE,
                     __HIP_MEMORY_SCOPE_AGENT);
  return prefix;
}

// Block-wide exclusive scan of one value per thread (256 threads); returns the total too.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* s_wave, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += s_wave[w];
    total += s_wave[w];
  }
  return before + incl - x;
}

template <int M, int BITS, bool SYM>
__global__ __launch_bounds__(256) void k_encode_ol(EncodeArgs a) {
  constexpr int LPV = M / 8, VPW = 64 / LPV, U = kOutlierIters, TILE = outlier_tile<M>();
  static_assert(TILE <= 256, "one count per thread");
  __shared__ uint32_t s_ticket;
  __shared__ uint32_t s_cnt[256];
  __shared__ uint32_t s_wave[4];
  __shared__ uint64_t s_prefix;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPV, c = lane % LPV;
  if (threadIdx.x == 0) s_ticket = atomicAdd(a.ws_ticket, 1u);
  s_cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t tile = s_ticket;
  const int64_t base = tile * TILE;
  uint32_t sm[4];
  chunk_sign_masks<M>(a.tab, c, sm);
  const float T = a.tab.T;
  float z[U][8];
  uint64_t om[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int local = (u * 4 + wave) * VPW + sub;
    const int64_t vec = base + local;
    const bool valid = vec < a.n;
    float v[8];
    const float ss = load_signed_chunk(a.x + vec * a.ld, c, sm, valid, v);
    const float n = sqrtf(vector_sum<LPV>(ss));
    fwht_vector<LPV>(v, c);
    quantize_store<M, BITS, SYM>(v, n, valid, vec, sub, c, a.tab, a.rec);
    const float rn = n > 0.0f ? 1.0f / n : 0.0f;
    uint32_t cl = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z[u][j] = v[j] * rn;
      const bool o = valid && fabsf(z[u][j]) > T;
      om[u][j] = ballot64(o);
      cl += o ? 1u : 0u;
    }
    const uint32_t cv = vector_sum_u32<LPV>(cl);
    if (c == 0) s_cnt[local] = cv;
  }
  __syncthreads();
  uint32_t agg = 0;
  const uint32_t excl = block_exclusive_scan(s_cnt[threadIdx.x], s_wave, agg);
  if (threadIdx.x == 0) s_prefix = tile_lookback(a.ws_status, a.ws_error, tile, agg);
  __syncthreads();  // every thread has read s_cnt; s_prefix is published
  const uint64_t prefix = s_prefix;
  s_cnt[threadIdx.x] = excl;  // reuse: exclusive offset inside the tile
  if (threadIdx.x < TILE && base + threadIdx.x < a.n)
    a.ol_off[base + threadIdx.x] = (uint32_t)(prefix + excl);
  if (threadIdx.x == 0 && base + TILE >= a.n) a.ol_off[a.n] = (uint32_t)(prefix + agg);
  __syncthreads();
  const uint64_t vec_lanes = low_mask(LPV) << (sub * LPV);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int local = (u * 4 + wave) * VPW + sub;
    const int64_t vec = base + local;
    if (vec >= a.n) continue;
    uint32_t below = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t mk = om[u][j] & vec_lanes;
      below += __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    }
    uint64_t pos = prefix + s_cnt[local] + below;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (fabsf(z[u][j]) > T) {
        if (pos < (uint64_t)a.ol_cap) {
          a.ol_idx[pos] = (uint8_t)(8 * c + j);
          a.ol_val[pos] = (uint16_t)f32_to_bf16_rne(z[u][j]);
        }
        ++pos;
      }
    }
  }
}

template <int M, int BITS, bool SYM>
static hipError_t launch_encode_ol_t(const EncodeArgs& a, int64_t n_tiles, hipStream_t st) {
  if (n_tiles < 1) return hipSuccess;
  if (n_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_encode_ol<M, BITS, SYM>), dim3((unsigned)n_tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_encode_ol_m(int bits, bool sym, const EncodeArgs& a, int64_t nt,
                                     hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_encode_ol_t<M, 1, false>(a, nt, st);
    case 3: return launch_encode_ol_t<M, 1, true>(a, nt, st);
    case 4: return launch_encode_ol_t<M, 2, false>(a, nt, st);
    case 5: return launch_encode_ol_t<M, 2, true>(a, nt, st);
    case 6: return launch_encode_ol_t<M, 3, false>(a, nt, st);
    case 7: return launch_encode_ol_t<M, 3, true>(a, nt, st);
    case 8: return launch_encode_ol_t<M, 4, false>(a, nt, st);
    case 9: return launch_encode_ol_t<M, 4, true>(a, nt, st);
  }
  return hipErrorInvalidValue;
}

int64_t encode_outlier_tile_vectors(int m) {
  switch (m) {
    case 32: return outlier_tile<32>();
    case 64: return outlier_tile<64>();
    case 128: return outlier_tile<128>();
    case 256: return outlier_tile<256>();
  }
  return 64;
}

hipError_t launch_encode_outliers(int m, int bits, bool sym, const EncodeArgs& a,
                                  int64_t n_tiles, hipStream_t st) {
  switch (m) {
    case 64: return launch_encode_ol_m<64>(bits, sym, a, n_tiles, st);
    case 128: return launch_encode_ol_m<128>(bits, sym, a, n_tiles, st);
    case 256: return launch_encode_ol_m<256>(bits, sym, a, n_tiles, st);
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
      const int64_t rr = r0 + j;
      return rr < ec.tail_len ? ec.tail + ((ec.tail_head + rr) % ec.tail_cap) * a.D
                              : ec.fresh + (rr - ec.tail_len) * a.D;
    }, tile);
    float v[L::K];
    const float ss = load_part<L::K>(tile + lane * St::S, part_signs<M>(a.tab, s_sign, q), v);
    const float n = sqrtf(part_sum<L::Q>(ss));
    fwht_regs<L::K, 8>(v);
    fwht_cross<L::Q, L::K>(v, q);
    quantize_store_lv<M, BITS, SYM>(v, n, true, q, a.tab,
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
  switch (m) {
    case 64: return launch_evict_m<64>(bits, sym, a, st);
    case 128: return launch_evict_m<128>(bits, sym, a, st);
    case 256: return launch_evict_m<256>(bits, sym, a, st);
    case 512: return launch_evict_m<512>(bits, sym, a, st);
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
  hipLaunchKernelGGL((k_encode<M, BITS, SYM>), dim3((unsigned)blocks), dim3(256), 0, st, a);
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
  if (encode_mx_supported(m)) return launch_encode_mx(m, bits, sym, a, st);
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
