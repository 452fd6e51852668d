// kvq_encode_kron.hip — Hadamard-path encode at coded lengths 256 and 512 with the 32-point
// blocks of the rotation on the matrix cores (plain encode and cache eviction).
//
// Per vector [kakeyaturbo PR #15, "M4 Phase A": rotate = H.D.x, code = #{k : z > t_k}; "M4 Phase
// B": the rotation as a product on the tensor cores; arc PR #98, "What landed" and "Eviction is
// chunked"]: n = ||x||, u = H_m (s . x), code_i = #{k : u_i > n t_k}, b bit-planes + the f32 norm.
//
// Rotation. Entry (i, j) of the Sylvester H_m is (-1)^popcount(i & j), which factors over any
// split of the index bits, so with i = 32 o + lo (o < O = m/32):
//   u[o, lo] = sum_o' (-1)^popcount(o & o') Y[o', lo],   Y[o'] = H_32 x'[o'],  x' = s . x.
// Y is formed on v_mfma_f32_16x16x32_bf16 from +-1 operands and the bf16 rows (every product
// exact, sums in f32); the O-point transform over o is log2(O) butterfly stages in registers.
// Against the lane-per-vector kernel this moves 5 of the 8 or 9 butterfly stages and the bf16
// to f32 conversions off the vector ALUs, which bind that kernel.
//
// Operands. B = x'^T (32 inputs x 16 vectors): lane l = 16 g + v holds inputs 32 o + 8 g + e of
// vector v, one 16-byte chunk of the staged row. A_t (16 outputs x 32 inputs) for the two output
// halves t: row r of half t is output coordinate lo(t, r) = (r >> 2) + 4 t + 8 (r & 3). The
// accumulator of lane (g, v) for block o then holds u at coordinates 32 o + 8 i + 4 t + g
// (i = 0..3): in the record's bit-plane order pi(c) = (c mod 8) m/8 + floor(c/8) these are plane
// position (4 t + g) m/8 + 4 o + i, so lane (g, v) owns whole record words — word group
// G = (4 t + g) m/256 + o/8, bit 4 (o mod 8) + i — and needs no other lane to pack them.
//
// Quantiser. A binary search over the sorted thresholds (b - 1 decisions on |u| for symmetric
// tables, b for general ones), each decision one compare whose result is shifted into that bit's
// word and selects the next threshold; equal to the count #{k : |u| > n tau_k} of the
// lane-per-vector kernel for sorted thresholds.
//
// Data path per wave: 16 rows staged through swizzled LDS by whole-row 16-byte loads (the next
// tile's loads in flight while the current one computes), the records staged in the same space
// and written as one contiguous piece.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_lanevec.h"
#include "kvq_mfma.h"

namespace kvq {

template <int M>
struct KR {
  static constexpr int O = M / 32;          // 32-coordinate blocks
  static constexpr int CH = M / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;       // rows per wave load instruction
  static constexpr int NI = 16 / RPI;       // load instructions per 16-row tile
  static constexpr int WAVES = 4;           // waves per block
  static constexpr int ROWS = 16;           // vectors per wave tile
  static constexpr int WG = M / 128;        // record word groups per lane
  // waves per SIMD the kernels are compiled for (registers: 64 accumulators per pass plus the
  // next tile's rows, 32 or 64; LDS: 8 or 16 KB per wave)
  static constexpr int OCC = 2;
};

// Binary-search quantiser. thr holds the NT = 2^LVL - 1 searched thresholds, ascending, already
// multiplied by the norm: symmetric tables the positive half tau_k (the code's top bit is the
// sign), general tables all 2^b - 1.
template <int BITS, bool SYM>
struct QuantBS {
  static constexpr int LVL = SYM ? BITS - 1 : BITS;
  static constexpr int NT = (1 << LVL) - 1;
  float thr[NT > 0 ? NT : 1];
  bool nz;

  __device__ __forceinline__ QuantBS(const Tables& tab, float n) {
    constexpr int L = 1 << BITS;
    nz = n > 0.0f;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      if constexpr (SYM) thr[k] = n * tab.t[L / 2 + k];
      else thr[k] = nz ? n * tab.t[k] : (tab.t[k] < 0.0f ? -1.0f : 1.0f);  // n = 0: u = 0
    }
  }

  // Shift the decisions for coordinate u into the words (w[p]: code bit p; sgn: sign bits).
  __device__ __forceinline__ void push(float u, uint32_t (&w)[LVL > 0 ? LVL : 1], uint32_t& sgn) const {
    if constexpr (SYM) sgn = shift_in_sign(sgn, u);
    if constexpr (LVL > 0) {
      const float a = SYM ? fabsf(u) : u;
      float s[NT];
#pragma unroll
      for (int k = 0; k < NT; ++k) s[k] = thr[k];
#pragma unroll
      for (int lv = 0; lv < LVL; ++lv) {
        const int cnt = (1 << (LVL - lv)) - 1, mid = cnt / 2;
        // the decision bit is the sign of (threshold - a) (a zero difference is +0: not
        // greater), shifted in with one alignbit; a compare only where a select follows
        w[LVL - 1 - lv] = shift_in_sign(w[LVL - 1 - lv], s[mid] - a);
        if (mid == 0) continue;
        const bool c = a > s[mid];
#pragma unroll
        for (int k = 0; k < mid; ++k) {
          // both candidates as opaque register values: a select of two array elements would be
          // folded into an indexed read, which expands into compares against every position
          float hi = s[mid + 1 + k], lo = s[k];
          asm("" : "+v"(hi), "+v"(lo));
          s[k] = c ? hi : lo;
        }
      }
    }
  }

  // Plane words. Symmetric: top plane = (u > 0) (nothing for a zero vector); the lower planes
  // are the magnitude count's bits, complemented where u <= 0 (code L/2 - 1 - count).
  __device__ __forceinline__ void planes(const uint32_t (&w)[LVL > 0 ? LVL : 1], uint32_t sgn,
                                         uint32_t (&pl)[BITS]) const {
    if constexpr (SYM) {
      const uint32_t pos = nz ? ~sgn : 0u;
#pragma unroll
      for (int p = 0; p < BITS - 1; ++p) pl[p] = ~(w[p] ^ pos);
      pl[BITS - 1] = pos;
    } else {
#pragma unroll
      for (int p = 0; p < BITS; ++p) pl[p] = w[p];
    }
  }
};

__device__ __forceinline__ uint4 neg_bf16(const uint4& a) {
  return make_uint4(a.x ^ 0x80008000u, a.y ^ 0x80008000u, a.z ^ 0x80008000u, a.w ^ 0x80008000u);
}

// A_t for lane l: row r = l % 16, inputs k = 8 (l / 16) + e; entry (-1)^popcount(lo(t, r) & k).
__device__ __forceinline__ uint4 kron_fragment(int t, int l) {
  const int r = l & 15, lo = (r >> 2) + 4 * t + 8 * (r & 3);
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = 8 * (l >> 4) + 2 * h + q;
      v |= (0x3F80u | ((uint32_t)(__builtin_popcount(lo & k) & 1) << 15)) << (16 * q);
    }
    w[h] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One wave tile: the 16 rows staged in `reg` by the caller (signs already flipped); writes the
// 16 records (NWT words each) into rec_lds, which aliases reg and is written only after every
// operand read. The caller stores rec_lds.
// RULE: the stored scale is the codec's scale rule (scale_rule, from the chosen centroids) instead
// of the norm.
template <int M, int BITS, bool SYM, bool RULE = false>
__device__ __forceinline__ void kron_tile(const Tables& tab, const uint4 (&A)[2], const uint4* reg,
                                          uint32_t* rec_lds, int ln, int scale_rule = 0) {
  using K = KR<M>;
  constexpr int O = K::O, CH = K::CH, NWC = (M / 32) * BITS, NWT = NWC + 1;
  const int v = ln & 15, g = ln >> 4;
  // output halves per pass: both at m = 256; one at a time at m = 512 (64 accumulators live,
  // the operands read from LDS again for the second half)
  constexpr int TP = O > 8 ? 1 : 2;
  // top bits of the block index o whose butterfly stages run on the matrix cores (one fewer at
  // m = 512 for general tables of 3 and 4 bits, whose 7 or 15 thresholds need the registers, and
  // with a scale rule, whose centroid selection needs them)
  constexpr int FB = O > 8 && (SYM || BITS < 3) && !RULE ? 2 : 1, NH = 1 << FB, NL = O / NH;
  const uint4 AN[2] = {neg_bf16(A[0]), neg_bf16(A[1])};
  constexpr int LV = QuantBS<BITS, SYM>::LVL > 0 ? QuantBS<BITS, SYM>::LVL : 1;
  uint32_t* rec = rec_lds + v * NWT;
  uint32_t pl[2][O / 8][BITS];  // plane words of word group (4 t + g) m/256 + oh
  float n = 0.0f;
  float zu = 0.0f, zz = 0.0f;   // RULE
#pragma unroll
  for (int t0 = 0; t0 < 2; t0 += TP) {
    // Y[o] for the pass's output halves, with the transform's stages over the top FB bits of o
    // taken in the accumulation (acc[o] = sum_o' +-A Y-operand[o'] over the o' that differ from
    // o in those bits only); in the first pass also the norm's sum of squares
    floatx4 acc[TP][O];
    float ss = 0.0f;
#pragma unroll
    for (int ol = 0; ol < NL; ++ol) {
      uint4 X[NH];
#pragma unroll
      for (int oh = 0; oh < NH; ++oh) {
        X[oh] = reg[swz<CH>(v, 4 * (oh * NL + ol) + g)];
        if (t0 == 0) {
          const uint32_t xw[4] = {X[oh].x, X[oh].y, X[oh].z, X[oh].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[e]),
                                                 __builtin_bit_cast(bf16x2_t, xw[e]), ss, false);
        }
      }
#pragma unroll
      for (int tt = 0; tt < TP; ++tt)
#pragma unroll
        for (int oh = 0; oh < NH; ++oh) {
          floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int oi = 0; oi < NH; ++oi)
            c = mfma_bf16((__builtin_popcount(oh & oi) & 1) ? AN[t0 + tt] : A[t0 + tt], X[oi], c);
          acc[tt][oh * NL + ol] = c;
        }
    }
    if (t0 == 0) {
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      n = __builtin_amdgcn_sqrtf(ss);
      const bool bad = ss_out_of_range(ss);
      if (wave_any(bad)) {  // rescaled sum of squares (kvq_device.h), wave-uniform
        uint32_t mb = 0;
#pragma unroll
        for (int o = 0; o < O; ++o) {
          const uint32_t m = chunk_max_mag_bits(reg[swz<CH>(v, 4 * o + g)]);
          mb = mb > m ? mb : m;
        }
        uint32_t ot = (uint32_t)__shfl_xor((int)mb, 16, 64);
        mb = mb > ot ? mb : ot;
        ot = (uint32_t)__shfl_xor((int)mb, 32, 64);
        mb = mb > ot ? mb : ot;
        const int ex = max_exp_of_bits(mb);
        const float sc = pow2f(-ex);
        float s2 = 0.0f;
#pragma unroll
        for (int o = 0; o < O; ++o) s2 = chunk_scaled_ss(reg[swz<CH>(v, 4 * o + g)], sc, s2);
        s2 += __shfl_xor(s2, 16, 64);
        s2 += __shfl_xor(s2, 32, 64);
        n = bad ? __builtin_amdgcn_sqrtf(s2) * pow2f(ex) : n;
      }
    }
    // the rest of the O-point transform over the blocks (the low bits of o), in place
#pragma unroll
    for (int h = 1; h < NL; h <<= 1)
#pragma unroll
      for (int o = 0; o < O; ++o)
        if ((o & h) == 0)
#pragma unroll
          for (int tt = 0; tt < TP; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = acc[tt][o][i], y = acc[tt][o + h][i];
              acc[tt][o][i] = x + y;
              acc[tt][o + h][i] = x - y;
            }
    // quantise word group by word group: bits 4 (o mod 8) + i pushed from 31 down
    const QuantBS<BITS, SYM> q(tab, n);
#pragma unroll
    for (int tt = 0; tt < TP; ++tt)
#pragma unroll
      for (int oh = 0; oh < O / 8; ++oh) {
        uint32_t w[LV], sgn = 0u;
#pragma unroll
        for (int p = 0; p < LV; ++p) w[p] = 0u;
#pragma unroll
        for (int o = 8 * oh + 7; o >= 8 * oh; --o) {
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            q.push(acc[tt][o][i], w, sgn);
            if constexpr (RULE) {
              const float zh = chosen_centroid<BITS, SYM>(acc[tt][o][i], q, tab);
              zu = fmaf(acc[tt][o][i], zh, zu);
              zz = fmaf(zh, zh, zz);
            }
          }
          // general tables of 3 and 4 bits, or a scale rule: a few coordinates' searches at a
          // time (scheduled wide, their candidate thresholds exhaust the registers)
          if constexpr ((!SYM && BITS >= 3) || RULE) __builtin_amdgcn_sched_barrier(0);
        }
        q.planes(w, sgn, pl[t0 + tt][oh]);
      }
  }
  // every operand read is done (the record space aliases the staged rows)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int oh = 0; oh < O / 8; ++oh) {
      const int G = (4 * t + g) * (M / 256) + oh;
#pragma unroll
      for (int p = 0; p < BITS; ++p) rec[G * BITS + p] = pl[t][oh][p];
    }
  float stored = n;
  if constexpr (RULE) {
    zu += __shfl_xor(zu, 16, 64);
    zu += __shfl_xor(zu, 32, 64);
    zz += __shfl_xor(zz, 16, 64);
    zz += __shfl_xor(zz, 32, 64);
    stored = n > 0.0f ? rule_scale(scale_rule, n, zu, zz, M) : 0.0f;
  }
  if (g == 0) rec[NWC] = __float_as_uint(stored);
}

// Load piece k of a tile into registers: row RPI k + l / CH, chunk l % CH (the rows' 16-byte
// chunks in order: whole rows per instruction), its signs already flipped.
template <int M, class RowFn>
__device__ __forceinline__ void kron_load(RowFn row_of, const uint4& sm, int ln, uint4 (&in)[KR<M>::NI]) {
  using K = KR<M>;
  const int j0 = ln / K::CH, c = ln % K::CH;
#pragma unroll
  for (int k = 0; k < K::NI; ++k) {
    const uint4 x = ld_stream(row_of(K::RPI * k + j0) + 8 * c);
    in[k] = make_uint4(x.x ^ sm.x, x.y ^ sm.y, x.z ^ sm.z, x.w ^ sm.w);
  }
}

// The same for 16 rows ld elements apart starting at row0 (wave-uniform): the lane's first
// address plus a fixed stride per piece.
template <int M>
__device__ __forceinline__ void kron_load_linear(const uint16_t* row0, int64_t ld, const uint4& sm, int ln,
                                                 uint4 (&in)[KR<M>::NI]) {
  using K = KR<M>;
  const uint16_t* p = row0 + (ln / K::CH) * ld + 8 * (ln % K::CH);
  const int64_t step = K::RPI * ld;
#pragma unroll
  for (int k = 0; k < K::NI; ++k) {
    const uint4 x = ld_stream(p);
    in[k] = make_uint4(x.x ^ sm.x, x.y ^ sm.y, x.z ^ sm.z, x.w ^ sm.w);
    p += step;
    asm("" : "+v"(p));  // one address live: bumped per load, not all formed ahead
  }
}

template <int M>
__device__ __forceinline__ void kron_stage(const uint4 (&in)[KR<M>::NI], uint4* reg, int ln) {
  using K = KR<M>;
  const int j0 = ln / K::CH, c = ln % K::CH;
#pragma unroll
  for (int k = 0; k < K::NI; ++k) reg[swz<K::CH>(K::RPI * k + j0, c)] = in[k];
}

// The 16 records staged at rec_lds (NWT words each) to dst, records [0, valid) only.
template <int NWT>
__device__ __forceinline__ void kron_store(uint32_t* __restrict__ dst, const uint32_t* rec_lds, int valid,
                                           int ln) {
  constexpr int CHR = 16 * NWT / 4;  // 16-byte pieces (16 NWT is a multiple of 4)
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  const uint4* s4 = reinterpret_cast<const uint4*>(rec_lds);
  if (valid == 16) {
#pragma unroll
    for (int k = 0; k < (CHR + 63) / 64; ++k) {
      const int id = k * 64 + ln;
      if (id < CHR) st_stream(d4 + id, s4[id]);
    }
  } else {
    const int valid_w = valid * NWT;
#pragma unroll
    for (int k = 0; k < (CHR + 63) / 64; ++k) {
      const int id = k * 64 + ln;
      if (4 * id + 4 <= valid_w) st_stream(d4 + id, s4[id]);
    }
    const int tw = valid_w % 4, w0 = valid_w - tw;  // a partial last piece, word by word
    if (ln < tw) dst[w0 + ln] = rec_lds[w0 + ln];
  }
}

// Lane sign masks of its staged chunk (coordinates 8 (l % CH) .. + 7).
template <int M>
__device__ __forceinline__ uint4 kron_signs(const Tables& tab, int ln) {
  const int c = ln % KR<M>::CH;
  return make_uint4(tab.sign_pairs[4 * c], tab.sign_pairs[4 * c + 1], tab.sign_pairs[4 * c + 2],
                    tab.sign_pairs[4 * c + 3]);
}

// Plain encode: wave tiles of 16 rows (rows past the end repeat the last row), tile w of the
// grid's 4 G waves then w + 4 G, ...
template <int M, int BITS, bool SYM, bool RULE>
__global__ __launch_bounds__(64 * KR<M>::WAVES) __attribute__((amdgpu_waves_per_eu(KR<M>::OCC)))
void k_encode_kron(EncodeArgs a) {
  using K = KR<M>;
  constexpr int NWT = (M / 32) * BITS + 1;
  __shared__ uint4 s_reg[K::WAVES * 16 * K::CH];
  // the wave index as a scalar: tile indices, cache lookups and row bases stay wave-uniform
  const int ln = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* reg = s_reg + wave * 16 * K::CH;
  const uint4 A[2] = {kron_fragment(0, ln), kron_fragment(1, ln)};
  const uint4 sm = kron_signs<M>(a.tab, ln);
  const int64_t n_tiles = (a.n + 15) / 16, stride = (int64_t)gridDim.x * K::WAVES;
  auto load = [&](int64_t tile, uint4 (&in)[K::NI]) {
    const int64_t r0 = tile * 16;
    if (r0 + 16 <= a.n) {  // wave-uniform
      kron_load_linear<M>(a.x + r0 * a.ld, a.ld, sm, ln, in);
    } else {
      kron_load<M>([&](int j) {
        const int64_t r = r0 + j < a.n ? r0 + j : a.n - 1;
        return a.x + r * a.ld;
      }, sm, ln, in);
    }
  };
  int64_t tile = (int64_t)blockIdx.x * K::WAVES + wave;
  uint4 nxt[K::NI];
  if (tile < n_tiles) load(tile, nxt);
  for (; tile < n_tiles; tile += stride) {
    kron_stage<M>(nxt, reg, ln);
    if (tile + stride < n_tiles) load(tile + stride, nxt);
    __builtin_amdgcn_wave_barrier();
    uint32_t* rec_lds = reinterpret_cast<uint32_t*>(reg);
    kron_tile<M, BITS, SYM, RULE>(a.tab, A, reg, rec_lds, ln, a.scale_rule);
    __builtin_amdgcn_wave_barrier();
    const int64_t r0 = tile * 16;
    const int valid = a.n - r0 < 16 ? (int)(a.n - r0) : 16;
    kron_store<NWT>(reinterpret_cast<uint32_t*>(a.rec) + r0 * NWT, rec_lds, valid, ln);
    __builtin_amdgcn_wave_barrier();
  }
}

// Eviction [arc PR #98, "Eviction is chunked, on purpose"]: row r of cache k is row r of the
// concatenation (tail ring from its head, then the new rows); chunks are 128 rows, so a 16-row
// tile never straddles two caches.
template <int M, int BITS, bool SYM>
__global__ __launch_bounds__(64 * KR<M>::WAVES) __attribute__((amdgpu_waves_per_eu(KR<M>::OCC)))
void k_evict_kron(EvictArgs a) {
  using K = KR<M>;
  constexpr int NWT = (M / 32) * BITS + 1;
  __shared__ uint4 s_reg[K::WAVES * 16 * K::CH];
  // the wave index as a scalar: tile indices, cache lookups and row bases stay wave-uniform
  const int ln = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* reg = s_reg + wave * 16 * K::CH;
  const uint4 A[2] = {kron_fragment(0, ln), kron_fragment(1, ln)};
  const uint4 sm = kron_signs<M>(a.tab, ln);
  const int64_t n_tiles = a.total_rows / 16, stride = (int64_t)gridDim.x * K::WAVES;
  auto cache_of = [&](int64_t tile) {
    const int64_t g0 = tile * 16;
    int k = 0;
    while (k + 1 < a.n_caches && g0 >= a.c[k + 1].row_begin) ++k;
    return k;
  };
  // the tile's rows: one run of the ring without a wrap, or of the new rows (the usual cases:
  // a fixed stride), else row by row
  auto load = [&](int64_t tile, uint4 (&in)[K::NI]) {
    const EvictCache& ec = a.c[cache_of(tile)];
    const int64_t r0 = tile * 16 - ec.row_begin;
    const int64_t s0 = ec.tail_head + r0 >= ec.tail_cap ? ec.tail_head + r0 - ec.tail_cap : ec.tail_head + r0;
    if (r0 + 16 <= ec.tail_len && s0 + 16 <= ec.tail_cap) {  // wave-uniform
      kron_load_linear<M>(ec.tail + s0 * M, M, sm, ln, in);
    } else if (r0 >= ec.tail_len) {
      kron_load_linear<M>(ec.fresh + (r0 - ec.tail_len) * M, M, sm, ln, in);
    } else {
      kron_load<M>([&](int j) {
        // ring slot tail_head + rr < 2 tail_cap: one conditional subtract wraps it
        const int64_t rr = r0 + j, slot = ec.tail_head + rr;
        return rr < ec.tail_len ? ec.tail + (slot >= ec.tail_cap ? slot - ec.tail_cap : slot) * M
                                : ec.fresh + (rr - ec.tail_len) * M;
      }, sm, ln, in);
    }
  };
  int64_t tile = (int64_t)blockIdx.x * K::WAVES + wave;
  uint4 nxt[K::NI];
  if (tile < n_tiles) load(tile, nxt);
  for (; tile < n_tiles; tile += stride) {
    kron_stage<M>(nxt, reg, ln);
    const int k = cache_of(tile);
    if (tile + stride < n_tiles) load(tile + stride, nxt);
    __builtin_amdgcn_wave_barrier();
    uint32_t* rec_lds = reinterpret_cast<uint32_t*>(reg);
    kron_tile<M, BITS, SYM>(a.tab, A, reg, rec_lds, ln);
    __builtin_amdgcn_wave_barrier();
    const EvictCache& ec = a.c[k];
    const int64_t r0 = tile * 16 - ec.row_begin;
    kron_store<NWT>(reinterpret_cast<uint32_t*>(ec.dst) + r0 * NWT, rec_lds, 16, ln);
    __builtin_amdgcn_wave_barrier();
  }
}

// Resident blocks per CU of a kernel, from the occupancy query (taken once per kernel by the
// caller), times the CUs: the grid, or fewer blocks when there are fewer block tiles.
template <class Kern>
static int kron_per_cu(Kern kern, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, 0) != hipSuccess || nb <= 0) nb = 1;
  return nb;
}

static int64_t kron_grid(int per_cu, int64_t block_tiles) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t resident = (int64_t)per_cu * cus;
  return block_tiles < resident ? block_tiles : resident;
}

template <int M, int BITS, bool SYM, bool RULE>
static hipError_t launch_encode_kron_r(const EncodeArgs& a, hipStream_t st) {
  constexpr int W = KR<M>::WAVES;
  static const int per_cu = kron_per_cu(k_encode_kron<M, BITS, SYM, RULE>, 64 * W);
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t blocks = kron_grid(per_cu, (tiles + W - 1) / W);
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((k_encode_kron<M, BITS, SYM, RULE>), dim3((unsigned)blocks), dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

template <int M, int BITS, bool SYM>
static hipError_t launch_encode_kron_t(const EncodeArgs& a, hipStream_t st) {
  return a.scale_rule != 0 ? launch_encode_kron_r<M, BITS, SYM, true>(a, st)
                           : launch_encode_kron_r<M, BITS, SYM, false>(a, st);
}

template <int M, int BITS, bool SYM>
static hipError_t launch_evict_kron_t(const EvictArgs& a, hipStream_t st) {
  constexpr int W = KR<M>::WAVES;
  static const int per_cu = kron_per_cu(k_evict_kron<M, BITS, SYM>, 64 * W);
  const int64_t tiles = a.total_rows / 16;
  const int64_t blocks = kron_grid(per_cu, (tiles + W - 1) / W);
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((k_evict_kron<M, BITS, SYM>), dim3((unsigned)blocks), dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_encode_kron_m(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_encode_kron_t<M, 1, false>(a, st);
    case 3: return launch_encode_kron_t<M, 1, true>(a, st);
    case 4: return launch_encode_kron_t<M, 2, false>(a, st);
    case 5: return launch_encode_kron_t<M, 2, true>(a, st);
    case 6: return launch_encode_kron_t<M, 3, false>(a, st);
    case 7: return launch_encode_kron_t<M, 3, true>(a, st);
    case 8: return launch_encode_kron_t<M, 4, false>(a, st);
    case 9: return launch_encode_kron_t<M, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int M>
static hipError_t launch_evict_kron_m(int bits, bool sym, const EvictArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_evict_kron_t<M, 1, false>(a, st);
    case 3: return launch_evict_kron_t<M, 1, true>(a, st);
    case 4: return launch_evict_kron_t<M, 2, false>(a, st);
    case 5: return launch_evict_kron_t<M, 2, true>(a, st);
    case 6: return launch_evict_kron_t<M, 3, false>(a, st);
    case 7: return launch_evict_kron_t<M, 3, true>(a, st);
    case 8: return launch_evict_kron_t<M, 4, false>(a, st);
    case 9: return launch_evict_kron_t<M, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

bool encode_kron_supported(int m) { return m == 256 || m == 512; }

hipError_t launch_encode_kron(int m, int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (m == 256) return launch_encode_kron_m<256>(bits, sym, a, st);
  if (m == 512) return launch_encode_kron_m<512>(bits, sym, a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_evict_kron(int m, int bits, bool sym, const EvictArgs& a, hipStream_t st) {
  if (a.total_rows <= 0) return hipSuccess;
  if (m == 256) return launch_evict_kron_m<256>(bits, sym, a, st);
  if (m == 512) return launch_evict_kron_m<512>(bits, sym, a, st);
  return hipErrorInvalidValue;
}

}  // namespace kvq
