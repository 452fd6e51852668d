// kvq_lanevec.h — lane-per-vector building blocks of the gfx950 codec kernels.
//
// A vector of coded length M lives in the registers of Q = max(1, M/128) consecutive lanes;
// lane part q (= lane % Q) holds the K = M/Q consecutive coordinates [qK, qK + K). So for
// head_dim <= 128 a lane owns a whole vector and the rotation
//   u = H_M (s (.) v)   [kakeyaturbo PR #15, "M4 Phase A": rotate = H.D.x; "M4 Phase B":
//                        Sylvester Hadamard]
// is log2(K) in-register butterfly stages (one add or sub per coordinate per stage) plus
// log2(Q) stages across the lanes of a quad (quad_perm DPP). Quantiser compares are shifted
// straight into per-lane record words, so no word ever crosses from scalar to vector registers.
//
// Record bit layout (format v1): plane position of coordinate i is
//   pi(i) = (i mod 8) * (M/8) + floor(i/8),  word g*b + p, bit pi mod 32 (g = pi / 32).
#pragma once

#include "kvq_device.h"

namespace kvq {

template <int M>
struct LV {
  static constexpr int Q = M > 128 ? M / 128 : 1;   // lanes per vector
  static constexpr int K = M / Q;                    // coordinates per lane
  static constexpr int VPW = 64 / Q;                 // vectors per wave
  // waves per SIMD the kernels are compiled for: 128 live coordinates per lane fit in 256
  // VGPRs (2 waves) without spilling; 64 fit in 168 (3 waves)
  static constexpr int WAVES = K <= 64 ? 3 : 2;
};

__host__ __device__ constexpr int plane_pos(int i, int M) { return (i % 8) * (M / 8) + i / 8; }
__host__ __device__ constexpr int coord_at(int pos, int M) { return 8 * (pos % (M / 8)) + pos / (M / 8); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two f32 -> packed bf16 (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// bf16-pair sign masks of lane part q. One lane per vector: the kernel-argument table itself
// (uniform index -> scalar loads). Several lanes per vector: an LDS copy indexed by part.
template <int M>
__device__ __forceinline__ void build_sign_table(const Tables& tab, uint32_t* s_sign) {
  if constexpr (LV<M>::Q > 1)
    for (int w = threadIdx.x; w < M / 2; w += blockDim.x) s_sign[w] = tab.sign_pairs[w];
}

template <int M>
__device__ __forceinline__ const uint32_t* part_signs(const Tables& tab, const uint32_t* s_sign, int q) {
  if constexpr (LV<M>::Q == 1) return tab.sign_pairs;
  else return s_sign + q * (LV<M>::K / 2);
}

// Load K bf16 coordinates from `row` (16-byte aligned, always readable: callers pass a clamped
// row for lanes past the end), flip signs with the masks `sm` (entry 0 = coordinates 0, 1 of
// this part), convert to f32; returns the sum of squares.
// Materialise every value of v here: an empty asm that reads and writes each register, so no
// arithmetic of a later phase can be hoisted above this point (the unrolled transform is one
// large DAG; scheduled freely it needs far more registers than the K values it updates).
template <int K>
__device__ __forceinline__ void pin(float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" : "+v"(v[i]));
}

// Radix-8 butterflies (index bits 0..2) of the 8 consecutive values v[b .. b+8).
template <int K>
__device__ __forceinline__ void fwht8(float (&v)[K], int b) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((e & h) == 0) {
        const float x = v[b + e], y = v[b + e + h];
        v[b + e] = x + y;
        v[b + e + h] = x - y;
      }
}

// Wave staging tile in LDS: the 64 lane parts of a wave, part p as K/8 16-byte chunks plus one
// chunk of padding (row stride = 4 mod 64 dwords: the 16-byte accesses of 16 lanes hit 64
// distinct banks). Global memory is touched in 1 KB contiguous pieces (chunk id = 64 k + lane),
// registers row by row (lane p reads part p).
template <int K>
struct Stage {
  static constexpr int CH = K / 8;      // chunks per lane part
  static constexpr int S = CH + 1;      // padded row stride, chunks
  static constexpr int WORDS = 64 * S;  // uint4 per wave
};

// Coalesced load of the bf16 row parts of the wave's 64/Q vectors into its tile; row_of(j)
// gives the first element of vector j of the wave (always a readable row).
template <int M, class RowFn>
__device__ __forceinline__ void stage_rows_in(RowFn row_of, uint4* tile) {
  using L = LV<M>;
  using St = Stage<L::K>;
  const int lane = threadIdx.x & 63;
  uint4 r[St::CH];
#pragma unroll
  for (int k = 0; k < St::CH; ++k) {
    const int id = k * 64 + lane, p = id / St::CH, c = id % St::CH;
    r[k] = ld_stream(reinterpret_cast<const uint4*>(row_of(p / L::Q) + (p % L::Q) * L::K) + c);
  }
#pragma unroll
  for (int k = 0; k < St::CH; ++k) {
    const int id = k * 64 + lane, p = id / St::CH, c = id % St::CH;
    tile[p * St::S + c] = r[k];
  }
  __builtin_amdgcn_wave_barrier();
}

// stage_rows_in for the rows x + (vec0 + j) ld, rows >= n repeating the last row. Part k of the
// lane is a fixed row and column offset plus k (64 / (CH Q)) rows, so every load adds a uniform
// stride to the lane's first row instead of forming a 64-bit row product.
template <int M>
__device__ __forceinline__ void stage_rows_linear(const uint16_t* __restrict__ x, int64_t ld,
                                                  int64_t vec0, int64_t n, uint4* tile) {
  using L = LV<M>;
  using St = Stage<L::K>;
  constexpr int CH = St::CH, JK = 64 / (CH * L::Q);  // vectors advanced per load
  static_assert(64 % CH == 0 && (64 / CH) % L::Q == 0, "row parts per load");
  const int lane = threadIdx.x & 63;
  const int j0 = (lane / CH) / L::Q, col = ((lane / CH) % L::Q) * L::K + 8 * (lane % CH);
  const uint16_t* first = x + (vec0 + j0) * ld + col;
  const uint16_t* last = x + (n - 1) * ld + col;
  uint4 r[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const bool in = vec0 + j0 + JK * k < n;
    r[k] = ld_stream(in ? first + JK * k * ld : last);
  }
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int id = k * 64 + lane, p = id / CH, c = id % CH;
    tile[p * St::S + c] = r[k];
  }
  __builtin_amdgcn_wave_barrier();
}

// Coalesced store of the wave's tile (bf16 row parts) to rows vec0 .. (rows >= n skipped).
template <int M>
__device__ __forceinline__ void stage_rows_out(uint16_t* __restrict__ y, int64_t ld, int64_t vec0,
                                               int64_t n, const uint4* tile) {
  using L = LV<M>;
  using St = Stage<L::K>;
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < St::CH; ++k) {
    const int id = k * 64 + lane, p = id / St::CH, c = id % St::CH;
    const int64_t vec = vec0 + p / L::Q;
    const uint4 d = tile[p * St::S + c];
    if (vec < n) st_stream(reinterpret_cast<uint4*>(y + vec * ld + (p % L::Q) * L::K) + c, d);
  }
}

template <int K>
__device__ __forceinline__ float load_part(const uint4* row, const uint32_t* sm, float (&v)[K]) {
  float ss = 0.0f;
  uint4 raw[K / 8];
#pragma unroll
  for (int c = 0; c < K / 8; ++c) raw[c] = row[c];
#pragma unroll
  for (int c = 0; c < K / 8; ++c) {
    const uint4 m = *reinterpret_cast<const uint4*>(sm + 4 * c);
    const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
    const uint32_t f[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]),
                                           __builtin_bit_cast(bf16x2_t, w[e]), ss, false);
      const uint32_t x = w[e] ^ f[e];
      v[8 * c + 2 * e] = __uint_as_float(x << 16);
      v[8 * c + 2 * e + 1] = __uint_as_float(x & 0xFFFF0000u);
    }
    fwht8<K>(v, 8 * c);  // first radix-8 pass of the rotation, as soon as the chunk is here
  }
  pin<K>(v);
  asm volatile("" : "+v"(ss));  // finish the sum now: the raw chunks must die here
  return ss;
}

// In-register unnormalised Walsh-Hadamard transform of K values (Sylvester order), from index
// bit log2(FIRST) on (FIRST = 8: the first radix-8 pass was done by load_part).
template <int K, int FIRST = 1>
__device__ __forceinline__ void fwht_regs(float (&v)[K]) {
  // Radix-8 passes over index bits [s, s+3): each group of 8 elements with stride 2^s runs its
  // three butterfly stages to completion before the next group, so the working set stays small
  // and every value is updated in place.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = FIRST; s < K; s <<= 3) {
    const int span = (s << 3) <= K ? 8 : K / s;  // elements per group in this pass
#pragma unroll
    for (int hi = 0; hi < K / (s * span); ++hi)
#pragma unroll
      for (int lo = 0; lo < s; ++lo) {
        const int base = hi * s * span + lo;  // lowest element of the group
#pragma unroll
        for (int h = 1; h < span; h <<= 1)
#pragma unroll
          for (int e = 0; e < span; ++e)
            if ((e & h) == 0) {
              const int j = base + e * s, k = base + (e + h) * s;
              const float a = v[j], b = v[k];
              v[j] = a + b;
              v[k] = a - b;
            }
      }
    pin<K>(v);
  }
}

// Partner value across a quad: mask 1 -> lane ^ 1, mask 2 -> lane ^ 2.
template <int MASK>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int ctrl = MASK == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, true));
}

// Butterfly stages over the lane-part bits (coordinate bits log2 K ..): the part whose bit is 0
// receives a + b, the other a - b; written as fma(v, sign, partner) so the DPP move folds.
template <int Q, int K>
__device__ __forceinline__ void fwht_cross(float (&v)[K], int q) {
  if constexpr (Q >= 2) {
    const float sg = (q & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = fmaf(v[k], sg, quad_xor<1>(v[k]));
  }
  if constexpr (Q >= 4) {
    const float sg = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = fmaf(v[k], sg, quad_xor<2>(v[k]));
  }
}

template <int Q>
__device__ __forceinline__ float part_sum(float x) {
  if constexpr (Q >= 2) x += quad_xor<1>(x);
  if constexpr (Q >= 4) x += quad_xor<2>(x);
  return x;
}

template <int Q>
__device__ __forceinline__ uint32_t part_max_u32(uint32_t x) {
  if constexpr (Q >= 2) {
    const uint32_t y = __float_as_uint(quad_xor<1>(__uint_as_float(x)));
    x = x > y ? x : y;
  }
  if constexpr (Q >= 4) {
    const uint32_t y = __float_as_uint(quad_xor<2>(__uint_as_float(x)));
    x = x > y ? x : y;
  }
  return x;
}

// Norm of a vector whose lane part's raw bf16 chunks sit at `row` (K/8 chunks, LDS), given the
// plain f32 sum of squares already summed over the vector's Q lanes; rescaled (see
// ss_out_of_range) where that sum left the f32 range. Call from wave-uniform control flow.
template <int K, int Q>
__device__ __forceinline__ float safe_norm_lv(float ss, const uint4* row) {
  const bool bad = ss_out_of_range(ss);
  float n = sqrtf(ss);
  if (wave_any(bad)) {
    uint32_t mb = 0;
#pragma unroll
    for (int c = 0; c < K / 8; ++c) {
      const uint32_t m = chunk_max_mag_bits(row[c]);
      mb = mb > m ? mb : m;
    }
    const int e = max_exp_of_bits(part_max_u32<Q>(mb));
    const float sc = pow2f(-e);
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < K / 8; ++c) s2 = chunk_scaled_ss(row[c], sc, s2);
    const float n2 = sqrtf(part_sum<Q>(s2)) * pow2f(e);
    n = bad ? n2 : n;
  }
  return n;
}

// The same for a vector held as f32 coordinates (K per lane, Q lanes; projection outputs).
template <int K, int Q>
__device__ __forceinline__ float safe_norm_f32(float ss, const float (&v)[K]) {
  const bool bad = ss_out_of_range(ss);
  float n = sqrtf(ss);
  if (wave_any(bad)) {
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t m = __float_as_uint(v[i]) & 0x7FFFFFFFu;
      mb = mb > m ? mb : m;
    }
    const int e = max_exp_of_bits(part_max_u32<Q>(mb));
    const float sc = pow2f(-e);
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float a = v[i] * sc;
      s2 = fmaf(a, a, s2);
    }
    const float n2 = sqrtf(part_sum<Q>(s2)) * pow2f(e);
    n = bad ? n2 : n;
  }
  return n;
}

__device__ __forceinline__ uint32_t shift_in(uint32_t w, bool bit) { return w + w + (bit ? 1u : 0u); }

// (acc << 1) | sign bit of x: one v_alignbit_b32.
__device__ __forceinline__ uint32_t shift_in_sign(uint32_t acc, float x) {
  return __builtin_amdgcn_alignbit(acc, __float_as_uint(x), 31);
}

// Keeps the compiler from hoisting work across a phase boundary (register pressure).
__device__ __forceinline__ void phase_fence() { __builtin_amdgcn_sched_barrier(0); }

// Quantiser. For a coordinate x of the rotated vector (norm n) the code is
// #{k : x/n > t_k} [kakeyaturbo PR #15, "M4 Phase A": nearest centroid, ties to the lower cell].
// Each compare is made arithmetic: (n t_k - x) is negative exactly when x > n t_k (a zero
// difference is +0, i.e. "not greater"), so its sign bit, shifted into a per-threshold word
// with one v_alignbit, is the compare result — no divide, no compare mask, no scalar register.
//   SYM (antisymmetric table: middle threshold 0, the others in +-tau pairs): top plane =
//   (x > 0), taken from the sign bit of x; lower planes = bits of #{k : |x| > n tau_k},
//   complemented where x <= 0. Equal to the count above except exactly on a threshold.
//   otherwise: thermometer words x > n t_k for all 2^b - 1 thresholds.
// The plane words are then formed with word-wide logic (32 coordinates per operation).
template <int BITS, bool SYM>
struct Quant {
  static constexpr int L = 1 << BITS;
  static constexpr int NT = SYM ? L / 2 - 1 : L - 1;  // thresholds compared per coordinate
  float thr[NT > 0 ? NT : 1];
  bool nz;

  __device__ __forceinline__ Quant(const Tables& tab, float n) {
    nz = n > 0.0f;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      if constexpr (SYM) {
        thr[k] = n * tab.t[L / 2 + k];
      } else {  // n == 0: x = 0 and z = 0, so the compare is just 0 > t_k
        thr[k] = nz ? n * tab.t[k] : (tab.t[k] < 0.0f ? -1.0f : 1.0f);
      }
    }
  }
};

template <int BITS, bool SYM>
struct QuantAcc {
  static constexpr int NT = Quant<BITS, SYM>::NT;
  uint32_t sgn;
  uint32_t a[NT > 0 ? NT : 1];

  __device__ __forceinline__ QuantAcc() : sgn(0u) {
#pragma unroll
    for (int k = 0; k < (NT > 0 ? NT : 1); ++k) a[k] = 0u;
  }

  __device__ __forceinline__ void push(float x, const Quant<BITS, SYM>& q) {
    if constexpr (SYM) {
      sgn = shift_in_sign(sgn, x);
#pragma unroll
      for (int k = 0; k < NT; ++k) a[k] = shift_in_sign(a[k], q.thr[k] - fabsf(x));
    } else {
#pragma unroll
      for (int k = 0; k < NT; ++k) a[k] = shift_in_sign(a[k], q.thr[k] - x);
    }
  }

  // Plane words of the collected bits (valid = mask of the bit positions pushed).
  __device__ __forceinline__ void planes(const Quant<BITS, SYM>& q, uint32_t valid,
                                         uint32_t (&pl)[BITS]) const {
    constexpr int L = 1 << BITS;
    if constexpr (SYM) {
      const uint32_t pos = q.nz ? (~sgn & valid) : 0u;
#pragma unroll
      for (int p = 0; p < BITS - 1; ++p) {
        uint32_t cp = 0u;
#pragma unroll
        for (int v = 1; v <= NT; ++v)
          if ((v >> p) & 1) cp |= a[v - 1] & (v < NT ? ~a[v] : ~0u);
        pl[p] = ~(cp ^ pos) & valid;
      }
      pl[BITS - 1] = pos;
    } else {
#pragma unroll
      for (int p = 0; p < BITS; ++p) {
        uint32_t cp = 0u;
#pragma unroll
        for (int v = 1; v < L; ++v)
          if ((v >> p) & 1) cp |= a[v - 1] & (v < L - 1 ? ~a[v] : ~0u);
        pl[p] = cp & valid;
      }
    }
  }
};

// The centroid the quantiser picks for rotated coordinate u (code = #{k : u > n t_k}), decided
// with the quantiser's own thresholds. Symmetric tables: the magnitude cell from |u|, the sign
// from u (u <= 0 takes the lower half: c[L/2 - 1 - j] = -c[L/2 + j]).
// QT: a quantiser holding those thresholds times the norm in thr[] (Quant, or the binary-search
// one of the Kronecker encode: both keep the same NT thresholds) and whether the norm is > 0.
template <int BITS, bool SYM, class QT>
__device__ __forceinline__ float chosen_centroid(float u, const QT& q, const Tables& tab) {
  constexpr int L = 1 << BITS, NT = SYM ? L / 2 - 1 : L - 1;
  int cnt = 0;
  if constexpr (SYM) {
#pragma unroll
    for (int k = 0; k < NT; ++k) cnt += fabsf(u) > q.thr[k] ? 1 : 0;
    float mag = tab.c[L / 2];
#pragma unroll
    for (int j = 1; j < L / 2; ++j) mag = cnt == j ? tab.c[L / 2 + j] : mag;
    return (q.nz && u > 0.0f) ? mag : -mag;
  } else {
#pragma unroll
    for (int k = 0; k < NT; ++k) cnt += u > q.thr[k] ? 1 : 0;
    float c = tab.c[0];
#pragma unroll
    for (int j = 1; j < L; ++j) c = cnt == j ? tab.c[j] : c;
    return c;
  }
}

// Stored scale of a rule from n = ||v||, zu = sum_i u_i z^_i (u = H (s .* v) = n z) and
// zz = sum_i z^_i^2 [turboquant_plus log: EDEN and matched-norm scales]. Decode gives
// x^ = (scale/m) s .* H z^, so: 1 matched norm n sqrt(m / zz) (||x^|| = ||v||); 2 inner-product
// preserving n^2 m / zu (<x^, v> = ||v||^2); 3 least squares zu / zz (<v - x^, x^> = 0).
// A rule whose denominator is not positive keeps the norm.
__device__ __forceinline__ float rule_scale(int rule, float n, float zu, float zz, int m) {
  if (rule == 1 && zz > 0.0f) return n * sqrtf((float)m / zz);
  if (rule == 2 && zu > 0.0f) return n * (n * (float)m / zu);
  if (rule == 3 && zz > 0.0f) return zu / zz;
  return n;
}

// All record code words of a lane-owned vector (Q == 1): out[g*BITS + p]. Word g, bit t holds
// the coordinate at plane position 32g + t; bits are shifted in from t = 31 down to 0.
template <int M, int BITS, bool SYM>
__device__ __forceinline__ void pack_vector(float (&u)[M], float n, const Tables& tab,
                                            uint32_t (&out)[(M / 32) * BITS]) {
  const Quant<BITS, SYM> q(tab, n);
#pragma unroll
  for (int g = 0; g < M / 32; ++g) {
    QuantAcc<BITS, SYM> acc;
#pragma unroll
    for (int t = 31; t >= 0; --t) acc.push(u[coord_at(32 * g + t, M)], q);
    uint32_t pl[BITS];
    acc.planes(q, 0xFFFFFFFFu, pl);
#pragma unroll
    for (int p = 0; p < BITS; ++p) out[g * BITS + p] = pl[p];
    // the later words' compares may not be hoisted above this word: pin only the coordinates
    // still to be quantised (pinning used ones would keep them alive)
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (plane_pos(i, M) / 32 > g) asm volatile("" : "+v"(u[i]));
  }
}

// Q > 1: this part's 16-bit halves of its 8 words per plane. Part q holds coordinates
// qK + k; coordinate k with k mod 8 = s sits at bit 16 (q mod 2) + k/8 of word
// s (M = 256) or 2s + q/2 (M = 512). half[s][p] holds those 16 bits in its low half.
template <int M, int BITS, bool SYM>
__device__ __forceinline__ void pack_part(float (&u)[128], float n, const Tables& tab,
                                          uint32_t (&half)[8][BITS]) {
  const Quant<BITS, SYM> q(tab, n);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    QuantAcc<BITS, SYM> acc;
#pragma unroll
    for (int t = 15; t >= 0; --t) acc.push(u[8 * t + s], q);
    acc.planes(q, 0xFFFFu, half[s]);
#pragma unroll
    for (int k = 0; k < 128; ++k)
      if (k % 8 > s) asm volatile("" : "+v"(u[k]));
  }
}

// Store a record held entirely by one lane (NWT dwords, 4-byte aligned) with 16-byte pieces.
template <int NWT>
__device__ __forceinline__ void store_words(uint32_t* __restrict__ dst, const uint32_t (&w)[NWT]) {
#pragma unroll
  for (int i = 0; i + 4 <= NWT; i += 4)
    *reinterpret_cast<uint4*>(dst + i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
  if constexpr (NWT % 4 == 3)
    *reinterpret_cast<uint3*>(dst + NWT - 3) = make_uint3(w[NWT - 3], w[NWT - 2], w[NWT - 1]);
  if constexpr (NWT % 4 == 2)
    *reinterpret_cast<uint2*>(dst + NWT - 2) = make_uint2(w[NWT - 2], w[NWT - 1]);
  if constexpr (NWT % 4 == 1) dst[NWT - 1] = w[NWT - 1];
}

template <int NWT>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ src, uint32_t (&w)[NWT]) {
#pragma unroll
  for (int i = 0; i + 4 <= NWT; i += 4) {
    const uint4 x = ld_stream(src + i);
    w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
  }
#pragma unroll
  for (int i = (NWT / 4) * 4; i < NWT; ++i) w[i] = src[i];
}

// Encode one vector part (rotated coordinates u, norm n) and store the record with `stored` as
// its scale (the norm itself, or a scale rule's value).
// Q == 1: the lane writes its whole record. Q > 1: lanes of a pair (q, q^1) merge their
// halves; each lane of the pair stores the words of every other slot s; part 0 writes the norm.
template <int M, int BITS, bool SYM>
__device__ __forceinline__ void quantize_store_lv(float (&u)[LV<M>::K], float n, float stored,
                                                  bool valid, int q, const Tables& tab,
                                                  uint32_t* __restrict__ rec) {
  constexpr int Q = LV<M>::Q, NWC = (M / 32) * BITS, NWT = NWC + 1;
  if constexpr (Q == 1) {
    uint32_t w[NWT];
    uint32_t (&cw)[NWC] = *reinterpret_cast<uint32_t(*)[NWC]>(w);
    pack_vector<M, BITS, SYM>(u, n, tab, cw);
    w[NWC] = __float_as_uint(stored);
    if (valid) store_words<NWT>(rec, w);
  } else {
    uint32_t half[8][BITS];
    pack_part<M, BITS, SYM>(u, n, tab, half);
    const bool odd = q & 1;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t word[BITS];
#pragma unroll
      for (int p = 0; p < BITS; ++p) {
        const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)half[s][p], 0xB1, 0xF, 0xF, true);
        word[p] = odd ? (other | (half[s][p] << 16)) : (half[s][p] | (other << 16));
      }
      const int g = (M == 256) ? s : 2 * s + (q >> 1);
      if (valid && ((s & 1) == (int)odd)) {
        uint32_t* d = rec + g * BITS;
        if constexpr (BITS == 4) *reinterpret_cast<uint4*>(d) = make_uint4(word[0], word[1], word[2], word[3]);
        if constexpr (BITS == 3) *reinterpret_cast<uint3*>(d) = make_uint3(word[0], word[1], word[2]);
        if constexpr (BITS == 2) *reinterpret_cast<uint2*>(d) = make_uint2(word[0], word[1]);
        if constexpr (BITS == 1) d[0] = word[0];
      }
    }
    if (valid && q == 0) rec[NWC] = __float_as_uint(stored);
  }
}

// Centroid tables for the unpacking below: in LDS, or held by lanes 0..15 of one register and
// fetched with a cross-lane permute (no LDS space needed).
struct LdsLut {
  const float* p;
  __device__ __forceinline__ float operator()(uint32_t code) const { return p[code]; }
};
struct LaneLut {
  int v;  // bits of centroid (lane % 16)
  __device__ __forceinline__ explicit LaneLut(const Tables& tab) : v(0) {
    const int l = __lane_id() & 15;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k) v = l == k ? __float_as_int(tab.c[k]) : v;
  }
  __device__ __forceinline__ float operator()(uint32_t code) const {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)(code << 2), v));
  }
};

// Codes of a whole record (one lane per vector) looked up in lut, the record's code words
// already in registers (lets a caller load them early).
template <int M, int BITS, class Lut>
__device__ __forceinline__ void unpack_lookup_words(const uint32_t (&w)[(M / 32) * BITS],
                                                    const Lut& lut, float (&zh)[M]) {
#pragma unroll
  for (int k = 0; k < M; ++k) {
    const int pos = plane_pos(k, M);
    uint32_t code = 0;
#pragma unroll
    for (int p = 0; p < BITS; ++p) code |= ((w[(pos >> 5) * BITS + p] >> (pos & 31)) & 1u) << p;
    zh[k] = lut(code);
  }
}

}  // namespace kvq
