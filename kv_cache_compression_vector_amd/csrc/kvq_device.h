// kvq_device.h — device-side building blocks shared by the gfx950 codec kernels.
//
// Lane layout used by every kernel that works on whole vectors: a vector of coded length M is
// held by LPV = M/8 consecutive lanes, lane c holding the 8 consecutive coordinates 8c..8c+7
// (one 16-byte bf16 load). A 64-wide wavefront therefore holds VPW = 64/LPV vectors.
//
// With that layout, ballot of "bit p of the code of slot j" over the wave gives, for each
// vector, the M/8 bits of plane positions j*(M/8) + c, c = 0..M/8-1 — the record's bit-plane
// order pi(i) = (i mod 8)*(M/8) + floor(i/8) — so packing needs only scalar bit moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kMaxLevels = 16;

// Codec tables, passed by value as kernel arguments (they live in the kernarg segment).
struct Tables {
  float t[15];            // decision thresholds, ascending (2^b - 1 used)
  float c[16];            // centroids (2^b used)
  uint32_t sign_words[16];// bit i of the M-bit string = 1 where s_i = -1
  float T;                // outlier threshold (0 = off)
  float inv_m;            // 1/M
  int32_t pad[2];
  // bf16-pair sign masks: entry w flips coordinate 2w (bit 15) and 2w + 1 (bit 31); read with
  // wave-uniform indices, so they come in through scalar loads.
  uint32_t sign_pairs[256];
};

// PCA bases: basis k is bf16 [D][r] at basis + k*D*r, its mean f32 [D] at mean + k*D.
// Rows are grouped in blocks of block_rows; block i uses basis index[i] (count > 1).
struct Basis {
  const uint16_t* basis;
  const float* mean;        // may be null (zero mean)
  const int32_t* index;     // may be null when count <= 1
  int32_t count;
  int32_t block_rows;
};

// Basis of the block holding `row`; an out-of-range index is clamped into [0, count).
__device__ __forceinline__ int basis_of_row(const Basis& b, int64_t row) {
  if (b.count <= 1) return 0;
  int k = b.index[row / b.block_rows];
  k = k < 0 ? 0 : k;
  return k >= b.count ? b.count - 1 : k;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte load / store (data touched once).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, static_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Per-lane XOR masks that flip the bf16 sign bits of the 8 coordinates held by chunk c
// (dword k holds coordinates 2k, 2k+1 in its low / high half).
template <int M>
__device__ __forceinline__ void chunk_sign_masks(const Tables& tab, int c, uint32_t (&sm)[4]) {
  const uint32_t byte = (tab.sign_words[(c >> 2) & 15] >> (8 * (c & 3))) & 0xFFu;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    sm[k] = (((byte >> (2 * k)) & 1u) << 15) | (((byte >> (2 * k + 1)) & 1u) << 31);
}

// Partner value across lanes: lane ^ mask within the wave.
__device__ __forceinline__ float lane_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// lane ^ MASK for a compile-time MASK. Inside a row of 16 lanes the exchange is a DPP move:
// quad permutes [1,0,3,2] (xor 1) and [2,3,0,1] (xor 2), the row rotation by 8 (xor 8), and for
// xor 4 the half-row mirror (xor 7) followed by the quad permute [3,2,1,0] (xor 3). Wider masks
// use the lane-permute path.
template <int MASK>
__device__ __forceinline__ float lane_xor_c(float v) {
  const int x = __float_as_int(v);
  if constexpr (MASK == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  } else if constexpr (MASK == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  } else if constexpr (MASK == 4) {
    const int m = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);
    return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true));
  } else if constexpr (MASK == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));
  } else {
    return __shfl_xor(v, MASK, 64);
  }
}

// Cross-lane butterfly stages MASK, 2 MASK, .. < LPV of fwht_vector.
template <int MASK, int LPV>
__device__ __forceinline__ void fwht_lane_stages(float (&v)[8], int c) {
  if constexpr (MASK < LPV) {
    const bool upper = (c & MASK) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = lane_xor_c<MASK>(v[j]);
      v[j] = upper ? (p - v[j]) : (v[j] + p);
    }
    fwht_lane_stages<2 * MASK, LPV>(v, c);
  }
}

// Unnormalised Walsh-Hadamard transform (Sylvester order) of the M coordinates held by the
// LPV lanes of a vector: coordinate bits 0..2 are the slot index inside the lane, bits 3.. are
// the lane index c. The element whose butterfly bit is 0 receives a + b, the other a - b.
template <int LPV>
__device__ __forceinline__ void fwht_vector(float (&v)[8], int c) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
  fwht_lane_stages<1, LPV>(v, c);
}

// Sum over the LPV lanes of one vector (all of them receive the total).
template <int LPV>
__device__ __forceinline__ float vector_sum(float x) {
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) x += lane_xor(x, m);
  return x;
}

// Integer sum over the LPV lanes of one vector.
template <int LPV>
__device__ __forceinline__ uint32_t vector_sum_u32(uint32_t x) {
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) x += (uint32_t)__shfl_xor((int)x, m, 64);
  return x;
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// v_writelane_b32 through the LLVM intrinsic (not inline asm), so that the compiler's hazard
// recognizer inserts the wait state needed after a VALU write of the SGPR it reads.
extern "C" __device__ int kvq_llvm_writelane_i32(int, int, int) __asm("llvm.amdgcn.writelane.i32");

// Write the wave-uniform value `val` into lane LANE of `old`.
template <int LANE>
__device__ __forceinline__ uint32_t write_lane(uint32_t val, uint32_t old) {
  return (uint32_t)kvq_llvm_writelane_i32((int)__builtin_amdgcn_readfirstlane(val), LANE, (int)old);
}

// Low `bits` bits set.
__host__ __device__ constexpr uint64_t low_mask(int bits) {
  return bits >= 64 ? ~0ull : ((1ull << bits) - 1ull);
}

// ---- Norms over the whole bf16 range ----------------------------------------------------------
// An f32 sum of squares overflows once a row's largest magnitude passes about 2^60 and loses its
// relative precision (then flushes to zero) below about 2^-60, while bf16 rows reach 2^+-127. The
// kernels form the plain sum first; in the rare wave where some vector's sum lies outside
// [2^-100, 2^100) every lane forms its vector's sum again over values multiplied by 2^-e, e the
// exponent of the vector's largest magnitude (a power of two: exact), and that vector's norm is
// sqrt(sum) 2^e. The branch is wave-uniform, so the cross-lane reductions inside it see every lane.

__device__ __forceinline__ bool ss_out_of_range(float ss) { return !(ss >= 0x1p-100f && ss < 0x1p100f); }

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// 2^e as an f32, e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Exponent e of the largest magnitude, from its f32 bit pattern (sign cleared), clamped to
// [-126, 126] so that both 2^e and 2^-e are normal f32 values; 0 for a zero vector.
__device__ __forceinline__ int max_exp_of_bits(uint32_t mag_bits) {
  const int E = (int)(mag_bits >> 23);
  const int e = E == 0 ? -126 : E - 127;
  return e > 126 ? 126 : e;
}

// Largest bf16 magnitude of the 8 coordinates in a 16-byte chunk, as f32 bits.
__device__ __forceinline__ uint32_t chunk_max_mag_bits(const uint4& c) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    m = m > (w[k] & 0x7FFFu) ? m : (w[k] & 0x7FFFu);
    m = m > ((w[k] >> 16) & 0x7FFFu) ? m : ((w[k] >> 16) & 0x7FFFu);
  }
  return m << 16;
}

// Sum of squares of the 8 bf16 coordinates of a chunk, each multiplied by sc first.
__device__ __forceinline__ float chunk_scaled_ss(const uint4& c, float sc, float acc) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = bf16lo_to_f32(w[k]) * sc, b = bf16hi_to_f32(w[k]) * sc;
    acc = fmaf(a, a, acc);
    acc = fmaf(b, b, acc);
  }
  return acc;
}

}  // namespace kvq
