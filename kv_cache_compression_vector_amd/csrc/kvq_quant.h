// kvq_quant.h — quantiser + record writer shared by every encode kernel.
//
// code_i = #{k : z_i > t_k} (nearest centroid, ties to the lower cell) [kakeyaturbo PR #15,
// "M4 Phase A"]; the compare masks are wave ballots; with the lane layout of kvq_device.h the
// ballot of bit p of slot j's code is the record's plane p at positions j*(M/8) + c.
#pragma once

#include "kvq_device.h"

namespace kvq {

// Bit-planes of the codes of one slot (one coordinate per lane) for the whole wave.
//  SYM: the table is antisymmetric (c_{L-1-k} = -c_k exactly, so the middle threshold is 0 and
//       the thresholds come in +-pairs). Top plane = (z > 0); the remaining planes come from the
//       count of positive thresholds below |z|, complemented for negative z. This agrees with
//       #{k : z > t_k} everywhere except exactly on a threshold.
//  otherwise: thermometer masks z > t_k and the planes of their count.
template <int BITS, bool SYM>
__device__ __forceinline__ void code_planes(float z, const Tables& tab, uint64_t (&pl)[BITS]) {
  constexpr int L = 1 << BITS;
  if constexpr (SYM) {
    const uint64_t pos = ballot64(z > 0.0f);
    const float az = fabsf(z);
    uint64_t a[L / 2 + 1];
    a[0] = ~0ull;
#pragma unroll
    for (int k = 1; k < L / 2; ++k) a[k] = ballot64(az > tab.t[L / 2 - 1 + k]);
    a[L / 2] = 0ull;
#pragma unroll
    for (int p = 0; p < BITS - 1; ++p) {
      uint64_t cp = 0;
#pragma unroll
      for (int v = 1; v < L / 2; ++v)
        if ((v >> p) & 1) cp |= a[v] & ~a[v + 1];
      pl[p] = ~(cp ^ pos);
    }
    pl[BITS - 1] = pos;
  } else {
    uint64_t mk[L];
#pragma unroll
    for (int k = 0; k < L - 1; ++k) mk[k] = ballot64(z > tab.t[k]);
    mk[L - 1] = 0ull;
#pragma unroll
    for (int p = 0; p < BITS; ++p) {
      uint64_t cp = 0;
#pragma unroll
      for (int v = 1; v < L; ++v)
        if ((v >> p) & 1) cp |= mk[v - 1] & ~mk[v];
      pl[p] = cp;
    }
  }
}

// Record word (g, p) of the vector held by lanes [s*LPV, s*LPV + LPV), from the per-slot planes.
template <int M, int BITS>
__device__ __forceinline__ uint32_t record_word(const uint64_t (&pl)[8][BITS], int s, int g, int p) {
  constexpr int LPV = M / 8;
  if constexpr (LPV >= 32) {
    const int j = (32 * g) / LPV, c0 = (32 * g) % LPV;
    return (uint32_t)(pl[j][p] >> (s * LPV + c0));
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 32 / LPV; ++e) {
      const int j = (32 * g) / LPV + e;
      w |= (uint32_t)((pl[j][p] >> (s * LPV)) & low_mask(LPV)) << (e * LPV);
    }
    return w;
  }
}

// Move every record word of the wave's vectors from scalar registers into its storing lane:
// word w of vector s goes to lane s*LPV + w % LPV of out[w / LPV].
template <int M, int BITS, int IDX, int NOUT>
__device__ __forceinline__ void store_words(const uint64_t (&pl)[8][BITS], uint32_t (&out)[NOUT]) {
  constexpr int LPV = M / 8, VPW = 64 / LPV, NWC = (M / 32) * BITS;
  if constexpr (IDX < VPW * NWC) {
    constexpr int s = IDX / NWC, w = IDX % NWC, g = w / BITS, p = w % BITS;
    out[w / LPV] = write_lane<s * LPV + (w % LPV)>(record_word<M, BITS>(pl, s, g, p), out[w / LPV]);
    store_words<M, BITS, IDX + 1, NOUT>(pl, out);
  }
}

// Quantise the rotated coordinates u[8] (norm n) of every vector of the wave and store the
// records. Lanes of vectors that do not exist (valid == false) take part in the ballots only.
template <int M, int BITS, bool SYM>
__device__ __forceinline__ void quantize_store(const float (&u)[8], float n, bool valid,
                                               int64_t vec, int sub, int c, const Tables& tab,
                                               uint8_t* __restrict__ rec) {
  constexpr int LPV = M / 8, NWC = (M / 32) * BITS, NWT = NWC + 1;
  constexpr int NOUT = (NWT + LPV - 1) / LPV;
  const float rn = n > 0.0f ? 1.0f / n : 0.0f;
  uint64_t pl[8][BITS];
#pragma unroll
  for (int j = 0; j < 8; ++j) code_planes<BITS, SYM>(u[j] * rn, tab, pl[j]);
  uint32_t out[NOUT];
#pragma unroll
  for (int r = 0; r < NOUT; ++r) out[r] = 0u;
  store_words<M, BITS, 0, NOUT>(pl, out);
  // the norm word: lane (NWC % LPV) of each vector, register NWC / LPV
  if (c == NWC % LPV) out[NWC / LPV] = __float_as_uint(n);
  if (valid) {
    uint32_t* r32 = reinterpret_cast<uint32_t*>(rec + vec * (int64_t)(NWT * 4));
#pragma unroll
    for (int r = 0; r < NOUT; ++r) {
      const int w = r * LPV + c;
      if (w < NWT) r32[w] = out[r];
    }
  }
}

// Load the 8 coordinates of chunk c of row `vec`, apply the sign diagonal, return f32 values
// and the lane's partial sum of squares.
__device__ __forceinline__ float load_signed_chunk(const uint16_t* __restrict__ row, int c,
                                                   const uint32_t (&sm)[4], bool valid,
                                                   float (&v)[8]) {
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (valid) raw = *reinterpret_cast<const uint4*>(row + 8 * c);
  const uint32_t w[4] = {raw.x ^ sm[0], raw.y ^ sm[1], raw.z ^ sm[2], raw.w ^ sm[3]};
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16lo_to_f32(w[k]);
    v[2 * k + 1] = bf16hi_to_f32(w[k]);
    ss = fmaf(v[2 * k], v[2 * k], ss);
    ss = fmaf(v[2 * k + 1], v[2 * k + 1], ss);
  }
  return ss;
}

}  // namespace kvq
