// kvq_decode.hip — records (+ optional outlier lists) -> f32 / bf16 rows.
//
// x^ = (n/M) s (.) H_M z^, z^_i = centroid[code_i], outlier entries replacing their coordinate
// before the inverse rotation [kakeyaturbo PR #15, commit "M5": LUT, outlier scatter, y = z^ n,
// x = H y sign / wht_len]. The Hadamard network runs in place (H is its own inverse up to
// 1/M). This file holds the decode with an outlier list at m = 256, 512: the 8-coordinates-
// per-lane layout lets each lane test the entries of its vector. Every other Hadamard shape
// decodes on the matrix cores (kvq_decode_h.hip).
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_lanevec.h"

namespace kvq {

// Codes of the 8 coordinates of chunk c, looked up in the centroid table in LDS.
template <int M, int BITS>
__device__ __forceinline__ void unpack_lookup(const uint32_t* __restrict__ r32, int c,
                                              const float* __restrict__ lut, float (&zh)[8]) {
  constexpr int LPV = M / 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = j * LPV + c;
    const int g = pos >> 5, bit = pos & 31;
    uint32_t code = 0;
#pragma unroll
    for (int p = 0; p < BITS; ++p) code |= ((r32[g * BITS + p] >> bit) & 1u) << p;
    zh[j] = lut[code];
  }
}

template <int M, int BITS, bool OL, bool BF16>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
  constexpr int LPV = M / 8, VPW = 64 / LPV, NWC = (M / 32) * BITS, NWT = NWC + 1;
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = a.tab.c[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPV, c = lane % LPV;
  const uint32_t sbyte = (a.tab.sign_words[(c >> 2) & 15] >> (8 * (c & 3))) & 0xFFu;
  const int64_t n_iter = (a.n + VPW - 1) / VPW;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < n_iter; it += (int64_t)gridDim.x * 4) {
    const int64_t vec = it * VPW + sub;
    if (vec >= a.n) continue;  // no cross-vector communication below: whole vectors drop out
    const uint32_t* r32 = reinterpret_cast<const uint32_t*>(a.rec) + vec * NWT;
    float zh[8];
    unpack_lookup<M, BITS>(r32, c, lut, zh);
    const float nrm = __uint_as_float(r32[NWC]);
    if constexpr (OL) {
      int64_t e0 = a.ol_off[vec], e1 = a.ol_off[vec + 1];
      if (e1 > a.ol_cap) e1 = a.ol_cap;
      for (int64_t e = e0; e < e1; ++e) {
        const int idx = M > 256 ? (int)static_cast<const uint16_t*>(a.ol_idx)[e]
                                : (int)static_cast<const uint8_t*>(a.ol_idx)[e];
        const float val = __uint_as_float((uint32_t)a.ol_val[e] << 16);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (idx == 8 * c + j) zh[j] = val;
      }
    }
    fwht_vector<LPV>(zh, c);
    const float scale = nrm * a.tab.inv_m;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      zh[j] = __uint_as_float(__float_as_uint(zh[j] * scale) ^ (((sbyte >> j) & 1u) << 31));
    if constexpr (BF16) {
      uint4 o;
      o.x = pack_bf16x2(zh[0], zh[1]);
      o.y = pack_bf16x2(zh[2], zh[3]);
      o.z = pack_bf16x2(zh[4], zh[5]);
      o.w = pack_bf16x2(zh[6], zh[7]);
      st_stream(static_cast<uint16_t*>(a.y) + vec * a.ld + 8 * c, o);  // rows are written once
    } else {
      float* yr = static_cast<float*>(a.y) + vec * a.ld + 8 * c;
      *reinterpret_cast<float4*>(yr) = make_float4(zh[0], zh[1], zh[2], zh[3]);
      *reinterpret_cast<float4*>(yr + 4) = make_float4(zh[4], zh[5], zh[6], zh[7]);
    }
  }
}

template <int M, int BITS>
static hipError_t launch_decode_t(bool bf16, const DecodeArgs& a, hipStream_t st) {
  const int vpw = 64 / (M / 8);
  const int64_t n_iter = (a.n + vpw - 1) / vpw;
  int64_t blocks = (n_iter + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return hipSuccess;
  const dim3 g((unsigned)blocks), b(256);
  if (bf16) hipLaunchKernelGGL((k_decode<M, BITS, true, true>), g, b, 0, st, a);
  else hipLaunchKernelGGL((k_decode<M, BITS, true, false>), g, b, 0, st, a);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_decode_m(int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return launch_decode_t<M, 1>(bf16, a, st);
    case 2: return launch_decode_t<M, 2>(bf16, a, st);
    case 3: return launch_decode_t<M, 3>(bf16, a, st);
    case 4: return launch_decode_t<M, 4>(bf16, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int D, int m, bool proj, int bits, bool ol, bool bf16, const DecodeArgs& a,
                         hipStream_t st) {
  if (!proj && decode_h_supported(D, m, ol)) return launch_decode_h(m, bits, bf16, a, st);
  if (proj) {
    if (ol) return hipErrorInvalidValue;  // projection codecs carry no outlier list
    if (decode_pca_h_supported(D, m)) return launch_decode_pca_h(D, m, bits, bf16, a, st);
    return launch_decode_pca(D, m, bits, bf16, a, st);
  }
  if (!ol) return hipErrorInvalidValue;  // every Hadamard shape without a list is above
  // Hadamard codec with an outlier list at m = 256, 512 (two-byte indices)
  switch (m) {
    case 256: return launch_decode_m<256>(bits, bf16, a, st);
    case 512: return launch_decode_m<512>(bits, bf16, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
