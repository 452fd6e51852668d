// kvq_score.hip — raw attention logits straight from packed K records.
//
// score[b][h][t] = q[b][h] . x^[b][kv][t] = (n_t/M) sum_i q'_i z^_{t,i},  q' = H_M (s (.) q):
// the sign diagonal and the Hadamard matrix are symmetric, so rotating the query once replaces
// decoding every key [arc PR #98/#94 kernel commit: attention reads packed K directly;
// turboquant_plus MLX notes: decode attention on a compact cache]. The query heads that share
// a KV head (GQA) are scored together so every record is read once.
#include "kvq_device.h"
#include "kvq_kernels.h"

namespace kvq {

constexpr int kScoreThreads = 256;

// q' of the G query heads of one (batch, kv head), written to LDS in plane-position order:
// qs[pos * G + h] = q'_h[i] with pos = (i mod 8) * (M/8) + i/8.
template <int M, int G>
__device__ __forceinline__ void rotate_queries(const ScoreArgs& a, int b, int kv, float* qs) {
  constexpr int LPV = M / 8;
  constexpr int HPB = kScoreThreads / LPV;  // heads per pass
  const int c = threadIdx.x % LPV;
  uint32_t sm[4];
  chunk_sign_masks<M>(a.tab, c, sm);
  for (int h0 = 0; h0 < G; h0 += HPB) {
    const int h = h0 + (int)threadIdx.x / LPV;
    const bool active = h < G;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (active)
      raw = *reinterpret_cast<const uint4*>(a.q + b * a.q_sb + (int64_t)(kv * G + h) * a.q_sh + 8 * c);
    const uint32_t w[4] = {raw.x ^ sm[0], raw.y ^ sm[1], raw.z ^ sm[2], raw.w ^ sm[3]};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16lo_to_f32(w[k]);
      v[2 * k + 1] = bf16hi_to_f32(w[k]);
    }
    fwht_vector<LPV>(v, c);
    if (active) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qs[(j * LPV + c) * G + h] = v[j];
    }
  }
}

template <int M, int BITS, int G>
__global__ __launch_bounds__(kScoreThreads) void k_score(ScoreArgs a) {
  constexpr int NWC = (M / 32) * BITS, NWT = NWC + 1;
  __shared__ float qs[M * G];
  __shared__ float lut[16];
  const int pair = blockIdx.y;
  const int b = pair / a.Hkv, kv = pair % a.Hkv;
  if (threadIdx.x < 16) lut[threadIdx.x] = a.tab.c[threadIdx.x];
  rotate_queries<M, G>(a, b, kv, qs);
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kScoreThreads + threadIdx.x;
  if (t >= a.T) return;
  const uint32_t* r32 =
      reinterpret_cast<const uint32_t*>(a.rec) + (b * a.rec_sb + kv * a.rec_sh + t) * NWT;
  float acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.0f;
#pragma unroll
  for (int g = 0; g < M / 32; ++g) {
    uint32_t W[BITS];
#pragma unroll
    for (int p = 0; p < BITS; ++p) W[p] = r32[g * BITS + p];
#pragma unroll 4
    for (int jb = 0; jb < 32; ++jb) {
      uint32_t code = 0;
#pragma unroll
      for (int p = 0; p < BITS; ++p) code |= ((W[p] >> jb) & 1u) << p;
      const float cv = lut[code];
      const float* qrow = qs + (32 * g + jb) * G;
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(qrow[h], cv, acc[h]);
    }
  }
  const float scale = __uint_as_float(r32[NWC]) * a.tab.inv_m;
  float* srow = a.s + b * a.s_sb + t;
#pragma unroll
  for (int h = 0; h < G; ++h) srow[(int64_t)(kv * G + h) * a.s_sh] = acc[h] * scale;
}

template <int M, int BITS>
static hipError_t launch_score_t(int group, const ScoreArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.T + kScoreThreads - 1) / kScoreThreads), (unsigned)(a.B * a.Hkv));
  const dim3 blk(kScoreThreads);
  switch (group) {
    case 1: hipLaunchKernelGGL((k_score<M, BITS, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_score<M, BITS, 2>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_score<M, BITS, 4>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_score<M, BITS, 8>), grid, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int M>
static hipError_t launch_score_m(int bits, int group, const ScoreArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return launch_score_t<M, 1>(group, a, st);
    case 2: return launch_score_t<M, 2>(group, a, st);
    case 3: return launch_score_t<M, 3>(group, a, st);
    case 4: return launch_score_t<M, 4>(group, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score(int D, int m, int bits, int group, const ScoreArgs& a, hipStream_t st) {
  if (D != m) return hipErrorInvalidValue;
  if (a.T <= 0 || a.B <= 0 || a.Hkv <= 0) return hipSuccess;
  switch (m) {
    case 64: return launch_score_m<64>(bits, group, a, st);
    case 128: return launch_score_m<128>(bits, group, a, st);
    case 256: return launch_score_m<256>(bits, group, a, st);
    case 512: return launch_score_m<512>(bits, group, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
