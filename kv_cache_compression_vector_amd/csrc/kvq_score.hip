// kvq_score.hip — raw attention logits straight from packed K records.
//
// score[b][h][t] = q[b][h] . x^[b][kv][t] = (n_t/M) sum_i q'_i z^_{t,i},  q' = H_M (s (.) q):
// the sign diagonal and the Hadamard matrix are symmetric, so rotating the query once replaces
// decoding every key [arc PR #98 / #94 kernel commit: attention reads packed K directly]. With
// a projection, x^ = mu + B v^ gives q.x^ = q.mu + (n/r) sum_i q''_i z^_i, q'' = H_r(s (.) B^T q).
// The query heads that share a KV head (GQA) are scored together so each record is read once.
#include "kvq_device.h"
#include "kvq_kernels.h"

namespace kvq {

constexpr int kScoreThreads = 256;

// Rotated queries of the G (<= GMAX) heads of one (batch, kv head) into LDS, plane-position
// order: qs[pos * GMAX + h], pos = (i mod 8) * (M/8) + i/8; heads h >= G are zero.
// PCA: also qmu[h] = q . mu.
template <int D, int M, int GMAX, bool PCA>
__device__ __forceinline__ void rotate_queries(const ScoreArgs& a, int b, int kv, int G, int64_t row0,
                                               float* qs, float* qf, float* uq, float* qmu) {
  constexpr int LPV = M / 8;
  constexpr int HPB = kScoreThreads / LPV;  // heads per pass
  const int tid = threadIdx.x, c = tid % LPV;
  const uint32_t sbyte = (a.tab.sign_words[(c >> 2) & 15] >> (8 * (c & 3))) & 0xFFu;
  if constexpr (PCA) {
    for (int e = tid; e < GMAX * D; e += kScoreThreads) {
      const int h = e / D, d = e % D;
      qf[e] = h < G ? __uint_as_float((uint32_t)a.q[b * a.q_sb + (int64_t)(kv * G + h) * a.q_sh + d] << 16)
                    : 0.0f;
    }
    __syncthreads();
    const int bi = basis_of_row(a.pca, row0);
    const uint16_t* Bk = a.pca.basis + (int64_t)bi * D * M;
    for (int e = tid; e < GMAX * M; e += kScoreThreads) {
      const int h = e / M, j = e % M;
      float u = 0.0f;
      for (int d = 0; d < D; ++d) u = fmaf(__uint_as_float((uint32_t)Bk[d * M + j] << 16), qf[h * D + d], u);
      uq[e] = u;
    }
    if (tid < GMAX) {
      float s = 0.0f;
      if (a.pca.mean) {
        const float* mu = a.pca.mean + (int64_t)bi * D;
        for (int d = 0; d < D; ++d) s = fmaf(mu[d], qf[tid * D + d], s);
      }
      qmu[tid] = s;
    }
    __syncthreads();
  }
  for (int h0 = 0; h0 < GMAX; h0 += HPB) {
    const int h = h0 + tid / LPV;
    const bool active = h < G;
    float v[8];
    if constexpr (PCA) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = h < GMAX ? uq[h * M + 8 * c + j] : 0.0f;
        v[j] = __uint_as_float(__float_as_uint(x) ^ (((sbyte >> j) & 1u) << 31));
      }
    } else {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (active)
        raw = *reinterpret_cast<const uint4*>(a.q + b * a.q_sb + (int64_t)(kv * G + h) * a.q_sh + 8 * c);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float((w[k] << 16) ^ (((sbyte >> (2 * k)) & 1u) << 31));
        v[2 * k + 1] = __uint_as_float((w[k] & 0xFFFF0000u) ^ (((sbyte >> (2 * k + 1)) & 1u) << 31));
      }
    }
    fwht_vector<LPV>(v, c);
    if (h < GMAX) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qs[(j * LPV + c) * GMAX + h] = active ? v[j] : 0.0f;
    }
  }
}

template <int D, int M, int BITS, int GMAX, bool PCA>
__global__ __launch_bounds__(kScoreThreads) void k_score(ScoreArgs a) {
  constexpr int NWC = (M / 32) * BITS, NWT = NWC + 1;
  __shared__ float qs[M * GMAX];
  __shared__ float qf[PCA ? GMAX * D : 1];
  __shared__ float uq[PCA ? GMAX * M : 1];
  __shared__ float qmu[GMAX];
  __shared__ float lut[16];
  const int pair = blockIdx.y;
  const int b = pair / a.Hkv, kv = pair % a.Hkv;
  const int G = a.Hq / a.Hkv;
  if (threadIdx.x < 16) lut[threadIdx.x] = a.tab.c[threadIdx.x];
  if (!PCA && threadIdx.x < GMAX) qmu[threadIdx.x] = 0.0f;
  const int64_t row0 = b * a.rec_sb + kv * a.rec_sh + (int64_t)blockIdx.x * kScoreThreads;
  rotate_queries<D, M, GMAX, PCA>(a, b, kv, G, row0, qs, qf, uq, qmu);
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kScoreThreads + threadIdx.x;
  if (t >= a.T) return;
  const uint32_t* r32 =
      reinterpret_cast<const uint32_t*>(a.rec) + (b * a.rec_sb + kv * a.rec_sh + t) * NWT;
  float acc[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) acc[h] = 0.0f;
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
      const float* qrow = qs + (32 * g + jb) * GMAX;
#pragma unroll
      for (int h = 0; h < GMAX; ++h) acc[h] = fmaf(qrow[h], cv, acc[h]);
    }
  }
  const float scale = __uint_as_float(r32[NWC]) * a.tab.inv_m;
  float* srow = a.s + b * a.s_sb + t;
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
    if (h < G) srow[(int64_t)(kv * G + h) * a.s_sh] = fmaf(acc[h], scale, qmu[h]);
}

template <int D, int M, int BITS, bool PCA>
static hipError_t launch_score_t(int group, const ScoreArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.T + kScoreThreads - 1) / kScoreThreads), (unsigned)(a.B * a.Hkv));
  const dim3 blk(kScoreThreads);
  if (group <= 4) hipLaunchKernelGGL((k_score<D, M, BITS, 4, PCA>), grid, blk, 0, st, a);
  else hipLaunchKernelGGL((k_score<D, M, BITS, 8, PCA>), grid, blk, 0, st, a);
  return hipGetLastError();
}

template <int D, int M, bool PCA>
static hipError_t launch_score_dm(int bits, int group, const ScoreArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return launch_score_t<D, M, 1, PCA>(group, a, st);
    case 2: return launch_score_t<D, M, 2, PCA>(group, a, st);
    case 3: return launch_score_t<D, M, 3, PCA>(group, a, st);
    case 4: return launch_score_t<D, M, 4, PCA>(group, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score(int D, int m, int bits, int group, const ScoreArgs& a, hipStream_t st) {
  if (a.T <= 0 || a.B <= 0 || a.Hkv <= 0) return hipSuccess;
  if (group < 1 || group > 8) return hipErrorInvalidValue;
  if (D == m) {
    switch (m) {
      case 64: return launch_score_dm<64, 64, false>(bits, group, a, st);
      case 128: return launch_score_dm<128, 128, false>(bits, group, a, st);
      case 256: return launch_score_dm<256, 256, false>(bits, group, a, st);
      case 512: return launch_score_dm<512, 512, false>(bits, group, a, st);
    }
    return hipErrorInvalidValue;
  }
#define KVQ_CASE(d, r) \
  if (D == d && m == r) return launch_score_dm<d, r, true>(bits, group, a, st);
  KVQ_CASE(64, 32) KVQ_CASE(128, 32) KVQ_CASE(128, 64) KVQ_CASE(256, 32) KVQ_CASE(256, 64)
  KVQ_CASE(256, 128) KVQ_CASE(512, 32) KVQ_CASE(512, 64)
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
