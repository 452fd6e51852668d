// kvq_pca.hip — projection (PCA) codec: v = B^T (x - mu) on MFMA, then the Hadamard codec
// over the r projected coordinates; decode x^ = mu + B v^ on MFMA.
//
// The projection follows the pages' per-token pipeline project -> rotate -> scale ->
// Lloyd-Max [kakeyaturbo PR #15, commits "M4 Phase A" ((X - mu) @ basis^T) and "M5" (unproject
// on the matrix engine)]. It is a genuine dense contraction, so it runs on
// v_mfma_f32_16x16x32_bf16: x and B are bf16, so every product is exact and accumulates in f32.
// The decode splits v^ into two bf16 halves (hi + lo) so the unprojection keeps ~2^-17 relative
// precision. Rows are processed in tiles of 64; the basis of a tile stays in LDS until a tile
// needs another basis.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_quant.h"

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kPcaTile = 64;

__device__ __forceinline__ floatx4 mfma_bf16(const uint4& a, const uint4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------------------------------
// Encode.
//   LDS: bT[r][D] = transposed basis (B operand: 8 consecutive k = input dims per lane),
//        mp[r] = B^T mu, y[64][r] = projected tile.
//   MFMA 16x16x32: lane l holds A[row l%16][k 8(l/16)..+7], B[k 8(l/16)..+7][col l%16] and
//   returns D[row 4(l/16)+i][col l%16], i = 0..3.
template <int D, int R, int BITS, bool SYM>
__global__ __launch_bounds__(256) void k_encode_pca(EncodeArgs a) {
  constexpr int KS = D / 32, NT = R / 16, LPV = R / 8, VPW = 64 / LPV;
  constexpr int BTS = D + 8;  // padded row (bf16 elements): 16-byte aligned rows, fewer conflicts
  constexpr int YS = R + 4;   // padded f32 row
  __shared__ __attribute__((aligned(16))) uint16_t bT[R * BTS];
  __shared__ float mp[R];
  __shared__ __attribute__((aligned(16))) float y[kPcaTile * YS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPV, c = lane % LPV;
  const uint32_t sbyte = (a.tab.sign_words[(c >> 2) & 15] >> (8 * (c & 3))) & 0xFFu;
  int cur = -1;
  const int64_t n_tiles = (a.n + kPcaTile - 1) / kPcaTile;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t row0 = tile * kPcaTile;
    const int bi = basis_of_row(a.pca, row0);
    if (bi != cur) {
      __syncthreads();
      const uint16_t* Bk = a.pca.basis + (int64_t)bi * D * R;
      for (int e = tid; e < D * R; e += 256) {  // B[d][j] -> bT[j][d]
        const int d = e / R, j = e % R;
        bT[j * BTS + d] = Bk[e];
      }
      __syncthreads();
      if (tid < R) {
        float s = 0.0f;
        if (a.pca.mean) {
          const float* mu = a.pca.mean + (int64_t)bi * D;
          for (int d = 0; d < D; ++d) s = fmaf(__uint_as_float((uint32_t)bT[tid * BTS + d] << 16), mu[d], s);
        }
        mp[tid] = s;
      }
      cur = bi;
      __syncthreads();
    }
    // projection of rows row0 + 16*wave .. +15
    {
      const int64_t row = row0 + 16 * wave + (lane & 15);
      const bool ok = row < a.n;
      floatx4 acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int k0 = ks * 32 + 8 * (lane >> 4);
        uint4 av = make_uint4(0, 0, 0, 0);
        if (ok) av = *reinterpret_cast<const uint4*>(a.x + row * a.ld + k0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 bv = *reinterpret_cast<const uint4*>(&bT[(t * 16 + (lane & 15)) * BTS + k0]);
          acc[t] = mfma_bf16(av, bv, acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[(16 * wave + 4 * (lane >> 4) + i) * YS + t * 16 + (lane & 15)] = acc[t][i];
    }
    __syncthreads();
    // Hadamard codec over the r projected coordinates, VPW vectors per wave step
#pragma unroll
    for (int st = 0; st < 16 / VPW; ++st) {
      const int local = 16 * wave + st * VPW + sub;
      const int64_t vec = row0 + local;
      const bool valid = vec < a.n;
      float v[8];
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = y[local * YS + 8 * c + j] - mp[8 * c + j];
        v[j] = __uint_as_float(__float_as_uint(p) ^ (((sbyte >> j) & 1u) << 31));
        ss = fmaf(p, p, ss);
      }
      const float n = sqrtf(vector_sum<LPV>(ss));
      fwht_vector<LPV>(v, c);
      quantize_store<R, BITS, SYM>(v, n, valid, vec, sub, c, a.tab, a.rec);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode.
//   LDS: Bs[D][r] = basis as stored (B operand of the unprojection: k = j contiguous),
//        mu[D], vh/vl[64][r] = bf16 hi / lo halves of v^.
template <int D, int R, int BITS, bool BF16>
__global__ __launch_bounds__(256) void k_decode_pca(DecodeArgs a) {
  constexpr int KS = R / 32, NT = D / 16, LPV = R / 8, VPW = 64 / LPV;
  constexpr int NWC = (R / 32) * BITS, NWT = NWC + 1;
  constexpr int BS = R + 8;   // padded bf16 row
  __shared__ __attribute__((aligned(16))) uint16_t Bs[D * BS];
  __shared__ float mu[D];
  __shared__ __attribute__((aligned(16))) uint16_t vh[kPcaTile * BS];
  __shared__ __attribute__((aligned(16))) uint16_t vl[kPcaTile * BS];
  __shared__ float lut[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPV, c = lane % LPV;
  if (tid < 16) lut[tid] = a.tab.c[tid];
  const uint32_t sbyte = (a.tab.sign_words[(c >> 2) & 15] >> (8 * (c & 3))) & 0xFFu;
  int cur = -1;
  const int64_t n_tiles = (a.n + kPcaTile - 1) / kPcaTile;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t row0 = tile * kPcaTile;
    const int bi = basis_of_row(a.pca, row0);
    if (bi != cur) {
      __syncthreads();
      const uint16_t* Bk = a.pca.basis + (int64_t)bi * D * R;
      for (int e = tid; e < D * R; e += 256) Bs[(e / R) * BS + (e % R)] = Bk[e];
      for (int d = tid; d < D; d += 256) mu[d] = a.pca.mean ? a.pca.mean[(int64_t)bi * D + d] : 0.0f;
      cur = bi;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 16 / VPW; ++st) {
      const int local = 16 * wave + st * VPW + sub;
      const int64_t vec = row0 + local;
      float zh[8];
      float nrm = 0.0f;
      if (vec < a.n) {
        const uint32_t* r32 = reinterpret_cast<const uint32_t*>(a.rec) + vec * NWT;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pos = j * LPV + c;
          uint32_t code = 0;
#pragma unroll
          for (int p = 0; p < BITS; ++p) code |= ((r32[(pos >> 5) * BITS + p] >> (pos & 31)) & 1u) << p;
          zh[j] = lut[code];
        }
        nrm = __uint_as_float(r32[NWC]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) zh[j] = 0.0f;
      }
      fwht_vector<LPV>(zh, c);
      const float scale = nrm * a.tab.inv_m;
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = __uint_as_float(__float_as_uint(zh[j] * scale) ^ (((sbyte >> j) & 1u) << 31));
        hi[j] = f32_to_bf16_rne(v);
        lo[j] = f32_to_bf16_rne(v - __uint_as_float(hi[j] << 16));
      }
      uint4 h4 = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
      uint4 l4 = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
      *reinterpret_cast<uint4*>(&vh[local * BS + 8 * c]) = h4;
      *reinterpret_cast<uint4*>(&vl[local * BS + 8 * c]) = l4;
    }
    __syncthreads();
    {
      const int arow = 16 * wave + (lane & 15);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int k0 = ks * 32 + 8 * (lane >> 4);
          const uint4 bv = *reinterpret_cast<const uint4*>(&Bs[(t * 16 + (lane & 15)) * BS + k0]);
          acc = mfma_bf16(*reinterpret_cast<const uint4*>(&vh[arow * BS + k0]), bv, acc);
          acc = mfma_bf16(*reinterpret_cast<const uint4*>(&vl[arow * BS + k0]), bv, acc);
        }
        const int col = t * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t vec = row0 + 16 * wave + 4 * (lane >> 4) + i;
          if (vec < a.n) {
            const float val = acc[i] + mu[col];
            if constexpr (BF16)
              static_cast<uint16_t*>(a.y)[vec * a.ld + col] = (uint16_t)f32_to_bf16_rne(val);
            else
              static_cast<float*>(a.y)[vec * a.ld + col] = val;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launchers. Supported (D, r): r in {32, 64, 128}, r < D, D*r <= 32768.

static int64_t pca_blocks(int64_t n) {
  int64_t tiles = (n + kPcaTile - 1) / kPcaTile;
  if (tiles > 8192) tiles = 8192;
  return tiles < 1 ? 1 : tiles;
}

template <int D, int R, int BITS, bool SYM>
static hipError_t enc_t(const EncodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_encode_pca<D, R, BITS, SYM>), dim3((unsigned)pca_blocks(a.n)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t enc_dr(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return enc_t<D, R, 1, false>(a, st);
    case 3: return enc_t<D, R, 1, true>(a, st);
    case 4: return enc_t<D, R, 2, false>(a, st);
    case 5: return enc_t<D, R, 2, true>(a, st);
    case 6: return enc_t<D, R, 3, false>(a, st);
    case 7: return enc_t<D, R, 3, true>(a, st);
    case 8: return enc_t<D, R, 4, false>(a, st);
    case 9: return enc_t<D, R, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int D, int R, int BITS>
static hipError_t dec_t(bool bf16, const DecodeArgs& a, hipStream_t st) {
  const dim3 g((unsigned)pca_blocks(a.n)), b(256);
  if (bf16) hipLaunchKernelGGL((k_decode_pca<D, R, BITS, true>), g, b, 0, st, a);
  else hipLaunchKernelGGL((k_decode_pca<D, R, BITS, false>), g, b, 0, st, a);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t dec_dr(int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return dec_t<D, R, 1>(bf16, a, st);
    case 2: return dec_t<D, R, 2>(bf16, a, st);
    case 3: return dec_t<D, R, 3>(bf16, a, st);
    case 4: return dec_t<D, R, 4>(bf16, a, st);
  }
  return hipErrorInvalidValue;
}

#define KVQ_PCA_PAIRS(X) X(64, 32) X(128, 32) X(128, 64) X(256, 32) X(256, 64) X(256, 128) \
                         X(512, 32) X(512, 64)

bool pca_shape_supported(int D, int r) {
#define KVQ_PCA_CASE(d, rr) if (D == d && r == rr) return true;
  KVQ_PCA_PAIRS(KVQ_PCA_CASE)
#undef KVQ_PCA_CASE
  return false;
}

hipError_t launch_encode_pca(int D, int r, int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
#define KVQ_PCA_CASE(d, rr) if (D == d && r == rr) return enc_dr<d, rr>(bits, sym, a, st);
  KVQ_PCA_PAIRS(KVQ_PCA_CASE)
#undef KVQ_PCA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_pca(int D, int r, int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
#define KVQ_PCA_CASE(d, rr) if (D == d && r == rr) return dec_dr<d, rr>(bits, bf16, a, st);
  KVQ_PCA_PAIRS(KVQ_PCA_CASE)
#undef KVQ_PCA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
