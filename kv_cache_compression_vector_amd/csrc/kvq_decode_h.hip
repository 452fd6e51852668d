// kvq_decode_h.hip — Hadamard-codec decode (m = 64 .. 512) with the inverse rotation split between
// the matrix cores and the vector ALUs.
//
// x^ = (n/m) s (.) H_m z^ [kakeyaturbo PR #15, "M4 Phase A" (inverse rotation, then the norm),
// "M5" (decode)]. In Sylvester order H_m = H_NB (x) H_32 with NB = m/32 (coordinate i = 32a + b,
// H_m[32a' + b'][32a + b] = H_NB[a'][a] H_32[b'][b]), so
//   y_a = H_32 z^_a           on MFMA for each 32-coordinate block a (entries +-1, exact in bf16;
//                             z^ as bf16 hi + lo),
//   x^_a' = sum_a H_NB[a'][a] y_a   as log2(NB) butterfly stages in registers,
// which leaves log2(NB) of the log2(m) butterfly stages on the vector ALUs (2 of 7 at m = 128)
// and needs no LDS operands: the H_32 fragments are formed once per wave in registers.
//
// Layout (16 vectors per MFMA tile, lane l: vector n = l % 16, group q = l / 16):
//  - H_32's columns are permuted so that the 8 k-values of lane group q are the coordinates
//    b = 8 q' + e' with e' = 2q + e/4, q' = e % 4, e = 0..7. Coordinate 32a + 8q' + e' has plane
//    position e' m/8 + 4a + q', so for every block a the lane's coordinates are two runs of 4
//    consecutive bits, (2q + r) m/8 mod 32 + 4a + [0, 4) for r = 0, 1, of one record word group
//    (q m/128). A lane reads b + 1 words of its vector's record, and two coordinates' bit pairs
//    index a table of their centroids' bf16 hi pair and lo pair (the MFMA operand words).
//  - H_32's rows are permuted so that the two 16-row output tiles t give lane group q the
//    output coordinates b' = 8q + 4t + [0, 4): after both, 8 consecutive outputs per block, one
//    16-byte chunk. bf16 rows are assembled in LDS and leave as whole rows, 1 KB per store
//    instruction.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_mfma.h"

namespace kvq {

namespace {

constexpr int kDhWaves = 4;
constexpr int kDhVT = 2;  // 16-vector tiles per wave step (m <= 128)

// 16-vector tiles per wave step: one at m = 256, 512 (the bf16 staging of 16 rows is 8 or 16 KB)
template <int M>
constexpr int dh_vt() { return M <= 128 ? kDhVT : 1; }

template <int BITS>
constexpr int dh_copies() { return BITS <= 3 ? 32 : 4; }

// Pair index of the coordinates at bits sh + pr, sh + pr + 1 of the BITS plane words w
// (bit 2p + i = plane p of coordinate i), from the planes' bytes at sh gathered into y.
template <int BITS>
__device__ __forceinline__ uint32_t gather_bytes(const uint32_t* w, int sh) {
  uint32_t y = __builtin_amdgcn_ubfe(w[0], sh, 8);
  if constexpr (BITS >= 2) y |= __builtin_amdgcn_ubfe(w[1], sh, 8) << 8;
  if constexpr (BITS >= 3) y |= __builtin_amdgcn_ubfe(w[2], sh, 8) << 16;
  if constexpr (BITS >= 4) y |= __builtin_amdgcn_ubfe(w[3], sh, 8) << 24;
  return y;
}

// Word offset (index times C) in the pair table of the coordinates at bits pr, pr + 1 of the
// plane bytes y (byte p = plane p). For b = 2, 3 the index sum_p 4^p (plane-p bit pair) is one
// byte dot product of the masked bytes with the weights (1, 4, 16); at pr = 2 it comes out times
// 4, which the shift into the table offset absorbs.
template <int BITS, int C>
__device__ __forceinline__ uint32_t pair_word(uint32_t y, int pr) {
  if constexpr (BITS == 1) {
    return ((y >> pr) & 3u) * C;
  } else if constexpr ((BITS == 2 || BITS == 3) && C == 32) {
    constexpr uint32_t mask = BITS == 3 ? 0x030303u : 0x0303u;
    constexpr uint32_t wts = BITS == 3 ? 0x100401u : 0x0401u;
    const uint32_t d = __builtin_amdgcn_udot4(y & (mask << pr), wts, 0u, false);  // idx 4^(pr/2)
    return d << (5 - pr);
  } else {
    uint32_t idx = 0;
#pragma unroll
    for (int p = 0; p < BITS; ++p) idx |= ((y >> (8 * p + pr)) & 3u) << (2 * p);
    return idx * C;
  }
}

// Pair table: entry e (bit 2p + i = plane p of code i) = the two centroids as a bf16 hi pair
// (lut[e C + c]) and lo pair (lut[(NPAIR + e) C + c]), copy c read by lanes l % C == c. Filled
// in two phases around a block barrier: pair_entries forms each entry once (copy 0) and
// pair_copies replicates it, consecutive threads writing consecutive words.
template <int BITS, int C>
__device__ __forceinline__ void pair_entries(const Tables& tab, uint32_t* lut, int tid, int nthr) {
  constexpr int NPAIR = 1 << (2 * BITS);
  for (int e = tid; e < NPAIR; e += nthr) {
    uint32_t ca = 0, cb = 0;
#pragma unroll
    for (int p = 0; p < BITS; ++p) {
      ca |= ((e >> (2 * p)) & 1u) << p;
      cb |= ((e >> (2 * p + 1)) & 1u) << p;
    }
    float va = 0.0f, vb = 0.0f;
#pragma unroll
    for (int k = 0; k < (1 << BITS); ++k) {
      va = (uint32_t)k == ca ? tab.c[k] : va;
      vb = (uint32_t)k == cb ? tab.c[k] : vb;
    }
    const uint32_t ha = f32_to_bf16_rne(va), hb = f32_to_bf16_rne(vb);
    const uint32_t la = f32_to_bf16_rne(va - __uint_as_float(ha << 16));
    const uint32_t lb = f32_to_bf16_rne(vb - __uint_as_float(hb << 16));
    lut[e * C] = ha | (hb << 16);
    lut[(NPAIR + e) * C] = la | (lb << 16);
  }
}

template <int BITS, int C>
__device__ __forceinline__ void pair_copies(uint32_t* lut, int tid, int nthr) {
  constexpr int WORDS = 2 * (1 << (2 * BITS)) * C;
  for (int i = tid; i < WORDS; i += nthr)
    if (i % C != 0) lut[i] = lut[i - i % C];
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

}  // namespace

// With OL, the vector's outlier entries [kakeyaturbo PR #15, calibrated Lloyd-Max + outlier
// commit: sparse (index, value) overrides of the scaled residual] replace their coordinates'
// centroids before the rotation. Element e of lane (q, vector) in block ab is coordinate
// i = 32 ab + 8 (e % 4) + 2 q + e / 4, so an entry belongs to lane group q = (i % 8) / 2 at slot
// 8 ab + e; each lane scans its vector's entries into a per-lane LDS slot row and a slot mask,
// and merges the flagged slots into its B operands (bf16 value as the hi half, lo half 0).
//
// m = 256, 512 (no outlier list): the same structure with NB = 8, 16 blocks. Plane position
// (2q + h) m/8 + 4a + q' of a lane's coordinates then lies in word group 2q + h (m = 256) or
// 4q + 2h + a / 8 (m = 512), bits 4 (a mod 8) + q': the lane loads m/64 word groups. One
// 16-vector tile per step, and the output signs come from LDS (16 blocks x 4 words per lane
// would not fit beside the 128 accumulators).
template <int M, int BITS, bool BF16, bool OL = false>
__global__ __launch_bounds__(64 * kDhWaves) void k_decode_h(DecodeArgs a) {
  static_assert(!OL || M <= 128, "outlier lists at m <= 128 only");
  constexpr int NB = M / 32, NWC = (M / 32) * BITS, NWT = NWC + 1;
  constexpr int C = dh_copies<BITS>(), NPAIR = 1 << (2 * BITS);
  constexpr int NS = 8 * NB;  // override slots per lane (coordinates of its group)
  constexpr int VT = dh_vt<M>();
  constexpr int NWG = M <= 128 ? 1 : M / 64;  // record word groups a lane reads
  constexpr bool SG_LDS = M > 128;
  __shared__ uint32_t lut[2 * NPAIR * C];
  __shared__ uint4 s_sg[SG_LDS ? NB * 4 : 1];  // sign masks of block a', lane group q
  // bf16 rows of a wave's step (16 VT rows of M bf16 = M/8 16-byte chunks, chunk index
  // XOR-swizzled with the row so the row-wise writes and chunk-wise reads spread over banks)
  constexpr int RCH = M / 8;
  __shared__ uint4 stage[BF16 ? kDhWaves * 16 * VT * RCH : 1];
  // override values: with bf16 rows they live in the last tile's row slice of the wave's stage
  // (16 rows of M bf16 = 64 lanes x NS bf16), free until that tile's rows are assembled
  __shared__ __attribute__((aligned(16))) uint16_t ov_own[(OL && !BF16) ? kDhWaves * 64 * NS : 8];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint16_t* const ovv =
      (BF16 ? reinterpret_cast<uint16_t*>(stage + (wave * 16 * VT + 16 * (VT - 1)) * RCH)
            : ov_own + wave * 64 * NS) + lane * NS;
  static_assert(!OL || 16 * M * 2 == 64 * NS * 2, "override slots fill one tile's row slice");
  constexpr int RPK = 64 / RCH;  // rows per whole-row store instruction
  const int64_t lane_off = (int64_t)(lane / RCH) * a.ld + 8 * (lane % RCH);
  uint16_t* const ylast = static_cast<uint16_t*>(a.y) + (a.n - 1) * a.ld + 8 * (lane % RCH);
  const int n16 = lane & 15, q = lane >> 4;
  pair_entries<BITS, C>(a.tab, lut, tid, 64 * kDhWaves);
  // A operands (H_32, permuted) of the two output tiles: row m -> b' = 8 (m/4) + 4t + m % 4,
  // column k = 8q + e -> b = 8 (e % 4) + 2q + e / 4
  uint4 A[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bo = 8 * (n16 >> 2) + 4 * t + (n16 & 3);
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t v = 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int e = 2 * h + s;
        const int bi = 8 * (e & 3) + 2 * q + (e >> 2);
        v |= (0x3F80u | (((uint32_t)__builtin_popcount(bo & bi) & 1u) << 15)) << (16 * s);
      }
      w[h] = v;
    }
    A[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // signs of this lane's outputs d = 32 a' + 8q + [0, 8), as bf16-pair (or f32) sign masks:
  // byte q of sign word a' (a wave-uniform index, so a scalar load)
  uint32_t sg[SG_LDS ? 1 : NB][4];
  auto sign_masks = [&](int ap, int qq, uint32_t (&m4)[4]) {
    const uint32_t byte = (a.tab.sign_words[ap] >> (8 * qq)) & 0xFFu;
#pragma unroll
    for (int h = 0; h < 4; ++h) {  // outputs 2h, 2h + 1 of the byte
      const uint32_t s0 = (byte >> (2 * h)) & 1u, s1 = (byte >> (2 * h + 1)) & 1u;
      m4[h] = BF16 ? ((s0 << 15) | (s1 << 31)) : (s0 | (s1 << 1));
    }
  };
  if constexpr (SG_LDS) {
    for (int i = tid; i < NB * 4; i += 64 * kDhWaves) {
      uint32_t m4[4];
      sign_masks(i / 4, i % 4, m4);
      s_sg[i] = make_uint4(m4[0], m4[1], m4[2], m4[3]);
    }
  } else {
#pragma unroll
    for (int ap = 0; ap < NB; ++ap) sign_masks(ap, q, sg[ap]);
  }
  __syncthreads();
  pair_copies<BITS, C>(lut, tid, 64 * kDhWaves);
  __syncthreads();
  const uint32_t* rec32 = reinterpret_cast<const uint32_t*>(a.rec);
  const int64_t n_steps = (a.n + 16 * VT - 1) / (16 * VT);
  const int64_t stride = (int64_t)gridDim.x * kDhWaves;
  // the lane's words (word groups q m/128 .. + NWG - 1, all planes) and the norm of the vectors
  // of a step
  constexpr int NW = NWG * BITS;
  auto load = [&](int64_t st, uint32_t (&w)[VT][NW + 1]) {
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      int64_t v = st * 16 * VT + 16 * vt + n16;
      v = v < a.n ? v : a.n - 1;
      const uint32_t* r = rec32 + v * NWT;
#pragma unroll
      for (int p = 0; p < NW; ++p) w[vt][p] = r[(q * M / 128) * BITS + p];
      w[vt][NW] = r[NWC];
    }
  };
  int64_t st = (int64_t)blockIdx.x * kDhWaves + wave;
  uint32_t wn[VT][NW + 1];
  if (st < n_steps) load(st, wn);
  // let the first step's words land before the loop, so the wait at the loop head only covers
  // the path round the loop, where the previous step's stores may stay in flight
  // (vmcnt(0) expcnt(7) lgkmcnt(15))
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (; st < n_steps; st += stride) {
    uint32_t w[VT][NW + 1];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int p = 0; p <= NW; ++p) w[vt][p] = wn[vt][p];
    if (st + stride < n_steps) load(st + stride, wn);  // in flight during this step
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      uint32_t ovm = 0;  // slots of this lane overridden by outlier entries
      if constexpr (OL) {
        // a lane past the end decodes the last record, whose row it stores again: with that
        // record's entries, so the bytes are the same
        int64_t v = st * 16 * VT + 16 * vt + n16;
        v = v < a.n ? v : a.n - 1;
        int64_t k = a.ol_off[v], e = a.ol_off[v + 1];
        if (e > a.ol_cap) e = a.ol_cap;
        for (; k < e; ++k) {
          const uint32_t i = static_cast<const uint8_t*>(a.ol_idx)[k];
          if (i < (uint32_t)M && ((i & 7u) >> 1) == (uint32_t)q) {  // indices past m: ignored
            const uint32_t slot = 8 * (i >> 5) + 4 * (i & 1u) + ((i & 31u) >> 3);
            ovv[slot] = a.ol_val[k];
            ovm |= 1u << slot;
          }
        }
      }
      floatx4 y[NB][2];
#pragma unroll
      for (int ab = 0; ab < NB; ++ab) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // word group (local j) and bit of plane position (2q + half) m/8 + 4 ab
          const int j = M <= 128 ? 0 : M == 256 ? half : 2 * half + (ab >> 3);
          const int sh = M <= 128 ? ((2 * q + half) * (M / 8)) % 32 + 4 * ab : 4 * (ab & 7);
          const uint32_t yb = gather_bytes<BITS>(w[vt] + j * BITS, sh);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint32_t off = pair_word<BITS, C>(yb, 2 * s) + (lane & (C - 1));
            hi[2 * half + s] = lut[off];
            lo[2 * half + s] = lut[NPAIR * C + off];
          }
        }
        if constexpr (OL) {
          const uint32_t mab = (ovm >> (8 * ab)) & 0xFFu;
          if (mab != 0u) {
            const uint4 ov = *reinterpret_cast<const uint4*>(ovv + 8 * ab);
            const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {  // word w4 holds elements 2 w4 (low), 2 w4 + 1
              const uint32_t msk = (((mab >> (2 * w4)) & 1u) ? 0x0000FFFFu : 0u) |
                                   (((mab >> (2 * w4 + 1)) & 1u) ? 0xFFFF0000u : 0u);
              hi[w4] = (hi[w4] & ~msk) | (ow[w4] & msk);
              lo[w4] &= ~msk;
            }
          }
        }
        const uint4 bh = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        const uint4 bl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          floatx4 c = {0.f, 0.f, 0.f, 0.f};
          c = mfma_bf16(A[t], bh, c);
          c = mfma_bf16(A[t], bl, c);
          y[ab][t] = c;
        }
      }
      // H_NB across the blocks (Sylvester: the partner of block a at stage h is a ^ h)
#pragma unroll
      for (int h = 1; h < NB; h <<= 1)
#pragma unroll
        for (int ab = 0; ab < NB; ++ab)
          if ((ab & h) == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const floatx4 u = y[ab][t], v = y[ab + h][t];
              y[ab][t] = u + v;
              y[ab + h][t] = u - v;
            }
          }
      const float sc = __uint_as_float(w[vt][NW]) * a.tab.inv_m;
      auto sgn = [&](int ap, int h) -> uint32_t {
        if constexpr (SG_LDS) {
          const uint4 m4 = s_sg[ap * 4 + q];
          return h == 0 ? m4.x : h == 1 ? m4.y : h == 2 ? m4.z : m4.w;
        } else {
          return sg[ap][h];
        }
      };
      if constexpr (BF16) {
        const int row = 16 * vt + n16;
#pragma unroll
        for (int ap = 0; ap < NB; ++ap) {
          const floatx4 y0 = y[ap][0], y1 = y[ap][1];
          const int ch = 4 * ap + q;  // columns 32 a' + 8q .. + 7
          stage[(wave * 16 * VT + row) * RCH + (ch ^ (row & (RCH - 1)))] =
              make_uint4(bf16_pair(y0[0] * sc, y0[1] * sc) ^ sgn(ap, 0),
                         bf16_pair(y0[2] * sc, y0[3] * sc) ^ sgn(ap, 1),
                         bf16_pair(y1[0] * sc, y1[1] * sc) ^ sgn(ap, 2),
                         bf16_pair(y1[2] * sc, y1[3] * sc) ^ sgn(ap, 3));
        }
      } else {
        int64_t v = st * 16 * VT + 16 * vt + n16;
        // a lane past the end decoded the last record: it stores the last row's own bytes again
        v = v < a.n ? v : a.n - 1;
#pragma unroll
        for (int ap = 0; ap < NB; ++ap) {
          const floatx4 y0 = y[ap][0], y1 = y[ap][1];
          const float o[8] = {y0[0] * sc, y0[1] * sc, y0[2] * sc, y0[3] * sc,
                              y1[0] * sc, y1[1] * sc, y1[2] * sc, y1[3] * sc};
          float* yp = static_cast<float*>(a.y) + v * a.ld + 32 * ap + 8 * q;
          float r[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            r[j] = __uint_as_float(__float_as_uint(o[j]) ^ (((sgn(ap, j >> 1) >> (j & 1)) & 1u) << 31));
          *reinterpret_cast<float4*>(yp) = make_float4(r[0], r[1], r[2], r[3]);
          *reinterpret_cast<float4*>(yp + 4) = make_float4(r[4], r[5], r[6], r[7]);
        }
      }
    }
    if constexpr (BF16) {
      // whole rows: each instruction writes 64 consecutive 16-byte chunks of the step's rows,
      // as streaming (nontemporal) stores: the rows are not read again by this kernel
      __builtin_amdgcn_wave_barrier();
      constexpr int CH = 16 * VT * RCH / 64;
      uint4 out[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int id = 64 * k + lane, row = id / RCH, ch = id % RCH;
        out[k] = stage[(wave * 16 * VT + row) * RCH + (ch ^ (row & (RCH - 1)))];
      }
      const int64_t v0 = st * 16 * VT;  // the step's first row
      uint16_t* const yp = static_cast<uint16_t*>(a.y) + v0 * a.ld + lane_off;
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        // row v0 + RPK k + lane / RCH; rows past the end hold the last row's own bytes
        const bool in = v0 + RPK * k + lane / RCH < a.n;
        st_stream(in ? yp + RPK * k * a.ld : ylast, out[k]);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Projection-codec decode, x^ = mu + B diag(s) v', v' = (n/r) H_r z^ [kakeyaturbo PR #15, "M5":
// inverse rotation, then the unprojection on the matrix engine]. The rotation is split as above
// (H_r = H_{r/32} (x) H_32). After it each lane holds, for every 32-coordinate block, the 8
// consecutive coordinates 32a + 8q + [0, 8) of its vector, which is exactly the unprojection's
// MFMA B operand for k-step a; so v' goes from the accumulators into the second product without
// leaving the registers (split into bf16 hi + lo: the basis is exact in bf16, v' is not). The
// basis (signs folded into its columns, exact) is the A operand from LDS; the accumulator starts
// at mu. Its rows are permuted within each pair of 16-row tiles so that a lane ends with 8
// consecutive output columns (one 16-byte chunk); bf16 rows are assembled in LDS and stored
// whole. A block takes 128 consecutive vectors per tile (one basis: basis blocks are multiples
// of 256 rows) and re-stages the basis only when it changes.

constexpr int kDpWaves = 4;
constexpr int kDpVT = 2;                           // 16-vector tiles per wave and block tile
constexpr int kDpRows = 16 * kDpVT * kDpWaves;     // vectors per block tile

__device__ __forceinline__ int dp_out_col(int mt, int m) {
  return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

template <int D, int R, int BITS, bool BF16>
__global__ __launch_bounds__(64 * kDpWaves) void k_decode_pca_h(DecodeArgs a, int64_t tiles_per_block) {
  constexpr int NB = R / 32, MT = D / 16, HCH = R / 8, RCH = D / 8;
  constexpr int NWC = (R / 32) * BITS, NWT = NWC + 1;
  constexpr int C = dh_copies<BITS>(), NPAIR = 1 << (2 * BITS);
  constexpr int HMASK = (HCH < 16 ? HCH : 16) - 1;
  __shared__ uint32_t lut[2 * NPAIR * C];
  __shared__ uint4 s_B[D * HCH];                      // basis rows, chunk c at c ^ (row & HMASK)
  __shared__ __attribute__((aligned(16))) float s_mu[D];
  __shared__ uint4 stage[BF16 ? kDpWaves * 16 * RCH : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int RPK = 64 / RCH;  // rows per whole-row store instruction
  const int64_t lane_off = (int64_t)(lane / RCH) * a.ld + 8 * (lane % RCH);
  uint16_t* const ylast = static_cast<uint16_t*>(a.y) + (a.n - 1) * a.ld + 8 * (lane % RCH);
  const int n16 = lane & 15, q = lane >> 4;
  pair_entries<BITS, C>(a.tab, lut, tid, 64 * kDpWaves);  // copies with the first basis
  uint4 Ah[2];  // H_32 fragments, as in k_decode_h
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bo = 8 * (n16 >> 2) + 4 * t + (n16 & 3);
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t v = 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int e = 2 * h + s;
        const int bi = 8 * (e & 3) + 2 * q + (e >> 2);
        v |= (0x3F80u | (((uint32_t)__builtin_popcount(bo & bi) & 1u) << 15)) << (16 * s);
      }
      w[h] = v;
    }
    Ah[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  const uint32_t* rec32 = reinterpret_cast<const uint32_t*>(a.rec);
  const int64_t n_tiles = (a.n + kDpRows - 1) / kDpRows;
  const int64_t t0 = blockIdx.x * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < n_tiles ? t0 + tiles_per_block : n_tiles;
  auto load = [&](int64_t tile, uint32_t (&w)[kDpVT][BITS + 1]) {
#pragma unroll
    for (int vt = 0; vt < kDpVT; ++vt) {
      int64_t v = tile * kDpRows + 32 * wave + 16 * vt + n16;
      v = v < a.n ? v : a.n - 1;
      const uint32_t* r = rec32 + v * NWT;
#pragma unroll
      for (int p = 0; p < BITS; ++p) w[vt][p] = r[(q * R / 128) * BITS + p];
      w[vt][BITS] = r[NWC];
    }
  };
  // basis-index entry of a tile, loaded with its records and range-checked where it is used;
  // tiles advance by kDpRows <= block_rows rows, so the entry advances by at most one per tile
  const bool multi = a.pca.count > 1;
  int64_t ib = multi ? t0 * kDpRows / a.pca.block_rows : 0;
  int64_t ib_end = multi ? (ib + 1) * a.pca.block_rows : 0;
  auto basis_raw = [&](int64_t tile) -> int {
    if (!multi) return 0;
    if (tile * kDpRows >= ib_end) {
      ++ib;
      ib_end += a.pca.block_rows;
    }
    return a.pca.index[ib];
  };
  uint32_t wn[kDpVT][BITS + 1];
  int bn = 0, cur = -1;
  if (t0 < t1) {
    load(t0, wn);
    bn = basis_raw(t0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop head then waits only for its own loads
  for (int64_t tile = t0; tile < t1; ++tile) {
    int bi = __builtin_amdgcn_readfirstlane(bn);  // block-uniform
    bi = bi < 0 ? 0 : (bi >= a.pca.count ? a.pca.count - 1 : bi);
    if (bi != cur) {
      __syncthreads();
      if (cur < 0) pair_copies<BITS, C>(lut, tid, 64 * kDpWaves);
      const uint4* Bk = reinterpret_cast<const uint4*>(a.pca.basis + (int64_t)bi * D * R);
      for (int e = tid; e < D * HCH; e += 64 * kDpWaves) {
        const uint4 w = Bk[e];
        const int row = e / HCH, c = e % HCH, j0 = 8 * c;  // signs of columns j0 .. j0 + 7
        s_B[row * HCH + (c ^ (row & HMASK))] =
            make_uint4(w.x ^ a.tab.sign_pairs[j0 / 2], w.y ^ a.tab.sign_pairs[j0 / 2 + 1],
                       w.z ^ a.tab.sign_pairs[j0 / 2 + 2], w.w ^ a.tab.sign_pairs[j0 / 2 + 3]);
      }
      const float* mu = a.pca.mean ? a.pca.mean + (int64_t)bi * D : nullptr;
      for (int i = tid; i < D; i += 64 * kDpWaves) s_mu[i] = mu ? mu[i] : 0.0f;
      cur = bi;
      __syncthreads();
    }
    uint32_t w[kDpVT][BITS + 1];
#pragma unroll
    for (int vt = 0; vt < kDpVT; ++vt)
#pragma unroll
      for (int p = 0; p <= BITS; ++p) w[vt][p] = wn[vt][p];
    if (tile + 1 < t1) {  // in flight during this tile
      load(tile + 1, wn);
      bn = basis_raw(tile + 1);
    }
#pragma unroll
    for (int vt = 0; vt < kDpVT; ++vt) {
      // v' = (n/r) H_r z^ as B operands of the unprojection (k-step a: coordinates 32a + [0, 32))
      floatx4 y[NB][2];
#pragma unroll
      for (int ab = 0; ab < NB; ++ab) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t yb = gather_bytes<BITS>(w[vt], ((2 * q + half) * (R / 8)) % 32 + 4 * ab);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint32_t off = pair_word<BITS, C>(yb, 2 * s) + (lane & (C - 1));
            hi[2 * half + s] = lut[off];
            lo[2 * half + s] = lut[NPAIR * C + off];
          }
        }
        const uint4 bh = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        const uint4 bl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          floatx4 c = {0.f, 0.f, 0.f, 0.f};
          c = mfma_bf16(Ah[t], bh, c);
          c = mfma_bf16(Ah[t], bl, c);
          y[ab][t] = c;
        }
      }
      // H_NB across the blocks (Sylvester: the partner of block a at stage h is a ^ h)
#pragma unroll
      for (int h = 1; h < NB; h <<= 1)
#pragma unroll
        for (int ab = 0; ab < NB; ++ab)
          if ((ab & h) == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const floatx4 u = y[ab][t], v = y[ab + h][t];
              y[ab][t] = u + v;
              y[ab + h][t] = u - v;
            }
          }
      const float sc = __uint_as_float(w[vt][BITS]) * a.tab.inv_m;
      uint4 vh[NB], vl[NB];
#pragma unroll
      for (int ab = 0; ab < NB; ++ab) {
        const float x[8] = {y[ab][0][0] * sc, y[ab][0][1] * sc, y[ab][0][2] * sc, y[ab][0][3] * sc,
                            y[ab][1][0] * sc, y[ab][1][1] * sc, y[ab][1][2] * sc, y[ab][1][3] * sc};
        uint32_t h[4], l[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h[k] = bf16_pair(x[2 * k], x[2 * k + 1]);
          l[k] = bf16_pair(x[2 * k] - __uint_as_float(h[k] << 16),
                           x[2 * k + 1] - __uint_as_float(h[k] & 0xFFFF0000u));
        }
        vh[ab] = make_uint4(h[0], h[1], h[2], h[3]);
        vl[ab] = make_uint4(l[0], l[1], l[2], l[3]);
      }
      int64_t v = (tile * kDpRows + 32 * wave + 16 * vt + n16);
      v = v < a.n ? v : a.n - 1;  // a lane past the end decoded the last record
#pragma unroll
      for (int ap = 0; ap < MT / 2; ++ap) {
        floatx4 o[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int mt = 2 * ap + hh;
          const float4 m4 = *reinterpret_cast<const float4*>(s_mu + dp_out_col(mt, 4 * q));
          floatx4 c = {m4.x, m4.y, m4.z, m4.w};
          const int row = dp_out_col(mt, n16);
#pragma unroll
          for (int ks = 0; ks < NB; ++ks) {
            const uint4 A = s_B[row * HCH + ((4 * ks + q) ^ (row & HMASK))];
            c = mfma_bf16(A, vh[ks], c);
            c = mfma_bf16(A, vl[ks], c);
          }
          o[hh] = c;
        }
        // columns 32 ap + 8q + [0, 8) of vector n16
        if constexpr (BF16) {
          stage[(wave * 16 + n16) * RCH + ((4 * ap + q) ^ (n16 & (RCH - 1)))] =
              make_uint4(bf16_pair(o[0][0], o[0][1]), bf16_pair(o[0][2], o[0][3]),
                         bf16_pair(o[1][0], o[1][1]), bf16_pair(o[1][2], o[1][3]));
        } else {
          float* yp = static_cast<float*>(a.y) + v * a.ld + 32 * ap + 8 * q;
          *reinterpret_cast<float4*>(yp) = make_float4(o[0][0], o[0][1], o[0][2], o[0][3]);
          *reinterpret_cast<float4*>(yp + 4) = make_float4(o[1][0], o[1][1], o[1][2], o[1][3]);
        }
      }
      if constexpr (BF16) {
        // the 16 rows leave whole: each instruction writes 64 consecutive 16-byte chunks, as
        // streaming (nontemporal) stores
        __builtin_amdgcn_wave_barrier();
        constexpr int CH = 16 * RCH / 64;
        uint4 out[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const int id = 64 * k + lane, row = id / RCH, ch = id % RCH;
          out[k] = stage[(wave * 16 + row) * RCH + (ch ^ (row & (RCH - 1)))];
        }
        const int64_t v0 = tile * kDpRows + 32 * wave + 16 * vt;  // the 16 rows' first
        uint16_t* const yp = static_cast<uint16_t*>(a.y) + v0 * a.ld + lane_off;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          // row v0 + RPK k + lane / RCH; rows past the end hold the last row's own bytes
          const bool in = v0 + RPK * k + lane / RCH < a.n;
          st_stream(in ? yp + RPK * k * a.ld : ylast, out[k]);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

// Compute units of the current device (queried once per device).
static int dh_device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Blocks of k_decode_h<M, BITS, BF16, OL> that one compute unit holds at once (registers and
// LDS: the bf16 staging and the pair table leave 3 blocks at b = 3, 4 at b <= 2).
template <int M, int BITS, bool BF16, bool OL>
static int dh_blocks_per_cu() {
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_h<M, BITS, BF16, OL>, 64 * kDhWaves, 0) !=
            hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb < 4 ? nb : 4;
  }
  return per_cu;
}

template <int M, int BITS, bool BF16, bool OL>
static hipError_t launch_dh_k(const DecodeArgs& a, hipStream_t st) {
  // exactly one resident round (at most 4 blocks of 4 waves per compute unit, measured best
  // against 2 and 8), waves striding over the steps: a grid beyond what the chip holds at once
  // would leave its last blocks to run alone on part of the chip
  const int64_t steps = (a.n + 16 * dh_vt<M>() - 1) / (16 * dh_vt<M>());
  int64_t blocks = (steps + kDhWaves - 1) / kDhWaves;
  const int64_t resident = (int64_t)dh_blocks_per_cu<M, BITS, BF16, OL>() * dh_device_cus();
  if (blocks > resident) blocks = resident;
  hipLaunchKernelGGL((k_decode_h<M, BITS, BF16, OL>), dim3((unsigned)blocks), dim3(64 * kDhWaves), 0,
                     st, a);
  return hipGetLastError();
}

template <int M, int BITS>
static hipError_t launch_dh_t(bool bf16, const DecodeArgs& a, hipStream_t st) {
  if constexpr (M > 128) {  // no outlier list here (decode_h_supported)
    return bf16 ? launch_dh_k<M, BITS, true, false>(a, st) : launch_dh_k<M, BITS, false, false>(a, st);
  } else {
    const bool ol = a.ol_off != nullptr;
    if (bf16) return ol ? launch_dh_k<M, BITS, true, true>(a, st) : launch_dh_k<M, BITS, true, false>(a, st);
    return ol ? launch_dh_k<M, BITS, false, true>(a, st) : launch_dh_k<M, BITS, false, false>(a, st);
  }
}

template <int D, int R, int BITS>
static hipError_t launch_dp_t(bool bf16, const DecodeArgs& a, hipStream_t st) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_pca_h<D, R, BITS, true>,
                                                     64 * kDpWaves, 0) != hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  const int64_t tiles = (a.n + kDpRows - 1) / kDpRows;
  const int64_t resident = (int64_t)per_cu * dh_device_cus();
  const int64_t per = (tiles + resident - 1) / resident;
  const dim3 g((unsigned)((tiles + per - 1) / per)), b(64 * kDpWaves);
  if (bf16) hipLaunchKernelGGL((k_decode_pca_h<D, R, BITS, true>), g, b, 0, st, a, per);
  else hipLaunchKernelGGL((k_decode_pca_h<D, R, BITS, false>), g, b, 0, st, a, per);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t launch_dp_dr(int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return launch_dp_t<D, R, 1>(bf16, a, st);
    case 2: return launch_dp_t<D, R, 2>(bf16, a, st);
    case 3: return launch_dp_t<D, R, 3>(bf16, a, st);
    case 4: return launch_dp_t<D, R, 4>(bf16, a, st);
  }
  return hipErrorInvalidValue;
}

bool decode_pca_h_supported(int D, int r) {
  return (D == 64 && (r == 32 || r == 64)) || (D == 128 && (r == 32 || r == 64 || r == 128));
}

hipError_t launch_decode_pca_h(int D, int r, int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (D == 64 && r == 32) return launch_dp_dr<64, 32>(bits, bf16, a, st);
  if (D == 64 && r == 64) return launch_dp_dr<64, 64>(bits, bf16, a, st);
  if (D == 128 && r == 32) return launch_dp_dr<128, 32>(bits, bf16, a, st);
  if (D == 128 && r == 64) return launch_dp_dr<128, 64>(bits, bf16, a, st);
  if (D == 128 && r == 128) return launch_dp_dr<128, 128>(bits, bf16, a, st);
  return hipErrorInvalidValue;
}

template <int M>
static hipError_t launch_dh_m(int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return launch_dh_t<M, 1>(bf16, a, st);
    case 2: return launch_dh_t<M, 2>(bf16, a, st);
    case 3: return launch_dh_t<M, 3>(bf16, a, st);
    case 4: return launch_dh_t<M, 4>(bf16, a, st);
  }
  return hipErrorInvalidValue;
}

bool decode_h_supported(int D, int m, bool outliers) {
  // outlier lists are merged into the B operands at m <= 128 (one-byte indices)
  return D == m && (m == 64 || m == 128 || ((m == 256 || m == 512) && !outliers));
}

hipError_t launch_decode_h(int m, int bits, bool bf16, const DecodeArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (m == 64) return launch_dh_m<64>(bits, bf16, a, st);
  if (m == 128) return launch_dh_m<128>(bits, bf16, a, st);
  if (m == 256) return launch_dh_m<256>(bits, bf16, a, st);
  if (m == 512) return launch_dh_m<512>(bits, bf16, a, st);
  return hipErrorInvalidValue;
}

}  // namespace kvq
