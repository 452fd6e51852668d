// kvq_score.hip — raw attention logits straight from packed K records.
//
// score[b][h][t] = q[b][h] . x^[b][kv][t] = (n_t/M) sum_i q'_i z^_{t,i},  q' = H_M (s (.) q):
// the sign diagonal and the Hadamard matrix are symmetric, so rotating the query once replaces
// decoding every key [arc PR #98 / #94 kernel commit: attention reads packed K directly]. With
// a projection, x^ = mu + B v^ gives q.x^ = q.mu + (n/r) sum_i q''_i z^_i, q'' = H_r(s (.) B^T q).
// The query heads that share a KV head (GQA) are scored together so each record is read once.
//
// Work split: the products run on MFMA (v_mfma_f32_16x16x32_f16) as S^T = Q' Z^T for tiles of
// 16 heads (G <= 8 used) x 16 tokens x 32 coordinates. A = the rotated queries, scaled per head by
// a power of two into the f16 range and split into f16 hi + lo once per block; B = the
// dequantised keys: each lane expands 8 coordinates of one token through a 2^(2b)-entry LDS
// table indexed by the bit pairs of two coordinates, whose entries are the two centroids as an
// f16 pair (scaled by a power of two per table), i.e. MFMA operand words. hi*c + lo*c carry the
// query to ~2^-22 and the centroid to 2^-11, products exact in the f32 accumulator. A block
// takes a run of tokens of one (batch, KV head), so the query preparation is paid once per run.
#include "kvq_device.h"
#include "kvq_kernels.h"

namespace kvq {

constexpr int kScoreThreads = 256;
constexpr int kScoreSegment = 256;  // tokens per basis check (basis blocks are multiples of 256)
constexpr int kScoreHeads = 8;      // query heads per KV head handled (MFMA rows 8..15 idle)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma16(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Max / sum over the 16 lanes of a DPP row (quad swaps, then half-row and row mirrors: each step
// pairs every lane with one of the other half it has not yet combined with); every lane of the
// row gets the result.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  return x + dpp_f32<0x140>(x);
}

// bf16 hi + lo of an f32 (both round to nearest even): hi + lo = x to ~2^-17 relative.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - __uint_as_float(hi << 16));
}

// The same split of two f32 at once, as packed pairs (x0 in the low halves): two
// v_cvt_pk_bf16_f32 (round to nearest even, as above) around the two residuals.
__device__ __forceinline__ void split_bf16_pair(float x0, float x1, uint32_t& hp, uint32_t& lp) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {x0, x1};
  hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
  const f2 r = {x0 - __uint_as_float(hp << 16), x1 - __uint_as_float(hp & 0xFFFF0000u)};
  lp = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, b2));
}

// Pair-table index of the coordinates at bits sh + pr, sh + pr + 1 of the b plane words w:
// bit 2p + i of the index = plane p of coordinate i. For b = 2, 3 the planes' bit pairs are
// gathered into one word (byte p = plane p) and brought together by one 24-bit multiply:
// with y = a + b 2^8 + c 2^16 (a, b, c < 4), y * (2^16 + 2^10 + 2^4) holds a + 4 b + 16 c in bits
// 16..21 and nothing else reaches those bits or carries into them.
template <int BITS>
__device__ __forceinline__ uint32_t pair_index(const uint32_t* w, int sh, int pr) {
  if constexpr (BITS == 1) {
    return __builtin_amdgcn_ubfe(w[0], sh + pr, 2);
  } else if constexpr (BITS == 2 || BITS == 3) {
    uint32_t y = __builtin_amdgcn_ubfe(w[0], sh, 8) | (__builtin_amdgcn_ubfe(w[1], sh, 8) << 8);
    if constexpr (BITS == 3) y |= __builtin_amdgcn_ubfe(w[2], sh, 8) << 16;
    const uint32_t mask = (BITS == 3 ? 0x030303u : 0x0303u) << pr;
    const uint32_t prod = __umul24(y & mask, BITS == 3 ? 0x10410u : 0x10400u);
    return __builtin_amdgcn_ubfe(prod, 16 + pr, 2 * BITS);
  } else {
    uint32_t idx = 0;
#pragma unroll
    for (int p = 0; p < BITS; ++p) idx |= __builtin_amdgcn_ubfe(w[p], sh + pr, 2) << (2 * p);
    return idx;
  }
}

// Rotated queries of heads [0, 8) of one (batch, kv head) into qs[h * M + pos] (plane-position
// order pos = (i mod 8) * (M/8) + i/8; heads >= G are zero) and qmu[h] = q_h . mu (projection).
// The projection uq[h][j] = sum_d q[h][d] B[d][j] runs on the vector ALUs: the queries are
// staged in LDS as f32 [d][h] (qT), thread (row slice, column pair) reads its slice's basis rows
// two columns per 32-bit load straight from memory (a wave reads whole basis rows), and the
// slices' partial sums meet in LDS (part, [slice][h][M]). Every thread of the block calls this;
// it synchronises.
template <int D, int M>
constexpr int proj_slices() { return kScoreThreads / (M / 2); }

// hook(0) runs once the prologue's global loads are issued, hook(1) after a block barrier that
// follows it (the pair tables are filled in these two phases while the loads are in flight).
struct NoHook {
  __device__ void operator()(int) const {}
};

template <int D, int M, bool PCA, class Hook = NoHook>
__device__ __forceinline__ void prepare_queries(const ScoreArgs& a, int b, int kv, int G, int bi,
                                                float* qs, float* qmu, float* qT, float* part,
                                                float* qpow, Hook hook = Hook()) {
  float* qmp = part + proj_slices<D, M>() * kScoreHeads * M;  // q . mu pair products [h][D / 2]
  constexpr int H = kScoreHeads;
  constexpr int LPV = M / 8;
  constexpr int HPB = kScoreThreads / LPV;  // heads per rotation pass
  constexpr int NS = proj_slices<D, M>();
  const int tid = threadIdx.x;
  const uint16_t* qb = a.q + b * a.q_sb + (int64_t)kv * G * a.q_sh;
  if constexpr (PCA) {
    constexpr int CP = M / 2, RS = D / NS;
    constexpr int QP = D * H / 2 / kScoreThreads;  // query bf16 pairs staged per thread
    static_assert(kScoreThreads % CP == 0 && D % NS == 0 && QP >= 1, "projection split");
    const int cp = tid % CP, sl = tid / CP;
    // every global load first (one memory round trip): basis rows, query pairs, mean pairs
    uint32_t qw[QP];
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int e = tid + kScoreThreads * i, h = e / (D / 2), d = 2 * (e % (D / 2));
      qw[i] = h < G ? *reinterpret_cast<const uint32_t*>(qb + (int64_t)h * a.q_sh + d) : 0u;
    }
    const uint32_t* Bk = reinterpret_cast<const uint32_t*>(a.pca.basis + (int64_t)bi * D * M) + cp;
    uint32_t bw[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) bw[i] = Bk[(sl * RS + i) * CP];
    // the mean's coordinate pairs matching the staged query pairs, for q . mu
    const float* mub = a.pca.mean ? a.pca.mean + (int64_t)bi * D : nullptr;
    float2 mw[QP];
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int e = tid + kScoreThreads * i, d = 2 * (e % (D / 2));
      mw[i] = mub ? *reinterpret_cast<const float2*>(mub + d) : make_float2(0.0f, 0.0f);
    }
    hook(0);
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int e = tid + kScoreThreads * i, h = e / (D / 2), d = 2 * (e % (D / 2));
      const float q0 = bf16lo_to_f32(qw[i]), q1 = bf16hi_to_f32(qw[i]);
      qT[d * H + h] = q0;
      qT[(d + 1) * H + h] = q1;
      qmp[e] = fmaf(q1, mw[i].y, q0 * mw[i].x);  // [h][d / 2]
    }
    __syncthreads();
    hook(1);
    float p0[H], p1[H];
#pragma unroll
    for (int h = 0; h < H; ++h) p0[h] = p1[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int d = sl * RS + i;
      const float4 x0 = *reinterpret_cast<const float4*>(qT + d * H);
      const float4 x1 = *reinterpret_cast<const float4*>(qT + d * H + 4);
      const float qq[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float b0 = bf16lo_to_f32(bw[i]), b1 = bf16hi_to_f32(bw[i]);
#pragma unroll
      for (int h = 0; h < H; ++h) {
        p0[h] = fmaf(qq[h], b0, p0[h]);
        p1[h] = fmaf(qq[h], b1, p1[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < H; ++h)
      *reinterpret_cast<float2*>(part + (sl * H + h) * M + 2 * cp) = make_float2(p0[h], p1[h]);
    if (tid < 8 * H) {  // q . mu: 8 lanes per head sum the head's pair products
      const int hm = tid / 8, lm = tid % 8;
      float sm = 0.0f;
#pragma unroll
      for (int k = 0; k < D / 16; ++k) sm += qmp[hm * (D / 2) + lm * (D / 16) + k];
      sm += __shfl_xor(sm, 1, 64);
      sm += __shfl_xor(sm, 2, 64);
      sm += __shfl_xor(sm, 4, 64);
      if (lm == 0) qmu[hm] = sm;
    }
    __syncthreads();
  }
  // s (.) v, then the M-point Hadamard transform, LPV lanes per head with 8 coordinates each
  const int c = tid % LPV;
  uint4 raw0 = make_uint4(0, 0, 0, 0);  // the first pass's query coordinates (no projection)
  if constexpr (!PCA) {
    if (tid / LPV < G) raw0 = *reinterpret_cast<const uint4*>(qb + (int64_t)(tid / LPV) * a.q_sh + 8 * c);
    if (tid < H) qmu[tid] = 0.0f;
    hook(0);
    __syncthreads();
    hook(1);
  }
  const uint32_t sbyte = (a.tab.sign_words[(c >> 2) & 15] >> (8 * (c & 3))) & 0xFFu;
  for (int h0 = 0; h0 < H; h0 += HPB) {
    const int h = h0 + tid / LPV;
    float v[8];
    if constexpr (PCA) {
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (h < H) {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const float4 u0 = *reinterpret_cast<const float4*>(part + (sl * H + h) * M + 8 * c);
          const float4 u1 = *reinterpret_cast<const float4*>(part + (sl * H + h) * M + 8 * c + 4);
          x[0] += u0.x; x[1] += u0.y; x[2] += u0.z; x[3] += u0.w;
          x[4] += u1.x; x[5] += u1.y; x[6] += u1.z; x[7] += u1.w;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(__float_as_uint(x[j]) ^ (((sbyte >> j) & 1u) << 31));
    } else {
      uint4 raw = raw0;
      if (h0 > 0 && h < G) raw = *reinterpret_cast<const uint4*>(qb + (int64_t)h * a.q_sh + 8 * c);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float((w[k] << 16) ^ (((sbyte >> (2 * k)) & 1u) << 31));
        v[2 * k + 1] = __uint_as_float((w[k] & 0xFFFF0000u) ^ (((sbyte >> (2 * k + 1)) & 1u) << 31));
      }
    }
    fwht_vector<LPV>(v, c);
    // qpow[h] = the power of two 2^e with max_i |q'_h,i| / 2^e in [2^14, 2^15) (1 for a zero
    // query): scaled by it, the head's coordinates use the whole f16 range
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) mx = fmaxf(mx, lane_xor(mx, m));
    if (h < H) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qs[h * M + j * LPV + c] = v[j];
      if (c == 0) qpow[h] = mx > 0.0f ? ldexpf(1.0f, ilogbf(mx) - 14) : 1.0f;
    }
  }
  __syncthreads();
}

// Pair table: entry e (bit 2p + i = plane p of code i) holds the centroids of its two codes as
// their bf16 hi pair (lut[e COPIES + c]) and lo pair (lut[(NPAIR + e) COPIES + c]), copy c read by
// lanes l with l % COPIES == c, so the lookups of a half-wave never share an LDS bank. Filled in
// two phases around a block barrier: pair_entries forms each entry once (copy 0), and
// pair_replicate copies it, consecutive threads writing consecutive words.
template <int BITS, int COPIES>
__device__ __forceinline__ void pair_codes(int e, uint32_t& ca, uint32_t& cb) {
  ca = cb = 0;
#pragma unroll
  for (int p = 0; p < BITS; ++p) {
    ca |= ((e >> (2 * p)) & 1u) << p;
    cb |= ((e >> (2 * p + 1)) & 1u) << p;
  }
}

template <int BITS>
__device__ __forceinline__ float centroid_of(const Tables& tab, uint32_t code) {
  float v = 0.0f;
#pragma unroll
  for (int k = 0; k < (1 << BITS); ++k) v = (uint32_t)k == code ? tab.c[k] : v;
  return v;
}

template <int BITS, int COPIES>
__device__ __forceinline__ void pair_entries(const Tables& tab, uint32_t* lut, int tid) {
  constexpr int NPAIR = 1 << (2 * BITS);
  for (int e = tid; e < NPAIR; e += kScoreThreads) {
    uint32_t ca, cb, ha, la, hb, lb;
    pair_codes<BITS, COPIES>(e, ca, cb);
    split_bf16(centroid_of<BITS>(tab, ca), ha, la);
    split_bf16(centroid_of<BITS>(tab, cb), hb, lb);
    lut[e * COPIES] = ha | (hb << 16);
    lut[(NPAIR + e) * COPIES] = la | (lb << 16);
  }
}

// WORDS = table words per copy set (NPAIR, or 2 NPAIR with the lo pairs).
template <int WORDS, int COPIES>
__device__ __forceinline__ void pair_replicate(uint32_t* lut, int tid) {
  for (int i = tid; i < WORDS * COPIES; i += kScoreThreads)
    if (i % COPIES != 0) lut[i] = lut[i - i % COPIES];
}

// Copies per pair table: one per lane of a half-wave up to 3 bits (16 KB at 3 bits), 4 at 4 bits.
template <int BITS>
constexpr int pair_copies() { return BITS <= 3 ? 32 : 4; }

// ---- f16 products for the score kernel -------------------------------------------------
// The score multiplies each rotated query, scaled per head by a power of two into the f16
// range and split into f16 hi + lo, by the f16 centroids (scaled by one power of two per table):
// each product is exact in the f32 accumulator, q'_hi + q'_lo carries ~2^-22 of q', and the
// centroid's f16 rounding (<= 2^-11 relative) bounds the error of every term, so
// |score error| <= ~5e-4 * (n/m) sum_i |q'_i c_i|. One table word (a pair of f16 centroids)
// per two coordinates and two products per k-step.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4_t mfma16h(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                 __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// The power of two that brings the table's largest centroid magnitude into [2^14, 2^15).
template <int BITS>
__device__ __forceinline__ float table_pow(const Tables& tab) {
  float mx = 0.0f;
#pragma unroll
  for (int k = 0; k < (1 << BITS); ++k) mx = fmaxf(mx, fabsf(tab.c[k]));
  return mx > 0.0f ? ldexpf(1.0f, ilogbf(mx) - 14) : 1.0f;
}

// f16 pair table: word e COPIES + c = the two centroids of entry e (bit 2p + i = plane p of
// code i) divided by cpow, as an f16 pair; copy c read by lanes l % COPIES == c. With LO, words
// (NPAIR + e) COPIES + c hold the pair's f16 remainders (centroid to ~2^-22). Entries here,
// copies by pair_replicate after a barrier.
template <int BITS, int COPIES, bool LO>
__device__ __forceinline__ void pair_entries_f16(const Tables& tab, float inv_cpow, uint32_t* lut,
                                                 int tid) {
  constexpr int NPAIR = 1 << (2 * BITS);
  for (int e = tid; e < NPAIR; e += kScoreThreads) {
    uint32_t ca, cb;
    pair_codes<BITS, COPIES>(e, ca, cb);
    const float va = centroid_of<BITS>(tab, ca) * inv_cpow, vb = centroid_of<BITS>(tab, cb) * inv_cpow;
    const _Float16 ha = (_Float16)va, hb = (_Float16)vb;
    lut[e * COPIES] = (uint32_t)__builtin_bit_cast(uint16_t, ha) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
    if constexpr (LO)
      lut[(NPAIR + e) * COPIES] = f16_bits(va - (float)ha) | (f16_bits(vb - (float)hb) << 16);
  }
}

// A operands of the rotated queries (head tok, coordinates 32 ks + 8 oct + [0, 8)) divided by
// their head's power of two, as f16 hi and lo halves.
template <int M>
__device__ __forceinline__ void query_operands_f16(const float* qs, const float* qpow, int tok,
                                                   int oct, uint4 (&qa_hi)[M / 32],
                                                   uint4 (&qa_lo)[M / 32]) {
  constexpr int H = kScoreHeads;
  const float inv = tok < H ? 1.0f / qpow[tok] : 0.0f;
#pragma unroll
  for (int ks = 0; ks < M / 32; ++ks) {
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = tok < H ? qs[tok * M + 32 * ks + 8 * oct + e] * inv : 0.0f;
      const _Float16 xh = (_Float16)x;
      hi[e] = (uint32_t)__builtin_bit_cast(uint16_t, xh);
      lo[e] = f16_bits(x - (float)xh);
    }
    qa_hi[ks] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                           hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    qa_lo[ks] = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                           lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
  }
}

// Byte permute selectors that gather, for lane group oct, byte oct of plane words w[0], w[1]
// (sel01) and then w[2] (sel2) into bytes 0, 1, 2 of one word.
__device__ __forceinline__ uint32_t planes_sel01(int oct) {
  return 0x0c0c0000u | ((uint32_t)(4 + oct) << 8) | (uint32_t)oct;
}
__device__ __forceinline__ uint32_t planes_sel2(int oct) {
  return 0x0c000100u | ((uint32_t)(4 + oct) << 16);
}

// Raw logits (divided by the head's and the table's powers of two) of one 16-token record tile:
// acc[k] for head 4 oct + k and token tok. For b = 2, 3 the lane's plane bytes sit side by side
// in one word y (byte p = plane p of its 8 coordinates); the pair index of coordinates 2 pr,
// 2 pr + 1 is sum_p 4^p (plane-p bit pair), one byte dot product of the masked word with the
// weights (1, 4, 16), which for odd pr comes out times 4 and is scaled into the table address.
template <int M, int BITS, int COPIES, bool LO>
__device__ __forceinline__ floatx4_t tile_dots_f16(const uint32_t* w, const uint32_t* lut, int lane,
                                                   int oct, uint32_t sel01, uint32_t sel2,
                                                   const uint4 (&qa_hi)[M / 32],
                                                   const uint4 (&qa_lo)[M / 32]) {
  static_assert(COPIES == 32 || BITS > 3, "pair-table address shifts assume 32 copies");
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* lc = lut + (lane & (COPIES - 1));
#pragma unroll
  for (int ks = 0; ks < M / 32; ++ks) {
    const uint32_t* wk = w + ks * BITS;
    uint32_t z[4], zl[4];
    if constexpr (BITS == 2 || BITS == 3) {
      uint32_t y = __builtin_amdgcn_perm(wk[1], wk[0], sel01);
      if constexpr (BITS == 3) y = __builtin_amdgcn_perm(wk[2], y, sel2);
      const uint32_t y2 = y >> 4;
      constexpr uint32_t mask = BITS == 3 ? 0x030303u : 0x0303u;
      constexpr uint32_t wts = BITS == 3 ? 0x100401u : 0x0401u;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t src = pr < 2 ? y : y2;
        const uint32_t d = __builtin_amdgcn_udot4(src & (mask << (2 * (pr & 1))), wts, 0u, false);
        const uint32_t off = d << ((pr & 1) ? 3 : 5);
        z[pr] = lc[off];
        if constexpr (LO) zl[pr] = lc[(1 << (2 * BITS)) * COPIES + off];
      }
    } else {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t off = pair_index<BITS>(wk, 8 * oct, 2 * pr) * COPIES;
        z[pr] = lc[off];
        if constexpr (LO) zl[pr] = lc[(1 << (2 * BITS)) * COPIES + off];
      }
    }
    const uint4 bz = make_uint4(z[0], z[1], z[2], z[3]);
    acc = mfma16h(qa_hi[ks], bz, acc);
    acc = mfma16h(qa_lo[ks], bz, acc);
    if constexpr (LO) acc = mfma16h(qa_hi[ks], make_uint4(zl[0], zl[1], zl[2], zl[3]), acc);
  }
  return acc;
}

// ---- The packed score's tile: both query halves in one product --------------------------
// Row m of the A operand holds head h = m / 4 + 4 ((m % 4) / 2) as its f16 hi half (m even) or lo
// half (m odd), divided by the head's power of two. The accumulator of lane (oct, tok) then holds
// head oct's hi and lo partial sums in acc[0], acc[1] and head oct + 4's in acc[2], acc[3]: one
// product per k-step instead of two, and at up to 4 heads per KV head every lane owns one score.
template <int M>
__device__ __forceinline__ void query_rows_f16(const float* qs, const float* qpow, int m, int oct,
                                               uint4 (&qa)[M / 32]) {
  const int h = (m >> 2) + 4 * ((m & 3) >> 1);
  const bool lo = m & 1;
  const float inv = 1.0f / qpow[h];
#pragma unroll
  for (int ks = 0; ks < M / 32; ++ks) {
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = qs[h * M + 32 * ks + 8 * oct + e] * inv;
      const _Float16 xh = (_Float16)x;
      v[e] = lo ? f16_bits(x - (float)xh) : (uint32_t)__builtin_bit_cast(uint16_t, xh);
    }
    qa[ks] = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                        v[6] | (v[7] << 16));
  }
}

// Raw logits of one 16-token record tile against the query rows above (divided by the heads' and
// the table's powers of two). The pair table has one copy: entry e (bit 2p + i = plane p of code
// i) is word e. For b = 2, 3 the entry's byte address 4 e is one byte dot product of the masked
// plane bytes with weights (4, 16, 64) (coordinates at bits 0, 1 of each byte) or (1, 4, 16)
// (bits 2, 3, whose bytes already carry a factor 4); the table's own address folds into the load.
template <int M, int BITS>
__device__ __forceinline__ floatx4_t tile_dots_rows(const uint32_t* w, const uint32_t* lut, int oct,
                                                    uint32_t sel01, uint32_t sel2,
                                                    const uint4 (&qa)[M / 32]) {
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  const char* lb = reinterpret_cast<const char*>(lut);
#pragma unroll
  for (int ks = 0; ks < M / 32; ++ks) {
    const uint32_t* wk = w + ks * BITS;
    uint32_t z[4];
    if constexpr (BITS == 2 || BITS == 3) {
      uint32_t y = __builtin_amdgcn_perm(wk[1], wk[0], sel01);
      if constexpr (BITS == 3) y = __builtin_amdgcn_perm(wk[2], y, sel2);
      const uint32_t y2 = y >> 4;
      constexpr uint32_t mask = BITS == 3 ? 0x030303u : 0x0303u;
      constexpr uint32_t w_even = BITS == 3 ? 0x401004u : 0x1004u;
      constexpr uint32_t w_odd = BITS == 3 ? 0x100401u : 0x0401u;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t src = pr < 2 ? y : y2;
        const uint32_t d = (pr & 1) ? __builtin_amdgcn_udot4(src & (mask << 2), w_odd, 0u, false)
                                    : __builtin_amdgcn_udot4(src & mask, w_even, 0u, false);
        z[pr] = *reinterpret_cast<const uint32_t*>(lb + d);
      }
    } else {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) z[pr] = lut[pair_index<BITS>(wk, 8 * oct, 2 * pr)];
    }
    acc = mfma16h(qa[ks], make_uint4(z[0], z[1], z[2], z[3]), acc);
  }
  return acc;
}

// Steps of the score loop. A wave takes the 64 consecutive tokens s0 + 64 wave + [0, 64) of each
// 256-token segment, in steps of TPS 16-token tiles. A step's records are one contiguous byte
// range: they leave memory as dword loads spread over the wave's lanes (SW per lane, no lane
// loading what another lane loads) and reach the lanes that multiply them through the wave's
// LDS slice. PF steps are in flight while one computes.
template <int NWT>
struct ScoreSteps {
  static constexpr int TPS = NWT <= 16 ? 4 : (NWT <= 32 ? 2 : 1);  // tiles per step
  static constexpr int WORDS = 16 * TPS * NWT;                      // record dwords per step
  static constexpr int SW = (WORDS + 63) / 64;                      // dwords per lane
  static constexpr int PF = (32 / SW) < 1 ? 1 : ((32 / SW) > 4 ? 4 : 32 / SW);
  static constexpr int SPS = 4 / TPS;                               // steps per segment
};

template <int D, int M, int BITS, bool PCA>
__global__ __launch_bounds__(kScoreThreads) void k_score(ScoreArgs a, int64_t chunks_per_pair) {
  constexpr int H = kScoreHeads;
  constexpr int KS = M / 32;              // MFMA k-steps (one 32-coordinate word group each)
  constexpr int NWC = KS * BITS, NWT = NWC + 1;
  using St = ScoreSteps<NWT>;
  constexpr int TPS = St::TPS, SW = St::SW, PF = St::PF, SPS = St::SPS, WORDS = St::WORDS;
  __shared__ __attribute__((aligned(16))) float qs[H * M];
  __shared__ float qmu[H];
  __shared__ float qpow[H];
  __shared__ uint32_t lut[1 << (2 * BITS)];  // entry e: f16 centroid pair
  // the projection's staging (queries, partial sums) and the loop's record staging share LDS:
  // the former is live only inside prepare_queries, between barriers, before a step's records
  // are staged
  constexpr int PRE = PCA ? D * H + proj_slices<D, M>() * H * M + H * D / 2 : 0;
  constexpr int STG = (kScoreThreads / 64) * WORDS;
  __shared__ __attribute__((aligned(16))) float work[PRE > STG ? PRE : STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* qT = work;
  float* part = work + D * H;
  uint32_t* stage = reinterpret_cast<uint32_t*>(work) + wave * WORDS;
  const int tok = lane & 15, oct = lane >> 4;
  const int64_t pair = blockIdx.x / chunks_per_pair;
  const int b = (int)(pair / a.Hkv), kv = (int)(pair % a.Hkv);
  const int G = a.Hq / a.Hkv;
  // the block's 256-token segments of its (batch, KV head): j, j + cpp, j + 2 cpp, ...: the
  // blocks of a pair advance through its records side by side
  const int64_t cpp = chunks_per_pair, jseg = blockIdx.x % chunks_per_pair;
  const int64_t segs = (a.T + kScoreSegment - 1) / kScoreSegment;
  const int64_t my_segs = jseg < segs ? (segs - jseg + cpp - 1) / cpp : 0;
  const int64_t t_end = a.T;
  auto seg_t0 = [&](int64_t k) { return kScoreSegment * (jseg + cpp * k); };
  const int64_t rowbase = b * a.rec_sb + kv * a.rec_sh;
  const int64_t n_steps = my_segs * SPS;
  const uint32_t* rec32 = reinterpret_cast<const uint32_t*>(a.rec);
  // first token of step g of this wave
  auto step_t0 = [&](int64_t g) {
    return seg_t0(g / SPS) + 64 * wave + 16 * TPS * (g % SPS);
  };
  auto load_step = [&](int64_t g, uint32_t (&buf)[SW]) {
    const int64_t t0 = step_t0(g), left = t_end - t0;
    const int lim = left >= 16 * TPS ? WORDS : (left > 0 ? (int)left * NWT : 0);  // uniform
    const uint32_t* src = rec32 + (rowbase + t0) * NWT + lane;
    // records are read once: streaming (nontemporal) loads keep them from displacing the
    // score rows in the caches (measured 124 -> 117 us on the long-context score)
    if (lim == WORDS && WORDS == 64 * SW) {
#pragma unroll
      for (int i = 0; i < SW; ++i) buf[i] = __builtin_nontemporal_load(src + 64 * i);
    } else {
#pragma unroll
      for (int i = 0; i < SW; ++i)
        buf[i] = lane + 64 * i < lim ? __builtin_nontemporal_load(src + 64 * i) : 0u;
    }
  };
  int bi = PCA ? basis_of_row(a.pca, rowbase + (my_segs > 0 ? seg_t0(0) : 0)) : 0;
  uint32_t ring[PF][SW];
  const float cpow = table_pow<BITS>(a.tab);
  prepare_queries<D, M, PCA>(a, b, kv, G, bi, qs, qmu, qT, part, qpow, [&](int phase) {
    if (phase == 0) {
      // the first steps' record loads go out behind the prologue's own loads, which the
      // prologue then waits for alone
#pragma unroll
      for (int r = 0; r < PF; ++r)
        if (r < n_steps) load_step(r, ring[r]);
      pair_entries_f16<BITS, 1, false>(a.tab, 1.0f / cpow, lut, tid);
    }
  });
  uint4 qa[KS];     // A operand: row tok (a head's hi or lo half), coordinates 32 ks + 8 oct .. + 7
  float qm[2], qsc[2];  // q . mu and the product's scale of heads oct and oct + 4
  auto operands = [&]() {
    query_rows_f16<M>(qs, qpow, tok, oct, qa);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      qm[k] = qmu[oct + 4 * k];
      qsc[k] = qpow[oct + 4 * k] * cpow * a.tab.inv_m;
    }
  };
  operands();
  const uint32_t sel01 = planes_sel01(oct), sel2 = planes_sel2(oct);
  int bnext = bi;
  for (int64_t g0 = 0; g0 < n_steps; g0 += PF) {
#pragma unroll
    for (int r = 0; r < PF; ++r) {
      const int64_t g = g0 + r;
      if (g >= n_steps) break;  // uniform
      if constexpr (PCA) {
        if (g % SPS == 0) {
          if (g > 0 && bnext != bi) {  // block-uniform: a new basis from this segment on
            __syncthreads();
            prepare_queries<D, M, PCA>(a, b, kv, G, bnext, qs, qmu, qT, part, qpow);
            operands();
            bi = bnext;
          }
          // the next segment's basis, looked up one segment ahead
          bnext = g / SPS + 1 < my_segs ? basis_of_row(a.pca, rowbase + seg_t0(g / SPS + 1)) : bi;
        }
      }
      // this step's records to the wave's LDS slice, then the slot refills
#pragma unroll
      for (int i = 0; i < SW; ++i)
        if (lane + 64 * i < WORDS) stage[lane + 64 * i] = ring[r][i];
      if (g + PF < n_steps) load_step(g + PF, ring[r]);
      __builtin_amdgcn_wave_barrier();
      const int64_t t0 = step_t0(g);
      float* srow = a.s + b * a.s_sb + (int64_t)kv * G * a.s_sh + t0 + tok;
#pragma unroll
      for (int tt = 0; tt < TPS; ++tt) {
        uint32_t w[NWT];
#pragma unroll
        for (int k = 0; k < NWT; ++k) w[k] = stage[(16 * tt + tok) * NWT + k];
        const floatx4_t acc = tile_dots_rows<M, BITS>(w, lut, oct, sel01, sel2, qa);
        const float nrm = __uint_as_float(w[NWC]);
        const bool tv = t0 + 16 * tt + tok < t_end;
        if (tv && oct < G) srow[(int64_t)oct * a.s_sh + 16 * tt] = fmaf(acc[0] + acc[1], nrm * qsc[0], qm[0]);
        if (tv && oct + 4 < G)
          srow[(int64_t)(oct + 4) * a.s_sh + 16 * tt] = fmaf(acc[2] + acc[3], nrm * qsc[1], qm[1]);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode attention over packed K and V [arc PR #98 / #94 kernel commit: the attention kernel
// reads the packed cache directly; arc PR #98, "Also: two silently-ignored kernel parameters":
// the soft cap acts after the scale multiply and before the running maximum].
//
// A block takes a run of tokens of one (batch, KV head) and the G <= 8 query heads of its
// group. Each wave walks 32-token units: the logits of two 16-token tiles on MFMA exactly as in
// k_score, an online softmax per head (running maximum m and sum l), and
//   acc[h][P] += sum_t p[h][t] (n_t / m) z^_t[P]     (P = plane position of the V codec)
// in the V codec's rotated domain, also on MFMA: A = the centroids of 16 positions x 32 tokens
// expanded from the V records' bit planes (two tokens per pair-table entry, bf16 hi + lo), B =
// the unit's weights p (n/m), transposed through LDS. The inverse rotation is linear, so it is
// applied once per query head after the partials are merged (k_attend_combine):
//   out = s (.) H (sum_c e^{m_c - M} acc_c) / (sum_c e^{m_c - M} l_c).

constexpr int kAttnWaves = kScoreThreads / 64;

template <int D>
constexpr int attend_stride() { return D + 4; }  // partial of one head: m, l, pad, acc[D]

template <int D, int M, int BK, bool PCA, int BV>
__global__ __launch_bounds__(kScoreThreads) void k_attend(AttendArgs a) {
  constexpr int H = kScoreHeads;
  constexpr int KS = M / 32, NWK = KS * BK + 1;
  constexpr int CK = pair_copies<BK>();
  constexpr int GV = D / 32, NWV = GV * BV + 1;  // V word groups, V record words
  constexpr int NPV = 1 << (2 * BV), CV = pair_copies<BV>();
  constexpr int CT = D / 16;                     // 16-position tiles of the V accumulator
  constexpr int VPL = (32 * NWV + 63) / 64;      // V record dwords staged per lane
  constexpr int S = attend_stride<D>();
  __shared__ __attribute__((aligned(16))) float qs[H * M];
  __shared__ float qmu[H];
  __shared__ float qpow[H];
  __shared__ uint32_t lutk[2 * (1 << (2 * BK)) * CK];  // f16 centroid pairs (hi | lo) of the K codec
  __shared__ uint32_t lutv[2 * NPV * CV];
  __shared__ __attribute__((aligned(16))) float qT[PCA ? D * H : 1];
  __shared__ __attribute__((aligned(16))) float part[PCA ? proj_slices<D, M>() * H * M + H * D / 2 : 1];
  __shared__ uint32_t vst[kAttnWaves][32 * NWV];                         // the unit's V records
  __shared__ __attribute__((aligned(16))) float pst[kAttnWaves][16][32];  // p (n/m) [head][token]
  __shared__ float cst[kAttnWaves][16];                                   // accumulator rescale
  const ScoreArgs& k = a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = lane & 15, oct = lane >> 4;
  const int64_t pair = blockIdx.x / a.chunks;
  const int b = (int)(pair / k.Hkv), kv = (int)(pair % k.Hkv);
  const int G = k.Hq / k.Hkv;
  const int64_t t_begin = (blockIdx.x % a.chunks) * a.chunk;
  const int64_t t_end = t_begin + a.chunk < k.T ? t_begin + a.chunk : k.T;
  const int64_t rowbase = b * k.rec_sb + kv * k.rec_sh;
  const uint32_t* krec32 = reinterpret_cast<const uint32_t*>(k.rec);
  const uint32_t* vrec32 = reinterpret_cast<const uint32_t*>(a.vrec);
  uint4 qa_hi[KS], qa_lo[KS];
  float qm[4], qsc[4], mrun[4], lrun[4];  // q . mu, product scale, softmax state of heads 4 oct + kk
  const float cpow = table_pow<BK>(k.tab);
  const uint32_t sel01 = planes_sel01(oct), sel2 = planes_sel2(oct);
  // V gather: rotation that brings bit tok (and 16 + tok) of a plane word to slot sl (16 + sl)
  uint32_t vrot[2 * BV];
#pragma unroll
  for (int sl = 0; sl < 2 * BV; ++sl) vrot[sl] = (uint32_t)(tok - sl) & 31u;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    mrun[kk] = -INFINITY;
    lrun[kk] = 0.0f;
  }
  floatx4_t acc[CT];  // acc[ct][i]: position 16 ct + 4 oct + i of head tok
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // records of the unit starting at token t0: K words of token tok of both tiles, V record
  // dwords of the 32 tokens (tokens past the end read the last record and get weight 0)
  constexpr int kUnits = kScoreSegment / (32 * kAttnWaves);  // units per wave and segment
  uint32_t wk_n[2][NWK], vv_n[VPL];
  auto load_unit = [&](int64_t t0) {
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      int64_t t = t0 + 16 * tile + tok;
      t = t < t_end ? t : t_end - 1;
      const uint32_t* r32 = krec32 + (rowbase + t) * NWK;
#pragma unroll
      for (int i = 0; i < NWK; ++i) wk_n[tile][i] = r32[i];
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int idx = lane + 64 * i;
      int64_t t = t0 + idx / NWV;
      t = t < t_end ? t : t_end - 1;
      vv_n[i] = idx < 32 * NWV ? vrec32[(rowbase + t) * NWV + idx % NWV] : 0u;
    }
  };
  if (t_begin + 32 * wave < t_end) load_unit(t_begin + 32 * wave);
  int cur = -1;
  const int64_t n_seg = (t_end - t_begin + kScoreSegment - 1) / kScoreSegment;
  for (int64_t sg = 0; sg < n_seg; ++sg) {
    const int64_t s0 = t_begin + kScoreSegment * sg;
    const int bi = PCA ? basis_of_row(k.pca, rowbase + s0) : 0;
    if (bi != cur) {  // block-uniform
      __syncthreads();
      prepare_queries<D, M, PCA>(k, b, kv, G, bi, qs, qmu, qT, part, qpow, [&](int phase) {
        if (cur >= 0) return;  // the pair tables are filled with the first basis
        if (phase == 0) {
          pair_entries_f16<BK, CK, true>(k.tab, 1.0f / cpow, lutk, tid);
          pair_entries<BV, CV>(a.tv, lutv, tid);
        } else {
          pair_replicate<2 * (1 << (2 * BK)), CK>(lutk, tid);
          pair_replicate<2 * NPV, CV>(lutv, tid);
        }
      });
      query_operands_f16<M>(qs, qpow, tok, oct, qa_hi, qa_lo);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        qm[kk] = 4 * oct + kk < H ? qmu[4 * oct + kk] : 0.0f;
        qsc[kk] = 4 * oct + kk < H ? qpow[4 * oct + kk] * cpow * k.tab.inv_m : 0.0f;
      }
      cur = bi;
    }
    for (int u = 0; u < kUnits; ++u) {
      const int64_t t0 = s0 + 32 * (kAttnWaves * u + wave);
      if (t0 >= t_end) break;  // wave-uniform
      // this unit's records (prefetched during the previous one) to LDS / registers, and the
      // next unit's loads in flight while this one computes
      uint32_t wk[2][NWK];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int i = 0; i < NWK; ++i) wk[tile][i] = wk_n[tile][i];
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i < 32 * NWV) vst[wave][lane + 64 * i] = vv_n[i];
      {
        const int un = u + 1 < kUnits ? u + 1 : 0;
        const int64_t tn = (u + 1 < kUnits ? s0 : s0 + kScoreSegment) + 32 * (kAttnWaves * un + wave);
        if (tn < t_end) load_unit(tn);
      }
      // logits of heads 4 oct + kk for tokens t0 + tok and t0 + 16 + tok
      float lg[2][4];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const floatx4_t d =
            tile_dots_f16<M, BK, CK, true>(wk[tile], lutk, lane, oct, sel01, sel2, qa_hi, qa_lo);
        const int64_t t = t0 + 16 * tile + tok;
        const float nk = __uint_as_float(wk[tile][NWK - 1]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          float x = fmaf(d[kk], nk * qsc[kk], qm[kk]) * a.scale;
          if (a.softcap > 0.0f) x = a.softcap * tanhf(x / a.softcap);
          lg[tile][kk] = (t < t_end && 4 * oct + kk < G) ? x : -INFINITY;
        }
      }
      __builtin_amdgcn_wave_barrier();
      // online softmax; weights times the V norm scale into pst
      const float nv0 = __uint_as_float(vst[wave][tok * NWV + NWV - 1]) * a.tv.inv_m;
      const float nv1 = __uint_as_float(vst[wave][(16 + tok) * NWV + NWV - 1]) * a.tv.inv_m;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float mx = row16_max(fmaxf(lg[0][kk], lg[1][kk]));
        const float mn = fmaxf(mrun[kk], mx);
        // mn = -inf: no token of this head so far (or a head slot >= G); nothing to rescale
        const float corr = mn == -INFINITY ? 1.0f : __expf(mrun[kk] - mn);
        const float p0 = lg[0][kk] == -INFINITY ? 0.0f : __expf(lg[0][kk] - mn);
        const float p1 = lg[1][kk] == -INFINITY ? 0.0f : __expf(lg[1][kk] - mn);
        const float ps = row16_sum(p0 + p1);
        lrun[kk] = fmaf(lrun[kk], corr, ps);
        mrun[kk] = mn;
        pst[wave][4 * oct + kk][tok] = p0 * nv0;
        pst[wave][4 * oct + kk][16 + tok] = p1 * nv1;
        if (tok == 0) cst[wave][4 * oct + kk] = corr;
      }
      __builtin_amdgcn_wave_barrier();
      // B operand: weights of head tok for tokens 8 oct + [0, 8), bf16 hi and lo
      const float c = cst[wave][tok];
      if (__ballot(c != 1.0f) != 0ull) {  // some head's running maximum moved (rare once settled)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] *= c;
      }
      // B operands: the unit's weights of head tok for tokens 8 oct + [0, 8) as bf16 hi and lo.
      // Interleaved form (low code widths): for A = {hi, lo, hi, lo} of two token pairs (an
      // entry's two table words as one read returns them), bh[q] = {hi(pair 2q), hi(2q),
      // hi(2q + 1), hi(2q + 1)} takes hi + lo of the centroids times hi of the weights and
      // bl[q] = {lo(2q), 0, lo(2q + 1), 0} hi times lo. Otherwise A = all hi or all lo (fewer
      // registers) with bhi, blo = the weights' hi and lo.
      constexpr bool IL = BV <= 2 && BK <= 3;
      uint4 bh[2], bl[2];
      {
        const float4 w0 = *reinterpret_cast<const float4*>(&pst[wave][tok][8 * oct]);
        const float4 w1 = *reinterpret_cast<const float4*>(&pst[wave][tok][8 * oct + 4]);
        const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) split_bf16_pair(w[2 * d], w[2 * d + 1], hp[d], lp[d]);
        if constexpr (IL) {
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            bh[qq] = make_uint4(hp[2 * qq], hp[2 * qq], hp[2 * qq + 1], hp[2 * qq + 1]);
            bl[qq] = make_uint4(lp[2 * qq], 0u, lp[2 * qq + 1], 0u);
          }
        } else {
          bh[0] = make_uint4(hp[0], hp[1], hp[2], hp[3]);  // bhi
          bl[0] = make_uint4(lp[0], lp[1], lp[2], lp[3]);  // blo
        }
      }
      // A operands: centroids at positions P = 32 g + 16 h2 + tok of tokens 8 oct + [0, 8). The
      // pair index of tokens (2 e2, 2 e2 + 1) at both positions of a lane comes from one pass:
      // plane p of token t of the pair is rotated so that its bits tok and 16 + tok land on
      // slot 2 p + t and 16 + 2 p + t, the rotated words are merged by bit masks, and the two
      // indices are the low and high 16-bit halves.
#pragma unroll
      for (int g = 0; g < GV; ++g) {
        uint32_t wv[8][BV];
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int p = 0; p < BV; ++p) wv[e][p] = vst[wave][(8 * oct + e) * NWV + g * BV + p];
        uint32_t ah[2][4], al[2][4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint32_t y = 0u;  // only the placed slots' bits are set: each slot is one v_and_or
#pragma unroll
          for (int sl = 2 * BV - 1; sl >= 0; --sl) {
            const uint32_t w = wv[2 * e2 + (sl & 1)][sl >> 1];
            y |= __builtin_amdgcn_alignbit(w, w, vrot[sl]) & ((1u << sl) | (1u << (16 + sl)));
          }
          const uint32_t i0 = y & 0xFFFFu, i1 = y >> 16;
          ah[0][e2] = lutv[i0 * CV + (lane & (CV - 1))];
          al[0][e2] = lutv[(NPV + i0) * CV + (lane & (CV - 1))];
          ah[1][e2] = lutv[i1 * CV + (lane & (CV - 1))];
          al[1][e2] = lutv[(NPV + i1) * CV + (lane & (CV - 1))];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          floatx4_t& c4 = acc[2 * g + h2];
          if constexpr (IL) {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              const uint4 av = make_uint4(ah[h2][2 * qq], al[h2][2 * qq], ah[h2][2 * qq + 1],
                                          al[h2][2 * qq + 1]);
              c4 = mfma16(av, bh[qq], c4);
              c4 = mfma16(av, bl[qq], c4);
            }
          } else {
            const uint4 ahi = make_uint4(ah[h2][0], ah[h2][1], ah[h2][2], ah[h2][3]);
            const uint4 alo = make_uint4(al[h2][0], al[h2][1], al[h2][2], al[h2][3]);
            c4 = mfma16(ahi, bh[0], c4);
            c4 = mfma16(ahi, bl[0], c4);
            c4 = mfma16(alo, bh[0], c4);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // vst, pst and cst are refilled by the next unit
    }
  }
  // this wave's partial of each head: [m, l, -, -, acc by plane position]
  float* pw = a.part + ((int64_t)blockIdx.x * kAttnWaves + wave) * H * S;
  if (tok < G) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      *reinterpret_cast<float4*>(pw + tok * S + 4 + 16 * ct + 4 * oct) =
          make_float4(acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]);
  }
  if (tok == 0) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int h = 4 * oct + kk;
      if (h < G) {
        pw[h * S] = mrun[kk];
        pw[h * S + 1] = lrun[kk];
      }
    }
  }
}

// Merge of the partials of one (batch, query head) and the inverse rotation of the V codec:
// out = s (.) H a, a[i] = sum_w e^{m_w - M} acc_w[pi(i)] / sum_w e^{m_w - M} l_w.
template <int D>
__global__ __launch_bounds__(64) void k_attend_combine(AttendArgs a) {
  constexpr int LPV = D / 8, H = kScoreHeads, S = attend_stride<D>();
  const ScoreArgs& k = a.k;
  const int lane = threadIdx.x, c = lane % LPV;
  const int b = blockIdx.x / k.Hq, hq = blockIdx.x % k.Hq, G = k.Hq / k.Hkv;
  const int kv = hq / G, h = hq % G;
  const int64_t pair = (int64_t)b * k.Hkv + kv;
  const int64_t np = a.chunks * kAttnWaves;
  const float* base = a.part + pair * np * H * S + h * S;
  float mx = -INFINITY;
  for (int64_t w = 0; w < np; ++w) mx = fmaxf(mx, base[w * H * S]);
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.0f;
  for (int64_t w = 0; w < np; ++w) {
    const float* pw = base + w * H * S;
    const float mw = pw[0];
    if (mw == -INFINITY) continue;  // a wave that saw no token
    const float f = __expf(mw - mx);
    l = fmaf(f, pw[1], l);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(f, pw[4 + j * (D / 8) + c], v[j]);  // pi(8c + j)
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] *= inv;
  fwht_vector<LPV>(v, c);
  if (lane < LPV) {
    float* o = a.out + b * a.o_sb + hq * a.o_sh;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 8 * c + j;
      const bool neg = (a.tv.sign_words[i >> 5] >> (i & 31)) & 1u;
      o[i] = neg ? -v[j] : v[j];
    }
  }
}

int64_t attend_chunk(int64_t pairs, int64_t T) {
  const int64_t segs = (T + kScoreSegment - 1) / kScoreSegment;
  int64_t cpp = pairs > 0 ? 512 / pairs : 1;  // about two blocks per compute unit
  if (cpp > segs) cpp = segs;
  if (cpp < 1) cpp = 1;
  return ((segs + cpp - 1) / cpp) * kScoreSegment;
}

int64_t attend_partial_floats(int64_t pairs, int64_t T, int D) {
  const int64_t chunk = attend_chunk(pairs, T);
  return pairs * ((T + chunk - 1) / chunk) * kAttnWaves * kScoreHeads * (D + 4);
}

template <int D, int M, int BK, bool PCA, int BV>
static hipError_t launch_attend_t(AttendArgs a, hipStream_t st) {
  const int64_t pairs = (int64_t)a.k.B * a.k.Hkv;
  a.chunk = attend_chunk(pairs, a.k.T);
  a.chunks = (a.k.T + a.chunk - 1) / a.chunk;
  const int64_t blocks = pairs * a.chunks;
  if (blocks > 0x7FFFFFFF || (int64_t)a.k.B * a.k.Hq > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_attend<D, M, BK, PCA, BV>), dim3((unsigned)blocks), dim3(kScoreThreads), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_attend_combine<D>), dim3((unsigned)(a.k.B * a.k.Hq)), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D, int M, bool PCA>
static hipError_t launch_attend_dm(int bk, int bv, const AttendArgs& a, hipStream_t st) {
#define KVQ_BV(K)                                                  \
  switch (bv) {                                                    \
    case 1: return launch_attend_t<D, M, K, PCA, 1>(a, st);        \
    case 2: return launch_attend_t<D, M, K, PCA, 2>(a, st);        \
    case 3: return launch_attend_t<D, M, K, PCA, 3>(a, st);        \
  }                                                                \
  return hipErrorInvalidValue;
  switch (bk) {
    case 1: KVQ_BV(1)
    case 2: KVQ_BV(2)
    case 3: KVQ_BV(3)
    case 4: KVQ_BV(4)
  }
#undef KVQ_BV
  return hipErrorInvalidValue;
}

// K: Hadamard (mk = D) or a projection to mk in {32, 64} or mk = D.
bool attend_supported(int D, int mk, bool proj, int bk, int bv) {
  if (bk < 1 || bk > 4 || bv < 1 || bv > 3) return false;
  if (D != 64 && D != 128) return false;
  if (!proj) return mk == D;
  return mk == 32 || mk == 64 || mk == D;
}

hipError_t launch_attend(int D, int mk, bool proj, int bk, int bv, const AttendArgs& a, hipStream_t st) {
  if (a.k.T <= 0 || a.k.B <= 0 || a.k.Hq <= 0) return hipSuccess;
  if (!attend_supported(D, mk, proj, bk, bv)) return hipErrorInvalidValue;
  if (D == 64) {
    if (!proj) return launch_attend_dm<64, 64, false>(bk, bv, a, st);
    if (mk == 64) return launch_attend_dm<64, 64, true>(bk, bv, a, st);
    return launch_attend_dm<64, 32, true>(bk, bv, a, st);
  }
  if (!proj) return launch_attend_dm<128, 128, false>(bk, bv, a, st);
  if (mk == 128) return launch_attend_dm<128, 128, true>(bk, bv, a, st);
  if (mk == 64) return launch_attend_dm<128, 64, true>(bk, bv, a, st);
  return launch_attend_dm<128, 32, true>(bk, bv, a, st);
}

// Compute units of the current device (queried once per device).
static int device_cus() {
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

// Launch: one round of resident blocks. Each (batch, KV head) pair gets as many blocks as the
// chip holds blocks per pair; block j of a pair takes the pair's 256-token segments j, j + cpp,
// ..., so every block pays the query preparation once, and the blocks of a pair read its records
// side by side (a narrow window of addresses at any moment streams faster on this chip than as
// many separate contiguous runs).
template <int D, int M, int BITS, bool PCA>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t st) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_score<D, M, BITS, PCA>, kScoreThreads, 0) !=
            hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  const int64_t pairs = (int64_t)a.B * a.Hkv;
  const int64_t segs = (a.T + kScoreSegment - 1) / kScoreSegment;
  int64_t cpp = ((int64_t)per_cu * device_cus()) / pairs;
  if (cpp > segs) cpp = segs;
  if (cpp < 1) cpp = 1;
  const int64_t chunks = cpp;
  const int64_t blocks = chunks * pairs;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_score<D, M, BITS, PCA>), dim3((unsigned)blocks), dim3(kScoreThreads), 0, st,
                     a, chunks);
  return hipGetLastError();
}

template <int D, int M, bool PCA>
static hipError_t launch_score_dm(int bits, const ScoreArgs& a, hipStream_t st) {
  switch (bits) {
    case 1: return launch_score_t<D, M, 1, PCA>(a, st);
    case 2: return launch_score_t<D, M, 2, PCA>(a, st);
    case 3: return launch_score_t<D, M, 3, PCA>(a, st);
    case 4: return launch_score_t<D, M, 4, PCA>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score(int D, int m, bool proj, int bits, int group, const ScoreArgs& a, hipStream_t st) {
  if (a.T <= 0 || a.B <= 0 || a.Hkv <= 0) return hipSuccess;
  if (group < 1 || group > 8) return hipErrorInvalidValue;
  if (!proj) {
    if (D != m) return hipErrorInvalidValue;
    switch (m) {
      case 64: return launch_score_dm<64, 64, false>(bits, a, st);
      case 128: return launch_score_dm<128, 128, false>(bits, a, st);
      case 256: return launch_score_dm<256, 256, false>(bits, a, st);
      case 512: return launch_score_dm<512, 512, false>(bits, a, st);
    }
    return hipErrorInvalidValue;
  }
#define KVQ_CASE(d, r) \
  if (D == d && m == r) return launch_score_dm<d, r, true>(bits, a, st);
  KVQ_CASE(64, 32) KVQ_CASE(64, 64) KVQ_CASE(128, 32) KVQ_CASE(128, 64) KVQ_CASE(128, 128)
  KVQ_CASE(256, 32) KVQ_CASE(256, 64) KVQ_CASE(256, 128) KVQ_CASE(512, 32) KVQ_CASE(512, 64)
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
