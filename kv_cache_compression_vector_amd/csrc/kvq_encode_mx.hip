// kvq_encode_mx.hip — Hadamard-path encode with the rotation on the matrix cores (m <= 128).
//
// u = H_m (s (.) x) [kakeyaturbo PR #15, "M4 Phase A": rotate = H.D.x; "M4 Phase B": the rotation
// as a dense product on the tensor cores] is formed on v_mfma_f32_16x16x32_bf16 from +-1 operands
// (exact in bf16; x is bf16, so every product is exact and sums in f32). The in-register
// butterfly would cost log2(m) adds per coordinate on the vector ALUs, which bind first on this
// chip; the product costs them nothing.
//
// m = 128 (k_encode_t128): the transposed product U^T = Bm^T X^T, arranged so that each lane ends
// with one whole record word group of one vector (no cross-lane packing), and the rotation held
// as 16 register fragments (see below). m = 64 (k_encode_mx): U = X Bm with the output columns
// permuted so each lane holds NT consecutive plane positions of each of its rows; the quantiser
// builds NT-bit fields per plane and LPW = 32/NT lanes OR them into a record word over DPP.
//
// Rows arrive through swizzled LDS with 1 KB-contiguous loads, the next tile's loads in flight
// while the current one computes. Norms come from bf16 dot products of the staged rows.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_lanevec.h"
#include "kvq_mfma.h"

namespace kvq {

template <int M>
struct MX {
  static constexpr int NT = M / 16;    // n-tiles = coordinates per lane per row
  static constexpr int KS = M / 32;    // k-steps
  static constexpr int LPW = 32 / NT;  // lanes per record word
  static constexpr int ROWS = 16;      // rows per wave tile
  static constexpr int RT = ROWS / 16; // MFMA row tiles per wave tile
  static constexpr int RCH = M / 8;    // staged row, 16-byte chunks
  static constexpr int WAVES = 8;     // waves per block, sharing the staged rotation
  static constexpr int LDS = M * M * 2 + WAVES * ROWS * RCH * 16;
};

// B fragment (ks, nt) of lane l: k = 32 ks + 8 (l / 16) + e, column j = pi^-1(NT (l % 16) + nt);
// entry e = s_k (-1)^popcount(k & j) as bf16.
template <int M>
__device__ __forceinline__ uint4 rotation_fragment(const Tables& tab, int ks, int nt, int l) {
  constexpr int NT = MX<M>::NT;
  const int j = coord_at(NT * (l & 15) + nt, M);
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = 32 * ks + 8 * (l >> 4) + 2 * h + q;
      const uint32_t s = (tab.sign_pairs[k >> 1] >> (16 * (k & 1))) & 0x8000u;  // s_k = -1
      const uint32_t par = (uint32_t)(__builtin_popcount(k & j) & 1) << 15;
      v |= (0x3F80u | (s ^ par)) << (16 * q);
    }
    w[h] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int M, int BITS, bool SYM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void k_encode_mx(EncodeArgs a, int64_t tiles_per_block) {
  using X = MX<M>;
  constexpr int NT = X::NT, KS = X::KS, LPW = X::LPW, RT = X::RT, RCH = X::RCH;
  constexpr int ROWS = X::ROWS, NWC = (M / 32) * BITS, NWT = NWC + 1;
  constexpr int TILE = X::WAVES * ROWS;
  __shared__ uint4 sB[KS * NT * 64];
  __shared__ uint4 s_reg[X::WAVES * ROWS * RCH];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int f = tid; f < KS * NT * 64; f += 64 * X::WAVES)
    sB[f] = rotation_fragment<M>(a.tab, f / (NT * 64), (f / 64) % NT, f % 64);
  __syncthreads();
  uint4* reg = s_reg + wave * ROWS * RCH;
  const int64_t n_tiles = (a.n + TILE - 1) / TILE;
  const int64_t t0 = blockIdx.x * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < n_tiles ? t0 + tiles_per_block : n_tiles;
  constexpr int PER = ROWS * RCH / 64;  // 16-byte input pieces per lane and tile
  // rows of a tile, 1 KB-contiguous per instruction (rows past the end repeat the last row)
  auto load_tile = [&](int64_t tile, uint4 (&in)[PER]) {
    const int64_t rw = tile * TILE + ROWS * wave;
    const int l = opaque_lane();
    // piece k of lane l is chunk l % RCH of row rw + (64 / RCH) k + l / RCH: a uniform row base
    // plus the lane's offset, and the last row's chunk for rows past the end
    const uint16_t* xp = a.x + (rw + l / RCH) * a.ld + 8 * (l % RCH);
    const uint16_t* xlast = a.x + (a.n - 1) * a.ld + 8 * (l % RCH);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const bool inr = rw + (64 / RCH) * k + l / RCH < a.n;
      in[k] = ld_stream(inr ? xp + (64 / RCH) * k * a.ld : xlast);
    }
  };
  uint4 nxt[PER];
  if (t0 < t1) load_tile(t0, nxt);
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int64_t rw0 = tile * TILE + ROWS * wave;
    const int ln = opaque_lane();
    const int c = ln & 15, grp = ln >> 4;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int id = k * 64 + ln, p = id / RCH, ch = id % RCH;
      reg[swz<RCH>(p, ch)] = nxt[k];
    }
    if (tile + 1 < t1) load_tile(tile + 1, nxt);  // in flight while this tile computes
    __builtin_amdgcn_wave_barrier();
    uint4 A[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) A[rt][ks] = reg[swz<RCH>(16 * rt + c, 4 * ks + grp)];
    __builtin_amdgcn_wave_barrier();
    // norms: row 16 rt + c from this lane's chunks, summed over the 4 lane groups, then moved to
    // the accumulator layout (rows 16 rt + 4 grp + i)
    float nC[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float ss = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t w[4] = {A[rt][ks].x, A[rt][ks].y, A[rt][ks].z, A[rt][ks].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]),
                                               __builtin_bit_cast(bf16x2_t, w[e]), ss, false);
      }
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      float nr = sqrtf(ss);
      const bool bad = ss_out_of_range(ss);
      if (wave_any(bad)) {  // rescaled sum of squares (kvq_device.h), wave-uniform
        uint32_t mb = 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t m = chunk_max_mag_bits(A[rt][ks]);
          mb = mb > m ? mb : m;
        }
        uint32_t o = (uint32_t)__shfl_xor((int)mb, 16, 64);
        mb = mb > o ? mb : o;
        o = (uint32_t)__shfl_xor((int)mb, 32, 64);
        mb = mb > o ? mb : o;
        const int ex = max_exp_of_bits(mb);
        const float sc = pow2f(-ex);
        float s2 = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s2 = chunk_scaled_ss(A[rt][ks], sc, s2);
        s2 += __shfl_xor(s2, 16, 64);
        s2 += __shfl_xor(s2, 32, 64);
        nr = bad ? sqrtf(s2) * pow2f(ex) : nr;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) nC[rt][i] = __shfl(nr, 4 * grp + i, 64);
    }
    // rotation
    floatx4 acc[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 bfrag = sB[(ks * NT + nt) * 64 + ln];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = mfma_bf16(A[rt][ks], bfrag, acc[rt][nt]);
      }
    // quantise this lane's NT plane positions per row, join LPW lanes per word, and collect
    // the tile's records in the (now free) LDS region
    const int e = c % LPW, g = c / LPW;
    uint32_t* rec_lds = reinterpret_cast<uint32_t*>(reg);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * grp + i;
        const float n = nC[rt][i];
        const Quant<BITS, SYM> q(a.tab, n);
        QuantAcc<BITS, SYM> qa;
#pragma unroll
        for (int nt = NT - 1; nt >= 0; --nt) qa.push(acc[rt][nt][i], q);
        uint32_t pl[BITS];
        qa.planes(q, (1u << NT) - 1u, pl);
        uint32_t mine = 0;
#pragma unroll
        for (int p = 0; p < BITS; ++p) {
          const uint32_t wd = group_or<LPW>(pl[p] << (NT * e));
          mine = (e == p) ? wd : mine;
        }
        if (e < BITS) rec_lds[r * NWT + g * BITS + e] = mine;
        if (c == 0) rec_lds[r * NWT + NWC] = __float_as_uint(n);
      }
    __builtin_amdgcn_wave_barrier();
    // the tile's records are contiguous (and 16-byte aligned) in memory: coalesced stores
    {
      constexpr int CH = ROWS * NWT / 4;  // 16-byte pieces
      const int64_t valid_rows = a.n - rw0 < ROWS ? a.n - rw0 : ROWS;
      const int64_t valid_ch = (valid_rows * NWT) / 4;  // whole pieces of valid records
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint32_t*>(a.rec) + rw0 * NWT);
      const uint4* src = reinterpret_cast<const uint4*>(rec_lds);
#pragma unroll
      for (int k = 0; k < (CH + 63) / 64; ++k) {
        const int id = k * 64 + ln;
        if (id < CH && id < valid_ch) st_stream(dst + id, src[id]);
      }
      // a partial last piece (only when the tile ends inside it): its words one by one
      const int64_t tail_w = valid_rows * NWT - valid_ch * 4;
      if (ln < tail_w)
        reinterpret_cast<uint32_t*>(a.rec)[(rw0 * NWT) + valid_ch * 4 + ln] = rec_lds[valid_ch * 4 + ln];
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---- m = 128: the transposed product --------------------------------------------------------
// U^T = Bm^T X^T with A = Bm^T (16 output coordinates x 32 inputs) and B = X^T (32 inputs x 16
// vectors): the accumulator of lane l = 16 grp + c holds vector c, rows m = 4 grp + i of the
// m-tile. Row m of m-tile mt is assigned plane position P = 32 grp + 4 mt + i, so lane (grp, c)
// ends with exactly the 32 plane positions of record word group grp of vector c: its b plane
// words need no other lane, and its norm is the one its own group already summed.
//
// Structure of the operand. With j = coord_at(P) = 32 (mt % 4) + 8 i + 2 grp + (mt >> 2) and an
// input index k = 32 ks + kappa (kappa < 32), popcount(k & j) splits into popcount(ks & (mt % 4))
// and popcount(kappa & (8 i + 2 grp + (mt >> 2))): the fragment (mt, ks) of Bm^T is
// (-1)^popcount(ks & (mt % 4)) F(mt >> 2, ks), with F holding s_k and the second factor. The whole
// 128 x 128 rotation is the 8 fragments F and their negations, kept in registers.

// F(h, ks) for lane l: row m = l % 16, inputs k = 32 ks + kappa, kappa = 8 (l / 16) + e.
__device__ __forceinline__ uint4 t128_fragment(const Tables& tab, int h, int ks, int l) {
  const int m = l & 15, jl = 8 * (m & 3) + 2 * (m >> 2) + h;
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int kappa = 8 * (l >> 4) + 2 * hh + q, k = 32 * ks + kappa;
      const uint32_t s = (tab.sign_pairs[k >> 1] >> (16 * (k & 1))) & 0x8000u;  // s_k = -1
      const uint32_t par = (uint32_t)(__builtin_popcount(kappa & jl) & 1) << 15;
      v |= (0x3F80u | (s ^ par)) << (16 * q);
    }
    w[hh] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

constexpr int kT128Waves = 4;   // waves per block
constexpr int kT128Rows = 16;   // vectors per wave tile

// Block b takes the block tiles b, b + G, b + 2G, ... (G = the grid): at any moment the resident
// blocks stream through one window of the rows.
//
// Outlier side lists [kakeyaturbo PR #15, calibrated Lloyd-Max + outlier commit] take two passes
// of this kernel around the scan of the counts (kvq_encode.hip): OL = 1 writes the records and
// each vector's count of coordinates with |z| > T into offsets[v]; OL = 2 (after the scan) writes
// only the entries. A lane holds the coordinates j = 8 J + 2 grp + h (J < 16, h < 2) of its
// vector, the outlier bit of j at bit 2 J + h of its mask: with the four groups' masks, the rank
// of an entry among the vector's outliers in ascending coordinate order is the number of set
// bits of lower coordinates, counted group by group. Both passes decide |u / n| > T with the
// same instructions, so their counts agree.
// Read once: the first pass also stages each 16-vector wave tile's entries, in CSR order, in the
// workspace (the tile-local offset of a vector is the prefix of its tile's counts), when the
// tile has at most kOutlierStage of them, and flags the tile. After the scan k_outlier_copy
// moves a staged tile's entries to [offsets[first vector], + count) without touching its rows,
// and the second pass visits only the tiles over the budget (found 64 flags at a time).
// RULE: the record stores the codec's scale rule (from zu = sum u z^, zz = sum z^^2 over the
// chosen centroids, summed over the vector's four lane groups) instead of the norm.
template <int BITS, bool SYM, int OL = 0, bool RULE = false>
__global__ __launch_bounds__(64 * kT128Waves) __attribute__((amdgpu_waves_per_eu(RULE ? 2 : 3)))
void k_encode_t128(EncodeArgs a) {
  constexpr int M = 128, KS = 4, RCH = M / 8, ROWS = kT128Rows;
  constexpr int NWC = (M / 32) * BITS, NWT = NWC + 1, TILE = kT128Waves * ROWS;
  __shared__ uint4 s_reg[kT128Waves * ROWS * RCH];
  __shared__ float s_z[OL != 0 ? kT128Waves * 32 * 64 : 1];  // outlier passes: z[t] of each lane
  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int c = ln & 15, grp = ln >> 4;
  uint4 F[2][KS], FN[2][KS];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      F[h][ks] = t128_fragment(a.tab, h, ks, ln);
      FN[h][ks] = make_uint4(F[h][ks].x ^ 0x80008000u, F[h][ks].y ^ 0x80008000u,
                             F[h][ks].z ^ 0x80008000u, F[h][ks].w ^ 0x80008000u);
    }
  uint4* reg = s_reg + wave * ROWS * RCH;
  uint32_t* rec_lds = reinterpret_cast<uint32_t*>(reg);
  // LDS places (uint4) of the 4 staged pieces (row 4 k + grp, chunk c) and of the 4 operand
  // chunks (row c, chunk 4 ks + grp): swizzled so 16 lanes of one row or one chunk column hit
  // distinct banks
  int woff[4], roff[KS];
#pragma unroll
  for (int k = 0; k < 4; ++k) woff[k] = swz<RCH>(4 * k + grp, c);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = swz<RCH>(c, 4 * ks + grp);
  const int64_t n_tiles = (a.n + TILE - 1) / TILE;
  const int64_t G = gridDim.x;
  const int64_t lane_off = (int64_t)grp * a.ld + 8 * c;
  // piece k of the lane: row rw + 4 k + grp, chunk c (1 KB contiguous per instruction); rows past
  // the end repeat the last row
  auto load_tile = [&](int64_t tile, uint4 (&in)[4]) {
    const int64_t rw = tile * TILE + ROWS * wave;
    if (rw + ROWS <= a.n) {  // wave-uniform
      const uint16_t* xp = a.x + rw * a.ld + lane_off;
#pragma unroll
      for (int k = 0; k < 4; ++k) in[k] = ld_stream(xp + 4 * k * a.ld);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int64_t row = rw + 4 * k + grp;
        row = row < a.n ? row : a.n - 1;
        in[k] = ld_stream(a.x + row * a.ld + 8 * c);
      }
    }
  };
  // the block tiles this wave computes: b, b + G, ...; in the entry pass only those whose wave
  // tile was not staged, from ballots over the flags of 64 block tiles at a time
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int64_t fl_base = (int64_t)blockIdx.x - 64 * G;  // block tile of mask bit 0
  uint64_t fl_mask = 0;
  auto next_tile = [&](int64_t tile) -> int64_t {
    if constexpr (OL != 2) {
      return tile + G;
    } else {
      while (fl_mask == 0) {
        fl_base += 64 * G;
        if (fl_base >= n_tiles) return n_tiles;
        const int64_t tl = fl_base + (int64_t)ln * G;
        const int64_t r = tl * TILE + ROWS * wave_u;
        fl_mask = __ballot(tl < n_tiles && r < a.n && a.stg_flag[r / ROWS] != 0u);
      }
      const int j = __builtin_ctzll(fl_mask);
      fl_mask &= fl_mask - 1;
      return fl_base + (int64_t)j * G;
    }
  };
  // lane (grp, c)'s entries of the vector whose CSR entries start at base, clipped to [., end),
  // from its outlier mask olm and its LDS column of z values
  auto emit = [&](uint32_t olm, const float* zc, uint8_t* idx, uint16_t* val, int64_t base, int64_t end) {
    uint32_t mg[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) mg[g] = (uint32_t)__shfl((int)olm, c + 16 * g, 64);
    for (uint32_t rem = olm; rem != 0u; rem &= rem - 1u) {
      const int t = __builtin_ctz(rem), J = t >> 1;
      // set bits of coordinates below 8 J (lo) and below 8 J + 8 (lo_pair; all ones at J = 15)
      const uint32_t lo = (1u << (2 * J)) - 1u, lo_pair = (4u << (2 * J)) - 1u;
      uint32_t rank = __builtin_popcount(olm & ((1u << t) - 1u));
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g != grp) rank += __builtin_popcount(mg[g] & (g < grp ? lo_pair : lo));
      const int64_t pos = base + rank;
      if (pos < end) {
        idx[pos] = (uint8_t)(8 * J + 2 * grp + (t & 1));
        val[pos] = (uint16_t)f32_to_bf16_rne(zc[64 * t]);
      }
    }
  };
  const int64_t first = OL == 2 ? next_tile(0) : (int64_t)blockIdx.x;
  uint4 nxt[4];
  if (first < n_tiles) load_tile(first, nxt);
  for (int64_t tile = first, tn; tile < n_tiles; tile = tn) {
    const int64_t rw0 = tile * TILE + ROWS * wave;
#pragma unroll
    for (int k = 0; k < 4; ++k) reg[woff[k]] = nxt[k];
    tn = next_tile(tile);
    if (tn < n_tiles) load_tile(tn, nxt);  // in flight while this tile computes
    __builtin_amdgcn_wave_barrier();
    uint4 X[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) X[ks] = reg[roff[ks]];
    __builtin_amdgcn_wave_barrier();
    // norm of vector c: this lane's 32 coordinates, summed over the 4 groups
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t w[4] = {X[ks].x, X[ks].y, X[ks].z, X[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]),
                                             __builtin_bit_cast(bf16x2_t, w[e]), ss, false);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    float n = __builtin_amdgcn_sqrtf(ss);
    const bool bad = ss_out_of_range(ss);
    if (wave_any(bad)) {  // rescaled sum of squares (kvq_device.h), wave-uniform
      uint32_t mb = 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t m = chunk_max_mag_bits(X[ks]);
        mb = mb > m ? mb : m;
      }
      uint32_t o = (uint32_t)__shfl_xor((int)mb, 16, 64);
      mb = mb > o ? mb : o;
      o = (uint32_t)__shfl_xor((int)mb, 32, 64);
      mb = mb > o ? mb : o;
      const int ex = max_exp_of_bits(mb);
      const float sc = pow2f(-ex);
      float s2 = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s2 = chunk_scaled_ss(X[ks], sc, s2);
      s2 += __shfl_xor(s2, 16, 64);
      s2 += __shfl_xor(s2, 32, 64);
      n = bad ? __builtin_amdgcn_sqrtf(s2) * pow2f(ex) : n;
    }
    // rotation and quantiser, one m-tile at a time: plane bits t = 4 mt + i, pushed from t = 31
    auto mtile = [&](int mt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bool neg = __builtin_popcount(ks & (mt & 3)) & 1;  // compile-time
        acc = mfma_bf16(neg ? FN[mt >> 2][ks] : F[mt >> 2][ks], X[ks], acc);
      }
      return acc;
    };
    // row i of m-tile mt is coordinate 8 (4 (mt % 4) + i) + 2 grp + (mt >> 2): its mask bit
    auto ol_bit = [](int mt, int i) { return 2 * (4 * (mt & 3) + i) + (mt >> 2); };
    const float rn = n > 0.0f ? 1.0f / n : 0.0f;
    const int64_t vec = rw0 + c;
    if constexpr (OL == 2) {
      // the lane's z values go to its LDS column (z[t] at row t), the outlier bits to olm
      float* zc = s_z + wave * 32 * 64 + ln;
      uint32_t olm = 0;
#pragma unroll
      for (int mt = 7; mt >= 0; --mt) {
        const floatx4 acc = mtile(mt);
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          const float z = acc[i] * rn;
          zc[64 * ol_bit(mt, i)] = z;
          olm |= (fabsf(z) > a.tab.T ? 1u : 0u) << ol_bit(mt, i);
        }
      }
      if (vec >= a.n) olm = 0u;
      int64_t base = 0, end = 0;
      if (vec < a.n) {
        base = a.ol_off[vec];
        end = a.ol_off[vec + 1];
        if (end > a.ol_cap) end = a.ol_cap;
      }
      emit(olm, zc, static_cast<uint8_t*>(a.ol_idx), a.ol_val, base, end);
      __builtin_amdgcn_wave_barrier();
      continue;  // the records were written by the first pass
    }
    const Quant<BITS, SYM> q(a.tab, n);
    QuantAcc<BITS, SYM> qa;
    uint32_t olm = 0;
    float* zc1 = s_z + wave * 32 * 64 + ln;  // OL = 1: z of this lane's coordinates
    float zu = 0.0f, zz = 0.0f;              // RULE
#pragma unroll
    for (int mt = 7; mt >= 0; --mt) {
      const floatx4 acc = mtile(mt);
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        qa.push(acc[i], q);
        if constexpr (RULE) {
          const float zh = chosen_centroid<BITS, SYM>(acc[i], q, a.tab);
          zu = fmaf(acc[i], zh, zu);
          zz = fmaf(zh, zh, zz);
        }
        if constexpr (OL == 1) {
          const float z = acc[i] * rn;
          const bool o = fabsf(z) > a.tab.T;
          olm |= (o ? 1u : 0u) << ol_bit(mt, i);
          // every z, not only the outliers': a branch per coordinate would cost exec-mask
          // switching and split the rotation products the compiler shares across m-tiles
          zc1[64 * ol_bit(mt, i)] = z;
        }
      }
    }
    if constexpr (OL == 1) {
      if (vec >= a.n) olm = 0u;
      const uint32_t own = __builtin_popcount(olm);
      uint32_t cnt = own;
      cnt += (uint32_t)__shfl_xor((int)cnt, 16, 64);
      cnt += (uint32_t)__shfl_xor((int)cnt, 32, 64);
      if (grp == 0 && vec < a.n) a.ol_off[vec] = cnt;
      // tile-local CSR offsets: prefix of the 16 vectors' counts (every group computes it)
      uint32_t incl = cnt;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, d, 16);
        if (c >= d) incl += y;
      }
      const uint32_t total = (uint32_t)__shfl((int)incl, 15, 16);
      if (rw0 < a.n) {  // wave-uniform
        const int64_t t16 = rw0 / ROWS;
        if (total <= (uint32_t)kOutlierStage)
          emit(olm, zc1, a.stg_idx + t16 * kOutlierStage, a.stg_val + t16 * kOutlierStage,
               incl - cnt, kOutlierStage);
        if (ln == 0) a.stg_flag[t16] = total <= (uint32_t)kOutlierStage ? 0u : 1u;
      }
    }
    uint32_t pl[BITS];
    qa.planes(q, 0xFFFFFFFFu, pl);
    float stored = n;
    if constexpr (RULE) {
      zu += __shfl_xor(zu, 16, 64);
      zu += __shfl_xor(zu, 32, 64);
      zz += __shfl_xor(zz, 16, 64);
      zz += __shfl_xor(zz, 32, 64);
      stored = n > 0.0f ? rule_scale(a.scale_rule, n, zu, zz, M) : 0.0f;
    }
    // the tile's records, staged in the (now free) region: lane (grp, c) writes words
    // grp * b .. grp * b + b - 1 of record c; group 0 writes the stored scale
#pragma unroll
    for (int p = 0; p < BITS; ++p) rec_lds[c * NWT + grp * BITS + p] = pl[p];
    if (grp == 0) rec_lds[c * NWT + NWC] = __float_as_uint(stored);
    __builtin_amdgcn_wave_barrier();
    // the wave tile's records are contiguous in memory: coalesced 16-byte stores
    {
      constexpr int CH = ROWS * NWT / 4;  // 16-byte pieces (ROWS * NWT is a multiple of 4)
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint32_t*>(a.rec) + rw0 * NWT);
      const uint4* src = reinterpret_cast<const uint4*>(rec_lds);
      if (rw0 + ROWS <= a.n) {  // wave-uniform
#pragma unroll
        for (int k = 0; k < (CH + 63) / 64; ++k) {
          const int id = k * 64 + ln;
          if (id < CH) st_stream(dst + id, src[id]);
        }
      } else if (rw0 < a.n) {
        const int valid_w = (int)(a.n - rw0) * NWT;  // words of whole valid records
#pragma unroll
        for (int k = 0; k < (CH + 63) / 64; ++k) {
          const int id = k * 64 + ln;
          if (4 * id + 4 <= valid_w) st_stream(dst + id, src[id]);
        }
        const int tw = valid_w % 4, w0 = valid_w - tw;  // a partial last piece, word by word
        if (ln < tw) reinterpret_cast<uint32_t*>(a.rec)[rw0 * NWT + w0 + ln] = rec_lds[w0 + ln];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int BITS, bool SYM, int OL = 0, bool RULE = false>
static hipError_t launch_t128(const EncodeArgs& a, hipStream_t st) {
  constexpr int TILE = kT128Waves * kT128Rows;
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_encode_t128<BITS, SYM, OL, RULE>, 64 * kT128Waves, 0) !=
            hipSuccess || nb <= 0)
      nb = 1;
    per_cu = nb;
  }
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t tiles = (a.n + TILE - 1) / TILE;
  const int64_t resident = (int64_t)per_cu * cus;
  const int64_t blocks = tiles < resident ? tiles : resident;
  hipLaunchKernelGGL((k_encode_t128<BITS, SYM, OL, RULE>), dim3((unsigned)blocks), dim3(64 * kT128Waves), 0,
                     st, a);
  return hipGetLastError();
}

// The two outlier passes of coded length 128 (OL = 1: records and counts; OL = 2: entries,
// which use neither the bit width nor the table's symmetry).
template <int OL>
hipError_t launch_t128_outlier_pass(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  if constexpr (OL == 2) {
    return launch_t128<1, true, 2>(a, st);
  } else {
    switch (bits * 2 + (sym ? 1 : 0)) {
      case 2: return launch_t128<1, false, OL>(a, st);
      case 3: return launch_t128<1, true, OL>(a, st);
      case 4: return launch_t128<2, false, OL>(a, st);
      case 5: return launch_t128<2, true, OL>(a, st);
      case 6: return launch_t128<3, false, OL>(a, st);
      case 7: return launch_t128<3, true, OL>(a, st);
      case 8: return launch_t128<4, false, OL>(a, st);
      case 9: return launch_t128<4, true, OL>(a, st);
    }
    return hipErrorInvalidValue;
  }
}
template hipError_t launch_t128_outlier_pass<1>(int, bool, const EncodeArgs&, hipStream_t);
template hipError_t launch_t128_outlier_pass<2>(int, bool, const EncodeArgs&, hipStream_t);

// Staged outlier entries into the CSR (after the scan): wave tile t of 16 vectors, when its
// flag is 0, copies its entries to [offsets[16 t], offsets[min(16 t + 16, n)]), clipped to the
// capacity. Each 16-lane group takes its own tile, so a wave has the flag, offset and entry
// loads of four tiles in flight.
__global__ __launch_bounds__(256) void k_outlier_copy(EncodeArgs a) {
  const int ln = threadIdx.x & 63, sub = ln & 15;
  const int64_t tiles = (a.n + kT128Rows - 1) / kT128Rows;
  for (int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (ln >> 4); t < tiles;
       t += (int64_t)gridDim.x * 16) {
    if (a.stg_flag[t] != 0u) continue;
    const int64_t r0 = t * kT128Rows, vend = r0 + kT128Rows < a.n ? r0 + kT128Rows : a.n;
    const int64_t base = a.ol_off[r0], total = (int64_t)a.ol_off[vend] - base;
    const uint8_t* si = a.stg_idx + t * kOutlierStage;
    const uint16_t* sv = a.stg_val + t * kOutlierStage;
    for (int64_t i = sub; i < total; i += 16)
      if (base + i < a.ol_cap) {
        static_cast<uint8_t*>(a.ol_idx)[base + i] = si[i];
        a.ol_val[base + i] = sv[i];
      }
  }
}

hipError_t launch_outlier_copy(const EncodeArgs& a, hipStream_t st) {
  const int64_t tiles = (a.n + kT128Rows - 1) / kT128Rows;
  int64_t blocks = (tiles + 15) / 16;  // 16 tiles per block
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(k_outlier_copy, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool RULE>
static hipError_t launch_t128_r(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_t128<1, false, 0, RULE>(a, st);
    case 3: return launch_t128<1, true, 0, RULE>(a, st);
    case 4: return launch_t128<2, false, 0, RULE>(a, st);
    case 5: return launch_t128<2, true, 0, RULE>(a, st);
    case 6: return launch_t128<3, false, 0, RULE>(a, st);
    case 7: return launch_t128<3, true, 0, RULE>(a, st);
    case 8: return launch_t128<4, false, 0, RULE>(a, st);
    case 9: return launch_t128<4, true, 0, RULE>(a, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_t128_b(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  return a.scale_rule != 0 ? launch_t128_r<true>(bits, sym, a, st) : launch_t128_r<false>(bits, sym, a, st);
}

template <int M, int BITS, bool SYM>
static hipError_t launch_mx_t(const EncodeArgs& a, hipStream_t st) {
  constexpr int TILE = MX<M>::WAVES * MX<M>::ROWS;
  const int64_t tiles = (a.n + TILE - 1) / TILE;
  const int64_t resident = 256 * (160 * 1024 / MX<M>::LDS);
  const int64_t per = (tiles + resident - 1) / resident;
  const int64_t blocks = (tiles + per - 1) / per;
  hipLaunchKernelGGL((k_encode_mx<M, BITS, SYM>), dim3((unsigned)blocks), dim3(64 * MX<M>::WAVES), 0,
                     st, a, per);
  return hipGetLastError();
}

template <int M>
static hipError_t launch_mx_m(int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  switch (bits * 2 + (sym ? 1 : 0)) {
    case 2: return launch_mx_t<M, 1, false>(a, st);
    case 3: return launch_mx_t<M, 1, true>(a, st);
    case 4: return launch_mx_t<M, 2, false>(a, st);
    case 5: return launch_mx_t<M, 2, true>(a, st);
    case 6: return launch_mx_t<M, 3, false>(a, st);
    case 7: return launch_mx_t<M, 3, true>(a, st);
    case 8: return launch_mx_t<M, 4, false>(a, st);
    case 9: return launch_mx_t<M, 4, true>(a, st);
  }
  return hipErrorInvalidValue;
}

bool encode_mx_supported(int m, int scale_rule) { return m == 128 || (m == 64 && scale_rule == 0); }

hipError_t launch_encode_mx(int m, int bits, bool sym, const EncodeArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (m == 64) return launch_mx_m<64>(bits, sym, a, st);
  if (m == 128) return launch_t128_b(bits, sym, a, st);
  return hipErrorInvalidValue;
}

}  // namespace kvq
