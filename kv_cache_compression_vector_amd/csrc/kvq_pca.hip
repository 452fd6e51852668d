// kvq_pca.hip — projection (PCA) codec: v = B^T (x - mu) on MFMA, then the Hadamard codec
// over the r projected coordinates; decode x^ = mu + B v^ on MFMA.
//
// The projection follows the pages' per-token pipeline project -> rotate -> scale ->
// Lloyd-Max [kakeyaturbo PR #15, commits "M4 Phase A" ((X - mu) @ basis^T) and "M5" (unproject
// on the matrix engine)]. It is a genuine dense contraction, so it runs on
// v_mfma_f32_16x16x32_bf16: x and B are bf16, every product is exact and sums in f32; B^T mu
// enters as the accumulator's initial value. The decode multiplies B by v^ split into two bf16
// halves (hi + lo), keeping ~2^-17 relative precision, with mu as the initial value.
//
// A block of W waves (4, or 2 for the largest bases) takes 64 W consecutive rows, all under one
// basis (basis blocks are multiples of 256 rows). Each wave owns 64 rows and one LDS region
// that holds, in turn, its swizzled input chunk, the MFMA output and the staged output rows,
// so global traffic moves in 256-byte row segments, 1 KB per instruction. After the
// projection each lane owns one vector (r <= 128 coordinates in registers) for the rotation
// and quantiser of kvq_lanevec.h. LDS at (D, r) = (128, 64): basis 16 KB + 4 x 16 KB, so two
// blocks share a CU.
//
// MFMA 16x16x32 operand layout (lane l): A[row l%16][k 8(l/16)..+7], B[k 8(l/16)..+7][col l%16],
// result D[row 4(l/16)+i][col l%16], i = 0..3.
#include "kvq_device.h"
#include "kvq_kernels.h"
#include "kvq_lanevec.h"
#include "kvq_mfma.h"

namespace kvq {


// Per-shape constants. Input (encode) and output (decode) rows move through LDS in column
// chunks of 256 bytes: 128 bf16 (or 64 f32) columns, the whole row when it is shorter.
template <int D, int R>
struct PcaShape {
  static constexpr int DC = D < 128 ? D : 128;            // bf16 columns per staged chunk
  static constexpr int CCH = DC / 8;                      // 16-byte chunks per staged row
  static constexpr int RCH = CCH > R / 4 ? CCH : R / 4;   // region row stride (f32 y, hi|lo v^)
  static constexpr int BASIS_BYTES = D * R * 2;
  static constexpr int REGION_BYTES = 64 * RCH * 16;
  static constexpr int W = BASIS_BYTES + 4 * REGION_BYTES <= 128 * 1024 ? 4 : 2;  // waves
  static constexpr int ROWS = 64 * W;                     // rows per block tile
};

// Mean used when a codec gives none (read only).
__device__ const float kZeroMean[512] = {};


// ------------------------------------------------------------------------------------------
// Encode. The random signs are folded into the staged basis (column j of B times s_j, exact
// in bf16), so the MFMA yields s (.) B^T x directly. The product is formed transposed,
// (B^T)(x^T), so that lane l receives 4 consecutive projected coordinates of one row.
template <int D, int R, int BITS, bool SYM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_encode_pca(EncodeArgs a, int64_t tiles_per_block) {
  using P = PcaShape<D, R>;
  constexpr int W = P::W, DC = P::DC, CCH = P::CCH, RCH = P::RCH;
  constexpr int BCH = D / 8;   // B^T row (one basis column, D bf16) in chunks
  constexpr int NT = R / 16, NWT = (R / 32) * BITS + 1;
  __shared__ uint4 s_bT[R * BCH];
  __shared__ uint4 s_reg[W * 64 * RCH];
  const int tid = threadIdx.x, wave = tid >> 6;
  uint4* reg = s_reg + wave * 64 * RCH;
  float4 mp[NT];  // -(s (.) B^T mu) at this lane's output columns 16 t + 4 (l / 16) .. +3
  int cur = -1;
  const int64_t n_tiles = (a.n + P::ROWS - 1) / P::ROWS;
  const int64_t t0 = blockIdx.x * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < n_tiles ? t0 + tiles_per_block : n_tiles;
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int64_t row0 = tile * P::ROWS;
    const int bi = basis_of_row(a.pca, row0);  // block tiles never straddle basis blocks
    if (bi != cur) {
      __syncthreads();
      const uint16_t* Bk = a.pca.basis + (int64_t)bi * D * R;
      uint16_t* bt16 = reinterpret_cast<uint16_t*>(s_bT);
      for (int e = tid; e < D * R; e += 64 * W) {
        const int d = e / R, j = e % R;
        const uint32_t flip = (a.tab.sign_pairs[j >> 1] >> (16 * (j & 1))) & 0x8000u;
        bt16[swz<BCH>(j, d / 8) * 8 + d % 8] = (uint16_t)(Bk[e] ^ flip);
      }
      __syncthreads();
      // -(s (.) B^T mu) through the (idle) regions: one column per thread, then each lane
      // takes the 4 NT columns its accumulators start from
      if (tid < R) {
        float s = 0.0f;
        if (a.pca.mean) {
          const float* mu = a.pca.mean + (int64_t)bi * D;
          for (int c = 0; c < BCH; ++c) {
            const uint4 w = s_bT[swz<BCH>(tid, c)];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s = fmaf(bf16lo_to_f32(u[e]), mu[8 * c + 2 * e], s);
              s = fmaf(bf16hi_to_f32(u[e]), mu[8 * c + 2 * e + 1], s);
            }
          }
        }
        reinterpret_cast<float*>(s_reg)[tid] = -s;
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < NT; ++t) mp[t] = reinterpret_cast<const float4*>(s_reg)[4 * t + ((tid & 63) >> 4)];
      __syncthreads();
      cur = bi;
    }
    const int64_t rw0 = row0 + 64 * wave;
    const int ln = opaque_lane();
    floatx4 acc[4][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][t] = floatx4{mp[t].x, mp[t].y, mp[t].z, mp[t].w};
#pragma unroll
    for (int dc = 0; dc < D / DC; ++dc) {
      // coalesced, swizzled input chunk: 64 rows x DC bf16 (rows past the end repeat the last);
      // all loads are issued before the first LDS write: one memory round trip per chunk
      uint4 in[CCH];
#pragma unroll
      for (int k = 0; k < CCH; ++k) {
        const int id = k * 64 + ln, p = id / CCH, c = id % CCH;
        const int64_t row = rw0 + p < a.n ? rw0 + p : a.n - 1;
        in[k] = ld_stream(reinterpret_cast<const uint4*>(a.x + row * a.ld + dc * DC) + c);
      }
#pragma unroll
      for (int k = 0; k < CCH; ++k) {
        const int id = k * 64 + ln, p = id / CCH, c = id % CCH;
        reg[swz<RCH>(p, c)] = in[k];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int ks = 0; ks < DC / 32; ++ks) {
        const int ck = 4 * ks + (ln >> 4);
        uint4 xf[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) xf[rt] = reg[swz<RCH>(16 * rt + (ln & 15), ck)];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 bf = s_bT[swz<BCH>(16 * t + (ln & 15), dc * CCH + ck)];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[rt][t] = mfma_bf16(bf, xf[rt], acc[rt][t]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // projected rows (f32) into the region: acc[rt][t] = y[16 rt + l % 16][16 t + 4 (l / 16) ..+3]
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        reg[swz<RCH>(16 * rt + (ln & 15), 4 * t + (ln >> 4))] =
            make_uint4(__float_as_uint(acc[rt][t][0]), __float_as_uint(acc[rt][t][1]),
                       __float_as_uint(acc[rt][t][2]), __float_as_uint(acc[rt][t][3]));
    __builtin_amdgcn_wave_barrier();
    // one vector per lane: norm, rotation, quantiser
    const int64_t vec = rw0 + ln;
    float v[R];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < R / 4; ++c) {
      const uint4 f = reg[swz<RCH>(ln, c)];
      v[4 * c + 0] = __uint_as_float(f.x);
      v[4 * c + 1] = __uint_as_float(f.y);
      v[4 * c + 2] = __uint_as_float(f.z);
      v[4 * c + 3] = __uint_as_float(f.w);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(v[4 * c + e], v[4 * c + e], ss);
    }
    __builtin_amdgcn_wave_barrier();
    const float n = safe_norm_f32<R, 1>(ss, v);
    fwht_regs<R>(v);
    quantize_store_lv<R, BITS, SYM>(v, n, n, vec < a.n, 0, a.tab,
                                    reinterpret_cast<uint32_t*>(a.rec) + vec * NWT);
  }
}

// ------------------------------------------------------------------------------------------
// Encode at r = 64, D <= 128 with two lanes per vector. Registers, not LDS or bandwidth, set
// the occupancy of the kernel above (about 200 registers for a lane that owns 64 coordinates:
// 2 waves per SIMD, 8 per CU, too few loads in flight to stream HBM). Here a wave takes 32 rows
// and lane pair (2p, 2p+1) owns vector p: lane q holds the 32 coordinates whose index bit 2 is
// q, i = 8j + 4q + e (j < 8, e < 4), locally k = 4j + e. The rotation is the Sylvester
// transform over the five in-lane index bits plus one butterfly across the pair (index bit 2);
// the bit order of a Hadamard transform's stages is free. With this split the word group of
// the record's plane layout (g = pi(i) / 32 = bit 2 of i) is the lane: lane q quantises exactly
// the 32 coordinates of word group q, bit t of its words holding k = 4 (t mod 8) + t / 8.
// Rows are not staged: each lane loads its MFMA B operands (16 bytes of one row per k-step)
// straight from memory, with ordinary loads (a streaming hint that bypasses the caches costs
// 7 % here, since the 64-byte pieces of one 128-byte line arrive from two instructions), and
// the next tile's operands stay in flight while a tile computes. LDS holds the basis (16 KB)
// and 8 KB per wave for the projected rows and the records; a block of 4 waves takes 128 rows
// under one basis, and three blocks (12 waves, 140-155 registers each) share a CU.
constexpr int kPqWaves = 4;
constexpr int kPqRows = 32;                       // rows per wave tile
constexpr int kPqTile = kPqWaves * kPqRows;       // rows per block tile

template <int D, int BITS, bool SYM>
__global__ __launch_bounds__(64 * kPqWaves) __attribute__((amdgpu_waves_per_eu(3)))
void k_encode_pq(EncodeArgs a, int64_t tiles_per_block) {
  constexpr int R = 64, NT = R / 16, BCH = D / 8;
  constexpr int RCH = 16;                          // region row stride: 16 chunks (64 f32)
  constexpr int NWC = 2 * BITS, NWT = NWC + 1;
  constexpr int KS = D / 32;                       // k-steps of the projection
  __shared__ uint4 s_bT[R * BCH];
  __shared__ uint4 s_reg[kPqWaves * kPqRows * RCH];
  __shared__ float4 s_mp[R / 4];  // -(s (.) B^T mu), the projection's initial value
  __shared__ float s_muf[D];
  const int tid = threadIdx.x, wave = tid >> 6;
  uint4* reg = s_reg + wave * kPqRows * RCH;
  int cur = -1;
  const int64_t n_tiles = (a.n + kPqTile - 1) / kPqTile;
  const int64_t t0 = blockIdx.x * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < n_tiles ? t0 + tiles_per_block : n_tiles;
  // The MFMA B operands straight from memory: lane l takes row 16 rt + l % 16, bytes
  // 64 ks + 16 (l / 16) .. +15 (rows past the end repeat the last); the next tile's are in flight
  // while a tile computes.
  auto load_x = [&](int64_t tile, uint4 (&dst)[2][KS]) {
    const int l = opaque_lane();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      int64_t row = tile * kPqTile + kPqRows * wave + 16 * rt + (l & 15);
      row = row < a.n ? row : a.n - 1;
      const uint4* src = reinterpret_cast<const uint4*>(a.x + row * a.ld) + (l >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[rt][ks] = src[4 * ks];
    }
  };
  uint4 nxt[2][KS];
  if (t0 < t1) load_x(t0, nxt);
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int64_t row0 = tile * kPqTile;
    const int bi = basis_of_row(a.pca, row0);  // block tiles never straddle basis blocks
    if (bi != cur) {
      __syncthreads();
      const uint16_t* Bk = a.pca.basis + (int64_t)bi * D * R;
      uint16_t* bt16 = reinterpret_cast<uint16_t*>(s_bT);
      for (int e = tid; e < D * R; e += 64 * kPqWaves) {
        const int d = e / R, j = e % R;
        const uint32_t flip = (a.tab.sign_pairs[j >> 1] >> (16 * (j & 1))) & 0x8000u;
        bt16[swz<BCH>(j, d / 8) * 8 + d % 8] = (uint16_t)(Bk[e] ^ flip);
      }
      const float* mu = a.pca.mean ? a.pca.mean + (int64_t)bi * D : nullptr;
      if (tid < D) s_muf[tid] = mu ? mu[tid] : 0.0f;
      __syncthreads();
      // -(s (.) B^T mu): TPC threads per column j, each over BCH / TPC chunks, then summed
      {
        constexpr int TPC = 64 * kPqWaves / R;
        static_assert(TPC * R == 64 * kPqWaves && BCH % TPC == 0 && TPC <= 8, "column split");
        const int j = tid / TPC, part = tid % TPC;
        float acc = 0.0f;
#pragma unroll
        for (int c2 = 0; c2 < BCH / TPC; ++c2) {
          const int c = part * (BCH / TPC) + c2;
          const uint4 w = s_bT[swz<BCH>(j, c)];
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = fmaf(bf16lo_to_f32(u[e]), s_muf[8 * c + 2 * e], acc);
            acc = fmaf(bf16hi_to_f32(u[e]), s_muf[8 * c + 2 * e + 1], acc);
          }
        }
#pragma unroll
        for (int o = 1; o < TPC; o <<= 1) acc += __shfl_xor(acc, o, 64);
        if (part == 0) reinterpret_cast<float*>(s_mp)[j] = -acc;
      }
      __syncthreads();
      cur = bi;
    }
    const int64_t rw0 = row0 + kPqRows * wave;
    const int ln = opaque_lane();
    uint4 xf[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) xf[rt][ks] = nxt[rt][ks];
    if (tile + 1 < t1) load_x(tile + 1, nxt);  // in flight while this tile computes
    // y^T = (s (.) B^T) x^T - s (.) B^T mu: acc[rt][t] = y[16 rt + l % 16][16 t + 4 (l / 16) ..+3]
    floatx4 acc[2][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4 m = s_mp[4 * t + (ln >> 4)];  // columns 16 t + 4 (l / 16) .. +3
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[rt][t] = floatx4{m.x, m.y, m.z, m.w};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ck = 4 * ks + (ln >> 4);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 bf = s_bT[swz<BCH>(16 * t + (ln & 15), ck)];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[rt][t] = mfma_bf16(bf, xf[rt][ks], acc[rt][t]);
      }
    }
    phase_fence();
    // projected rows (f32) into the region: chunk c of a row holds coordinates 4c .. 4c + 3
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        reg[swz<RCH>(16 * rt + (ln & 15), 4 * t + (ln >> 4))] =
            make_uint4(__float_as_uint(acc[rt][t][0]), __float_as_uint(acc[rt][t][1]),
                       __float_as_uint(acc[rt][t][2]), __float_as_uint(acc[rt][t][3]));
    __builtin_amdgcn_wave_barrier();
    // lane pair per vector: lane q takes chunks 2j + q (coordinates 8j + 4q + e)
    const int p = ln >> 1, q = ln & 1;
    float v[32];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 f = reg[swz<RCH>(p, 2 * j + q)];
      v[4 * j + 0] = __uint_as_float(f.x);
      v[4 * j + 1] = __uint_as_float(f.y);
      v[4 * j + 2] = __uint_as_float(f.z);
      v[4 * j + 3] = __uint_as_float(f.w);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(v[4 * j + e], v[4 * j + e], ss);
    }
    __builtin_amdgcn_wave_barrier();
    phase_fence();
    ss += quad_xor<1>(ss);
    const float n = safe_norm_f32<32, 2>(ss, v);
    fwht_regs<32>(v);          // index bits 0, 1, 3, 4, 5 (local bits 0 .. 4)
    fwht_cross<2, 32>(v, q);   // index bit 2, across the pair
    // quantise word group q: bit t of each plane word is local coordinate 4 (t mod 8) + t / 8
    uint32_t pl[BITS];
    {
      const Quant<BITS, SYM> qz(a.tab, n);
      QuantAcc<BITS, SYM> qa;
#pragma unroll
      for (int t = 31; t >= 0; --t) qa.push(v[4 * (t % 8) + t / 8], qz);
      qa.planes(qz, 0xFFFFFFFFu, pl);
    }
    // the tile's records through the (now free) region, then coalesced 16-byte stores
    uint32_t* rec_lds = reinterpret_cast<uint32_t*>(reg);
#pragma unroll
    for (int pp = 0; pp < BITS; ++pp) rec_lds[p * NWT + q * BITS + pp] = pl[pp];
    if (q == 0) rec_lds[p * NWT + NWC] = __float_as_uint(n);
    __builtin_amdgcn_wave_barrier();
    {
      constexpr int CH = kPqRows * NWT / 4;  // 16-byte pieces of the tile's records
      const int64_t valid_rows = a.n - rw0 < kPqRows ? (a.n - rw0 > 0 ? a.n - rw0 : 0) : kPqRows;
      const int64_t valid_ch = (valid_rows * NWT) / 4;
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint32_t*>(a.rec) + rw0 * NWT);
      const uint4* src = reinterpret_cast<const uint4*>(rec_lds);
#pragma unroll
      for (int k = 0; k < (CH + 63) / 64; ++k) {
        const int id = k * 64 + ln;
        if (id < CH && id < valid_ch) st_stream(dst + id, src[id]);
      }
      const int64_t tail_w = valid_rows * NWT - valid_ch * 4;  // words of a partial last piece
      if (ln < tail_w)
        reinterpret_cast<uint32_t*>(a.rec)[rw0 * NWT + valid_ch * 4 + ln] = rec_lds[valid_ch * 4 + ln];
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------------------------------
// Encode at r = 128 (D = 128, 256): the projection formed transposed, U^T = (s (.) B^T) x^T, as
// the Hadamard encode at m = 128 forms its rotation, so that each lane ends with one whole
// record word group of one vector. Row m of m-tile mt is projected coordinate
// j = 8 (4 (mt mod 4) + i) + 2 g + (mt >> 2) for m = 4 g + i; lane l = 16 g + v then holds the
// 32 coordinates of vector v whose index bits 1, 2 equal g, at plane positions 32 g + 4 mt + i.
// The Sylvester rotation over the projected coordinates is five butterfly stages in registers
// (index bits 0, 3..6: the bits of mt and i) and two across the lane groups (bits 1, 2: lanes
// l ^ 16, l ^ 32); then the quantiser packs the lane's words with no other lane. No f32 staging
// region: LDS holds the sign-folded basis (D r bf16), the mean term and each wave's records.
constexpr int kPtWaves = 4;
// 16-row MFMA column tiles per wave tile (two, sharing each basis read, measured no faster: the
// kernel is bound by vector-ALU issue, not by the basis reads from LDS)
constexpr int kPtRT = 1;

// Projected coordinate of row m of m-tile mt.
__host__ __device__ constexpr int pt_coord(int mt, int m) {
  return 8 * (4 * (mt & 3) + (m & 3)) + 2 * (m >> 2) + (mt >> 2);
}

// LDS place (uint4) of chunk c of basis column j: the XOR key (j >> 1) mod 16 gives the 16
// columns of one m-tile's A operand (index bits 1..4 varying) 16 distinct bank groups.
template <int BCH>
__device__ __forceinline__ int pt_swz(int j, int c) { return j * BCH + (c ^ ((j >> 1) & 15)); }

template <int D, int BITS, bool SYM>
__global__ __launch_bounds__(64 * kPtWaves) __attribute__((amdgpu_waves_per_eu(2)))
void k_encode_pt(EncodeArgs a, int64_t tiles_per_block) {
  constexpr int R = 128, BCH = D / 8, KS = D / 32, NMT = R / 16;
  constexpr int RT = kPtRT, ROWS = 16 * RT;
  constexpr int NWC = (R / 32) * BITS, NWT = NWC + 1, TILE = ROWS * kPtWaves;
  __shared__ uint4 s_bT[R * BCH];
  __shared__ float4 s_mp[NMT * 4];  // -(s (.) B^T mu) at (mt, g): coordinates pt_coord(mt, 4 g + i)
  __shared__ float s_mu[D];
  __shared__ uint32_t s_rec[kPtWaves][ROWS * NWT];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
  const int v = ln & 15, g = ln >> 4;
  uint32_t* rec_lds = s_rec[wave];
  int cur = -1;
  const int64_t n_tiles = (a.n + TILE - 1) / TILE;
  const int64_t t0 = blockIdx.x * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < n_tiles ? t0 + tiles_per_block : n_tiles;
  // B operands: row 16 wave + v of the tile, chunk 4 ks + g (rows past the end repeat the last)
  auto load_x = [&](int64_t tile, uint4 (&dst)[RT][KS]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      int64_t row = tile * TILE + ROWS * wave + 16 * rt + v;
      row = row < a.n ? row : a.n - 1;
      const uint4* src = reinterpret_cast<const uint4*>(a.x + row * a.ld) + g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[rt][ks] = src[4 * ks];
    }
  };
  uint4 nxt[RT][KS];
  if (t0 < t1) load_x(t0, nxt);
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int bi = basis_of_row(a.pca, tile * TILE);  // block tiles never straddle basis blocks
    if (bi != cur) {
      __syncthreads();
      const uint16_t* Bk = a.pca.basis + (int64_t)bi * D * R;
      uint16_t* bt16 = reinterpret_cast<uint16_t*>(s_bT);
      if ((reinterpret_cast<uintptr_t>(Bk) & 15) == 0) {  // 16-byte pieces: 8 columns of one row d
        for (int e8 = tid; e8 < D * R / 8; e8 += 64 * kPtWaves) {
          const int d = e8 / (R / 8), j0 = 8 * (e8 % (R / 8));
          const uint4 w = *reinterpret_cast<const uint4*>(Bk + (int64_t)d * R + j0);
          // the sign masks of columns j0 .. j0 + 7 are the pair words j0/2 .. j0/2 + 3 (bits 15, 31)
          const uint32_t f[4] = {w.x ^ a.tab.sign_pairs[j0 / 2], w.y ^ a.tab.sign_pairs[j0 / 2 + 1],
                                 w.z ^ a.tab.sign_pairs[j0 / 2 + 2], w.w ^ a.tab.sign_pairs[j0 / 2 + 3]};
#pragma unroll
          for (int t = 0; t < 8; ++t)
            bt16[pt_swz<BCH>(j0 + t, d / 8) * 8 + d % 8] = (uint16_t)(f[t >> 1] >> (16 * (t & 1)));
        }
      } else {
        for (int e = tid; e < D * R; e += 64 * kPtWaves) {
          const int d = e / R, j = e % R;
          const uint32_t flip = (a.tab.sign_pairs[j >> 1] >> (16 * (j & 1))) & 0x8000u;
          bt16[pt_swz<BCH>(j, d / 8) * 8 + d % 8] = (uint16_t)(Bk[e] ^ flip);
        }
      }
      const float* mu = a.pca.mean ? a.pca.mean + (int64_t)bi * D : nullptr;
      for (int d = tid; d < D; d += 64 * kPtWaves) s_mu[d] = mu ? mu[d] : 0.0f;
      __syncthreads();
      // -(s (.) B^T mu)_j: two threads per column, halves of the column summed
      {
        const int j = tid >> 1, part = tid & 1;
        float acc = 0.0f;
        for (int c = part * (BCH / 2); c < (part + 1) * (BCH / 2); ++c) {
          const uint4 w = s_bT[pt_swz<BCH>(j, c)];
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = fmaf(bf16lo_to_f32(u[e]), s_mu[8 * c + 2 * e], acc);
            acc = fmaf(bf16hi_to_f32(u[e]), s_mu[8 * c + 2 * e + 1], acc);
          }
        }
        acc += __shfl_xor(acc, 1, 64);
        // coordinate j sits at (mt, g, i) with j = pt_coord(mt, 4 g + i)
        const int mt = 4 * (j & 1) + (j >> 5), gg = (j >> 1) & 3, i = (j >> 3) & 3;
        if (part == 0) reinterpret_cast<float*>(s_mp)[(4 * mt + gg) * 4 + i] = -acc;
      }
      __syncthreads();
      cur = bi;
    }
    const int64_t rw0 = tile * TILE + ROWS * wave;
    uint4 X[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) X[rt][ks] = nxt[rt][ks];
    if (tile + 1 < t1) load_x(tile + 1, nxt);  // in flight while this tile computes
    // the projection: accs[rt][mt][i] = y_j, j = pt_coord(mt, 4 g + i), of vector 16 rt + v
    floatx4 accs[RT][NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const float4 m0 = s_mp[4 * mt + g];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) accs[rt][mt] = floatx4{m0.x, m0.y, m0.z, m0.w};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const uint4 A = s_bT[pt_swz<BCH>(pt_coord(mt, ln & 15), 4 * ks + (ln >> 4))];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) accs[rt][mt] = mfma_bf16(A, X[rt][ks], accs[rt][mt]);
      }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
    floatx4 (&acc)[NMT] = accs[rt];
    // norm of the projected vector: this lane's 32 coordinates, summed over the 4 groups
    float ss = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = fmaf(acc[mt][i], acc[mt][i], ss);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    float n = __builtin_amdgcn_sqrtf(ss);
    const bool bad = ss_out_of_range(ss);
    if (wave_any(bad)) {  // rescaled sum of squares (kvq_device.h), wave-uniform
      uint32_t mb = 0;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t m = __float_as_uint(acc[mt][i]) & 0x7FFFFFFFu;
          mb = mb > m ? mb : m;
        }
      uint32_t ot = (uint32_t)__shfl_xor((int)mb, 16, 64);
      mb = mb > ot ? mb : ot;
      ot = (uint32_t)__shfl_xor((int)mb, 32, 64);
      mb = mb > ot ? mb : ot;
      const int ex = max_exp_of_bits(mb);
      const float sc = pow2f(-ex);
      float s2 = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y = acc[mt][i] * sc;
          s2 = fmaf(y, y, s2);
        }
      s2 += __shfl_xor(s2, 16, 64);
      s2 += __shfl_xor(s2, 32, 64);
      n = bad ? __builtin_amdgcn_sqrtf(s2) * pow2f(ex) : n;
    }
    // rotation: in-lane stages over the bits of i and mt, then the two lane-group bits
#pragma unroll
    for (int h = 1; h < 4; h <<= 1)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((i & h) == 0) {
            const float x = acc[mt][i], y = acc[mt][i + h];
            acc[mt][i] = x + y;
            acc[mt][i + h] = x - y;
          }
#pragma unroll
    for (int h = 1; h < NMT; h <<= 1)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        if ((mt & h) == 0)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = acc[mt][i], y = acc[mt + h][i];
            acc[mt][i] = x + y;
            acc[mt + h][i] = x - y;
          }
#pragma unroll
    for (int gb = 1; gb < 4; gb <<= 1) {
      const float sg = (g & gb) ? -1.0f : 1.0f;  // the upper lane of the pair takes a - b
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = fmaf(acc[mt][i], sg, __shfl_xor(acc[mt][i], 16 * gb, 64));
    }
    // quantiser: plane bits t = 4 mt + i, pushed from t = 31 down
    uint32_t pl[BITS];
    {
      const Quant<BITS, SYM> q(a.tab, n);
      QuantAcc<BITS, SYM> qa;
#pragma unroll
      for (int mt = NMT - 1; mt >= 0; --mt)
#pragma unroll
        for (int i = 3; i >= 0; --i) qa.push(acc[mt][i], q);
      qa.planes(q, 0xFFFFFFFFu, pl);
    }
#pragma unroll
    for (int p = 0; p < BITS; ++p) rec_lds[(16 * rt + v) * NWT + g * BITS + p] = pl[p];
    if (g == 0) rec_lds[(16 * rt + v) * NWT + NWC] = __float_as_uint(n);
    }
    __builtin_amdgcn_wave_barrier();
    {
      constexpr int CH = ROWS * NWT / 4;  // 16-byte pieces of the wave tile's records
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

template <int D, int BITS, bool SYM>
static hipError_t enc_pt_t(const EncodeArgs& a, hipStream_t st) {
  constexpr int TILE = 16 * kPtRT * kPtWaves;
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_encode_pt<D, BITS, SYM>, 64 * kPtWaves, 0) !=
            hipSuccess || nb <= 0)
      nb = 1;
    return nb;
  }();
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t tiles = (a.n + TILE - 1) / TILE;
  const int64_t resident = (int64_t)per_cu * cus;
  const int64_t per = (tiles + resident - 1) / resident;
  hipLaunchKernelGGL((k_encode_pt<D, BITS, SYM>), dim3((unsigned)((tiles + per - 1) / per)),
                     dim3(64 * kPtWaves), 0, st, a, per);
  return hipGetLastError();
}

template <int D, int BITS, bool SYM>
static hipError_t enc_pq_t(const EncodeArgs& a, hipStream_t st) {
  const int64_t tiles = (a.n + kPqTile - 1) / kPqTile;
  const int64_t resident = 256 * 3;  // three blocks per CU (registers and LDS: 16 KB + 32 KB)
  const int64_t per = (tiles + resident - 1) / resident;
  hipLaunchKernelGGL((k_encode_pq<D, BITS, SYM>), dim3((unsigned)((tiles + per - 1) / per)),
                     dim3(64 * kPqWaves), 0, st, a, per);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Decode: out^T[d][row] = sum_j B[d][j] v^[row][j] + mu[d]. The A operand is B as stored (row d,
// k = j contiguous) with the signs folded into its columns, the B operand the rows of
// scale * H z^, so lane l receives 4 consecutive d of one row.
template <int D, int R, int BITS, bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_decode_pca(DecodeArgs a, int64_t tiles_per_block) {
  using P = PcaShape<D, R>;
  constexpr int W = P::W, CCH = P::CCH, RCH = P::RCH;
  constexpr int HCH = R / 8;                      // basis row (R bf16) in chunks = v^ half row
  constexpr int OCOLS = BF16 ? P::DC : P::DC / 2; // output columns per staged chunk (256 B)
  constexpr int ES = BF16 ? 2 : 4;                // output element bytes
  constexpr int KS = R / 32, NWC = (R / 32) * BITS, NWT = NWC + 1;
  __shared__ uint4 s_B[D * HCH];
  __shared__ uint4 s_reg[W * 64 * RCH];
  const int tid = threadIdx.x, wave = tid >> 6;
  const LaneLut lut(a.tab);
  uint4* reg = s_reg + wave * 64 * RCH;
  const float* mu = kZeroMean;
  int cur = -1;
  const int64_t n_tiles = (a.n + P::ROWS - 1) / P::ROWS;
  const int64_t t0 = blockIdx.x * tiles_per_block;
  const int64_t t1 = t0 + tiles_per_block < n_tiles ? t0 + tiles_per_block : n_tiles;
  // lanes past the end decode the last record (their rows are not stored)
  auto rec_of = [&](int64_t tile) {
    const int64_t vec = tile * P::ROWS + 64 * wave + opaque_lane();
    return reinterpret_cast<const uint32_t*>(a.rec) + (vec < a.n ? vec : a.n - 1) * NWT;
  };
  uint32_t wn[NWT];
  if (t0 < t1) load_words<NWT>(rec_of(t0), wn);
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int64_t row0 = tile * P::ROWS;
    const int bi = basis_of_row(a.pca, row0);
    if (bi != cur) {
      __syncthreads();
      const uint4* Bk = reinterpret_cast<const uint4*>(a.pca.basis + (int64_t)bi * D * R);
      for (int e = tid; e < D * HCH; e += 64 * W) {
        const uint4 w = Bk[e];
        const int j0 = 8 * (e % HCH);  // the chunk's first basis column; signs folded in
        s_B[swz<HCH>(e / HCH, e % HCH)] =
            make_uint4(w.x ^ a.tab.sign_pairs[j0 / 2], w.y ^ a.tab.sign_pairs[j0 / 2 + 1],
                       w.z ^ a.tab.sign_pairs[j0 / 2 + 2], w.w ^ a.tab.sign_pairs[j0 / 2 + 3]);
      }
      if (a.pca.mean) mu = a.pca.mean + (int64_t)bi * D;
      cur = bi;
      __syncthreads();
    }
    const int64_t rw0 = row0 + 64 * wave;
    const int ln = opaque_lane();
    uint32_t w[NWC];
#pragma unroll
    for (int i = 0; i < NWC; ++i) w[i] = wn[i];
    const float scale = __uint_as_float(wn[NWC]) * a.tab.inv_m;
    if (tile + 1 < t1) load_words<NWT>(rec_of(tile + 1), wn);  // in flight during this tile
    float zh[R];
    unpack_lookup_words<R, BITS>(w, lut, zh);
    fwht_regs<R>(zh);
    // scale * (H z^) as bf16 hi | lo halves of the lane's region row (the signs s are in s_B)
#pragma unroll
    for (int c = 0; c < HCH; ++c) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = zh[8 * c + 2 * e] * scale;
        const float x1 = zh[8 * c + 2 * e + 1] * scale;
        hi[e] = pack_bf16x2(x0, x1);
        lo[e] = pack_bf16x2(x0 - __uint_as_float(hi[e] << 16), x1 - __uint_as_float(hi[e] & 0xFFFF0000u));
      }
      reg[swz<RCH>(ln, c)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      reg[swz<RCH>(ln, HCH + c)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __builtin_amdgcn_wave_barrier();
    uint4 bh[4][KS], bl[4][KS];  // B-operand fragments: row tile nt, k step ks
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = 16 * nt + (ln & 15), ck = 4 * ks + (ln >> 4);
        bh[nt][ks] = reg[swz<RCH>(row, ck)];
        bl[nt][ks] = reg[swz<RCH>(row, HCH + ck)];
      }
    __builtin_amdgcn_wave_barrier();
    uint32_t* reg32 = reinterpret_cast<uint32_t*>(reg);
#pragma unroll
    for (int oc = 0; oc < D / OCOLS; ++oc) {
#pragma unroll
      for (int mt = 0; mt < OCOLS / 16; ++mt) {
        const int dl = 16 * mt + 4 * (ln >> 4);  // column within the staged chunk
        const float4 m4 = *reinterpret_cast<const float4*>(mu + oc * OCOLS + dl);
        const floatx4 init = floatx4{m4.x, m4.y, m4.z, m4.w};
        uint4 af[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          af[ks] = s_B[swz<HCH>(oc * OCOLS + 16 * mt + (ln & 15), 4 * ks + (ln >> 4))];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          floatx4 acc = init;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            acc = mfma_bf16(af[ks], bh[nt][ks], acc);
            acc = mfma_bf16(af[ks], bl[nt][ks], acc);
          }
          const int row = 16 * nt + (ln & 15);  // acc = out[row][d0 .. d0 + 3]
          if constexpr (BF16) {
            uint32_t* slot = reg32 + swz<RCH>(row, dl / 8) * 4 + 2 * ((dl / 4) & 1);
            slot[0] = pack_bf16x2(acc[0], acc[1]);
            slot[1] = pack_bf16x2(acc[2], acc[3]);
          } else {
            reg[swz<RCH>(row, dl / 4)] = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                                    __float_as_uint(acc[2]), __float_as_uint(acc[3]));
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      uint4 out[CCH];
#pragma unroll
      for (int k = 0; k < CCH; ++k) {
        const int id = k * 64 + ln, p = id / CCH, c = id % CCH;
        out[k] = reg[swz<RCH>(p, c)];
      }
#pragma unroll
      for (int k = 0; k < CCH; ++k) {
        const int id = k * 64 + ln, p = id / CCH, c = id % CCH;
        if (rw0 + p < a.n)
          st_stream(static_cast<uint8_t*>(a.y) + ((rw0 + p) * a.ld + oc * OCOLS) * ES + 16 * c, out[k]);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launchers. Supported (D, r): r in {32, 64, 128}, r <= D/2, D*r <= 32768, and r = D for D in
// {64, 128} (a square transform such as a whitening factor, then the rotation over all D).

// Blocks take consecutive tiles (consecutive tiles share a basis), as many as keeps the grid
// within what the chip holds at once.
struct PcaGrid {
  unsigned blocks;
  int64_t per_block;
};

template <int D, int R>
static PcaGrid pca_grid(int64_t n) {
  using P = PcaShape<D, R>;
  const int64_t tiles = (n + P::ROWS - 1) / P::ROWS;
  const int64_t resident = 256 * (160 * 1024 / (P::BASIS_BYTES + P::W * P::REGION_BYTES));
  const int64_t per = (tiles + resident - 1) / resident;
  return PcaGrid{(unsigned)((tiles + per - 1) / per), per};
}

template <int D, int R, int BITS, bool SYM>
static hipError_t enc_t(const EncodeArgs& a, hipStream_t st) {
  if constexpr (R == 64 && D <= 128) {
    return enc_pq_t<D, BITS, SYM>(a, st);
  } else if constexpr (R == 128) {
    return enc_pt_t<D, BITS, SYM>(a, st);
  } else {
    const PcaGrid g = pca_grid<D, R>(a.n);
    hipLaunchKernelGGL((k_encode_pca<D, R, BITS, SYM>), dim3(g.blocks), dim3(64 * PcaShape<D, R>::W), 0,
                       st, a, g.per_block);
    return hipGetLastError();
  }
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
  const PcaGrid pg = pca_grid<D, R>(a.n);
  const dim3 g(pg.blocks), b(64 * PcaShape<D, R>::W);
  if (bf16) hipLaunchKernelGGL((k_decode_pca<D, R, BITS, true>), g, b, 0, st, a, pg.per_block);
  else hipLaunchKernelGGL((k_decode_pca<D, R, BITS, false>), g, b, 0, st, a, pg.per_block);
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

#define KVQ_PCA_PAIRS(X) X(64, 32) X(64, 64) X(128, 32) X(128, 64) X(128, 128) X(256, 32) \
                         X(256, 64) X(256, 128) X(512, 32) X(512, 64)

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
