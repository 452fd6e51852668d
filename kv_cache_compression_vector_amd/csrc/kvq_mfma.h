// kvq_mfma.h — MFMA operand helpers shared by the gfx950 codec kernels.
//
// v_mfma_f32_16x16x32_bf16 operand layout (lane l of a wave64):
//   A[m = l % 16][k = 8 (l / 16) + e],  B[k = 8 (l / 16) + e][n = l % 16],  e = 0..7 (one uint4)
//   D[m = 4 (l / 16) + i][n = l % 16],  i = 0..3 (one floatx4)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma_bf16(const uint4& a, const uint4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16-byte chunk c of row r in an LDS tile whose rows are CH chunks apart, XOR-swizzled so that
// 16 lanes reading one chunk column (or one row each) hit distinct banks.
template <int CH>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int mask = (CH < 16 ? CH : 16) - 1;
  return r * CH + (c ^ (r & mask));
}

// The lane index as a value the compiler cannot see through: addresses derived from it inside a
// tile loop are recomputed each tile instead of being hoisted out of the loop (and spilled).
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// OR over aligned groups of G lanes (G = 2, 4, 8 or 16); every lane of a group gets the result.
template <int G>
__device__ __forceinline__ uint32_t group_or(uint32_t x) {
  if constexpr (G >= 2) x |= dpp_u32<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x |= dpp_u32<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x |= dpp_u32<0x141>(x);  // row_half_mirror: quad 0 <-> quad 1
  if constexpr (G >= 16) x |= dpp_u32<0x140>(x); // row_mirror: half-row 0 <-> half-row 1
  return x;
}

}  // namespace kvq
