// kvq_misc.hip — small helper kernels: tail-ring append, word clearing, and a streaming copy
// (the bandwidth control a measurement runs next to the codec kernels).
#include "kvq_device.h"
#include "kvq_kernels.h"

namespace kvq {

// Copy new rows into the dense tail rings of several caches (16 bytes per lane).
__global__ __launch_bounds__(256) void k_tail_copy(TailCopyArgs a) {
  const int64_t per_row = a.D / 8;  // uint4 per row
  const int64_t total = a.total_rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t g = i / per_row, q = i % per_row;
    int k = 0;
    while (k + 1 < a.n_caches && g >= a.c[k + 1].row_begin) ++k;
    const TailCopyCache& tc = a.c[k];
    const int64_t r = g - tc.row_begin;
    const int64_t slot = (tc.first_slot + r) % tc.cap;
    const uint4 v = reinterpret_cast<const uint4*>(tc.src + r * a.D)[q];
    reinterpret_cast<uint4*>(tc.ring + slot * a.D)[q] = v;
  }
}

__global__ __launch_bounds__(256) void k_clear_u32(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// Streaming copy of n16 16-byte words: each thread moves 4 words per pass, all four loads
// issued before the stores, grid-stride over the array.
__global__ __launch_bounds__(256) void k_stream_copy(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                     int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i + 256 * k < n16) v[k] = ld_stream(src + i + 256 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i + 256 * k < n16) st_stream(dst + i + 256 * k, v[k]);
  }
}

// Grid of a streaming control: at most per_cu blocks per CU (measured on MI355X at 1 GiB: the
// read peaks at 4 blocks per CU, 7.0 TB/s, where fewer blocks also mean fewer atomics; the fill
// at 32, 5.3 TB/s; the copy is flat from 4 to 32 at 5.9 TB/s).
static int64_t stream_blocks(int64_t n16, int per_cu) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t blocks = (n16 + 1023) / 1024, cap = (int64_t)cus * per_cu;
  return blocks > cap ? cap : blocks;
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)stream_blocks(n16, 8)), dim3(256), 0, st,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

// Streaming read of n16 16-byte words, folded by XOR: each thread keeps four words in flight
// per pass, and each block adds its fold to *sink with one atomic XOR.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, int64_t n16,
                                                     uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = i + 256 * k < n16 ? ld_stream(src + i + 256 * k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(sink, part[0] ^ part[1] ^ part[2] ^ part[3]);
}

// Streaming fill of n16 16-byte words with one 32-bit value.
__global__ __launch_bounds__(256) void k_stream_fill(uint4* __restrict__ dst, int64_t n16, uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  const uint4 v = make_uint4(value, value, value, value);
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i + 256 * k < n16) st_stream(dst + i + 256 * k, v);
  }
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)stream_blocks(n16, 4)), dim3(256), 0, st,
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_fill(void* dst, int64_t bytes, uint32_t value, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_fill, dim3((unsigned)stream_blocks(n16, 32)), dim3(256), 0, st,
                     static_cast<uint4*>(dst), n16, value);
  return hipGetLastError();
}

hipError_t launch_tail_copy(const TailCopyArgs& a, hipStream_t st) {
  const int64_t total = a.total_rows * (a.D / 8);
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_tail_copy, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_clear_u32(uint32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_clear_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace kvq
