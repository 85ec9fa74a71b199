// Packed storage of GPTQ codes at b bits (b = 2..8).
//
// CLHA summary, section 2.3 (CLHA-MP): shared experts are stored at b+1 bits
// and routed experts at b, so storage follows the bit width of each matrix.
// GPTQ writes one byte per code; packed, code j of the stream occupies bits
// j*b .. j*b+b-1 of a little-endian bit stream (bit 0 is the least
// significant bit of byte 0).  Eight codes fill exactly b bytes, so a row of c
// codes (c a multiple of 8) is c*b/8 bytes and rows can be packed as one flat
// stream: each thread turns 8 codes into b bytes, with no carry between threads.
#include "kernels.h"

namespace clha {

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ packed, int64_t n8,
                                                         int bits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint2 v = *reinterpret_cast<const uint2*>(codes + 8 * i);
  const uint64_t mask = (1u << bits) - 1u;
  uint64_t acc = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t c = ((u < 4 ? v.x : v.y) >> (8 * (u & 3))) & 0xffu;
    acc |= ((uint64_t)c & mask) << (u * bits);
  }
  uint8_t* o = packed + i * bits;
  for (int k = 0; k < bits; ++k) o[k] = (uint8_t)(acc >> (8 * k));
}

__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint8_t* __restrict__ packed,
                                                           uint8_t* __restrict__ codes, int64_t n8,
                                                           int bits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint8_t* p = packed + i * bits;
  uint64_t acc = 0;
  for (int k = 0; k < bits; ++k) acc |= (uint64_t)p[k] << (8 * k);
  const uint64_t mask = (1u << bits) - 1u;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t c = (uint32_t)((acc >> (u * bits)) & mask);
    if (u < 4) lo |= c << (8 * u); else hi |= c << (8 * (u - 4));
  }
  *reinterpret_cast<uint2*>(codes + 8 * i) = make_uint2(lo, hi);
}

void launch_pack_codes(const uint8_t* codes, uint8_t* packed, int64_t n_codes, int bits, hipStream_t s) {
  const int64_t n8 = n_codes / 8;
  if (n8 == 0) return;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, codes, packed,
                     n8, bits);
}

void launch_unpack_codes(const uint8_t* packed, uint8_t* codes, int64_t n_codes, int bits, hipStream_t s) {
  const int64_t n8 = n_codes / 8;
  if (n8 == 0) return;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, packed, codes,
                     n8, bits);
}

}  // namespace clha
