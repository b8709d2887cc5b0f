// mx_quantize: block quantization of a row-major matrix to MX codes + E8M0 scales.
//
// One lane owns one 32-element block: it reads the block (64 B of bf16 or
// 128 B of fp32), takes the largest magnitude on the integer bits, derives the
// shared exponent, encodes the 32 elements and writes them packed (16 B of
// E2M1, 24 B of E3M2 or 32 B of E4M3) plus one scale byte.  Consecutive lanes
// own consecutive blocks of a row, so a wave reads and writes contiguous
// memory.  The kernel is bound by HBM bandwidth.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mx_device.h"

namespace moe_mx {

template <int FMT, bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ src, int64_t rows,
                                                  int64_t nblk_row, int64_t src_ld,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  using F = Fmt<FMT>;
  const int64_t total = rows * nblk_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / nblk_row;
    const int64_t b = i - r * nblk_row;
    uint32_t v[32];  // fp32 bits
    if (BF16) {
      const uint16_t* p = (const uint16_t*)src + r * src_ld + b * 32;
      if (VEC) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 d = ((const uint4*)p)[q];
          uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[q * 8 + 2 * j] = w[j] << 16;
            v[q * 8 + 2 * j + 1] = w[j] & 0xffff0000u;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = (uint32_t)p[j] << 16;
      }
    } else {
      const uint32_t* p = (const uint32_t*)src + r * src_ld + b * 32;
      if (VEC) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint4 d = ((const uint4*)p)[q];
          v[4 * q] = d.x; v[4 * q + 1] = d.y; v[4 * q + 2] = d.z; v[4 * q + 3] = d.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = p[j];
      }
    }
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = max(amax, v[j] & 0x7fffffffu);
    const int s = block_exponent<FMT>(amax);
    const float inv = exp2_neg(s);
    uint32_t c[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = encode<FMT>(__uint_as_float(v[j]) * inv);
    scales[i] = (uint8_t)(s + 127);
    if (FMT == 1) {  // 16 bytes
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc |= c[q * 8 + j] << (4 * j);
        w[q] = acc;
      }
      *(uint4*)(codes + i * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if (FMT == 2) {  // 24 bytes: six dwords of contiguous 6-bit fields
      uint32_t w[6];
#pragma unroll
      for (int q = 0; q < 6; ++q) w[q] = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int bit = 6 * j, wi = bit >> 5, sh = bit & 31;
        w[wi] |= c[j] << sh;
        if (sh > 26) w[wi + 1] |= c[j] >> (32 - sh);
      }
      uint2* o = (uint2*)(codes + i * 24);
      o[0] = make_uint2(w[0], w[1]);
      o[1] = make_uint2(w[2], w[3]);
      o[2] = make_uint2(w[4], w[5]);
    } else {  // 32 bytes, two codes per hardware conversion
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        w[q] = e4m3_pair(__uint_as_float(v[4 * q]) * inv, __uint_as_float(v[4 * q + 1]) * inv) |
               (e4m3_pair(__uint_as_float(v[4 * q + 2]) * inv, __uint_as_float(v[4 * q + 3]) * inv) << 16);
      }
      uint4* o = (uint4*)(codes + i * 32);
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

template <int FMT>
static void launch_fmt(const void* src, bool bf16, bool vec, int64_t rows, int64_t nb, int64_t ld,
                       uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t total = rows * nb;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (bf16 && vec) k_quantize<FMT, true, true><<<blocks, 256, 0, st>>>(src, rows, nb, ld, codes, scales);
  else if (bf16) k_quantize<FMT, true, false><<<blocks, 256, 0, st>>>(src, rows, nb, ld, codes, scales);
  else if (vec) k_quantize<FMT, false, true><<<blocks, 256, 0, st>>>(src, rows, nb, ld, codes, scales);
  else k_quantize<FMT, false, false><<<blocks, 256, 0, st>>>(src, rows, nb, ld, codes, scales);
}

hipError_t launch_quantize(const void* src, moe_src_t src_dtype, int64_t rows, int64_t cols,
                           int64_t src_ld, mx_elem_t fmt, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const bool bf16 = src_dtype == MOE_SRC_BF16;
  const int64_t esz = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)src % 16 == 0) && ((src_ld * esz) % 16 == 0);
  const int64_t nb = cols / 32;
  switch (fmt) {
    case MX_E2M1: launch_fmt<1>(src, bf16, vec, rows, nb, src_ld, codes, scales, stream); break;
    case MX_E3M2: launch_fmt<2>(src, bf16, vec, rows, nb, src_ld, codes, scales, stream); break;
    default: launch_fmt<3>(src, bf16, vec, rows, nb, src_ld, codes, scales, stream); break;
  }
  return hipGetLastError();
}

}  // namespace moe_mx
