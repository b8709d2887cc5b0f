// Grouped FC1 / FC2 GEMMs of the routed MoE layer, "stream" variant.
//
// One wave owns one M-tile of up to 16 rows of one expert and 4 blocks of 16
// output columns, and walks the whole contraction K in chunks of 128.  Weight
// fragments are loaded straight from HBM into the MFMA operand layout (no LDS):
// each lane reads one 32-element MX block of one weight row per chunk (16 B of
// E2M1 or 24 B of E3M2) plus its E8M0 scale, so every weight byte is read once
// per M-tile and the wave's loads cover whole 64-byte row segments.  This is
// the decode-shaped path: few rows per expert, bound by weight streaming
// (mxfp6-sm120 page, "Execution model": weights stay packed in the mainloop).
//
// Operand layouts of the gfx950 MFMAs used (measured on the device):
//  * v_mfma_f32_16x16x32_bf16: lane l supplies row (l%16), k = 8*(l/16)+j,
//    j = 0..7, of A and of B; C lane l element i is (row 4*(l/16)+i, col l%16).
//    The contraction order is free, so lane group g = l/16 takes the actual K
//    range [128c + 32g, +32) of chunk c, 8 elements per MFMA step.
//  * v_mfma_scale_f32_16x16x128_f8f6f4: an E2M1/E3M2 lane holds the 32
//    contiguous k of block g = l/16; an E4M3 lane holds k [16g, +16) and
//    [64+16g, +16); lane l's scale byte applies to (row l%16, k block l/16).
//
// bf16 activations: weights are dequantized in registers with
// v_cvt_scalef32_pk_bf16_fp4 (E2M1) or v_cvt_scalef32_pk32_bf16_bf6 (E3M2, the "bf6" format),
// exact for E8M0 scales, and multiplied on the bf16 MFMA.  MXFP8 activations: codes and scales feed the scaled MFMA
// directly (TokenSpeed SiTU page, "Activation precision": MXFP8 activation x
// MXFP4 weight; mxfp6-sm120 page: block-scaled MMA with FP32 accumulation).
#include <hip/hip_runtime.h>

#include "gemm.h"
#include "mx_device.h"

namespace moe_mx {

namespace {

constexpr int NB = 4;  // 16-column MFMA blocks per wave
typedef int v6i __attribute__((ext_vector_type(6)));
typedef __bf16 v32bf __attribute__((ext_vector_type(32)));

struct AFrag {
  uint4 d[4];      // bf16: 32 values; MX: d[0], d[1] = the two 16-byte code halves
  uint32_t scale;  // MX: scale dword of the chunk
};
struct BFrag {
  uint32_t d[6];   // E2M1: d[0..3]; E3M2: d[0..5]
  uint32_t scale;
};

template <bool MXA>
__device__ __forceinline__ void load_a(AFrag& f, const uint8_t* row, const uint8_t* srow, int c, int g) {
  if (row == nullptr) {
#pragma unroll
    for (int q = 0; q < 4; ++q) f.d[q] = make_uint4(0, 0, 0, 0);
    f.scale = 0x7f7f7f7fu;
    return;
  }
  if (MXA) {
    f.d[0] = *(const uint4*)(row + 128 * c + 16 * g);
    f.d[1] = *(const uint4*)(row + 128 * c + 64 + 16 * g);
    f.scale = *(const uint32_t*)(srow + 4 * c);
  } else {
    const uint4* p = (const uint4*)(row + 2 * (128 * c + 32 * g));
#pragma unroll
    for (int q = 0; q < 4; ++q) f.d[q] = p[q];
  }
}

template <int WF>
__device__ __forceinline__ void load_b(BFrag& f, const uint8_t* row, const uint8_t* srow, int c, int g) {
  if (WF == 1) {
    const uint4 v = *(const uint4*)(row + 64 * c + 16 * g);
    f.d[0] = v.x; f.d[1] = v.y; f.d[2] = v.z; f.d[3] = v.w; f.d[4] = 0; f.d[5] = 0;
  } else {
    const uint2* p = (const uint2*)(row + 24 * (4 * c + g));
    const uint2 a = p[0], b = p[1], d = p[2];
    f.d[0] = a.x; f.d[1] = a.y; f.d[2] = b.x; f.d[3] = b.y; f.d[4] = d.x; f.d[5] = d.y;
  }
  f.scale = *(const uint32_t*)(srow + 4 * c);
}

template <bool MXA, int WF>
__device__ __forceinline__ void mma_chunk(v4f (&acc)[NB], const AFrag& a, const BFrag (&b)[NB], int g) {
  if (MXA) {
    const v8i av = {(int)a.d[0].x, (int)a.d[0].y, (int)a.d[0].z, (int)a.d[0].w,
                    (int)a.d[1].x, (int)a.d[1].y, (int)a.d[1].z, (int)a.d[1].w};
    const int asc = (int)((a.scale >> (8 * g)) & 0xffu);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const v8i bv = {(int)b[n].d[0], (int)b[n].d[1], (int)b[n].d[2], (int)b[n].d[3],
                      (int)b[n].d[4], (int)b[n].d[5], 0, 0};
      const int bsc = (int)((b[n].scale >> (8 * g)) & 0xffu);
      acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[n], 0, Fmt<WF>::MFMA, 0, asc,
                                                                0, bsc);
    }
  } else if (WF == 2) {
    // E3M2: the lane's 32 codes (24 bytes, element i in bits 6i..6i+5) to 32
    // bf16 values in one conversion, exact for E8M0 scales
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const float sc = e8m0_to_f32((b[n].scale >> (8 * g)) & 0xffu);
      const v6i src = {(int)b[n].d[0], (int)b[n].d[1], (int)b[n].d[2], (int)b[n].d[3], (int)b[n].d[4],
                       (int)b[n].d[5]};
      const v32bf wv = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(src, sc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v8bf bv = {wv[8 * s], wv[8 * s + 1], wv[8 * s + 2], wv[8 * s + 3],
                         wv[8 * s + 4], wv[8 * s + 5], wv[8 * s + 6], wv[8 * s + 7]};
        const uint4 ad = a.d[s];
        v8bf av;
        __builtin_memcpy(&av, &ad, 16);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const float sc = e8m0_to_f32((b[n].scale >> (8 * g)) & 0xffu);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w = b[n].d[s];
        const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
        const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
        const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
        const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
        const v8bf bv = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        const uint4 ad = a.d[s];
        v8bf av;
        __builtin_memcpy(&av, &ad, 16);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
      }
    }
  }
}

// Full-K mainloop with the next chunk's loads issued before the current MFMAs.
template <bool MXA, int WF>
__device__ __forceinline__ void mainloop(v4f (&acc)[NB], const uint8_t* arow, const uint8_t* asrow,
                                         const uint8_t* const (&brow)[NB],
                                         const uint8_t* const (&bsrow)[NB], int nchunk, int g) {
  AFrag a0, a1;
  BFrag b0[NB], b1[NB];
  load_a<MXA>(a0, arow, asrow, 0, g);
#pragma unroll
  for (int n = 0; n < NB; ++n) load_b<WF>(b0[n], brow[n], bsrow[n], 0, g);
  int c = 0;
  for (; c + 2 <= nchunk; c += 2) {
    if (c + 1 < nchunk) {
      load_a<MXA>(a1, arow, asrow, c + 1, g);
#pragma unroll
      for (int n = 0; n < NB; ++n) load_b<WF>(b1[n], brow[n], bsrow[n], c + 1, g);
    }
    mma_chunk<MXA, WF>(acc, a0, b0, g);
    if (c + 2 < nchunk) {
      load_a<MXA>(a0, arow, asrow, c + 2, g);
#pragma unroll
      for (int n = 0; n < NB; ++n) load_b<WF>(b0[n], brow[n], bsrow[n], c + 2, g);
    }
    mma_chunk<MXA, WF>(acc, a1, b1, g);
  }
  if (c < nchunk) mma_chunk<MXA, WF>(acc, a0, b0, g);
}

__device__ __forceinline__ bool tile_of(const FcArgs& p, int ti, Tile& t) {
  if (p.dense_rows > 0) {
    t.expert = 0;
    t.p0 = 16 * ti;
    t.rows = min(16, p.dense_rows - 16 * ti);
    return t.rows > 0;
  }
  if (ti >= *p.num_tiles) return false;
  t = p.tiles[ti];
  return true;
}

}  // namespace

// FC1: h[p, n] = SiLU(A W1_gate^T)[p, n] * (A W1_up^T)[p, n] for the wave's
// 32 columns n; rows of A are gathered tokens.  bf16 mode stores h as bf16;
// MX mode quantizes each row's 32 columns to one E4M3 block with its scale.
template <bool MXA, int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_fc1_stream(FcArgs p) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = gw % p.nchunks, ti = gw / p.nchunks;
  Tile t;
  if (!tile_of(p, ti, t)) return;
  const int I = p.N, K = p.K;
  const int col0 = nch * 32;

  const uint8_t* arow = nullptr;
  const uint8_t* asrow = nullptr;
  if (r < t.rows) {
    const int prow = t.p0 + r;
    const int tok = p.dense_rows > 0 ? prow : p.sorted_assign[prow] / p.k;
    arow = (const uint8_t*)p.a + (int64_t)tok * (MXA ? K : 2 * K);
    if (MXA) asrow = p.a_scale + (int64_t)tok * (K / 32);
  }
  const uint8_t* wb = p.w + (int64_t)t.expert * p.w_estride;
  const uint8_t* sb = p.w_scale + (int64_t)t.expert * p.ws_estride;
  const int64_t wrow = (int64_t)K * Fmt<WF>::BITS / 8;
  const uint8_t* brow[NB];
  const uint8_t* bsrow[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int row = (n < NB / 2 ? 0 : I) + col0 + 16 * (n % (NB / 2)) + r;
    brow[n] = wb + (int64_t)row * wrow;
    bsrow[n] = sb + (int64_t)row * (K / 32);
  }
  v4f acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = (v4f){0.f, 0.f, 0.f, 0.f};
  mainloop<MXA, WF>(acc, arow, asrow, brow, bsrow, K / 128, g);

  // epilogue: lane holds rows 4g+i, columns col0 + 16h + r (h = 0, 1)
  float hv[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[h][i] = gated_act(p.act_fn, acc[h][i], acc[h + 2][i]);
  if (!MXA) {
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i;
      if (row < t.rows) {
        const int64_t o = (int64_t)(t.p0 + row) * I + col0 + r;
        out[o] = f32_to_bf16_rne(hv[0][i]);
        out[o + 16] = f32_to_bf16_rne(hv[1][i]);
      }
    }
  } else {
    uint8_t* out = (uint8_t*)p.out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t m = max(__float_as_uint(hv[0][i]) & 0x7fffffffu, __float_as_uint(hv[1][i]) & 0x7fffffffu);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
      const int s = block_exponent<3>(m);
      const float inv = exp2_neg(s);
      const int row = 4 * g + i;
      if (row < t.rows) {
        const int64_t prow = t.p0 + row;
        const int64_t o = prow * I + col0 + r;
        out[o] = (uint8_t)encode<3>(hv[0][i] * inv);
        out[o + 16] = (uint8_t)encode<3>(hv[1][i] * inv);
        if (r == 0) p.out_scale[prow * (I / 32) + col0 / 32] = (uint8_t)(s + 127);
      }
    }
  }
}

// FC2: obuf[a(p), n] = w(p) * (A W2^T)[p, n] for the wave's 64 columns n;
// rows of A are rows of h in permuted order.
template <bool MXA, int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_fc2_stream(FcArgs p) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = gw % p.nchunks, ti = gw / p.nchunks;
  Tile t;
  if (!tile_of(p, ti, t)) return;
  const int H = p.N, K = p.K;
  const int col0 = nch * 64;

  const uint8_t* arow = nullptr;
  const uint8_t* asrow = nullptr;
  if (r < t.rows) {
    const int64_t prow = t.p0 + r;
    arow = (const uint8_t*)p.a + prow * (MXA ? K : 2 * K);
    if (MXA) asrow = p.a_scale + prow * (K / 32);
  }
  const uint8_t* wb = p.w + (int64_t)t.expert * p.w_estride;
  const uint8_t* sb = p.w_scale + (int64_t)t.expert * p.ws_estride;
  const int64_t wrow = (int64_t)K * Fmt<WF>::BITS / 8;
  const uint8_t* brow[NB];
  const uint8_t* bsrow[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    // columns past N (a dense GEMM with N % 64 != 0) read the last weight
    // row and are not stored
    const int row = min(col0 + 16 * n + r, H - 1);
    brow[n] = wb + (int64_t)row * wrow;
    bsrow[n] = sb + (int64_t)row * (K / 32);
  }
  v4f acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = (v4f){0.f, 0.f, 0.f, 0.f};
  mainloop<MXA, WF>(acc, arow, asrow, brow, bsrow, K / 128, g);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    if (row >= t.rows) continue;
    const int prow = t.p0 + row;
    int64_t orow;
    float w;
    if (p.dense_rows > 0) {
      orow = prow;
      w = p.dense_weight;
    } else {
      const int a = p.sorted_assign[prow];
      orow = a;
      w = p.topk_w[a];
    }
    uint16_t* o = p.obuf + orow * H + col0 + r;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      if (col0 + 16 * n + r < H) o[16 * n] = f32_to_bf16_rne(w * acc[n][i]);
  }
}

template <bool MXA, int WF>
static hipError_t launch_pair(const FcArgs& p, bool fc1, hipStream_t st) {
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + 15) / 16 : p.max_tiles;
  const int64_t waves = (int64_t)ntiles * p.nchunks;
  if (waves == 0) return hipSuccess;
  const int64_t blocks = (waves + 3) / 4;
  if (fc1) k_fc1_stream<MXA, WF><<<blocks, 256, 0, st>>>(p);
  else k_fc2_stream<MXA, WF><<<blocks, 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_fc_stream(const FcArgs& p, bool fc1, bool mx_act, int wfmt, hipStream_t st) {
  if (mx_act) return wfmt == 1 ? launch_pair<true, 1>(p, fc1, st) : launch_pair<true, 2>(p, fc1, st);
  return wfmt == 1 ? launch_pair<false, 1>(p, fc1, st) : launch_pair<false, 2>(p, fc1, st);
}

}  // namespace moe_mx
