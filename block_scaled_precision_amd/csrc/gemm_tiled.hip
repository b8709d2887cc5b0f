// Grouped FC1 / FC2 GEMMs of the routed MoE layer for MXFP8 activations,
// "tiled" variant: LDS-staged tiles on the gfx950 block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 (mxfp6-sm120 page, "Execution model":
// E4M3 activations and packed MX weights, each with one UE8M0 scale per 32 K
// values, block-scaled MMA with FP32 accumulation; TokenSpeed SiTU page,
// "Activation precision": MXFP8 activation x MXFP4 weight).
//
// Work item = (M-tile, N-block).  An M-tile holds up to 256 permuted rows of one
// expert, so an expert with <= 256 assignments streams its weights from HBM
// exactly once; the N-block is 128 weight rows (FC1: 64 gate rows and the 64
// matching up rows, i.e. 64 columns of h; FC2: 128 output columns).  The grid is
// persistent: one workgroup of 4 waves per CU walks the items of its XCD (the
// M-tiles x, x+8, ... of XCD x), so the N-blocks of one M-tile run together on
// one XCD and its activation rows stay in that XCD's L2.
//
// Per K-stage of 128: every thread loads its share of the A tile (gathered rows
// of E4M3 codes, 128 B per row), of the B tile (packed weights, 64 B per row for
// E2M1, 96 B for E3M2) and of the per-row scale words into registers, one stage
// ahead of the MFMAs, and writes them to the other half of a double-buffered
// LDS tile.  Waves are laid out 2 (M) x 2 (N): wave (wm, wn) owns the 32-row
// sub-blocks wm, wm+2, wm+4, wm+6 of the tile (interleaved, so both M halves
// stay busy when a tile is partly filled) and two 32-column MFMA tiles.
//
// MFMA operand layouts (v_mfma_scale_f32_32x32x64_f8f6f4, measured on the
// device): lane l supplies row l%32 of its operand and the scale of (row l%32,
// 32-k block l/32); an E4M3 lane holds k [16g, 16g+16) and [32+16g, 32+16g+16)
// of the 64-k step (g = l/32), an E2M1/E3M2 lane holds k [32g, 32g+32).  So the
// natural memory order of each row serves both operands: 32-k block b of the
// stage is bytes [32b, 32b+32) of an E4M3 row, [16b, 16b+16) of an E2M1 row and
// [24b, 24b+24) of an E3M2 row.  Accumulator element i of lane l is
// (row 8*(i/4) + 4*(l/32) + i%4, column l%32).
#include <hip/hip_runtime.h>

#include "gemm.h"
#include "mx_device.h"

namespace moe_mx {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int TBM = kTiledRows;  // rows per M-tile (8 sub-blocks of 32)
constexpr int TBN = 128;         // weight rows per work item
constexpr int TBK = 128;         // K per stage
constexpr int kThreads = 256;

template <int WF> struct BLay {
  static constexpr int ROW = WF == 1 ? 64 : 96;  // bytes of one weight row per stage
  static constexpr int CHUNKS = ROW / 16;        // 16-byte chunks per row
  static constexpr int PER_THREAD = TBN * CHUNKS / kThreads;  // 2 (E2M1) or 3 (E3M2)
};

template <int WF> struct Lds {
  static constexpr int A = TBM * TBK;               // E4M3 codes
  static constexpr int B = TBN * BLay<WF>::ROW;     // packed weights
  static constexpr int SA = TBM * 4;                // 4 scale codes per row and stage
  static constexpr int SB = TBN * 4;
  static constexpr int STAGE = A + B + SA + SB;
  static constexpr int TOTAL = 2 * STAGE;
};

// A tile: row r holds 8 chunks of 16 B; chunk c sits at slot c ^ (r & 7) so
// that 8 consecutive rows read at the same k land in 8 different bank groups.
__device__ __forceinline__ int a_off(int r, int c) { return r * TBK + 16 * (c ^ (r & 7)); }
// E2M1 B tile: 4 chunks per 64-B row, chunk c at slot c ^ ((r >> 1) & 3).
__device__ __forceinline__ int b4_off(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

template <int WF>
struct Staged {
  uint4 a[8];
  uint4 b[BLay<WF>::PER_THREAD];
  uint32_t sa, sb;
};

struct ItemGeom {
  int expert, p0, rows, nb;
};

__device__ __forceinline__ bool tiled_tile(const FcArgs& p, int ti, ItemGeom& g) {
  if (p.dense_rows > 0) {
    g.expert = 0;
    g.p0 = TBM * ti;
    g.rows = min(TBM, p.dense_rows - TBM * ti);
    return g.rows > 0;
  }
  const Tile t = p.tiles[ti];
  g.expert = t.expert;
  g.p0 = t.p0;
  g.rows = t.rows;
  return true;
}

}  // namespace

template <bool FC1, int WF>
__global__ __launch_bounds__(kThreads, 1) void k_fc_tiled(FcArgs p) {
  using L = Lds<WF>;
  using BL = BLay<WF>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::TOTAL];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int K = p.K, nk = K / TBK, NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + TBM - 1) / TBM : *p.num_tiles;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3, Q = gridDim.x >> 3;
  const int xt = ntiles > xcd ? (ntiles - xcd + 7) / 8 : 0;
  const int nitems = xt * NB;
  const int64_t wrow = (int64_t)K * Fmt<WF>::BITS / 8;  // bytes of one weight row
  const int ksc = K / 32;                                // scale bytes per row

  for (int j = q; j < nitems; j += Q) {
    ItemGeom it;
    tiled_tile(p, xcd + 8 * (j / NB), it);
    it.nb = j % NB;
    const int nsub = (it.rows + 31) >> 5;

    // ---- per-item load addresses (nullptr / -1: row outside the tile) ----
    const uint8_t* arow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      arow[i] = nullptr;
      if (r < it.rows) {
        const int prow = it.p0 + r;
        const int64_t src = FC1 ? (p.dense_rows > 0 ? prow : p.sorted_assign[prow] / p.k) : prow;
        arow[i] = (const uint8_t*)p.a + src * K + 16 * (tid & 7);
      }
    }
    const uint8_t* asrow = nullptr;
    if (tid < it.rows) {
      const int prow = it.p0 + tid;
      const int64_t src = FC1 ? (p.dense_rows > 0 ? prow : p.sorted_assign[prow] / p.k) : prow;
      asrow = p.a_scale + src * ksc;
    }
    const uint8_t* wb = p.w + (int64_t)it.expert * p.w_estride;
    const uint8_t* sb = p.w_scale + (int64_t)it.expert * p.ws_estride;
    // weight row held at B-tile row j
    auto wrow_of = [&](int jr) -> int64_t {
      if (FC1) return jr < TBN / 2 ? (int64_t)it.nb * (TBN / 2) + jr : (int64_t)p.N + it.nb * (TBN / 2) + jr - TBN / 2;
      return (int64_t)it.nb * TBN + jr;
    };
    const uint8_t* brow[BL::PER_THREAD];
    int bslot[BL::PER_THREAD];
#pragma unroll
    for (int i = 0; i < BL::PER_THREAD; ++i) {
      const int c = tid + kThreads * i;
      const int jr = c / BL::CHUNKS, ch = c % BL::CHUNKS;
      brow[i] = wb + wrow_of(jr) * wrow + 16 * ch;
      bslot[i] = WF == 1 ? b4_off(jr, ch) : jr * BL::ROW + 16 * ch;
    }
    const uint8_t* bsrow = tid < TBN ? sb + wrow_of(tid) * ksc : nullptr;

    auto load = [&](Staged<WF>& st, int s) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        st.a[i] = arow[i] ? *(const uint4*)(arow[i] + s * TBK) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < BL::PER_THREAD; ++i) st.b[i] = *(const uint4*)(brow[i] + s * (TBK * Fmt<WF>::BITS / 8));
      st.sa = asrow ? *(const uint32_t*)(asrow + 4 * s) : 0x7f7f7f7fu;
      st.sb = bsrow ? *(const uint32_t*)(bsrow + 4 * s) : 0u;
    };
    auto store = [&](const Staged<WF>& st, int buf) {
      uint8_t* base = smem + buf * L::STAGE;
#pragma unroll
      for (int i = 0; i < 8; ++i) *(uint4*)(base + a_off((tid >> 3) + 32 * i, tid & 7)) = st.a[i];
#pragma unroll
      for (int i = 0; i < BL::PER_THREAD; ++i) *(uint4*)(base + L::A + bslot[i]) = st.b[i];
      *(uint32_t*)(base + L::A + L::B + 4 * tid) = st.sa;
      if (tid < TBN) *(uint32_t*)(base + L::A + L::B + L::SA + 4 * tid) = st.sb;
    };

    v16f acc[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.f;

    // B-tile rows of this wave's two column tiles
    const int brow0 = FC1 ? 32 * wn : 64 * wn;
    const int brow1 = FC1 ? TBN / 2 + 32 * wn : 64 * wn + 32;

    auto compute = [&](int buf) {
      const uint8_t* base = smem + buf * L::STAGE;
      const uint8_t* As = base;
      const uint8_t* Bs = base + L::A;
      const uint32_t* SAs = (const uint32_t*)(base + L::A + L::B);
      const uint32_t* SBs = (const uint32_t*)(base + L::A + L::B + L::SA);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v8i bv[2];
        int bsc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int jr = (n == 0 ? brow0 : brow1) + l32;
          const int blk = 2 * kk + g;
          if (WF == 1) {
            const uint4 v = *(const uint4*)(Bs + b4_off(jr, blk));
            bv[n] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          } else {
            const uint8_t* rp = Bs + jr * BL::ROW + 24 * blk;
            uint4 v;
            uint2 d;
            if ((blk & 1) == 0) {
              v = *(const uint4*)rp;
              d = *(const uint2*)(rp + 16);
              bv[n] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, (int)d.x, (int)d.y, 0, 0};
            } else {
              d = *(const uint2*)rp;
              v = *(const uint4*)(rp + 8);
              bv[n] = (v8i){(int)d.x, (int)d.y, (int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0};
            }
          }
          bsc[n] = (int)((SBs[jr] >> (8 * blk)) & 0xffu);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int sbk = wm + 2 * m;
          if (sbk < nsub) {
            const int r = 32 * sbk + l32;
            const uint4 lo = *(const uint4*)(As + a_off(r, 4 * kk + g));
            const uint4 hi = *(const uint4*)(As + a_off(r, 4 * kk + 2 + g));
            const v8i av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int asc = (int)((SAs[r] >> (8 * (2 * kk + g))) & 0xffu);
#pragma unroll
            for (int n = 0; n < 2; ++n)
              acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv[n], acc[m][n], 0, Fmt<WF>::MFMA,
                                                                          0, asc, 0, bsc[n]);
          }
        }
      }
    };

    // ---- mainloop: stage s+1 is loaded into registers while stage s computes ----
    Staged<WF> st;
    load(st, 0);
    store(st, 0);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
      const bool more = s + 1 < nk;
      if (more) load(st, s + 1);
      compute(s & 1);
      if (more) store(st, (s + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int sbk = wm + 2 * m;
      if (sbk >= nsub) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * sbk + 8 * (i >> 2) + 4 * g + (i & 3);
        if (FC1) {
          // h = SiLU(gate) * up for column nb*64 + 32*wn + l32, then one E4M3
          // block per (row, 32 columns) with its E8M0 scale
          const float h = silu_mul(acc[m][0][i], acc[m][1][i]);
          uint32_t mx = __float_as_uint(h) & 0x7fffffffu;
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
          const int sexp = block_exponent<3>(mx);
          if (row < it.rows) {
            const int64_t prow = it.p0 + row;
            const int col0 = it.nb * (TBN / 2) + 32 * wn;
            ((uint8_t*)p.out)[prow * p.N + col0 + l32] = (uint8_t)encode<3>(h * exp2_neg(sexp));
            if (l32 == 0) p.out_scale[prow * (p.N / 32) + col0 / 32] = (uint8_t)(sexp + 127);
          }
        } else {
          if (row < it.rows) {
            const int prow = it.p0 + row;
            int tok;
            float w;
            if (p.dense_rows > 0) {
              tok = prow;
              w = p.dense_weight;
            } else {
              const int a = p.sorted_assign[prow];
              tok = a / p.k;
              w = p.topk_w[a];
            }
            float* y = p.y_acc + (int64_t)tok * p.N + it.nb * TBN + 64 * wn + l32;
            unsafeAtomicAdd(y, w * acc[m][0][i]);
            unsafeAtomicAdd(y + 32, w * acc[m][1][i]);
          }
        }
      }
    }
  }
}

template <bool FC1, int WF>
static hipError_t launch_tiled_t(const FcArgs& p, int grid, hipStream_t st) {
  k_fc_tiled<FC1, WF><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_fc_tiled(const FcArgs& p, bool fc1, int wfmt, int grid, hipStream_t st) {
  if (grid < 8) grid = 8;
  grid &= ~7;
  if (fc1) return wfmt == 1 ? launch_tiled_t<true, 1>(p, grid, st) : launch_tiled_t<true, 2>(p, grid, st);
  return wfmt == 1 ? launch_tiled_t<false, 1>(p, grid, st) : launch_tiled_t<false, 2>(p, grid, st);
}

}  // namespace moe_mx
