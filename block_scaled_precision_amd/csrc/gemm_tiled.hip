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
// persistent: one workgroup of 8 waves per CU walks the items of its XCD (the
// M-tiles x, x+8, ... of XCD x), so the N-blocks of one M-tile run together on
// one XCD and its activation rows stay in that XCD's L2.
//
// Data movement: a K-stage (128 values of K) of the A tile (gathered rows of
// E4M3 codes, 128 B per row), of the B tile (packed weights, 64 B per row for
// E2M1, 96 B for E3M2) and of their per-row scale words is copied straight
// from global memory into LDS by global_load_lds (no register staging), into a
// ring of three stage buffers: while stage s is multiplied, stages s+1 and s+2
// are in flight.  The stream of (item, stage) steps is continuous across the
// items of a workgroup, so the next item's first stages load during the
// current item's last ones.  The copies are issued from inline assembly, so
// the only waits on them are the explicit per-stage vmcnt waits below.
//
// Eight waves (two per SIMD, so one wave's LDS reads overlap the other's MFMAs)
// are laid out 4 (M) x 2 (N): wave (wm, wn) owns the 32-row sub-blocks wm and
// wm+4 of the tile (so a partly filled tile still spreads over all SIMDs) and
// two 32-column MFMA tiles.
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
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <int WF> struct BLay {
  static constexpr int ROW = WF == 1 ? 64 : 96;  // bytes of one weight row per stage
  static constexpr int COPIES = TBN * ROW / 1024;  // 1-KB copies per stage: 8 (E2M1), 12 (E3M2)
  static constexpr int PER_WAVE = (COPIES + kWaves - 1) / kWaves;  // 1 or 2
};

template <int WF> struct Lds {
  static constexpr int A = TBM * TBK;            // E4M3 codes
  static constexpr int B = TBN * BLay<WF>::ROW;  // packed weights
  static constexpr int SA = TBM * 4;             // 4 scale codes per row and stage
  static constexpr int SB = TBN * 4;
  static constexpr int STAGE = A + B + SA + SB;
};

// Copies issued per wave and stage: 4 (A) + B + 1 scale copy.
template <int WF> constexpr int copies_per_stage() { return 4 + BLay<WF>::PER_WAVE + 1; }

// s_waitcnt with vmcnt(n) and lgkmcnt(0) (gfx9 encoding; expcnt left at its maximum).
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Asynchronous copies global -> LDS (global_load_lds): lane i of the wave writes
// its `size` bytes at lds + size*i; `lds` is a wave-uniform LDS byte address.
// M0 carries the LDS address; one wait state separates its write from the copy.
__device__ __forceinline__ void lds_copy16(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(src) : "memory");
}
__device__ __forceinline__ void lds_copy4(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds), "v"(src) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// A tile: row r holds 8 chunks of 16 B; chunk c sits at slot c ^ (r & 7) so
// that 8 consecutive rows read at the same k land in 8 different bank groups.
__device__ __forceinline__ int a_off(int r, int c) { return r * TBK + 16 * (c ^ (r & 7)); }
// E2M1 B tile: 4 chunks per 64-B row, chunk c at slot c ^ ((r >> 1) & 3).
__device__ __forceinline__ int b4_off(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

struct ItemGeom {
  int expert, p0, rows, nb;
};

__device__ __forceinline__ ItemGeom item_geom(const FcArgs& p, int xcd, int j, int NB) {
  ItemGeom g;
  const int ti = xcd + 8 * (j / NB);
  g.nb = j % NB;
  if (p.dense_rows > 0) {
    g.expert = 0;
    g.p0 = TBM * ti;
    g.rows = min(TBM, p.dense_rows - TBM * ti);
  } else {
    const Tile t = p.tiles[ti];
    g.expert = t.expert;
    g.p0 = t.p0;
    g.rows = t.rows;
  }
  return g;
}

// Per-thread source addresses of one item's copies at stage 0 (stage s adds a
// fixed stride) and the wave-uniform LDS offsets they land at.
template <int WF>
struct LoadGeom {
  const uint8_t* a[4];  // A: 16-B chunk of row 8*(4*wave + i) + lane/8
  const uint8_t* b[BLay<WF>::PER_WAVE];
  const uint8_t* sc;    // waves 0-3: A scale word of row 64*wave + lane;
                        // waves 4-7: B scale word of row 64*(wave & 1) + lane
};

// row of the gathered activations that feeds tile row r (r < it.rows)
template <bool FC1>
__device__ __forceinline__ int64_t a_src_row(const FcArgs& p, int prow) {
  if (!FC1 || p.dense_rows > 0) return prow;
  return p.sorted_assign[prow] / p.k;
}

// weight row held at B-tile row jr
template <bool FC1>
__device__ __forceinline__ int64_t w_row(const FcArgs& p, int nb, int jr) {
  if (FC1) return jr < TBN / 2 ? (int64_t)nb * (TBN / 2) + jr : (int64_t)p.N + nb * (TBN / 2) + jr - TBN / 2;
  return (int64_t)nb * TBN + jr;
}

template <int WF> __device__ __forceinline__ int b_copy(int wv, int i) {
  // E3M2: waves 0-3 take copies wv and 8+wv, waves 4-7 repeat their first copy
  // (the same bytes to the same place) so that every wave issues as many copies
  if (WF == 1) return wv;
  return i == 0 ? wv : (wv < 4 ? 8 + wv : wv);
}

template <bool FC1, int WF>
__device__ __forceinline__ void setup_loads(const FcArgs& p, const ItemGeom& it, LoadGeom<WF>& lg) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int K = p.K;
  // rows outside the tile copy the tile's last row (their results are never stored)
  const int c = (lane & 7) ^ (lane >> 3);  // chunk that lands in this lane's LDS slot
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(8 * (4 * wv + i) + (lane >> 3), it.rows - 1);
    lg.a[i] = (const uint8_t*)p.a + a_src_row<FC1>(p, it.p0 + r) * K + 16 * c;
  }
  const uint8_t* wb = p.w + (int64_t)it.expert * p.w_estride;
  const uint8_t* sb = p.w_scale + (int64_t)it.expert * p.ws_estride;
  const int64_t wrow = (int64_t)K * Fmt<WF>::BITS / 8;
#pragma unroll
  for (int i = 0; i < BLay<WF>::PER_WAVE; ++i) {
    const int t = b_copy<WF>(wv, i);
    int jr, ch;
    if (WF == 1) {
      jr = 16 * t + (lane >> 2);
      ch = (lane & 3) ^ ((jr >> 1) & 3);
    } else {
      const int cc = 64 * t + lane;
      jr = cc / 6;
      ch = cc % 6;
    }
    lg.b[i] = wb + w_row<FC1>(p, it.nb, jr) * wrow + 16 * ch;
  }
  if (wv < 4) {
    const int r = min(64 * wv + lane, it.rows - 1);
    lg.sc = p.a_scale + a_src_row<FC1>(p, it.p0 + r) * (K / 32);
  } else {
    lg.sc = sb + w_row<FC1>(p, it.nb, 64 * (wv & 1) + lane) * (K / 32);
  }
}

template <int WF>
__device__ __forceinline__ void issue_stage(const LoadGeom<WF>& lg, int s, uint32_t buf) {
  using L = Lds<WF>;
  const int wv = threadIdx.x >> 6;
  const int ao = s * TBK, bo = s * (TBK * Fmt<WF>::BITS / 8), so = 4 * s;
#pragma unroll
  for (int i = 0; i < 4; ++i) lds_copy16(lg.a[i] + ao, __builtin_amdgcn_readfirstlane(buf + 1024 * (4 * wv + i)));
#pragma unroll
  for (int i = 0; i < BLay<WF>::PER_WAVE; ++i)
    lds_copy16(lg.b[i] + bo, __builtin_amdgcn_readfirstlane(buf + L::A + 1024 * b_copy<WF>(wv, i)));
  const uint32_t so_lds = wv < 4 ? buf + L::A + L::B + 256 * wv : buf + L::A + L::B + L::SA + 256 * (wv & 1);
  lds_copy4(lg.sc + so, __builtin_amdgcn_readfirstlane(so_lds));
}

// One 128-K stage for a wave holding NM (1 or 2) sub-blocks: sub-block
// wm + 4m of the tile times the wave's two 32-column B tiles.
template <int WF, int NM>
__device__ __forceinline__ void compute_stage(v16f (&acc)[2][2], const uint8_t* base, int wm, int brow0,
                                              int brow1) {
  using L = Lds<WF>;
  using BL = BLay<WF>;
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const uint8_t* As = base;
  const uint8_t* Bs = base + L::A;
  const uint32_t* SAs = (const uint32_t*)(base + L::A + L::B);
  const uint32_t* SBs = (const uint32_t*)(base + L::A + L::B + L::SA);
  v8i bv[2][2];
  uint32_t bsw[2];
  v8i av[2][NM];
  uint32_t asw[NM];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int jr = (n == 0 ? brow0 : brow1) + l32;
    bsw[n] = SBs[jr];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int blk = 2 * kk + g;
      if (WF == 1) {
        const uint4 v = *(const uint4*)(Bs + b4_off(jr, blk));
        bv[kk][n] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      } else {
        const uint8_t* rp = Bs + jr * BL::ROW + 24 * blk;
        if ((blk & 1) == 0) {
          const uint4 v = *(const uint4*)rp;
          const uint2 d = *(const uint2*)(rp + 16);
          bv[kk][n] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, (int)d.x, (int)d.y, 0, 0};
        } else {
          const uint2 d = *(const uint2*)rp;
          const uint4 v = *(const uint4*)(rp + 8);
          bv[kk][n] = (v8i){(int)d.x, (int)d.y, (int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0};
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int r = 32 * (wm + 4 * m) + l32;
    asw[m] = SAs[r];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 lo = *(const uint4*)(As + a_off(r, 4 * kk + g));
      const uint4 hi = *(const uint4*)(As + a_off(r, 4 * kk + 2 + g));
      av[kk][m] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int sh = 8 * (2 * kk + g);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int asc = (int)((asw[m] >> sh) & 0xffu);
#pragma unroll
      for (int n = 0; n < 2; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[kk][m], bv[kk][n], acc[m][n], 0,
                                                                    Fmt<WF>::MFMA, 0, asc, 0,
                                                                    (int)((bsw[n] >> sh) & 0xffu));
    }
  }
}

}  // namespace

template <bool FC1, int WF>
__global__ __launch_bounds__(kThreads, 1) void k_fc_tiled(FcArgs p) {
  using L = Lds<WF>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * L::STAGE];
  constexpr int D = copies_per_stage<WF>();

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int nk = p.K / TBK, NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + TBM - 1) / TBM : *p.num_tiles;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3, Q = gridDim.x >> 3;
  const int xt = ntiles > xcd ? (ntiles - xcd + 7) / 8 : 0;
  const int nitems = xt * NB;
  const int my_items = nitems > q ? (nitems - q + Q - 1) / Q : 0;
  const int total = my_items * nk;  // (item, stage) steps of this workgroup
  if (total == 0) return;
  const uint32_t lds0 = lds_addr(smem);

  // load cursor: item li (j = q + li*Q), stage ls
  int li = 0, ls = 0;
  LoadGeom<WF> lg;
  setup_loads<FC1, WF>(p, item_geom(p, xcd, q, NB), lg);
  auto issue_next = [&](int bufi) {
    issue_stage<WF>(lg, ls, lds0 + bufi * L::STAGE);
    if (++ls == nk) {
      ls = 0;
      if (++li < my_items) setup_loads<FC1, WF>(p, item_geom(p, xcd, q + li * Q, NB), lg);
    }
  };
  issue_next(0);
  if (total > 1) issue_next(1);

  // compute cursor
  int ci = 0, cs = 0;
  ItemGeom cit = item_geom(p, xcd, q, NB);
  int nm = (wm < ((cit.rows + 31) >> 5)) + (wm + 4 < ((cit.rows + 31) >> 5));
  v16f acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.f;

  // B-tile rows of this wave's two column tiles
  const int brow0 = FC1 ? 32 * wn : 64 * wn;
  const int brow1 = FC1 ? TBN / 2 + 32 * wn : 64 * wn + 32;

  auto epilogue = [&]() {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m >= nm) continue;
      const int sbk = wm + 4 * m;
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
          if (row < cit.rows) {
            const int64_t prow = cit.p0 + row;
            const int col0 = cit.nb * (TBN / 2) + 32 * wn;
            ((uint8_t*)p.out)[prow * p.N + col0 + l32] = (uint8_t)encode<3>(h * exp2_neg(sexp));
            if (l32 == 0) p.out_scale[prow * (p.N / 32) + col0 / 32] = (uint8_t)(sexp + 127);
          }
        } else {
          if (row < cit.rows) {
            // routed: row of the assignment (weight applied here, in fp32);
            // dense: row of the token
            const int prow = cit.p0 + row;
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
            float* o = p.obuf + orow * p.N + cit.nb * TBN + 64 * wn + l32;
            o[0] = w * acc[m][0][i];
            o[32] = w * acc[m][1][i];
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.f;
  };

  // One step: stage gidx is complete once this wave's copies for it have
  // landed (at most D younger copies -- the next stage's -- may remain) and
  // every wave has passed the barrier; then the stage after next is issued
  // into the buffer read in the previous step, and stage gidx is multiplied.
  int cur = 0;
  for (int gidx = 0; gidx < total; ++gidx) {
    if (gidx + 1 < total) wait_vm_lgkm0<D>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (gidx + 2 < total) issue_next(cur == 0 ? 2 : cur - 1);
    const uint8_t* base = smem + cur * L::STAGE;
    if (nm == 2) compute_stage<WF, 2>(acc, base, wm, brow0, brow1);
    else if (nm == 1) compute_stage<WF, 1>(acc, base, wm, brow0, brow1);
    cur = cur == 2 ? 0 : cur + 1;
    if (++cs == nk) {
      epilogue();
      // the epilogue's stores are younger than the copies in flight; drain
      // them so that the copy counts above stay exact
      wait_vm_lgkm0<0>();
      cs = 0;
      if (++ci < my_items) {
        cit = item_geom(p, xcd, q + ci * Q, NB);
        const int nsub = (cit.rows + 31) >> 5;
        nm = (wm < nsub) + (wm + 4 < nsub);
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
