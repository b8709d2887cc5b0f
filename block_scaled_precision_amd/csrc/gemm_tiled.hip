// Grouped FC1 / FC2 GEMMs of the routed MoE layer for MXFP8 activations,
// "tiled" variant: LDS-staged tiles on the gfx950 block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 (mxfp6-sm120 page, "Execution model":
// E4M3 activations and packed MX weights, each with one UE8M0 scale per 32 K
// values, block-scaled MMA with FP32 accumulation; TokenSpeed SiTU page,
// "Activation precision": MXFP8 activation x MXFP4 weight).
//
// Work item = (M-tile, N-block).  An M-tile holds up to TM permuted rows of one
// expert (TM = 192 or 128, the host's choice: 128 when the experts average at
// most 96 rows; for a dense expert, per GEMM), so an expert with <= TM
// assignments streams its weights from HBM exactly once.  With TM = 192 the
// N-block is TN = 128 weight rows (FC1: 64 gate rows and the 64 matching up
// rows, i.e. 64 columns of h; FC2: 128 output columns); with TM = 128 it is
// TN = 256: the activation stages are a third smaller, so each 128-K step (one
// barrier) can carry twice the weight bytes and twice the multiply work of the
// few rows an expert has.  The grid is
// persistent: one workgroup per CU walks the items of its XCD (whole M-tiles
// x, x+8, ..., then an equal share of the N-blocks of the last ntiles % 8
// tiles), so the N-blocks of one M-tile run together on one XCD and its
// activation rows stay in that XCD's L2.  Items are consumed as one
// continuous stream of (item, 128-K stage) steps with one workgroup barrier per
// step.
//
// Waves have fixed roles (12 waves, three per SIMD):
//  * waves 0-7 multiply: with WN = TN / 64 waves along N and WM = 8 / WN
//    along M, wave (wm, wn) = (w / WN, w % WN) owns the 32-row sub-blocks
//    wm, wm + WM, ... of the tile (so a partly filled tile still spreads over
//    all SIMDs) and two 32-column MFMA tiles (64 weight rows), reads its
//    operands from LDS and writes the item's results;
//  * waves 8-9 copy the activation stage (gathered rows of E4M3 codes, 128 B per
//    row and stage) into a ring of 4 LDS buffers (3 for E3M2 weights with
//    128-row tiles), all but one stage ahead of the multiply, and the rows'
//    scale words in groups of 4 stages;
//  * waves 10-11 copy the weight stage (64 B per row and stage for E2M1, 96 B
//    for E3M2) into a ring that takes the rest of the LDS (with 192-row tiles
//    6 buffers for E2M1, 4 for E3M2; with 128-row tiles and 256-row N-blocks
//    5 and 4) so that weights, which come from HBM, are requested further
//    ahead, and the rows' scale words in groups of 4 stages.
// The copies are global_load_lds (global memory straight into LDS) issued from
// inline assembly; each copy wave waits for its own stage with an explicit
// vmcnt before the barrier.  Because a wave's memory counter drains in order,
// the near (activation) and far (weight) streams live in different waves, and
// the multiply waves issue no loads at all: the per-row metadata of an item
// (source row, routing weight) is copied into LDS one item ahead by the
// activation waves.
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

#include "copy_ring.h"
#include "gemm.h"
#include "mx_device.h"
#include "tiled_count.h"

namespace moe_mx {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int TBK = 128;         // K per stage
constexpr int kComputeWaves = 8;  // multiply waves
constexpr int kWaves = kComputeWaves + 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveA = kComputeWaves;      // first activation-copy wave
constexpr int kWaveB = kComputeWaves + 2;  // first weight-copy wave

// Work item shape for M-tiles of TM rows: TN weight rows, and the grid of
// multiply waves (each holds 64 weight rows: two 32-column MFMA tiles)
template <int TM> struct Grid {
  static constexpr int TN = tiled_weight_rows(TM);
  static constexpr int WN = TN / 64;               // multiply waves along N
  static constexpr int WM = kComputeWaves / WN;    // multiply waves along M
  static constexpr int MAX_SUB = (TM / 32 + WM - 1) / WM;  // 32-row sub-blocks per multiply wave
};

// LDS layout: [A ring: STAGES x codes TM x 128 B] [B ring: NBS x weight codes]
//             [A scale groups: 2 x TM x 16 B] [B scale groups: 2 x TN x 16 B]
//             [row tables: TABLES x (source row TM x 4 B + weight TM x 4 B)]
// for M-tiles of TM rows (kTiledRows or kTiledRowsLow).  Scales travel in
// groups of 4 stages: the 16 scale bytes of a row for 4 consecutive stages
// are contiguous in both operands, so one 16-byte copy per row serves 4
// stages (a 4-byte copy per row and stage costs one memory request per row
// for 4 bytes, as many requests as the codes themselves).  K is a multiple of
// 512, so an item's steps fill whole groups.
template <int WF, int TM> struct ALay {
  static_assert(TM % 64 == 0 && TM <= 256, "tile rows");
  // E3M2 stages of 256 weight rows (24 KB) leave room for 3 activation stages
  static constexpr int STAGES = Grid<TM>::TN == 256 && WF == 2 ? 3 : 4;
  // The row table of item i+1 is copied with item i's first stage, STAGES - 1
  // steps before item i starts, into the buffer of item i+1-TABLES, whose last
  // reader is its epilogue at the end of item i+2-TABLES: with items of at
  // least 2 steps the copy comes after that epilogue.
  static constexpr int TABLES = 4;
  static_assert((TABLES - 2) * 2 >= STAGES, "row table ring too short");
  static constexpr int CODE_COPIES = TM / 16;  // 1-KB code copies per activation-copy wave and stage
  static constexpr int SCALE_CHUNKS = TM / 64;  // 1-KB copies (64 rows x 16 B) in a scale group
  static constexpr int GROUP_COPIES = (SCALE_CHUNKS + 1) / 2;  // per activation-copy wave and group
  static constexpr int STAGE = TM * TBK;
  static constexpr int GROUP = TM * 16;
  static constexpr int TABLE = TM * 8;
};
// The weight ring takes what the activation ring, the scale groups and the
// tables leave of the LDS (all of its 160 KB in every shape), so that as many
// weight stages (which come from HBM) as fit are in flight.
template <int WF, int TM> struct BLay {
  static constexpr int TN = Grid<TM>::TN;
  static constexpr int ROW = WF == 1 ? 64 : 96;    // bytes of one weight row per stage
  static constexpr int STAGE = TN * ROW;
  static constexpr int COPIES = STAGE / 1024;      // 1-KB copies per stage: 8, 12, 16 or 24
  static constexpr int PER_WAVE = COPIES / 2;      // per weight-copy wave
  static constexpr int GROUP = TN * 16;
  static constexpr int GROUP_COPIES = GROUP / 2048;  // 1-KB copies (64 rows) per weight-copy wave and group
  static constexpr int NBS = TM == kTiledRows ? (WF == 1 ? 6 : 4) : (WF == 1 ? 5 : 4);  // ring depth
  static_assert(COPIES % 2 == 0 && GROUP_COPIES * 2048 == GROUP, "copy split");
};
template <int WF, int TM> struct Lds {
  static constexpr int A = 0;
  static constexpr int B = ALay<WF, TM>::STAGES * ALay<WF, TM>::STAGE;
  static constexpr int AS = B + BLay<WF, TM>::NBS * BLay<WF, TM>::STAGE;
  static constexpr int BS = AS + 2 * ALay<WF, TM>::GROUP;
  static constexpr int TBL = BS + 2 * BLay<WF, TM>::GROUP;
  static constexpr int TOTAL = TBL + ALay<WF, TM>::TABLES * ALay<WF, TM>::TABLE;
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

// s_waitcnt vmcnt(n) lgkmcnt(0) for a run-time n in [LO, HI] (a compare ladder)
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n) {
  if constexpr (LO == HI) {
    wait_vm_lgkm0<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vm_range<LO, MID>(n);
    else wait_vm_range<MID + 1, HI>(n);
  }
}

// A tile: row r holds 8 chunks of 16 B; chunk c sits at slot c ^ (r & 7) so
// that 8 consecutive rows read at the same k land in 8 different bank groups.
__device__ __forceinline__ int a_off(int r, int c) { return r * TBK + 16 * (c ^ (r & 7)); }
// E2M1 B tile: 4 chunks per 64-B row, chunk c at slot c ^ ((r >> 1) & 3).
__device__ __forceinline__ int b4_off(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

struct ItemGeom {
  int expert, p0, rows, nb;
};

// Item list of one XCD: first the N-blocks of M-tiles xcd, xcd+8, ... for the
// 8*full leading tiles (whole tiles per XCD, so an M-tile's activation rows are
// shared in one L2), then an equal contiguous share [tail0, tail0 + ntail) of
// the N-blocks of the ntiles % 8 remaining tiles.
struct Sched {
  int xcd, full, tail0, q, Q, NB, nk, my_items, total;
};

template <int TM>
__device__ __forceinline__ ItemGeom item_geom(const FcArgs& p, const Sched& sc, int li) {
  const int j = sc.q + li * sc.Q;
  int ti;
  ItemGeom g;
  if (j < sc.full * sc.NB) {
    ti = sc.xcd + 8 * (j / sc.NB);
    g.nb = j % sc.NB;
  } else {
    const int u = sc.tail0 + j - sc.full * sc.NB;
    ti = 8 * sc.full + u / sc.NB;
    g.nb = u % sc.NB;
  }
  if (p.dense_rows > 0) {
    g.expert = 0;
    g.p0 = TM * ti;
    g.rows = min(TM, p.dense_rows - TM * ti);
  } else {
    const Tile t = load_tile(p.tiles, ti);
    g.expert = t.expert;
    g.p0 = t.p0;
    g.rows = t.rows;
  }
  return g;
}

// K stage copied at step ls of an item.  The N-blocks of one M-tile run at the
// same time on one XCD and read the same activation rows; starting each at a
// different K stage (rotated by its N-block index) means only the first to
// reach a stage misses in L2 and the others hit, instead of all of them
// waiting on the same miss.  The multiply is indifferent to the K order.  The
// rotation is a multiple of 4 stages, so a scale group's 4 steps are 4
// consecutive stages starting at a multiple of 4.
__device__ __forceinline__ int k_stage(const Sched& sc, int nb, int ls) {
  const int s = ls + ((nb * sc.nk / sc.NB) & ~3);
  return s < sc.nk ? s : s - sc.nk;
}

// weight row held at B-tile row jr of an N-block of TN rows
template <bool FC1, int TN>
__device__ __forceinline__ int64_t w_row(const FcArgs& p, int nb, int jr) {
  if (FC1) return jr < TN / 2 ? (int64_t)nb * (TN / 2) + jr : (int64_t)p.N + nb * (TN / 2) + jr - TN / 2;
  return (int64_t)nb * TN + jr;
}

// ------------------------------------------------------------ multiply ---

// One 128-K stage for a wave holding NM (1 to MAX_SUB) sub-blocks: sub-block
// wm + WM*m of the tile times the wave's two 32-column B tiles.  `ags`
// and `bgs` point at the stage's scale words in its scale group buffers (row
// r's word at 16 r).
template <int WF, int TM, int NM>
__device__ __forceinline__ void compute_stage(v16f (&acc)[Grid<TM>::MAX_SUB][2], const uint8_t* as, const uint8_t* bs,
                                              const uint8_t* ags, const uint8_t* bgs, int wm, int brow0, int brow1) {
  using BL = BLay<WF, TM>;
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  v8i bv[2][2];
  uint32_t bsw[2];
  v8i av[2][NM];
  uint32_t asw[NM];
  // scale words first, then the fragments of the first 64-K half, then the
  // second: the first half's MFMAs wait only for the reads issued before them
#pragma unroll
  for (int n = 0; n < 2; ++n) bsw[n] = *(const uint32_t*)(bgs + 16 * ((n == 0 ? brow0 : brow1) + l32));
#pragma unroll
  for (int m = 0; m < NM; ++m) asw[m] = *(const uint32_t*)(ags + 16 * (32 * (wm + Grid<TM>::WM * m) + l32));
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int blk = 2 * kk + g;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int jr = (n == 0 ? brow0 : brow1) + l32;
      if (WF == 1) {
        const uint4 v = *(const uint4*)(bs + b4_off(jr, blk));
        bv[kk][n] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      } else {
        const uint8_t* rp = bs + jr * BL::ROW + 24 * blk;
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
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int r = 32 * (wm + Grid<TM>::WM * m) + l32;
      const uint4 lo = *(const uint4*)(as + a_off(r, 4 * kk + g));
      const uint4 hi = *(const uint4*)(as + a_off(r, 4 * kk + 2 + g));
      av[kk][m] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
  // every fragment read of the stage is issued before the first MFMA (the
  // compiler would otherwise reuse one register set and wait between MFMAs)
  __builtin_amdgcn_sched_barrier(0);
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

template <bool FC1, int WF, int TM>
__device__ __forceinline__ void multiply_role(const FcArgs& p, const Sched& sc, uint8_t* smem) {
  using L = Lds<WF, TM>;
  using BL = BLay<WF, TM>;
  using AL = ALay<WF, TM>;
  using G = Grid<TM>;
  constexpr int kMaxSub = G::MAX_SUB;
  constexpr int TN = G::TN;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // (wm, wn) = (w / WN, w % WN), so the two multiply waves of a SIMD (w and
  // w + 4) hold different sub-blocks (TN = 128: {wm, wm + 4} and
  // {wm + 2, wm + 6}) or different rows of the same N-block (TN = 256:
  // sub-blocks {0, 2} and {1, 3}, so a 64-row tile keeps both busy)
  const int wm = wv / G::WN;
  const int wn = wv % G::WN;
  const int l32 = lane & 31, g = lane >> 5;
  const int brow0 = FC1 ? 32 * wn : 64 * wn;
  const int brow1 = FC1 ? TN / 2 + 32 * wn : 64 * wn + 32;

  v16f acc[kMaxSub][2];
#pragma unroll
  for (int m = 0; m < kMaxSub; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.f;

  // sub-blocks of this wave in a tile of `rows` rows
  auto wave_subs = [&](int rows) { return max(0, (((rows + 31) >> 5) - wm + G::WM - 1) / G::WM); };
  int ci = 0, cs = 0;
  ItemGeom it = item_geom<TM>(p, sc, 0);
  int nm = wave_subs(it.rows);
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_lgkm0();  // this wave's reads of the previous stage are done
    barrier();
    const uint8_t* as = smem + L::A + (gidx % AL::STAGES) * AL::STAGE;
    const uint8_t* bs = smem + L::B + (gidx % BL::NBS) * BL::STAGE;
    const int gb = (gidx >> 2) & 1, q = gidx & 3;
    const uint8_t* ags = smem + L::AS + gb * AL::GROUP + 4 * q;
    const uint8_t* bgs = smem + L::BS + gb * BL::GROUP + 4 * q;
    switch (nm) {
      case 4: if constexpr (kMaxSub >= 4) compute_stage<WF, TM, 4>(acc, as, bs, ags, bgs, wm, brow0, brow1); break;
      case 3: if constexpr (kMaxSub >= 3) compute_stage<WF, TM, 3>(acc, as, bs, ags, bgs, wm, brow0, brow1); break;
      case 2: if constexpr (kMaxSub >= 2) compute_stage<WF, TM, 2>(acc, as, bs, ags, bgs, wm, brow0, brow1); break;
      case 1: compute_stage<WF, TM, 1>(acc, as, bs, ags, bgs, wm, brow0, brow1); break;
      default: break;
    }
    if (++cs < sc.nk) continue;

    // ---- epilogue of item ci ----
    const int32_t* tsrc = (const int32_t*)(smem + L::TBL + (ci % AL::TABLES) * AL::TABLE);
    const float* twt = (const float*)(smem + L::TBL + (ci % AL::TABLES) * AL::TABLE + TM * 4);
#pragma unroll
    for (int m = 0; m < kMaxSub; ++m) {
      if (m >= nm) continue;
      const int sbk = wm + G::WM * m;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * sbk + 8 * (i >> 2) + 4 * g + (i & 3);
        if (FC1) {
          // h = SiLU(gate) * up for column nb*64 + 32*wn + l32, then one E4M3
          // block per (row, 32 columns) with its E8M0 scale
          const float h = gated_act(p.act_fn, acc[m][0][i], acc[m][1][i]);
          uint32_t mx = __float_as_uint(h) & 0x7fffffffu;
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
          const int sexp = block_exponent<3>(mx);
          if (row < it.rows) {
            const int64_t prow = it.p0 + row;
            const int col0 = it.nb * (TN / 2) + 32 * wn;
            ((uint8_t*)p.out)[prow * p.N + col0 + l32] = (uint8_t)encode<3>(h * exp2_neg(sexp));
            if (l32 == 0) p.out_scale[prow * (p.N / 32) + col0 / 32] = (uint8_t)(sexp + 127);
          }
        } else if (row < it.rows) {
          // routed: row of the assignment, weight applied here in fp32;
          // dense: row of the token
          int64_t orow;
          float w;
          if (p.dense_rows > 0) {
            orow = it.p0 + row;
            w = p.dense_weight;
          } else {
            orow = tsrc[row];
            w = twt[row];
          }
          uint16_t* o = p.obuf + orow * p.N + it.nb * TN + 64 * wn + l32;
          o[0] = f32_to_bf16_rne(w * acc[m][0][i]);
          o[32] = f32_to_bf16_rne(w * acc[m][1][i]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kMaxSub; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.f;
    cs = 0;
    if (++ci < sc.my_items) {
      it = item_geom<TM>(p, sc, ci);
      nm = wave_subs(it.rows);
    }
  }
}

// ----------------------------------------------------- activation copies ---

// Copies the row table of an item (routed mode): the assignment id of each
// tile row (FC1: turned into the token of the activation row when read; FC2:
// the output row) and its routing weight.  Rows past the tile repeat its first
// row.  Both activation waves copy the ids (the same bytes to the same place),
// so each reads only what its own copies wrote; the first also copies the
// weights, which only the multiply waves read, barriers later.
template <int TM>
__device__ __forceinline__ void copy_table(const FcArgs& p, const ItemGeom& it, uint32_t tbl) {
  const int lane = threadIdx.x & 63, aw = (threadIdx.x >> 6) - kWaveA;
#pragma unroll
  for (int t = 0; t < TM / 64; ++t) {
    const int r = 64 * t + lane;
    const int prow = it.p0 + (r < it.rows ? r : 0);
    lds_copy4(p.sorted_assign + prow, tbl + 256 * t);
    if (aw == 0) lds_copy4(p.sorted_w + prow, tbl + TM * 4 + 256 * t);
  }
}

template <bool FC1, int WF, int TM>
__device__ __forceinline__ void activation_role(const FcArgs& p, const Sched& sc, uint8_t* smem) {
  using L = Lds<WF, TM>;
  using AL = ALay<WF, TM>;
  constexpr int kACodeCopies = AL::CODE_COPIES;
  constexpr int kGC = AL::GROUP_COPIES;
  constexpr int kMaxWait = (AL::STAGES - 1) * kACodeCopies + 2 * kGC;
  static_assert(kMaxWait < 64, "vmcnt range");
  const int lane = threadIdx.x & 63, aw = (threadIdx.x >> 6) - kWaveA;
  const int K = p.K;
  const bool routed = p.dense_rows == 0;
  const uint32_t lds0 = lds_addr(smem);
  const int c = (lane & 7) ^ (lane >> 3);  // chunk that lands in this lane's LDS slot
  const TiledCopyCount<AL::STAGES, kACodeCopies, kGC> cnt{sc.total, sc.total / 4};

  // activation row (token for FC1, permuted row for FC2) of tile row r of
  // item li, whose row table must have landed
  auto src_row = [&](const ItemGeom& it, int li, int r) -> int64_t {
    r = r < it.rows ? r : it.rows - 1;  // rows past the tile repeat its last row
    if (!routed) return it.p0 + r;
    const int32_t* tsrc = (const int32_t*)(smem + L::TBL + (li % AL::TABLES) * AL::TABLE);
    return FC1 ? tsrc[r] / p.k : (int64_t)it.p0 + r;
  };

  const uint8_t* asrc[kACodeCopies];
  int load_nb = 0;
  int li = 0, ls = 0, issued = 0;  // code cursor: item, step within it; stages issued
  int gli = 0, gls = 0;            // group cursor: item, first step of the group
  const uint8_t* gsrc[kGC];        // the group cursor's item: per-lane scale rows
  int gnb = 0;
  // the next code stage; at the start of an item, first copy the row table of
  // the item after it (older than the stage's copies, so the wait for the
  // stage covers it; tables 0 and 1 go out in the prologue)
  auto issue_stage = [&]() {
    if (ls == 0) {
      if (routed && li > 0 && li + 1 < sc.my_items)
        copy_table<TM>(p, item_geom<TM>(p, sc, li + 1), lds0 + L::TBL + ((li + 1) % AL::TABLES) * AL::TABLE);
      // item li's table went out with the first stage of item li-1, at least
      // nk >= STAGES - 1 stages before the one the last wait covered
      const ItemGeom it = item_geom<TM>(p, sc, li);
      load_nb = it.nb;
#pragma unroll
      for (int i = 0; i < kACodeCopies; ++i)
        asrc[i] = (const uint8_t*)p.a + src_row(it, li, 8 * (kACodeCopies * aw + i) + (lane >> 3)) * K + 16 * c;
    }
    const int ks = k_stage(sc, load_nb, ls);
    const uint32_t base = lds0 + L::A + (issued % AL::STAGES) * AL::STAGE;
#pragma unroll
    for (int i = 0; i < kACodeCopies; ++i) lds_copy16(asrc[i] + ks * TBK, base + 1024 * (kACodeCopies * aw + i));
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  // scale group G: 16 bytes per row (the 4 stages from the group's first K
  // stage) in 64-row chunks; wave aw copies chunks kGC*aw .. kGC*aw + kGC - 1
  // (a missing one repeats the last: the same bytes to the same place).  The
  // group opening item li is copied 4 steps before it, after the wait that
  // covers the stage copied with item li's row table.
  auto issue_group = [&](int G) {
    if (gls == 0) {
      const ItemGeom it = item_geom<TM>(p, sc, gli);
      gnb = it.nb;
#pragma unroll
      for (int i = 0; i < kGC; ++i)
        gsrc[i] = p.a_scale + src_row(it, gli, 64 * min(kGC * aw + i, AL::SCALE_CHUNKS - 1) + lane) * (K / 32);
    }
    const int ks = k_stage(sc, gnb, gls);
    const uint32_t base = lds0 + L::AS + (G & 1) * AL::GROUP;
#pragma unroll
    for (int i = 0; i < kGC; ++i)
      lds_copy16(gsrc[i] + 4 * ks, base + 1024 * min(kGC * aw + i, AL::SCALE_CHUNKS - 1));
    gls += 4;
    if (gls == sc.nk) {
      gls = 0;
      ++gli;
    }
  };

  if (routed) {
    copy_table<TM>(p, item_geom<TM>(p, sc, 0), lds0 + L::TBL);
    if (sc.my_items > 1) copy_table<TM>(p, item_geom<TM>(p, sc, 1), lds0 + L::TBL + AL::TABLE);
    wait_vm_lgkm0<0>();
  }
  for (int G = 0; G < 2 && G < cnt.ngroups; ++G) issue_group(G);
  for (int s = 0; s < AL::STAGES - 1 && s < sc.total; ++s) issue_stage();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_vm_range<0, kMaxWait>(min(cnt.allowed(gidx), kMaxWait));
    barrier();
    if (gidx >= 4 && (gidx & 3) == 0 && (gidx >> 2) + 1 < cnt.ngroups) issue_group((gidx >> 2) + 1);
    if (issued < sc.total) issue_stage();
  }
}

// --------------------------------------------------------- weight copies ---

template <bool FC1, int WF, int TM>
__device__ __forceinline__ void weight_role(const FcArgs& p, const Sched& sc, uint8_t* smem) {
  using L = Lds<WF, TM>;
  using BL = BLay<WF, TM>;
  constexpr int TN = BL::TN;
  constexpr int kGC = BL::GROUP_COPIES;
  constexpr int kMaxWait = (BL::NBS - 1) * BL::PER_WAVE + 2 * kGC;
  static_assert(kMaxWait < 64, "vmcnt range");
  const int lane = threadIdx.x & 63, bw = (threadIdx.x >> 6) - kWaveB;
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const int64_t wrow = (int64_t)K * Fmt<WF>::BITS / 8;
  const TiledCopyCount<BL::NBS, BL::PER_WAVE, kGC> cnt{sc.total, sc.total / 4};

  const uint8_t* bsrc[BL::PER_WAVE];
  int load_nb = 0;
  auto setup = [&](int li) {
    const ItemGeom it = item_geom<TM>(p, sc, li);
    load_nb = it.nb;
    const uint8_t* wb = p.w + (int64_t)it.expert * p.w_estride;
#pragma unroll
    for (int i = 0; i < BL::PER_WAVE; ++i) {
      const int t = BL::PER_WAVE * bw + i;  // 1-KB copy index within the stage
      int jr, ch;
      if (WF == 1) {
        jr = 16 * t + (lane >> 2);
        ch = (lane & 3) ^ ((jr >> 1) & 3);
      } else {
        const int cc = 64 * t + lane;
        jr = cc / 6;
        ch = cc % 6;
      }
      bsrc[i] = wb + w_row<FC1, TN>(p, it.nb, jr) * wrow + 16 * ch;
    }
  };
  int li = 0, ls = 0, issued = 0;  // code cursor
  int gli = 0, gls = 0;            // group cursor
  const uint8_t* gsrc[kGC];        // the group cursor's item: per-lane scale rows
  int gnb = 0;
  auto issue_stage = [&]() {
    if (ls == 0) setup(li);
    const uint32_t base = lds0 + L::B + (issued % BL::NBS) * BL::STAGE;
    const int ks = k_stage(sc, load_nb, ls);
    const int bo = ks * (TBK * Fmt<WF>::BITS / 8);
#pragma unroll
    for (int i = 0; i < BL::PER_WAVE; ++i) lds_copy16(bsrc[i] + bo, base + 1024 * (BL::PER_WAVE * bw + i));
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  // scale group G: 16 bytes (4 stages) of weight rows 64 (kGC bw + i) + lane
  auto issue_group = [&](int G) {
    if (gls == 0) {
      const ItemGeom it = item_geom<TM>(p, sc, gli);
      gnb = it.nb;
#pragma unroll
      for (int i = 0; i < kGC; ++i)
        gsrc[i] = p.w_scale + (int64_t)it.expert * p.ws_estride +
                  w_row<FC1, TN>(p, it.nb, 64 * (kGC * bw + i) + lane) * (K / 32);
    }
    const int ks = k_stage(sc, gnb, gls);
#pragma unroll
    for (int i = 0; i < kGC; ++i)
      lds_copy16(gsrc[i] + 4 * ks, lds0 + L::BS + (G & 1) * BL::GROUP + 1024 * (kGC * bw + i));
    gls += 4;
    if (gls == sc.nk) {
      gls = 0;
      ++gli;
    }
  };
  for (int G = 0; G < 2 && G < cnt.ngroups; ++G) issue_group(G);
  for (int s = 0; s < BL::NBS - 1 && s < sc.total; ++s) issue_stage();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_vm_range<0, kMaxWait>(min(cnt.allowed(gidx), kMaxWait));
    barrier();
    if (gidx >= 4 && (gidx & 3) == 0 && (gidx >> 2) + 1 < cnt.ngroups) issue_group((gidx >> 2) + 1);
    if (issued < sc.total) issue_stage();
  }
}

}  // namespace

// DENSE: the launch is a dense expert (p.dense_rows > 0).  The code is the
// same; the separate instantiation keeps the routed and dense launches apart
// in kernel traces.
template <bool FC1, int WF, int TM, bool DENSE>
__global__ __launch_bounds__(kThreads, 1) void k_fc_tiled(FcArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Lds<WF, TM>::TOTAL];
  Sched sc;
  sc.nk = p.K / TBK;
  sc.NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + TM - 1) / TM : *p.num_tiles;
  sc.xcd = blockIdx.x & 7;
  sc.q = blockIdx.x >> 3;
  sc.Q = gridDim.x >> 3;
  sc.full = ntiles / 8;
  const int tail_items = (ntiles % 8) * sc.NB;
  sc.tail0 = tail_items * sc.xcd / 8;
  const int nitems = sc.full * sc.NB + tail_items * (sc.xcd + 1) / 8 - sc.tail0;
  sc.my_items = nitems > sc.q ? (nitems - sc.q + sc.Q - 1) / sc.Q : 0;
  sc.total = sc.my_items * sc.nk;  // (item, stage) steps of this workgroup
  if (sc.total == 0) return;
  const int wv = threadIdx.x >> 6;
  if (wv < kComputeWaves) multiply_role<FC1, WF, TM>(p, sc, smem);
  else if (wv < kWaveB) activation_role<FC1, WF, TM>(p, sc, smem);
  else weight_role<FC1, WF, TM>(p, sc, smem);
}

template <bool FC1, int WF>
static hipError_t launch_tiled_t(const FcArgs& p, int rows, int grid, hipStream_t st) {
  const bool dense = p.dense_rows > 0;
  if (rows == kTiledRowsLow) {
    if (dense) k_fc_tiled<FC1, WF, kTiledRowsLow, true><<<grid, kThreads, 0, st>>>(p);
    else k_fc_tiled<FC1, WF, kTiledRowsLow, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (dense) k_fc_tiled<FC1, WF, kTiledRows, true><<<grid, kThreads, 0, st>>>(p);
    else k_fc_tiled<FC1, WF, kTiledRows, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_fc_tiled(const FcArgs& p, bool fc1, int wfmt, int rows, int grid, hipStream_t st) {
  if (rows != kTiledRows && rows != kTiledRowsLow) return hipErrorInvalidValue;
  if (grid < 8) grid = 8;
  grid &= ~7;
  if (fc1) return wfmt == 1 ? launch_tiled_t<true, 1>(p, rows, grid, st) : launch_tiled_t<true, 2>(p, rows, grid, st);
  return wfmt == 1 ? launch_tiled_t<false, 1>(p, rows, grid, st) : launch_tiled_t<false, 2>(p, rows, grid, st);
}

}  // namespace moe_mx
