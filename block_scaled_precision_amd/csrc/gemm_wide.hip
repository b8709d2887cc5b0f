// Grouped FC1 / FC2 GEMMs of the routed MoE layer for MXFP8 activations x
// MXFP4 (E2M1) weights, "wide" variant: 192 x 256 work items on the gfx950
// block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 (mxfp6-sm120 page,
// "Execution model": E4M3 activations and packed MX weights, each with one
// UE8M0 scale per 32 K values, block-scaled MMA with FP32 accumulation;
// TokenSpeed SiTU page, "Activation precision": MXFP8 activation x MXFP4
// weight).
//
// Work item = (M-tile, N-block).  An M-tile holds up to 192 permuted rows of one
// expert, so an expert with <= 192 assignments streams its weights from HBM
// once.  The N-block is 256 weight rows (FC1: 128 columns of h, i.e. 128 gate
// rows and the 128 matching up rows; FC2: 256 output columns).  The wide block
// halves how often an M-tile's activation rows are fetched from L2 (once per
// N-block) compared with 128-row blocks: for a prefill FC1 those re-reads are
// about three times the weight bytes and set the copy rate.  The grid is
// persistent: one workgroup per CU walks the items of its XCD (whole M-tiles
// x, x+8, ..., then an equal share of the N-blocks of the last ntiles % 8
// tiles), so the N-blocks of one M-tile run together on one XCD and its
// activation rows stay in that XCD's L2.  Items are consumed as one continuous
// stream of (item, 128-K step) steps with one workgroup barrier per step.
//
// Eight waves, two per SIMD, all multiply: wave (wm, wn) = (w % 4, w / 4)
// owns the 16-row sub-blocks wm, wm+4 and wm+8 of the tile (so the two waves
// of a SIMD share their activation rows and a partly filled tile still spreads
// over all SIMDs) and weight rows [128 wn, 128 wn + 128) of the block.  Each
// step multiplies fragments already held in registers while the fragments of
// the next step are read from LDS in between the MFMAs; the barrier at the top
// of step g certifies the stages of step g+1 and releases those of step g.
//
// The copies into LDS are global_load_lds (global memory straight into LDS)
// issued from inline assembly by the multiply waves themselves: waves with
// wn = 0 keep the activation ring (3 stages: gathered rows of E4M3 codes, 128 B
// per row and step, plus per-row scale words, and the row tables of the items
// ahead), waves with wn = 1 the weight ring (4 stages of 64 B per weight row
// plus scale words).  Each wave thus has one in-order stream of copies and
// waits for its own stage with an explicit vmcnt before the barrier.
//
// MFMA operand layouts (measured on the device): lane l supplies row l%16 of
// its operand and the scale of (row l%16, 32-k block l/16); an E4M3 lane holds
// k [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-k step (g = l/16), an
// E2M1 lane holds k [32g, 32g+32), i.e. bytes [16g, 16g+16) of the step's 64
// bytes of a weight row.  Accumulator element i of lane l is (row 4*(l/16) + i,
// column l%16).  The E2M1 operand is passed as 4 registers through the
// intrinsic's narrow overload.
#include <hip/hip_runtime.h>

#include "copy_ring.h"
#include "gemm.h"
#include "mx_device.h"
#include "wide_count.h"

namespace moe_mx {

typedef int v4i_w __attribute__((ext_vector_type(4)));

// Block-scaled MFMA 16x16x128, E4M3 A operand (8 registers) x E2M1 B operand (4
// registers: the intrinsic's own narrow overload).
__device__ v4f mfma16_f8_f4_w(v8i a, v4i_w b, v4f c, int fa, int fb, int opa, int sa, int opb, int sb)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v8i32.v4i32");

namespace {

typedef v4i_w v4i;

constexpr int TBM = kTiledRows;  // rows per M-tile (12 sub-blocks of 16)
constexpr int TBN = kWideCols;   // weight rows per work item (16 column tiles of 16)
constexpr int TBK = 128;         // K per step
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSubs = TBM / 16 / 4;  // 16-row sub-blocks per wave
constexpr int kTiles = TBN / 2 / 16; // column tiles per wave
static_assert(TBM == 192 && TBN == 256, "copy maps below assume 192 x 256 items");

// LDS layout: [A ring: 3 x codes TBM x 128 B] [B ring: 4 x codes TBN x 64 B]
//             [A scale groups: 2 x TBM x 16 B] [B scale groups: 2 x TBN x 16 B]
//             [row tables: 4 x (source row TBM x 4 B + weight TBM x 4 B)]
// Scales travel in groups of 4 K-steps: a row's 16 scale bytes for 4
// consecutive steps are contiguous in both operands, so one 16-byte copy per
// row serves 4 steps (per-step 4-byte copies cost as many memory requests as
// the codes themselves).
constexpr int kAStages = 3;
constexpr int kBStages = 4;
constexpr int kTables = 4;
constexpr int kGroup = kWideGroup;  // K-steps per scale group
// The row table of item i+1 is copied when item i's first stage is copied,
// kAStages steps before item i starts, into the buffer of item i+1-kTables,
// whose last reader is its epilogue at the end of item i+2-kTables: with items
// of at least 2 steps the copy comes after that epilogue.
static_assert((kTables - 2) * 2 >= kAStages, "row table ring too short");
constexpr int A_STAGE = TBM * TBK;
constexpr int B_ROW = TBK / 2;  // bytes of one E2M1 weight row per step
constexpr int B_STAGE = TBN * B_ROW;
constexpr int AS_GROUP = TBM * 4 * kGroup;
constexpr int BS_GROUP = TBN * 4 * kGroup;
constexpr int TABLE = TBM * 8;
constexpr int L_A = 0;
constexpr int L_B = L_A + kAStages * A_STAGE;
constexpr int L_AS = L_B + kBStages * B_STAGE;
constexpr int L_BS = L_AS + 2 * AS_GROUP;
constexpr int L_TBL = L_BS + 2 * BS_GROUP;
constexpr int L_TOTAL = L_TBL + kTables * TABLE;
static_assert(L_TOTAL <= 160 * 1024, "LDS");

// 1-KB code copies per wave and stage
constexpr int kACodeCopies = A_STAGE / 1024 / 4;
constexpr int kBCodeCopies = B_STAGE / 1024 / 4;

// A tile: row r holds 8 chunks of 16 B; chunk c sits at slot c ^ (r & 7), so
// that 8 consecutive rows read at the same k land in 8 different bank groups.
__device__ __forceinline__ int a_off(int r, int c) { return r * TBK + 16 * (c ^ (r & 7)); }
// B tile: row r holds 4 chunks of 16 B; chunk c sits at slot c ^ ((r >> 1) & 3)
// (rows are 64 B, so rows r and r+2 would otherwise share banks).
__device__ __forceinline__ int b_off(int r, int c) { return r * B_ROW + 16 * (c ^ ((r >> 1) & 3)); }

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
    g.p0 = TBM * ti;
    g.rows = min(TBM, p.dense_rows - TBM * ti);
  } else {
    const Tile t = load_tile(p.tiles, ti);
    g.expert = t.expert;
    g.p0 = t.p0;
    g.rows = t.rows;
  }
  return g;
}

// K step copied at step ls of an item: the steps run in K order, so the
// N-blocks of one M-tile, which run together on one XCD, read each activation
// stage at about the same time and one L2 fill serves them all.  (Starting
// each N-block at a different K step, which spreads the misses, measured
// slower with 256-row blocks and grouped scale copies.)
__device__ __forceinline__ int k_step(const Sched&, int, int ls) { return ls; }

// weight row held at B-tile row jr.  FC1: each half of the block (the rows of
// one wave) is 64 gate rows then the 64 matching up rows, so a wave holds both
// factors of its 64 h columns.
template <bool FC1>
__device__ __forceinline__ int64_t w_row(const FcArgs& p, int nb, int jr) {
  if (FC1) {
    const int half = jr >> 7, j = jr & 127;
    const int64_t col = (int64_t)nb * (TBN / 2) + 64 * half + (j & 63);
    return j < 64 ? col : (int64_t)p.N + col;
  }
  return (int64_t)nb * TBN + jr;
}

// ------------------------------------------------------------ copies ---

// Row table of an item (routed mode): the assignment id of each tile row (FC1:
// turned into the token of the activation row when read; FC2: the output row)
// and its routing weight.  Rows past the tile repeat its first row.  Every
// activation wave copies the ids (the same bytes to the same place), so each
// reads only what its own copies wrote; wave 0 also copies the weights, which
// are read by the epilogue, barriers later.
__device__ __forceinline__ void copy_table(const FcArgs& p, const ItemGeom& it, uint32_t tbl, bool weights) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < TBM / 64; ++t) {
    const int r = 64 * t + lane;
    const int prow = it.p0 + (r < it.rows ? r : 0);
    lds_copy4(p.sorted_assign + prow, tbl + 256 * t);
    if (weights) lds_copy4(p.sorted_w + prow, tbl + TBM * 4 + 256 * t);
  }
}

// Memory-counter bookkeeping of a copy stream: WideCopyCount (wide_count.h)
// gives, in closed form, how many copies may stay in flight before each
// barrier; its per-phase steady values are never looser than the exact count
// (checked here at compile time and, against a replay of the issue sequence,
// by a host program in the tests).  The last waits of a stream, from barrier
// total - kTailWaits on, wait for every copy.
constexpr int kTailWaits = kWideTailWaits;
static_assert(kTailWaits >= kAStages - 1 && kTailWaits >= kBStages - 1 && kGroup + 1 <= kTailWaits, "tail waits");

template <int NS, int C>
struct CopyCount : WideCopyCount<NS, C> {
  using W = WideCopyCount<NS, C>;
  static_assert(kGroup == 4 && W::steady_is_safe(), "per-phase waits");
  static __device__ __forceinline__ void wait_step(int g) {
    switch (g & (kGroup - 1)) {
      case 0: wait_vm_lgkm0<W::steady(0)>(); break;
      case 1: wait_vm_lgkm0<W::steady(1)>(); break;
      case 2: wait_vm_lgkm0<W::steady(2)>(); break;
      default: wait_vm_lgkm0<W::steady(3)>(); break;
    }
  }
};
// The activation stream of wave (wm, 0): codes of rows [48 wm, 48 wm + 48)
// (1-KB copy t = 6 wm + i holds rows 8t .. 8t+7, lane -> row 8t + lane/8,
// slot lane%8 receiving chunk (lane%8) ^ (row%8)), scale groups of rows
// 64 min(wm, 2) + lane (16 bytes per row: the 4 K-steps of the group), and
// the row tables.  A row table is read only after the per-step waits have
// covered the copy that wrote it: the table of item i goes out before item
// i-1's first code stage, which every wait from step nk*i - nk + 1 on includes.
template <bool FC1>
struct ACopier {
  using Count = CopyCount<kAStages, kACodeCopies>;
  uint32_t src[kACodeCopies];  // FC1 routed: byte offsets into the activations (< 4 GiB)
  int nb, p0, rows;            // the code cursor's item
  // Both streams advance one code stage / one scale group per call, so their
  // (item, step) cursors are counted instead of divided out of the step index.
  int cli = 0, cls = 0;        // code cursor: item, step within it
  int gli = 0, gls = 0;        // scale-group cursor: item, first step of the group
  int gitem = -1;              // item whose group source offsets are held below
  uint32_t goff;               // per-lane scale-row offset of that item
  int gnb;
  // FC1 gathers token rows through the row table (or, dense, rows p0 + r), and
  // keeps the per-lane row offsets for the item; FC2's tile row r is always
  // activation row p0 + r, so its offsets are recomputed at each issue (no
  // per-item registers)
  static constexpr bool kGather = FC1;

  // activation row (token for FC1, permuted row for FC2) of tile row r of item li
  __device__ __forceinline__ static uint32_t src_row(const FcArgs& p, const uint8_t* smem, const ItemGeom& it,
                                                     int li, int r) {
    r = r < it.rows ? r : it.rows - 1;  // rows past the tile repeat its last row
    if (p.dense_rows > 0) return (uint32_t)(it.p0 + r);
    const int32_t* tsrc = (const int32_t*)(smem + L_TBL + (li % kTables) * TABLE);
    if (!FC1) return (uint32_t)(it.p0 + r);
    return p.k == 1 ? (uint32_t)tsrc[r] : __umulhi((uint32_t)tsrc[r], p.kdiv);
  }

  // code stage of step s
  __device__ __forceinline__ void issue_code(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm, int s) {
    if (s >= sc.total) return;
    const int lane = threadIdx.x & 63;
    const uint32_t lds0 = lds_addr(smem);
    const int li = cli, ls = cls;
    if (++cls == sc.nk) {
      cls = 0;
      ++cli;
    }
    if (ls == 0) {
      // the next item's table goes out before this item's first stage
      if (p.dense_rows == 0 && li + 1 < sc.my_items)
        copy_table(p, item_geom(p, sc, li + 1), lds0 + L_TBL + ((li + 1) % kTables) * TABLE, wm == 0);
      const ItemGeom it = item_geom(p, sc, li);
      nb = it.nb;
      p0 = it.p0;
      rows = it.rows;
      if (kGather) {
        const int c = (lane & 7) ^ (lane >> 3);
#pragma unroll
        for (int i = 0; i < kACodeCopies; ++i)
          src[i] = src_row(p, smem, it, li, 8 * (kACodeCopies * wm + i) + (lane >> 3)) * (uint32_t)p.K + 16 * c;
      }
    }
    const int ks = k_step(sc, nb, ls);
    const uint8_t* a = (const uint8_t*)p.a + ks * TBK;
    const uint32_t base = lds0 + L_A + (s % kAStages) * A_STAGE;
    if (kGather) {
#pragma unroll
      for (int i = 0; i < kACodeCopies; ++i) lds_copy16_s(a, src[i], base + 1024 * (kACodeCopies * wm + i));
    } else {
      const uint32_t c16 = 16 * ((lane & 7) ^ (lane >> 3));
#pragma unroll
      for (int i = 0; i < kACodeCopies; ++i) {
        const int r = min(8 * (kACodeCopies * wm + i) + (lane >> 3), rows - 1);  // rows past the tile repeat its last row
        lds_copy16_s(a, (uint32_t)(p0 + r) * (uint32_t)p.K + c16, base + 1024 * (kACodeCopies * wm + i));
      }
    }
  }

  // scale group G (steps 4G .. 4G+3)
  __device__ __forceinline__ void issue_group(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm, int G) {
    if (kGroup * G >= sc.total) return;
    const int li = gli, ls = gls;
    gls += kGroup;
    if (gls == sc.nk) {
      gls = 0;
      ++gli;
    }
    const int u = min(wm, TBM / 64 - 1);
    if (li != gitem) {
      // a new item: its rows' scale offsets (the item's row table has landed:
      // it went out before the item's first code stage, which precedes this)
      const int lane = threadIdx.x & 63;
      const ItemGeom it = item_geom(p, sc, li);
      goff = src_row(p, smem, it, li, 64 * u + lane) * (uint32_t)(p.K / 32);
      gnb = it.nb;
      gitem = li;
    }
    lds_copy16_s(p.a_scale + 4 * k_step(sc, gnb, ls), goff, lds_addr(smem) + L_AS + (G % 2) * AS_GROUP + 1024 * u);
  }

  __device__ __forceinline__ void prologue(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm) {
    if (p.dense_rows == 0) {
      copy_table(p, item_geom(p, sc, 0), lds_addr(smem) + L_TBL, wm == 0);
      wait_vm_lgkm0<0>();
    }
    for (int s = 0; s < kAStages; ++s) issue_code(p, sc, smem, wm, s);
    issue_group(p, sc, smem, wm, 0);
    issue_group(p, sc, smem, wm, 1);
  }
  // after barrier g
  __device__ __forceinline__ void issue(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm, int g) {
    issue_code(p, sc, smem, wm, g + kAStages);
    if ((g & (kGroup - 1)) == kGroup - 1) issue_group(p, sc, smem, wm, (g + 1) / kGroup + 1);
  }
  __device__ __forceinline__ void wait_for(int g) { Count::wait_step(g); }
};

// The weight stream of wave (wm, 1): codes of B-tile rows [64 wm, 64 wm + 64)
// (1-KB copy t = 4 wm + i holds rows 16t .. 16t+15) and scale groups of rows
// 64 wm + lane.
template <bool FC1>
struct BCopier {
  using Count = CopyCount<kBStages, kBCodeCopies>;
  int nb, expert;  // of the code cursor's item; per-lane offsets are recomputed at each issue
  int cli = 0, cls = 0;  // code cursor: item, step within it (counted, as in ACopier)
  int gli = 0, gls = 0;  // scale-group cursor
  int gitem = -1;        // item whose scale-row base is held in gbase
  const uint8_t* gbase;

  // First weight row of the wave's 64 B-tile rows [64 wm, 64 wm + 64): FC1 takes
  // gate rows (even wm) or the matching up rows (odd wm) of h columns
  // nb*128 + 64 (wm/2) + [0, 64); FC2 takes output rows nb*256 + 64 wm + [0, 64).
  __device__ __forceinline__ static int64_t row0(const FcArgs& p, int nb_, int wm) {
    if (FC1) return (int64_t)nb_ * (TBN / 2) + 64 * (wm >> 1) + ((wm & 1) ? (int64_t)p.N : 0);
    return (int64_t)nb_ * TBN + 64 * wm;
  }

  __device__ __forceinline__ void issue_code(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm, int s) {
    if (s >= sc.total) return;
    const int lane = threadIdx.x & 63;
    const int li = cli, ls = cls;
    if (++cls == sc.nk) {
      cls = 0;
      ++cli;
    }
    if (ls == 0) {
      const ItemGeom it = item_geom(p, sc, li);
      nb = it.nb;
      expert = it.expert;
    }
    const int ks = k_step(sc, nb, ls);
    const uint8_t* w = p.w + (int64_t)expert * p.w_estride + row0(p, nb, wm) * (p.K / 2) + ks * B_ROW;
    // copy i: rows 16i + lane/4 of the wave's 64, slot lane%4 receiving chunk
    // (lane%4) ^ ((row/2)%4) = (lane%4) ^ ((lane/8)%4)
    const uint32_t lo = (uint32_t)(lane >> 2) * (uint32_t)(p.K / 2) + 16 * ((lane & 3) ^ ((lane >> 3) & 3));
    const uint32_t base = lds_addr(smem) + L_B + (s % kBStages) * B_STAGE;
#pragma unroll
    for (int i = 0; i < kBCodeCopies; ++i)
      lds_copy16_s(w, lo + (uint32_t)(16 * i) * (uint32_t)(p.K / 2), base + 1024 * (kBCodeCopies * wm + i));
  }

  __device__ __forceinline__ void issue_group(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm, int G) {
    if (kGroup * G >= sc.total) return;
    const int lane = threadIdx.x & 63;
    const int li = gli, ls = gls;
    gls += kGroup;
    if (gls == sc.nk) {
      gls = 0;
      ++gli;
    }
    if (li != gitem) {
      const ItemGeom it = item_geom(p, sc, li);
      gbase = p.w_scale + (int64_t)it.expert * p.ws_estride + row0(p, it.nb, wm) * (p.K / 32);
      gitem = li;
    }
    lds_copy16_s(gbase + 4 * ls, (uint32_t)lane * (uint32_t)(p.K / 32), lds_addr(smem) + L_BS + (G % 2) * BS_GROUP + 1024 * wm);
  }

  __device__ __forceinline__ void prologue(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm) {
    for (int s = 0; s < kBStages; ++s) issue_code(p, sc, smem, wm, s);
    issue_group(p, sc, smem, wm, 0);
    issue_group(p, sc, smem, wm, 1);
  }
  __device__ __forceinline__ void issue(const FcArgs& p, const Sched& sc, const uint8_t* smem, int wm, int g) {
    issue_code(p, sc, smem, wm, g + kBStages);
    if ((g & (kGroup - 1)) == kGroup - 1) issue_group(p, sc, smem, wm, (g + 1) / kGroup + 1);
  }
  __device__ __forceinline__ void wait_for(int g) { Count::wait_step(g); }
};

// ------------------------------------------------------------ epilogue ---

// ------------------------------------------------------------ multiply ---

// Operand fragments of one K-step for a wave: kSubs A sub-blocks and kTiles B
// column tiles, with the lane's scale byte of each.
struct Frags {
  v8i a[kSubs];
  int asc[kSubs];
  v4i b[kTiles];
  int bsc[kTiles];
};

// Per-lane LDS byte offsets of a wave's fragment reads, so that every read is
// this offset plus a compile-time constant (sub-block and column-tile offsets
// are multiples of 8 rows and leave the swizzles unchanged).
struct LaneOffs {
  int a_lo, a_hi, a_sc, b, b_sc;  // a_sc, b_sc: in a scale group buffer
};
__device__ __forceinline__ LaneOffs lane_offs(int wm, int wn) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int r = 16 * wm + l16, jr = 128 * wn + l16;
  LaneOffs o;
  o.a_lo = a_off(r, g);
  o.a_hi = a_off(r, 4 + g);
  o.a_sc = 4 * kGroup * r + g;
  o.b = b_off(jr, g);
  o.b_sc = 4 * kGroup * jr + g;
  return o;
}

// A sub-block m (rows 16 (wm + 4m) + l16), B column tile n (rows 128 wn + 16n + l16);
// `ass` / `bss` point at the step's scale words in its scale group buffer.
__device__ __forceinline__ void read_a(const uint8_t* as, const uint8_t* ass, const LaneOffs& o, int m, v8i& a,
                                       int& sc) {
  const int mo = 64 * m * TBK;
  const v4i lo = *(const v4i*)(as + o.a_lo + mo);
  const v4i hi = *(const v4i*)(as + o.a_hi + mo);
  a = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  sc = *(const uint8_t*)(ass + o.a_sc + 4 * kGroup * 64 * m);
}
__device__ __forceinline__ void read_b(const uint8_t* bs, const uint8_t* bss, const LaneOffs& o, int n, v4i& b,
                                       int& sc) {
  b = *(const v4i*)(bs + o.b + 16 * n * B_ROW);
  sc = *(const uint8_t*)(bss + o.b_sc + 4 * kGroup * 16 * n);
}

// One K-step for a wave holding NM (0 to kSubs) sub-blocks: the MFMAs of the
// fragments in `f`, column tile by column tile, with the reads of the next
// step's fragments (stages `nas`, `nbs`) placed between them: a column tile's
// B fragment is replaced right after its MFMAs, an A fragment right after its
// MFMA with the last column tile.
template <int NM>
__device__ __forceinline__ void mul_step(v4f (&acc)[kSubs][kTiles], Frags& f, const uint8_t* nas, const uint8_t* nbs,
                                         const uint8_t* nass, const uint8_t* nbss, const LaneOffs& o) {
#pragma unroll
  for (int n = 0; n < kTiles; ++n) {
#pragma unroll
    for (int m = 0; m < kSubs; ++m) {
      if (m < NM) acc[m][n] = mfma16_f8_f4_w(f.a[m], f.b[n], acc[m][n], 0, Fmt<1>::MFMA, 0, f.asc[m], 0, f.bsc[n]);
      if (n == kTiles - 1) read_a(nas, nass, o, m, f.a[m], f.asc[m]);
    }
    read_b(nbs, nbss, o, n, f.b[n], f.bsc[n]);
    // keep this order: the scheduler would otherwise hoist every read above
    // the MFMAs and need second register sets
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The nk steps of one item for a wave holding NM sub-blocks, from global step
// gbase.  Before barrier g the wave's own copies for step g+1 (code stage and,
// at a group start, scale group) have landed and its reads of step g's data
// are complete; after it, the wave copies its next stage into the buffer step g
// used (and, after a group's last step, the group after next into that group's
// buffer) and multiplies step g while reading step g+1's fragments (past the
// last step the reads hit a stale buffer and go unused).
template <int NM, class Copier>
__device__ __forceinline__ void item_steps(const FcArgs& p, const Sched& sc, v4f (&acc)[kSubs][kTiles], Frags& f,
                                           const LaneOffs& o, uint8_t* smem, Copier& cp, int wm, int gbase) {
  for (int s = 0; s < sc.nk; ++s) {
    const int g = gbase + s;
    if (g + kTailWaits < sc.total) cp.wait_for(g);
    else wait_vm_lgkm0<0>();
    barrier();
    cp.issue(p, sc, smem, wm, g);
    const int nx = g + 1;
    const int grp = (nx / kGroup) & 1, q = nx & (kGroup - 1);
    mul_step<NM>(acc, f, smem + L_A + (nx % kAStages) * A_STAGE, smem + L_B + (nx % kBStages) * B_STAGE,
                 smem + L_AS + grp * AS_GROUP + 4 * q, smem + L_BS + grp * BS_GROUP + 4 * q, o);
  }
}

template <bool FC1, int ACT, class Copier>
__device__ __forceinline__ void wave_main(const FcArgs& p, const Sched& sc, uint8_t* smem, int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  Copier cp;
  cp.prologue(p, sc, smem, wm);

  v4f acc[kSubs][kTiles];
#pragma unroll
  for (int m = 0; m < kSubs; ++m)
#pragma unroll
    for (int n = 0; n < kTiles; ++n) acc[m][n] = (v4f){0.f, 0.f, 0.f, 0.f};

  // sub-blocks wm, wm+4, wm+8 of a tile of `rows` rows that hold rows
  auto wave_subs = [&](int rows) { return max(0, (((rows + 15) >> 4) - wm + 3) / 4); };
  ItemGeom it = item_geom(p, sc, 0);
  int nm = wave_subs(it.rows);

  // step 0's fragments: its stages have landed at the first barrier
  Frags f;
  const LaneOffs o = lane_offs(wm, wn);
  wait_vm_lgkm0<0>();
  barrier();
#pragma unroll
  for (int n = 0; n < kTiles; ++n) read_b(smem + L_B, smem + L_BS, o, n, f.b[n], f.bsc[n]);
#pragma unroll
  for (int m = 0; m < kSubs; ++m) read_a(smem + L_A, smem + L_AS, o, m, f.a[m], f.asc[m]);

  int gbase = 0;
  for (int ci = 0; ci < sc.my_items; ++ci) {
    // one step loop per sub-block count, so that the accumulators stay in place
    switch (nm) {
      case 3: item_steps<3>(p, sc, acc, f, o, smem, cp, wm, gbase); break;
      case 2: item_steps<2>(p, sc, acc, f, o, smem, cp, wm, gbase); break;
      case 1: item_steps<1>(p, sc, acc, f, o, smem, cp, wm, gbase); break;
      default: item_steps<0>(p, sc, acc, f, o, smem, cp, wm, gbase); break;
    }
    gbase += sc.nk;

    // ---- epilogue of item ci ----
    const int32_t* tsrc = (const int32_t*)(smem + L_TBL + (ci % kTables) * TABLE);
    const float* twt = (const float*)(smem + L_TBL + (ci % kTables) * TABLE + TBM * 4);
#pragma unroll
    for (int m = 0; m < kSubs; ++m) {
      if (m >= nm) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * (wm + 4 * m) + 4 * g + i;
        if (FC1) {
          // h = SiLU(gate) * up: column tile n (< 4) holds gate columns, tile
          // n + 4 the matching up columns.  One E4M3 block per (row, 32
          // columns of h) = tiles 2b and 2b+1, with its E8M0 scale; the 16
          // lanes of a row are one DPP row.
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const float h0 = act_mul<ACT>(acc[m][2 * b][i], acc[m][2 * b + 4][i]);
            const float h1 = act_mul<ACT>(acc[m][2 * b + 1][i], acc[m][2 * b + 5][i]);
            const uint32_t mx = row16_max(max(__float_as_uint(h0) & 0x7fffffffu, __float_as_uint(h1) & 0x7fffffffu));
            const int sexp = block_exponent<3>(mx);
            const uint32_t codes = e4m3_pair(h0 * exp2_neg(sexp), h1 * exp2_neg(sexp));
            if (row < it.rows) {
              const int64_t prow = it.p0 + row;
              const int col0 = it.nb * (TBN / 2) + 64 * wn + 32 * b;
              uint8_t* out = (uint8_t*)p.out + prow * p.N + col0 + l16;
              out[0] = (uint8_t)codes;
              out[16] = (uint8_t)(codes >> 8);
              if (l16 == 0) p.out_scale[prow * (p.N / 32) + col0 / 32] = (uint8_t)(sexp + 127);
            }
          }
        } else if (row < it.rows) {
          // routed: row of the assignment, weight applied here in fp32;
          // dense: row of the token
          int64_t orow;
          float wt;
          if (p.dense_rows > 0) {
            orow = it.p0 + row;
            wt = p.dense_weight;
          } else {
            orow = tsrc[row];
            wt = twt[row];
          }
          uint16_t* out = p.obuf + orow * p.N + it.nb * TBN + 128 * wn + l16;
#pragma unroll
          for (int n = 0; n < kTiles; ++n) out[16 * n] = f32_to_bf16_rne(wt * acc[m][n][i]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kSubs; ++m)
#pragma unroll
      for (int n = 0; n < kTiles; ++n) acc[m][n] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (ci + 1 < sc.my_items) {
      it = item_geom(p, sc, ci + 1);
      nm = wave_subs(it.rows);
    }
  }
  wait_vm_lgkm0<0>();
}

template <bool FC1, int ACT>
__global__ __launch_bounds__(kThreads, 1) void k_fc_wide(FcArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L_TOTAL];
  Sched sc;
  sc.nk = p.K / TBK;
  sc.NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + TBM - 1) / TBM : *p.num_tiles;
  sc.xcd = blockIdx.x & 7;
  sc.q = blockIdx.x >> 3;
  sc.Q = gridDim.x >> 3;
  sc.full = ntiles / 8;
  const int tail_items = (ntiles % 8) * sc.NB;
  sc.tail0 = tail_items * sc.xcd / 8;
  const int nitems = sc.full * sc.NB + tail_items * (sc.xcd + 1) / 8 - sc.tail0;
  sc.my_items = nitems > sc.q ? (nitems - sc.q + sc.Q - 1) / sc.Q : 0;
  sc.total = sc.my_items * sc.nk;  // (item, step) steps of this workgroup
  if (sc.total == 0) return;
  // the wave index is uniform; saying so keeps everything derived from it
  // (copy cursors, sub-block counts, branches) in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w < 4) wave_main<FC1, ACT, ACopier<FC1>>(p, sc, smem, w, 0);
  else wave_main<FC1, ACT, BCopier<FC1>>(p, sc, smem, w - 4, 1);
}

}  // namespace

hipError_t launch_fc_wide(const FcArgs& p, bool fc1, int grid, hipStream_t st) {
  if (grid < 8) grid = 8;
  grid &= ~7;
  if (!fc1) k_fc_wide<false, MOE_FN_SILU><<<grid, kThreads, 0, st>>>(p);
  else if (p.act_fn == MOE_FN_RELU2) k_fc_wide<true, MOE_FN_RELU2><<<grid, kThreads, 0, st>>>(p);
  else if (p.act_fn == MOE_FN_SWIGLU_OAI) k_fc_wide<true, MOE_FN_SWIGLU_OAI><<<grid, kThreads, 0, st>>>(p);
  else k_fc_wide<true, MOE_FN_SILU><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe_mx
