// Grouped FC1 / FC2 GEMMs of the routed MoE layer for bf16 activations and
// E2M1 weights ("w4a16": TokenSpeed SiTU page, "Activation precision") when
// the local experts see many rows each, as under skewed routing where a few
// experts take most assignments.  The 16-row small-M kernel streams an
// expert's whole weight matrix once per 16 rows; here an M-tile holds up to
// 64 rows and an N-block 256 weight rows, so weights are re-read once per 64
// rows and activation rows once per 256 weight rows, cutting the traffic the
// caches serve about threefold.  M-tiles still follow each expert's own row
// count (one partial tile per expert), the persistent grid walks them as they
// come from the tile list, and the weights stay packed in the mainloop
// (mxfp6-sm120 page, "Execution model").
//
// Work item = (M-tile of one expert, N-block of 256 weight rows: FC1 128 gate
// + 128 up rows, i.e. 128 columns of h; FC2 256 output columns).  Per 128-K
// stage the weight tile (256 rows x 64 B of E2M1 codes) and the activation
// tile (64 rows x 256 B of bf16) are copied global -> LDS into a ring of 4
// stage buffers (3 stages in flight).  The E8M0 weight scales travel in
// groups of 4 stages (16 contiguous bytes per row), one copy per row and group.
//
// Waves (8): 0-3 multiply, 4-5 copy weights (8 code copies per stage each,
// plus 2 scale copies at the start of a group), 6-7 copy activations (8 per
// stage each).  Multiply wave w owns rows [32*(w>>1), +32) (two 16-row
// sub-tiles) and half of the N-block's column tiles; it dequantizes each
// weight column tile once per stage (v_cvt_scalef32_pk_bf16_fp4, exact for
// E8M0 scales) and feeds it to both row sub-tiles, i.e. two conversions per
// MFMA.  A wave whose rows lie past the tile skips its MFMAs for that item.
//
// MFMA: v_mfma_f32_16x16x32_bf16 (lane l supplies row l%16 and 8 consecutive
// k-slots 8*(l/16) .. +8; accumulator element i of lane l is (row 4*(l/16)+i,
// column l%16)).  Lane group g = l/16 takes the actual k range [32g, 32g + 32)
// of the stage, 8 values per MFMA step: one MX block of weight codes (16 B,
// one scale byte) and a 64-B activation run.
#include <hip/hip_runtime.h>

#include "copy_ring.h"
#include "gemm.h"
#include "mx_device.h"

namespace moe_mx {

namespace {

constexpr int MBN = kWideCols;  // weight rows per item
constexpr int MBK = 128;        // K per stage
constexpr int GS = 4;           // stages per scale group
constexpr int NG = 2;           // scale-group buffers
constexpr int B_ROW = MBK / 2;  // 64 B of codes per weight row and stage
constexpr int A_ROW = MBK * 2;  // 256 B of bf16 per activation row and stage
constexpr int S_B = MBN * B_ROW;
constexpr int SROW = MBK / 32;       // scale bytes per row and stage
constexpr int GROW = SROW * GS;      // scale bytes per row and group
constexpr int G_BYTES = MBN * GROW;  // one scale-group buffer
constexpr int kBCopies = S_B / 1024 / 2;      // 1-KB code copies per weight wave and stage
constexpr int kGCopies = G_BYTES / 1024 / 2;  // 1-KB scale copies per weight wave and group
static_assert(MBK * 4 == kMidK, "the host checks K divisibility against kMidK");
static_assert(kBCopies * 2048 == S_B && kGCopies * 2048 == G_BYTES, "copy split");

// Layout for M-tiles of TM rows (kMidRows or kMidRowsHigh): TM / 16 multiply
// waves (TM / 32 row groups x 2 column halves), then 2 weight-copy and 2
// activation-copy waves; a ring of NSTG stages [weights | activations] and
// the scale-group ring.
template <int TM> struct ML {
  static constexpr int NSTG = TM == kMidRows ? 4 : 3;
  static constexpr int S_A = TM * A_ROW;
  static constexpr int S_STAGE = S_B + S_A;
  static constexpr int L_SG = NSTG * S_STAGE;
  static constexpr int L_TOTAL = L_SG + NG * G_BYTES;
  static constexpr int MUL_WAVES = TM / 16;
  static constexpr int THREADS = 64 * (MUL_WAVES + 4);
  static constexpr int A_COPIES = S_A / 1024 / 2;  // 1-KB copies per activation wave and stage
  static constexpr int A_ROWS = TM / 2;            // tile rows per activation wave
  static_assert(A_COPIES * 2048 == S_A && 4 * A_COPIES == A_ROWS, "copy split");
  static_assert(L_TOTAL <= 160 * 1024, "LDS");
  // Group G (stages GS*G ..) is copied just before the codes of its first
  // stage, into buffer G % NG, whose previous group was last read at stage
  // GS*(G-NG) + GS - 1; stage GS*G is copied after barrier GS*G - NSTG + 1.
  static_assert(GS * (NG - 1) >= NSTG - 1, "scale-group ring too short");
};

// weight tile: row r holds 4 chunks of 16 B; chunk c sits at slot c ^ ((r >> 1) & 3)
__device__ __forceinline__ int mb_off(int r, int c) { return r * B_ROW + 16 * (c ^ ((r >> 1) & 3)); }
// activation tile: row r holds 16 chunks of 16 B (8 bf16); chunk c at slot c ^ (r & 7)
__device__ __forceinline__ int ma_off(int r, int c) { return r * A_ROW + 16 * (c ^ (r & 7)); }

struct MGeom {
  int expert, p0, rows, nb;
};

// Item list of one XCD: the M-tiles go to the XCDs in groups of G consecutive
// tiles (group i to XCD i % 8), all N-blocks of a tile on one XCD, so its
// activation rows are shared in one L2; G is about the number of tiles whose
// items the XCD's workgroups hold at once, so that consecutive tiles of one
// expert run together and share its weight N-blocks in L2 too.  The tiles
// past the last whole round of 8 groups are split as items: each XCD takes an
// equal contiguous share of their N-blocks.
struct MSched {
  int xcd, G, full, tail0, q, Q, NB, nk, my_items, total;
};

template <int TM>
__device__ __forceinline__ MGeom m_geom(const FcArgs& p, const MSched& sc, int li) {
  const int j = sc.q + li * sc.Q;
  int ti;
  MGeom g;
  if (j < sc.full * sc.G * sc.NB) {
    const int idx = j / sc.NB;  // tile of this XCD's list
    ti = (idx / sc.G) * 8 * sc.G + sc.xcd * sc.G + idx % sc.G;
    g.nb = j % sc.NB;
  } else {
    const int u = sc.tail0 + j - sc.full * sc.G * sc.NB;
    ti = 8 * sc.G * sc.full + u / sc.NB;
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

// weight row (within the expert's matrix) of row jr of N-block nb
template <bool FC1>
__device__ __forceinline__ int64_t m_wrow(const FcArgs& p, int nb, int jr) {
  if (FC1) return jr < MBN / 2 ? (int64_t)nb * (MBN / 2) + jr : (int64_t)p.N + nb * (MBN / 2) + jr - MBN / 2;
  return (int64_t)nb * MBN + jr;
}

// s_waitcnt vmcnt(n) lgkmcnt(0) for a run-time n in [LO, HI] (n above HI waits
// for HI, which is stricter)
template <int LO, int HI>
__device__ __forceinline__ void wait_n(int n) {
  if constexpr (LO == HI) {
    wait_vm_lgkm0<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_n<MID, HI>(n);
    else wait_n<LO, MID - 1>(n);
  }
}

// ------------------------------------------------------------ multiply ---

// B-tile row of column tile n (0..7) of the wave in column half wc: FC1 tiles
// 0-3 are gate rows and 4-7 the up rows of the same 64 h columns
template <bool FC1>
__device__ __forceinline__ int m_btile(int wc, int n) {
  if (FC1) return n < 4 ? 64 * wc + 16 * n : MBN / 2 + 64 * wc + 16 * (n - 4);
  return 128 * wc + 16 * n;
}

// one stage of one multiply wave: acc[m][n] += A(sub-tile m) * B(column tile n)^T
template <bool FC1>
__device__ __forceinline__ void m_stage(const uint8_t* st, const uint8_t* sg, int wr, int wc, int r16, int g,
                                        v4f (&acc)[2][8]) {
  const uint8_t* as = st + S_B;
  uint4 a[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int ar = 32 * wr + 16 * m + r16;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) a[m][kq] = *(const uint4*)(as + ma_off(ar, 4 * g + kq));
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int jr = m_btile<FC1>(wc, n) + r16;
    const uint4 b = *(const uint4*)(st + mb_off(jr, g));
    const float s = e8m0_to_f32(sg[GROW * jr]);
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const v2bf q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], s, 0);
      const v2bf q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], s, 1);
      const v2bf q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], s, 2);
      const v2bf q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], s, 3);
      const v8bf bv = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        v8bf av;
        __builtin_memcpy(&av, &a[m][kq], 16);
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[m][n], 0, 0, 0);
      }
    }
  }
}

template <bool FC1, int TM>
__device__ __forceinline__ void mid_multiply(const FcArgs& p, const MSched& sc, uint8_t* smem, int w) {
  using L = ML<TM>;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = w >> 1, wc = w & 1;
  v4f acc[2][8];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[m][n] = (v4f){0.f, 0.f, 0.f, 0.f};
  int ci = 0, cs = 0;
  MGeom it = m_geom<TM>(p, sc, 0);
  // routed FC2: the lane's row metadata for the item (output row and routing
  // weight of rows 32 wr + 16 m + 4 g + i), loaded when the item starts so
  // that the epilogue does not wait for it (rows past the tile read row 0)
  int m_row[2][4];
  float m_wt[2][4];
  auto load_meta = [&]() {
    if (!FC1 && p.dense_rows == 0) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 32 * wr + 16 * m + 4 * g + i;
          const int64_t pr = it.p0 + (row < it.rows ? row : 0);
          m_row[m][i] = p.sorted_assign[pr];
          m_wt[m][i] = p.sorted_w[pr];
        }
    }
  };
  load_meta();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_lgkm0();
    barrier();
    if (it.rows > 32 * wr) {
      const uint8_t* st = smem + (gidx % L::NSTG) * L::S_STAGE;
      // scale byte of row jr, this stage, MX block g: sg[GROW * jr]
      const uint8_t* sg = smem + L::L_SG + ((gidx / GS) % NG) * G_BYTES + (gidx % GS) * SROW + g;
      m_stage<FC1>(st, sg, wr, wc, r16, g, acc);
    }
    if (++cs < sc.nk) continue;

    // ---- epilogue: lane holds rows 32wr + 16m + 4g + i, column r16 of each tile ----
    if (it.rows > 32 * wr) {
      if (FC1) {
        uint16_t* out = (uint16_t*)p.out;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 32 * wr + 16 * m + 4 * g + i;
            if (row < it.rows) {
              uint16_t* o = out + (int64_t)(it.p0 + row) * p.N + it.nb * (MBN / 2) + 64 * wc + r16;
#pragma unroll
              for (int n = 0; n < 4; ++n) o[16 * n] = f32_to_bf16_rne(gated_act(p.act_fn, acc[m][n][i], acc[m][n + 4][i]));
            }
          }
      } else {
        // row metadata by plain per-lane loads (the multiply waves issue no
        // copies, so their memory counter holds nothing else)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 32 * wr + 16 * m + 4 * g + i;
            if (row < it.rows) {
              int64_t orow = it.p0 + row;
              float wt = p.dense_weight;
              if (p.dense_rows == 0) {
                orow = m_row[m][i];
                wt = m_wt[m][i];
              }
              uint16_t* o = p.obuf + orow * p.N + it.nb * MBN + 128 * wc + r16;
#pragma unroll
              for (int n = 0; n < 8; ++n) o[16 * n] = f32_to_bf16_rne(wt * acc[m][n][i]);
            }
          }
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[m][n] = (v4f){0.f, 0.f, 0.f, 0.f};
    cs = 0;
    if (++ci < sc.my_items) {
      it = m_geom<TM>(p, sc, ci);
      load_meta();
    }
  }
}

// -------------------------------------------------------- weight copies ---

template <bool FC1, int TM>
__device__ __forceinline__ void mid_weights(const FcArgs& p, const MSched& sc, uint8_t* smem, int bw) {
  using L = ML<TM>;
  const int lane = threadIdx.x & 63;
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const int64_t wrow = (int64_t)K / 2;
  const uint8_t* src[kBCopies];
  const uint8_t* ssrc[kGCopies];
  auto setup = [&](int li) {
    const MGeom it = m_geom<TM>(p, sc, li);
    const uint8_t* wb = p.w + (int64_t)it.expert * p.w_estride;
    const uint8_t* sb = p.w_scale + (int64_t)it.expert * p.ws_estride;
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) {
      // copy t lands rows 16t .. 16t + 15, four 16-B slots per row
      const int t = kBCopies * bw + i;
      const int jr = 16 * t + lane / 4;
      const int ch = (lane % 4) ^ ((jr >> 1) & 3);
      src[i] = wb + m_wrow<FC1>(p, it.nb, jr) * wrow + 16 * ch;
    }
#pragma unroll
    for (int i = 0; i < kGCopies; ++i) {
      // scale copy s lands rows 64s .. 64s + 63, 16 B (4 stages) per row
      const int jr = 64 * (kGCopies * bw + i) + lane;
      ssrc[i] = sb + m_wrow<FC1>(p, it.nb, jr) * (K / 32);
    }
  };
  int li = 0, ls = 0, issued = 0;
  auto issue_next = [&]() {
    if (ls == 0) setup(li);
    // the scale group first: the wait for its first stage then covers it
    if (issued % GS == 0) {
      const uint32_t gb = lds0 + L::L_SG + ((issued / GS) % NG) * G_BYTES;
#pragma unroll
      for (int i = 0; i < kGCopies; ++i) lds_copy16(ssrc[i] + ls * SROW, gb + 1024 * (kGCopies * bw + i));
    }
    const uint32_t base = lds0 + (issued % L::NSTG) * L::S_STAGE;
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) lds_copy16(src[i] + ls * B_ROW, base + 1024 * (kBCopies * bw + i));
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  for (int s = 0; s < L::NSTG - 1 && s < sc.total; ++s) issue_next();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    // stage gidx (and its group, copied before it) has landed once at most the
    // copies of the stages issued after it remain
    const int after = (issued - 1 - gidx) * kBCopies + kGCopies * ((issued - 1) / GS - gidx / GS);
    wait_n<0, (L::NSTG - 2) * (kBCopies + kGCopies)>(after);
    barrier();
    if (issued < sc.total) issue_next();
  }
}

// ---------------------------------------------------- activation copies ---

template <bool FC1, int TM>
__device__ __forceinline__ void mid_activations(const FcArgs& p, const MSched& sc, uint8_t* smem, int aw) {
  using L = ML<TM>;
  constexpr int kACopies = L::A_COPIES;
  const int lane = threadIdx.x & 63;
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const bool gather = FC1 && p.dense_rows == 0;
  const uint8_t* a = (const uint8_t*)p.a;
  const uint8_t* src[kACopies];
  auto setup = [&](int li) {
    const MGeom it = m_geom<TM>(p, sc, li);
    // this wave's A_ROWS tile rows: tokens (FC1 routed) from the scalar cache
    Dw16 ids[L::A_ROWS / 16];
#pragma unroll
    for (int h = 0; h < L::A_ROWS / 16; ++h)
      if (gather && it.rows > L::A_ROWS * aw + 16 * h)
        ids[h] = load_dw16(p.sorted_assign + it.p0 + L::A_ROWS * aw + 16 * h);
#pragma unroll
    for (int i = 0; i < kACopies; ++i) {
      // copy i lands tile rows A_ROWS*aw + 4i .. +4, sixteen 16-B slots per row
      const int q = 4 * i + lane / 16;  // row within the wave's A_ROWS
      const int lr = L::A_ROWS * aw + q;
      int64_t row = 0;                  // rows past the tile copy row 0 of the operand
      if (lr < it.rows) {
        if (gather) {
          // q = 4i + lane/16: one of the 4 entries 4i .. 4i + 3
          int id = ids[(4 * i) / 16].v[(4 * i) % 16];
#pragma unroll
          for (int e = 1; e < 4; ++e)
            if (lane / 16 == e) id = ids[(4 * i + e) / 16].v[(4 * i + e) % 16];
          row = p.k > 1 ? (int64_t)__umulhi((uint32_t)id, p.kdiv) : id;
        } else {
          row = it.p0 + lr;
        }
      }
      const int c = (lane % 16) ^ (lr & 7);
      src[i] = a + row * (2 * (int64_t)K) + 16 * c;
    }
  };
  int li = 0, ls = 0, issued = 0;
  auto issue_next = [&]() {
    if (ls == 0) setup(li);
    const uint32_t base = lds0 + (issued % L::NSTG) * L::S_STAGE + S_B;
#pragma unroll
    for (int i = 0; i < kACopies; ++i) lds_copy16(src[i] + ls * A_ROW, base + 1024 * (kACopies * aw + i));
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  for (int s = 0; s < L::NSTG - 1 && s < sc.total; ++s) issue_next();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_n<0, (L::NSTG - 2) * kACopies>((issued - 1 - gidx) * kACopies);
    barrier();
    if (issued < sc.total) issue_next();
  }
}

template <bool FC1, int TM>
__global__ __launch_bounds__(ML<TM>::THREADS, 1) void k_fc_mid(FcArgs p) {
  using L = ML<TM>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::L_TOTAL];
  MSched sc;
  sc.nk = p.K / MBK;
  sc.NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + TM - 1) / TM : *p.num_tiles;
  sc.xcd = blockIdx.x & 7;
  sc.q = blockIdx.x >> 3;
  sc.Q = gridDim.x >> 3;
  sc.G = (sc.Q + sc.NB - 1) / sc.NB;
  sc.full = ntiles / (8 * sc.G);
  const int tail_items = (ntiles - 8 * sc.G * sc.full) * sc.NB;
  sc.tail0 = tail_items * sc.xcd / 8;
  const int nitems = sc.full * sc.G * sc.NB + tail_items * (sc.xcd + 1) / 8 - sc.tail0;
  sc.my_items = nitems > sc.q ? (nitems - sc.q + sc.Q - 1) / sc.Q : 0;
  sc.total = sc.my_items * sc.nk;
  if (sc.total == 0) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w < L::MUL_WAVES) mid_multiply<FC1, TM>(p, sc, smem, w);
  else if (w < L::MUL_WAVES + 2) mid_weights<FC1, TM>(p, sc, smem, w - L::MUL_WAVES);
  else mid_activations<FC1, TM>(p, sc, smem, w - L::MUL_WAVES - 2);
}

}  // namespace

template <int TM>
static hipError_t launch_mid_t(const FcArgs& p, bool fc1, int grid, hipStream_t st) {
  if (fc1) k_fc_mid<true, TM><<<grid, ML<TM>::THREADS, 0, st>>>(p);
  else k_fc_mid<false, TM><<<grid, ML<TM>::THREADS, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_fc_mid(const FcArgs& p, bool fc1, int rows, int grid, hipStream_t st) {
  if (rows != kMidRows && rows != kMidRowsHigh) return hipErrorInvalidValue;
  if (grid < 8) grid = 8;
  grid &= ~7;
  return rows == kMidRows ? launch_mid_t<kMidRows>(p, fc1, grid, st) : launch_mid_t<kMidRowsHigh>(p, fc1, grid, st);
}

}  // namespace moe_mx
