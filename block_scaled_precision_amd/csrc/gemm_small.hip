// Grouped FC1 / FC2 GEMMs of the routed MoE layer for bf16 activations and
// E2M1 weights ("w4a16": TokenSpeed SiTU page, "Activation precision"), for
// M-tiles of at most 16 rows: the decode shape, where each expert sees a
// handful of tokens and the layer is bound by streaming the packed weights
// from HBM (mxfp6-sm120 page, "Execution model": weights stay packed in the
// mainloop).
//
// Work item = (16-row M-tile of one expert, N-block of 128 weight rows: FC1
// 64 gate + 64 up rows, i.e. 64 columns of h; FC2 128 output columns).  The
// grid is persistent (one workgroup per CU).  Per 256-K stage the weight
// tile (128 rows x 128 B of E2M1 codes) and the activation tile (16 rows x
// 512 B of bf16) are copied global -> LDS into a ring of 6 stage buffers, so
// up to 5 stages (about 100 KB per CU) are in flight: enough to cover HBM
// latency at full bandwidth.  Reading 128 contiguous bytes of every weight row
// per stage streams HBM markedly faster than 64 (measured: the decode FC1 went
// from 4.7 to 5.5 TB/s).  The E8M0 weight scales (8 bytes per row and stage)
// travel in groups of GS stages (4, 2 or 1, the largest dividing the stages
// of an item): a row's scales for consecutive stages are contiguous, and one
// copy per row and group costs a quarter of the memory requests of one per
// row and stage (measured: without any scale copies the decode FC1 ran 14%
// faster).
//
// Waves (7): 0-3 multiply, 4-5 copy weights (8 copies per stage each, plus
// the scale copies at the start of a group), 6 copies activations (8 copies
// per stage).  Each copy wave owns one in-order stream
// and waits for its own stage before the per-stage barrier; the multiply
// waves issue no loads (item geometry and row metadata come through the
// scalar cache).
//
// MFMA: v_mfma_f32_16x16x32_bf16 (lane l supplies row l%16 and 8 consecutive
// k-slots 8*(l/16) .. +8; accumulator element i of lane l is (row 4*(l/16)+i,
// column l%16)).  The contraction order is free, so lane group g = l/16 takes
// the actual k range [64g, 64g + 64) of the stage, 8 values per MFMA step: its
// weight bytes are two 16-B chunks (two MX blocks, two scale bytes) and its
// activation values one 128-B run.  Weights are dequantized in registers with
// v_cvt_scalef32_pk_bf16_fp4 (exact for E8M0 scales).
#include <hip/hip_runtime.h>

#include "copy_ring.h"
#include "gemm.h"
#include "mx_device.h"
#include "batch_route.h"

namespace moe_mx {

namespace {

constexpr int SBM = kStreamRows;  // 16 rows per M-tile
constexpr int SBN = 128;          // weight rows per item
constexpr int SBK = kSmallK;      // K per stage (the host checks K divisibility against it)
static_assert(SBK == 128 || SBK == 256, "stage K");
constexpr int NSTAGE = SBK == 128 ? 12 : 6;  // ring depth (about 150 KB either way)
constexpr int KPL = SBK / 4;      // k values per lane group and stage (one or two MX blocks)
constexpr int BROW = SBK / 2;     // weight bytes per row and stage
constexpr int kMulW = 4;
constexpr int kWaveB = 4;         // weight-copy waves 4, 5
constexpr int kWaveA = 6;         // activation-copy wave
constexpr int kThreadsS = 64 * 7;

// stage layout: [weights 128 rows x BROW][activations 16 rows x 2*SBK];
// then the scale-group ring: NG(GS) buffers of 128 rows x GS*SBK/32 bytes
constexpr int S_B = SBN * BROW;
constexpr int S_A = SBM * SBK * 2;
constexpr int S_STAGE = S_B + S_A;
constexpr int kBData = S_B / 1024 / 2;        // 1-KB weight copies per weight-copy wave
constexpr int kACopiesS = S_A / 1024;
constexpr int SROW = SBK / 32;                // scale bytes per row and stage
constexpr int L_SG = NSTAGE * S_STAGE;        // scale-group ring
constexpr int L_SG_SIZE = 4 * SBN * SROW * 3; // room for the largest ring (GS = 4, 3 buffers)
// Scale groups of GS stages: group G (stages GS*G ..) is copied just before
// the code copies of its first stage, into buffer G % NG, whose previous
// group was last read at stage GS*(G-NG) + GS - 1; stage GS*G is copied
// after barrier GS*G - NSTAGE + 1, so GS*(NG-1) >= NSTAGE - 1 keeps them apart.
template <int GS> struct SGroup {
  static constexpr int NG = (NSTAGE - 1 + GS - 1) / GS + 1;
  static constexpr int BYTES = SBN * SROW * GS;           // one group buffer
  static constexpr int LW = SROW * GS >= 16 ? 16 : 4;     // bytes per lane and copy
  static constexpr int COPIES = BYTES / 2 / (64 * LW);    // per weight-copy wave
  static_assert(NG * BYTES <= L_SG_SIZE, "scale-group ring");
  static_assert(GS * (NG - 1) >= NSTAGE - 1, "scale-group ring too short");
};

// Routing tables of the few-token FC1 (after the scale-group ring): tile j is
// active local expert j (T <= 16 tokens, so one 16-row tile holds all its
// rows), and the token of each permuted row (the activation row it gathers).
struct RouteTables {
  Tile tile[kSmallRoutedAssign];
  int32_t tok[kSmallRoutedAssign];
};
constexpr int L_RT = L_SG + L_SG_SIZE;
static_assert(L_RT + sizeof(RouteTables) <= 160 * 1024, "LDS");
static_assert(kSmallRoutedTokens <= SBM && kSmallRoutedTokens <= 32, "one tile per expert, 32-bit token masks");

// weight tile: 16-B chunk c of row r at slot c ^ swz(r), so that 8 rows read
// at the same chunk fall in 8 different 16-B bank groups
__device__ __forceinline__ int wb_swz(int r) { return BROW == 64 ? ((r >> 1) & 3) : (r & 7); }
__device__ __forceinline__ int wb_off(int r, int c) { return r * BROW + 16 * (c ^ wb_swz(r)); }
// activation tile: 16-B chunk c (8 bf16) of row r at slot c ^ (r & 7)
__device__ __forceinline__ int wa_off(int r, int c) { return r * (2 * SBK) + 16 * (c ^ (r & 7)); }

struct SGeom {
  int expert, p0, rows, nb, ks;
};
// NB N-blocks and S K-ranges per M-tile (S > 1 only for split dense GEMMs)
struct SSched {
  int q, Q, NB, S, nk, my_items, total;
};

// RT: the tile list is the workgroup's own routing tables in LDS
template <bool RT>
__device__ __forceinline__ SGeom s_geom(const FcArgs& p, const SSched& sc, int li, const uint8_t* smem) {
  const int j = sc.q + li * sc.Q;
  const int ti = j / (sc.NB * sc.S), r = j % (sc.NB * sc.S);
  SGeom g;
  g.nb = r / sc.S;
  g.ks = r % sc.S;
  if (p.dense_rows > 0) {
    g.expert = 0;
    g.p0 = SBM * ti;
    g.rows = min(SBM, p.dense_rows - SBM * ti);
  } else if (RT) {
    const Tile t = ((const RouteTables*)(smem + L_RT))->tile[ti];  // the same word in every lane
    g.expert = __builtin_amdgcn_readfirstlane(t.expert);
    g.p0 = __builtin_amdgcn_readfirstlane(t.p0);
    g.rows = __builtin_amdgcn_readfirstlane(t.rows);
  } else {
    const Tile t = load_tile(p.tiles, ti);
    g.expert = t.expert;
    g.p0 = t.p0;
    g.rows = t.rows;
  }
  return g;
}

template <bool FC1>
__device__ __forceinline__ int64_t s_wrow(const FcArgs& p, int nb, int jr) {
  if (FC1) return jr < SBN / 2 ? (int64_t)nb * (SBN / 2) + jr : (int64_t)p.N + nb * (SBN / 2) + jr - SBN / 2;
  return (int64_t)nb * SBN + jr;
}

// at most n (<= N) stages of COPIES copies each may stay in flight
template <int COPIES, int N>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vm_lgkm0<N * COPIES>();
      return;
    }
    wait_stages<COPIES, N - 1>(n);
  } else {
    wait_vm_lgkm0<0>();
  }
}

// s_waitcnt vmcnt(n) lgkmcnt(0) for a run-time n in [LO, HI] (binary search
// over the immediate forms; n above HI waits for HI, which is stricter)
template <int LO, int HI>
__device__ __forceinline__ void wait_ops(int n) {
  if constexpr (LO == HI) {
    wait_vm_lgkm0<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_ops<MID, HI>(n);
    else wait_ops<LO, MID - 1>(n);
  }
}

// ------------------------------------------------------------ multiply ---

template <bool FC1, int GS, bool RT>
__device__ __forceinline__ void small_multiply(const FcArgs& p, const SSched& sc, uint8_t* smem) {
  using SG = SGroup<GS>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  // B-tile rows of this wave's two 16-column tiles
  const int t0 = FC1 ? 16 * w : 32 * w;
  const int t1 = FC1 ? SBN / 2 + 16 * w : 32 * w + 16;
  v4f acc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
  int ci = 0, cs = 0;
  SGeom it = s_geom<RT>(p, sc, 0, smem);
  // routed FC2: the item's row metadata, loaded when the item starts (scalar
  // cache) so that its epilogue does not wait for it
  const bool routed2 = !FC1 && p.dense_rows == 0;
  Dw16 m_ids = {}, m_wts = {};
  if (routed2) {
    m_ids = load_dw16(p.sorted_assign + it.p0);
    m_wts = load_dw16(p.sorted_w + it.p0);
  }
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_lgkm0();
    barrier();
    const uint8_t* st = smem + (gidx % NSTAGE) * S_STAGE;
    // this stage's scale bytes of row jr: sb[jr * SROW * GS + ...]
    const uint8_t* sb = smem + L_SG + ((gidx / GS) % SG::NG) * SG::BYTES + (gidx % GS) * SROW;
    const uint8_t* as = st + S_B;
    // activation run of this lane: row r16, k [KPL*g, KPL*(g+1)) = chunks
    // (KPL/8)*g .. +KPL/8
    constexpr int NA = KPL / 8;  // 16-B activation chunks (MFMA steps) per lane
    uint4 a[NA];
#pragma unroll
    for (int ks = 0; ks < NA; ++ks) a[ks] = *(const uint4*)(as + wa_off(r16, NA * g + ks));
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int jr = (n == 0 ? t0 : t1) + r16;
#pragma unroll
      for (int blk = 0; blk < KPL / 32; ++blk) {
        // one MX block: 16 B of codes, one scale byte
        const uint4 b = *(const uint4*)(st + wb_off(jr, (KPL / 32) * g + blk));
        const float sc = e8m0_to_f32(sb[jr * SROW * GS + (KPL / 32) * g + blk]);
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
          const v2bf q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], sc, 0);
          const v2bf q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], sc, 1);
          const v2bf q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], sc, 2);
          const v2bf q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[kq], sc, 3);
          const v8bf bv = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
          v8bf av;
          __builtin_memcpy(&av, &a[4 * blk + kq], 16);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
        }
      }
    }
    if (++cs < sc.nk) continue;

    // ---- epilogue: lane holds rows 4g + i, columns r16 of its two tiles ----
    if (FC1) {
      uint16_t* out = (uint16_t*)p.out;
      const int col = it.nb * (SBN / 2) + 16 * w + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row < it.rows) out[(int64_t)(it.p0 + row) * p.N + col] = f32_to_bf16_rne(gated_act(p.act_fn, acc[0][i], acc[1][i]));
      }
    } else {
      int orow[4];
      float wt[4];
      if (sc.S > 1) {
        // split dense GEMM: this K range's unscaled fp32 sums
        float* o = p.part + ((int64_t)it.ks * p.dense_rows + it.p0) * p.N + it.nb * SBN + 32 * w + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (4 * g + i < it.rows) {
            o[(int64_t)(4 * g + i) * p.N] = acc[0][i];
            o[(int64_t)(4 * g + i) * p.N + 16] = acc[1][i];
          }
        }
      } else if (p.dense_rows > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          orow[i] = it.p0 + 4 * g + i;
          wt[i] = p.dense_weight;
        }
      } else {
        // row metadata of the tile through the scalar cache (16 entries from p0;
        // entries past the tile are never used)
        const Dw16& ids = m_ids;
        const Dw16& wts = m_wts;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          orow[i] = 0;
          wt[i] = 0.f;
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (4 * g + i == q) {
              orow[i] = ids.v[q];
              wt[i] = __int_as_float(wts.v[q]);
            }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (sc.S == 1 && 4 * g + i < it.rows) {
          uint16_t* o = p.obuf + (int64_t)orow[i] * p.N + it.nb * SBN + 32 * w + r16;
          o[0] = f32_to_bf16_rne(wt[i] * acc[0][i]);
          o[16] = f32_to_bf16_rne(wt[i] * acc[1][i]);
        }
      }
    }
    acc[0] = (v4f){0.f, 0.f, 0.f, 0.f};
    acc[1] = (v4f){0.f, 0.f, 0.f, 0.f};
    cs = 0;
    if (++ci < sc.my_items) {
      it = s_geom<RT>(p, sc, ci, smem);
      if (routed2) {
        m_ids = load_dw16(p.sorted_assign + it.p0);
        m_wts = load_dw16(p.sorted_w + it.p0);
      }
    }
  }
}

// -------------------------------------------------------- weight copies ---

template <bool FC1, int GS, bool RT>
__device__ __forceinline__ void small_weights(const FcArgs& p, const SSched& sc, uint8_t* smem) {
  using SG = SGroup<GS>;
  const int lane = threadIdx.x & 63, bw = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) - kWaveB);
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const int64_t wrow = (int64_t)K / 2;
  constexpr int CPR = BROW / 16;  // 16-B chunks per weight row and stage
  constexpr int GROW = SROW * GS; // scale bytes per row and group
  const uint8_t* src[kBData];
  const uint8_t* ssrc[SG::COPIES];
  auto setup = [&](int li) {
    const SGeom it = s_geom<RT>(p, sc, li, smem);
    const int64_t k0 = (int64_t)it.ks * sc.nk * SBK;  // first k of the item's range
    const uint8_t* wb = p.w + (int64_t)it.expert * p.w_estride + k0 / 2;
    const uint8_t* sb = p.w_scale + (int64_t)it.expert * p.ws_estride + k0 / 32;
#pragma unroll
    for (int i = 0; i < kBData; ++i) {
      const int t = kBData * bw + i;  // 1-KB copy index within the stage
      const int jr = (64 / CPR) * t + lane / CPR;
      const int ch = (lane % CPR) ^ wb_swz(jr);
      src[i] = wb + s_wrow<FC1>(p, it.nb, jr) * wrow + 16 * ch;
    }
    // scale group: GROW bytes per row, SG::LW per lane; copy t covers bytes
    // [64 LW t, 64 LW (t+1)) of the group buffer (row-major)
#pragma unroll
    for (int i = 0; i < SG::COPIES; ++i) {
      const int byte = SG::LW * (64 * (SG::COPIES * bw + i) + lane);
      const int jr = byte / GROW, within = byte % GROW;
      ssrc[i] = sb + s_wrow<FC1>(p, it.nb, jr) * (K / 32) + within;
    }
  };
  int li = 0, ls = 0, issued = 0;
  auto issue_next = [&]() {
    if (ls == 0) setup(li);
    // the scale group first: the stage's own wait then covers it
    if (issued % GS == 0) {
      const uint32_t gb = lds0 + L_SG + ((issued / GS) % SG::NG) * SG::BYTES;
#pragma unroll
      for (int i = 0; i < SG::COPIES; ++i) {
        if constexpr (SG::LW == 16) lds_copy16(ssrc[i] + ls * SROW, gb + 64 * SG::LW * (SG::COPIES * bw + i));
        else lds_copy4(ssrc[i] + ls * SROW, gb + 64 * SG::LW * (SG::COPIES * bw + i));
      }
    }
    const uint32_t base = lds0 + (issued % NSTAGE) * S_STAGE;
#pragma unroll
    for (int i = 0; i < kBData; ++i) lds_copy16(src[i] + ls * BROW, base + 1024 * (kBData * bw + i));
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  for (int s = 0; s < NSTAGE - 1 && s < sc.total; ++s) issue_next();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    // stage gidx (and its group, copied before it) has landed once at most the
    // copies of the stages issued after it remain
    const int after = (issued - 1 - gidx) * kBData + SG::COPIES * ((issued - 1) / GS - gidx / GS);
    wait_ops<0, (NSTAGE - 2) * (kBData + SG::COPIES)>(after);
    barrier();
    if (issued < sc.total) issue_next();
  }
}

// ---------------------------------------------------- activation copies ---

template <bool FC1, bool RT>
__device__ __forceinline__ void small_activations(const FcArgs& p, const SSched& sc, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const bool gather = FC1 && p.dense_rows == 0;
  constexpr int RPC = 1024 / (2 * SBK);  // activation rows per 1-KB copy
  constexpr int CPA = 2 * SBK / 16;      // 16-B chunks per activation row and stage
  const uint8_t* src[kACopiesS];
  auto setup = [&](int li) {
    const SGeom it = s_geom<RT>(p, sc, li, smem);
    int tok[16];
    if (gather && RT) {
      // the same words in every lane (entries past the tile are never used)
      const int32_t* lt = ((const RouteTables*)(smem + L_RT))->tok;
#pragma unroll
      for (int q = 0; q < 16; ++q) tok[q] = __builtin_amdgcn_readfirstlane(lt[min(it.p0 + q, kSmallRoutedAssign - 1)]);
    } else if (gather) {
      const Dw16 ids = load_dw16(p.sorted_assign + it.p0);
#pragma unroll
      for (int q = 0; q < 16; ++q) tok[q] = ids.v[q] / p.k;
    }
#pragma unroll
    for (int i = 0; i < kACopiesS; ++i) {
      // copy i lands rows RPC*i ..; rows past the tile repeat its first row
      const int lr = RPC * i + lane / CPA;  // LDS row
      const int r = lr < it.rows ? lr : 0;
      int64_t row = it.p0 + r;
      if (gather) {
        int tr = tok[0];
#pragma unroll
        for (int q = 1; q < 16; ++q)
          if (r == q) tr = tok[q];
        row = tr;
      }
      const int c = (lane % CPA) ^ (lr & 7);  // chunk for this lane's LDS slot
      src[i] = (const uint8_t*)p.a + row * (2 * (int64_t)K) + 2 * (int64_t)it.ks * sc.nk * SBK + 16 * c;
    }
  };
  int li = 0, ls = 0, issued = 0;
  auto issue_next = [&]() {
    if (ls == 0) setup(li);
    const uint32_t base = lds0 + (issued % NSTAGE) * S_STAGE + S_B;
#pragma unroll
    for (int i = 0; i < kACopiesS; ++i) lds_copy16(src[i] + ls * (2 * SBK), base + 1024 * i);
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  for (int s = 0; s < NSTAGE - 1 && s < sc.total; ++s) issue_next();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_stages<kACopiesS, NSTAGE - 2>(issued - 1 - gidx);
    barrier();
    if (issued < sc.total) issue_next();
  }
}

}  // namespace

template <bool FC1, int GS>
__global__ __launch_bounds__(kThreadsS, 1) void k_fc_small(FcArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L_SG + L_SG_SIZE];
  SSched sc;
  sc.S = p.ksplit > 1 ? p.ksplit : 1;
  sc.nk = p.K / SBK / sc.S;
  sc.NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + SBM - 1) / SBM : *p.num_tiles;
  sc.q = blockIdx.x;
  sc.Q = gridDim.x;
  const int nitems = ntiles * sc.NB * sc.S;
  sc.my_items = nitems > sc.q ? (nitems - sc.q + sc.Q - 1) / sc.Q : 0;
  sc.total = sc.my_items * sc.nk;
  if (sc.total == 0) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w < kMulW) small_multiply<FC1, GS, false>(p, sc, smem);
  else if (w < kWaveA) small_weights<FC1, GS, false>(p, sc, smem);
  else small_activations<FC1, false>(p, sc, smem);
}

// Routing of the batch in the prologue of the few-token FC1: every workgroup
// routes it into LDS (scratch in the stage ring, which no copy has reached
// yet: top-k, token masks and the expert scan of batch_route.h) and keeps the
// tile list and the token of each permuted row; workgroup 0 also writes the
// routing out, with the top-k and the expert offsets, exactly as the routing
// and permutation kernels would.  Returns the number of tiles (active local
// experts), uniform; ends with a barrier.
template <int NS>
__device__ int route_in_fc1(const FcArgs& p, uint8_t* smem) {
  using R = BatchRoute<kSmallRoutedAssign>;
  static_assert(sizeof(R) + 4 * (kMaxExperts + 1) <= L_SG, "routing scratch");
  R& r = *(R*)smem;
  int32_t* start = (int32_t*)(smem + sizeof(R));  // first permuted row of each local expert, [L + 1]
  RouteTables& rt = *(RouteTables*)(smem + L_RT);
  route_batch<NS, kThreadsS>(p.logits, nullptr, nullptr, p.T, p.E, p.k, p.off, p.L, r, start);
  const bool pub = blockIdx.x == 0;
  for (int j = threadIdx.x; j < r.nact; j += kThreadsS) {
    Tile t;
    t.expert = r.act_e[j];
    t.p0 = r.act_off[j];
    t.rows = r.act_off[j + 1] - r.act_off[j];  // at most T <= 16: one tile per expert
    t.pad = 0;
    rt.tile[j] = t;
    if (pub) p.tiles_out[j] = t;
  }
  const int A = p.T * p.k;
  for (int a = threadIdx.x; a < A; a += kThreadsS) {
    if (pub) {
      p.ids_out[a] = r.ids[a];
      p.w_out[a] = r.wts[a];
    }
    const int el = r.ids[a] - p.off;
    if (el < 0 || el >= p.L) continue;
    // rows of an expert are its tokens in ascending order
    const int t = a / p.k;
    const int pos = start[el] + __popc(r.mask[el] & ((1u << t) - 1u));
    rt.tok[pos] = t;
    if (pub) {
      p.sorted_out[pos] = a;
      p.sorted_w_out[pos] = r.wts[a];
    }
  }
  if (pub) {
    for (int e = threadIdx.x; e <= p.L; e += kThreadsS) p.offsets_out[e] = start[e];
    if (threadIdx.x == 0) *p.ntiles_out = r.nact;
  }
  const int n = __builtin_amdgcn_readfirstlane(r.nact);
  __syncthreads();  // the tables are complete and the scratch is free for the stage ring
  return n;
}

template <int GS, int NS>
__global__ __launch_bounds__(kThreadsS, 1) void k_fc_small_routed(FcArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L_RT + sizeof(RouteTables)];
  const int ntiles = route_in_fc1<NS>(p, smem);
  SSched sc;
  sc.S = 1;
  sc.nk = p.K / SBK;
  sc.NB = p.nchunks;
  sc.q = blockIdx.x;
  sc.Q = gridDim.x;
  const int nitems = ntiles * sc.NB;
  sc.my_items = nitems > sc.q ? (nitems - sc.q + sc.Q - 1) / sc.Q : 0;
  sc.total = sc.my_items * sc.nk;
  if (sc.total == 0) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w < kMulW) small_multiply<true, GS, true>(p, sc, smem);
  else if (w < kWaveA) small_weights<true, GS, true>(p, sc, smem);
  else small_activations<true, true>(p, sc, smem);
}

template <bool FC1>
static hipError_t launch_small_t(const FcArgs& p, int grid, hipStream_t st) {
  // scale groups: the largest of 4, 2, 1 stages that divides the stages of an item
  const int nk = p.K / SBK / (p.ksplit > 1 ? p.ksplit : 1);
  if (nk % 4 == 0) k_fc_small<FC1, 4><<<grid, kThreadsS, 0, st>>>(p);
  else if (nk % 2 == 0) k_fc_small<FC1, 2><<<grid, kThreadsS, 0, st>>>(p);
  else k_fc_small<FC1, 1><<<grid, kThreadsS, 0, st>>>(p);
  return hipGetLastError();
}

// Sum of the K-range partials of a split dense GEMM: 4 columns per thread,
// the ranges added in ascending order, then alpha, then one bf16 rounding.
__global__ void k_splitk_reduce(const float4* __restrict__ part, int ksplit, int64_t n4, float alpha,
                                uint2* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  float4 s = part[i];
  for (int k = 1; k < ksplit; ++k) {
    const float4 v = part[(int64_t)k * n4 + i];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(alpha * s.x) | ((uint32_t)f32_to_bf16_rne(alpha * s.y) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(alpha * s.z) | ((uint32_t)f32_to_bf16_rne(alpha * s.w) << 16);
  y[i] = o;
}

hipError_t launch_splitk_reduce(const float* part, int ksplit, int64_t n4, float alpha, uint16_t* y,
                                hipStream_t st) {
  if (n4 <= 0) return hipSuccess;
  k_splitk_reduce<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>((const float4*)part, ksplit, n4, alpha, (uint2*)y);
  return hipGetLastError();
}

hipError_t launch_fc_small(const FcArgs& p, bool fc1, int grid, hipStream_t st) {
  if (grid < 1) grid = 1;
  return fc1 ? launch_small_t<true>(p, grid, st) : launch_small_t<false>(p, grid, st);
}

template <int GS>
static hipError_t launch_small_routed_t(const FcArgs& p, int grid, hipStream_t st) {
  // key slots per lane of the top-k: the fewest of 1, 2, 4, 6, 8, 16 covering E
  const int ns = (p.E + 63) / 64;
  if (ns <= 1) k_fc_small_routed<GS, 1><<<grid, kThreadsS, 0, st>>>(p);
  else if (ns <= 2) k_fc_small_routed<GS, 2><<<grid, kThreadsS, 0, st>>>(p);
  else if (ns <= 4) k_fc_small_routed<GS, 4><<<grid, kThreadsS, 0, st>>>(p);
  else if (ns <= 6) k_fc_small_routed<GS, 6><<<grid, kThreadsS, 0, st>>>(p);
  else if (ns <= 8) k_fc_small_routed<GS, 8><<<grid, kThreadsS, 0, st>>>(p);
  else k_fc_small_routed<GS, 16><<<grid, kThreadsS, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_fc_small_routed(const FcArgs& p, int grid, hipStream_t st) {
  if (grid < 1) grid = 1;
  const int nk = p.K / SBK;
  if (nk % 4 == 0) return launch_small_routed_t<4>(p, grid, st);
  if (nk % 2 == 0) return launch_small_routed_t<2>(p, grid, st);
  return launch_small_routed_t<1>(p, grid, st);
}

}  // namespace moe_mx
