// Grouped FC1 / FC2 GEMMs of the routed MoE layer for bf16 activations and
// E2M1 weights ("w4a16": TokenSpeed SiTU page, "Activation precision"), for
// M-tiles of at most 16 rows: the decode shape, where each expert sees a
// handful of tokens and the layer is bound by streaming the packed weights
// from HBM (mxfp6-sm120 page, "Execution model": weights stay packed in the
// mainloop).
//
// Work item = (16-row M-tile of one expert, N-block of 128 weight rows: FC1
// 64 gate + 64 up rows, i.e. 64 columns of h; FC2 128 output columns).  The
// grid is persistent (one workgroup per CU).  Per 128-K stage the weight
// tile (128 rows x 64 B of E2M1 codes + one E8M0 scale word per row) and the
// activation tile (16 rows x 256 B of bf16) are copied global -> LDS into a
// ring of 12 stage buffers, so up to 11 stages (about 100 KB per CU) are in
// flight: enough to cover HBM latency at full bandwidth.
//
// Waves (7): 0-3 multiply, 4-5 copy weights (5 copies per stage each), 6 copies
// activations (4 copies per stage).  Each copy wave owns one in-order stream
// and waits for its own stage before the per-stage barrier; the multiply
// waves issue no loads (item geometry and row metadata come through the
// scalar cache).
//
// MFMA: v_mfma_f32_16x16x32_bf16 (lane l supplies row l%16 and 8 consecutive
// k-slots 8*(l/16) .. +8; accumulator element i of lane l is (row 4*(l/16)+i,
// column l%16)).  The contraction order is free, so lane group g = l/16 takes
// the actual k range [32g, 32g + 32) of the stage, 8 values per MFMA step: its
// weight bytes are one 16-B chunk (one MX block, one scale byte) and its
// activation values one 64-B run.  Weights are dequantized in registers with
// v_cvt_scalef32_pk_bf16_fp4 (exact for E8M0 scales).
#include <hip/hip_runtime.h>

#include "copy_ring.h"
#include "gemm.h"
#include "mx_device.h"

namespace moe_mx {

namespace {

constexpr int SBM = kStreamRows;  // 16 rows per M-tile
constexpr int SBN = 128;          // weight rows per item
constexpr int SBK = 128;          // K per stage
constexpr int NSTAGE = 12;        // ring depth
constexpr int kMulW = 4;
constexpr int kWaveB = 4;         // weight-copy waves 4, 5
constexpr int kWaveA = 6;         // activation-copy wave
constexpr int kThreadsS = 64 * 7;

// stage layout: [weights 128 x 64 B][scale words 128 x 4 B][activations 16 x 256 B]
constexpr int S_B = SBN * SBK / 2;
constexpr int S_BS = SBN * 4;
constexpr int S_A = SBM * SBK * 2;
constexpr int S_STAGE = S_B + S_BS + S_A;
constexpr int kBCopies = S_B / 1024 / 2 + 1;  // per weight-copy wave: 4 x 1 KB + 1 scale copy
constexpr int kACopiesS = S_A / 1024;         // 4 x 1 KB

// weight tile: 16-B chunk c of row r at slot c ^ ((r >> 1) & 3)
__device__ __forceinline__ int wb_off(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }
// activation tile: 16-B chunk c (8 bf16) of row r at slot c ^ (r & 7)
__device__ __forceinline__ int wa_off(int r, int c) { return r * 256 + 16 * (c ^ (r & 7)); }

struct SGeom {
  int expert, p0, rows, nb;
};
struct SSched {
  int q, Q, NB, nk, my_items, total;
};

__device__ __forceinline__ SGeom s_geom(const FcArgs& p, const SSched& sc, int li) {
  const int j = sc.q + li * sc.Q;
  const int ti = j / sc.NB;
  SGeom g;
  g.nb = j % sc.NB;
  if (p.dense_rows > 0) {
    g.expert = 0;
    g.p0 = SBM * ti;
    g.rows = min(SBM, p.dense_rows - SBM * ti);
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

// ------------------------------------------------------------ multiply ---

template <bool FC1>
__device__ __forceinline__ void small_multiply(const FcArgs& p, const SSched& sc, uint8_t* smem) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  // B-tile rows of this wave's two 16-column tiles
  const int t0 = FC1 ? 16 * w : 32 * w;
  const int t1 = FC1 ? SBN / 2 + 16 * w : 32 * w + 16;
  v4f acc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
  int ci = 0, cs = 0;
  SGeom it = s_geom(p, sc, 0);
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_lgkm0();
    barrier();
    const uint8_t* st = smem + (gidx % NSTAGE) * S_STAGE;
    const uint32_t* sw = (const uint32_t*)(st + S_B);
    const uint8_t* as = st + S_B + S_BS;
    // activation run of this lane: row r16, k [32g, 32g + 32) = chunks 4g .. 4g+3
    uint4 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = *(const uint4*)(as + wa_off(r16, 4 * g + ks));
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int jr = (n == 0 ? t0 : t1) + r16;
      const uint4 b = *(const uint4*)(st + wb_off(jr, g));
      const float sc = e8m0_to_f32((sw[jr] >> (8 * g)) & 0xffu);
      const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const v2bf q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[ks], sc, 0);
        const v2bf q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[ks], sc, 1);
        const v2bf q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[ks], sc, 2);
        const v2bf q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[ks], sc, 3);
        const v8bf bv = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
        v8bf av;
        __builtin_memcpy(&av, &a[ks], 16);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
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
        if (row < it.rows) out[(int64_t)(it.p0 + row) * p.N + col] = f32_to_bf16_rne(silu_mul(acc[0][i], acc[1][i]));
      }
    } else {
      int orow[4];
      float wt[4];
      if (p.dense_rows > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          orow[i] = it.p0 + 4 * g + i;
          wt[i] = p.dense_weight;
        }
      } else {
        // row metadata of the tile through the scalar cache (16 entries from p0;
        // entries past the tile are never used)
        const Dw16 ids = load_dw16(p.sorted_assign + it.p0);
        const Dw16 wts = load_dw16(p.sorted_w + it.p0);
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
        if (4 * g + i < it.rows) {
          float* o = p.obuf + (int64_t)orow[i] * p.N + it.nb * SBN + 32 * w + r16;
          o[0] = wt[i] * acc[0][i];
          o[16] = wt[i] * acc[1][i];
        }
      }
    }
    acc[0] = (v4f){0.f, 0.f, 0.f, 0.f};
    acc[1] = (v4f){0.f, 0.f, 0.f, 0.f};
    cs = 0;
    if (++ci < sc.my_items) it = s_geom(p, sc, ci);
  }
}

// -------------------------------------------------------- weight copies ---

template <bool FC1>
__device__ __forceinline__ void small_weights(const FcArgs& p, const SSched& sc, uint8_t* smem) {
  const int lane = threadIdx.x & 63, bw = (threadIdx.x >> 6) - kWaveB;
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const int64_t wrow = (int64_t)K / 2;
  const uint8_t* src[4];
  const uint8_t* ssrc;
  auto setup = [&](int li) {
    const SGeom it = s_geom(p, sc, li);
    const uint8_t* wb = p.w + (int64_t)it.expert * p.w_estride;
    const uint8_t* sb = p.w_scale + (int64_t)it.expert * p.ws_estride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * bw + i;
      const int jr = 16 * t + (lane >> 2);
      const int ch = (lane & 3) ^ ((jr >> 1) & 3);
      src[i] = wb + s_wrow<FC1>(p, it.nb, jr) * wrow + 16 * ch;
    }
    ssrc = sb + s_wrow<FC1>(p, it.nb, 64 * bw + lane) * (K / 32);
  };
  int li = 0, ls = 0, issued = 0;
  auto issue_next = [&]() {
    if (ls == 0) setup(li);
    const uint32_t base = lds0 + (issued % NSTAGE) * S_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(src[i] + ls * (SBK / 2), base + 1024 * (4 * bw + i));
    lds_copy4(ssrc + 4 * ls, base + S_B + 256 * bw);
    ++issued;
    if (++ls == sc.nk) {
      ls = 0;
      ++li;
    }
  };
  for (int s = 0; s < NSTAGE - 1 && s < sc.total; ++s) issue_next();
  for (int gidx = 0; gidx < sc.total; ++gidx) {
    wait_stages<kBCopies, NSTAGE - 2>(issued - 1 - gidx);
    barrier();
    if (issued < sc.total) issue_next();
  }
}

// ---------------------------------------------------- activation copies ---

template <bool FC1>
__device__ __forceinline__ void small_activations(const FcArgs& p, const SSched& sc, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int K = p.K;
  const uint32_t lds0 = lds_addr(smem);
  const bool gather = FC1 && p.dense_rows == 0;
  const uint8_t* src[4];
  auto setup = [&](int li) {
    const SGeom it = s_geom(p, sc, li);
    int tok[16];
    if (gather) {
      const Dw16 ids = load_dw16(p.sorted_assign + it.p0);
#pragma unroll
      for (int q = 0; q < 16; ++q) tok[q] = ids.v[q] / p.k;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy i lands rows 4i .. 4i+3; rows past the tile repeat its first row
      int r = 4 * i + (lane >> 4);
      r = r < it.rows ? r : 0;
      int64_t row = it.p0 + r;
      if (gather) {
        int tr = tok[0];
#pragma unroll
        for (int q = 1; q < 16; ++q)
          if (r == q) tr = tok[q];
        row = tr;
      }
      const int c = (lane & 15) ^ ((4 * i + (lane >> 4)) & 7);  // chunk for this lane's LDS slot
      src[i] = (const uint8_t*)p.a + row * (2 * (int64_t)K) + 16 * c;
    }
  };
  int li = 0, ls = 0, issued = 0;
  auto issue_next = [&]() {
    if (ls == 0) setup(li);
    const uint32_t base = lds0 + (issued % NSTAGE) * S_STAGE + S_B + S_BS;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(src[i] + ls * (2 * SBK), base + 1024 * i);
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

template <bool FC1>
__global__ __launch_bounds__(kThreadsS, 1) void k_fc_small(FcArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * S_STAGE];
  SSched sc;
  sc.nk = p.K / SBK;
  sc.NB = p.nchunks;
  const int ntiles = p.dense_rows > 0 ? (p.dense_rows + SBM - 1) / SBM : *p.num_tiles;
  sc.q = blockIdx.x;
  sc.Q = gridDim.x;
  const int nitems = ntiles * sc.NB;
  sc.my_items = nitems > sc.q ? (nitems - sc.q + sc.Q - 1) / sc.Q : 0;
  sc.total = sc.my_items * sc.nk;
  if (sc.total == 0) return;
  const int w = threadIdx.x >> 6;
  if (w < kMulW) small_multiply<FC1>(p, sc, smem);
  else if (w < kWaveA) small_weights<FC1>(p, sc, smem);
  else small_activations<FC1>(p, sc, smem);
}

hipError_t launch_fc_small(const FcArgs& p, bool fc1, int grid, hipStream_t st) {
  if (grid < 1) grid = 1;
  if (fc1) k_fc_small<true><<<grid, kThreadsS, 0, st>>>(p);
  else k_fc_small<false><<<grid, kThreadsS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe_mx
