// Fused small-batch path of the routed MoE layer (bf16 activations, E2M1
// weights, at most 8 tokens and 64 assignments), taken on request: two
// kernels instead of the default path's three (FC1 with the routing in its
// prologue, FC2, combine).
//
// The mxfp6-sm120 page ("Execution model") runs batches of a few tokens on a
// separate path: allocation-free routing, a split W1 and a fused W2
// routed/shared reduction.  Here (without the split of W1, see below):
//
// k_micro_fc1  Every workgroup routes the batch itself in LDS (top-k of each
//              token by one wave, then the active local experts in ascending
//              order with their token masks): no routing launch and no
//              permutation kernels.  Workgroup 0 publishes the routing (the
//              caller's top-k outputs and the active-expert list k_micro_fc2
//              reads).  The workgroups then walk the items (active expert,
//              64 h columns), and after them the shared expert's items,
//              as one stream of 512-K steps: each of the four waves holds the
//              16 gate and 16 up weight rows of its 16 h columns, loads their
//              E2M1 codes and E8M0 scales straight from HBM into registers
//              three steps ahead (across item boundaries), and multiplies
//              them against the batch's x rows, staged once in LDS, on the
//              bf16 MFMA.  A tile's rows are the tokens; rows of tokens the
//              expert does not see are zero.  The epilogue applies the gated
//              activation and stores h in bf16.  (Splitting each item's K
//              between two waves per SIMD, with the halves added through LDS,
//              measured slower: 38.9 against 32.4 us at one token of the
//              decode shapes.)
//
// k_micro_fc2  One workgroup per 32 output columns.  Each of the 8 waves walks
//              its share of the work (the active experts j = wave, wave + 8,
//              ..., all of K, then every eighth 256-K chunk of the shared
//              expert)
//              and multiplies the h rows, again as token-indexed tiles,
//              against 32 rows of W2 streamed into registers three chunks
//              ahead.  After each expert the wave adds w(token, expert) times
//              the expert's output to its per-token fp32 accumulators (the
//              shared expert: shared_weight times its partial sums); the
//              waves' accumulators are added in a fixed order and each y
//              element is rounded to bf16 once.  No per-assignment output
//              rows and no combine launch; the result does not depend on
//              scheduling.
//
// MFMA operand layout of v_mfma_f32_16x16x32_bf16 (as in the other bf16
// kernels): lane l supplies row l%16 and 8 consecutive k-slots; the
// contraction order is free, so lane group g = l/16 takes the actual k ranges
// [32g, 32g + 32) and [128 + 32g, +32) of each 256-K chunk, 8 values per MFMA
// step: one MX block of its weight row in each 128-K half (16 bytes and one
// scale byte each), so that a load instruction reads a contiguous 64-byte run
// of each of 16 rows.  Accumulator element i of lane l is (row 4*(l/16) + i,
// column l%16).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "micro.h"
#include "mx_device.h"
#include "batch_route.h"

namespace moe_mx {

namespace {

constexpr int kWaves = 8;  // k_micro_fc2, and the routing of k_micro_fc1
constexpr int kThreads = 64 * kWaves;
constexpr int kThreads1 = 256;  // k_micro_fc1: four waves, one per 16 h columns of an item

// LDS routing state of one workgroup (k_micro_fc1)
using Route = BatchRoute<kMicroMaxAssign>;
static_assert(sizeof(Route) <= kMicroFc1StaticLds, "routing state");

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *(const uint4*)p; }


// Dequantize 8 E2M1 codes (one dword) with scale sc and multiply-accumulate
// them against 8 bf16 activation values.
__device__ __forceinline__ void mma8(v4f& acc, uint32_t w, float sc, const uint4& a) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  const v8bf bv = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  v8bf av;
  __builtin_memcpy(&av, &a, 16);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Publish the routing (workgroup 0): the caller's top-k outputs, and for
// k_micro_fc2 the active experts with their token masks, h row bases and the
// weight of each (expert, token).
template <int NT>
__device__ void publish(const MicroArgs& p, const Route& r) {
  const int A = p.T * p.k;
  for (int i = threadIdx.x; i < A; i += NT) {
    if (p.ids_out) p.ids_out[i] = r.ids[i];
    if (p.w_out) p.w_out[i] = r.wts[i];
  }
  MicroList* l = p.list;
  if (threadIdx.x == 0) l->nact = r.nact;
  for (int j = threadIdx.x; j < r.nact; j += NT) {
    const int e = r.act_e[j];
    l->expert[j] = e;
    l->mask[j] = r.mask[e];
    l->off[j] = r.act_off[j];
  }
  // the weight of every (active expert, token): its slot's weight, or 0 for a
  // token the expert does not see (one writer per entry)
  for (int i = threadIdx.x; i < r.nact * kMicroMaxTokens; i += NT) {
    const int j = i / kMicroMaxTokens, t = i % kMicroMaxTokens;
    const int eg = r.act_e[j] + p.off;
    float w = 0.f;
    if (t < p.T)
      for (int q = 0; q < p.k; ++q)
        if (r.ids[t * p.k + q] == eg) w = r.wts[t * p.k + q];
    l->w[i] = w;
  }
}

// ---------------------------------------------------------------- FC1 ----

// One 512-K step of a wave: codes of its gate and up rows (two 256-K
// chunks, 32 bytes each per lane) and their scale bytes (16 per row: both
// chunks).
struct Step1 {
  uint4 c[2][4];  // [tile][chunk u * 2 + half]
  uint4 s[2];     // [tile] scale bytes of the two chunks
};

struct Item1 {
  const uint8_t* w;   // code row of the lane's gate row (up row: + up_off)
  const uint8_t* sc;  // scale row
  int64_t up_off, up_soff;
};

// weights of item `it` for this lane (wave wv, row r16)
__device__ __forceinline__ Item1 item1(const MicroArgs& p, const Route& r, int it, int wv, int r16) {
  const int nb1 = p.I / 64;
  const int nr = r.nact * nb1;
  Item1 g;
  const int64_t rowb = (int64_t)p.H / 2, srow = p.H / 32;
  if (it < nr) {
    const int j = it / nb1, nb = it - j * nb1;
    const int e = r.act_e[j];
    const int64_t row = (int64_t)nb * 64 + 16 * wv + r16;
    g.w = p.w1 + (int64_t)e * p.w1_estride + row * rowb;
    g.sc = p.s1 + (int64_t)e * p.s1_estride + row * srow;
    g.up_off = (int64_t)p.I * rowb;
    g.up_soff = (int64_t)p.I * srow;
  } else {
    const int nb = it - nr;
    const int64_t row = (int64_t)nb * 64 + 16 * wv + r16;
    g.w = p.ws1 + row * rowb;
    g.sc = p.ss1 + row * srow;
    g.up_off = (int64_t)p.Is * rowb;
    g.up_soff = (int64_t)p.Is * srow;
  }
  return g;
}

// Within a 256-K chunk, lane group g4 takes k [32 g4, +32) of each 128-K half:
// its 16-byte MX block of half h sits at byte 64 h + 16 g4 of the row's 128,
// so each load instruction reads one contiguous 64-byte run of every row.
__device__ __forceinline__ void load1(Step1& b, const Item1& g, int q, int g4) {
  const uint8_t* w0 = g.w + 256 * q + 16 * g4;
  const uint8_t* w1 = w0 + g.up_off;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      b.c[0][2 * u + h] = ld16(w0 + 128 * u + 64 * h);
      b.c[1][2 * u + h] = ld16(w1 + 128 * u + 64 * h);
    }
  }
  b.s[0] = ld16(g.sc + 16 * q);
  b.s[1] = ld16(g.sc + g.up_soff + 16 * q);
}

// multiply step q of an item: x rows from LDS (row stride xs bytes), valid
// rows `rows_ok` (bit r: the lane's token row r takes part)
__device__ __forceinline__ void mul1(v4f (&acc)[2], const Step1& b, const uint8_t* xl, int xs, bool row_ok,
                                     int r16, int g4, int q) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sb = 8 * u + 4 * h + g4;  // scale byte within the step's 16
      const float sc0 = e8m0_to_f32((word(b.s[0], sb >> 2) >> (8 * (sb & 3))) & 0xffu);
      const float sc1 = e8m0_to_f32((word(b.s[1], sb >> 2) >> (8 * (sb & 3))) & 0xffu);
      const int k0 = 512 * q + 256 * u + 128 * h + 32 * g4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 a = make_uint4(0, 0, 0, 0);
        if (row_ok) a = *(const uint4*)(xl + r16 * xs + 2 * (k0 + 8 * s));
        mma8(acc[0], word(b.c[0][2 * u + h], s), sc0, a);
        mma8(acc[1], word(b.c[1][2 * u + h], s), sc1, a);
      }
    }
  }
}

template <int NS>
__global__ __launch_bounds__(kThreads1, 1) void k_micro_fc1(MicroArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];  // x rows, stride xs
  __shared__ Route r;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int xs = 2 * p.H + 16;

  // x rows of the batch into LDS (16 B per thread and copy)
  const int chunks = p.H / 8;
  for (int i = threadIdx.x; i < p.T * chunks; i += kThreads1) {
    const int t = i / chunks, c = i - t * chunks;
    *(uint4*)(xl + t * xs + 16 * c) = *(const uint4*)((const uint8_t*)p.x + ((int64_t)t * p.H + 8 * c) * 2);
  }
  route_batch<NS, kThreads1>(p.ids_in ? nullptr : p.logits, p.ids_in, p.w_in, p.T, p.E, p.k, p.off, p.L, r,
                             nullptr);  // ends with a barrier
  if (blockIdx.x == 0) publish<kThreads1>(p, r);

  const int nb1 = p.I / 64;
  const int items = r.nact * nb1 + p.Is / 64;
  const int my = items > (int)blockIdx.x ? (items - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
  // wave wc holds 16 h columns of the item (its gate and up rows) over all of K
  const int wc = wv;
  const int nq = p.H / 512;  // steps per item
  const int q0 = 0;
  const int total = my * nq;
  if (total == 0) return;  // uniform over the workgroup

  // the load cursor runs three steps ahead of the multiply cursor
  int lli = 0, lq = 0;
  Item1 lg = item1(p, r, blockIdx.x, wc, r16);
  auto load_next = [&](Step1& b) {
    load1(b, lg, q0 + lq, g4);
    if (++lq == nq) {
      lq = 0;
      if (lli + 1 < my) {
        ++lli;
        lg = item1(p, r, blockIdx.x + lli * gridDim.x, wc, r16);
      } else {
        lq = nq - 1;  // past the end: reload the last step (not used)
      }
    }
  };
  Step1 b0, b1, b2;
  load_next(b0);
  load_next(b1);
  load_next(b2);

  v4f acc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
  int mli = 0, mq = 0;  // multiply cursor
  int it = blockIdx.x;
  // the item's token rows: routed items use the expert's token mask, the
  // shared expert's items every token of the batch
  auto row_mask = [&](int item) -> uint32_t {
    const int nr = r.nact * nb1;
    return item < nr ? r.mask[r.act_e[item / nb1]] : ((1u << p.T) - 1u);
  };
  uint32_t mask = row_mask(it);

  auto step = [&](const Step1& b) {
    mul1(acc, b, xl, xs, r16 < p.T && (mask >> r16 & 1u), r16, g4, q0 + mq);
    if (++mq < nq) return;
    {
      // epilogue: lane holds token rows 4*g4 + i, column r16
      const int nr = r.nact * nb1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * g4 + i;
        if (t >= p.T || !(mask >> t & 1u)) continue;
        const float h = gated_act(p.act_fn, acc[0][i], acc[1][i]);
        if (it < nr) {
          const int j = it / nb1, nb = it - j * nb1;
          const int prow = r.act_off[j] + __popc(mask & ((1u << t) - 1u));
          p.h[(int64_t)prow * p.I + nb * 64 + 16 * wc + r16] = f32_to_bf16_rne(h);
        } else {
          const int nb = it - nr;
          p.hs[(int64_t)t * p.Is + nb * 64 + 16 * wc + r16] = f32_to_bf16_rne(h);
        }
      }
    }
    acc[0] = (v4f){0.f, 0.f, 0.f, 0.f};
    acc[1] = (v4f){0.f, 0.f, 0.f, 0.f};
    mq = 0;
    ++mli;
    it = blockIdx.x + mli * gridDim.x;
    if (mli < my) mask = row_mask(it);
  };

  // the loads are issued on every path (past the end they repeat the last
  // step), so each buffer's wait counts the same later loads on all paths
  for (int s = 0; s < total; s += 3) {
    step(b0);
    load_next(b0);
    if (s + 1 < total) step(b1);
    load_next(b1);
    if (s + 2 < total) step(b2);
    load_next(b2);
  }
}

// ---------------------------------------------------------------- FC2 ----

// One 256-K chunk of a wave: codes of its 32 W2 rows (two tiles, 32 bytes
// per lane each), the dword holding the lane's two scale bytes of each, and
// the lane's 64 h values of its token row.
struct Step2 {
  uint4 c[2][2];
  uint2 s[2];  // the row's 8 scale bytes of the chunk: .x half 0, .y half 1
  uint4 a[8];
};

// the wave's chunk stream: work unit u < n_r * kc: routed expert j = wave +
// 4 (u / kc), chunk u % kc; then the shared expert's chunks wave, wave + 4, ...
struct Stream2 {
  int nr_units, kc, kcs;
};

// The published list, copied to LDS by every workgroup of k_micro_fc2.
struct ListLds {
  int32_t expert[kMicroMaxL];
  uint32_t mask[kMicroMaxL];
  int32_t off[kMicroMaxL];
  float w[kMicroMaxL][kMicroMaxTokens];
};

template <bool kShared>
__device__ __forceinline__ void load2(Step2& b, const MicroArgs& p, const ListLds* l, int j, int c, int n0,
                                      int r16, int g4, bool& row_ok) {
  const uint8_t* wb;
  const uint8_t* sb;
  const uint16_t* hrow;
  int K;
  // lanes whose token row takes no part load a valid row (the first) and
  // zero it, so that every path issues the same loads
  if (!kShared) {
    const int e = l->expert[j];
    K = p.I;
    wb = p.w2 + (int64_t)e * p.w2_estride;
    sb = p.s2 + (int64_t)e * p.s2_estride;
    const uint32_t m = l->mask[j];
    row_ok = r16 < p.T && (m >> r16 & 1u);
    hrow = p.h + (int64_t)(l->off[j] + (row_ok ? __popc(m & ((1u << r16) - 1u)) : 0)) * p.I;
  } else {
    K = p.Is;
    wb = p.ws2;
    sb = p.ss2;
    row_ok = r16 < p.T;
    hrow = p.hs + (int64_t)(row_ok ? r16 : 0) * p.Is;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    // lane group g4: k [32 g4, +32) of each 128-K half h (bytes 64 h + 16 g4)
    const int64_t row = n0 + 16 * t + r16;
    const uint8_t* w = wb + row * (K / 2) + 128 * c + 16 * g4;
    b.c[t][0] = ld16(w);
    b.c[t][1] = ld16(w + 64);
    b.s[t] = *(const uint2*)(sb + row * (K / 32) + 8 * c);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint8_t* a = (const uint8_t*)(hrow + 256 * c + 128 * h + 32 * g4);
#pragma unroll
    for (int i = 0; i < 4; ++i) b.a[4 * h + i] = ld16(a + 16 * i);
  }
}

__device__ __forceinline__ void mul2(v4f (&acc)[2], const Step2& b, int g4, bool row_ok) {
  const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sh = 8 * g4;
    const float sc0 = e8m0_to_f32(((h ? b.s[0].y : b.s[0].x) >> sh) & 0xffu);
    const float sc1 = e8m0_to_f32(((h ? b.s[1].y : b.s[1].x) >> sh) & 0xffu);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 a = row_ok ? b.a[4 * h + s] : zero;
      mma8(acc[0], word(b.c[0][h], s), sc0, a);
      mma8(acc[1], word(b.c[1][h], s), sc1, a);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_micro_fc2(MicroArgs p) {
  __shared__ float part[kWaves][kMicroMaxTokens][32];
  __shared__ ListLds ll;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = blockIdx.x * 32;
  const MicroList* gl = p.list;
  const int nact = gl->nact;
  for (int i = threadIdx.x; i < nact * kMicroMaxTokens; i += kThreads)
    ll.w[i / kMicroMaxTokens][i % kMicroMaxTokens] = gl->w[i];
  for (int j = threadIdx.x; j < nact; j += kThreads) {
    ll.expert[j] = gl->expert[j];
    ll.mask[j] = gl->mask[j];
    ll.off[j] = gl->off[j];
  }
  __syncthreads();
  const ListLds* l = &ll;

  const int kc = p.I / 256;
  const int mine = nact > wv ? (nact - wv + kWaves - 1) / kWaves : 0;  // routed experts of this wave
  const int nr = mine * kc;
  const int kcs = p.Is / 256;
  const int ns = kcs > wv ? (kcs - wv + kWaves - 1) / kWaves : 0;  // shared chunks of this wave
  const int total = nr + ns;

  v4f tot[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
  if (total > 0) {
    // load cursor three units ahead of the multiply cursor
    int lu = 0;
    auto load_unit = [&](Step2& b, bool& ok) {
      const int u = min(lu, total - 1);
      ++lu;
      if (u < nr) load2<false>(b, p, l, wv + kWaves * (u / kc), u % kc, n0, r16, g4, ok);
      else load2<true>(b, p, l, 0, wv + kWaves * (u - nr), n0, r16, g4, ok);
    };
    Step2 b0, b1, b2;
    bool o0, o1, o2;
    load_unit(b0, o0);
    load_unit(b1, o1);
    load_unit(b2, o2);
    v4f acc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
    int mu = 0;
    auto step = [&](const Step2& b, bool ok) {
      mul2(acc, b, g4, ok);
      const int u = mu++;
      const bool last_routed = u < nr && (u % kc) == kc - 1;
      const bool last = u == total - 1;
      if (last_routed) {
        // expert j done: tot[row] += w(token row, j) * its output
        const int j = wv + kWaves * (u / kc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w = 4 * g4 + i < kMicroMaxTokens ? ll.w[j][4 * g4 + i] : 0.f;
          tot[0][i] += w * acc[0][i];
          tot[1][i] += w * acc[1][i];
        }
        acc[0] = (v4f){0.f, 0.f, 0.f, 0.f};
        acc[1] = (v4f){0.f, 0.f, 0.f, 0.f};
      } else if (last && u >= nr) {
        // the wave's share of the shared expert, with its weight
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tot[0][i] += p.shared_weight * acc[0][i];
          tot[1][i] += p.shared_weight * acc[1][i];
        }
      }
    };
    for (int s = 0; s < total; s += 3) {
      step(b0, o0);
      load_unit(b0, o0);
      if (s + 1 < total) step(b1, o1);
      load_unit(b1, o1);
      if (s + 2 < total) step(b2, o2);
      load_unit(b2, o2);
    }
  }
  // rows 4*g4 + i < T of the wave's totals into LDS, then the fixed-order sum
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * g4 + i;
    if (t < kMicroMaxTokens) {
      part[wv][t][r16] = tot[0][i];
      part[wv][t][16 + r16] = tot[1][i];
    }
  }
  __syncthreads();
  uint16_t* y = p.y;
  for (int i = threadIdx.x; i < p.T * 32; i += kThreads) {
    const int t = i / 32, c = i % 32;
    float v = part[0][t][c];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) v += part[q][t][c];  // fixed order
    y[(int64_t)t * p.H + n0 + c] = f32_to_bf16_rne(v);
  }
}

}  // namespace

size_t micro_fc1_lds(int T, int H) { return (size_t)T * (2 * (size_t)H + 16); }

hipError_t launch_micro(const MicroArgs& p, int cus, hipStream_t st, hipEvent_t fc2_mark) {
  const int nb1 = p.I / 64;
  // at most min(A, L) active experts: enough workgroups for every item, at most one per CU
  const int max_act = min(p.T * p.k, p.L);
  int g1 = max_act * nb1 + p.Is / 64;
  g1 = min(g1, cus);
  if (g1 < 1) g1 = 1;
  const size_t lds = micro_fc1_lds(p.T, p.H);
  const int ns = (p.E + 63) / 64;
  if (ns <= 1) k_micro_fc1<1><<<g1, kThreads1, lds, st>>>(p);
  else if (ns <= 2) k_micro_fc1<2><<<g1, kThreads1, lds, st>>>(p);
  else if (ns <= 4) k_micro_fc1<4><<<g1, kThreads1, lds, st>>>(p);
  else if (ns <= 6) k_micro_fc1<6><<<g1, kThreads1, lds, st>>>(p);
  else if (ns <= 8) k_micro_fc1<8><<<g1, kThreads1, lds, st>>>(p);
  else k_micro_fc1<16><<<g1, kThreads1, lds, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (fc2_mark && hipEventRecord(fc2_mark, st) != hipSuccess) return hipErrorUnknown;
  k_micro_fc2<<<p.H / 32, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe_mx
