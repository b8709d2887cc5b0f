// Host side of libmoe_mx: argument validation, architecture check, workspace
// planning and the launch sequence of moe_fused, plus the public entry points
// mx_quantize and moe_route.
//
// The boundary follows the pages' interfaces: the keyword call of the
// TokenSpeed SiTU page ("Runtime API": physical intermediate size, global
// expert count, local expert offset and count; "Supported contract": MXFP8
// activations with a block-scale tensor, precomputed top-k), the op names of
// the TokenSpeed-kernel page ("Public API": moe_route ... moe_fused), the
// caller-owned, graph-safe workspaces of the mxfp6-sm120 page ("Execution
// model", "Python API") and its fail-closed validation ("Validated scope").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "gemm.h"
#include "internal.h"
#include "micro.h"
#include "mx_device.h"

namespace moe_mx {

// ------------------------------------------------------------------ arch ---

moe_status_t check_arch() {
  static std::atomic<int> cache[256];  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_ARCH;
  if (dev < 256) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return MOE_OK;
    if (c == 2) return MOE_ERR_ARCH;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_ARCH;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 256) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MOE_OK : MOE_ERR_ARCH;
}

// Compute units of the current device (cached per device), for persistent grids.
static int device_cus() {
  static std::atomic<int> cache[256];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 256) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 256) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// ------------------------------------------------------- small kernels ----

// Unpermute-combine (TokenSpeed SiTU page, "Supported contract": the layer
// output is the routing-weighted sum over the selected experts; mxfp6-sm120
// page, "Routed MoE": routed/shared reduction).  obuf row t*k + j holds
// w[t,j] * FC2 output of assignment (t, j) rounded to bf16; sbuf row t the
// weighted shared-expert output (or nullptr), likewise.  y[t] = bf16 RNE of the
// fp32 sum over the assignments whose expert lies in the local range
// [off, off + L) (rows of other experts were never written), added in slot
// order, plus sbuf[t].  Each thread takes 8 columns (16 bytes per row) and
// issues the loads of up to 4 slots before adding them: the rows of slots
// whose expert is not local are loaded too (they lie in the workspace) and
// dropped.
__device__ __forceinline__ void add_bf16x8(float (&s)[8], uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s[2 * q] += __uint_as_float(w[q] << 16);
    s[2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
  }
}
constexpr int kCombineBatch = 8;  // slots in flight per thread
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte load that need not stay in the caches (the data is read once)
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__global__ __launch_bounds__(256) void k_combine(const uint4* __restrict__ obuf, const uint4* __restrict__ sbuf,
                                                 const int32_t* __restrict__ ids, int k, int off, int L,
                                                 int H8, int64_t n8, uint4* __restrict__ y) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const int64_t t = i / H8;
    const int64_t c = i - t * H8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // up to kCombineBatch slots in flight per thread; each obuf row is read
    // once, so the loads bypass the caches' retention (non-temporal)
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
      uint4 v[kCombineBatch];
      bool use[kCombineBatch];
#pragma unroll
      for (int q = 0; q < kCombineBatch; ++q) {
        const int j = j0 + q < k ? j0 + q : j0;
        const int e = ids[t * k + j] - off;
        use[q] = j0 + q < k && e >= 0 && e < L;
        v[q] = load_once(obuf + (t * k + j) * H8 + c);
      }
#pragma unroll
      for (int q = 0; q < kCombineBatch; ++q)
        if (use[q]) add_bf16x8(s, v[q]);
    }
    if (sbuf) add_bf16x8(s, sbuf[i]);
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (uint32_t)f32_to_bf16_rne(s[2 * q]) | ((uint32_t)f32_to_bf16_rne(s[2 * q + 1]) << 16);
    y[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void k_copy_routing(const int32_t* __restrict__ ids_in,
                                                      const float* __restrict__ w_in,
                                                      int32_t* __restrict__ ids_out,
                                                      float* __restrict__ w_out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (ids_out) ids_out[i] = ids_in[i];
  if (w_out) w_out[i] = w_in[i];
}

static int64_t grid_for(int64_t n, int64_t per_block, int64_t cap) {
  int64_t b = (n + per_block - 1) / per_block;
  return b < 1 ? 1 : (b > cap ? cap : b);
}

// ------------------------------------------------------------ layouts ----

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int wbits(mx_elem_t f) { return f == MX_E2M1 ? 4 : (f == MX_E3M2 ? 6 : 8); }

// Routed GEMMs run tiled (LDS-staged, M-tiles of up to kTiledRows rows) when the
// activations are MXFP8, H and I are multiples of kTiledKMultiple and the
// local experts average at least this many rows; otherwise the stream kernels
// (16-row tiles, weights straight from HBM) run.
constexpr int kTiledMinRowsPerExpert = 16;
// ... in M-tiles of kTiledRowsLow rows while the local experts average at most
// this many rows (nearly every expert then fits one such tile)
constexpr int kTiledLowMaxRowsPerExpert = 96;
// bf16 activations: the mid-M kernel when the local experts average at least
// this many rows (else the small-M kernel, 16-row tiles), with 128-row tiles
// from the second threshold on (64-row tiles below it)
constexpr int kMidMinRowsPerExpert = 32;
constexpr int kMidHighMinRowsPerExpert = 96;

// GEMM kernel family of one FC1/FC2 pair
enum class Fc { kStream, kSmall, kMid, kTiled, kWide };

// N-block width: FC1 in h columns, FC2 in output columns (`rows`: the M-tile
// height the kernel runs with)
static int fc_cols(Fc k, bool fc1, int rows) {
  switch (k) {
    case Fc::kWide:
    case Fc::kMid: return fc1 ? kWideCols / 2 : kWideCols;
    case Fc::kTiled: return fc1 ? tiled_weight_rows(rows) / 2 : tiled_weight_rows(rows);
    case Fc::kSmall: return fc1 ? kSmallColsFc1 : kSmallColsFc2;
    default: return fc1 ? kStreamColsFc1 : kStreamColsFc2;
  }
}

// M-tile height of a dense GEMM (the shared expert) on the tiled kernel: M
// rows, N output columns (FC1: h columns), `grid` persistent workgroups.
// 128-row tiles with 256-row N-blocks carry more multiply work per step;
// 192-row tiles with 128-row N-blocks split the work more finely.  Take the
// one whose busiest workgroup has the smaller area to multiply (ties: 128).
static int dense_tiled_rows(int M, int N, bool fc1, int grid) {
  int best = kTiledRowsLow;
  int64_t best_cost = -1;
  for (const int rows : {kTiledRowsLow, kTiledRows}) {
    const int tn = tiled_weight_rows(rows);
    const int64_t items = (int64_t)((M + rows - 1) / rows) * (N / (fc1 ? tn / 2 : tn));
    const int64_t cost = (items + grid - 1) / grid * rows * tn;
    if (best_cost < 0 || cost < best_cost) {
      best = rows;
      best_cost = cost;
    }
  }
  return best;
}

// The small-batch path (micro.hip): bf16 activations and E2M1 weights, at
// most kMicroMaxTokens tokens and kMicroMaxAssign assignments, H a multiple
// of 1024 (two K halves of 512-K FC1 steps), I and I_shared multiples of 256,
// and the batch's x rows within the LDS of a workgroup.
static bool micro_ok(const moe_problem_t& p) {
  return p.act == MOE_ACT_BF16 && p.w_fmt == MX_E2M1 && p.T >= 1 && p.T <= kMicroMaxTokens &&
         (int64_t)p.T * p.k <= kMicroMaxAssign && p.H % kMicroHMultiple == 0 && p.I % 256 == 0 && p.I_shared % 256 == 0 &&
         micro_fc1_lds(p.T, p.H) + kMicroFc1StaticLds <= 160 * 1024;
}

struct FusedPlan {
  int L, off;
  int64_t A;
  bool micro;
  Fc routed, shared;
  int bm;         // M-tile height of the routed tile list
  int shared_bm;  // M-tile height of the shared expert on the mid-M kernel
  int nblk, max_tiles;
  size_t ids, w, rank, hist, offsets, sorted, sorted_w, tiles, ntiles, xq, xs, h, hsc, hs, hssc, obuf, sbuf, micro_list,
      total;
};

static FusedPlan plan(const moe_problem_t& p) {
  FusedPlan f;
  f.off = p.local_expert_offset;
  f.L = p.local_num_experts == 0 ? p.E : p.local_num_experts;
  f.A = (int64_t)p.T * p.k;
  f.nblk = (p.T + kTokensPerRouteBlock - 1) / kTokensPerRouteBlock;
  // tokens from assignment ids by multiplication (FC1 gathers of the wide and
  // mid kernels) need A*k < 2^32
  const bool kdiv_ok = (double)f.A * p.k < 4294967296.0;
  if (p.act == MOE_ACT_MXFP8) {
    const bool tiled_h = p.H % kTiledKMultiple == 0;
    const bool tiled = f.L > 0 && f.A >= (int64_t)kTiledMinRowsPerExpert * f.L && tiled_h &&
                       p.I % kTiledKMultiple == 0;
    const bool shared_tiled = p.T >= kTiledMinRowsPerExpert && tiled_h && p.I_shared % kTiledKMultiple == 0;
    // E2M1 weights take the wide tiled kernel (256-row weight blocks)
    // (K a multiple of 512 and at least 1024: scale groups of 4 K-steps, items
    // of at least 8 steps)
    // The wide kernel addresses activation rows by 32-bit byte offsets from
    // the operand's base: token * H for FC1 (x codes), permuted row * I for FC2
    // (h codes), which must stay below 4 GiB.
    const double lim = 4294967296.0;
    const bool wide_h = p.w_fmt == MX_E2M1 && p.H % 512 == 0 && p.H >= 1024 && (double)p.T * p.H < lim;
    const bool wide = tiled && wide_h && p.I % 512 == 0 && p.I >= 1024 && kdiv_ok && (double)f.A * p.I < lim;
    const bool shared_wide = shared_tiled && wide_h && p.I_shared % 512 == 0 && p.I_shared >= 1024 &&
                             (double)p.T * p.I_shared < lim;
    f.routed = wide ? Fc::kWide : (tiled ? Fc::kTiled : Fc::kStream);
    f.shared = shared_wide ? Fc::kWide : (shared_tiled ? Fc::kTiled : Fc::kStream);
  } else {
    // bf16 activations, E2M1 weights: the small-M kernel, or the mid-M kernel
    // for experts with many rows; the stream kernels when K does not fit them.
    // E3M2 weights take the stream kernels.
    const bool small = p.w_fmt == MX_E2M1 && p.H % kSmallK == 0 && p.I % kSmallK == 0 &&
                       p.I_shared % kSmallK == 0;
    const bool mid_h = small && p.H % kMidK == 0;
    const bool mid = mid_h && p.I % kMidK == 0 && f.L > 0 && f.A >= (int64_t)kMidMinRowsPerExpert * f.L && kdiv_ok;
    const bool shared_mid = mid_h && p.I_shared % kMidK == 0 && p.T >= kMidMinRowsPerExpert;
    f.routed = mid ? Fc::kMid : (small ? Fc::kSmall : Fc::kStream);
    f.shared = shared_mid ? Fc::kMid : (small ? Fc::kSmall : Fc::kStream);
  }
  if (f.routed == Fc::kWide) f.bm = kTiledRows;
  else if (f.routed == Fc::kTiled)
    f.bm = f.A <= (int64_t)kTiledLowMaxRowsPerExpert * f.L ? kTiledRowsLow : kTiledRows;
  else if (f.routed == Fc::kMid)
    f.bm = f.A >= (int64_t)kMidHighMinRowsPerExpert * f.L ? kMidRowsHigh : kMidRows;
  else f.bm = kStreamRows;
  // (a dense shared expert on the tiled kernel picks its tile height per GEMM
  // at launch, from the grid: dense_tiled_rows)
  f.shared_bm = f.shared == Fc::kMid ? (p.T >= kMidHighMinRowsPerExpert ? kMidRowsHigh : kMidRows) : kTiledRows;
  f.max_tiles = (int)(f.A / f.bm + (f.A < f.L ? f.A : f.L));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = align_up(o + bytes, 256);
    return r;
  };
  const bool mx = p.act == MOE_ACT_MXFP8;
  const size_t T = (size_t)p.T, H = (size_t)p.H, I = (size_t)p.I, Is = (size_t)p.I_shared;
  f.ids = take(f.A * 4);
  f.w = take(f.A * 4);
  f.rank = take(f.A * 4);
  f.hist = take((size_t)f.nblk * f.L * 4);
  f.offsets = take((size_t)(f.L + 1) * 4);
  f.sorted = take(f.A * 4);
  f.sorted_w = take(f.A * 4);
  f.tiles = take((size_t)f.max_tiles * sizeof(Tile));
  f.ntiles = take(4);
  f.xq = mx ? take(T * H) : 0;
  f.xs = mx ? take(T * H / 32) : 0;
  f.h = take(f.A * I * (mx ? 1 : 2));
  f.hsc = mx ? take(f.A * I / 32) : 0;
  f.hs = Is ? take(T * Is * (mx ? 1 : 2)) : 0;
  f.hssc = (Is && mx) ? take(T * Is / 32) : 0;
  f.obuf = take(f.A * H * 2);
  f.sbuf = Is ? take(T * H * 2) : 0;
  f.micro = (p.flags & MOE_FLAG_FUSED_SMALL_BATCH) != 0;
  f.micro_list = take(sizeof(MicroList));
  f.total = o;
  return f;
}

static moe_status_t validate(const moe_problem_t* p, const moe_tensors_t* t) {
  if (!p || !t) return MOE_ERR_INVALID_ARG;
  if (p->T < 0 || p->H <= 0 || p->I <= 0 || p->I_shared < 0) return MOE_ERR_INVALID_ARG;
  if (p->H % 32 || p->I % 32 || p->I_shared % 32) return MOE_ERR_INVALID_ARG;
  if (p->E < 1 || p->E > kMaxExperts || p->k < 1 || p->k > p->E) return MOE_ERR_INVALID_ARG;
  if (p->w_fmt != MX_E2M1 && p->w_fmt != MX_E3M2 && p->w_fmt != MX_E4M3) return MOE_ERR_INVALID_ARG;
  if (p->act != MOE_ACT_BF16 && p->act != MOE_ACT_MXFP8) return MOE_ERR_INVALID_ARG;
  if (p->act_fn != MOE_FN_SILU && p->act_fn != MOE_FN_RELU2 && p->act_fn != MOE_FN_SWIGLU_OAI)
    return MOE_ERR_INVALID_ARG;
  if (p->flags & ~MOE_FLAG_FUSED_SMALL_BATCH) return MOE_ERR_INVALID_ARG;
  const int L = p->local_num_experts == 0 ? p->E : p->local_num_experts;
  if (p->local_expert_offset < 0 || L < 0 || (int64_t)p->local_expert_offset + L > p->E)
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)p->T * p->k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  if (p->T > 0) {
    if (!t->x || !t->y || !t->w1 || !t->w1_scale || !t->w2 || !t->w2_scale) return MOE_ERR_INVALID_ARG;
    const bool have_in = t->topk_ids_in || t->topk_w_in;
    if (have_in && !(t->topk_ids_in && t->topk_w_in)) return MOE_ERR_INVALID_ARG;
    if (!have_in && !t->router_logits) return MOE_ERR_INVALID_ARG;
    if (p->I_shared > 0 && (!t->ws1 || !t->ws1_scale || !t->ws2 || !t->ws2_scale)) return MOE_ERR_INVALID_ARG;
    const void* ptrs[] = {t->x, t->y, t->w1, t->w1_scale, t->w2, t->w2_scale};
    for (const void* q : ptrs)
      if (!aligned16(q)) return MOE_ERR_INVALID_ARG;
    if (p->I_shared > 0) {
      const void* sp[] = {t->ws1, t->ws1_scale, t->ws2, t->ws2_scale};
      for (const void* q : sp)
        if (!aligned16(q)) return MOE_ERR_INVALID_ARG;
    }
  }
  // valid, but outside what the kernels implement
  if (p->w_fmt == MX_E4M3) return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_FUSED_SMALL_BATCH) && !micro_ok(*p)) return MOE_ERR_UNSUPPORTED;
  if (p->H % 128 || p->I % 128 || p->I_shared % 128) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// ----------------------------------------------------- no-alloc scratch ----

// Workspace of moe_fused_noalloc: one array per device that loads the
// library, held until the process ends.  In host code `scratch` names a
// host-side stand-in, so its device address is looked up once per device
// (scratch_ptr) and only that address is passed to kernels.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up on the first
// call per device (nullptr if the lookup fails).
static void* scratch_ptr(moe_status_t* st) {
  static std::atomic<void*> ptrs[256];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
    *st = MOE_ERR_ARCH;
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    *st = MOE_ERR_HIP;
    return nullptr;
  }
  ptrs[dev].store(p, std::memory_order_release);  // the same address however many threads race here
  return p;
}

}  // namespace moe_mx

using namespace moe_mx;

// ------------------------------------------------------- public entry points

extern "C" const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_ARCH: return "no gfx950 device";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char* moe_mx_version(void) { return "0.1.0"; }

extern "C" moe_status_t mx_quantize(const void* src, moe_src_t src_dtype, int64_t rows, int64_t cols,
                                    int64_t src_ld, mx_elem_t fmt, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 32 || src_ld < cols) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_SRC_BF16 && src_dtype != MOE_SRC_FP32) return MOE_ERR_INVALID_ARG;
  if (fmt != MX_E2M1 && fmt != MX_E3M2 && fmt != MX_E4M3) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!src || !codes || !scales)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  moe_status_t a = check_arch();
  if (a != MOE_OK) return a;
  return launch_quantize(src, src_dtype, rows, cols, src_ld, fmt, codes, scales, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

extern "C" size_t moe_route_workspace_bytes(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  const size_t nblk = ((size_t)T + kTokensPerRouteBlock - 1) / kTokensPerRouteBlock;
  return align_up(nblk * E * 4, 256) + align_up((size_t)T * k * 4, 256) + 256;
}

extern "C" moe_status_t moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                                  float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (!expert_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_assign)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_route_workspace_bytes(T, E, k);
  if (workspace_bytes < need || (!workspace && need > 0)) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_INVALID_ARG;
  moe_status_t a = check_arch();
  if (a != MOE_OK) return a;
  const size_t nblk = ((size_t)T + kTokensPerRouteBlock - 1) / kTokensPerRouteBlock;
  char* ws = (char*)workspace;
  int32_t* hist = (int32_t*)ws;
  int32_t* rank = (int32_t*)(ws + align_up(nblk * E * 4, 256));
  if (T <= kSmallFusedRouteTokens && k <= 64)
    return launch_route_permute_small(logits, T, E, k, topk_ids, topk_w, 0, E, expert_offsets, sorted_assign,
                                      nullptr, nullptr, nullptr, 0, stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
  if (launch_topk(logits, T, E, k, topk_ids, topk_w, stream) != hipSuccess) return MOE_ERR_HIP;
  if (launch_permute(topk_ids, nullptr, T, k, 0, E, hist, rank, expert_offsets, sorted_assign, nullptr, nullptr,
                     nullptr, 0,
                     stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" size_t moe_fused_workspace_bytes(const moe_problem_t* p) {
  if (!p || p->T < 0 || p->E < 1 || p->k < 1 || p->H <= 0 || p->I <= 0 || p->I_shared < 0) return 0;
  return plan(*p).total;
}

// ----------------------------------------------------------- dense GEMM --

// Kernel and M-tile height of a dense GEMM C[M, N] = A W^T with K = K on the
// FC2 instantiations (bf16 rows of dense_weight * A W^T): the families that
// the layer's shared expert takes, where N fits their N-blocks; the stream
// kernels (16-row tiles, N masked to a multiple of 8) otherwise.
static Fc dense_kind(int64_t M, int64_t N, int64_t K, bool mx, mx_elem_t wf, int grid, int* rows) {
  *rows = kStreamRows;
  if (mx) {
    if (M >= kTiledMinRowsPerExpert && K % kTiledKMultiple == 0) {
      if (wf == MX_E2M1 && K % 512 == 0 && K >= 1024 && N % kWideCols == 0 && (double)M * K < 4294967296.0) {
        *rows = kTiledRows;
        return Fc::kWide;
      }
      const int r = dense_tiled_rows((int)M, (int)N, false, grid);
      for (const int rr : {r, r == kTiledRows ? kTiledRowsLow : kTiledRows}) {
        if (N % tiled_weight_rows(rr) == 0) {
          *rows = rr;
          return Fc::kTiled;
        }
      }
    }
    return Fc::kStream;
  }
  if (wf == MX_E2M1) {
    if (M >= kMidMinRowsPerExpert && K % kMidK == 0 && N % kWideCols == 0) {
      *rows = M >= kMidHighMinRowsPerExpert ? kMidRowsHigh : kMidRows;
      return Fc::kMid;
    }
    if (K % kSmallK == 0 && N % kSmallColsFc2 == 0) return Fc::kSmall;
  }
  return Fc::kStream;
}

// K split of a dense GEMM on the small-M kernel (bf16 activations, E2M1
// weights, few rows): the number of equal K ranges, each of whole stages and at
// least two, that best fills kSplitTargetItems workgroup items (ties: fewer
// ranges); 1 when the items already fill them.  A function of the shape only,
// so that the workspace size does not depend on the device.
constexpr int kSplitTargetItems = 256;
static int dense_ksplit(int64_t M, int64_t N, int64_t K, moe_act_t act, mx_elem_t wf) {
  if (act != MOE_ACT_BF16 || wf != MX_E2M1 || M <= 0 || M >= kMidMinRowsPerExpert) return 1;
  if (K % kSmallK || N % kSmallColsFc2 || N % 4) return 1;
  const int64_t items = (M + kStreamRows - 1) / kStreamRows * (N / kSmallColsFc2);
  if (items * 2 > kSplitTargetItems) return 1;
  const int64_t nk = K / kSmallK;
  int best = 1;
  double best_fill = (double)items / kSplitTargetItems;
  for (int64_t s = 2; s <= nk / 2 && s <= 64; ++s) {
    if (nk % s) continue;
    const int64_t n = items * s;
    const double fill = (double)n / (double)(((n + kSplitTargetItems - 1) / kSplitTargetItems) * kSplitTargetItems);
    if (fill > best_fill + 1e-9) {
      best = (int)s;
      best_fill = fill;
    }
  }
  return best;
}

static size_t gemm_quant_bytes(int64_t M, int64_t K) {
  return align_up((size_t)(M * K), 256) + align_up((size_t)(M * K / 32), 256);
}

extern "C" size_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, moe_act_t act, mx_elem_t w_fmt) {
  if (M < 0 || N <= 0 || K <= 0 || K % 32) return 0;
  if (act == MOE_ACT_MXFP8) return gemm_quant_bytes(M, K);
  const int s = dense_ksplit(M, N, K, act, w_fmt);
  return s > 1 ? align_up((size_t)s * (size_t)M * (size_t)N * 4, 256) : 0;
}

extern "C" moe_status_t mx_gemm(const void* a, const uint8_t* a_scale, int64_t M, int64_t N, int64_t K,
                                moe_act_t act, const uint8_t* w, const uint8_t* w_scale, mx_elem_t w_fmt,
                                float alpha, void* c, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (act != MOE_ACT_BF16 && act != MOE_ACT_MXFP8) return MOE_ERR_INVALID_ARG;
  if (w_fmt != MX_E2M1 && w_fmt != MX_E3M2 && w_fmt != MX_E4M3) return MOE_ERR_INVALID_ARG;
  if (act == MOE_ACT_BF16 && a_scale) return MOE_ERR_INVALID_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || (double)M * N > 9.0e15) return MOE_ERR_INVALID_ARG;
  if (M > 0) {
    if (!a || !w || !w_scale || !c) return MOE_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(w) || !aligned16(c) || (a_scale && !aligned16(a_scale)))
      return MOE_ERR_INVALID_ARG;
  }
  if (w_fmt == MX_E4M3 || N % 8 || K % 128) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  const bool quant = act == MOE_ACT_MXFP8 && !a_scale;
  const size_t need = quant ? gemm_quant_bytes(M, K) : 0;
  if (quant && (workspace_bytes < need || !workspace)) return MOE_ERR_WORKSPACE;
  if (quant && ((uintptr_t)workspace & 255u) != 0) return MOE_ERR_INVALID_ARG;
  // a K split only when the caller's workspace holds its partial sums
  int ksplit = dense_ksplit(M, N, K, act, w_fmt);
  if (ksplit > 1 && (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
                     workspace_bytes < (size_t)ksplit * (size_t)M * (size_t)N * 4))
    ksplit = 1;
  moe_status_t st = check_arch();
  if (st != MOE_OK) return st;

  const bool mx = act == MOE_ACT_MXFP8;
  const uint8_t* codes = (const uint8_t*)a;
  const uint8_t* scales = a_scale;
  if (quant) {
    uint8_t* qc = (uint8_t*)workspace;
    uint8_t* qs = qc + align_up((size_t)(M * K), 256);
    if (launch_quantize(a, MOE_SRC_BF16, M, K, K, MX_E4M3, qc, qs, stream) != hipSuccess) return MOE_ERR_HIP;
    codes = qc;
    scales = qs;
  }
  const int cus = device_cus();
  const int tgrid = cus < 8 ? 8 : cus & ~7;
  int rows = 0;
  const Fc kind = dense_kind(M, N, K, mx, w_fmt, tgrid, &rows);
  FcArgs g = {};
  g.dense_rows = (int)M;
  g.dense_weight = alpha;
  g.k = 1;
  g.a = mx ? (const void*)codes : a;
  g.a_scale = scales;
  g.w = w;
  g.w_scale = w_scale;
  g.K = (int)K;
  g.N = (int)N;
  const int cols = fc_cols(kind, false, rows);
  g.nchunks = (int)((N + cols - 1) / cols);  // the stream kernels mask the last chunk's columns
  g.obuf = (uint16_t*)c;
  if (kind == Fc::kSmall && ksplit > 1) {
    g.ksplit = ksplit;
    g.part = (float*)workspace;
  }
  const int wf = w_fmt == MX_E2M1 ? 1 : 2;
  hipError_t e = hipSuccess;
  switch (kind) {
    case Fc::kSmall:
      e = launch_fc_small(g, false, cus, stream);
      if (e == hipSuccess && g.ksplit > 1) e = launch_splitk_reduce(g.part, g.ksplit, M * N / 4, alpha, (uint16_t*)c, stream);
      break;
    case Fc::kMid: e = launch_fc_mid(g, false, rows, cus, stream); break;
    case Fc::kWide: e = launch_fc_wide(g, false, cus, stream); break;
    case Fc::kTiled: e = launch_fc_tiled(g, false, wf, rows, cus, stream); break;
    default: e = launch_fc_stream(g, false, mx, wf, stream); break;
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" size_t moe_fused_workspace_offset(const moe_problem_t* p, moe_ws_part_t part) {
  const size_t none = ~(size_t)0;
  if (!p || p->T < 0 || p->E < 1 || p->k < 1 || p->k > p->E || p->H <= 0 || p->I <= 0 || p->I_shared < 0)
    return none;
  const int L = p->local_num_experts == 0 ? p->E : p->local_num_experts;
  if (p->local_expert_offset < 0 || L < 0 || (int64_t)p->local_expert_offset + L > p->E) return none;
  const FusedPlan f = plan(*p);
  switch (part) {
    case MOE_WS_EXPERT_OFFSETS: return f.offsets;
    case MOE_WS_SORTED_ASSIGN: return f.sorted;
    case MOE_WS_H: return f.h;
    case MOE_WS_H_SCALE: return p->act == MOE_ACT_MXFP8 ? f.hsc : none;
  }
  return none;
}

extern "C" moe_status_t moe_fused(const moe_problem_t* p, const moe_tensors_t* t, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  moe_status_t v = validate(p, t);
  if (v != MOE_OK) return v;
  if (p->T == 0) return MOE_OK;
  const FusedPlan f = plan(*p);
  if (!workspace || workspace_bytes < f.total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_INVALID_ARG;
  moe_status_t a = check_arch();
  if (a != MOE_OK) return a;

  char* ws = (char*)workspace;
  const bool mx = p->act == MOE_ACT_MXFP8;
  const int wf = p->w_fmt == MX_E2M1 ? 1 : 2;
  const int T = p->T, H = p->H, I = p->I, k = p->k, Is = p->I_shared;
  uint16_t* obuf = (uint16_t*)(ws + f.obuf);
  uint16_t* sbuf = Is ? (uint16_t*)(ws + f.sbuf) : nullptr;
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t r) {
    if (r != hipSuccess && e == hipSuccess) e = r;
    return r == hipSuccess;
  };
  // optional instrumentation: event i marks the start of stage i
  auto mark = [&](int stage) {
    return t->stage_events == nullptr || hipEventRecord(t->stage_events[stage], stream) == hipSuccess;
  };
  if (!mark(MOE_STAGE_ROUTE)) return MOE_ERR_HIP;

  if (f.micro) {
    // small batch: routing + FC1 in one kernel, FC2 + combine (+ shared) in another
    const int64_t bh = (int64_t)H / 2, bi = (int64_t)I / 2;
    MicroArgs m = {};
    m.logits = t->topk_ids_in ? nullptr : t->router_logits;
    m.ids_in = t->topk_ids_in;
    m.w_in = t->topk_w_in;
    m.T = T;
    m.E = p->E;
    m.k = k;
    m.off = f.off;
    m.L = f.L;
    m.ids_out = t->topk_ids_out;
    m.w_out = t->topk_w_out;
    m.x = t->x;
    m.H = H;
    m.I = I;
    m.Is = Is;
    m.act_fn = p->act_fn;
    m.w1 = t->w1;
    m.s1 = t->w1_scale;
    m.w1_estride = 2 * (int64_t)I * bh;
    m.s1_estride = 2 * (int64_t)I * (H / 32);
    m.ws1 = t->ws1;
    m.ss1 = t->ws1_scale;
    m.h = (uint16_t*)(ws + f.h);
    m.hs = Is ? (uint16_t*)(ws + f.hs) : nullptr;
    m.list = (MicroList*)(ws + f.micro_list);
    m.w2 = t->w2;
    m.s2 = t->w2_scale;
    m.w2_estride = (int64_t)H * bi;
    m.s2_estride = (int64_t)H * (I / 32);
    m.ws2 = t->ws2;
    m.ss2 = t->ws2_scale;
    m.shared_weight = p->shared_weight;
    m.y = (uint16_t*)t->y;
    // stages: routing, permutation and FC1 are the first kernel; FC2, the
    // shared expert and the combine the second
    if (!mark(MOE_STAGE_PERMUTE) || !mark(MOE_STAGE_QUANT_X) || !mark(MOE_STAGE_FC1)) return MOE_ERR_HIP;
    const hipEvent_t fc2 = t->stage_events ? t->stage_events[MOE_STAGE_FC2] : nullptr;
    if (launch_micro(m, device_cus(), stream, fc2) != hipSuccess) return MOE_ERR_HIP;
    if (!mark(MOE_STAGE_SHARED) || !mark(MOE_STAGE_FINALIZE) || !mark(MOE_NUM_STAGES)) return MOE_ERR_HIP;
    return MOE_OK;
  }

  // 1. routing
  const int32_t* ids;
  const float* wts;
  int32_t* sorted = (int32_t*)(ws + f.sorted);
  Tile* tiles = (Tile*)(ws + f.tiles);
  int32_t* ntiles = (int32_t*)(ws + f.ntiles);
  float* sorted_w = (float*)(ws + f.sorted_w);
  // a few tokens on the small-M kernel: its FC1 routes the batch itself (no
  // routing launch; k <= 64: one 64-lane selection round per token);
  // otherwise, for a few tokens, top-k and the permutation in one workgroup
  const bool route_in_fc1 = !t->topk_ids_in && !mx && f.routed == Fc::kSmall && T <= kSmallRoutedTokens &&
                            k <= 64 && (int64_t)T * k <= kSmallRoutedAssign;
  const bool fused_route = !route_in_fc1 && !t->topk_ids_in && T <= kSmallFusedRouteTokens && k <= 64;
  if (route_in_fc1) {
    ids = t->topk_ids_out ? t->topk_ids_out : (int32_t*)(ws + f.ids);
    wts = t->topk_w_out ? t->topk_w_out : (float*)(ws + f.w);
  } else if (fused_route) {
    int32_t* ids_w = t->topk_ids_out ? t->topk_ids_out : (int32_t*)(ws + f.ids);
    float* w_w = t->topk_w_out ? t->topk_w_out : (float*)(ws + f.w);
    if (!ok(launch_route_permute_small(t->router_logits, T, p->E, k, ids_w, w_w, f.off, f.L,
                                       (int32_t*)(ws + f.offsets), sorted, sorted_w, tiles, ntiles, f.bm, stream)))
      return MOE_ERR_HIP;
    ids = ids_w;
    wts = w_w;
  } else if (t->topk_ids_in) {
    ids = t->topk_ids_in;
    wts = t->topk_w_in;
    if (t->topk_ids_out || t->topk_w_out) {
      k_copy_routing<<<grid_for(f.A, 256, 1 << 30), 256, 0, stream>>>(ids, wts, t->topk_ids_out, t->topk_w_out, f.A);
      if (!ok(hipGetLastError())) return MOE_ERR_HIP;
    }
  } else {
    int32_t* ids_w = t->topk_ids_out ? t->topk_ids_out : (int32_t*)(ws + f.ids);
    float* w_w = t->topk_w_out ? t->topk_w_out : (float*)(ws + f.w);
    if (!ok(launch_topk(t->router_logits, T, p->E, k, ids_w, w_w, stream))) return MOE_ERR_HIP;
    ids = ids_w;
    wts = w_w;
  }
  // 2. permutation by local expert + tile list (done above for a few tokens)
  if (!mark(MOE_STAGE_PERMUTE)) return MOE_ERR_HIP;
  if (!fused_route && !route_in_fc1 &&
      !ok(launch_permute(ids, wts, T, k, f.off, f.L, (int32_t*)(ws + f.hist), (int32_t*)(ws + f.rank),
                         (int32_t*)(ws + f.offsets), sorted, sorted_w, tiles, ntiles, f.bm, stream)))
    return MOE_ERR_HIP;
  // 3. MXFP8 activations
  if (!mark(MOE_STAGE_QUANT_X)) return MOE_ERR_HIP;
  const uint8_t* xq = (const uint8_t*)(ws + f.xq);
  const uint8_t* xs = (const uint8_t*)(ws + f.xs);
  if (mx && !ok(launch_quantize(t->x, MOE_SRC_BF16, T, H, H, MX_E4M3, (uint8_t*)xq, (uint8_t*)xs, stream)))
    return MOE_ERR_HIP;

  const int64_t bytes_h = (int64_t)H * wbits(p->w_fmt) / 8;
  const int64_t bytes_i = (int64_t)I * wbits(p->w_fmt) / 8;
  // 4-5. FC1 + SiLU(gate)*up (+ MXFP8 requantization)
  if (!mark(MOE_STAGE_FC1)) return MOE_ERR_HIP;
  FcArgs a1 = {};
  a1.tiles = tiles;
  a1.num_tiles = ntiles;
  a1.max_tiles = f.max_tiles;
  a1.dense_rows = 0;
  a1.sorted_assign = sorted;
  a1.k = k;
  a1.kdiv = k > 1 ? (uint32_t)(((1ull << 32) + k - 1) / k) : 0u;  // unused for k = 1
  a1.topk_w = wts;
  a1.sorted_w = sorted_w;
  a1.a = mx ? (const void*)xq : t->x;
  a1.a_scale = xs;
  a1.w = t->w1;
  a1.w_scale = t->w1_scale;
  a1.w_estride = 2 * (int64_t)I * bytes_h;
  a1.ws_estride = 2 * (int64_t)I * (H / 32);
  a1.act_fn = p->act_fn;
  a1.K = H;
  a1.N = I;
  a1.nchunks = I / fc_cols(f.routed, true, f.bm);
  a1.out = ws + f.h;
  a1.out_scale = (uint8_t*)(ws + f.hsc);
  const int cus = device_cus();
  // rows: M-tile height (the routed tile list's, or the dense GEMM's)
  auto launch_fc = [&](const FcArgs& a, bool fc1, Fc kind, int rows) {
    switch (kind) {
      case Fc::kSmall: return launch_fc_small(a, fc1, cus, stream);
      case Fc::kMid: return launch_fc_mid(a, fc1, rows, cus, stream);
      case Fc::kWide: return launch_fc_wide(a, fc1, cus, stream);
      case Fc::kTiled: return launch_fc_tiled(a, fc1, wf, rows, cus, stream);
      default: return launch_fc_stream(a, fc1, mx, wf, stream);
    }
  };
  if (route_in_fc1) {
    a1.logits = t->router_logits;
    a1.T = T;
    a1.E = p->E;
    a1.off = f.off;
    a1.L = f.L;
    a1.ids_out = (int32_t*)ids;
    a1.w_out = (float*)wts;
    a1.offsets_out = (int32_t*)(ws + f.offsets);
    a1.sorted_out = sorted;
    a1.sorted_w_out = sorted_w;
    a1.tiles_out = tiles;
    a1.ntiles_out = ntiles;
    if (!ok(launch_fc_small_routed(a1, cus, stream))) return MOE_ERR_HIP;
  } else if (!ok(launch_fc(a1, true, f.routed, f.bm))) {
    return MOE_ERR_HIP;
  }
  // 6-7. FC2 + weighted combine into the fp32 accumulator
  if (!mark(MOE_STAGE_FC2)) return MOE_ERR_HIP;
  FcArgs a2 = a1;
  a2.logits = nullptr;
  a2.a = ws + f.h;
  a2.a_scale = (const uint8_t*)(ws + f.hsc);
  a2.w = t->w2;
  a2.w_scale = t->w2_scale;
  a2.w_estride = (int64_t)H * bytes_i;
  a2.ws_estride = (int64_t)H * (I / 32);
  a2.K = I;
  a2.N = H;
  a2.nchunks = H / fc_cols(f.routed, false, f.bm);
  a2.out = nullptr;
  a2.obuf = obuf;
  if (!ok(launch_fc(a2, false, f.routed, f.bm))) return MOE_ERR_HIP;
  // shared expert: a dense expert over all T tokens with its own weight
  if (!mark(MOE_STAGE_SHARED)) return MOE_ERR_HIP;
  if (Is > 0) {
    const bool st = f.shared == Fc::kTiled;
    const int tgrid = cus < 8 ? 8 : cus & ~7;  // the tiled kernel's grid
    const int rows1 = st ? dense_tiled_rows(T, Is, true, tgrid) : f.shared_bm;
    const int rows2 = st ? dense_tiled_rows(T, H, false, tgrid) : f.shared_bm;
    FcArgs s1 = a1;
    s1.logits = nullptr;
    s1.dense_rows = T;
    s1.w = t->ws1;
    s1.w_scale = t->ws1_scale;
    s1.w_estride = 0;
    s1.ws_estride = 0;
    s1.N = Is;
    s1.nchunks = Is / fc_cols(f.shared, true, rows1);
    s1.out = ws + f.hs;
    s1.out_scale = (uint8_t*)(ws + f.hssc);
    if (!ok(launch_fc(s1, true, f.shared, rows1))) return MOE_ERR_HIP;
    FcArgs s2 = a2;
    s2.dense_rows = T;
    s2.dense_weight = p->shared_weight;
    s2.a = ws + f.hs;
    s2.a_scale = (const uint8_t*)(ws + f.hssc);
    s2.w = t->ws2;
    s2.w_scale = t->ws2_scale;
    s2.w_estride = 0;
    s2.ws_estride = 0;
    s2.K = Is;
    s2.nchunks = H / fc_cols(f.shared, false, rows2);
    s2.obuf = sbuf;
    if (!ok(launch_fc(s2, false, f.shared, rows2))) return MOE_ERR_HIP;
  }
  // 8. y = bf16(accumulator)
  if (!mark(MOE_STAGE_FINALIZE)) return MOE_ERR_HIP;
  const int64_t n8 = (int64_t)T * H / 8;
  k_combine<<<grid_for(n8, 256, 16384), 256, 0, stream>>>((const uint4*)obuf, (const uint4*)sbuf, ids, k, f.off,
                                                          f.L, H / 8, n8, (uint4*)t->y);
  if (!ok(hipGetLastError())) return MOE_ERR_HIP;
  if (!mark(MOE_NUM_STAGES)) return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" moe_status_t moe_fused_noalloc(const moe_problem_t* p, const moe_tensors_t* t, hipStream_t stream) {
  moe_status_t v = validate(p, t);
  if (v != MOE_OK) return v;
  if (p->T == 0) return MOE_OK;
  if (plan(*p).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  moe_status_t a = check_arch();
  if (a != MOE_OK) return a;
  moe_status_t st = MOE_OK;
  void* ws = scratch_ptr(&st);
  if (!ws) return st;
  return moe_fused(p, t, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
