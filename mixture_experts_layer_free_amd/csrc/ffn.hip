// Grouped SwiGLU experts.
//
// Lesson "专家组合 (MoE)" (AI Engineering from Scratch), Concept: each expert
// is an independent FFN, usually SwiGLU; Shared experts: an always-on expert
// is the same FFN applied to every token.  The AREX article on The Ultimate
// MoE Training Handbook (paragraph on the expert-count sweet spot) notes that
// finer experts mean smaller GEMMs that cost step time: the kernels below are
// built so that many small, unequal expert GEMMs still fill the chip.
//
// bf16 path: two grouped GEMMs (gemm.h) on v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation, both "NT" (activations and nn.Linear weights are both
// contiguous along the reduction dimension):
//   up:   [G | U] = X W_gu^T, epilogue H = silu(G) * U (bf16), optionally G, U
//   down: Y = H W_down^T (fp32 out)
// The row-tile prefix sums are built on the device from the expert offsets
// (no host sync); the GEMM kernel is persistent and XCD-aware (gemm.h).
//
// Fused permute (moe_grouped_ffn_gather): the AREX article on The Ultimate
// MoE Training Handbook reports, in its paragraph on the handbook's section
// 3.7, that fusing the permute shrank the permute/copy kernels' share of the
// step.  Here the up-projection's operand loads fetch row token_of[r] of x
// for GEMM row r, so no permuted copy of x is written or read.
#include "gemm.h"

namespace {

// mt_prefix[g] = sum over g' < g of ceil(n_g' / bm); one workgroup.
__global__ __launch_bounds__(1024) void tile_schedule_kernel(const int32_t* __restrict__ offsets, int G, int bm,
                                                             int32_t* __restrict__ mt_prefix) {
  __shared__ int32_t s_wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = tid < G ? (offsets[tid + 1] - offsets[tid] + bm - 1) / bm : 0;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, MOE_WAVE);
    if (lane >= o) inc += u;
  }
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  if (tid < G) mt_prefix[tid] = base + inc - v;
  if (tid == G - 1) mt_prefix[G] = base + inc;
}

// ---------------------------------------------------------------------------
// K-grouped chunk schedule (see moe_gemm::KgPlan in gemm.h).  One workgroup
// of 1024 threads, one group per thread (G <= 1024).

__device__ __forceinline__ int block_excl_scan_1024(int v, int32_t* s_w, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, MOE_WAVE);
    if (lane >= o) inc += u;
  }
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += s_w[w];
    total += s_w[w];
  }
  __syncthreads();
  return base + inc - v;
}

__global__ __launch_bounds__(1024) void kg_schedule_kernel(const int32_t* __restrict__ offsets, int G, int C, int tpg,
                                                           int gmax, int32_t* __restrict__ ks) {
  __shared__ int32_t s_w[16];
  __shared__ int32_t s_rrows[1024];      // remainder rows (or -1: none), per group
  __shared__ int64_t s_rcost[1024];      // remainder chunk cost by rank, then its prefix sums
  const int e = threadIdx.x;
  const int64_t full_cost = (int64_t)C + moe_gemm::KG_OVERHEAD_ROWS;
  const int n = e < G ? offsets[e + 1] - offsets[e] : 0;
  const int q = n / C, r = n - q * C;
  const bool has_rem = e < G && (r > 0 || n == 0);   // an empty group keeps one (empty) chunk: its output is zeros
  const int nc = e < G ? q + (has_rem ? 1 : 0) : 0;
  const bool split = nc > 1;
  int Qtot, nslot, ns, nrem;
  const int fbase = block_excl_scan_1024(q, s_w, Qtot);
  const int sbase = block_excl_scan_1024(split ? nc : 0, s_w, nslot);
  const int sidx = block_excl_scan_1024(split ? 1 : 0, s_w, ns);
  (void)block_excl_scan_1024(has_rem ? 1 : 0, s_w, nrem);
  s_rrows[e] = has_rem ? r : -1;
  __syncthreads();
  // rank of this group's remainder chunk: more rows first, then the lower group
  int rank = 0;
  if (has_rem)
    for (int o = 0; o < G; ++o) {
      const int ro = s_rrows[o];
      rank += ro > r || (ro == r && o < e);
    }
  int32_t* g_e = ks + moe_gemm::KG_HDR;
  int32_t* g_kb = g_e + gmax;
  int32_t* g_ke = g_kb + gmax;
  int32_t* g_out = g_ke + gmax;
  int32_t* s_e = g_out + gmax;
  int32_t* s_s0 = s_e + G;
  int32_t* s_nc = s_s0 + G;
  const int off = e < G ? offsets[e] : 0;
  for (int c = 0; c < q; ++c) {
    const int g = fbase + c;
    g_e[g] = e;
    g_kb[g] = off + c * C;
    g_ke[g] = off + (c + 1) * C;
    g_out[g] = split ? sbase + c : -1;
  }
  if (has_rem) {
    const int g = Qtot + rank;
    g_e[g] = e;
    g_kb[g] = off + q * C;
    g_ke[g] = off + n;
    g_out[g] = split ? sbase + q : -1;
    s_rcost[rank] = (int64_t)((r + 63) / 64 * 64) + moe_gemm::KG_OVERHEAD_ROWS;
  }
  if (split) {
    s_e[sidx] = e;
    s_s0[sidx] = sbase;
    s_nc[sidx] = nc;
  }
  __syncthreads();
  // inclusive prefix of the remainder costs, in rank order (serial: at most G values)
  if (e == 0) {
    int64_t acc = 0;
    for (int i = 0; i < nrem; ++i) {
      acc += s_rcost[i];
      s_rcost[i] = acc;
    }
  }
  __syncthreads();
  const int ng = Qtot + nrem;
  // cost of the chunks before chunk g (each of its tpg tiles costs the chunk's cost)
  auto before = [&](int g) -> int64_t {
    if (g <= Qtot) return (int64_t)g * full_cost;
    return (int64_t)Qtot * full_cost + s_rcost[g - Qtot - 1];
  };
  if (e < 9) {
    int64_t item;
    if (e == 0) {
      item = 0;
    } else if (e == 8) {
      item = (int64_t)ng * tpg;
    } else {
      const int64_t target = before(ng) * e / 8;   // in chunk-cost units (per tile)
      int lo = 0, hi = ng;                          // last chunk starting at or before target
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (before(mid) <= target) lo = mid; else hi = mid;
      }
      const int64_t cst = before(lo + 1) - before(lo);
      const int64_t t = cst > 0 ? ((target - before(lo)) * tpg + cst - 1) / cst : 0;
      item = (int64_t)lo * tpg + (t < tpg ? t : tpg);
    }
    ks[e] = (int32_t)item;
    if (e < 8) ks[9 + e] = (int32_t)item;
  }
  if (e == 0) {
    ks[17] = ns;
    ks[18] = ng;
    ks[19] = gmax;
  }
}

// out[e] = sum over the chunks c of split group e of partial[slot0 + c], in
// chunk order; grid-stride over (split group, 4-float vector).
__global__ __launch_bounds__(256) void kg_reduce_kernel(const int32_t* __restrict__ ks, int G,
                                                        const f32x4* __restrict__ partial, int64_t mn4,
                                                        f32x4* __restrict__ out, int64_t out_group4) {
  const int ns = ks[17], gmax = ks[19];
  const int32_t* s_e = ks + moe_gemm::KG_HDR + 4 * gmax;
  const int32_t* s_s0 = s_e + G;
  const int32_t* s_nc = s_s0 + G;
  const int64_t total = (int64_t)ns * mn4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int sgi = (int)(i / mn4);
    const int64_t v = i - (int64_t)sgi * mn4;
    const int64_t s0 = s_s0[sgi];
    const int nc = s_nc[sgi];
    f32x4 acc = __builtin_nontemporal_load(partial + s0 * mn4 + v);
    for (int c = 1; c < nc; ++c) acc += __builtin_nontemporal_load(partial + (s0 + c) * mn4 + v);
    __builtin_nontemporal_store(acc, out + (int64_t)s_e[sgi] * out_group4 + v);
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per output element, serial fp32 FMA along the
// reduction (used for fp32 layers, which are small).

__device__ __forceinline__ int group_of_row(const int32_t* __restrict__ offsets, int G, int row) {
  int lo = 0, hi = G;  // largest g with offsets[g] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// row_token (or null): GEMM row r reads row row_token[r] of X, which has
// x_total rows (an index outside [0, x_total) reads as a zero row)
__global__ __launch_bounds__(256) void ffn_up_f32_kernel(const float* __restrict__ X, int64_t rows, int64_t d,
                                                         const int32_t* __restrict__ row_token, int64_t x_total,
                                                         const int32_t* __restrict__ offsets, int G, int64_t f,
                                                         const float* __restrict__ Wgu, float* __restrict__ gu,
                                                         float* __restrict__ H) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * f) return;
  const int64_t row = id / f, n = id % f;
  if (row >= offsets[G]) return;   // rows past the last group (e.g. dropped by a capacity) are not touched
  const int g = group_of_row(offsets, G, (int)row);
  const int64_t xrow = row_token ? (int64_t)row_token[row] : row;
  const bool in = xrow >= 0 && xrow < x_total;
  const float* xr = X + (in ? xrow : 0) * d;
  const float* wg = Wgu + (int64_t)g * 2 * f * d + n * d;
  const float* wu = wg + f * d;
  float a = 0.f, b = 0.f;
  for (int64_t i = 0; in && i < d; ++i) {
    a = fmaf(xr[i], wg[i], a);
    b = fmaf(xr[i], wu[i], b);
  }
  H[row * f + n] = a / (1.0f + expf(-a)) * b;
  if (gu) {
    gu[row * 2 * f + n] = a;
    gu[row * 2 * f + f + n] = b;
  }
}

__global__ __launch_bounds__(256) void ffn_down_f32_kernel(const float* __restrict__ H, int64_t rows, int64_t d,
                                                           const int32_t* __restrict__ offsets, int G, int64_t f,
                                                           const float* __restrict__ Wd, float* __restrict__ Y) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * d) return;
  const int64_t row = id / d, n = id % d;
  if (row >= offsets[G]) return;
  const int g = group_of_row(offsets, G, (int)row);
  const float* hr = H + row * f;
  const float* w = Wd + (int64_t)g * d * f + n * f;
  float a = 0.f;
  for (int64_t j = 0; j < f; ++j) a = fmaf(hr[j], w[j], a);
  Y[row * d + n] = a;
}

// Expert weights in the order the 256 x 256 bf16 GEMM tile streams them
// (Args::b_packed): block (g, nb, s) holds, for r < 256, row rowmap(nb, r)
// of group g's [rows, K] weight, columns 32 s .. 32 s + 31 (64 bytes at
// r * 64 in the block); a row at or past `rows` is zero.  swiglu (the
// up-projection): column block nb holds gate rows nb*128 .. +127 and up
// rows f + nb*128 .. +127 in 32-row blocks alternating gate, up -- the
// order the SwiGLU tile pairs them in.  One 16-byte chunk per thread and
// step, written in order.
__global__ __launch_bounds__(256) void pack_b_kernel(const u32x4* __restrict__ src, int64_t G, int64_t rows,
                                                     int64_t K, int NB, int swiglu, int64_t f, u32x4* __restrict__ dst) {
  const int64_t nslab = K / 32;
  const int64_t total = G * NB * nslab * 1024;   // 16-byte chunks: 256 rows x 4 per block
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i & 3), r = (int)((i >> 2) & 255);
    int64_t b = i >> 10;
    const int64_t sl = b % nslab;
    b /= nslab;
    const int nb = (int)(b % NB);
    const int64_t g = b / NB;
    const int64_t n = swiglu ? ((r >> 5) & 1 ? f : 0) + (int64_t)nb * 128 + (r >> 6) * 32 + (r & 31)
                             : (int64_t)nb * 256 + r;
    dst[i] = n < rows ? src[((g * rows + n) * K + sl * 32) / 8 + c] : u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

size_t moe_ffn_workspace(int G) { return align256((size_t)(G + 1) * sizeof(int32_t)); }

namespace moe_gemm {
moe_status lds_attr(const void* fn, int bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int grid_for(int64_t tiles_upper, int per_cu) {
  const int max_wg = (per_cu * moe_num_cus()) & ~7;
  const int64_t t = (tiles_upper + 7) & ~int64_t(7);
  return (int)std::max<int64_t>(8, std::min<int64_t>(max_wg, t));
}
}  // namespace moe_gemm

namespace moe_gemm {
moe_status kg_schedule_launch(const int32_t* offsets, int G, const KgPlan& k, int32_t* sched, hipStream_t s) {
  kg_schedule_kernel<<<1, 1024, 0, s>>>(offsets, G, (int)k.chunk, (int)k.tpg, (int)k.gmax, sched);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status kg_reduce_launch(const int32_t* sched, const KgPlan& k, int G, const float* partial, float* out,
                            int64_t out_group, hipStream_t s) {
  // enough workgroups for the largest possible sum; most exit at once when
  // no group was split
  const int64_t work = std::min<int64_t>(k.smax / 2, G) * (k.mn / 4);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(2048, ceil_div(work, 256)));
  kg_reduce_kernel<<<grid, 256, 0, s>>>(sched, G, reinterpret_cast<const f32x4*>(partial), k.mn / 4,
                                         reinterpret_cast<f32x4*>(out), out_group / 4);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
}  // namespace moe_gemm

moe_status moe_tile_schedule_launch(const int32_t* offsets, int G, int bm, int32_t* mt_prefix, hipStream_t s) {
  tile_schedule_kernel<<<1, 1024, 0, s>>>(offsets, G, bm, mt_prefix);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Tile schedule plus the two bf16 expert GEMMs of a grouped SwiGLU FFN.
// row_token (or null): GEMM row r of the up-projection reads row
// row_token[r] of x_rows, which then has x_total rows.
// packed: wgu and wd are the tile-order copies of moe_pack_expert_weights
// (the 256 x 256 tile only).
namespace {

// Events for the next grouped FFN call of this host thread (moe_ffn_stage_events).
thread_local void* const* t_ffn_events = nullptr;

// Records stage event i of a grouped FFN call (when the caller asked for it).
moe_status ffn_mark(void* const* events, int i, hipStream_t s) {
  if (events && events[i] && hipEventRecord(static_cast<hipEvent_t>(events[i]), s) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_ffn_stage_events(void* const* events) {
  t_ffn_events = events;
  return MOE_OK;
}

moe_status moe_ffn_bf16_launch(const bf16_t* x_rows, int64_t rows, int64_t d, const int32_t* row_token, int64_t x_total,
                               const int32_t* offsets, int32_t* mt_prefix, int G, int64_t f, const bf16_t* wgu,
                               const bf16_t* wd, bf16_t* gu, bf16_t* h, float* y, hipStream_t s, bool packed,
                               void* const* events) {
  using namespace moe_gemm;
  const bool large = use_large_tile(f);
  if (packed && !large) return MOE_ENOTSUP;
  moe_status st = moe_tile_schedule_launch(offsets, G, large ? BM_LARGE : BM, mt_prefix, s);
  if (st != MOE_OK) return st;
  Args a{};
  a.A = x_rows;
  a.lda = d;
  a.B = wgu;
  a.ldb = d;
  a.b_group = 2 * f * d;
  a.b_rows = 2 * f;
  a.K = d;
  a.N = f;
  a.offsets = offsets;
  a.mt_prefix = mt_prefix;
  a.G = G;
  a.out = h;
  a.ldo = f;
  a.gu_out = gu;
  a.a_rows = row_token;
  a.a_rows_total = x_total;
  a.b_packed = packed;
  st = launch_gemm<true, true, false, EPI_SWIGLU>(a, large, rows, s);
  if (st == MOE_OK) st = ffn_mark(events, MOE_FFN_STAGE_UP, s);
  if (st != MOE_OK) return st;
  Args b{};
  b.A = h;
  b.lda = f;
  b.B = wd;
  b.ldb = f;
  b.b_group = d * f;
  b.b_rows = d;
  b.K = f;
  b.N = d;
  b.offsets = offsets;
  b.mt_prefix = mt_prefix;
  b.G = G;
  b.out = y;
  b.ldo = d;
  b.b_packed = packed;
  st = launch_gemm<true, true, false, EPI_F32>(b, large, rows, s);
  if (st != MOE_OK) return st;
  return ffn_mark(events, MOE_FFN_STAGE_DOWN, s);
}

namespace {

moe_status grouped_ffn_impl(const void* x, int64_t x_total, const int32_t* row_token, int64_t rows, int64_t d,
                            int dtype, const int32_t* offsets, int G, int64_t f, const void* w_gate_up,
                            const void* w_down, void* gu_saved, void* h, float* y, void* workspace,
                            size_t workspace_bytes, void* stream, bool packed = false) {
  void* const* events = t_ffn_events;   // one call's worth: taken here whatever the call returns
  t_ffn_events = nullptr;
  if (!x || !offsets || !w_gate_up || !w_down || !h || !y) return MOE_EINVAL;
  if (rows < 1 || d < 1 || f < 1 || G < 1 || x_total < 1) return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EINVAL;
  if (G > MOE_MAX_EXPERTS || rows >= (1ll << 31)) return MOE_ENOTSUP;
  hipStream_t s = moe_stream(stream);
  if (dtype == MOE_BF16) {
    if (d % 64 != 0 || f % 64 != 0) return MOE_ENOTSUP;
    if (2 * f * d * 2 >= (1ll << 31)) return MOE_ENOTSUP;   // one expert's weight must fit a buffer resource
    // gathered rows are addressed through one buffer resource over all of x
    if (row_token && x_total * d * 2 >= (1ll << 31)) return MOE_ENOTSUP;
    if (!workspace || workspace_bytes < moe_ffn_workspace(G)) return MOE_EWORKSPACE;
    int32_t* mt_prefix = static_cast<int32_t*>(workspace);
    return moe_ffn_bf16_launch(static_cast<const bf16_t*>(x), rows, d, row_token, x_total, offsets, mt_prefix, G, f,
                               static_cast<const bf16_t*>(w_gate_up), static_cast<const bf16_t*>(w_down),
                               static_cast<bf16_t*>(gu_saved), static_cast<bf16_t*>(h), y, s, packed, events);
  }
  if (packed) return MOE_ENOTSUP;   // packed weights: bf16 only
  if (d % 4 != 0) return MOE_ENOTSUP;
  ffn_up_f32_kernel<<<(unsigned)ceil_div(rows * f, 256), 256, 0, s>>>(
      static_cast<const float*>(x), rows, d, row_token, x_total, offsets, G, f, static_cast<const float*>(w_gate_up),
      static_cast<float*>(gu_saved), static_cast<float*>(h));
  MOE_LAUNCH_CHECK();
  moe_status st = ffn_mark(events, MOE_FFN_STAGE_UP, s);
  if (st != MOE_OK) return st;
  ffn_down_f32_kernel<<<(unsigned)ceil_div(rows * d, 256), 256, 0, s>>>(static_cast<const float*>(h), rows, d, offsets, G,
                                                                        f, static_cast<const float*>(w_down), y);
  MOE_LAUNCH_CHECK();
  return ffn_mark(events, MOE_FFN_STAGE_DOWN, s);
}

}  // namespace

extern "C" moe_status moe_grouped_ffn(const void* x_rows, int64_t rows, int64_t d, int dtype, const int32_t* offsets, int G,
                                      int64_t f, const void* w_gate_up, const void* w_down, void* gu_saved, void* h, float* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_ffn_impl(x_rows, rows, nullptr, rows, d, dtype, offsets, G, f, w_gate_up, w_down, gu_saved, h, y,
                          workspace, workspace_bytes, stream);
}

extern "C" moe_status moe_grouped_ffn_gather(const void* x, int64_t T, const int32_t* token_of, int64_t rows, int64_t d,
                                             int dtype, const int32_t* offsets, int G, int64_t f, const void* w_gate_up,
                                             const void* w_down, void* gu_saved, void* h, float* y, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  if (!token_of) return MOE_EINVAL;
  return grouped_ffn_impl(x, T, token_of, rows, d, dtype, offsets, G, f, w_gate_up, w_down, gu_saved, h, y, workspace,
                          workspace_bytes, stream);
}

extern "C" size_t moe_packed_weight_bytes(int which, int64_t G, int64_t d, int64_t f) {
  if (G < 1 || d < 1 || f < 1) return 0;
  if (which == 0) return (size_t)G * 2 * f * d * 2;                 // f/128 column blocks, d/32 slabs of 16 KB
  if (which == 1) return (size_t)G * ceil_div(d, 256) * 256 * f * 2;   // ceil(d/256) column blocks, f/32 slabs
  return 0;
}

extern "C" moe_status moe_pack_expert_weights(const void* w_gate_up, const void* w_down, int64_t G, int64_t d,
                                              int64_t f, void* packed_gate_up, void* packed_down, void* stream) {
  if (!w_gate_up || !w_down || !packed_gate_up || !packed_down) return MOE_EINVAL;
  if (G < 1 || d < 1 || f < 1) return MOE_EINVAL;
  if (G > MOE_MAX_EXPERTS || d % 64 != 0 || f % 128 != 0) return MOE_ENOTSUP;
  hipStream_t s = moe_stream(stream);
  const int nb_gu = (int)(f / 128), nb_d = (int)ceil_div(d, 256);
  auto grid = [](int64_t chunks) { return (unsigned)std::min<int64_t>(65536, std::max<int64_t>(1, ceil_div(chunks, 256))); };
  pack_b_kernel<<<grid(G * nb_gu * (d / 32) * 1024), 256, 0, s>>>(static_cast<const u32x4*>(w_gate_up), G, 2 * f, d,
                                                                 nb_gu, 1, f, static_cast<u32x4*>(packed_gate_up));
  MOE_LAUNCH_CHECK();
  pack_b_kernel<<<grid(G * nb_d * (f / 32) * 1024), 256, 0, s>>>(static_cast<const u32x4*>(w_down), G, d, f, nb_d, 0,
                                                                f, static_cast<u32x4*>(packed_down));
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_grouped_ffn_packed(const void* x, int64_t T, const int32_t* token_of, int64_t rows,
                                             int64_t d, const int32_t* offsets, int G, int64_t f,
                                             const void* packed_gate_up, const void* packed_down, void* gu_saved,
                                             void* h, float* y, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (f % 128 != 0) return MOE_ENOTSUP;
  return grouped_ffn_impl(x, token_of ? T : rows, token_of, rows, d, MOE_BF16, offsets, G, f, packed_gate_up,
                          packed_down, gu_saved, h, y, workspace, workspace_bytes, stream, true);
}
