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

moe_status moe_tile_schedule_launch(const int32_t* offsets, int G, int bm, int32_t* mt_prefix, hipStream_t s) {
  tile_schedule_kernel<<<1, 1024, 0, s>>>(offsets, G, bm, mt_prefix);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Tile schedule plus the two bf16 expert GEMMs of a grouped SwiGLU FFN.
// row_token (or null): GEMM row r of the up-projection reads row
// row_token[r] of x_rows, which then has x_total rows.
moe_status moe_ffn_bf16_launch(const bf16_t* x_rows, int64_t rows, int64_t d, const int32_t* row_token, int64_t x_total,
                               const int32_t* offsets, int32_t* mt_prefix, int G, int64_t f, const bf16_t* wgu,
                               const bf16_t* wd, bf16_t* gu, bf16_t* h, float* y, hipStream_t s) {
  using namespace moe_gemm;
  const bool large = use_large_tile(f);
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
  st = launch_gemm<true, true, false, EPI_SWIGLU>(a, large, rows, s);
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
  return launch_gemm<true, true, false, EPI_F32>(b, large, rows, s);
}

namespace {

moe_status grouped_ffn_impl(const void* x, int64_t x_total, const int32_t* row_token, int64_t rows, int64_t d,
                            int dtype, const int32_t* offsets, int G, int64_t f, const void* w_gate_up,
                            const void* w_down, void* gu_saved, void* h, float* y, void* workspace,
                            size_t workspace_bytes, void* stream) {
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
                               static_cast<bf16_t*>(gu_saved), static_cast<bf16_t*>(h), y, s);
  }
  if (d % 4 != 0) return MOE_ENOTSUP;
  ffn_up_f32_kernel<<<(unsigned)ceil_div(rows * f, 256), 256, 0, s>>>(
      static_cast<const float*>(x), rows, d, row_token, x_total, offsets, G, f, static_cast<const float*>(w_gate_up),
      static_cast<float*>(gu_saved), static_cast<float*>(h));
  MOE_LAUNCH_CHECK();
  ffn_down_f32_kernel<<<(unsigned)ceil_div(rows * d, 256), 256, 0, s>>>(static_cast<const float*>(h), rows, d, offsets, G,
                                                                        f, static_cast<const float*>(w_down), y);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
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
