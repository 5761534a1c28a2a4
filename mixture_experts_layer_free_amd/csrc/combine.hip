// Combine (unpermute + gate-weighted sum) and the loss-free bias controller.
//
// Lesson "专家组合 (MoE)" (AI Engineering from Scratch): Concept (the layer
// adds gate * expert output over the chosen experts), Shared experts (their
// output is added for every token), Load balancing item 3 and Build it step 2
// (the bias moves by -gamma for over-used experts, +gamma for under-used).
#include "moe_common.h"

namespace {

// One wave per token: out[t] = shared[t] + sum_j gate[t,j] * y[row_of[t,j]],
// fp32, j ascending, 16-byte vectors along the row; the K row loads of a
// vector are issued together.  A slot whose row_of is negative (dropped by
// the expert capacity, or an invalid expert) adds nothing: its load goes to
// row 0 and the value is replaced by zero, never multiplied (y rows that no
// expert computed may hold anything).
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const f32x4* __restrict__ y, const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate, const f32x4* __restrict__ shared,
                                                      int64_t T, int64_t nv, void* __restrict__ out, int out_bf16) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myr = lane < K ? row_of[t * K + lane] : 0;
  const float myg = lane < K ? gate[t * K + lane] : 0.f;
  const f32x4* yr[K];
  float g[K];
  bool live[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = __shfl(myr, j, MOE_WAVE);
    live[j] = r >= 0;
    yr[j] = y + (int64_t)(live[j] ? r : 0) * nv;
    g[j] = __shfl(myg, j, MOE_WAVE);
  }
  for (int64_t v = lane; v < nv; v += MOE_WAVE) {
    f32x4 yv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const f32x4 l = __builtin_nontemporal_load(yr[j] + v);
      yv[j] = live[j] ? l : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 acc = shared ? shared[t * nv + v] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      acc[0] = fmaf(g[j], yv[j][0], acc[0]);
      acc[1] = fmaf(g[j], yv[j][1], acc[1]);
      acc[2] = fmaf(g[j], yv[j][2], acc[2]);
      acc[3] = fmaf(g[j], yv[j][3], acc[3]);
    }
    if (out_bf16) {
      uint2 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      static_cast<uint2*>(out)[t * nv + v] = o;
    } else {
      static_cast<f32x4*>(out)[t * nv + v] = acc;
    }
  }
}

__global__ void bias_update_kernel(float* __restrict__ b, const int32_t* __restrict__ counts, int E, int64_t Tk,
                                   float gamma) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)E * counts[e];
  if (load > Tk) b[e] = b[e] - gamma;
  else if (load < Tk) b[e] = b[e] + gamma;
}

}  // namespace

extern "C" moe_status moe_combine(const float* y_perm, const int32_t* row_of, const float* topk_gate, const float* shared_y,
                                  int64_t T, int k, int64_t d, void* out, int out_dtype, void* stream) {
  if (!y_perm || !row_of || !topk_gate || !out) return MOE_EINVAL;
  if (T < 1 || d < 1 || k < 1) return MOE_EINVAL;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_EINVAL;
  if (k > MOE_MAX_TOPK || d % 4 != 0) return MOE_ENOTSUP;
#define MOE_COMBINE(K)                                                                                      \
  combine_kernel<K><<<(unsigned)ceil_div(T, 4), 256, 0, moe_stream(stream)>>>(                              \
      reinterpret_cast<const f32x4*>(y_perm), row_of, topk_gate, reinterpret_cast<const f32x4*>(shared_y), T, d / 4, \
      out, out_dtype == MOE_BF16)
  MOE_DISPATCH_K(k, MOE_COMBINE);
#undef MOE_COMBINE
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_bias_update(float* sel_bias, const int32_t* counts, int E, int64_t T, int k, float gamma,
                                      void* stream) {
  if (!sel_bias || !counts) return MOE_EINVAL;
  if (E < 1 || T < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS) return MOE_ENOTSUP;
  bias_update_kernel<<<(unsigned)ceil_div(E, 256), 256, 0, moe_stream(stream)>>>(sel_bias, counts, E, T * k, gamma);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
