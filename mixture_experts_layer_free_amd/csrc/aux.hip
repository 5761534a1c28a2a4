// Auxiliary load-balancing loss and the dense router gradient it needs.
//
// Lesson "专家组合 (MoE)", Load balancing item 1 and Key terms: an extra loss
// term that penalises uneven expert usage (a hyperparameter and a second
// gradient signal).  The pages give no formula; the Switch/GShard form is
// used:
//   L_aux = alpha * E / (T*k) * sum_e counts[e] * P[e],  P[e] = mean_t p[t,e]
// with p the router probabilities over all E experts (softmax of the logits
// for softmax scoring, each score over the sum of all E scores otherwise)
// and counts the top-k assignments (held fixed).  Its gradient reaches every
// logit, so with it on the router weight gradient and the router part of dx
// use the dense [T, E] logit gradient.  Every reduction here runs in a fixed
// order: results are bit-reproducible.
#include "aux.h"

#include <float.h>

namespace {

constexpr int AUX_TPC = 256;                            // tokens per probability partial
constexpr int AUX_NV = MOE_MAX_EXPERTS / MOE_WAVE;      // experts per lane
constexpr int DW_TCH = 512;                             // tokens per router-wgrad partial
constexpr int DW_EB = 64;                               // experts per router-wgrad workgroup

__device__ __forceinline__ float aux_score(float l, int fn) {
  if (fn == MOE_SIGMOID_NORM) return 1.0f / (1.0f + expf(-l));
  return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));   // MOE_SQRT_SOFTPLUS_NORM
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

// p[t, e] for the experts e = lane + 64*m held by this lane (0 past E).
__device__ __forceinline__ void token_probs(const float* __restrict__ lrow, int E, int fn, float (&p)[AUX_NV]) {
  const int lane = threadIdx.x & 63;
  if (fn == MOE_SOFTMAX_CHOSEN) {
    float m = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) {
      const int e = lane + MOE_WAVE * i;
      p[i] = e < E ? lrow[e] : -FLT_MAX;
      m = fmaxf(m, p[i]);
    }
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) {
      const int e = lane + MOE_WAVE * i;
      p[i] = e < E ? expf(p[i] - m) : 0.f;
      s += p[i];
    }
    const float inv = 1.0f / wave_sum(s);
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) p[i] *= inv;
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) {
      const int e = lane + MOE_WAVE * i;
      p[i] = e < E ? aux_score(lrow[e], fn) : 0.f;
      s += p[i];
    }
    const float S = wave_sum(s);
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) p[i] /= S;
  }
}

// part[c][e] = sum of p[t, e] over the AUX_TPC tokens of chunk c: wave w sums
// its tokens c*AUX_TPC + w + 4i in order, the 4 waves are added in order.
__global__ __launch_bounds__(256) void aux_prob_partial_kernel(const float* __restrict__ logits, int T, int E, int fn,
                                                               float* __restrict__ part) {
  __shared__ float s_acc[4][MOE_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[AUX_NV];
#pragma unroll
  for (int i = 0; i < AUX_NV; ++i) acc[i] = 0.f;
  for (int q = wave; q < AUX_TPC; q += 4) {
    const int t = blockIdx.x * AUX_TPC + q;
    if (t >= T) break;
    float p[AUX_NV];
    token_probs(logits + (int64_t)t * E, E, fn, p);
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) acc[i] += p[i];
  }
#pragma unroll
  for (int i = 0; i < AUX_NV; ++i) {
    const int e = lane + MOE_WAVE * i;
    if (e < E) s_acc[wave][e] = acc[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    part[(int64_t)blockIdx.x * E + e] = (s_acc[0][e] + s_acc[1][e]) + (s_acc[2][e] + s_acc[3][e]);
}

// One workgroup of 1024 threads (E <= 1024): P[e] = sum of the partials in
// order / T; L = alpha * E/(T*k) * sum_e counts[e] * P[e].
__global__ __launch_bounds__(1024) void aux_loss_final_kernel(const float* __restrict__ part, int nchunks,
                                                              const int32_t* __restrict__ counts, int T, int E, int k,
                                                              float alpha, float* __restrict__ loss,
                                                              float* __restrict__ p_mean) {
  __shared__ float s_w[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  float P = 0.f;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) P += part[(int64_t)c * E + e];
    P /= (float)T;
    if (p_mean) p_mean[e] = P;
  }
  float v = e < E ? (float)counts[e] * P : 0.f;
  v = wave_sum(v);
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  if (e == 0) {
    float s = 0.f;
    for (int w = 0; w < 16; ++w) s += s_w[w];
    loss[0] = alpha * (float)E / ((float)T * (float)k) * s;
  }
}

// Dense logit gradient of one token (one wave): the aux part on every expert
// plus the main-loss dl of the chosen experts.
__global__ __launch_bounds__(256) void aux_dl_dense_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                           int T, int E, int k, int fn, float alpha,
                                                           float* __restrict__ dl_dense) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lrow = logits + (int64_t)t * E;
  float p[AUX_NV];
  token_probs(lrow, E, fn, p);
  const float cs = alpha * (float)E / ((float)T * (float)k) / (float)T;   // dL/dp[t,e] = cs * counts[e]
  float c[AUX_NV];
  float pc = 0.f;
#pragma unroll
  for (int i = 0; i < AUX_NV; ++i) {
    const int e = lane + MOE_WAVE * i;
    c[i] = e < E ? cs * (float)counts[e] : 0.f;
    pc += p[i] * c[i];
  }
  pc = wave_sum(pc);
  float Sinv = 0.f;
  if (fn != MOE_SOFTMAX_CHOSEN) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < AUX_NV; ++i) {
      const int e = lane + MOE_WAVE * i;
      s += e < E ? aux_score(lrow[e], fn) : 0.f;
    }
    Sinv = 1.0f / wave_sum(s);
  }
  const int myi = lane < k ? idx[(int64_t)t * k + lane] : -1;
  const float myl = lane < k ? dl[(int64_t)t * k + lane] : 0.f;
#pragma unroll
  for (int i = 0; i < AUX_NV; ++i) {
    const int e = lane + MOE_WAVE * i;
    float g;
    if (fn == MOE_SOFTMAX_CHOSEN) {
      g = p[i] * (c[i] - pc);
    } else {
      const float l = e < E ? lrow[e] : 0.f;
      const float ds = (c[i] - pc) * Sinv;
      if (fn == MOE_SIGMOID_NORM) {
        const float s = 1.0f / (1.0f + expf(-l));
        g = ds * s * (1.0f - s);
      } else {
        g = ds * (1.0f / (1.0f + expf(-l))) / (2.0f * aux_score(l, fn));
      }
    }
    for (int j = 0; j < k; ++j) {   // add the main-loss dl if e is chosen (a token holds e at most once)
      const int ej = __shfl(myi, j, MOE_WAVE);
      const float lj = __shfl(myl, j, MOE_WAVE);
      if (ej == e) g += lj;
    }
    if (e < E) dl_dense[(int64_t)t * E + e] = g;
  }
}

// part[p][e][c] = sum over the DW_TCH tokens of chunk p of dl_dense[t][e] * x[t][c]:
// one column per thread, DW_EB experts per workgroup, token order within the chunk.
__global__ __launch_bounds__(256) void router_dense_wgrad_part_kernel(const bf16_t* __restrict__ x,
                                                                      const float* __restrict__ dl_dense, int T, int E,
                                                                      int64_t d, float* __restrict__ part) {
  __shared__ float s_dl[64][DW_EB];
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * DW_EB;
  const int t0 = blockIdx.z * DW_TCH;
  float acc[DW_EB];
#pragma unroll
  for (int i = 0; i < DW_EB; ++i) acc[i] = 0.f;
  for (int tb = t0; tb < t0 + DW_TCH && tb < T; tb += 64) {
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * DW_EB; i += 256) {
      const int tt = tb + i / DW_EB, e = e0 + i % DW_EB;
      s_dl[i / DW_EB][i % DW_EB] = tt < T && e < E ? dl_dense[(int64_t)tt * E + e] : 0.f;
    }
    __syncthreads();
    const int nt = T - tb < 64 ? T - tb : 64;
    if (c < d) {
      for (int q = 0; q < nt; ++q) {
        const float xv = bf16_to_f32(x[(int64_t)(tb + q) * d + c]);
#pragma unroll
        for (int i = 0; i < DW_EB; ++i) acc[i] = fmaf(s_dl[q][i], xv, acc[i]);
      }
    }
  }
  if (c < d) {
    float* o = part + ((int64_t)blockIdx.z * E + e0) * d + c;
#pragma unroll
    for (int i = 0; i < DW_EB; ++i)
      if (e0 + i < E) o[(int64_t)i * d] = acc[i];
  }
}

__global__ __launch_bounds__(256) void router_dense_wgrad_reduce_kernel(const float* __restrict__ part, int nparts,
                                                                        int E, int64_t d, float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E * d) return;
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += part[(int64_t)p * E * d + i];
  dw[i] = s;
}

// dx[t] = sum_j dx_perm[row_of[t,j]] + sum_e dl_dense[t,e] * w_router[e]
// (dropped slots, row_of < 0, have no dx_perm row).
template <int K>
__global__ __launch_bounds__(256) void unpermute_bwd_dense_kernel(const u32x2* __restrict__ dx_perm,
                                                                  const int32_t* __restrict__ row_of,
                                                                  const float* __restrict__ dl_dense,
                                                                  const f32x4* __restrict__ w_router,
                                                                  const f32x4* __restrict__ extra, int T, int E,
                                                                  int64_t nv, f32x4* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myr = lane < K ? row_of[t * K + lane] : 0;
  const u32x2* xr[K];
  bool live[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = __shfl(myr, j, MOE_WAVE);
    live[j] = r >= 0;
    xr[j] = dx_perm + (int64_t)(live[j] ? r : 0) * nv;
  }
  const float* dlr = dl_dense + t * E;
  for (int64_t v = lane; v < nv; v += MOE_WAVE) {
    f32x4 acc = extra ? __builtin_nontemporal_load(extra + t * nv + v) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (live[j]) {
        const u32x2 b = xr[j][v];   // four bf16 of the row, summed in fp32
        acc += f32x4{bf16_to_f32(b[0] & 0xFFFFu), bf16_to_f32(b[0] >> 16), bf16_to_f32(b[1] & 0xFFFFu),
                     bf16_to_f32(b[1] >> 16)};
      }
    }
    for (int e = 0; e < E; ++e) {
      const float w = dlr[e];
      const f32x4 wr = w_router[(int64_t)e * nv + v];
      acc[0] = fmaf(w, wr[0], acc[0]);
      acc[1] = fmaf(w, wr[1], acc[1]);
      acc[2] = fmaf(w, wr[2], acc[2]);
      acc[3] = fmaf(w, wr[3], acc[3]);
    }
    dx[t * nv + v] = acc;
  }
}

}  // namespace

size_t moe_aux_workspace(int64_t T, int E) { return align256((size_t)ceil_div(T, AUX_TPC) * E * sizeof(float)); }

size_t moe_aux_bwd_workspace(int64_t T, int E, int64_t d) {
  return align256((size_t)T * E * sizeof(float)) + align256((size_t)ceil_div(T, DW_TCH) * E * d * sizeof(float));
}

moe_status moe_aux_backward_launch(const float* logits, const int32_t* counts, const int32_t* idx, const float* dl,
                                   const bf16_t* x, const float* w_router, const u32x4* dx_perm,
                                   const f32x4* extra, const int32_t* row_of, int64_t T, int E, int k, int64_t d,
                                   int fn, float alpha, float* dw_router, float* dx, void* ws, hipStream_t s) {
  float* dl_dense = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)T * E * sizeof(float)));
  aux_dl_dense_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(logits, counts, idx, dl, (int)T, E, k, fn, alpha,
                                                               dl_dense);
  MOE_LAUNCH_CHECK();
  const int nparts = (int)ceil_div(T, DW_TCH);
  router_dense_wgrad_part_kernel<<<dim3((unsigned)ceil_div(d, 256), (unsigned)ceil_div(E, DW_EB), (unsigned)nparts),
                                   256, 0, s>>>(x, dl_dense, (int)T, E, d, part);
  MOE_LAUNCH_CHECK();
  router_dense_wgrad_reduce_kernel<<<(unsigned)ceil_div((int64_t)E * d, 256), 256, 0, s>>>(part, nparts, E, d,
                                                                                            dw_router);
  MOE_LAUNCH_CHECK();
#define MOE_UBWD_DENSE(K)                                                                                  \
  unpermute_bwd_dense_kernel<K><<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(                                  \
      reinterpret_cast<const u32x2*>(dx_perm), row_of, dl_dense, reinterpret_cast<const f32x4*>(w_router),  \
      extra, (int)T, E, d / 4,                                                                              \
      reinterpret_cast<f32x4*>(dx))
  MOE_DISPATCH_K(k, MOE_UBWD_DENSE);
#undef MOE_UBWD_DENSE
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_aux_loss(const float* logits, const int32_t* counts, int64_t T, int E, int k, int score_fn,
                                   float alpha, float* loss_out, float* p_mean_out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!logits || !counts || !loss_out) return MOE_EINVAL;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (score_fn < MOE_SOFTMAX_CHOSEN || score_fn > MOE_SQRT_SOFTPLUS_NORM) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || T >= (1ll << 31)) return MOE_ENOTSUP;
  if (!workspace || workspace_bytes < moe_aux_workspace(T, E)) return MOE_EWORKSPACE;
  hipStream_t s = moe_stream(stream);
  const int nchunks = (int)ceil_div(T, AUX_TPC);
  float* part = static_cast<float*>(workspace);
  aux_prob_partial_kernel<<<(unsigned)nchunks, 256, 0, s>>>(logits, (int)T, E, score_fn, part);
  MOE_LAUNCH_CHECK();
  aux_loss_final_kernel<<<1, 1024, 0, s>>>(part, nchunks, counts, (int)T, E, k, alpha, loss_out, p_mean_out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
