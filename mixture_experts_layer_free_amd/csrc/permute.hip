// Permute: group the T*k (token, expert) assignments by expert, stably and
// without atomics, and copy each token's row to its k expert rows.
//
// The expert GEMMs want every expert's rows contiguous; this is the permute
// whose fusion the AREX article on The Ultimate MoE Training Handbook reports
// in its paragraph on hiding all-to-all (permute/copy kernels took 11.45% of
// the step unfused, 7.14% fused).
//
// Assignments are numbered i = t*k + j.  Chunks of 256 consecutive
// assignments (one workgroup, one assignment per lane) are the unit of the
// histogram.  Inside a wave, lanes holding the same expert find each other
// with one ballot per bit of the expert id (a match-any), which gives both the
// per-wave count and each lane's rank among equal experts in lane order.
// Lane order is assignment order, and a token never holds an expert twice, so
// ranks follow token order: the sort is stable and the result unique.
#include "moe_common.h"

namespace {

constexpr int PCH = 256;  // assignments per chunk (= threads per workgroup)

__device__ __forceinline__ int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// Lanes of this wave that hold the same expert as this lane (valid lanes only).
__device__ __forceinline__ uint64_t match_expert(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Per-chunk, per-wave expert counts into LDS; returns this lane's rank among
// the lanes of its wave with the same expert.
__device__ __forceinline__ int chunk_counts(const int32_t* __restrict__ idx, int64_t A, int E, int32_t (*s_cnt)[MOE_MAX_EXPERTS],
                                            int& e_out, bool& valid_out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * E; i += PCH) s_cnt[i / E][i % E] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * PCH + tid;
  const int ev = i < A ? idx[i] : 0;
  const bool valid = i < A && ev >= 0 && ev < E;   // out-of-range ids are dropped, never indexed
  const int e = valid ? ev : 0;
  const uint64_t m = match_expert(e, valid, bits_for(E));
  const int rank = __popcll(m & lanemask_lt());
  if (valid && rank == 0) s_cnt[wave][e] = __popcll(m);
  __syncthreads();
  e_out = e;
  valid_out = valid;
  return rank;
}

// hist[e * nchunks + c] = assignments of chunk c that chose expert e
__global__ __launch_bounds__(PCH) void perm_hist_kernel(const int32_t* __restrict__ idx, int64_t A, int E, int nchunks,
                                                        int32_t* __restrict__ hist) {
  __shared__ int32_t s_cnt[4][MOE_MAX_EXPERTS];
  int e;
  bool valid;
  chunk_counts(idx, A, E, s_cnt, e, valid);
  for (int x = threadIdx.x; x < E; x += PCH)
    hist[(int64_t)x * nchunks + blockIdx.x] = s_cnt[0][x] + s_cnt[1][x] + s_cnt[2][x] + s_cnt[3][x];
}

// Inclusive scan across one wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, MOE_WAVE);
    if (lane >= o) v += u;
  }
  return v;
}

// One workgroup of 1024 threads.  Each expert's column of the histogram is
// turned into exclusive chunk bases (within the expert); the expert totals
// become counts and their exclusive scan the offsets.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ hist, int E, int nchunks,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int32_t s_tot[MOE_MAX_EXPERTS];
  __shared__ int32_t s_wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = wave; e < E; e += 16) {
    int32_t* col = hist + (int64_t)e * nchunks;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < nchunks ? col[c] : 0;
      const int inc = wave_incl_scan(v);
      if (c < nchunks) col[c] = carry + inc - v;
      carry += __shfl(inc, 63, MOE_WAVE);
    }
    if (lane == 0) s_tot[e] = carry;
  }
  __syncthreads();
  // exclusive scan of s_tot[0..E) (E <= 1024: one value per thread)
  const int v = tid < E ? s_tot[tid] : 0;
  const int inc = wave_incl_scan(v);
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  if (tid < E) {
    counts[tid] = v;
    offsets[tid] = base + inc - v;
  }
  if (tid == E - 1) offsets[E] = base + inc;
}

// row_of[i] and token_of[row] for every assignment of chunk blockIdx.x.
__global__ __launch_bounds__(PCH) void perm_index_kernel(const int32_t* __restrict__ idx, int64_t A, int k, int E, int nchunks,
                                                         const int32_t* __restrict__ hist, const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ row_of, int32_t* __restrict__ token_of) {
  __shared__ int32_t s_cnt[4][MOE_MAX_EXPERTS];
  int e;
  bool valid;
  const int rank = chunk_counts(idx, A, E, s_cnt, e, valid);
  const int64_t i = (int64_t)blockIdx.x * PCH + threadIdx.x;
  if (i < A && !valid) row_of[i] = -1;
  if (!valid) return;
  const int wave = threadIdx.x >> 6;
  int r = offsets[e] + hist[(int64_t)e * nchunks + blockIdx.x] + rank;
  for (int w = 0; w < wave; ++w) r += s_cnt[w][e];
  row_of[i] = r;
  token_of[r] = (int32_t)(i / k);
}

// Token-major row copy: one wave per token reads its row once (16-byte
// vectors) and writes it to the token's K expert rows.
template <int K>
__global__ __launch_bounds__(256) void perm_copy_kernel(const u32x4* __restrict__ src, int64_t T, int64_t nvec,
                                                        const int32_t* __restrict__ row_of, u32x4* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int my = lane < K ? row_of[t * K + lane] : 0;
  int rows[K];
  bool ok = true;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = __shfl(my, j, MOE_WAVE);
    ok = ok && rows[j] >= 0;   // an out-of-range expert id left its row unset
  }
  const u32x4* s = src + t * nvec;
  if (ok) {
    for (int64_t v = lane; v < nvec; v += MOE_WAVE) {
      const u32x4 val = s[v];
#pragma unroll
      for (int j = 0; j < K; ++j) dst[(int64_t)rows[j] * nvec + v] = val;
    }
  } else {
    for (int64_t v = lane; v < nvec; v += MOE_WAVE) {
      const u32x4 val = s[v];
#pragma unroll
      for (int j = 0; j < K; ++j)
        if (rows[j] >= 0) dst[(int64_t)rows[j] * nvec + v] = val;
    }
  }
}

}  // namespace

size_t moe_permute_workspace(int64_t T, int k, int E) {
  const int64_t nchunks = ceil_div(T * k, PCH);
  return align256((size_t)nchunks * (size_t)E * sizeof(int32_t));
}

extern "C" moe_status moe_permute(const int32_t* topk_idx, int64_t T, int k, int E, const void* x, int x_dtype, int64_t d,
                                  int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of, void* x_perm,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!topk_idx || !x || !counts || !offsets || !row_of || !token_of || !x_perm) return MOE_EINVAL;
  if (T < 1 || d < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EINVAL;
  const int64_t es = x_dtype == MOE_BF16 ? 2 : 4;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || T * k >= (1ll << 31) || (d * es) % 16 != 0) return MOE_ENOTSUP;
  const size_t need = moe_permute_workspace(T, k, E);
  if (!workspace || workspace_bytes < need) return MOE_EWORKSPACE;
  hipStream_t s = moe_stream(stream);
  const int64_t A = T * k;
  const int nchunks = (int)ceil_div(A, PCH);
  int32_t* hist = static_cast<int32_t*>(workspace);
  perm_hist_kernel<<<nchunks, PCH, 0, s>>>(topk_idx, A, E, nchunks, hist);
  MOE_LAUNCH_CHECK();
  perm_scan_kernel<<<1, 1024, 0, s>>>(hist, E, nchunks, counts, offsets);
  MOE_LAUNCH_CHECK();
  perm_index_kernel<<<nchunks, PCH, 0, s>>>(topk_idx, A, k, E, nchunks, hist, offsets, row_of, token_of);
  MOE_LAUNCH_CHECK();
  const int64_t nvec = d * es / 16;
#define MOE_PCOPY(K)                                                                                       \
  perm_copy_kernel<K><<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(static_cast<const u32x4*>(x), T, nvec, row_of, \
                                                               static_cast<u32x4*>(x_perm))
  MOE_DISPATCH_K(k, MOE_PCOPY);
#undef MOE_PCOPY
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
