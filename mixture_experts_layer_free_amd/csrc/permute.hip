// Permute: group the T*k (token, expert) assignments by expert, stably and
// without atomics, and copy each token's row to its k expert rows (or, with
// x_perm NULL, only the indices: an expert GEMM that gathers rows through
// token_of needs no copy).
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
//
// Expert capacity (lesson "专家组合 (MoE)", Load balancing item 2: an expert
// takes at most a fixed number of tokens and the overflow skips the layer):
// with a capacity c >= 0, the first c assignments of an expert in token order
// are kept and the rest dropped.  Kept rows fill x_perm[0, A_kept) grouped by
// expert (offsets); dropped rows follow in x_perm[A_kept, A), grouped by
// expert in the same order, and are still copied (the router weight gradient
// runs over every assignment).  row_of holds r for a kept row and ~r (< 0)
// for a dropped one; an out-of-range expert id gets INT32_MIN and no row.
#include <atomic>

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
__device__ __forceinline__ void block_excl_scan(int v, int E, int32_t* s_wsum, int32_t* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  if (tid < E) out[tid] = base + inc - v;
  if (tid == E - 1) out[E] = base + inc;
  __syncthreads();
}

// cap < 0: no capacity.  counts = assignments per expert (the router's
// demand); offsets = exclusive scan of the kept counts min(counts, cap);
// doff (capacity only) = exclusive scan of the dropped counts.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ hist, int E, int nchunks, int cap,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ doff) {
  __shared__ int32_t s_tot[MOE_MAX_EXPERTS];
  __shared__ int32_t s_wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int SB = 8;   // 64-chunk groups whose loads are issued together
  for (int e = wave; e < E; e += 16) {
    int32_t* col = hist + (int64_t)e * nchunks;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64 * SB) {
      int v[SB];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int c = c0 + 64 * b + lane;
        v[b] = c < nchunks ? col[c] : 0;
      }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        if (c0 + 64 * b >= nchunks) break;   // empty groups past the column's end
        const int c = c0 + 64 * b + lane;
        const int inc = wave_incl_scan(v[b]);
        if (c < nchunks) col[c] = carry + inc - v[b];
        carry += __shfl(inc, 63, MOE_WAVE);
      }
    }
    if (lane == 0) s_tot[e] = carry;
  }
  __syncthreads();
  // exclusive scans over experts (E <= 1024: one value per thread)
  const int v = tid < E ? s_tot[tid] : 0;
  const int kept = cap >= 0 && v > cap ? cap : v;
  if (tid < E) counts[tid] = v;
  block_excl_scan(kept, E, s_wsum, offsets);
  if (cap >= 0) block_excl_scan(v - kept, E, s_wsum, doff);
}

// row_of[i] and token_of[row] for every assignment of chunk blockIdx.x.
__global__ __launch_bounds__(PCH) void perm_index_kernel(const int32_t* __restrict__ idx, int64_t A, int k, int E, int nchunks,
                                                         int cap, const int32_t* __restrict__ hist,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ doff,
                                                         int32_t* __restrict__ row_of, int32_t* __restrict__ token_of) {
  __shared__ int32_t s_cnt[4][MOE_MAX_EXPERTS];
  int e;
  bool valid;
  const int rank = chunk_counts(idx, A, E, s_cnt, e, valid);
  const int64_t i = (int64_t)blockIdx.x * PCH + threadIdx.x;
  if (i < A && !valid) row_of[i] = INT32_MIN;
  if (!valid) return;
  const int wave = threadIdx.x >> 6;
  int q = hist[(int64_t)e * nchunks + blockIdx.x] + rank;   // rank among expert e's assignments
  for (int w = 0; w < wave; ++w) q += s_cnt[w][e];
  if (cap < 0 || q < cap) {
    const int r = offsets[e] + q;
    row_of[i] = r;
    token_of[r] = (int32_t)(i / k);
  } else {
    const int r = offsets[E] + doff[e] + (q - cap);
    row_of[i] = ~r;
    token_of[r] = (int32_t)(i / k);
  }
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
    const int r = __shfl(my, j, MOE_WAVE);
    rows[j] = r >= 0 || r == INT32_MIN ? r : ~r;   // dropped rows are copied too
    ok = ok && rows[j] >= 0;                        // an out-of-range expert id has no row
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
  return align256((size_t)nchunks * (size_t)E * sizeof(int32_t)) + align256((size_t)(E + 1) * sizeof(int32_t));
}

extern "C" moe_status moe_permute(const int32_t* topk_idx, int64_t T, int k, int E, const void* x, int x_dtype, int64_t d,
                                  int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of, void* x_perm,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return moe_permute_capacity(topk_idx, T, k, E, -1, x, x_dtype, d, counts, offsets, row_of, token_of, x_perm,
                              workspace, workspace_bytes, stream);
}

// Scratch of moe_permute_noalloc: one copy per GPU, for the life of the
// process.  Host code never names it: it takes the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) int32_t scratch[MOE_PERMUTE_NOALLOC_SCRATCH / sizeof(int32_t)];

namespace {

// The permute's kernels after the argument checks; hist/doff: its scratch
// (the chunk histogram, then the dropped-row bases), nothing of which has to
// start at zero (every entry is written before it is read).
moe_status permute_launch(const int32_t* topk_idx, int64_t T, int k, int E, int cap, const void* x, int64_t es,
                          int64_t d, int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of,
                          void* x_perm, int32_t* hist, int32_t* doff, hipStream_t s) {
  const int64_t A = T * k;
  const int nchunks = (int)ceil_div(A, PCH);
  perm_hist_kernel<<<nchunks, PCH, 0, s>>>(topk_idx, A, E, nchunks, hist);
  MOE_LAUNCH_CHECK();
  perm_scan_kernel<<<1, 1024, 0, s>>>(hist, E, nchunks, cap, counts, offsets, doff);
  MOE_LAUNCH_CHECK();
  perm_index_kernel<<<nchunks, PCH, 0, s>>>(topk_idx, A, k, E, nchunks, cap, hist, offsets, doff, row_of, token_of);
  MOE_LAUNCH_CHECK();
  if (!x_perm) return MOE_OK;
  const int64_t nvec = d * es / 16;
#define MOE_PCOPY(K)                                                                                       \
  perm_copy_kernel<K><<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(static_cast<const u32x4*>(x), T, nvec, row_of, \
                                                               static_cast<u32x4*>(x_perm))
  MOE_DISPATCH_K(k, MOE_PCOPY);
#undef MOE_PCOPY
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Argument checks shared by every permute entry point; es = element bytes.
moe_status permute_check(const int32_t* topk_idx, int64_t T, int k, int E, const void* x, int x_dtype, int64_t d,
                         const int32_t* counts, const int32_t* offsets, const int32_t* row_of,
                         const int32_t* token_of, const void* x_perm, int64_t& es) {
  // x_perm NULL: indices only (a consumer that gathers rows through token_of
  // needs no copy), and then x may be NULL too
  if (!topk_idx || !counts || !offsets || !row_of || !token_of || (x_perm && !x)) return MOE_EINVAL;
  if (T < 1 || d < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EINVAL;
  es = x_dtype == MOE_BF16 ? 2 : 4;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || T * k >= (1ll << 31) || (d * es) % 16 != 0) return MOE_ENOTSUP;
  return MOE_OK;
}

constexpr int kMaxScratchDevices = 64;
std::atomic<uintptr_t> g_scratch[kMaxScratchDevices];   // 0: not yet looked up

// This device's copy of `scratch` (looked up once per device, with that
// device current), or nullptr if the lookup failed.
int32_t* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    p = reinterpret_cast<uintptr_t>(ptr);
    g_scratch[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  return reinterpret_cast<int32_t*>(p);
}

}  // namespace

extern "C" moe_status moe_permute_capacity(const int32_t* topk_idx, int64_t T, int k, int E, int64_t capacity,
                                           const void* x, int x_dtype, int64_t d, int32_t* counts, int32_t* offsets,
                                           int32_t* row_of, int32_t* token_of, void* x_perm, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  int64_t es = 0;
  const moe_status st = permute_check(topk_idx, T, k, E, x, x_dtype, d, counts, offsets, row_of, token_of, x_perm, es);
  if (st != MOE_OK) return st;
  const size_t need = moe_permute_workspace(T, k, E);
  if (!workspace || workspace_bytes < need) return MOE_EWORKSPACE;
  const int64_t A = T * k;
  // a capacity of A or more drops nothing: the same as none
  const int cap = capacity < 0 || capacity >= A ? -1 : (int)capacity;
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* doff = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                             align256((size_t)ceil_div(A, PCH) * (size_t)E * sizeof(int32_t)));
  return permute_launch(topk_idx, T, k, E, cap, x, es, d, counts, offsets, row_of, token_of, x_perm, hist, doff,
                        moe_stream(stream));
}

extern "C" moe_status moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int k, int E, const void* x, int x_dtype,
                                          int64_t d, int32_t* counts, int32_t* offsets, int32_t* row_of,
                                          int32_t* token_of, void* x_perm, void* stream) {
  int64_t es = 0;
  const moe_status st = permute_check(topk_idx, T, k, E, x, x_dtype, d, counts, offsets, row_of, token_of, x_perm, es);
  if (st != MOE_OK) return st;
  // the histogram must fit the static scratch (no capacity: doff is not used)
  const size_t hist_bytes = (size_t)ceil_div(T * k, PCH) * (size_t)E * sizeof(int32_t);
  if (hist_bytes > MOE_PERMUTE_NOALLOC_SCRATCH) return MOE_ENOTSUP;
  int32_t* hist = noalloc_scratch();
  if (!hist) return MOE_EHIP;
  return permute_launch(topk_idx, T, k, E, -1, x, es, d, counts, offsets, row_of, token_of, x_perm, hist, nullptr,
                        moe_stream(stream));
}
