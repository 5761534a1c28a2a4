// Backward of the routed MoE layer.
//
// The pages give no backward; this is the chain rule through the forward of
// the lesson "专家组合 (MoE)" (AI Engineering from Scratch: Concept, Build it
// step 1).  The selection bias and the logit offset get no gradient (Key
// terms: the loss-free bias adds no gradient signal) and the top-k choice is
// held fixed.  Kernels, in stream order:
//   1. combine_bwd   one wave per token t: for each kept slot j, row
//                    r = row_of[t,j] gets dY_perm[r] = bf16(g*dy[t]) and gperm[r] = g
//   2. dgrad down    dH' = dy[t] W_down (dy rows read through token_of);
//                    epilogue: gate-gradient partials dg += <dH', H> over 32
//                    columns (dg = <dy, y_perm row> = <dy W_down, H>, so the
//                    fp32 expert output is never read back), then
//                    dH = g dH' and the SwiGLU backward -> dG|dU
//   3. gate_bwd      one wave per token: dg from the partials, dl on the
//                    chosen experts; router weight gradient dW_r[e] = sum over
//                    e's rows of dl * x rows (row-chunk partials, then an
//                    ordered reduction: deterministic)
//   4. wgrad down    dW_down[e] = dY_perm^T H over e's rows
//   5. wgrad up      dW_gate_up[e] = [dG|dU]^T X_perm over e's rows (with
//                    no X_perm given, its rows are read from x through
//                    token_of inside the GEMM's slab loads)
//   6. dgrad up      dX_perm = [dG|dU] W_gate_up (stored in bf16, like the
//                    other per-row activation gradients; summed in fp32 below)
//   7. shared expert (optional) the same products over all tokens
//   8. unpermute_bwd one wave per token: dx = sum_j dX_perm[row_of[t,j]]
//                    + sum_j dl*W_r[e] (+ the shared expert's input gradient)
// With an expert capacity (moe_permute_capacity), a dropped assignment has
// no expert output: it gets dg = 0 and no dY_perm / dX_perm row, but its
// logit still has a gradient through the gate normalisation, and the router
// weight gradient runs over the kept and the dropped rows of x_perm.
#include "aux.h"
#include "gemm.h"

#include <cstddef>

moe_status moe_tile_schedule_launch(const int32_t* offsets, int G, int bm, int32_t* mt_prefix, hipStream_t s);

namespace {

constexpr int RCH = 256;  // rows per router-wgrad partial

__device__ __forceinline__ float score_of(float l, int fn) {
  if (fn == MOE_SIGMOID_NORM) return 1.0f / (1.0f + expf(-l));
  if (fn == MOE_SQRT_SOFTPLUS_NORM) return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));
  return l;
}

// Combine backward, one wave per token t: its dy row is read once and each
// of its K kept expert rows r = row_of[t,j] gets dY_perm[r] = bf16(g[t,j] *
// dy[t]) (16-byte stores, the K rows' stores of a vector issued together;
// ordinary stores measured faster than non-temporal ones here, 0.110 against
// 0.138 ms at 16384 tokens, top-8) and gperm[r] = g[t,j].  A slot without a kept row (row_of < 0: dropped by
// an expert capacity, or an invalid expert id) writes nothing.
template <int K>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const u32x4* __restrict__ dy, const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ gate, int64_t T, int64_t nv8,
                                                          u32x4* __restrict__ dy_perm, float* __restrict__ gperm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myr = lane < K ? row_of[t * K + lane] : -1;
  const float myg = lane < K ? gate[t * K + lane] : 0.f;
  if (lane < K && myr >= 0) gperm[myr] = myg;
  u32x4* out[K];
  float g[K];
  bool live[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = __shfl(myr, j, MOE_WAVE);
    live[j] = r >= 0;
    out[j] = dy_perm + (int64_t)(live[j] ? r : 0) * nv8;
    g[j] = __shfl(myg, j, MOE_WAVE);
  }
  const u32x4* src = dy + t * nv8;
  for (int64_t v = lane; v < nv8; v += MOE_WAVE) {
    const u32x4 raw = __builtin_nontemporal_load(src + v);
    float a[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[2 * q] = bf16_to_f32(raw[q] & 0xFFFFu);
      a[2 * q + 1] = bf16_to_f32(raw[q] >> 16);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (!live[j]) continue;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(g[j] * a[2 * q], g[j] * a[2 * q + 1]);
      out[j][v] = o;
    }
  }
}

// Gate backward, one wave per token (lanes 0..k-1 hold the chosen experts):
// dg = the sum of the row's np32 partials from the dgrad-down epilogue, then
// dl on the chosen experts.  The k rows' partials are read by the whole
// wave at once: slot j's row goes to the L lanes j*L .. j*L+L-1 (L the
// largest power of two with k*L <= 64), lane j*L+i sums partials i, i+L,
// i+2L, ..., and the L lane sums are added by a butterfly (a fixed order).
// dg and dl are written for every slot.  An expert id outside [0, E) is
// invalid input (its token's results are unspecified); such a slot is never
// used as an index.
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ dg_part, int np32,
                                                       const int32_t* __restrict__ row_of,
                                                       const float* __restrict__ gate, const int32_t* __restrict__ idx,
                                                       const float* __restrict__ logits, int T, int k, int E, int fn,
                                                       float* __restrict__ dg_out, float* __restrict__ dl_out,
                                                       float* __restrict__ dl_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // an expert id outside [0, E) is never used as an index: its slot is left
  // out of the sums below
  const bool slot = lane < k;
  const int e_in = slot ? idx[t * k + lane] : -1;
  const bool act = slot && e_in >= 0 && e_in < E;
  const int myr = slot ? row_of[t * k + lane] : 0;
  const float myg = act ? gate[t * k + lane] : 0.f;
  const int mye = act ? e_in : 0;
  // a dropped slot (no row) adds nothing to the output: dg = 0
  int L = 64;
  while (L * k > 64) L >>= 1;
  const int js = lane / L, sub = lane - js * L;
  const int rj = __shfl(act ? myr : -1, js < k ? js : 0, MOE_WAVE);   // slot js's row, or -1
  float part = 0.f;
  if (js < k && rj >= 0) {
    const float* pr = dg_part + (int64_t)rj * np32;
    for (int b = sub; b < np32; b += L) part += pr[b];
  }
  for (int m = 1; m < L; m <<= 1) part += __shfl_xor(part, m, MOE_WAVE);
  float dg = __shfl(part, (lane < k ? lane : 0) * L, MOE_WAVE);
  if (!(act && myr >= 0)) dg = 0.f;
  const int prow = myr >= 0 ? myr : (myr == INT32_MIN ? -1 : ~myr);   // its x_perm row, kept or dropped
  const float D = wave_sum(act ? myg * dg : 0.f);
  float dl;
  if (fn == MOE_UNIFORM_GATES) {
    dl = 0.f;   // constant gates: no logit gradient
  } else if (fn == MOE_SOFTMAX_CHOSEN) {
    dl = myg * (dg - D);
  } else {
    const float l = act ? logits[t * E + mye] : 0.f;
    const float s = act ? score_of(l, fn) : 0.f;
    const float S = wave_sum(s);
    const float ds = (dg - D) / S;
    if (fn == MOE_SIGMOID_NORM) dl = ds * s * (1.0f - s);
    else dl = ds * (1.0f / (1.0f + expf(-l))) / (2.0f * s);
  }
  if (slot) {
    dg_out[t * k + lane] = act ? dg : 0.f;
    dl_out[t * k + lane] = act ? dl : 0.f;
    if (act && prow >= 0) dl_perm[prow] = dl;
  }
}

// Row segments of the router weight gradient: segment s < E holds the kept
// rows of expert s (offsets), segment E+s its dropped rows, which follow all
// kept rows (none without a capacity: counts may be NULL).  rc_prefix[s] =
// row chunks of RCH before segment s.  One workgroup of 1024 threads, E <= 1024.
__device__ __forceinline__ int excl_scan_1024(int v, int32_t* s_w, int& total) {
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

__global__ __launch_bounds__(1024) void router_seg_schedule_kernel(const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ counts, int E,
                                                                   int32_t* __restrict__ seg_beg,
                                                                   int32_t* __restrict__ seg_end,
                                                                   int32_t* __restrict__ rc_prefix) {
  __shared__ int32_t s_w[16];
  const int e = threadIdx.x;
  const int kept = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int drop = e < E && counts ? counts[e] - kept : 0;
  int tot_drop, tot_kp, tot_dp;
  const int dstart = excl_scan_1024(drop, s_w, tot_drop);
  const int kp = (kept + RCH - 1) / RCH, dp = (drop + RCH - 1) / RCH;
  const int kpx = excl_scan_1024(kp, s_w, tot_kp);
  const int dpx = excl_scan_1024(dp, s_w, tot_dp);
  if (e < E) {
    const int kept_all = offsets[E];
    seg_beg[e] = offsets[e];
    seg_end[e] = offsets[e + 1];
    seg_beg[E + e] = kept_all + dstart;
    seg_end[E + e] = kept_all + dstart + drop;
    rc_prefix[e] = kpx;
    rc_prefix[E + e] = tot_kp + dpx;
  }
  if (e == 0) rc_prefix[2 * E] = tot_kp + tot_dp;
}

// Partial router weight gradient over one chunk of at most RCH rows of one
// segment: part[p][c] = sum over the chunk's rows of dl_perm[r] * x_perm[r][c].
// Row r of x_perm is row token_of[r] of x, and x is read there: the k copies
// of a token row come from one row of x, which stays in the caches, instead
// of k rows streamed from HBM (147 -> 69 us on 16384 tokens, top-8).
// Eight columns (one 16-byte vector) per thread, 2048 columns per workgroup,
// four rows in flight per thread.
__global__ __launch_bounds__(256) void router_wgrad_part_kernel(const bf16_t* __restrict__ x,
                                                                const int32_t* __restrict__ token_of,
                                                                const float* __restrict__ dl_perm,
                                                                const int32_t* __restrict__ seg_beg,
                                                                const int32_t* __restrict__ seg_end,
                                                                const int32_t* __restrict__ rc_prefix, int S, int64_t d,
                                                                float* __restrict__ part) {
  const int p = blockIdx.x;
  if (p >= rc_prefix[S]) return;
  int lo = 0, hi = S;  // segment of chunk p: largest s with rc_prefix[s] <= p
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (rc_prefix[mid] <= p) lo = mid; else hi = mid;
  }
  const int sg = lo;
  const int64_t r0 = seg_beg[sg] + (int64_t)(p - rc_prefix[sg]) * RCH;
  const int64_t r1 = min((int64_t)seg_end[sg], r0 + RCH);
  const int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    u32x4 xv[4];
    float w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xv[u] = *reinterpret_cast<const u32x4*>(x + (int64_t)token_of[r + u] * d + c);
      w[u] = dl_perm[r + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w[u], bf16_to_f32(xv[u][q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w[u], bf16_to_f32(xv[u][q] >> 16), acc[2 * q + 1]);
      }
  }
  for (; r < r1; ++r) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (int64_t)token_of[r] * d + c);
    const float w = dl_perm[r];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(w, bf16_to_f32(xv[q] & 0xFFFFu), acc[2 * q]);
      acc[2 * q + 1] = fmaf(w, bf16_to_f32(xv[q] >> 16), acc[2 * q + 1]);
    }
  }
  f32x4* o = reinterpret_cast<f32x4*>(part + (int64_t)p * d + c);
  o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// dW_r[e] = the partials of e's kept segment, then of its dropped segment, in order
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ part,
                                                                  const int32_t* __restrict__ rc_prefix, int E,
                                                                  int64_t d, float* __restrict__ dw) {
  const int e = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;
  if (c >= d) return;
  float s = 0.f;
  for (int p = rc_prefix[e]; p < rc_prefix[e + 1]; ++p) s += part[(int64_t)p * d + c];
  for (int p = rc_prefix[E + e]; p < rc_prefix[E + e + 1]; ++p) s += part[(int64_t)p * d + c];
  dw[(int64_t)e * d + c] = s;
}

// The router weight gradient on the bf16 MFMA (E <= 64, d a multiple of
// 256): dW_r = dL^T x, with dL [T, E] the slots' dl placed at their experts
// (a slot counts when its expert id is valid and it has a row, kept or
// dropped, as in dl_perm).  Each fp32 dl is split exactly into three bf16
// parts (split3x2: 8 + 8 + 8 bits of its significand) and x is bf16, so
// every product is exact in fp32 and three MFMAs per 16-deep step add them
// in fp32.  x is read once (T * d * 2 bytes) instead of k gathered copies.
// Workgroup: all 64 expert rows x 256 columns over a chunk of RW_TCH
// tokens, 4 waves of 64 x 64, two workgroups per CU; per 32-token slab the
// three dL planes ([64 experts][32 tokens], K-contiguous) are built in LDS
// and x's slab ([32 tokens][256 columns], K-strided) is copied in,
// double-buffered, its loads two slabs ahead.
// part[chunk][e][c]; router_wgrad_chunks_reduce_kernel adds the chunks in
// order (deterministic).
constexpr int RW_TCH = 256, RW_EMAX = 64;
constexpr int RW_PLANE = RW_EMAX * 32 * 2;          // bytes of one dL plane
constexpr int RW_BUF = 3 * RW_PLANE + 32 * 256 * 2; // dL planes + x slab
__global__ __launch_bounds__(256) void router_wgrad_mfma_kernel(const bf16_t* __restrict__ x,
                                                                const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ row_of,
                                                                const float* __restrict__ dl, int T, int k, int E,
                                                                int64_t d, float* __restrict__ part) {
  using namespace moe_gemm;
  __shared__ __attribute__((aligned(16))) char smem[2 * RW_BUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 256;
  const int t0 = blockIdx.y * RW_TCH, t1 = min(T, t0 + RW_TCH);
  const int nslab = (t1 - t0 + 31) / 32;
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};
  // x slab: 32 rows x 256 columns = 1024 16-byte chunks, 4 per thread; chunk
  // q of thread tid is row (tid + 256 q) / 32, column chunk (tid + 256 q) % 32
  auto load_x = [&](int slab, u32x4 (&v)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + 256 * q, r = i >> 5, cc = i & 31;
      const int t = t0 + slab * 32 + r;
      v[q] = t < t1 ? *reinterpret_cast<const u32x4*>(x + (int64_t)t * d + c0 + cc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](char* buf, const u32x4 (&v)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + 256 * q, r = i >> 5, cc = i & 31;
      *reinterpret_cast<u32x4*>(buf + 3 * RW_PLANE + r * 512 + ((cc ^ swz_ks(r)) << 4)) = v[q];
    }
  };
  // A slab's 32 * k slots (32 tokens), at most two per thread (k <= 16):
  // expert id, row and dl, loaded two slabs ahead like x
  struct Slots {
    int e[2], row[2];
    float v[2];
  };
  auto load_slots = [&](int slab, Slots& sl) {
    const int tb = t0 + slab * 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 256 * u, t = tb + i / k;
      const bool in = i < 32 * k && t < t1;
      const int64_t q = in ? (int64_t)t * k + i % k : 0;
      sl.e[u] = in ? idx[q] : -1;
      sl.row[u] = row_of[q];
      sl.v[u] = dl[q];
    }
  };
  // dL planes of a slab (zeroed before): one bf16 part per slot and plane
  // at (expert, token) -- the k experts of a token are distinct
  auto build_dl = [&](char* buf, const Slots& sl) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 256 * u, e = sl.e[u];
      if (e < 0 || e >= E || sl.row[u] == INT32_MIN) continue;
      uint32_t h, m, l;
      split3x2(sl.v[u], 0.f, h, m, l);
      const int r = i / k, off = e * 64 + (((r >> 3) ^ swz_kc(e)) << 4) + (r & 7) * 2;
      *reinterpret_cast<uint16_t*>(buf + off) = (uint16_t)h;
      *reinterpret_cast<uint16_t*>(buf + RW_PLANE + off) = (uint16_t)m;
      *reinterpret_cast<uint16_t*>(buf + 2 * RW_PLANE + off) = (uint16_t)l;
    }
  };
  auto zero_dl = [&](char* buf) {
    for (int i = tid; i < 3 * RW_PLANE / 16; i += 256) reinterpret_cast<u32x4*>(buf)[i] = u32x4{0u, 0u, 0u, 0u};
  };
  u32x4 xv[2][4];
  Slots sv[2];
  load_x(0, xv[0]);
  load_slots(0, sv[0]);
  load_x(1, xv[1]);
  load_slots(1, sv[1]);
  for (int sl = 0; sl < nslab; ++sl) {
    char* buf = smem + (sl & 1) * RW_BUF;
    zero_dl(buf);
    if (sl & 1) store_x(buf, xv[1]);   // register sets by parity, so both stay in registers
    else store_x(buf, xv[0]);
    __syncthreads();
    if (sl & 1) build_dl(buf, sv[1]);
    else build_dl(buf, sv[0]);
    if (sl + 2 < nslab) {
      if (sl & 1) {
        load_x(sl + 2, xv[1]);
        load_slots(sl + 2, sv[1]);
      } else {
        load_x(sl + 2, xv[0]);
        load_slots(sl + 2, sv[0]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 16 * h;
      bf16x8 fa[3][2], fb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = mi * 32 + (lane & 31), cch = (kk >> 3) + (lane >> 5);
        const int off = row * 64 + ((cch ^ swz_kc(row)) << 4);
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) fa[pl][mi] = *reinterpret_cast<const bf16x8*>(buf + pl * RW_PLANE + off);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col0 = wave * 64 + ni * 32;
        s16x4 p2[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int g = lane >> 4, a = lane & 15;
          const int kr = kk + 8 * (g >> 1) + 4 * tt + (a >> 2);
          const int m = col0 + 16 * (g & 1) + 4 * (a & 3);
          const int off = 3 * RW_PLANE + kr * 512 + (((m >> 3) ^ swz_ks(kr)) << 4) + ((m & 7) << 1);
          p2[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + off));
        }
        fb[ni] = join8(p2[0], p2[1]);
      }
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[pl][mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
  }
  // MFMA layout: register r of a lane is row 8(r/4) + 4(lane/32) + r%4 of
  // its 32 x 32 block, column lane % 32
  float* pb = part + (int64_t)blockIdx.y * E * d;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (e < E) pb[(int64_t)e * d + c0 + wave * 64 + ni * 32 + (lane & 31)] = acc[mi][ni][r];
      }
}

// dW_r[e][c] = sum over the token chunks, in order, of part[chunk][e][c];
// eight chunks' loads in flight at a time, added in chunk order
__global__ __launch_bounds__(256) void router_wgrad_chunks_reduce_kernel(const float* __restrict__ part, int nchunk,
                                                                         int E, int64_t d, float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x, n = (int64_t)E * d;
  if (i >= n) return;
  float s = 0.f;
  int c = 0;
  for (; c + 8 <= nchunk; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(c + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; c < nchunk; ++c) s += part[(int64_t)c * n + i];
  dw[i] = s;
}

// dx[t] = extra[t] + sum_j dx_perm[row_of[t,j]] + sum_j dl[t,j] * w_router[idx[t,j]]
// (dx_perm: bf16 rows, summed in fp32; extra: the shared expert's input
// gradient in fp32, or null; a slot without a row, row_of < 0, is never
// read).  Eight columns (16 bytes of dx_perm) per lane and step.
template <int K, bool ROUTER>
__global__ __launch_bounds__(256) void unpermute_bwd_kernel(const u32x4* __restrict__ dx_perm,
                                                            const int32_t* __restrict__ row_of,
                                                            const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                            const f32x4* __restrict__ w_router,
                                                            const f32x4* __restrict__ extra, int T, int E,
                                                            int64_t nv8, f32x4* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myr = lane < K ? row_of[t * K + lane] : 0;
  const int e_in = lane < K ? idx[t * K + lane] : 0;
  const int mye = e_in >= 0 && e_in < E ? e_in : 0;   // an invalid id is never used as an index
  const float myl = lane < K ? dl[t * K + lane] : 0.f;
  const u32x4* xr[K];
  const f32x4* wr[K];
  float w[K];
  bool live[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = __shfl(myr, j, MOE_WAVE);
    live[j] = r >= 0;
    xr[j] = dx_perm + (int64_t)(live[j] ? r : 0) * nv8;
    wr[j] = ROUTER ? w_router + (int64_t)__shfl(mye, j, MOE_WAVE) * 2 * nv8 : nullptr;
    w[j] = __shfl(myl, j, MOE_WAVE);
  }
  for (int64_t v = lane; v < nv8; v += MOE_WAVE) {
    u32x4 xs[K];
#pragma unroll
    for (int j = 0; j < K; ++j) xs[j] = live[j] ? __builtin_nontemporal_load(xr[j] + v) : u32x4{0u, 0u, 0u, 0u};
    f32x4 a0 = extra ? __builtin_nontemporal_load(extra + t * 2 * nv8 + 2 * v) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 a1 = extra ? __builtin_nontemporal_load(extra + t * 2 * nv8 + 2 * v + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a0 += f32x4{bf16_to_f32(xs[j][0] & 0xFFFFu), bf16_to_f32(xs[j][0] >> 16), bf16_to_f32(xs[j][1] & 0xFFFFu),
                  bf16_to_f32(xs[j][1] >> 16)};
      a1 += f32x4{bf16_to_f32(xs[j][2] & 0xFFFFu), bf16_to_f32(xs[j][2] >> 16), bf16_to_f32(xs[j][3] & 0xFFFFu),
                  bf16_to_f32(xs[j][3] >> 16)};
    }
#pragma unroll
    for (int j = 0; j < K && ROUTER; ++j) {
      const f32x4 w0 = wr[j][2 * v], w1 = wr[j][2 * v + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a0[q] = fmaf(w[j], w0[q], a0[q]);
        a1[q] = fmaf(w[j], w1[q], a1[q]);
      }
    }
    dx[t * 2 * nv8 + 2 * v] = a0;
    dx[t * 2 * nv8 + 2 * v + 1] = a1;
  }
}

// The same sum with the router weights staged in LDS, for E <= UPL_EMAX: a
// workgroup owns a UPL_CW-column slice of dx for UPL_TB tokens and first
// copies that slice of all E router rows into LDS, so each router row is
// read from L2 once per workgroup instead of once per token that chose it
// (16384 tokens, top-8, d = 2048: 134 MB instead of 1 GB).  Each wave
// takes two tokens at a time, 32 lanes each, 8 columns (16 bytes of
// dx_perm) per lane; UPL_NT / 64 waves share the slice.  Sums as
// unpermute_bwd_kernel: the K rows in slot order in fp32, then the K
// router terms in slot order.
constexpr int UPL_CW = 256, UPL_TB = 128, UPL_EMAX = 64, UPL_NT = 512;
template <int K>
__global__ __launch_bounds__(UPL_NT) __attribute__((amdgpu_waves_per_eu(4))) void unpermute_bwd_lds_kernel(const u32x4* __restrict__ dx_perm,
                                                                const int32_t* __restrict__ row_of,
                                                                const int32_t* __restrict__ idx,
                                                                const float* __restrict__ dl,
                                                                const f32x4* __restrict__ w_router,
                                                                const f32x4* __restrict__ extra, int T, int E,
                                                                int64_t d, f32x4* __restrict__ dx) {
  __shared__ f32x4 s_w[UPL_EMAX * UPL_CW / 4];
  const int64_t c0 = (int64_t)blockIdx.x * UPL_CW;   // this workgroup's columns c0 .. c0 + UPL_CW - 1
  const int64_t nv4 = d / 4;
  for (int i = threadIdx.x; i < E * UPL_CW / 4; i += UPL_NT) {
    const int e = i / (UPL_CW / 4), v = i % (UPL_CW / 4);
    s_w[i] = w_router[(int64_t)e * nv4 + c0 / 4 + v];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;   // token of the pair, lane within it
  const int64_t nv8 = d / 8, col8 = c0 / 8 + hl;   // this lane's 8 columns, as a 16-byte vector index
  const int64_t tbeg = (int64_t)blockIdx.y * UPL_TB;
  for (int64_t tp = tbeg + 2 * wave; tp < tbeg + UPL_TB && tp < T; tp += 2 * (UPL_NT / 64)) {
    const int64_t t = tp + half;
    const bool tok = t < T;
    const int64_t tt = tok ? t : tp;
    const int myr = hl < K ? row_of[tt * K + hl] : 0;
    const int e_in = hl < K ? idx[tt * K + hl] : 0;
    const int mye = e_in >= 0 && e_in < E ? e_in : 0;   // an invalid id is never used as an index
    const float myl = hl < K ? dl[tt * K + hl] : 0.f;
    u32x4 xs[K];
    bool live[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int r = __shfl(myr, half * 32 + j, MOE_WAVE);
      live[j] = r >= 0;
      const u32x4 l = __builtin_nontemporal_load(dx_perm + (int64_t)(live[j] ? r : 0) * nv8 + col8);
      xs[j] = live[j] ? l : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 a0 = extra ? __builtin_nontemporal_load(extra + tt * 2 * nv8 + 2 * col8) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 a1 = extra ? __builtin_nontemporal_load(extra + tt * 2 * nv8 + 2 * col8 + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a0 += f32x4{bf16_to_f32(xs[j][0] & 0xFFFFu), bf16_to_f32(xs[j][0] >> 16), bf16_to_f32(xs[j][1] & 0xFFFFu),
                  bf16_to_f32(xs[j][1] >> 16)};
      a1 += f32x4{bf16_to_f32(xs[j][2] & 0xFFFFu), bf16_to_f32(xs[j][2] >> 16), bf16_to_f32(xs[j][3] & 0xFFFFu),
                  bf16_to_f32(xs[j][3] >> 16)};
    }
#pragma unroll 1
    for (int j = 0; j < K; ++j) {   // one router row at a time: its LDS reads are not hoisted into registers
      const float w = __shfl(myl, half * 32 + j, MOE_WAVE);
      const int e = __shfl(mye, half * 32 + j, MOE_WAVE);
      const f32x4 w0 = s_w[e * (UPL_CW / 4) + 2 * hl], w1 = s_w[e * (UPL_CW / 4) + 2 * hl + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a0[q] = fmaf(w, w0[q], a0[q]);
        a1[q] = fmaf(w, w1[q], a1[q]);
      }
    }
    if (tok) {
      dx[t * 2 * nv8 + 2 * col8] = a0;
      dx[t * 2 * nv8 + 2 * col8 + 1] = a1;
    }
  }
}

// offsets {0, T} of the shared expert's one row group
__global__ void shared_offsets_kernel(int32_t* __restrict__ o, int32_t T) {
  if (threadIdx.x < 2) o[threadIdx.x] = threadIdx.x ? T : 0;
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

inline bool router_mfma(int E, int64_t d) { return E <= RW_EMAX && d % 256 == 0; }

struct BwdLayout {
  size_t dy_perm, dgu, dx_perm, dg, dl, dl_perm, gperm, dg_part, mt_prefix, rc_prefix, seg_beg, seg_end, rpart, aux,
      kg_sched, kg_partial, total;
};

// Tile choices and chunk plans of the two weight-gradient GEMMs (M x N
// outputs over `rows` reduction rows in G groups).
inline bool wgrad_down_large(int64_t d, int64_t f) { return d >= moe_gemm::BM_LARGE && f >= moe_gemm::BN_LARGE; }
inline bool wgrad_up_large(int64_t d, int64_t f) { return 2 * f >= moe_gemm::BM_LARGE && d >= moe_gemm::BN_LARGE; }
inline size_t kg_sched_need(int64_t rows, int G, int64_t d, int64_t f) {
  using namespace moe_gemm;
  return std::max(kg_sched_bytes(kg_plan(d, f, rows, G, wgrad_down_large(d, f)), G),
                  kg_sched_bytes(kg_plan(2 * f, d, rows, G, wgrad_up_large(d, f)), G));
}
inline size_t kg_partial_need(int64_t rows, int G, int64_t d, int64_t f) {
  using namespace moe_gemm;
  return std::max(kg_partial_bytes(kg_plan(d, f, rows, G, wgrad_down_large(d, f))),
                  kg_partial_bytes(kg_plan(2 * f, d, rows, G, wgrad_up_large(d, f))));
}

BwdLayout layout(int64_t T, int k, int E, int64_t d, int64_t f) {
  const int64_t A = T * k;
  BwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.dy_perm = take((size_t)A * d * 2);
  L.dgu = take((size_t)A * 2 * f * 2);
  L.dx_perm = take((size_t)A * d * 2);
  L.dg = take((size_t)T * k * 4);
  L.dl = take((size_t)T * k * 4);
  L.dl_perm = take((size_t)A * 4);
  L.gperm = take((size_t)A * 4);
  L.dg_part = take((size_t)A * (size_t)(f / 32) * 4);
  L.mt_prefix = take((size_t)(E + 1) * 4);
  L.rc_prefix = take((size_t)(2 * E + 1) * 4);
  L.seg_beg = take((size_t)2 * E * 4);
  L.seg_end = take((size_t)2 * E * 4);
  L.rpart = take(std::max((size_t)(ceil_div(A, RCH) + 2 * E) * d * 4,
                           router_mfma(E, d) ? (size_t)ceil_div(T, RW_TCH) * E * d * 4 : 0));
  L.aux = take(moe_aux_bwd_workspace(T, E, d));
  L.kg_sched = take(kg_sched_need(A, E, d, f));
  L.kg_partial = take(kg_partial_need(A, E, d, f));
  L.total = o;
  return L;
}

// Workspace of the shared expert's backward: dG|dU [T, 2fs] bf16, its input
// gradient [T, d] f32, and its one-group offsets and tile prefix.
struct SharedLayout {
  size_t dgu, dx, offs, mt_prefix, kg_sched, kg_partial, total;
};

SharedLayout shared_layout(int64_t T, int64_t d, int64_t fs) {
  SharedLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.dgu = take((size_t)T * 2 * fs * 2);
  L.dx = take((size_t)T * d * 4);
  L.offs = take(2 * 4);
  L.mt_prefix = take(2 * 4);
  L.kg_sched = take(kg_sched_need(T, 1, d, fs));
  L.kg_partial = take(kg_partial_need(T, 1, d, fs));
  L.total = o;
  return L;
}

}  // namespace

size_t moe_backward_workspace(int64_t T, int k, int E, int64_t d, int64_t f) {
  if (d < 1 || f < 1) return 0;
  return layout(T, k, E, d, f).total;
}

size_t moe_backward_shared_workspace(int64_t T, int64_t d, int64_t fs) {
  if (d < 1 || fs < 1) return 0;
  return shared_layout(T, d, fs).total;
}

extern "C" moe_status moe_backward(const moe_bwd_args* a, void* stream) {
  // struct_size: the full struct, or one that ends before an appended field
  if (!a || (a->struct_size != sizeof(moe_bwd_args) && a->struct_size != offsetof(moe_bwd_args, counts) &&
             a->struct_size != offsetof(moe_bwd_args, aux_alpha) &&
             a->struct_size != offsetof(moe_bwd_args, f_shared) &&
             a->struct_size != offsetof(moe_bwd_args, stage_events)))
    return MOE_EINVAL;
  const int32_t* counts = a->struct_size > offsetof(moe_bwd_args, counts) ? a->counts : nullptr;
  const float aux_alpha = a->struct_size > offsetof(moe_bwd_args, aux_alpha) ? a->aux_alpha : 0.0f;
  const bool shared = a->struct_size > offsetof(moe_bwd_args, f_shared) && a->w_gate_up_shared;
  void* const* events = a->struct_size > offsetof(moe_bwd_args, stage_events) ? a->stage_events : nullptr;
  const int64_t T = a->T, d = a->d, f = a->f;
  const int E = a->E, k = a->k;
  if (T < 1 || d < 1 || f < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (a->score_fn < MOE_SOFTMAX_CHOSEN || a->score_fn > MOE_UNIFORM_GATES) return MOE_EINVAL;
  const bool router = a->score_fn != MOE_UNIFORM_GATES;
  if (!a->dy || !a->x || !a->topk_idx || !a->topk_gate || !a->row_of || !a->token_of || !a->offsets ||
      !a->gu_saved || !a->h || !a->w_gate_up || !a->w_down || !a->dx || !a->dw_gate_up || !a->dw_down)
    return MOE_EINVAL;
  if (router && (!a->w_router || !a->logits || !a->dw_router)) return MOE_EINVAL;
  const bool aux = aux_alpha != 0.0f;
  if (aux && (!router || !counts)) return MOE_EINVAL;   // the aux loss needs a router and the expert counts
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || d % 64 != 0 || f % 64 != 0 || T * k >= (1ll << 31) || T >= (1ll << 31))
    return MOE_ENOTSUP;
  // the weight-gradient GEMMs address one expert's rows of the permuted
  // activations, and the data-gradient GEMMs one expert's weight, through
  // 32-bit buffer resources
  if (T * k * std::max(d, 2 * f) * 2 >= (1ll << 31) || 2 * f * d * 2 >= (1ll << 31)) return MOE_ENOTSUP;
  const int64_t fs = shared ? a->f_shared : 0;
  if (shared) {
    if (!a->w_down_shared || !a->gu_shared || !a->h_shared || !a->dw_gate_up_shared || !a->dw_down_shared || fs < 1)
      return MOE_EINVAL;
    if (fs % 64 != 0 || T * std::max(d, 2 * fs) * 2 >= (1ll << 31) || 2 * fs * d * 2 >= (1ll << 31))
      return MOE_ENOTSUP;
  }
  const BwdLayout Lo = layout(T, k, E, d, f);
  if (!a->workspace || a->workspace_bytes < Lo.total) return MOE_EWORKSPACE;
  const SharedLayout Ls = shared_layout(T, d, fs);
  if (shared && (!a->workspace_shared || a->workspace_shared_bytes < Ls.total)) return MOE_EWORKSPACE;
  hipStream_t s = moe_stream(stream);
  // event of stage st (enum moe_bwd_stage), recorded after the stage's kernels
  auto mark = [&](int st) -> moe_status {
    if (events && events[st] && hipEventRecord(static_cast<hipEvent_t>(events[st]), s) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_EHIP;
    }
    return MOE_OK;
  };
#define MOE_MARK(st_)                      \
  do {                                     \
    const moe_status m_ = mark(st_);       \
    if (m_ != MOE_OK) return m_;           \
  } while (0)
  const int64_t A = T * k;
  char* ws = static_cast<char*>(a->workspace);
  bf16_t* dy_perm = reinterpret_cast<bf16_t*>(ws + Lo.dy_perm);
  bf16_t* dgu = reinterpret_cast<bf16_t*>(ws + Lo.dgu);
  bf16_t* dx_perm = reinterpret_cast<bf16_t*>(ws + Lo.dx_perm);
  float* dg = a->dgate ? a->dgate : reinterpret_cast<float*>(ws + Lo.dg);
  float* dl = a->dlogit ? a->dlogit : reinterpret_cast<float*>(ws + Lo.dl);
  float* dl_perm = reinterpret_cast<float*>(ws + Lo.dl_perm);
  float* gperm = reinterpret_cast<float*>(ws + Lo.gperm);
  float* dg_part = reinterpret_cast<float*>(ws + Lo.dg_part);
  int32_t* kg_sched = reinterpret_cast<int32_t*>(ws + Lo.kg_sched);
  float* kg_partial = reinterpret_cast<float*>(ws + Lo.kg_partial);
  int32_t* mt_prefix = reinterpret_cast<int32_t*>(ws + Lo.mt_prefix);
  int32_t* rc_prefix = reinterpret_cast<int32_t*>(ws + Lo.rc_prefix);
  int32_t* seg_beg = reinterpret_cast<int32_t*>(ws + Lo.seg_beg);
  int32_t* seg_end = reinterpret_cast<int32_t*>(ws + Lo.seg_end);
  float* rpart = reinterpret_cast<float*>(ws + Lo.rpart);
  const bf16_t* x_perm = static_cast<const bf16_t*>(a->x_perm);
  const bf16_t* wgu = static_cast<const bf16_t*>(a->w_gate_up);
  const bf16_t* wd = static_cast<const bf16_t*>(a->w_down);

  using namespace moe_gemm;
  const bool large = use_large_tile(f);
  const int np32 = (int)(f / 32);
  // 1. combine backward (permuted domain): dY_perm and each row's gate
#define MOE_CBWD(K)                                                                                          \
  combine_bwd_kernel<K><<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(static_cast<const u32x4*>(a->dy), a->row_of, \
                                                                  a->topk_gate, T, d / 8,                      \
                                                                  reinterpret_cast<u32x4*>(dy_perm), gperm)
  MOE_DISPATCH_K(k, MOE_CBWD);
#undef MOE_CBWD
  MOE_LAUNCH_CHECK();
  MOE_MARK(MOE_BWD_COMBINE);
  // 2. dH' = dy W_down over each expert's rows (dy rows gathered through
  //    token_of); epilogue: dg partials against H, dH = g dH', SwiGLU
  //    backward -> dG|dU
  moe_status st = moe_tile_schedule_launch(a->offsets, E, large ? BM_LARGE : BM, mt_prefix, s);
  if (st != MOE_OK) return st;
  {
    Args g{};
    g.A = static_cast<const bf16_t*>(a->dy); g.lda = d;
    g.a_rows = a->token_of; g.a_rows_total = T;
    g.B = wd; g.ldb = f; g.b_group = d * f;
    g.K = d; g.N = f;
    g.offsets = a->offsets; g.mt_prefix = mt_prefix; g.G = E;
    g.gu_in = static_cast<const bf16_t*>(a->gu_saved);
    g.gu_out = dgu;
    g.row_scale = gperm;
    g.h_in = static_cast<const bf16_t*>(a->h);
    g.dg_part = dg_part;
    st = launch_gemm<true, false, false, EPI_SWIGLU_BWD>(g, large, A, s);
    if (st != MOE_OK) return st;
  }
  MOE_MARK(MOE_BWD_DGRAD_DOWN);
  // 3. gate backward (dg, dl), then the router weight gradient (with the aux
  //    loss: dense, together with dx below)
  gate_bwd_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(dg_part, np32, a->row_of, a->topk_gate, a->topk_idx,
                                                           a->logits, (int)T, k, E, a->score_fn, dg, dl, dl_perm);
  MOE_LAUNCH_CHECK();
  if (aux) {
  } else if (router && router_mfma(E, d)) {
    const int nchunk = (int)ceil_div(T, RW_TCH);
    router_wgrad_mfma_kernel<<<dim3((unsigned)(d / 256), (unsigned)nchunk), 256, 0, s>>>(
        static_cast<const bf16_t*>(a->x), a->topk_idx, a->row_of, dl, (int)T, k, E, d, rpart);
    MOE_LAUNCH_CHECK();
    router_wgrad_chunks_reduce_kernel<<<(unsigned)ceil_div((int64_t)E * d, 256), 256, 0, s>>>(rpart, nchunk, E, d,
                                                                                           a->dw_router);
    MOE_LAUNCH_CHECK();
  } else if (router) {
    router_seg_schedule_kernel<<<1, 1024, 0, s>>>(a->offsets, counts, E, seg_beg, seg_end, rc_prefix);
    MOE_LAUNCH_CHECK();
    router_wgrad_part_kernel<<<dim3((unsigned)(ceil_div(A, RCH) + 2 * E), (unsigned)ceil_div(d, 2048)), 256, 0, s>>>(
        static_cast<const bf16_t*>(a->x), a->token_of, dl_perm, seg_beg, seg_end, rc_prefix, 2 * E, d, rpart);
    MOE_LAUNCH_CHECK();
    router_wgrad_reduce_kernel<<<dim3((unsigned)E, (unsigned)ceil_div(d, 256)), 256, 0, s>>>(rpart, rc_prefix, E, d,
                                                                                              a->dw_router);
    MOE_LAUNCH_CHECK();
  } else if (a->dw_router) {
    fill_zero_kernel<<<(unsigned)std::min<int64_t>(1024, ceil_div((int64_t)E * d, 256)), 256, 0, s>>>(a->dw_router,
                                                                                                      (int64_t)E * d);
    MOE_LAUNCH_CHECK();
  }
  MOE_MARK(MOE_BWD_ROUTER);
  {  // 4. dW_down[e] = dY_perm^T H
    Args g{};
    g.A = dy_perm; g.lda = d;
    g.B = static_cast<const bf16_t*>(a->h); g.ldb = f;
    g.M = d; g.N = f;
    g.offsets = a->offsets; g.G = E;
    g.out = a->dw_down; g.ldo = f; g.out_group = d * f;
    g.kg_sched = kg_sched; g.kg_partial = kg_partial;
    st = launch_gemm<false, false, true, EPI_F32>(g, wgrad_down_large(d, f), A, s);
    if (st != MOE_OK) return st;
  }
  MOE_MARK(MOE_BWD_WGRAD_DOWN);
  {  // 5. dW_gate_up[e] = [dG|dU]^T X_perm
    Args g{};
    g.A = dgu; g.lda = 2 * f;
    g.ldb = d;
    g.M = 2 * f; g.N = d;
    g.offsets = a->offsets; g.G = E;
    g.out = a->dw_gate_up; g.ldo = d; g.out_group = 2 * f * d;
    g.kg_sched = kg_sched; g.kg_partial = kg_partial;
    const bool large = wgrad_up_large(d, f);
    if (x_perm) {
      g.B = x_perm;
      st = launch_gemm<false, false, true, EPI_F32>(g, large, A, s);
    } else {
      g.B = static_cast<const bf16_t*>(a->x);
      g.b_gather = a->token_of;
      g.b_gather_rows = T;
      st = launch_gemm<false, false, true, EPI_F32, true>(g, large, A, s);
    }
    if (st != MOE_OK) return st;
  }
  MOE_MARK(MOE_BWD_WGRAD_UP);
  {  // 6. dX_perm = [dG|dU] W_gate_up
    Args g{};
    g.A = dgu; g.lda = 2 * f;
    g.B = wgu; g.ldb = d; g.b_group = 2 * f * d;
    g.K = 2 * f; g.N = d;
    g.offsets = a->offsets; g.mt_prefix = mt_prefix; g.G = E;
    g.out = dx_perm; g.ldo = d;
    st = launch_gemm<true, false, false, EPI_BF16>(g, large, A, s);
    if (st != MOE_OK) return st;
  }
  MOE_MARK(MOE_BWD_DGRAD_UP);
  // shared expert: the same four products over all T rows with dY_perm = dy
  // and X = x (gate 1), on one row group {0, T}
  char* wss = static_cast<char*>(a->workspace_shared);
  float* dx_sh = shared ? reinterpret_cast<float*>(wss + Ls.dx) : nullptr;
  if (shared) {
    bf16_t* dgu_sh = reinterpret_cast<bf16_t*>(wss + Ls.dgu);
    int32_t* offs_sh = reinterpret_cast<int32_t*>(wss + Ls.offs);
    int32_t* mt_sh = reinterpret_cast<int32_t*>(wss + Ls.mt_prefix);
    int32_t* kg_sched_sh = reinterpret_cast<int32_t*>(wss + Ls.kg_sched);
    float* kg_partial_sh = reinterpret_cast<float*>(wss + Ls.kg_partial);
    const bf16_t* dyb = static_cast<const bf16_t*>(a->dy);
    const bf16_t* xb = static_cast<const bf16_t*>(a->x);
    const bool large_sh = use_large_tile(fs);
    shared_offsets_kernel<<<1, 64, 0, s>>>(offs_sh, (int32_t)T);
    MOE_LAUNCH_CHECK();
    st = moe_tile_schedule_launch(offs_sh, 1, large_sh ? BM_LARGE : BM, mt_sh, s);
    if (st != MOE_OK) return st;
    {  // dH = dy W_down_sh -> dG|dU (SwiGLU backward from the saved G|U)
      Args g{};
      g.A = dyb; g.lda = d;
      g.B = static_cast<const bf16_t*>(a->w_down_shared); g.ldb = fs;
      g.K = d; g.N = fs;
      g.offsets = offs_sh; g.mt_prefix = mt_sh; g.G = 1;
      g.gu_in = static_cast<const bf16_t*>(a->gu_shared);
      g.gu_out = dgu_sh;
      st = launch_gemm<true, false, false, EPI_SWIGLU_BWD>(g, large_sh, T, s);
      if (st != MOE_OK) return st;
    }
    {  // dW_down_sh = dy^T H_sh
      Args g{};
      g.A = dyb; g.lda = d;
      g.B = static_cast<const bf16_t*>(a->h_shared); g.ldb = fs;
      g.M = d; g.N = fs;
      g.offsets = offs_sh; g.G = 1;
      g.out = a->dw_down_shared; g.ldo = fs; g.out_group = 0;
      g.kg_sched = kg_sched_sh; g.kg_partial = kg_partial_sh;
      st = launch_gemm<false, false, true, EPI_F32>(g, wgrad_down_large(d, fs), T, s);
      if (st != MOE_OK) return st;
    }
    {  // dW_gate_up_sh = [dG|dU]^T x
      Args g{};
      g.A = dgu_sh; g.lda = 2 * fs;
      g.B = xb; g.ldb = d;
      g.M = 2 * fs; g.N = d;
      g.offsets = offs_sh; g.G = 1;
      g.out = a->dw_gate_up_shared; g.ldo = d; g.out_group = 0;
      g.kg_sched = kg_sched_sh; g.kg_partial = kg_partial_sh;
      st = launch_gemm<false, false, true, EPI_F32>(g, wgrad_up_large(d, fs), T, s);
      if (st != MOE_OK) return st;
    }
    {  // dx_sh = [dG|dU] W_gate_up_sh (f32; added to dx by the unpermute below)
      Args g{};
      g.A = dgu_sh; g.lda = 2 * fs;
      g.B = static_cast<const bf16_t*>(a->w_gate_up_shared); g.ldb = d; g.b_group = 0;
      g.K = 2 * fs; g.N = d;
      g.offsets = offs_sh; g.mt_prefix = mt_sh; g.G = 1;
      g.out = dx_sh; g.ldo = d;
      st = launch_gemm<true, false, false, EPI_F32>(g, large_sh, T, s);
      if (st != MOE_OK) return st;
    }
  }
  MOE_MARK(MOE_BWD_SHARED);
  // 7. unpermute + router input gradient (+ the shared expert's)
  if (aux) {
    st = moe_aux_backward_launch(a->logits, counts, a->topk_idx, dl, static_cast<const bf16_t*>(a->x), a->w_router,
                                 reinterpret_cast<const u32x4*>(dx_perm), reinterpret_cast<const f32x4*>(dx_sh),
                                 a->row_of, T, E, k, d, a->score_fn, aux_alpha, a->dw_router, a->dx, ws + Lo.aux, s);
    if (st != MOE_OK) return st;
  } else {
#define MOE_UBWD(K)                                                                                             \
  do {                                                                                                          \
    if (router && E <= UPL_EMAX && d % UPL_CW == 0)                                                             \
      unpermute_bwd_lds_kernel<K><<<dim3((unsigned)(d / UPL_CW), (unsigned)ceil_div(T, UPL_TB)), UPL_NT, 0, s>>>( \
          reinterpret_cast<const u32x4*>(dx_perm), a->row_of, a->topk_idx, dl,                                  \
          reinterpret_cast<const f32x4*>(a->w_router), reinterpret_cast<const f32x4*>(dx_sh), (int)T, E, d,     \
          reinterpret_cast<f32x4*>(a->dx));                                                                     \
    else if (router)                                                                                            \
      unpermute_bwd_kernel<K, true><<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(                                   \
          reinterpret_cast<const u32x4*>(dx_perm), a->row_of, a->topk_idx, dl,                                  \
          reinterpret_cast<const f32x4*>(a->w_router), reinterpret_cast<const f32x4*>(dx_sh), (int)T, E, d / 8, \
          reinterpret_cast<f32x4*>(a->dx));                                                                     \
    else                                                                                                        \
      unpermute_bwd_kernel<K, false><<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(                                  \
          reinterpret_cast<const u32x4*>(dx_perm), a->row_of, a->topk_idx, dl, nullptr,                        \
          reinterpret_cast<const f32x4*>(dx_sh), (int)T, E, d / 8, reinterpret_cast<f32x4*>(a->dx));            \
  } while (0)
    MOE_DISPATCH_K(k, MOE_UBWD);
#undef MOE_UBWD
    MOE_LAUNCH_CHECK();
  }
  MOE_MARK(MOE_BWD_UNPERMUTE);
#undef MOE_MARK
  return MOE_OK;
}
