// Router: fp32 logits on MFMA, then one wavefront per token for scoring,
// loss-free-biased top-k and gates.
//
// Method: lesson "专家组合 (MoE)" (AI Engineering from Scratch), Concept and
// Build it step 1; score functions and the fp32 rule from the AREX article on
// The Ultimate MoE Training Handbook, router-precision paragraph (a bf16
// router can round two close logits to one value and change the winner).
#include "moe_common.h"

#include <float.h>
#include <limits.h>

namespace {

// ---------------------------------------------------------------------------
// logits[t, e] = sum_i x[t, i] * w[e, i] (+ off[e]), fp32.
//
// Workgroup tile: 32 tokens x 64 experts, 4 waves.  Each wave owns the whole
// 32x64 tile but a quarter of every 64-wide K slab (k in [16w, 16w+16)), so
// the four partial tiles are summed at the end.  Inside a wave the products
// go through v_mfma_f32_16x16x4_f32 into a chunk accumulator that is folded
// into the running total every 64 products: every fp32 partial sum covers at
// most 64 products (blocked accumulation keeps the logit error near 1e-7
// relative at d = 7168).
constexpr int RT_M = 32, RT_N = 64, RT_K = 64, RT_LD = RT_K + 4;  // +4 floats: conflict-free b128 reads

template <bool XBF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv, const float* __restrict__ w,
                                                            const float* __restrict__ off, float* __restrict__ logits,
                                                            int T, int d, int E) {
  __shared__ __attribute__((aligned(16))) float sA[RT_M * RT_LD];
  __shared__ __attribute__((aligned(16))) float sB[RT_N * RT_LD];
  __shared__ __attribute__((aligned(16))) float sR[4][RT_M][RT_N + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_M, e0 = blockIdx.y * RT_N;

  // global -> register staging (prefetch of the next K slab)
  f32x4 ra[2];   // A: 32 rows x 64 k = 512 float4, 2 per thread
  f32x4 rb[4];   // B: 64 rows x 64 k = 1024 float4, 4 per thread

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 4, kc = (c & 15) * 4;
      const int t = t0 + row, k = k0 + kc;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (t < T && k < d) {
        if (XBF16) {
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(xv) + (int64_t)t * d + k);
          v[0] = bf16_to_f32(u.x & 0xFFFFu);
          v[1] = bf16_to_f32(u.x >> 16);
          v[2] = bf16_to_f32(u.y & 0xFFFFu);
          v[3] = bf16_to_f32(u.y >> 16);
        } else {
          v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(xv) + (int64_t)t * d + k);
        }
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 4, kc = (c & 15) * 4;
      const int e = e0 + row, k = k0 + kc;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (e < E && k < d) v = *reinterpret_cast<const f32x4*>(w + (int64_t)e * d + k);
      rb[i] = v;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<f32x4*>(&sA[(c >> 4) * RT_LD + (c & 15) * 4]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<f32x4*>(&sB[(c >> 4) * RT_LD + (c & 15) * 4]) = rb[i];
    }
  };

  f32x4 tot[2][4], chk[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) tot[m][n] = chk[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (d + RT_K - 1) / RT_K;
  gload(0);
  for (int it = 0; it < nk; ++it) {
    sstore();
    __syncthreads();
    if (it + 1 < nk) gload((it + 1) * RT_K);
    // this wave's 16 k: lane group g = lane/16 holds k = 16*wave + 4g + s, s = 0..3
    const int kb = 16 * wave + 4 * (lane >> 4);
    f32x4 a[2], b[4];
#pragma unroll
    for (int m = 0; m < 2; ++m) a[m] = *reinterpret_cast<const f32x4*>(&sA[(16 * m + (lane & 15)) * RT_LD + kb]);
#pragma unroll
    for (int n = 0; n < 4; ++n) b[n] = *reinterpret_cast<const f32x4*>(&sB[(16 * n + (lane & 15)) * RT_LD + kb]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          chk[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m][s], b[n][s], chk[m][n], 0, 0, 0);
    if ((it & 3) == 3 || it + 1 == nk) {   // 4 slabs x 16 k = 64 products per chunk
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          tot[m][n] += chk[m][n];
          chk[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();
  }

  // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16)+r, column lane%16
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) sR[wave][16 * m + 4 * (lane >> 4) + r][16 * n + (lane & 15)] = tot[m][n][r];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < (RT_M * RT_N) / 256; ++i) {
    const int c = tid + 256 * i, row = c / RT_N, col = c % RT_N;
    const int t = t0 + row, e = e0 + col;
    if (t < T && e < E) {
      float v = (sR[0][row][col] + sR[1][row][col]) + (sR[2][row][col] + sR[3][row][col]);
      if (off) v += off[e];
      logits[(int64_t)t * E + e] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// The same logits for bf16 x on the bf16 MFMA.  Each fp32 router weight is
// split exactly into three bf16 parts, w = hi + mid + lo (hi = w with its
// significand cut to 8 bits, mid the next 8 bits of the remainder, lo what is
// left; 8 + 8 + 8 bits hold the 24-bit fp32 significand).  x is bf16, so
// every product x*hi, x*mid, x*lo is exact in fp32 and the three
// v_mfma_f32_32x32x16_bf16 per 16-deep step add exact products in fp32 --
// an fp32 dot product, at the bf16 matrix rate.  As in the fp32 kernel, the
// products go into a chunk accumulator folded into the running total every
// 64 k (every partial sum covers at most 64 x 3 exact products).
// This kernel serves the grids too small for the LDS-shared kernel below
// (fewer than 256 tiles of 64 x 64, e.g. 8192 tokens x 64 experts) and
// d >= 2^22.
// Workgroup: 2 x RKS waves, 32 tokens x 64 experts; wave w owns experts
// e0 + 32(w%2) .. +31 and the (w/2)-th of RKS contiguous ranges of the
// reduction.  RKS = 4 when the grid would otherwise hold fewer than 1024
// waves (e.g. 8192 tokens x 64 experts), so a small grid still keeps the
// SIMDs busy; 1 otherwise (more waves measured slower there).  Operands come
// straight from global memory by buffer loads in the MFMA operand layout
// (16-byte x loads, 32-byte w loads, 32-bit offsets within the tile's rows, so
// d < 2^24); the next four 16-deep steps load while the current four
// multiply.  The RKS partial tiles are added in range order through LDS.
// (split3x2, in moe_common.h, splits each weight into its three bf16 parts.)

constexpr int RB_STEPS = 4;   // 16-deep steps in flight

template <int RKS>
__global__ __launch_bounds__(128 * RKS) void router_logits_bf16_kernel(const bf16_t* __restrict__ x,
                                                                       const float* __restrict__ w,
                                                                       const float* __restrict__ off,
                                                                       float* __restrict__ logits, int T, int d, int E) {
  __shared__ f32x4 s_part[RKS > 1 ? RKS - 1 : 1][2][4][64];   // partial tiles of ranges 1..RKS-1
  const int lane = threadIdx.x & 63, wave = (int)uni((uint32_t)(threadIdx.x >> 6));   // uniform: scalar offsets
  const int eh = wave & 1, ks = wave >> 1;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 64 + eh * 32;
  const int row = lane & 31, kh = 8 * (lane >> 5);        // MFMA operand layout: row l%32, k 8*(l/32)..+7
  // Buffer resources over the tile's 32 token rows of x and 32 expert rows of
  // W_r: a row past T (E) lies past the resource and reads zeros.  A lane's
  // x offset is pushed past the end for a k beyond d or a step beyond this
  // wave's range, so its products are zero whatever W_r holds there.
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(uni((const void*)(x + (int64_t)t0 * d)), uni((int64_t)(T - t0 < 32 ? T - t0 : 32) * d * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(uni((const void*)(w + (int64_t)(e0 < E ? e0 : 0) * d)),
                uni((int64_t)(E - e0 < 32 ? (E - e0 > 0 ? E - e0 : 0) : 32) * d * 4));
  const uint32_t xo = (uint32_t)(row * d + kh) * 2u, wo = (uint32_t)(row * d + kh) * 4u;
  const int klim = d - kh;   // this lane's k = 16*s + kh is inside d while 16*s < klim
  f32x16 tot = {}, chk = {};
  // this wave's steps: range ks of RKS, each a whole number of load batches
  const int nall = (d + 15) / 16;
  const int per = ((nall + RKS - 1) / RKS + RB_STEPS - 1) / RB_STEPS * RB_STEPS;
  const int sbeg = ks * per < nall ? ks * per : nall;
  const int nsteps = sbeg + per < nall ? sbeg + per : nall;   // end of the range
  // batch b = steps b*RB_STEPS .. +RB_STEPS-1; batch b+1 loads while batch b multiplies
  auto load = [&](int s0, u32x4 (&xa)[RB_STEPS], f32x4 (&wa)[RB_STEPS][2]) {
#pragma unroll
    for (int u = 0; u < RB_STEPS; ++u) {
      const int st = s0 + u;
      const bool kin = st < nsteps && 16 * st < klim;   // d % 8 == 0: the 8 values are all in or all out
      const uint32_t so = (uint32_t)st * 32u;           // bytes of x per 16-deep step (W_r: twice that)
      xa[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, kin ? xo : 0x80000000u, so, 0));
      wa[u][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 2 * so, 0));
      wa[u][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo + 16u, 2 * so, 0));
    }
  };
  auto compute = [&](const u32x4 (&xa)[RB_STEPS], const f32x4 (&wa)[RB_STEPS][2]) {
#pragma unroll
    for (int u = 0; u < RB_STEPS; ++u) {
      uint32_t h[4], m[4], l[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        split3x2(wa[u][0][2 * q], wa[u][0][2 * q + 1], h[q], m[q], l[q]);
        split3x2(wa[u][1][2 * q], wa[u][1][2 * q + 1], h[2 + q], m[2 + q], l[2 + q]);
      }
      const u32x4 hv = {h[0], h[1], h[2], h[3]}, mv = {m[0], m[1], m[2], m[3]}, lv = {l[0], l[1], l[2], l[3]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, xa[u]);
      // D[token][expert]: A = x (tokens x k), B = w parts (k x experts)
      chk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, lv), chk, 0, 0, 0);
      chk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, mv), chk, 0, 0, 0);
      chk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, hv), chk, 0, 0, 0);
    }
    tot += chk;   // RB_STEPS * 16 = 64 k per chunk
    chk = f32x16{};
  };
  u32x4 xa0[RB_STEPS], xa1[RB_STEPS];
  f32x4 wa0[RB_STEPS][2], wa1[RB_STEPS][2];
  load(sbeg, xa0, wa0);
  for (int s0 = sbeg; s0 < nsteps; s0 += 2 * RB_STEPS) {   // batches past the end load and add zeros
    load(s0 + RB_STEPS, xa1, wa1);
    compute(xa0, wa0);
    load(s0 + 2 * RB_STEPS, xa0, wa0);
    compute(xa1, wa1);
  }
  // add the ranges' partial tiles in range order (deterministic)
  if (RKS > 1 && ks > 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) s_part[ks - 1][eh][q][lane] = f32x4{tot[4 * q], tot[4 * q + 1], tot[4 * q + 2], tot[4 * q + 3]};
  if (RKS > 1) __syncthreads();
  if (ks > 0) return;
#pragma unroll
  for (int j = 0; j < RKS - 1; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = s_part[j][eh][q][lane];
      tot[4 * q] += v[0]; tot[4 * q + 1] += v[1]; tot[4 * q + 2] += v[2]; tot[4 * q + 3] += v[3];
    }
  // D layout: register r of a lane = row (token) 8*(r/4) + 4*(lane/32) + r%4, column (expert) lane%32
  const int ec = e0 + (lane & 31);
  if (ec < E) {
    const float o = off ? off[ec] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = t0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (tr < T) logits[(int64_t)tr * E + ec] = tot[r] + o;
    }
  }
}

// ---------------------------------------------------------------------------
// LDS writes done, then the workgroup barrier; the compiler moves no memory
// access across either.
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same logits and the same sums (bit for bit) on larger grids, with the
// operands shared through LDS.  The kernel above is bound by its texture
// addresser: each wave fetches its own fragments in the MFMA operand layout
// (32 rows per load), and the two waves of a workgroup fetch the same x rows.
// Here a 4-wave workgroup owns 64 tokens x 64 experts (wave w: tokens
// 32(w/2).., experts 32(w%2)..) and stages each 64-deep batch of x and W_r
// once, with every load covering whole 128-byte lines; W_r is split into its
// three bf16 parts once, on the way into LDS (three [64][64] bf16 planes).
// Each 16-deep step then reads one x and three W_r fragments from LDS and
// issues the same three MFMAs, in the same order, on the same lane-to-k
// mapping as the kernel above; the chunk accumulator folds every 64 k.
// Batches run two ahead in registers; the LDS holds two stages (64 KB).
// Offsets are 32-bit within the tile's rows: d < 2^22.
constexpr int RL_T = 64, RL_E = 64, RL_K = 64;                  // tile and batch depth
constexpr int RL_XB = RL_T * RL_K * 2, RL_PB = RL_E * RL_K * 2;  // bytes: x stage, one W_r plane
constexpr int RL_STAGE = RL_XB + 3 * RL_PB;                      // 32 KB

__device__ __forceinline__ int rl_swz(int row) { return (row >> 1) & 7; }   // 16-byte chunk swizzle, [64][64] bf16

__global__ __launch_bounds__(256) void router_logits_lds_kernel(const bf16_t* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ off,
                                                                float* __restrict__ logits, int T, int d, int E) {
  __shared__ __attribute__((aligned(16))) char smem[2 * RL_STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = (int)uni((uint32_t)(tid >> 6));
  const int tm = wave >> 1, te = wave & 1;
  const int ntb = (T + RL_T - 1) / RL_T;
  const int t0 = (int)(blockIdx.x % ntb) * RL_T, e0 = (int)(blockIdx.x / ntb) * RL_E;
  const int nb = (d + RL_K - 1) / RL_K;   // 64-deep batches

  // Loads: x rows of 128 bytes (8 chunks) -> thread chunks c = tid, tid+256
  // (row c/8, chunk c%8); W_r rows of 256 bytes (16 chunks of 4 floats) ->
  // c = tid + 256j, j < 4 (row c/16, chunk c%16).  Rows past T (E) lie past
  // the buffer resource and read zeros; an x chunk past d is pushed past it
  // too, so its products are zero whatever W_r holds there.
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(uni((const void*)(x + (int64_t)t0 * d)), uni((int64_t)(T - t0 < RL_T ? T - t0 : RL_T) * d * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(uni((const void*)(w + (int64_t)e0 * d)), uni((int64_t)(E - e0 < RL_E ? E - e0 : RL_E) * d * 4));
  uint32_t xo[2], wo[4];
  int xk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + 256 * j, r = c >> 3, ch = c & 7;
    xo[j] = (uint32_t)(r * d + 8 * ch) * 2u;
    xk[j] = 8 * ch;   // k of the chunk inside its batch
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j, r = c >> 4, ch = c & 15;
    wo[j] = (uint32_t)(r * d + 4 * ch) * 4u;
  }
  auto gload = [&](int b, u32x4 (&xr)[2], f32x4 (&wr)[4]) {
    const int kb = (int)uni((uint32_t)(b * RL_K));   // uniform: a scalar offset, no loop over the lanes
#pragma unroll
    for (int j = 0; j < 2; ++j)
      xr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rx, kb + xk[j] < d ? xo[j] : 0x80000000u, (uint32_t)kb * 2u, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wr[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo[j], (uint32_t)kb * 4u, 0));
  };
  // LDS stage: x [64][64] bf16, then the hi, mid, lo planes of W_r [64][64] bf16
  auto swrite = [&](char* st, const u32x4 (&xr)[2], const f32x4 (&wr)[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + 256 * j, r = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(st + r * 128 + ((ch ^ rl_swz(r)) << 4)) = xr[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j, r = c >> 4, ch = c & 15;   // 4 floats: half of a 16-byte plane chunk
      const int o = r * 128 + (((ch >> 1) ^ rl_swz(r)) << 4) + 8 * (ch & 1);
      uint32_t h0, m0, l0, h1, m1, l1;
      split3x2(wr[j][0], wr[j][1], h0, m0, l0);
      split3x2(wr[j][2], wr[j][3], h1, m1, l1);
      *reinterpret_cast<u32x2*>(st + RL_XB + o) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(st + RL_XB + RL_PB + o) = u32x2{m0, m1};
      *reinterpret_cast<u32x2*>(st + RL_XB + 2 * RL_PB + o) = u32x2{l0, l1};
    }
  };
  // fragments: row l%32 of the wave's 32, k 8*(l/32).. of the 16-deep step
  const int fr = lane & 31, fsw = rl_swz(fr);
  const int xa_row = (32 * tm + fr) * 128, wb_row = (32 * te + fr) * 128;
  f32x16 tot = {}, chk = {};
  auto compute = [&](const char* st) {
#pragma unroll
    for (int u = 0; u < RL_K / 16; ++u) {
      const int ch = ((2 * u + (lane >> 5)) ^ fsw) << 4;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + xa_row + ch);
      const bf16x8 hv = *reinterpret_cast<const bf16x8*>(st + RL_XB + wb_row + ch);
      const bf16x8 mv = *reinterpret_cast<const bf16x8*>(st + RL_XB + RL_PB + wb_row + ch);
      const bf16x8 lv = *reinterpret_cast<const bf16x8*>(st + RL_XB + 2 * RL_PB + wb_row + ch);
      chk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lv, chk, 0, 0, 0);
      chk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, mv, chk, 0, 0, 0);
      chk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hv, chk, 0, 0, 0);
    }
    tot += chk;
    chk = f32x16{};
  };
  // batch j lives in register set j % 2 until it is written to LDS stage j % 2
  u32x4 xr0[2], xr1[2];
  f32x4 wr0[4], wr1[4];
  gload(0, xr0, wr0);
  gload(1, xr1, wr1);   // a batch past the end reads zeros
  swrite(smem, xr0, wr0);
  wait_lgkm0();
  lds_barrier();
  for (int b = 0; b < nb; b += 2) {
    gload(b + 2, xr0, wr0);
    compute(smem);
    swrite(smem + RL_STAGE, xr1, wr1);
    wait_lgkm0();
    lds_barrier();
    if (b + 1 >= nb) break;
    gload(b + 3, xr1, wr1);
    compute(smem + RL_STAGE);
    swrite(smem, xr0, wr0);
    wait_lgkm0();
    lds_barrier();
  }
  // D layout: register r of a lane = row (token) 8*(r/4) + 4*(lane/32) + r%4, column (expert) lane%32
  const int ec = e0 + 32 * te + (lane & 31);
  if (ec < E) {
    const float o = off ? off[ec] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = t0 + 32 * tm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (tr < T) logits[(int64_t)tr * E + ec] = tot[r] + o;
    }
  }
}

// ---------------------------------------------------------------------------
// The same logits for E <= 16 (the few-expert layers, where the router reads
// x once and the 64-expert tile would idle most of its MFMA columns).
//
// Workgroup: 16 tokens x 16 experts, 4 waves splitting d into contiguous
// ranges of 32-wide k steps.  Each lane loads its operands straight from
// global memory into registers, 8 steps ahead: lane l holds row l%16 (token
// for A, expert for B) and k = 32*step + 8*(l/16) + s, s = 0..7, which is the
// k the lane feeds to MFMA s (any fixed k permutation is the same sum).  The
// chunk accumulator is folded every 2 steps (64 products); the 4 wave
// partials are added in a fixed order.
constexpr int RS_U = 8;   // k steps in flight per wave

template <bool XBF16>
__global__ __launch_bounds__(256) void router_logits_small_kernel(const void* __restrict__ xv,
                                                                  const float* __restrict__ w,
                                                                  const float* __restrict__ off,
                                                                  float* __restrict__ logits, int T, int d, int E) {
  __shared__ float sR[4][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * 16, t = t0 + r;
  const int nsteps = (d + 31) / 32;
  const int s0 = wave * nsteps / 4, s1 = (wave + 1) * nsteps / 4;
  const bool trow = t < T, erow = r < E;

  f32x4 tot = {0.f, 0.f, 0.f, 0.f}, chk = {0.f, 0.f, 0.f, 0.f};
  for (int st = s0; st < s1; st += RS_U) {
    float a[RS_U][8], b[RS_U][8];
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const int k = 32 * (st + u) + 8 * kq;
      const bool kin = st + u < s1 && k < d;   // d % 8 == 0: the 8 values are all in or all out
      if (XBF16) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kin && trow) v = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(xv) + (int64_t)t * d + k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[u][2 * q] = bf16_to_f32(v[q] & 0xFFFFu);
          a[u][2 * q + 1] = bf16_to_f32(v[q] >> 16);
        }
      } else {
        f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (kin && trow) {
          const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(xv) + (int64_t)t * d + k);
          v0 = p[0];
          v1 = p[1];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[u][q] = v0[q];
          a[u][4 + q] = v1[q];
        }
      }
      f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0;
      if (kin && erow) {
        const f32x4* p = reinterpret_cast<const f32x4*>(w + (int64_t)r * d + k);
        w0 = p[0];
        w1 = p[1];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b[u][q] = w0[q];
        b[u][4 + q] = w1[q];
      }
    }
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
#pragma unroll
      for (int q = 0; q < 8; ++q) chk = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][q], b[u][q], chk, 0, 0, 0);
      if (u & 1) {   // 2 steps x 32 k = 64 products per chunk
        tot += chk;
        chk = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i) sR[wave][4 * kq + i][r] = tot[i];
  __syncthreads();
  const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
  if (t0 + row < T && col < E) {
    float v = (sR[0][row][col] + sR[1][row][col]) + (sR[2][row][col] + sR[3][row][col]);
    if (off) v += off[col];
    logits[(int64_t)(t0 + row) * E + col] = v;
  }
}

// ---------------------------------------------------------------------------
// One wavefront per token.  Lane l holds experts l, l+64, ...; k rounds of a
// cross-lane argmax on (key desc, expert asc) pick the experts; lanes 0..k-1
// then hold one chosen expert each and form the gates with wave reductions.

__device__ __forceinline__ float score_of(float l, int fn) {
  if (fn == MOE_SIGMOID_NORM) return 1.0f / (1.0f + expf(-l));
  if (fn == MOE_SQRT_SOFTPLUS_NORM) return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));
  return l;
}

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

constexpr int TOPK_MAXV = MOE_MAX_EXPERTS / MOE_WAVE;  // experts per lane

// Gate of the chosen expert held by an active lane (raw logit l): softmax over
// the active lanes' logits, or the lane's score over the active lanes' sum.
__device__ __forceinline__ float chosen_gate(float l, bool act, int fn) {
  if (fn == MOE_SOFTMAX_CHOSEN) {
    float m = act ? l : -INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, MOE_WAVE));
    const float ex = act ? expf(l - m) : 0.0f;
    return ex / wave_sum(ex);
  }
  const float s = act ? score_of(l, fn) : 0.0f;
  return s / wave_sum(s);
}

__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                                                        int T, int E, int k, int fn, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lrow = logits + (int64_t)t * E;
  if (E <= MOE_WAVE) {
    // One key per lane: each lane counts the keys that beat its own (a
    // larger key, or an equal key at a lower expert index), which is its
    // place in the selection order; one permute then hands the k best to
    // lanes 0..k-1.  The order is read on a 64-bit integer: an
    // order-preserving image of the key (-0 taken as +0) above the
    // complemented lane, so ties go to the lower index and no two lanes tie.
    const bool valid = lane < E;
    const float kf = valid ? score_of(lrow[lane], fn) + (bias ? bias[lane] : 0.0f) + 0.0f : 0.0f;
    const uint32_t u = __float_as_uint(kf);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const uint64_t mykey = valid ? ((uint64_t)ord << 32) | (uint32_t)(MOE_WAVE - 1 - lane) : 0ull;
    const uint32_t khi = (uint32_t)(mykey >> 32), klo = (uint32_t)mykey;
    int rank = 0;
#pragma unroll
    for (int m = 0; m < MOE_WAVE; ++m) {
      const uint64_t km = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)khi, m) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)klo, m);
      rank += km > mykey ? 1 : 0;
    }
    // lanes past E keep their own id (their ranks are >= E, never sent)
    const int mine = __builtin_amdgcn_ds_permute((valid ? rank : lane) * 4, lane);
    const bool act = lane < k;
    const float g = chosen_gate(act ? lrow[mine] : 0.0f, act, fn);
    if (act) {
      idx[(int64_t)t * k + lane] = mine;
      gate[(int64_t)t * k + lane] = g;
    }
    return;
  }
  const int nv = (E + MOE_WAVE - 1) / MOE_WAVE;

  float key[TOPK_MAXV];
#pragma unroll
  for (int i = 0; i < TOPK_MAXV; ++i) {
    const int e = lane + MOE_WAVE * i;
    key[i] = -FLT_MAX;
    if (i < nv && e < E) key[i] = score_of(lrow[e], fn) + (bias ? bias[e] : 0.0f);
  }
  uint32_t taken = 0;
  int mine = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < TOPK_MAXV; ++i) {
      const int e = lane + MOE_WAVE * i;
      if (i < nv && e < E && !((taken >> i) & 1u) && better(key[i], e, bv, be)) {
        bv = key[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, MOE_WAVE);
      const int oe = __shfl_xor(be, o, MOE_WAVE);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) mine = be;
  }
  // gates over the chosen experts, from the unbiased values
  const bool act = lane < k;
  const float g = chosen_gate(act ? lrow[mine] : 0.0f, act, fn);
  if (act) {
    idx[(int64_t)t * k + lane] = mine;
    gate[(int64_t)t * k + lane] = g;
  }
}

// ---------------------------------------------------------------------------
// Routing replay (lesson "专家组合 (MoE)", Exercises item 3: record the
// experts fired at inference and force the same choice when computing
// gradients): gates of a given choice, one wave per token.  An id outside
// [0, E) gets gate 0 and takes no part in the normalisation.
__global__ __launch_bounds__(256) void replay_gate_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ idx, int T, int E, int k, int fn,
                                                          float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int e = lane < k ? idx[(int64_t)t * k + lane] : -1;
  const bool act = lane < k && e >= 0 && e < E;
  const float g = chosen_gate(act ? logits[(int64_t)t * E + e] : 0.0f, act, fn);
  if (lane < k) gate[(int64_t)t * k + lane] = act ? g : 0.0f;
}

// ---------------------------------------------------------------------------
// Hash router (lesson, Exercises item 2: a deterministic router with nothing
// learned).  Expert e's key for token id is the SplitMix64 output for the
// state id*2^32 + e advanced (salt+1) times (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", 2014):
//   z = id*2^32 + e + (salt+1)*0x9E3779B97F4A7C15
//   z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;  z = (z ^ z>>27) * 0x94D049BB133111EB;  z ^= z>>31
// and the token goes to the k experts with the smallest keys (ascending;
// the mix is a bijection, so keys of one token never tie), each with gate 1/k.
__device__ __forceinline__ uint64_t splitmix_key(uint32_t id, uint32_t e, uint32_t salt) {
  uint64_t z = ((uint64_t)id << 32 | e) + (uint64_t)(salt + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void hash_route_kernel(const int32_t* __restrict__ token_ids, int T, int E, int k,
                                                         uint32_t salt, int32_t* __restrict__ idx,
                                                         float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint32_t id = (uint32_t)token_ids[t];
  const int nv = (E + MOE_WAVE - 1) / MOE_WAVE;
  uint64_t key[TOPK_MAXV];
#pragma unroll
  for (int i = 0; i < TOPK_MAXV; ++i) {
    const int e = lane + MOE_WAVE * i;
    key[i] = i < nv && e < E ? splitmix_key(id, (uint32_t)e, salt) : ~0ull;
  }
  uint32_t taken = 0;
  int mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t bv = ~0ull;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < TOPK_MAXV; ++i) {
      const int e = lane + MOE_WAVE * i;
      if (i < nv && e < E && !((taken >> i) & 1u) && (key[i] < bv || (key[i] == bv && e < be))) {
        bv = key[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t ov = ((uint64_t)(uint32_t)__shfl_xor((int)(bv >> 32), o, MOE_WAVE) << 32) |
                          (uint32_t)__shfl_xor((int)(uint32_t)bv, o, MOE_WAVE);
      const int oe = __shfl_xor(be, o, MOE_WAVE);
      if (ov < bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) mine = be;
  }
  if (lane < k) {
    idx[(int64_t)t * k + lane] = mine;
    gate[(int64_t)t * k + lane] = 1.0f / (float)k;
  }
}

}  // namespace

static moe_status router_logits_launch(const void* x, int x_dtype, int64_t T, int64_t d, const float* w_router,
                                       const float* logit_offset, int E, float* logits_out, hipStream_t s);

extern "C" moe_status moe_route(const void* x, int x_dtype, int64_t T, int64_t d, const float* w_router,
                                const float* logit_offset, const float* sel_bias, int E, int k, int score_fn,
                                int32_t* topk_idx, float* topk_gate, float* logits_out, void* stream) {
  if (!x || !w_router || !topk_idx || !topk_gate || !logits_out) return MOE_EINVAL;
  if (T < 1 || d < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EINVAL;
  if (score_fn < MOE_SOFTMAX_CHOSEN || score_fn > MOE_SQRT_SOFTPLUS_NORM) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || d % 8 != 0 || T >= (1ll << 31) || d >= (1ll << 24))
    return MOE_ENOTSUP;
  hipStream_t s = moe_stream(stream);
  const moe_status st = router_logits_launch(x, x_dtype, T, d, w_router, logit_offset, E, logits_out, s);
  if (st != MOE_OK) return st;
  topk_gate_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(logits_out, sel_bias, (int)T, E, k, score_fn, topk_idx,
                                                            topk_gate);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

static moe_status router_logits_launch(const void* x, int x_dtype, int64_t T, int64_t d, const float* w_router,
                                       const float* logit_offset, int E, float* logits_out, hipStream_t s) {
  if (E <= 16) {
    const unsigned gs = (unsigned)ceil_div(T, 16);
    if (x_dtype == MOE_BF16)
      router_logits_small_kernel<true><<<gs, 256, 0, s>>>(x, w_router, logit_offset, logits_out, (int)T, (int)d, E);
    else
      router_logits_small_kernel<false><<<gs, 256, 0, s>>>(x, w_router, logit_offset, logits_out, (int)T, (int)d, E);
  } else if (x_dtype == MOE_BF16 && d < (1 << 22) && ceil_div(T, RL_T) * ceil_div(E, RL_E) >= 256) {
    // enough 64 x 64 tiles to fill the CUs: operands shared through LDS
    const unsigned g = (unsigned)(ceil_div(T, RL_T) * ceil_div(E, RL_E));
    router_logits_lds_kernel<<<g, 256, 0, s>>>(static_cast<const bf16_t*>(x), w_router, logit_offset, logits_out,
                                               (int)T, (int)d, E);
  } else if (x_dtype == MOE_BF16) {
    const dim3 g((unsigned)ceil_div(T, 32), (unsigned)ceil_div(E, 64));
    if ((int64_t)g.x * g.y * 2 < 1024)
      router_logits_bf16_kernel<4><<<g, 128 * 4, 0, s>>>(static_cast<const bf16_t*>(x), w_router, logit_offset,
                                                          logits_out, (int)T, (int)d, E);
    else
      router_logits_bf16_kernel<1><<<g, 128, 0, s>>>(static_cast<const bf16_t*>(x), w_router, logit_offset,
                                                      logits_out, (int)T, (int)d, E);
  } else {
    dim3 g1((unsigned)ceil_div(T, RT_M), (unsigned)ceil_div(E, RT_N));
    router_logits_kernel<false><<<g1, 256, 0, s>>>(x, w_router, logit_offset, logits_out, (int)T, (int)d, E);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_route_replay(const void* x, int x_dtype, int64_t T, int64_t d, const float* w_router,
                                       const float* logit_offset, int E, int k, int score_fn,
                                       const int32_t* topk_idx, float* topk_gate, float* logits_out, void* stream) {
  if (!x || !w_router || !topk_idx || !topk_gate || !logits_out) return MOE_EINVAL;
  if (T < 1 || d < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EINVAL;
  if (score_fn < MOE_SOFTMAX_CHOSEN || score_fn > MOE_SQRT_SOFTPLUS_NORM) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || d % 8 != 0 || T >= (1ll << 31) || d >= (1ll << 24))
    return MOE_ENOTSUP;
  hipStream_t s = moe_stream(stream);
  const moe_status st = router_logits_launch(x, x_dtype, T, d, w_router, logit_offset, E, logits_out, s);
  if (st != MOE_OK) return st;
  replay_gate_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, s>>>(logits_out, topk_idx, (int)T, E, k, score_fn, topk_gate);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_route_hash(const int32_t* token_ids, int64_t T, int E, int k, uint32_t salt,
                                     int32_t* topk_idx, float* topk_gate, void* stream) {
  if (!token_ids || !topk_idx || !topk_gate) return MOE_EINVAL;
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || T >= (1ll << 31)) return MOE_ENOTSUP;
  hash_route_kernel<<<(unsigned)ceil_div(T, 4), 256, 0, moe_stream(stream)>>>(token_ids, (int)T, E, k, salt, topk_idx,
                                                                             topk_gate);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
