// Grouped SwiGLU experts.
//
// Lesson "专家组合 (MoE)" (AI Engineering from Scratch), Concept: each expert
// is an independent FFN, usually SwiGLU; Shared experts: an always-on expert
// is the same FFN applied to every token.  The AREX article on The Ultimate
// MoE Training Handbook (paragraph on the expert-count sweet spot) notes that
// finer experts mean smaller GEMMs that cost step time: the kernels below are
// built so that many small, unequal expert GEMMs still fill the chip.
//
// bf16 path: two grouped GEMMs on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation, both "NT" (activations and nn.Linear weights are both
// contiguous along the reduction dimension):
//   up:   [G | U] = X W_gu^T, epilogue H = silu(G) * U (bf16), optionally G, U
//   down: Y = H W_down^T (fp32 out)
// Tiles are 128 rows x 128 weight rows x 64 deep, 4 waves of 64x64, LDS
// double-buffered with a register prefetch.  The tile list is built on the
// device from the expert offsets (no host sync): expert e owns
// ceil(n_e/128) row tiles; tiles are ordered (expert, column block, row
// tile), so consecutive tiles share the weight panel.  The kernel is
// persistent: workgroup i sits on XCD i%8 and takes, in each round, a tile
// from that XCD's contiguous share of the round, so tiles that reuse a weight
// panel run on one XCD and hit its L2.
#include "moe_common.h"

namespace {

constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;  // +8 bf16: conflict-free 16-byte reads

struct GemmArgs {
  const bf16_t* A;           // [rows, K]
  const bf16_t* B;           // group g: B + g*b_group, rows of K
  int64_t b_group;
  int64_t K;
  int64_t N;                 // output columns
  const int32_t* offsets;    // [G+1]
  const int32_t* mt_prefix;  // [G+1] row tiles before group g
  int G;
  int NB;                    // column blocks
  void* out;                 // bf16 H [rows, N] (SwiGLU) or f32 Y [rows, N]
  bf16_t* gu;                // [rows, 2N] or null (SwiGLU only)
};

enum { EPI_SWIGLU = 0, EPI_F32 = 1 };

template <int EPI>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(GBM + GBN) * GLD];
  __shared__ int32_t s_pref[MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  for (int i = tid; i <= p.G; i += 256) s_pref[i] = p.mt_prefix[i];
  __syncthreads();
  const int NB = p.NB;
  const int total = s_pref[p.G] * NB;
  const int per = gridDim.x >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int64_t K = p.K;
  const int nk = (int)(K / GBK);

  for (int base = 0;; base += gridDim.x) {
    const int L = base + xcd * per + slot;
    if (L >= total) break;
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] * NB <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int mte = s_pref[e + 1] - s_pref[e];
    const int local = L - s_pref[e] * NB;
    const int nb = local / mte, mt = local % mte;
    const int row0 = p.offsets[e] + mt * GBM;
    const int row_end = p.offsets[e + 1];
    const bf16_t* Bg = p.B + (int64_t)e * p.b_group;

    // per-thread source rows of the A and B tiles (4 x 16-byte chunks each)
    const bf16_t* asrc[4];
    const bf16_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, kc = (c & 7) * 8;
      int ar = row0 + r;
      if (ar >= row_end) ar = row_end - 1;   // ragged tail: valid row, result discarded
      asrc[i] = p.A + (int64_t)ar * K + kc;
      int64_t wr;
      if (EPI == EPI_SWIGLU) {
        const int jb = r >> 5;                 // 32-row blocks: gate, up, gate, up
        wr = ((jb & 1) ? p.N : 0) + (int64_t)nb * 64 + (jb >> 1) * 32 + (r & 31);
      } else {
        wr = (int64_t)nb * GBN + r;
        if (wr >= p.N) wr = p.N - 1;
      }
      bsrc[i] = Bg + wr * K + kc;
    }
    u32x4 ra[4], rb[4];
    auto gload = [&](int64_t k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(asrc[i] + k0);
        rb[i] = *reinterpret_cast<const u32x4*>(bsrc[i] + k0);
      }
    };
    auto sstore = [&](int buf) {
      bf16_t* sa = smem[buf];
      bf16_t* sb = smem[buf] + GBM * GLD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = (c & 7) * 8;
        *reinterpret_cast<u32x4*>(sa + r * GLD + kc) = ra[i];
        *reinterpret_cast<u32x4*>(sb + r * GLD + kc) = rb[i];
      }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

    gload(0);
    sstore(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      const int cur = it & 1;
      if (it + 1 < nk) gload((int64_t)(it + 1) * GBK);
      const bf16_t* sa = smem[cur] + (wm * 64 + (lane & 31)) * GLD + 8 * (lane >> 5);
      const bf16_t* sb = smem[cur] + GBM * GLD + (wn * 64 + (lane & 31)) * GLD + 8 * (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < GBK; kk += 16) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) a[mi] = *reinterpret_cast<const bf16x8*>(sa + mi * 32 * GLD + kk);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) b[ni] = *reinterpret_cast<const bf16x8*>(sb + ni * 32 * GLD + kk);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
      }
      if (it + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }

    // 32x32 MFMA result: register r of lane holds row 8*(r/4) + 4*(lane/32) + r%4, column lane%32
    if (EPI == EPI_SWIGLU) {
      bf16_t* H = static_cast<bf16_t*>(p.out);
      const int64_t col = (int64_t)nb * 64 + wn * 32 + (lane & 31);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < row_end) {
            const float g = acc[mi][0][r], u = acc[mi][1][r];
            H[(int64_t)row * p.N + col] = (bf16_t)f32_to_bf16(silu_f32(g) * u);
            if (p.gu) {
              p.gu[(int64_t)row * 2 * p.N + col] = (bf16_t)f32_to_bf16(g);
              p.gu[(int64_t)row * 2 * p.N + p.N + col] = (bf16_t)f32_to_bf16(u);
            }
          }
        }
    } else {
      float* Y = static_cast<float*>(p.out);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t col = (int64_t)nb * GBN + wn * 64 + ni * 32 + (lane & 31);
        if (col >= p.N) continue;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < row_end) Y[(int64_t)row * p.N + col] = acc[mi][ni][r];
          }
      }
    }
  }
}

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

__global__ __launch_bounds__(256) void ffn_up_f32_kernel(const float* __restrict__ X, int64_t rows, int64_t d,
                                                         const int32_t* __restrict__ offsets, int G, int64_t f,
                                                         const float* __restrict__ Wgu, float* __restrict__ gu,
                                                         float* __restrict__ H) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * f) return;
  const int64_t row = id / f, n = id % f;
  const int g = group_of_row(offsets, G, (int)row);
  const float* xr = X + row * d;
  const float* wg = Wgu + (int64_t)g * 2 * f * d + n * d;
  const float* wu = wg + f * d;
  float a = 0.f, b = 0.f;
  for (int64_t i = 0; i < d; ++i) {
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
  const int g = group_of_row(offsets, G, (int)row);
  const float* hr = H + row * f;
  const float* w = Wd + (int64_t)g * d * f + n * f;
  float a = 0.f;
  for (int64_t j = 0; j < f; ++j) a = fmaf(hr[j], w[j], a);
  Y[row * d + n] = a;
}

}  // namespace

size_t moe_ffn_workspace(int G) { return align256((size_t)(G + 1) * sizeof(int32_t)); }

// Launches the two bf16 grouped GEMMs (also used by the backward for the
// shared forward pieces); mt_prefix must already hold the tile schedule.
moe_status moe_ffn_bf16_launch(const bf16_t* x_rows, int64_t rows, int64_t d, const int32_t* offsets,
                               const int32_t* mt_prefix, int G, int64_t f, const bf16_t* wgu, const bf16_t* wd,
                               bf16_t* gu, bf16_t* h, float* y, hipStream_t s) {
  const int max_wg = (2 * moe_num_cus()) & ~7;
  const int64_t mtiles = ceil_div(rows, GBM) + G;
  GemmArgs a{};
  a.A = x_rows;
  a.B = wgu;
  a.b_group = 2 * f * d;
  a.K = d;
  a.N = f;
  a.offsets = offsets;
  a.mt_prefix = mt_prefix;
  a.G = G;
  a.NB = (int)(f / 64);
  a.out = h;
  a.gu = gu;
  int64_t grid = std::min<int64_t>(max_wg, (mtiles * a.NB + 7) & ~7ll);
  grouped_gemm_kernel<EPI_SWIGLU><<<(unsigned)grid, 256, 0, s>>>(a);
  MOE_LAUNCH_CHECK();
  GemmArgs b{};
  b.A = h;
  b.B = wd;
  b.b_group = d * f;
  b.K = f;
  b.N = d;
  b.offsets = offsets;
  b.mt_prefix = mt_prefix;
  b.G = G;
  b.NB = (int)ceil_div(d, GBN);
  b.out = y;
  b.gu = nullptr;
  grid = std::min<int64_t>(max_wg, (mtiles * b.NB + 7) & ~7ll);
  grouped_gemm_kernel<EPI_F32><<<(unsigned)grid, 256, 0, s>>>(b);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

moe_status moe_tile_schedule_launch(const int32_t* offsets, int G, int32_t* mt_prefix, hipStream_t s) {
  tile_schedule_kernel<<<1, 1024, 0, s>>>(offsets, G, GBM, mt_prefix);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" moe_status moe_grouped_ffn(const void* x_rows, int64_t rows, int64_t d, int dtype, const int32_t* offsets, int G,
                                      int64_t f, const void* w_gate_up, const void* w_down, void* gu_saved, void* h, float* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!x_rows || !offsets || !w_gate_up || !w_down || !h || !y) return MOE_EINVAL;
  if (rows < 1 || d < 1 || f < 1 || G < 1) return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EINVAL;
  if (G > MOE_MAX_EXPERTS || rows >= (1ll << 31)) return MOE_ENOTSUP;
  hipStream_t s = moe_stream(stream);
  if (dtype == MOE_BF16) {
    if (d % 64 != 0 || f % 64 != 0) return MOE_ENOTSUP;
    if (!workspace || workspace_bytes < moe_ffn_workspace(G)) return MOE_EWORKSPACE;
    int32_t* mt_prefix = static_cast<int32_t*>(workspace);
    moe_status st = moe_tile_schedule_launch(offsets, G, mt_prefix, s);
    if (st != MOE_OK) return st;
    return moe_ffn_bf16_launch(static_cast<const bf16_t*>(x_rows), rows, d, offsets, mt_prefix, G, f,
                               static_cast<const bf16_t*>(w_gate_up), static_cast<const bf16_t*>(w_down),
                               static_cast<bf16_t*>(gu_saved), static_cast<bf16_t*>(h), y, s);
  }
  if (d % 4 != 0) return MOE_ENOTSUP;
  ffn_up_f32_kernel<<<(unsigned)ceil_div(rows * f, 256), 256, 0, s>>>(
      static_cast<const float*>(x_rows), rows, d, offsets, G, f, static_cast<const float*>(w_gate_up),
      static_cast<float*>(gu_saved), static_cast<float*>(h));
  MOE_LAUNCH_CHECK();
  ffn_down_f32_kernel<<<(unsigned)ceil_div(rows * d, 256), 256, 0, s>>>(static_cast<const float*>(h), rows, d, offsets, G,
                                                                        f, static_cast<const float*>(w_down), y);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
