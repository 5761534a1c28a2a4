// Grouped bf16 GEMM on gfx950 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulation), shared by the expert forward and backward.
//
//   C[m][n] = sum_k A(m,k) * B(n,k)
//
// Operand access: "K-contiguous" (A(m,k) = A[m*lda + k]) is loaded straight
// into LDS with 16-byte vectors; "K-strided" (A(m,k) = A[k*lda + m]) is loaded
// as 8x8 bf16 blocks (eight 16-byte rows along m) and transposed in registers
// so that LDS always holds [m][k] with k contiguous, the layout the MFMA
// operand reads want (one 16-byte read per lane per 16-deep step).
//
// Grouping:
//   row-grouped: group g owns rows offsets[g]..offsets[g+1]-1 of A and the
//     weight B + g*b_group (expert forward and data gradients);
//   K-grouped:   group g reduces over rows offsets[g]..offsets[g+1]-1 of
//     both A and B and writes C_g = out + g*out_group (weight gradients).
//
// Tiles are 128x128x64 or 256x256x64 (chosen per call from the average rows
// per group), 4 waves, LDS double-buffered with register prefetch.  The
// kernel is persistent: grid = a multiple of 8 workgroups;
// workgroup i runs on XCD i%8 and, in each round, takes the tile at position
// i/8 of that XCD's contiguous share of the round, so neighbouring tiles
// (which share a weight panel or an activation panel) meet in one XCD's L2.
#pragma once

#include "moe_common.h"

namespace moe_gemm {

// Row tile of the small configuration: the tile schedule's unit for
// row-grouped GEMMs is chosen per call (TILE_SMALL or TILE_LARGE rows).
constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;  // +8 bf16 per LDS row: conflict-free b128 reads
constexpr int BM_LARGE = 256, BN_LARGE = 256;

enum Epi {
  EPI_SWIGLU = 0,      // H = silu(G)*U from paired gate/up columns; optional bf16 G|U save
  EPI_F32 = 1,         // plain fp32 store
  EPI_SWIGLU_BWD = 2,  // dG = dH*U*silu'(G), dU = dH*silu(G) from saved G|U, bf16 out
};

struct Args {
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B;
  int64_t ldb;
  int64_t b_group;           // row-grouped: elements between groups' weights
  int64_t K;                 // row-grouped: reduction length (multiple of BK)
  int64_t M;                 // K-grouped: output rows per group
  int64_t N;                 // output columns
  const int32_t* offsets;    // [G+1]
  const int32_t* mt_prefix;  // [G+1] row tiles before group g (row-grouped)
  int G;
  int NB;                    // column blocks
  int MT;                    // K-grouped: row tiles per group
  void* out;
  int64_t ldo;
  int64_t out_group;         // K-grouped: elements between groups' outputs
  const bf16_t* gu_in;       // SwiGLU-bwd: saved [rows, 2N] G|U
  bf16_t* gu_out;            // SwiGLU: G|U save (or null); SwiGLU-bwd: dG|dU out
};

// 8x8 bf16 transpose: in[r] holds row r (8 values along m), out[m] holds the
// 8 values of column m (along k).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = in[2 * j][c], hi = in[2 * j + 1][c];
      out[2 * c][j] = (lo & 0xFFFFu) | (hi << 16);
      out[2 * c + 1][j] = (lo >> 16) | (hi & 0xFFFF0000u);
    }
}

// TM x TN workgroup tile, 4 waves in 2x2, each wave (TM/2) x (TN/2) made of
// FM x FN blocks of 32x32.  128x128 tiles keep two workgroups per CU; 256x256
// tiles (one workgroup per CU, accumulators in AGPRs) halve the LDS bytes
// read per MFMA flop and give each 64-deep slab ~2k MFMA cycles per wave to
// hide the next slab's global loads.
template <int TM, int TN, bool AK, bool BKC, bool KG, int EPI>
__global__ __launch_bounds__(256, (TM * TN > 128 * 128) ? 1 : 2) void gemm_kernel(Args p) {
  constexpr int WTM = TM / 2, WTN = TN / 2, FM = WTM / 32, FN = WTN / 32;
  constexpr int CA = TM / 32, CB = TN / 32;      // 16-byte chunks per thread per slab (K-contiguous)
  constexpr int UA = TM / 128, UB = TN / 128;    // 8x8 transpose units per thread-half per slab
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(TM + TN) * LDK];
  __shared__ int32_t s_pref[MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (!KG) {
    for (int i = tid; i <= p.G; i += 256) s_pref[i] = p.mt_prefix[i];
    __syncthreads();
  }
  const int NB = p.NB;
  const int total = KG ? p.G * p.MT * NB : s_pref[p.G] * NB;
  const int per = gridDim.x >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  for (int base = 0;; base += gridDim.x) {
    const int L = base + xcd * per + slot;
    if (L >= total) break;
    int e, mt, nb;
    int64_t row0, row_end, kbeg, kend;
    if (KG) {
      e = L / (p.MT * NB);
      const int r = L - e * p.MT * NB;
      nb = r / p.MT;
      mt = r - nb * p.MT;
      row0 = (int64_t)mt * TM;
      row_end = p.M;
      kbeg = p.offsets[e];
      kend = p.offsets[e + 1];
    } else {
      int lo = 0, hi = p.G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] * NB <= L) lo = mid; else hi = mid;
      }
      e = lo;
      const int mte = s_pref[e + 1] - s_pref[e];
      const int local = L - s_pref[e] * NB;
      nb = local / mte;
      mt = local - nb * mte;
      row0 = p.offsets[e] + (int64_t)mt * TM;
      row_end = p.offsets[e + 1];
      kbeg = 0;
      kend = p.K;
    }
    const int nk = (int)((kend - kbeg + BK - 1) / BK);
    const bf16_t* Bg = KG ? p.B : p.B + (int64_t)e * p.b_group;

    // ---- loader set-up
    // K-contiguous operands: 16-byte chunks, chunk c -> tile row c/8, k (c%8)*8
    const bf16_t* a_row[CA];
    const bf16_t* b_row[CB];
    if (AK) {
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int c = tid + 256 * i;
        int64_t r = row0 + (c >> 3);
        if (r >= row_end) r = row_end - 1;   // ragged tail: a valid row, its result is discarded
        a_row[i] = p.A + r * p.lda + (c & 7) * 8;
      }
    }
    if (BKC) {
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int c = tid + 256 * i, r = c >> 3;
        int64_t n;
        if (EPI == EPI_SWIGLU) {
          const int jb = r >> 5;   // 32-row blocks of the tile: gate, up, gate, up, ...
          n = ((jb & 1) ? p.N : 0) + (int64_t)nb * (TN / 2) + (jb >> 1) * 32 + (r & 31);
        } else {
          n = (int64_t)nb * TN + r;
          if (n >= p.N) n = p.N - 1;
        }
        b_row[i] = Bg + n * p.ldb + (c & 7) * 8;
      }
    }
    // K-strided operands: 8(k) x 8(m) units; unit u -> k block u/(T/8), m block
    // u%(T/8).  Threads 0..127 serve A, threads 128..255 serve B.
    const bool t_is_a = tid < 128;
    constexpr int UMAX = UA > UB ? UA : UB;
    const int nunits = t_is_a ? (AK ? 0 : UA) : (BKC ? 0 : UB);
    const int tdim = t_is_a ? TM : TN;
    const bf16_t* t_src[UMAX];
    bool t_mvalid[UMAX];
    int t_kb[UMAX], t_mb[UMAX];
    const int64_t t_ld = t_is_a ? p.lda : p.ldb;
#pragma unroll
    for (int q = 0; q < UMAX; ++q) {
      const int u = (tid & 127) + 128 * q;
      t_kb[q] = u / (tdim / 8);
      t_mb[q] = u % (tdim / 8);
      t_src[q] = nullptr;
      t_mvalid[q] = false;
      if (q < nunits) {
        if (t_is_a) {
          const int64_t m = row0 + 8 * t_mb[q];
          t_mvalid[q] = m < row_end;
          t_src[q] = p.A + (kbeg + 8 * t_kb[q]) * p.lda + m;
        } else {
          const int64_t n = (int64_t)nb * TN + 8 * t_mb[q];
          t_mvalid[q] = n < p.N;
          t_src[q] = Bg + (kbeg + 8 * t_kb[q]) * p.ldb + n;
        }
      }
    }

    u32x4 ra[AK ? CA : 1], rb[BKC ? CB : 1], rt[UMAX][8];
    auto gload = [&](int it) {
      const int64_t k0 = (int64_t)it * BK;
      if (AK) {
#pragma unroll
        for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_row[i] + k0);
      }
      if (BKC) {
#pragma unroll
        for (int i = 0; i < CB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_row[i] + k0);
      }
#pragma unroll
      for (int q = 0; q < UMAX; ++q) {
        if (q < nunits) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bool ok = t_mvalid[q] && (kbeg + k0 + 8 * t_kb[q] + i < kend);
            rt[q][i] = ok ? *reinterpret_cast<const u32x4*>(t_src[q] + (k0 + i) * t_ld) : u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    };
    auto sstore = [&](int buf) {
      bf16_t* sa = smem[buf];
      bf16_t* sb = smem[buf] + TM * LDK;
      if (AK) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
          const int c = tid + 256 * i;
          *reinterpret_cast<u32x4*>(sa + (c >> 3) * LDK + (c & 7) * 8) = ra[i];
        }
      }
      if (BKC) {
#pragma unroll
        for (int i = 0; i < CB; ++i) {
          const int c = tid + 256 * i;
          *reinterpret_cast<u32x4*>(sb + (c >> 3) * LDK + (c & 7) * 8) = rb[i];
        }
      }
#pragma unroll
      for (int q = 0; q < UMAX; ++q) {
        if (q < nunits) {
          u32x4 tr[8];
          transpose8x8(rt[q], tr);
          bf16_t* s = (t_is_a ? sa : sb) + (8 * t_mb[q]) * LDK + 8 * t_kb[q];
#pragma unroll
          for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(s + i * LDK) = tr[i];
        }
      }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = f32x16{};

    if (nk > 0) {
      gload(0);
      sstore(0);
      __syncthreads();
      for (int it = 0; it < nk; ++it) {
        const int cur = it & 1;
        if (it + 1 < nk) gload(it + 1);
        const bf16_t* sa = smem[cur] + (wm * WTM + (lane & 31)) * LDK + 8 * (lane >> 5);
        const bf16_t* sb = smem[cur] + TM * LDK + (wn * WTN + (lane & 31)) * LDK + 8 * (lane >> 5);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
          bf16x8 a[FM], b[FN];
#pragma unroll
          for (int mi = 0; mi < FM; ++mi) a[mi] = *reinterpret_cast<const bf16x8*>(sa + mi * 32 * LDK + kk);
#pragma unroll
          for (int ni = 0; ni < FN; ++ni) b[ni] = *reinterpret_cast<const bf16x8*>(sb + ni * 32 * LDK + kk);
#pragma unroll
          for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
        }
        if (it + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
      }
    }

    // ---- epilogue.  32x32 MFMA result: register r of a lane holds row
    // 8*(r/4) + 4*(lane/32) + r%4 and column lane%32 of the 32x32 block.
    if (EPI == EPI_SWIGLU) {
      bf16_t* H = static_cast<bf16_t*>(p.out);
#pragma unroll
      for (int pi = 0; pi < FN / 2; ++pi) {   // wave column blocks come in (gate, up) pairs
        const int64_t col = (int64_t)nb * (TN / 2) + (wn * (WTN / 64) + pi) * 32 + (lane & 31);
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = row0 + wm * WTM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < row_end) {
              const float g = acc[mi][2 * pi][r], u = acc[mi][2 * pi + 1][r];
              H[row * p.ldo + col] = (bf16_t)f32_to_bf16(silu_f32(g) * u);
              if (p.gu_out) {
                p.gu_out[row * 2 * p.N + col] = (bf16_t)f32_to_bf16(g);
                p.gu_out[row * 2 * p.N + p.N + col] = (bf16_t)f32_to_bf16(u);
              }
            }
          }
      }
    } else {
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const int64_t col = (int64_t)nb * TN + wn * WTN + ni * 32 + (lane & 31);
        if (col >= p.N) continue;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = row0 + wm * WTM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= row_end) continue;
            const float v = acc[mi][ni][r];
            if (EPI == EPI_F32) {
              float* C = static_cast<float*>(p.out) + (KG ? (int64_t)e * p.out_group : 0);
              C[row * p.ldo + col] = v;
            } else {  // EPI_SWIGLU_BWD: v = dH[row][col]
              const float g = bf16_to_f32(p.gu_in[row * 2 * p.N + col]);
              const float u = bf16_to_f32(p.gu_in[row * 2 * p.N + p.N + col]);
              const float sg = 1.0f / (1.0f + __expf(-g));
              p.gu_out[row * 2 * p.N + col] = (bf16_t)f32_to_bf16(v * u * sg * (1.0f + g * (1.0f - sg)));
              p.gu_out[row * 2 * p.N + p.N + col] = (bf16_t)f32_to_bf16(v * g * sg);
            }
          }
      }
    }
  }
}

// Persistent grid: at most `per_cu` workgroups per CU, a multiple of 8.
int grid_for(int64_t tiles_upper, int per_cu);

// Fills in the tile counts of `a` for a TM x TN tile and launches.  `rows`
// (row-grouped only) bounds the row tiles: sum over groups of
// ceil(n_g/TM) <= ceil(rows/TM) + G.  a.mt_prefix must have been built with
// bm = TM.
template <int TM, int TN, bool AK, bool BKC, bool KG, int EPI>
moe_status launch_cfg(Args a, int64_t rows, hipStream_t s) {
  a.NB = EPI == EPI_SWIGLU ? (int)(a.N / (TN / 2)) : (int)ceil_div(a.N, TN);
  int64_t tiles;
  if (KG) {
    a.MT = (int)ceil_div(a.M, TM);
    tiles = (int64_t)a.G * a.MT * a.NB;
  } else {
    tiles = (ceil_div(rows, TM) + a.G) * a.NB;
  }
  gemm_kernel<TM, TN, AK, BKC, KG, EPI><<<grid_for(tiles, TM * TN > 128 * 128 ? 1 : 2), 256, 0, s>>>(a);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

template <bool AK, bool BKC, bool KG, int EPI>
moe_status launch_gemm(const Args& a, bool large, int64_t rows, hipStream_t s) {
  return large ? launch_cfg<BM_LARGE, BN_LARGE, AK, BKC, KG, EPI>(a, rows, s)
               : launch_cfg<BM, BN, AK, BKC, KG, EPI>(a, rows, s);
}

// Row-grouped GEMMs use the large tile when groups average at least this many
// rows (fewer rows waste too much of a 256-row tile on ragged tails).
constexpr int64_t LARGE_MIN_ROWS = 512;

inline bool use_large_rows(int64_t rows, int G, int64_t f) {
  return rows >= LARGE_MIN_ROWS * G && f % (BN_LARGE / 2) == 0;
}

}  // namespace moe_gemm
