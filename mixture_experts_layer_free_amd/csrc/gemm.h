// Grouped bf16 GEMM on gfx950 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulation), shared by the expert forward and backward.
//
//   C[m][n] = sum_k A(m,k) * B(n,k)
//
// Operand access: "K-contiguous" (A(m,k) = A[m*lda + k]) or "K-strided"
// (A(m,k) = A[k*lda + m]); the same for B with n in place of m.
//
// Grouping:
//   row-grouped: group g owns rows offsets[g]..offsets[g+1]-1 of A and the
//     weight B + g*b_group (expert forward and data gradients);
//   K-grouped:   group g reduces over rows offsets[g]..offsets[g+1]-1 of
//     both A and B and writes C_g = out + g*out_group (weight gradients).
//
// Data movement.  Operand tiles go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging).  Each tile's buffer
// resource is bounded to the rows that tile may use, so reads past a group's
// last row (ragged row tiles, K tails of the weight gradients) return zeros.
// The LDS holds an S-stage ring of BK-deep slabs; one barrier per slab, with
// the loads for slab it+S-1 issued right after it, so S-1 slabs are in flight
// while the waves multiply.  LDS rows carry no padding; 16-byte chunks are
// XOR-swizzled by row so the MFMA operand reads are free of bank conflicts:
//   K-contiguous slab [T rows][BK]: fragments by ds_read_b128 (8 k of one row);
//   K-strided slab [BK rows][T]:    fragments by two ds_read_b64_tr_b16, which
//     gather 4 consecutive k of one column per lane (the transpose happens in
//     the LDS read, none in registers).
//
// Workgroup: 4 waves in 2x2, each wave (TM/2) x (TN/2) of 32x32 MFMA blocks
// (1x4 for the half tiles below).
// Measured on MI355X, the loop is bound by the operand stream from L2 into
// LDS (removing the in-loop loads alone lifts it from ~1.07 to ~1.75 PF/s):
// the slab loads of a step are spread between its MFMAs (issued together,
// the 4 waves' 32 loads queue behind one texture unit for ~500 cycles while
// the matrix cores idle), and the tile order below is chosen for L2 reuse.
// Two tile shapes: 256x256 (one workgroup per CU, accumulators in AGPRs,
// half the LDS bytes per MFMA flop) and 128x128 (two workgroups per CU);
// use_large_tile below picks one (the large one where it fits).  A row-grouped
// 256x256 tile whose group ends within its first 128 rows runs as 128x256
// with the four waves side by side (each 128 x 64), so small experts and
// ragged last tiles do half the MFMA work per wave and half the A loads
// while still reading their weights once.  The kernel is persistent: the
// grid is a multiple of 8 workgroups; workgroup i runs on XCD i%8 and in each
// round takes the tile at position i/8 of that XCD's contiguous share of the
// round, so neighbouring tiles (sharing a weight or activation panel) meet in
// one XCD's L2.
#pragma once
#include <algorithm>
#include <atomic>

#include "moe_common.h"

namespace moe_gemm {

constexpr int BM = 128, BN = 128;              // small tile
constexpr int BM_LARGE = 256, BN_LARGE = 256;  // large tile
constexpr int BK = 32;                         // slab depth
constexpr int STAGES = 4;                      // LDS ring depth

enum Epi {
  EPI_SWIGLU = 0,      // H = silu(G)*U from paired gate/up columns; optional bf16 G|U save
  EPI_F32 = 1,         // plain fp32 store
  EPI_SWIGLU_BWD = 2,  // dG = dH*U*silu'(G), dU = dH*silu(G) from saved G|U, bf16 out
  EPI_BF16 = 3,        // plain bf16 store (round to nearest even), row-grouped only
};

struct Args {
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B;
  int64_t ldb;
  int64_t b_group;           // row-grouped: elements between groups' weights
  int64_t b_rows;            // row-grouped: rows of one group's weight (its buffer bound)
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
  // SwiGLU (up-projection) only: when set, GEMM row r reads row a_rows[r] of
  // A, which has a_rows_total rows (the permute fused into the operand load)
  const int32_t* a_rows;
  int64_t a_rows_total;
  // K-grouped with a K-strided B only (GB kernels): reduction row r reads
  // row b_gather[r] of B, which has b_gather_rows rows
  const int32_t* b_gather;
  int64_t b_gather_rows;
  // SwiGLU-bwd only: the accumulator row r is scaled by row_scale[r] before
  // the SwiGLU backward (or by 1 when null); with h_in set, the epilogue also
  // writes dg_part[r * (N / 32) + c / 32] = sum over the 32 columns c.. of
  // acc[r][c] * h_in[r][c] (the unscaled accumulator against the saved H)
  const float* row_scale;
  const bf16_t* h_in;
  float* dg_part;
  // K-grouped only: the chunk schedule (kg_schedule_kernel) and the partial
  // outputs of experts split into several row chunks (see launch_cfg)
  int32_t* kg_sched;
  float* kg_partial;
  // Row-grouped with a K-contiguous B on the 256 x 256 tile only: B is held
  // in tile order (pack_b_kernel): the TN x BK slab s of group g's column
  // block nb is one contiguous block at B + ((g * NB + nb) * (K / BK) + s) *
  // TN * BK, its row r at r * BK -- each slab is one contiguous read
  int b_packed;
};

// K-grouped (weight-gradient) schedule.  Each group's reduction rows are cut
// into chunks of at most C rows; an item is one output tile of one chunk.
// A group of more than one chunk writes one partial output per chunk, and
// kg_reduce_kernel adds them in chunk order (deterministic).  Chunks go in
// order of decreasing cost; the item list is cut into 8 ranges of equal
// cost, one per XCD, and an XCD's workgroups take the range's items in order
// from an atomic counter, then help drain the other XCDs' ranges (which
// only spreads the work: each item is computed once, so results do not
// depend on the order).
// Schedule block (int32): [0..8] item range starts per XCD (9 = end),
// [9..16] the XCDs' next items, [17] split groups, [18] chunks, [19] gmax
// (the chunk arrays' length), then chunk expert / first row / end row /
// output slot (gmax each), then split group / first slot / chunk count (G each).
constexpr int KG_HDR = 32;
constexpr int KG_OVERHEAD_ROWS = 448;   // a tile's prologue and epilogue, in rows of K
struct KgPlan {
  int64_t tpg, chunk, gmax, smax, mn;
};
inline KgPlan kg_plan(int64_t M, int64_t N, int64_t rows, int G, bool large) {
  const int64_t tm = large ? BM_LARGE : BM, tn = large ? BN_LARGE : BN;
  KgPlan k{};
  k.tpg = ceil_div(M, tm) * ceil_div(N, tn);
  // a chunk's tile costs at most half a workgroup's share on a 256-workgroup grid
  const int64_t c = ceil_div(std::max<int64_t>(rows, 1) * k.tpg, 512);
  k.chunk = std::max<int64_t>(512, ceil_div(c, 64) * 64);
  k.gmax = G + ceil_div(rows, k.chunk);
  k.smax = 2 * ceil_div(rows, k.chunk);
  k.mn = M * N;
  return k;
}
inline size_t kg_sched_bytes(const KgPlan& k, int G) { return (size_t)(KG_HDR + 4 * k.gmax + 3 * (int64_t)G) * 4; }
inline size_t kg_partial_bytes(const KgPlan& k) { return (size_t)(k.smax * k.mn) * 4; }

typedef __attribute__((address_space(3))) void lds_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte chunk swizzles
__device__ __forceinline__ int swz_kc(int row) { return ((row >> 2) ^ (row >> 1)) & 3; }  // slab [T][32]
__device__ __forceinline__ int swz_ks(int k) { return (k & 3) << 2; }                     // slab [32][T]

template <int TM, int TN>
constexpr int lds_bytes() {
  return STAGES * (TM + TN) * BK * 2 + 16 * ((MOE_MAX_EXPERTS + 1 + 3) / 4);
}

__device__ __forceinline__ bf16x8 join8(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Order of one group's mt x nb tiles: bands of BAND column blocks; inside a
// band, row tiles in order with the column blocks fastest.  A persistent
// round hands each XCD a run of consecutive tiles, so its concurrent tiles
// form a compact (rows x BAND) block: every operand slab an XCD pulls into its
// L2 feeds several workgroups (row panels are shared by BAND tiles, column
// panels by all the block's row tiles).  The forward expert GEMMs use bands
// of 4 (an XCD's 32 tiles: 8 row tiles x 4 column blocks; 64-expert
// training shape, both forward GEMMs: 1.733 -> 1.688 ms against bands of 8),
// the others bands of 8.
template <int BAND>
__device__ __forceinline__ void band_order(int t, int mts, int nbs, int& mt, int& nb) {
  const int band = t / (mts * BAND);
  const int r = t - band * mts * BAND;
  const int w = nbs - band * BAND < BAND ? nbs - band * BAND : BAND;   // width of this band
  mt = r / w;
  nb = band * BAND + (r - mt * w);
}

// Scheduling pattern of one slab step with NM MFMAs, NR LDS fragment reads
// and NV slab loads: the reads go between the MFMAs of the first half, the
// loads between those of the second half.
template <int NM, int NR, int NV, int M = 0>
__device__ __forceinline__ void interleave() {
  constexpr int H = NM / 2;
  if constexpr (M < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    if constexpr (M < H) {
      constexpr int ds = (M + 1) * NR / H - M * NR / H;
      if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);   // LDS read
    } else {
      constexpr int vm = (M - H + 1) * NV / (NM - H) - (M - H) * NV / (NM - H);
      if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);   // buffer load
    }
    interleave<NM, NR, NV, M + 1>();
  }
}

// One output tile: TM x TN, the four waves WM x WN (WM = 4 / WN), each
// (TM / WM) x (TN / WN) of 32x32 MFMA blocks; operand slabs, main loop and
// epilogue as described at the top of this file.
template <int TM, int TN, int WN, bool AK, bool BKC, bool KG, int EPI, bool GB, int SPLIT = 1>
__device__ __forceinline__ void gemm_tile(const Args& p, char* smem, int e, int nb, int64_t row0, int64_t row_end,
                                          int64_t kbeg, int64_t kend, float* kg_out = nullptr) {
  constexpr int WTM = TM / (4 / WN), WTN = TN / WN, FM = WTM / 32, FN = WTN / 32;
  constexpr int SA = TM * BK * 2, SB = TN * BK * 2, STAGE = SA + SB;   // bytes
  constexpr int LA = SA / 4096, LB = SB / 4096;                         // 1 KB loads per wave per slab
  constexpr int LPS = LA + LB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // slabs: K / BK for a row-grouped GEMM (even: K is a multiple of 64);
  // rounded up to even for a K-grouped one (the extra slab reads zeros)
  const int nk = KG ? (int)((kend - kbeg + 2 * BK - 1) / (2 * BK)) * 2 : (int)((kend - kbeg) / BK);

  // ---- buffer resources and per-lane byte offsets of this tile's loads.
  // A K-contiguous: rows row0.. of A, bounded at the group's last row.
  // A K-strided:    rows kbeg.. of A, bounded at kend; columns from row0.
  const void* a_base;
  const void* b_base;
  int64_t a_bytes, b_bytes;
  uint32_t a_voff[LA], b_voff[LB];
  uint32_t a_step, b_step;   // bytes per slab
  if (AK && !KG && (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD) && p.a_rows) {   // row-grouped A gathered through a_rows
    // gathered rows: the buffer spans all of A (under 2^31 bytes), a row past
    // the group's end or an index outside [0, a_rows_total) gets an offset
    // past the buffer (its loads read zeros); a valid index's offset fits 32 bits
    a_base = p.A;
    a_bytes = p.a_rows_total * p.lda * 2;
    a_step = BK * 2;
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int r = (wave * LA + q) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz_kc(r);
      const uint32_t src = row0 + r < row_end ? (uint32_t)p.a_rows[row0 + r] : 0xFFFFFFFFu;
      a_voff[q] = src < (uint32_t)p.a_rows_total ? src * (uint32_t)(p.lda * 2) + c * 16 : 0x80000000u;
    }
  } else if (AK) {
    const int64_t a_rows = row_end - row0 < TM ? row_end - row0 : TM;
    a_base = p.A + row0 * p.lda;
    a_bytes = a_rows * p.lda * 2;
    a_step = BK * 2;
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int r = (wave * LA + q) * 16 + (lane >> 2);      // tile row of this lane
      const int c = (lane & 3) ^ swz_kc(r);                  // logical chunk it fetches
      a_voff[q] = (uint32_t)((int64_t)r * p.lda * 2 + c * 16);
    }
  } else {
    a_base = p.A + kbeg * p.lda;
    a_bytes = (kend - kbeg) * p.lda * 2;
    a_step = (uint32_t)(BK * p.lda * 2);
    constexpr int CPR = TM / 8;                              // chunks per slab row
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int idx = (wave * LA + q) * 64 + lane;           // physical chunk index in the slab
      const int k = idx / CPR, pc = idx % CPR;
      const int c = pc ^ swz_ks(k);
      a_voff[q] = (uint32_t)((int64_t)k * p.lda * 2 + (row0 + c * 8) * 2);
    }
  }
  if (BKC && p.b_packed) {
    // packed blocks are TN * SPLIT wide; a column part (SPLIT > 1) reads rows
    // (nb % SPLIT) * TN .. of its block's slabs
    constexpr int TNP = TN * SPLIT;
    const int64_t nslab = p.K / BK;
    const int64_t part_off = (int64_t)(nb % SPLIT) * TN * BK;
    b_base = p.B + ((int64_t)e * p.NB + nb / SPLIT) * nslab * (TNP * BK) + part_off;
    b_bytes = nslab * (TNP * BK * 2) - part_off * 2;
    b_step = TNP * BK * 2;
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int r = (wave * LB + q) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz_kc(r);
      b_voff[q] = (uint32_t)(r * (BK * 2) + c * 16);
    }
  } else if (BKC) {
    b_base = p.B + (int64_t)e * p.b_group;
    b_bytes = p.b_rows * p.ldb * 2;
    b_step = BK * 2;
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int r = (wave * LB + q) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz_kc(r);
      int64_t n;
      if (EPI == EPI_SWIGLU) {
        const int jb = r >> 5;   // 32-row blocks of the tile: gate, up, gate, up, ...
        n = ((jb & 1) ? p.N : 0) + (int64_t)nb * (TN / 2) + (jb >> 1) * 32 + (r & 31);
      } else {
        n = (int64_t)nb * TN + r;   // rows past the weight read as zeros
      }
      b_voff[q] = (uint32_t)(n * p.ldb * 2 + c * 16);
    }
  } else if (GB) {
    // gathered rows: the buffer spans all of B; b_voff holds the column part
    // of each load, the row part comes per slab from b_gather (gb_rows below)
    b_base = p.B;
    b_bytes = p.b_gather_rows * p.ldb * 2;
    b_step = 0;
    constexpr int CPR = TN / 8;
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int idx = (wave * LB + q) * 64 + lane;
      const int k = idx / CPR, pc = idx % CPR;
      const int c = pc ^ swz_ks(k);
      b_voff[q] = (uint32_t)(((int64_t)nb * TN + c * 8) * 2);
    }
  } else {
    const bf16_t* Bk = KG ? p.B + kbeg * p.ldb : p.B + (int64_t)e * p.b_group;
    b_base = Bk;
    b_bytes = (KG ? (kend - kbeg) : p.K) * p.ldb * 2;
    b_step = (uint32_t)(BK * p.ldb * 2);
    constexpr int CPR = TN / 8;
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int idx = (wave * LB + q) * 64 + lane;
      const int k = idx / CPR, pc = idx % CPR;
      const int c = pc ^ swz_ks(k);
      b_voff[q] = (uint32_t)((int64_t)k * p.ldb * 2 + ((int64_t)nb * TN + c * 8) * 2);
    }
  }

  // Loads of one BK-deep slab into its ring stage: LA (LB) 1 KB
  // buffer->LDS loads per wave for A (B), 16 bytes per lane placed
  // lane-linearly.  The host compilation pass only needs this kernel's
  // signature (for its launch stub) and cannot type the LDS-pointer cast,
  // so the statement exists in the device pass only.
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(uni(a_base), uni(a_bytes));
  const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(uni(b_base), uni(b_bytes));

  // Gathered B (GB): a wave's loads of one slab cover its rows 8*wave ..
  // 8*wave+7 (BK/4 rows, since each wave moves a quarter of the slab); lane
  // l of load q takes row q*RPL + l/(TN/8) of them.  Each lane reads the LB
  // row indices it needs with vector loads one slab ahead (gb_rows), over a
  // buffer holding the group's rows only; a row past the group's end gets
  // -1.  gb_voffs turns them into the per-lane byte offsets of a slab's
  // loads; a row outside B (or -1) gets an offset past the buffer, so its
  // load reads zeros.  (Scalar loads of the indices would bring the scalar
  // memory counter into the loop; those loads complete out of order with
  // the LDS reads, so every wait for a fragment read would then have to
  // wait for the scalar load just issued as well.)
  static_assert(!GB || (KG && !BKC && LB * 64 / (TN / 8) == 8), "gathered B: K-grouped, K-strided, 8 rows per wave");
  constexpr int RPL = 64 / (TN / 8);
  static_assert(!GB || RPL == 2 || RPL == 4, "gathered B: 2 or 4 rows per load");
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  const int wv = (int)uni((uint32_t)wave);
  const uint32_t gb_lrow = (uint32_t)(lane / (TN / 8));   // this lane's row within a load's RPL rows
  const uint32_t gb_nrel = (uint32_t)(kend - kbeg);        // the group's rows (under 2^31)
  const __amdgpu_buffer_rsrc_t rs_g =
      make_rsrc(uni((const void*)(GB ? p.b_gather + kbeg : p.offsets)), uni(GB ? (kend - kbeg) * 4 : (int64_t)0));
  // row of the group (from kbeg) that this lane's load q of a slab takes
  auto gb_rel = [&](int slab, int q) -> uint32_t {
    return uni((uint32_t)slab) * BK + 8 * wv + q * RPL + gb_lrow;
  };
  auto gb_rows = [&](int slab) -> i32x4 {
    i32x4 t = {0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < LB; ++q)
      t[q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs_g, gb_rel(slab, q) * 4u, 0, 0);
    return t;
  };
  const uint32_t gb_rb = (uint32_t)(p.ldb * 2), gb_nrows = (uint32_t)p.b_gather_rows;
  auto gb_voffs = [&](int slab, i32x4 t, uint32_t (&vo)[LB]) {
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int32_t row = gb_rel(slab, q) < gb_nrel ? t[q] : -1;   // rows past the group's end
      // B has under 2^31 bytes, so a row inside it gives a 32-bit offset;
      // -1 and any row outside B go past the buffer
      vo[q] = (uint32_t)row < gb_nrows ? (uint32_t)row * gb_rb + b_voff[q] : 0x80000000u;
    }
  };
#if defined(__HIP_DEVICE_COMPILE__)
#define MOE_ISSUE(slab_, gvo_)                                                                       \
do {                                                                                               \
  const int slab = (slab_);                                                                        \
  const bool live_ = slab < nk;   /* a slab past the end is pushed out of range: its loads read zeros */ \
  char* st_ = smem + (slab % STAGES) * STAGE;                                                      \
  _Pragma("unroll") for (int q = 0; q < LA; ++q)                                                   \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_t*)(st_ + (wave * LA + q) * 1024), 16, a_voff[q], \
                                             uni(live_ ? (uint32_t)slab * a_step : 0x80000000u), 0, 0); \
  _Pragma("unroll") for (int q = 0; q < LB; ++q)                                                   \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_t*)(st_ + SA + (wave * LB + q) * 1024), 16,      \
                                             GB ? (gvo_)[q] : b_voff[q],                           \
                                             uni(GB ? 0u : live_ ? (uint32_t)slab * b_step : 0x80000000u), 0, 0); \
} while (0)
#else
#define MOE_ISSUE(slab_, gvo_) ((void)(slab_), (void)(gvo_))
#endif

  // fragment byte offsets inside a stage for the 16-deep step kk
  auto frag_kc = [&](int region, int row, int kk) -> int {   // K-contiguous slab: ds_read_b128
    const int c = (kk >> 3) + (lane >> 5);
    return region + row * (BK * 2) + ((c ^ swz_kc(row)) << 4);
  };
  auto frag_ks = [&](int region, int T, int col0, int kk, int t) -> int {   // K-strided slab: ds_read_b64_tr_b16
    const int g = lane >> 4, a = lane & 15;
    const int k = kk + 8 * (g >> 1) + 4 * t + (a >> 2);
    const int m = col0 + 16 * (g & 1) + 4 * (a & 3);
    return region + k * (T * 2) + (((m >> 3) ^ swz_ks(k)) << 4) + ((m & 7) << 1);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = f32x16{};

  // Fragment reads of one slab into a register set (both 16-deep steps).
  auto read_frags = [&](const char* st, bf16x8 (&fa)[2][FM], bf16x8 (&fb)[2][FN]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 16 * h;
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) {
        const int m0 = wm * WTM + mi * 32;
        if (AK) {
          fa[h][mi] = *reinterpret_cast<const bf16x8*>(st + frag_kc(0, m0 + (lane & 31), kk));
        } else {
          fa[h][mi] = join8(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + frag_ks(0, TM, m0, kk, 0))),
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + frag_ks(0, TM, m0, kk, 1))));
        }
      }
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const int n0 = wn * WTN + ni * 32;
        if (BKC) {
          fb[h][ni] = *reinterpret_cast<const bf16x8*>(st + frag_kc(SA, n0 + (lane & 31), kk));
        } else {
          fb[h][ni] = join8(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + frag_ks(SA, TN, n0, kk, 0))),
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + frag_ks(SA, TN, n0, kk, 1))));
        }
      }
    }
  };
  // The same reads through a restrict pointer, for the kernels with a
  // K-strided operand.  Before a transposing read (ds_read_b64_tr_b16) the
  // compiler cannot tell which ring stage the LDS-DMA loads in flight
  // write, so it waits for all of them (vmcnt(0)), which leaves one slab of
  // prefetch instead of two; a read it knows to be distinct from those
  // loads (the alias scope that inlining a restrict parameter attaches)
  // gets no such wait.  The ring's own waits already order them: a step
  // reads the stage whose loads its vmcnt wait and barrier completed, and
  // the loads in flight fill other stages.  Training shape: dgrad-down
  // 0.89 -> 0.80 ms, W_down's gradient 0.71 -> 0.57, W_gate_up's 1.31 ->
  // 1.20, dgrad-up 1.18 -> 1.01.  (The K-contiguous reads of the forward
  // GEMMs never get the wait; their code is left as it is.)
  auto read_frags_r = [&](const char* __restrict__ st, bf16x8 (&fa)[2][FM], bf16x8 (&fb)[2][FN]) {
    read_frags(st, fa, fb);
  };
  auto mfmas = [&](const bf16x8 (&fa)[2][FM], const bf16x8 (&fb)[2][FN]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[h][mi], fb[h][ni], acc[mi][ni], 0, 0, 0);
  };
  // LDS reads per slab (a transposing fragment takes two) and MFMAs per slab
  constexpr int NREAD = 2 * (FM * (AK ? 1 : 2) + FN * (BKC ? 1 : 2));
  constexpr int NMFMA = 2 * FM * FN;

  // Slab step it: make slab it+1 visible, refill the ring three slabs
  // ahead, and multiply slab it (registers `ca/cb`, read one step earlier)
  // while the fragments of slab it+1 stream into `na/nb`.  Slab it+3 goes
  // into the stage slab it-1 used; every wave consumed those fragments
  // before this step's barrier.  The step has no branch: loads of slabs
  // past the end are out of range (they write zeros into a stage nobody
  // reads), so every step waits for the same count of loads, and the
  // MFMAs, fragment reads and slab loads form one scheduling region:
  // each MFMA is followed by its share of the reads (first half of the
  // step) or of the loads (second half; the compiler keeps the loads
  // behind the reads since both touch LDS).  Steps come in pairs that swap
  // the two register sets; the slab count is even (K of a row-grouped
  // GEMM is a multiple of 64; a K-grouped tile rounds up and its extra slab
  // reads zeros past the group's rows).  On the last step the reads fetch a
  // stage whose contents are never used.
  // With a gathered B, the step first starts the loads of the next slab's
  // row indices (tn), in a scheduling region of its own ahead of the slab
  // loads (so they are older than the slab loads that the next step's wait
  // leaves in flight), then turns the indices read one step earlier (tc)
  // into load offsets inside the MFMA region, where that chain of vector
  // instructions runs in the shadow of the MFMAs instead of before them.
#define MOE_STEP(it_, ca, cb, na, nb_, tc, tn)                                                    \
do {                                                                                          \
  const int it = (it_);                                                                       \
  wait_vmcnt<LPS>();                                                                          \
  block_barrier();                                                                            \
  uint32_t gvo[LB];                                                                           \
  if constexpr (GB) {                                                                         \
    tn = gb_rows(it + STAGES);                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    gb_voffs(it + STAGES - 1, tc, gvo);                                                       \
  }                                                                                           \
  if constexpr (AK && BKC) read_frags(smem + ((it + 1) % STAGES) * STAGE, na, nb_);           \
  else read_frags_r(smem + ((it + 1) % STAGES) * STAGE, na, nb_);                             \
  MOE_ISSUE(it + STAGES - 1, gvo);                                                            \
  mfmas(ca, cb);                                                                              \
  interleave<NMFMA, NREAD, LPS>();                                                            \
  __builtin_amdgcn_sched_barrier(0);                                                          \
} while (0)

  // Stores of the previous tile's epilogue may still be in flight: they are
  // older than this tile's loads, so the load waits below cover them too.
  if (nk > 0) {
    i32x4 tk0 = {}, tk1 = {};   // gathered B: row indices of the slab the next step loads, and of the one after
    if constexpr (GB) {
      static_assert(STAGES == 4, "gathered-B prologue");
      const i32x4 t0 = gb_rows(0), t1 = gb_rows(1), t2 = gb_rows(2);
      uint32_t v0[LB], v1[LB], v2[LB];
      gb_voffs(0, t0, v0);
      gb_voffs(1, t1, v1);
      gb_voffs(2, t2, v2);
      tk0 = gb_rows(3);
      MOE_ISSUE(0, v0);
      MOE_ISSUE(1, v1);
      MOE_ISSUE(2, v2);
    } else {
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) MOE_ISSUE(s, b_voff);
    }
    bf16x8 fa0[2][FM], fb0[2][FN], fa1[2][FM], fb1[2][FN];
    wait_vmcnt<(STAGES - 2) * LPS>();
    block_barrier();
    read_frags(smem, fa0, fb0);
    for (int it2 = 0; it2 < nk; it2 += 2) {
      MOE_STEP(it2, fa0, fb0, fa1, fb1, tk0, tk1);
      MOE_STEP(it2 + 1, fa1, fb1, fa0, fb0, tk1, tk0);
    }
    wait_vmcnt<0>();   // the out-of-range tail loads still land in the ring
    block_barrier();   // every wave is done with the ring before the epilogue stages in it
  }
#undef MOE_STEP
#undef MOE_ISSUE

  // ---- epilogue.  Each 32x32 result block goes through LDS (the ring is
  // idle now): the MFMA layout (register r of a lane = row 8*(r/4) +
  // 4*(lane/32) + r%4, column lane%32) is written out, then read back as
  // 4-column chunks so every global store is a row-contiguous vector
  // (16 bytes of fp32 or 8 bytes of bf16) and the SwiGLU math runs on them.
  // Results are stored non-temporally: they are far larger than the L2,
  // which is left to the operand panels the neighbouring tiles reuse.
  {
    constexpr int SLD = 36;   // floats per staged row (16-byte aligned rows, spread banks)
    float* stg0 = reinterpret_cast<float*>(smem) + wave * (2 * 32 * SLD);
    float* stg1 = stg0 + 32 * SLD;
    auto stage = [&](float* stg, const f32x16& v) {
#pragma unroll
      for (int r = 0; r < 16; ++r) stg[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SLD + (lane & 31)] = v[r];
    };
    if constexpr (EPI == EPI_SWIGLU && FN % 4 == 0) {
      // Two (gate, up) pairs at a time: their 64 H columns (and 64 of G and
      // of U) make whole 128-byte rows, 8 rows per store.  Four staged blocks
      // per wave (the ring is idle).
      bf16_t* H = static_cast<bf16_t*>(p.out);
      float* sg = reinterpret_cast<float*>(smem) + wave * (4 * 32 * SLD);
#pragma unroll
      for (int pi = 0; pi < FN / 2; pi += 2) {
        const int64_t col0 = (int64_t)nb * (TN / 2) + (wn * (WTN / 64) + pi) * 32;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
          for (int q = 0; q < 4; ++q) stage(sg + q * 32 * SLD, acc[mi][2 * pi + q]);   // gate, up, gate, up
#pragma unroll
          for (int j = 0; j < 4; ++j) {   // 8 columns (16 bytes of bf16) per lane
            const int idx = lane + 64 * j, rr = idx >> 3, c8 = (idx & 7) * 8;
            const int64_t row = row0 + wm * WTM + mi * 32 + rr;
            const float* gs = sg + (2 * (c8 >> 5)) * 32 * SLD + rr * SLD + (c8 & 31);
            const float* us = gs + 32 * SLD;
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(gs);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(gs + 4);
            const f32x4 u0 = *reinterpret_cast<const f32x4*>(us);
            const f32x4 u1 = *reinterpret_cast<const f32x4*>(us + 4);
            if (row < row_end) {
              const int64_t col = col0 + c8;
              const u32x4 h = {pack_bf16x2(silu_f32(g0[0]) * u0[0], silu_f32(g0[1]) * u0[1]),
                               pack_bf16x2(silu_f32(g0[2]) * u0[2], silu_f32(g0[3]) * u0[3]),
                               pack_bf16x2(silu_f32(g1[0]) * u1[0], silu_f32(g1[1]) * u1[1]),
                               pack_bf16x2(silu_f32(g1[2]) * u1[2], silu_f32(g1[3]) * u1[3])};
              __builtin_nontemporal_store(h, reinterpret_cast<u32x4*>(H + row * p.ldo + col));
              if (p.gu_out) {
                const u32x4 gg = {pack_bf16x2(g0[0], g0[1]), pack_bf16x2(g0[2], g0[3]), pack_bf16x2(g1[0], g1[1]),
                                  pack_bf16x2(g1[2], g1[3])};
                const u32x4 uu = {pack_bf16x2(u0[0], u0[1]), pack_bf16x2(u0[2], u0[3]), pack_bf16x2(u1[0], u1[1]),
                                  pack_bf16x2(u1[2], u1[3])};
                __builtin_nontemporal_store(gg, reinterpret_cast<u32x4*>(p.gu_out + row * 2 * p.N + col));
                __builtin_nontemporal_store(uu, reinterpret_cast<u32x4*>(p.gu_out + row * 2 * p.N + p.N + col));
              }
            }
          }
        }
      }
    } else if (EPI == EPI_SWIGLU) {
      bf16_t* H = static_cast<bf16_t*>(p.out);
#pragma unroll
      for (int pi = 0; pi < FN / 2; ++pi) {   // wave column blocks come in (gate, up) pairs
        const int64_t col0 = (int64_t)nb * (TN / 2) + (wn * (WTN / 64) + pi) * 32;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
          stage(stg0, acc[mi][2 * pi]);
          stage(stg1, acc[mi][2 * pi + 1]);
#pragma unroll
          for (int j = 0; j < 2; ++j) {   // 8 columns (16 bytes of bf16) per lane
            const int idx = lane + 64 * j, rr = idx >> 2, c8 = (idx & 3) * 8;
            const int64_t row = row0 + wm * WTM + mi * 32 + rr;
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(stg0 + rr * SLD + c8);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(stg0 + rr * SLD + c8 + 4);
            const f32x4 u0 = *reinterpret_cast<const f32x4*>(stg1 + rr * SLD + c8);
            const f32x4 u1 = *reinterpret_cast<const f32x4*>(stg1 + rr * SLD + c8 + 4);
            if (row < row_end) {
              const int64_t col = col0 + c8;
              const u32x4 h = {pack_bf16x2(silu_f32(g0[0]) * u0[0], silu_f32(g0[1]) * u0[1]),
                               pack_bf16x2(silu_f32(g0[2]) * u0[2], silu_f32(g0[3]) * u0[3]),
                               pack_bf16x2(silu_f32(g1[0]) * u1[0], silu_f32(g1[1]) * u1[1]),
                               pack_bf16x2(silu_f32(g1[2]) * u1[2], silu_f32(g1[3]) * u1[3])};
              __builtin_nontemporal_store(h, reinterpret_cast<u32x4*>(H + row * p.ldo + col));
              if (p.gu_out) {
                const u32x4 gg = {pack_bf16x2(g0[0], g0[1]), pack_bf16x2(g0[2], g0[3]), pack_bf16x2(g1[0], g1[1]),
                                  pack_bf16x2(g1[2], g1[3])};
                const u32x4 uu = {pack_bf16x2(u0[0], u0[1]), pack_bf16x2(u0[2], u0[3]), pack_bf16x2(u1[0], u1[1]),
                                  pack_bf16x2(u1[2], u1[3])};
                __builtin_nontemporal_store(gg, reinterpret_cast<u32x4*>(p.gu_out + row * 2 * p.N + col));
                __builtin_nontemporal_store(uu, reinterpret_cast<u32x4*>(p.gu_out + row * 2 * p.N + p.N + col));
              }
            }
          }
        }
      }
    } else if (EPI == EPI_F32) {
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const int64_t col0 = (int64_t)nb * TN + wn * WTN + ni * 32;
        if (col0 >= p.N) continue;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
          stage(stg0, acc[mi][ni]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int idx = lane + 64 * j, rr = idx >> 3, c4 = (idx & 7) * 4;
            const int64_t row = row0 + wm * WTM + mi * 32 + rr;
            const f32x4 v = *reinterpret_cast<const f32x4*>(stg0 + rr * SLD + c4);
            const int64_t col = col0 + c4;
            if (row < row_end && col < p.N) {
              float* C = KG ? kg_out : static_cast<float*>(p.out);   // K-grouped: this chunk's output
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(C + row * p.ldo + col));
            }
          }
        }
      }
    } else if (EPI == EPI_BF16) {
      // two neighbouring 32-column blocks at a time, so each store covers
      // whole 128-byte rows (8 rows of 64 columns per store)
      static_assert(EPI != EPI_BF16 || !KG, "bf16 store: row-grouped GEMMs only");
      static_assert(FN % 2 == 0, "column blocks in pairs");
      bf16_t* C = static_cast<bf16_t*>(p.out);
#pragma unroll
      for (int ni = 0; ni < FN; ni += 2) {
        const int64_t col0 = (int64_t)nb * TN + wn * WTN + ni * 32;
        if (col0 >= p.N) continue;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
          stage(stg0, acc[mi][ni]);
          stage(stg1, acc[mi][ni + 1]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {   // 8 columns (16 bytes of bf16) per lane
            const int idx = lane + 64 * j, rr = idx >> 3, c8 = (idx & 7) * 8;
            const int64_t row = row0 + wm * WTM + mi * 32 + rr;
            const float* src = (c8 < 32 ? stg0 : stg1 - 32) + rr * SLD + c8;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
            const int64_t col = col0 + c8;
            if (row < row_end && col < p.N) {
              const u32x4 o = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                               pack_bf16x2(v1[2], v1[3])};
              __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(C + row * p.ldo + col));
            }
          }
        }
      }
    } else {  // EPI_SWIGLU_BWD: dH block -> dG, dU from the saved G, U
      // Two neighbouring 32-column blocks at a time (a pair), so every load
      // and store covers whole 128-byte rows: each instruction moves 8 rows
      // of 64 columns (a unit; a pair is 4 units).  The saved G|U (and H,
      // for the gate-gradient partials) come from HBM by 16-byte loads (8
      // columns per lane) into a ring of 4 units in the registers the
      // fragments used in the loop: unit j of pair b is reloaded with unit j
      // of pair b + 1 as soon as it is consumed, so a pair's worth of loads
      // stays in flight.
      static_assert(FN % 2 == 0, "column blocks in pairs");
      constexpr int NPAIR = FM * FN / 2;
      const bool dgp = p.h_in != nullptr;
      const int64_t np32 = p.N / 32;   // gate-gradient partials per row
      u32x4 gq[4], uq[4], hq[4];
      float sq[4];
      // Every lane loads, from a clamped address when its row or column is
      // past the end (the value is then never used: the arithmetic and the
      // stores below keep to live lanes).  Loads under a per-lane branch,
      // into registers zeroed first, made the compiler wait for every load
      // in flight before each block, which emptied the prefetch.
      const bool scaled = p.row_scale != nullptr;
      const bf16_t* hsrc = dgp ? p.h_in : p.gu_in;                           // any readable rows when absent
      const float* ssrc = scaled ? p.row_scale : reinterpret_cast<const float*>(p.gu_in);
      auto load_unit = [&](int b, int j, u32x4& gb, u32x4& ub, u32x4& hb, float& sb) {
        const int mi = b / (FN / 2), ni = 2 * (b % (FN / 2));
        const int idx = lane + 64 * j, rr = idx >> 3, c8 = (idx & 7) * 8;
        int64_t row = row0 + wm * WTM + mi * 32 + rr;
        int64_t col = (int64_t)nb * TN + wn * WTN + ni * 32 + c8;
        row = row < row_end ? row : row_end - 1;
        col = col < p.N ? col : p.N - 8;
        gb = *reinterpret_cast<const u32x4*>(p.gu_in + row * 2 * p.N + col);
        ub = *reinterpret_cast<const u32x4*>(p.gu_in + row * 2 * p.N + p.N + col);
        hb = *reinterpret_cast<const u32x4*>(hsrc + (dgp ? row * p.N + col : 0));
        const float sv = ssrc[scaled ? row : 0];
        sb = scaled ? sv : 1.0f;
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) load_unit(0, j, gq[j], uq[j], hq[j], sq[j]);
#pragma unroll
      for (int b = 0; b < NPAIR; ++b) {
        const int mi = b / (FN / 2), ni = 2 * (b % (FN / 2));
        stage(stg0, acc[mi][ni]);
        stage(stg1, acc[mi][ni + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 gcj = gq[j], ucj = uq[j], hcj = hq[j];
          const float scj = sq[j];
          if (b + 1 < NPAIR) load_unit(b + 1, j, gq[j], uq[j], hq[j], sq[j]);
          const int idx = lane + 64 * j, rr = idx >> 3, c8 = (idx & 7) * 8;
          const int64_t row = row0 + wm * WTM + mi * 32 + rr;
          const int64_t col = (int64_t)nb * TN + wn * WTN + ni * 32 + c8;
          const float* src = (c8 < 32 ? stg0 : stg1 - 32) + rr * SLD + c8;
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
          const bool live = row < row_end && col < p.N;
          if (dgp) {
            // gate-gradient partial of this row's 32 columns: the four lanes
            // holding them (consecutive lanes) add their 8 products in a fixed order
            float part = 0.f;
            if (live) {
              const float vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                part = fmaf(vv[2 * q], bf16_to_f32(hcj[q] & 0xFFFFu), part);
                part = fmaf(vv[2 * q + 1], bf16_to_f32(hcj[q] >> 16), part);
              }
            }
            part += __shfl_xor(part, 1, MOE_WAVE);
            part += __shfl_xor(part, 2, MOE_WAVE);
            if (live && (lane & 3) == 0) p.dg_part[row * np32 + (col >> 5)] = part;
          }
          if (live) {
            const float s = scj;
            const float v[8] = {s * v0[0], s * v0[1], s * v0[2], s * v0[3], s * v1[0], s * v1[1], s * v1[2], s * v1[3]};
            u32x4 o1, o2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float dg[2], du[2];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const uint32_t gw = gcj[q], uw = ucj[q];
                const float g = bf16_to_f32(h ? gw >> 16 : gw & 0xFFFFu);
                const float u = bf16_to_f32(h ? uw >> 16 : uw & 0xFFFFu);
                const float sg = sigmoid_fast(g);
                dg[h] = v[2 * q + h] * u * sg * (1.0f + g * (1.0f - sg));
                du[h] = v[2 * q + h] * g * sg;
              }
              o1[q] = pack_bf16x2(dg[0], dg[1]);
              o2[q] = pack_bf16x2(du[0], du[1]);
            }
            __builtin_nontemporal_store(o1, reinterpret_cast<u32x4*>(p.gu_out + row * 2 * p.N + col));
            __builtin_nontemporal_store(o2, reinterpret_cast<u32x4*>(p.gu_out + row * 2 * p.N + p.N + col));
          }
        }
      }
    }
  }
  block_barrier();   // staging areas sit in the ring: free them before the next tile's loads
}

template <int TM, int TN, bool AK, bool BKC, bool KG, int EPI, bool GB>
__global__ __launch_bounds__(256, (TM * TN > 128 * 128) ? 1 : 2)
__attribute__((amdgpu_waves_per_eu((TM * TN > 128 * 128) ? 1 : 2, (TM * TN > 128 * 128) ? 1 : 2)))
void gemm_kernel(Args p) {
  constexpr int STAGE = (TM + TN) * BK * 2;   // bytes of one ring stage
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int32_t* s_pref = reinterpret_cast<int32_t*>(smem + STAGES * STAGE);

  const int tid = threadIdx.x;
  if (!KG) {
    for (int i = tid; i <= p.G; i += 256) s_pref[i] = p.mt_prefix[i];
    __syncthreads();
  }
  const int NB = p.NB;
  const int total = KG ? p.G * p.MT * NB : s_pref[p.G] * NB;
  const int per = gridDim.x >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  if constexpr (KG) {
    // items from this XCD's range of the chunk schedule, in order; once it is
    // drained, from the next XCDs' ranges (each range's tail holds its
    // cheapest items), so no workgroup idles while any item is left
    const int32_t* ks = p.kg_sched;
    const int tpg = p.MT * NB, gmax = ks[19];
    const int32_t* g_e = ks + KG_HDR;
    const int32_t* g_kb = g_e + gmax;
    const int32_t* g_ke = g_kb + gmax;
    const int32_t* g_out = g_ke + gmax;
    int32_t* s_item = s_pref;
    (void)total, (void)per, (void)slot;
    int src = xcd, hops = 0;   // thread 0's current range and the ranges it has left behind
    for (;;) {
      if (tid == 0) {
        int L = -1;
        while (hops < 8) {
          const int t = atomicAdd(p.kg_sched + 9 + src, 1);
          if (t < ks[src + 1]) {
            L = t;
            break;
          }
          src = (src + 1) & 7;
          ++hops;
        }
        *s_item = L;
      }
      __syncthreads();
      const int L = *s_item;
      if (L < 0) break;
      const int g = L / tpg;
      int mt, nb;
      // column blocks slowest: an XCD's concurrent tiles of one chunk share
      // its B panels (for W_gate_up's gradient, gathered x rows, the costlier
      // operand to fetch) and re-read A's instead (W_gate_up's gradient on
      // 16384 tokens, top-8: 1.36 -> 1.32 ms)
      band_order<8>(L - g * tpg, NB, p.MT, nb, mt);
      const int e = g_e[g], oslot = g_out[g];
      float* outp = oslot < 0 ? static_cast<float*>(p.out) + (int64_t)e * p.out_group
                              : p.kg_partial + (int64_t)oslot * p.M * p.N;
      gemm_tile<TM, TN, 2, AK, BKC, KG, EPI, GB>(p, smem, e, nb, (int64_t)mt * TM, p.M, g_kb[g], g_ke[g], outp);
    }
    return;
  }
  // Tile L of the row-grouped list: its group, row tile and column block.
  auto tile_at = [&](int L, int& e, int& mt, int& nb) {
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] * NB <= L) lo = mid; else hi = mid;
    }
    e = lo;
    band_order<BKC ? 4 : 8>(L - s_pref[e] * NB, s_pref[e + 1] - s_pref[e], NB, mt, nb);
  };
  const int grid = gridDim.x, pos = xcd * per + slot;
  int end = total;
  // The last round, when under half full, runs its tiles cut into `split`
  // parts (two column halves of 256 x 128, or four quarters of 128 x 128)
  // on the workgroups that would otherwise idle through it.  A part makes
  // each of its outputs by the same MFMA sequence along K as the whole tile,
  // so the results are the same bits.  A quarter moves half the operand
  // bytes per slab of a 256 x 64 column part for the same MFMA work; a
  // quarter below the group's last row has nothing to do and is skipped.
  // The parts run first, outside the persistent loop: inside it, the
  // compiler keeps their set-up values live across every tile, which costs
  // registers the whole-tile path needs.  An XCD's positions are
  // contiguous, so a tile's parts share its L2.
  if constexpr (TM == 256 && TN == 256 && AK && !KG) {
    const int full_end = total - total % grid, rem = total - full_end;
    int split = 1;
    while (rem > 0 && split < 4 && rem * split * 2 <= grid) split *= 2;
    split = (int)uni((uint32_t)split);
    if (split > 1) {
      end = full_end;
      if (pos < rem * split) {
        int e, mt, nb;
        tile_at(full_end + pos / split, e, mt, nb);
        const int part = pos % split;
        const int64_t row0 = p.offsets[e] + (int64_t)mt * TM, row_end = p.offsets[e + 1];
        if (split == 4) {
          const int64_t r0 = row0 + (int64_t)(part >> 1) * (TM / 2);
          if (uni(r0) < uni(row_end))
            gemm_tile<TM / 2, TN / 2, 2, AK, BKC, KG, EPI, GB, 2>(p, smem, e, nb * 2 + (part & 1), r0, row_end, 0,
                                                                 p.K);
        } else {
          gemm_tile<TM, TN / 2, 2, AK, BKC, KG, EPI, GB, 2>(p, smem, e, nb * 2 + part, row0, row_end, 0, p.K);
        }
      }
    }
  }
  for (int base = 0;; base += grid) {
    const int L = base + pos;
    if (L >= end) break;
    int e, mt, nb;
    tile_at(L, e, mt, nb);
    const int64_t row0 = p.offsets[e] + (int64_t)mt * TM, row_end = p.offsets[e + 1];
    const int64_t kbeg = 0, kend = p.K;
    // A 256-row tile whose group ends within its first 128 rows (a small
    // expert, or a group's ragged last tile) runs as 128 x 256 with the waves
    // side by side: half the MFMA work on each wave's path and half the A
    // loads, the same weight reads.
    if constexpr (TM == 256 && TN == 256 && AK && !KG) {
      if (uni(row_end - row0) <= TM / 2) {
        gemm_tile<TM / 2, TN, 4, AK, BKC, KG, EPI, GB>(p, smem, e, nb, row0, row_end, kbeg, kend);
        continue;
      }
    }
    gemm_tile<TM, TN, 2, AK, BKC, KG, EPI, GB>(p, smem, e, nb, row0, row_end, kbeg, kend);
  }
}

// Persistent grid: at most `per_cu` workgroups per CU, a multiple of 8.
int grid_for(int64_t tiles_upper, int per_cu);

// The K-grouped chunk schedule (into a.kg_sched) and, after the GEMM, the
// ordered sum of the split groups' partial outputs (ffn.hip).
moe_status kg_schedule_launch(const int32_t* offsets, int G, const KgPlan& k, int32_t* sched, hipStream_t s);
moe_status kg_reduce_launch(const int32_t* sched, const KgPlan& k, int G, const float* partial, float* out,
                            int64_t out_group, hipStream_t s);

// Raises a kernel's dynamic-LDS limit on the current device.
moe_status lds_attr(const void* fn, int bytes);

// Per device (the current one): 0 not yet set, 1 set, 2 failed.
constexpr int kMaxAttrDevices = 64;
template <typename K>
moe_status lds_attr_once(std::atomic<int> (&done)[kMaxAttrDevices], K* fn, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxAttrDevices) dev = 0;
  int st = done[dev].load(std::memory_order_acquire);
  if (st == 0) {
    st = lds_attr(reinterpret_cast<const void*>(fn), bytes) == MOE_OK ? 1 : 2;
    done[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MOE_OK : MOE_EHIP;
}

// Fills in the tile counts of `a` for a TM x TN tile and launches.  `rows`
// (row-grouped only) bounds the row tiles: sum over groups of
// ceil(n_g/TM) <= ceil(rows/TM) + G.  a.mt_prefix must have been built with
// bm = TM.
// K-grouped launches (rows = the reduction rows of all groups) run the chunk
// schedule first and the partial-output sum after; a.kg_sched and
// a.kg_partial must hold kg_sched_bytes / kg_partial_bytes of
// kg_plan(a.M, a.N, rows, a.G, TM == BM_LARGE).
template <int TM, int TN, bool AK, bool BKC, bool KG, int EPI, bool GB = false>
moe_status launch_cfg(Args a, int64_t rows, hipStream_t s) {
  a.NB = EPI == EPI_SWIGLU ? (int)(a.N / (TN / 2)) : (int)ceil_div(a.N, TN);
  int64_t tiles;
  KgPlan kp{};
  if (KG) {
    a.MT = (int)ceil_div(a.M, TM);
    kp = kg_plan(a.M, a.N, rows, a.G, TM == BM_LARGE);
    tiles = kp.gmax * a.MT * a.NB;
    const moe_status st = kg_schedule_launch(a.offsets, a.G, kp, a.kg_sched, s);
    if (st != MOE_OK) return st;
  } else {
    tiles = (ceil_div(rows, TM) + a.G) * a.NB;
  }
  constexpr int lds = lds_bytes<TM, TN>();
  static std::atomic<int> attr_done[kMaxAttrDevices];
  const moe_status attr = lds_attr_once(attr_done, &gemm_kernel<TM, TN, AK, BKC, KG, EPI, GB>, lds);
  if (attr != MOE_OK) return attr;
  gemm_kernel<TM, TN, AK, BKC, KG, EPI, GB><<<grid_for(tiles, TM * TN > 128 * 128 ? 1 : 2), 256, lds, s>>>(a);
  MOE_LAUNCH_CHECK();
  if (KG) return kg_reduce_launch(a.kg_sched, kp, a.G, a.kg_partial, static_cast<float*>(a.out), a.out_group, s);
  return MOE_OK;
}

template <bool AK, bool BKC, bool KG, int EPI, bool GB = false>
moe_status launch_gemm(const Args& a, bool large, int64_t rows, hipStream_t s) {
  return large ? launch_cfg<BM_LARGE, BN_LARGE, AK, BKC, KG, EPI, GB>(a, rows, s)
               : launch_cfg<BM, BN, AK, BKC, KG, EPI, GB>(a, rows, s);
}

// Tile choice of a row-grouped GEMM: the large tile whenever the SwiGLU
// columns allow it (f a multiple of 128).  It moves half the operand bytes
// per flop of the small one, reads each group's weights once per 256 rows
// (the small tile: once per 128), and a tile whose group ends within its
// first 128 rows runs as 128 x 256, so ragged tails waste little.  Measured
// on 64 experts (d = 2048, f = 1024), large against small, both expert GEMMs:
// 130-250 rows per expert 0.28 against 0.35 ms, 300-470 rows 0.50 against
// 0.58, 400-511 rows 0.52 against 0.68, 257-320 rows even; on 256 experts of
// ~128 rows, 7.7 -> 5.6 ms.  The small tile serves the other widths.
inline bool use_large_tile(int64_t f) { return f % (BN_LARGE / 2) == 0; }

}  // namespace moe_gemm
