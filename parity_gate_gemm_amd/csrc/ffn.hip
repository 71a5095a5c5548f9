// Grouped SwiGLU expert FFN over the dispatched segments (Composer 2 Technical
// Report, section 6.1 "Kernels", Figure 10: the MoE layer as one grouped GEMM per
// expert group).  Two launches:
//   GEMM1: h[j, n] = silu(sum_i x[tok(j), i] W1[e][n][i]) * (sum_i x[tok(j), i] W3[e][n][i])
//          with tok(j) = perm[j] / k for routed rows and j - T*k for the shared
//          expert's rows (the gather is fused into the A-tile loads);
//   GEMM2: out[j, c] = sum_n h[j, n] W2[e][c][n].
// A tile never mixes experts.  Every output element is produced by the same
// instruction sequence (one MFMA shape, K swept in ascending 64-wide steps, no
// split-K), so a row's result does not depend on which rows share its tile.
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = kGemmBM;   // 128 rows per tile
constexpr int BNR = 128;      // B rows (output features) staged per tile
constexpr int BK = 64;        // reduction step
constexpr int LDSS = BK + 8;  // LDS row stride in bf16 elements (144 B: conflict-free 16-B reads)

// Tuning knobs of the bf16 grouped GEMM (same results for every setting).
#ifndef MOE_GEMM_DEPTH
#define MOE_GEMM_DEPTH 1
#endif
#ifndef MOE_GEMM_NT_B
#define MOE_GEMM_NT_B 0
#endif
constexpr int kGemmDepth = MOE_GEMM_DEPTH;   // K-steps of loads in flight per thread
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 8
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;       // row tiles per raster group
constexpr bool kGemmNtB = MOE_GEMM_NT_B != 0; // nontemporal weight loads
// Widest tile (wavefronts along N) each bf16 GEMM uses where the shape divides; the
// narrower tiles give the same bits (each output is the same MFMA sequence over K).
#ifndef MOE_GEMM1_WN
#define MOE_GEMM1_WN 4
#endif
#ifndef MOE_GEMM2_WN
#define MOE_GEMM2_WN 4
#endif
// MXFP8 tile shape: wavefronts along M and N, 32-row B blocks per wavefront.
#ifndef MOE_MX_WM
#define MOE_MX_WM 2
#endif
#ifndef MOE_MX_WN
#define MOE_MX_WN 2
#endif
#ifndef MOE_MX_FN
#define MOE_MX_FN 2
#endif
#ifndef MOE_MX_WAVES
#define MOE_MX_WAVES 1   // minimum wavefronts per SIMD the register allocation must allow
#endif
#ifndef MOE_MX_RING
#define MOE_MX_RING 1   // MXFP8 GEMMs on the LDS ring where the shape tiles
#endif
#ifndef MOE_GEMM_DMA
#define MOE_GEMM_DMA 0
#endif
#ifndef MOE_GEMM_NARROW_WAVES
#define MOE_GEMM_NARROW_WAVES 1
#endif

#ifndef MOE_MX_XCD_CHUNK
#define MOE_MX_XCD_CHUNK 16
#endif
constexpr int kMxXcdChunk = MOE_MX_XCD_CHUNK;

// Segment table: segment s < E is routed expert s (rows offsets[s]..offsets[s+1]-1),
// segment E is the shared expert (rows T*k .. T*k+T-1).  mstart = exclusive prefix of
// the per-segment counts of tm-row tiles.  Offsets are clamped into [0, T*k] and flagged if
// they are not a valid segmentation.
__global__ __launch_bounds__(1024) void seg_table_kernel(const int32_t* __restrict__ offsets, int E,
                                                         long long Tk, int T, int has_shared, int tm,
                                                         int* __restrict__ mstart,
                                                         int* __restrict__ rowstart,
                                                         int* __restrict__ rowcount, int* flag) {
  __shared__ int cnt[kMaxExperts + 1];
  const int S = E + (has_shared ? 1 : 0);
  int bad = 0;
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    long long a, b;
    if (s < E) {
      a = offsets[s];
      b = offsets[s + 1];
      if (a < 0 || b < a || b > Tk || (s == 0 && a != 0) || (s == E - 1 && b != Tk)) bad = 1;
      a = a < 0 ? 0 : (a > Tk ? Tk : a);
      b = b < a ? a : (b > Tk ? Tk : b);
    } else {
      a = Tk;
      b = Tk + T;
    }
    rowstart[s] = (int)a;
    rowcount[s] = (int)(b - a);
    cnt[s] = (int)((b - a + tm - 1) / tm);
  }
  if (bad) raise_flag(flag, kFlagCorrupt);
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int s = 0; s < S; ++s) {
      mstart[s] = run;
      run += cnt[s];
    }
    mstart[S] = run;
  }
}

struct GemmArgs {
  const uint16_t* a;      // GEMM1: x [T][d]; GEMM2: h [rows][I]
  const int32_t* perm;    // GEMM1 only
  int T, k, E;
  long long Tk;
  const uint16_t* b0;     // GEMM1: W1 bank; GEMM2: W2 bank
  const uint16_t* b1;     // GEMM1: W3 bank
  const uint16_t* sb0;    // shared expert's matrices (may be null when S == E)
  const uint16_t* sb1;
  int K, N;               // reduction length; output width of one weight matrix
  int NT;                 // output-column tiles per segment
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  int S;
  uint16_t* out;          // GEMM1: h [rows][I]; GEMM2: out [rows][d]
  float* out_pre;         // MODE 2: pre-activations [rows][2I] (x W1, then x W3), fp32
  int* flag;
};

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + expf(-a)); }

// MODE 0: GEMM1 (W1 and W3, SwiGLU epilogue, 32 * WN output features per tile).
// MODE 1: GEMM2 (W2, 64 * WN output features per tile).
// MODE 2: GEMM1 without the epilogue: the fp32 pre-activations x W1 and x W3 (the
//         backward pass recomputes them; same MFMA sequence as MODE 0).
// 128 * WN threads = 2 x WN wavefronts; each wavefront owns a 64-row x 64-B-row part
// of the 128 x (64 * WN) tile as 2 x 2 MFMA 32x32x16 blocks.  In GEMM1 the staged B
// rows alternate 32-row blocks of W1 and W3 for the same features, so a wavefront's
// two column blocks are the W1 and W3 halves of 32 features.
// Wide tiles (WN >= 4) are held to 128 registers so that 4 wavefronts fit per SIMD.
template <int MODE, int DEPTH, bool NT_B, int WN>
__global__ __launch_bounds__(128 * WN)
__attribute__((amdgpu_waves_per_eu(WN >= 4 ? 4 : MOE_GEMM_NARROW_WAVES)))
void grouped_gemm_bf16_kernel(GemmArgs g) {
  constexpr bool G1 = MODE != 1;                // GEMM1 operands (gathered x; W1 / W3)
  constexpr int NTHR = 128 * WN;
  constexpr int BNW = 64 * WN;                  // staged B rows per tile
  constexpr int RSTEP = NTHR / 8;               // loader row stride
  constexpr int LA = BM / RSTEP, LB = BNW / RSTEP;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDSS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BNW * LDSS];

  // ---- tile decode: XCD-contiguous ranges of the segment-major tile list ----
  const int total = g.mstart[g.S] * g.NT;
  int tile;
  if (!xcd_tile<0>(total, tile)) return;
  int lo = 0, hi = g.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mstart[mid] * g.NT <= tile) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int mtiles = g.mstart[s + 1] - g.mstart[s];
  const int local = tile - g.mstart[s] * g.NT;
  // Row tiles in groups of kGroupM: within a group, consecutive tiles share a weight
  // slab (column tile) and the group's activation rows are reused by every column tile.
  const int grp = local / (kGroupM * g.NT), rem = local % (kGroupM * g.NT);
  const int gm = min(kGroupM, mtiles - grp * kGroupM);
  const int nt = rem / gm, mt = grp * kGroupM + rem % gm;
  const int row0 = g.rowstart[s] + mt * BM;
  const int mrows = min(BM, g.rowcount[s] - mt * BM);
  const int n0 = nt * (G1 ? BNW / 2 : BNW);
  const bool is_shared = (s == g.E);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = tid >> 3, lc = (tid & 7) * 8;   // loader: rows lr + RSTEP i, column chunk lc

  // ---- per-thread source rows.  A tile row r >= mrows only feeds output row r,
  //      which is never stored, so it re-reads the tile's first row instead. ----
  const uint16_t* aptr[LA];
  const uint16_t* bptr[LB];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = lr + RSTEP * i;
    const long long j = (long long)row0 + (r < mrows ? r : 0);
    long long src;
    if (G1) {
      if (is_shared) {
        src = j - g.Tk;
      } else {
        src = g.perm[j] / g.k;
      }
      if (src < 0 || src >= g.T) {
        bad = 1;
        src = 0;
      }
    } else {
      src = j;
    }
    aptr[i] = g.a + src * (long long)g.K + lc;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = lr + RSTEP * i;
    long long brow;
    const uint16_t* bank;
    if (G1) {
      const int blk = r >> 5, within = r & 31;
      bank = (blk & 1) ? (is_shared ? g.sb1 : g.b1) : (is_shared ? g.sb0 : g.b0);
      brow = (long long)n0 + (blk >> 1) * 32 + within;
    } else {
      bank = is_shared ? g.sb0 : g.b0;
      brow = (long long)n0 + r;
    }
    const long long e = is_shared ? 0 : s;
    bptr[i] = bank + (e * g.N + brow) * (long long)g.K + lc;
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // K loop: DEPTH register sets keep DEPTH K-steps of global loads in flight; each
  // step goes registers -> LDS -> MFMA.  Weight (B) loads may bypass L2 retention
  // (nontemporal): every weight byte is used by one tile only.
  u32x4_t ra[DEPTH][LA], rb[DEPTH][LB];
  auto gload = [&](u32x4_t(&A)[LA], u32x4_t(&B)[LB], int kofs) {
#pragma unroll
    for (int i = 0; i < LA; ++i) A[i] = *(const u32x4_t*)(aptr[i] + kofs);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      if (NT_B)
        B[i] = __builtin_nontemporal_load((const u32x4_t*)(bptr[i] + kofs));
      else
        B[i] = *(const u32x4_t*)(bptr[i] + kofs);
    }
  };
  auto step = [&](u32x4_t(&A)[LA], u32x4_t(&B)[LB], int knext) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(u32x4_t*)&sA[(lr + RSTEP * i) * LDSS + lc] = A[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(u32x4_t*)&sB[(lr + RSTEP * i) * LDSS + lc] = B[i];
    __syncthreads();
    if (knext < g.K) gload(A, B, knext);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const int kc = kk + (lane >> 5) * 8;
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4_t u = *(const u32x4_t*)&sA[(wm * 64 + mb * 32 + (lane & 31)) * LDSS + kc];
        af[mb] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const u32x4_t u = *(const u32x4_t*)&sB[(wn * 64 + nb * 32 + (lane & 31)) * LDSS + kc];
        bf[nb] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
    __syncthreads();
  };
#pragma unroll
  for (int s2 = 0; s2 < DEPTH; ++s2)
    if (s2 * BK < g.K) gload(ra[s2], rb[s2], s2 * BK);
  for (int k0 = 0; k0 < g.K; k0 += DEPTH * BK) {
#pragma unroll
    for (int s2 = 0; s2 < DEPTH; ++s2)
      if (k0 + s2 * BK < g.K) step(ra[s2], rb[s2], k0 + (s2 + DEPTH) * BK);
  }

  // ---- epilogue.  Accumulator element v of a lane is C[i][j] with
  //      j = lane % 32, i = 8 * (v / 4) + 4 * (lane / 32) + v % 4. ----
  const int j = lane & 31;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int r = wm * 64 + mb * 32 + i;
      if (r >= mrows) continue;
      const long long orow = (long long)row0 + r;
      if (MODE == 0) {
        const float a = acc[mb][0][v], gg = acc[mb][1][v];
        const int col = n0 + wn * 32 + j;
        g.out[orow * g.N + col] = f32_to_bf16(silu_f32(a) * gg);   // 32 features per wave
        if (g.out_pre) {   // saved for the backward pass
          g.out_pre[orow * 2 * g.N + col] = a;
          g.out_pre[orow * 2 * g.N + g.N + col] = gg;
        }
      } else if (MODE == 2) {
        const int col = n0 + wn * 32 + j;
        g.out_pre[orow * 2 * g.N + col] = acc[mb][0][v];
        g.out_pre[orow * 2 * g.N + g.N + col] = acc[mb][1][v];
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + wn * 64 + nb * 32 + j;
          g.out[orow * g.N + col] = f32_to_bf16(acc[mb][nb][v]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 grouped GEMM with a three-stage LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane l of a wavefront writes its 16 bytes at base + 16 l).
// No registers hold data in flight, so two K-steps of loads stay outstanding while a
// third is multiplied.  Same tile order, tile shape (128 x 64 WN), MFMA sequence and
// epilogue as grouped_gemm_bf16_kernel, hence the same bits.
// A stage holds the A tile (128 rows) then the B tile (64 WN rows), 128 bytes per row.
// The sixteen-byte chunk c of row r is stored in slot c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7:
// the 8 (or 16) consecutive rows one ds_read_b128 phase touches then fall in distinct banks.
// Synchronisation per K-step: wait for this wavefront's loads of the step (s_waitcnt
// vmcnt), then s_barrier, so every wavefront's loads of the step have landed and every
// wavefront has finished reading the stage that the next loads overwrite.
// ---------------------------------------------------------------------------
constexpr int kDmaStages = 3;

__device__ __forceinline__ int lds_swz(int r) { return (r ^ (r >> 3)) & 7; }

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MODE, int WN>
__global__ __launch_bounds__(128 * WN) void grouped_gemm_bf16_dma_kernel(GemmArgs g) {
  constexpr int NTHR = 128 * WN, NW = 2 * WN;
  constexpr int BNW = 64 * WN;
  constexpr int LA = BM / (8 * NW), LB = BNW / (8 * NW);   // 1 KB load instructions per wavefront
  constexpr int STAGE = (BM + BNW) * 128;                  // bytes per stage
  static_assert(LA * 8 * NW == BM && LB * 8 * NW == BNW, "loader shape");
  static_assert(kDmaStages * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];

  // ---- tile decode (identical to grouped_gemm_bf16_kernel) ----
  const int total = g.mstart[g.S] * g.NT;
  int tile;
  if (!xcd_tile<0>(total, tile)) return;
  int lo = 0, hi = g.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mstart[mid] * g.NT <= tile) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int mtiles = g.mstart[s + 1] - g.mstart[s];
  const int local = tile - g.mstart[s] * g.NT;
  const int grp = local / (kGroupM * g.NT), rem = local % (kGroupM * g.NT);
  const int gm = min(kGroupM, mtiles - grp * kGroupM);
  const int nt = rem / gm, mt = grp * kGroupM + rem % gm;
  const int row0 = g.rowstart[s] + mt * BM;
  const int mrows = min(BM, g.rowcount[s] - mt * BM);
  const int n0 = nt * (MODE == 0 ? BNW / 2 : BNW);
  const bool is_shared = (s == g.E);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- loader: instruction i of this wavefront fills stage rows 8 (wave LA + i) + lane / 8
  //      (A) or 8 (wave LB + i) + lane / 8 (B), slot lane % 8 <- chunk slot ^ swz(row). ----
  const uint16_t* aptr[LA];
  const uint16_t* bptr[LB];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = 8 * (wave * LA + i) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swz(r);
    const long long j = (long long)row0 + (r < mrows ? r : 0);
    long long src;
    if (MODE == 0) {
      src = is_shared ? j - g.Tk : (long long)(g.perm[j] / g.k);
      if (src < 0 || src >= g.T) {
        bad = 1;
        src = 0;
      }
    } else {
      src = j;
    }
    aptr[i] = g.a + src * (long long)g.K + chunk * 8;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = 8 * (wave * LB + i) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swz(r);
    long long brow;
    const uint16_t* bank;
    if (MODE == 0) {
      const int blk = r >> 5, within = r & 31;
      bank = (blk & 1) ? (is_shared ? g.sb1 : g.b1) : (is_shared ? g.sb0 : g.b0);
      brow = (long long)n0 + (blk >> 1) * 32 + within;
    } else {
      bank = is_shared ? g.sb0 : g.b0;
      brow = (long long)n0 + r;
    }
    const long long e = is_shared ? 0 : s;
    bptr[i] = bank + (e * g.N + brow) * (long long)g.K + chunk * 8;
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue = [&](uint8_t* st, int k0) {
#if defined(__HIP_DEVICE_COMPILE__)   // a gfx950 builtin: device pass only
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds(aptr[i] + k0, (lds_ptr)(st + (wave * LA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      __builtin_amdgcn_global_load_lds(bptr[i] + k0, (lds_ptr)(st + BM * 128 + (wave * LB + i) * 1024), 16,
                                       0, 0);
#endif
  };

  // ---- fragment addresses: lane reads row (block base + lane % 32), chunk 2 kk + lane / 32.
  //      Offsets within a stage, for A blocks [b][kk] and B blocks [b][kk]. ----
  uint32_t aof[2][4], bof[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int ra = wm * 64 + b * 32 + (lane & 31);
    const int rb = wn * 64 + b * 32 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = 2 * kk + (lane >> 5);
      aof[b][kk] = ra * 128 + ((chunk ^ lds_swz(ra)) << 4);
      bof[b][kk] = BM * 128 + rb * 128 + ((chunk ^ lds_swz(rb)) << 4);
    }
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // The fragment reads are issued from inline assembly, each batch ending in its own
  // lgkmcnt(0) wait, so that the compiler does not tie them to the outstanding
  // global->LDS loads of the other stages (it would wait for all of them); the
  // ordering against those loads is the explicit vmcnt wait and barrier of the K loop.
  auto compute = [&](uint32_t st) {
#pragma unroll
    for (int kp = 0; kp < 4; kp += 2) {
      u32x4_t f[8];
      asm volatile(
          "ds_read_b128 %0, %8\n\t"
          "ds_read_b128 %1, %9\n\t"
          "ds_read_b128 %2, %10\n\t"
          "ds_read_b128 %3, %11\n\t"
          "ds_read_b128 %4, %12\n\t"
          "ds_read_b128 %5, %13\n\t"
          "ds_read_b128 %6, %14\n\t"
          "ds_read_b128 %7, %15\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
            "=&v"(f[6]), "=&v"(f[7])
          : "v"(st + aof[0][kp]), "v"(st + aof[1][kp]), "v"(st + bof[0][kp]), "v"(st + bof[1][kp]),
            "v"(st + aof[0][kp + 1]), "v"(st + aof[1][kp + 1]), "v"(st + bof[0][kp + 1]),
            "v"(st + bof[1][kp + 1]));
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, f[4 * h + mb]), __builtin_bit_cast(bf16x8_t, f[4 * h + 2 + nb]),
                acc[mb][nb], 0, 0, 0);
    }
  };

  // ---- K loop over the ring; stage i lives in st[i % 3] ----
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t l0 = (uint32_t)(uintptr_t)(lds_u8*)st0, l1 = (uint32_t)(uintptr_t)(lds_u8*)st1,
                 l2 = (uint32_t)(uintptr_t)(lds_u8*)st2;
  const int nsteps = g.K / BK;
  issue(st0, 0);
  if (nsteps > 1) issue(st1, BK);
  auto kstep = [&](int i, uint32_t cur, uint8_t* nxt) {
    if (i + 1 < nsteps)
      wait_vmcnt<LA + LB>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (i + 2 < nsteps) issue(nxt, (i + 2) * BK);
    compute(cur);
  };
  for (int i = 0; i < nsteps; i += kDmaStages) {
    kstep(i, l0, st2);
    if (i + 1 < nsteps) kstep(i + 1, l1, st0);
    if (i + 2 < nsteps) kstep(i + 2, l2, st1);
  }

  // ---- epilogue (as grouped_gemm_bf16_kernel) ----
  const int j = lane & 31;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int r = wm * 64 + mb * 32 + i;
      if (r >= mrows) continue;
      const long long orow = (long long)row0 + r;
      if (MODE == 0) {
        const int col = n0 + wn * 32 + j;
        g.out[orow * g.N + col] = f32_to_bf16(silu_f32(acc[mb][0][v]) * acc[mb][1][v]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + wn * 64 + nb * 32 + j;
          g.out[orow * g.N + col] = f32_to_bf16(acc[mb][nb][v]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP8 path (OCP MX: E4M3 elements, one E8M0 scale per 32 elements along K) on the
// block-scaled matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4.  Lane l of an operand
// holds row (or column) l % 32; with h = l / 32, its bytes 0..15 are k = 16h..16h+15 of
// the instruction's 64-wide k range and bytes 16..31 are k = 32+16h..32+16h+15, so
// k-block 0 (k < 32) is split over both lane halves, and lane half h supplies the E8M0
// scale of k-block h.
// GEMM1 requantises h = silu(x W1) * (x W3) to MXFP8 row by row (one 32-column block per
// half wavefront) for GEMM2; GEMM2 writes bf16.
// ---------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int MBK = 128;               // reduction step in elements (= bytes)
constexpr int MLDS = MBK + 16;         // LDS row stride in bytes

struct MxArgs {
  const uint8_t* a;          // GEMM1: x codes [T][d]; GEMM2: h codes [rows][I]
  const uint8_t* as;         // matching E8M0 scales [.][K/32]
  const int32_t* perm;
  int T, k, E;
  long long Tk;
  const uint8_t* b0;         // GEMM1: W1 codes; GEMM2: W2 codes
  const uint8_t* b1;         // GEMM1: W3 codes
  const uint8_t* b0s;
  const uint8_t* b1s;
  const uint8_t* sb0;        // shared expert
  const uint8_t* sb1;
  const uint8_t* sb0s;
  const uint8_t* sb1s;
  int K, N, NT;
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  int S;
  void* out;                 // GEMM1: h codes [rows][I]; GEMM2: bf16 [rows][d]
  uint8_t* out_scale;        // GEMM1: h scales [rows][I/32]
  int* flag;
};

// fp32 (already divided by its block scale) -> E4M3 code, round to nearest even,
// saturating to +-448 (NaN -> 0x7F).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a != a) return 0x7Fu;
  if (!(a < 448.0f)) return sign | 0x7Eu;
  const uint32_t ua = __float_as_uint(a);
  if (ua < 0x00800000u) return sign;                 // below 2^-126: rounds to zero
  const int e = (int)(ua >> 23) - 127;
  const uint32_t full = (ua & 0x7FFFFFu) | 0x800000u;
  const int shift = e >= -6 ? 20 : 20 + (-6 - e);
  if (shift > 24) return sign;                       // below 2^-10: rounds to zero
  uint32_t keep = full >> shift;
  const uint32_t rem = full & ((1u << shift) - 1u), half = 1u << (shift - 1);
  keep += (rem > half || (rem == half && (keep & 1u))) ? 1u : 0u;
  if (e >= -6) {
    int ef = e + 7;
    if (keep == 16u) {
      ++ef;
      keep = 8u;
    }
    return sign | ((uint32_t)ef << 3) | (keep - 8u);
  }
  return sign | keep;                                // subnormal grid (keep == 8: 2^-6)
}

// Requantise one row's 32-feature MX block (this value and the 31 other lanes of the
// half wavefront) and store code and scale: OCP MX scale 2^(floor(log2 amax) - 8).
__device__ __forceinline__ void mx_store_h(float h, bool live, uint8_t* code, uint8_t* scale,
                                           bool first) {
  float amax = fabsf(h);
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int se;
  uint32_t scode;
  if (amax == 0.0f) {
    se = -127;
    scode = 0;
  } else if (!(amax <= 3.0e38f)) {
    se = 0;
    scode = 255;
  } else {
    se = min(max(ilogbf(amax) - 8, -127), 127);
    scode = (uint32_t)(se + 127);
  }
  if (live) {
    *code = (uint8_t)e4m3_rne_sat(ldexpf(h, -se));
    if (first) *scale = (uint8_t)scode;
  }
}

// Requantise one MX block (32 consecutive fp32 features of a row, at `src` in LDS, read
// by one lane) and store its 32 codes (two 16-byte stores) and its scale.  Same scale
// rule and encoding as mx_store_h.  Two passes over LDS (the block's amax, then the
// codes) keep few values live.
__device__ __forceinline__ void mx_store_block(const uint8_t* src, uint8_t* code, uint8_t* scale) {
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float4 t = *(const float4*)(src + 16 * c);
    amax = fmaxf(fmaxf(amax, fmaxf(fabsf(t.x), fabsf(t.y))), fmaxf(fabsf(t.z), fabsf(t.w)));
  }
  int se;
  uint32_t scode;
  if (amax == 0.0f) {
    se = -127;
    scode = 0;
  } else if (!(amax <= 3.0e38f)) {
    se = 0;
    scode = 255;
  } else {
    se = min(max(ilogbf(amax) - 8, -127), 127);
    scode = (uint32_t)(se + 127);
  }
  // v_cvt_pk_fp8_f32 rounds to nearest even onto the OCP E4M3 grid; with its input
  // clamped to +-448 it equals e4m3_rne_sat (checked on every rounding boundary of
  // every binade from 2^-20 to 2^10, the subnormal grid, +-0 and the infinities), and
  // NaN is kept as 0x7F explicitly
  u32x4_t w[2];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float4 t = *(const float4*)(src + 16 * c);
    const float v[4] = {ldexpf(t.x, -se), ldexpf(t.y, -se), ldexpf(t.z, -se), ldexpf(t.w, -se)};
    int d = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v[0], -448.0f), 448.0f),
                                            fminf(fmaxf(v[1], -448.0f), 448.0f), 0, false);
    d = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v[2], -448.0f), 448.0f),
                                        fminf(fmaxf(v[3], -448.0f), 448.0f), d, true);
    uint32_t du = (uint32_t)d;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (v[b] != v[b]) du = (du & ~(0xFFu << (8 * b))) | (0x7Fu << (8 * b));
    w[c >> 2][c & 3] = du;
  }
  *(u32x4_t*)code = w[0];
  *(u32x4_t*)(code + 16) = w[1];
  *scale = (uint8_t)scode;
}

// Tile: (64 WM) rows x (32 FN WN) staged B rows, WM x WN wavefronts; each wavefront
// owns 64 rows x 32 FN B rows as 2 x FN MFMA blocks.  K advances 128 bytes a step:
// registers -> LDS (144-byte rows) -> two 64-wide MFMA steps, with the next step's
// loads in flight.  GEMM1 (MODE 0): B rows alternate 32-row blocks of W1 and W3, so a
// wavefront's blocks 2p and 2p + 1 are the W1 and W3 halves of 32 features.
template <int MODE, int WM, int WN, int FN>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(MOE_MX_WAVES)))
void grouped_gemm_mx_kernel(MxArgs g) {
  constexpr int NTHR = 64 * WM * WN;
  constexpr int TM = 64 * WM;                 // tile rows
  constexpr int TB = 32 * FN * WN;            // staged B rows
  constexpr int RSTEP = NTHR / 8;             // loader row stride (8 threads per 128-byte row)
  constexpr int LA = TM / RSTEP, LB = TB / RSTEP;
  static_assert(LA * RSTEP == TM && LB * RSTEP == TB && FN % 2 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t sA[TM * MLDS];
  __shared__ __attribute__((aligned(16))) uint8_t sB[TB * MLDS];
  __shared__ uint32_t sAs[TM];
  __shared__ uint32_t sBs[TB];

  const int total = g.mstart[g.S] * g.NT;
  int tile;
  if (!xcd_tile<0>(total, tile)) return;
  int lo = 0, hi = g.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mstart[mid] * g.NT <= tile) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int mtiles = g.mstart[s + 1] - g.mstart[s];
  const int local = tile - g.mstart[s] * g.NT;
  const int grp = local / (kGroupM * g.NT), rem = local % (kGroupM * g.NT);
  const int gm = min(kGroupM, mtiles - grp * kGroupM);
  const int nt = rem / gm, mt = grp * kGroupM + rem % gm;
  const int row0 = g.rowstart[s] + mt * TM;
  const int mrows = min(TM, g.rowcount[s] - mt * TM);
  const int n0 = nt * (MODE == 0 ? TB / 2 : TB);
  const bool is_shared = (s == g.E);
  const long long e = is_shared ? 0 : s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = tid >> 3, lc = (tid & 7) * 16;     // loader: rows lr + RSTEP i, 16-byte chunk lc
  const int KB = g.K / 32;                           // scale bytes per row

  // source row of A tile row r (rows past the segment re-read the tile's first row)
  auto a_src = [&](int r, int& bad) -> long long {
    const long long jr = (long long)row0 + (r < mrows ? r : 0);
    long long src;
    if (MODE == 0) {
      src = is_shared ? jr - g.Tk : (long long)(g.perm[jr] / g.k);
      if (src < 0 || src >= g.T) {
        bad = 1;
        src = 0;
      }
    } else {
      src = jr;
    }
    return src;
  };
  // row (within expert e's matrix) of staged B row r, with its code and scale banks
  auto b_row = [&](int r, const uint8_t*& bank, const uint8_t*& sbank) -> long long {
    if (MODE == 0) {
      const int blk = r >> 5, within = r & 31;
      const bool w3 = blk & 1;
      bank = w3 ? (is_shared ? g.sb1 : g.b1) : (is_shared ? g.sb0 : g.b0);
      sbank = w3 ? (is_shared ? g.sb1s : g.b1s) : (is_shared ? g.sb0s : g.b0s);
      return (long long)n0 + (blk >> 1) * 32 + within;
    }
    bank = is_shared ? g.sb0 : g.b0;
    sbank = is_shared ? g.sb0s : g.b0s;
    return (long long)n0 + r;
  };

  int bad = 0;
  const uint8_t* aptr[LA];
  const uint8_t* bptr[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) aptr[i] = g.a + a_src(lr + RSTEP * i, bad) * (long long)g.K + lc;
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const uint8_t *bank, *sbank;
    const long long br = b_row(lr + RSTEP * i, bank, sbank);
    bptr[i] = bank + (e * g.N + br) * (long long)g.K + lc;
  }
  // Scale rows: thread t < TM stages A row t's four scale bytes of the step, threads
  // TM .. TM + TB - 1 those of B row t - TM (strided when there are fewer threads).
  constexpr int NS = (TM + TB + NTHR - 1) / NTHR;
  const uint8_t* sptr[NS];
  bool sact[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int sr = tid + NTHR * i;
    sact[i] = sr < TM + TB;
    if (sr < TM) {
      sptr[i] = g.as + a_src(sr, bad) * (long long)KB;
    } else {
      const uint8_t *bank, *sbank;
      const long long br = b_row(sact[i] ? sr - TM : 0, bank, sbank);
      sptr[i] = sbank + (e * g.N + br) * (long long)KB;
    }
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  f32x16_t acc[2][FN];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  u32x4_t ra[LA], rb[LB];
  uint32_t rs[NS];
#pragma unroll
  for (int i = 0; i < LA; ++i) ra[i] = *(const u32x4_t*)(aptr[i]);
#pragma unroll
  for (int i = 0; i < LB; ++i) rb[i] = *(const u32x4_t*)(bptr[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) rs[i] = sact[i] ? *(const uint32_t*)(sptr[i]) : 0u;

  for (int k0 = 0; k0 < g.K; k0 += MBK) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(u32x4_t*)&sA[(lr + RSTEP * i) * MLDS + lc] = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(u32x4_t*)&sB[(lr + RSTEP * i) * MLDS + lc] = rb[i];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int sr = tid + NTHR * i;
      if (sr < TM) sAs[sr] = rs[i];
      else if (sact[i]) sBs[sr - TM] = rs[i];
    }
    __syncthreads();
    const int kn = k0 + MBK;
    if (kn < g.K) {
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *(const u32x4_t*)(aptr[i] + kn);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = *(const u32x4_t*)(bptr[i] + kn);
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (sact[i]) rs[i] = *(const uint32_t*)(sptr[i] + kn / 32);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kc = sub * 64 + (lane >> 5) * 16;       // bytes 0..15; bytes 16..31 at kc + 32
      const int sh = 8 * (sub * 2 + (lane >> 5));       // scale byte of k-block (2 sub + half)
      i32x8_t af[2], bf[FN];
      int sa[2], sb[FN];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + (lane & 31);
        const u32x4_t u0 = *(const u32x4_t*)&sA[row * MLDS + kc];
        const u32x4_t u1 = *(const u32x4_t*)&sA[row * MLDS + kc + 32];
        af[mb] = (i32x8_t){(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                           (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
        sa[mb] = (int)((sAs[row] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int nb = 0; nb < FN; ++nb) {
        const int row = (wn * FN + nb) * 32 + (lane & 31);
        const u32x4_t u0 = *(const u32x4_t*)&sB[row * MLDS + kc];
        const u32x4_t u1 = *(const u32x4_t*)&sB[row * MLDS + kc + 32];
        bf[nb] = (i32x8_t){(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                           (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
        sb[nb] = (int)((sBs[row] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < FN; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[mb], bf[nb], acc[mb][nb], 0, 0, 0, sa[mb], 0, sb[nb]);
    }
    __syncthreads();
  }

  // ---- epilogue.  Accumulator element v of a lane is C[i][j], j = lane % 32,
  //      i = 8 (v / 4) + 4 (lane / 32) + v % 4. ----
  const int j = lane & 31;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int r = wm * 64 + mb * 32 + i;
      const long long orow = (long long)row0 + r;
      if (MODE == 0) {
        // One MX block = this row's 32 features, spread over the 32 lanes of a half.
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
          const float hv = silu_f32(acc[mb][2 * p][v]) * acc[mb][2 * p + 1][v];
          const int col = n0 + (wn * FN / 2 + p) * 32 + j;
          mx_store_h(hv, r < mrows, (uint8_t*)g.out + orow * g.N + col,
                     g.out_scale + orow * (g.N / 32) + col / 32, j == 0);
        }
      } else {
        if (r < mrows) {
#pragma unroll
          for (int nb = 0; nb < FN; ++nb) {
            const int col = n0 + (wn * FN + nb) * 32 + j;
            ((uint16_t*)g.out)[orow * g.N + col] = f32_to_bf16(acc[mb][nb][v]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP8 grouped GEMM on a four-stage LDS ring (the path for shapes it tiles: N of
// GEMM2 a multiple of 256).  Tiles are 256 rows x 256 staged B rows; K advances 64
// bytes (one MFMA k range) a step.  Eight wavefronts, 2 along M x 4 along N, each own
// 128 rows x 64 B rows as 4 x 2 MFMA blocks, two wavefronts per SIMD.
// Loads go straight from global memory into LDS (global_load_lds_dwordx4: lane l of a
// wavefront writes its 16 bytes at base + 16 l), three steps ahead of the step being
// multiplied.  A stage holds the A tile (256 rows x 64 B) and the B tile (256 x 64 B).
// E8M0 scales travel in groups of 16 bytes per row (512 K, eight steps), into one of two
// scale buffers, issued eight steps before their first use: a per-step scale load
// would cost one memory request per row for 2 bytes.
// The 16-byte chunk c of a row r is stored in slot c ^ ((r >> 2) & 3), so the sixteen
// rows that one ds_read_b128 phase touches fall in distinct banks.
// Row blocks past the tile's valid rows are not multiplied (a wavefront skips its
// 32-row blocks that hold no valid row), so a short tile costs MFMA time in
// proportion to its 32-row blocks.  Every output is the same MFMA chain as in
// grouped_gemm_mx_kernel (K ascending in 64-wide scaled MFMAs from zero), hence the
// same bits.
// The loads are issued from inline assembly: the compiler then treats the fragment
// reads as ordinary LDS loads (it does not wait for the ring's outstanding loads before
// each of them), and the K loop orders them itself with an explicit vmcnt wait and
// s_barrier per step.  No other global load is in flight inside the K loop.
// ---------------------------------------------------------------------------
constexpr int XR_M = 256;                        // tile rows
constexpr int XR_N = 256;                        // staged B rows
constexpr int XR_K = 128;                        // K bytes per ring step (two MFMA k ranges)
constexpr int XR_ST = 2;                         // ring stages
constexpr int XR_A = 0, XR_B = XR_M * XR_K;      // tile offsets within a stage
constexpr int XR_STAGE = (XR_M + XR_N) * XR_K;   // 64 KB
constexpr int XR_GS = 4;                         // steps per scale group (16 E8M0 bytes per row)
constexpr int XR_GB = XR_GS * XR_K;              // K per scale group
constexpr int XR_SC = XR_ST * XR_STAGE;          // two scale-group buffers after the stages
constexpr int XR_SCB = (XR_M + XR_N) * 16;       // bytes per scale-group buffer (A rows, then B)
constexpr int XR_LDS = XR_SC + 2 * XR_SCB;       // 144 KB
constexpr int XR_EPI_ROW = 144;                  // epilogue staging: bytes per local row
constexpr int XR_EPI = 128 * XR_EPI_ROW;         // epilogue staging per wavefront (18 KB)
static_assert(XR_LDS <= 160 * 1024 && 8 * XR_EPI <= XR_LDS, "LDS budget");

// slot of the 16-byte chunk c of row r: c ^ ((r >> 1) & 7); the sixteen rows that one
// ds_read_b128 phase touches (one chunk each) then fall in distinct banks
__device__ __forceinline__ int xr_swz(int r) { return (r >> 1) & 7; }

// global_load_lds_dwordx4 (lane l writes its 16 bytes at lds + 16 l) from a
// wavefront-uniform base plus a 32-bit per-lane offset, or from a per-lane address
__device__ __forceinline__ void xr_load16(uint32_t lds, uint32_t off, const void* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory");
}
__device__ __forceinline__ void xr_load16(uint32_t lds, const void* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory");
}
// Wait until at most N ring loads of this wavefront are outstanding and every LDS
// access of this wavefront has completed, then meet the other wavefronts.
template <int N>
__device__ __forceinline__ void xr_sync() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One 64-wide k range of fragments: NB of the wavefront's 4 row blocks, 2 B blocks.
template <int NB>
struct XrFrag {
  i32x8_t a[NB > 0 ? NB : 1], b[2];
};
// The E8M0 scales of one step for a lane: word w of a block holds, from its low byte, the
// scales of k-blocks 4 (j % 4) + lane / 32 + 0, 1, 2, ... of the row, so the first k range
// takes byte 0 (MFMA op_sel 0) and the second byte 2 (op_sel 2).
template <int NB>
struct XrScale {
  int a[NB > 0 ? NB : 1], b[2];
};

// Read k range `half` (0 or 1) of the stage at st.  aof/bof: this lane's chunk of k
// range 0 (k range 1 is XOR 64, the second 16 bytes XOR 32).
template <int NB>
__device__ __forceinline__ void xr_read(XrFrag<NB>& f, const uint8_t* st, uint32_t aof, uint32_t bof,
                                        int half) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint32_t o = (bof ^ (64 * half)) + nb * 32 * XR_K;
    const u32x4_t lo = *(const u32x4_t*)(st + o);
    const u32x4_t hi = *(const u32x4_t*)(st + (o ^ 32));
    f.b[nb] = (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    const uint32_t o = (aof ^ (64 * half)) + mb * 32 * XR_K;
    const u32x4_t lo = *(const u32x4_t*)(st + o);
    const u32x4_t hi = *(const u32x4_t*)(st + (o ^ 32));
    f.a[mb] = (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}
// asf/bsf: this lane's row's 16-byte scale group in the scale buffer scb; sc: the step's
// first k-block within the group (a multiple of 4); sh = 8 (lane / 32).
template <int NB>
__device__ __forceinline__ void xr_read_scales(XrScale<NB>& sc4, const uint8_t* scb, uint32_t asf,
                                               uint32_t bsf, int sc, int sh) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) sc4.b[nb] = (int)(*(const uint32_t*)(scb + bsf + nb * 32 * 16 + sc) >> sh);
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
    sc4.a[mb] = (int)(*(const uint32_t*)(scb + asf + mb * 32 * 16 + sc) >> sh);
}

// An empty asm that reads every accumulator: the MFMAs before it are issued before the
// ring loads and barriers that follow it in program order (the compiler would otherwise
// sink them next to their next use).
__device__ __forceinline__ void xr_pin(const f32x16_t (&acc)[4][2]) {
  asm volatile("" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[1][0]), "a"(acc[1][1]), "a"(acc[2][0]),
               "a"(acc[2][1]), "a"(acc[3][0]), "a"(acc[3][1]));
}

template <int NB, int SEL>
__device__ __forceinline__ void xr_mfma(const XrFrag<NB>& f, const XrScale<NB>& sc4, f32x16_t (&acc)[4][2]) {
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[mb], f.b[nb], acc[mb][nb], 0, 0, SEL,
                                                                   sc4.a[mb], SEL, sc4.b[nb]);
}

// Load sources: A rows at abase + aoff[i] (wavefront-uniform base, per-lane offset), B
// rows at bbase + boff[i], scale groups at sbase + soff (A rows, waves 0..3) or at the
// per-lane bsp (B rows, waves 4..7).
struct XrSrc {
  const uint8_t* abase;
  const uint8_t* bbase;
  const uint8_t* sbase;
  const uint8_t* bsp;
  uint32_t aoff[4], boff[4], soff;
};

// The K loop of a wavefront that multiplies NB of its 4 row blocks (NB = 0: it only
// loads and synchronises).  Step j (K bytes 128 j .. 128 j + 127) lives in stage j % 2.
// At step j: wait for its data, meet (every wavefront is then done with step j - 1, whose
// stage takes step j + 1's loads), multiply.  Scale group g (steps 4 g .. 4 g + 3) goes
// out at step 4 (g - 1), after that step's data, into buffer g % 2.
template <int NB>
__device__ __forceinline__ void xr_kloop(const uint8_t* ring, uint32_t ring_lds, int nsteps, const XrSrc& src,
                                         int wave, uint32_t aof, uint32_t bof, uint32_t asf, uint32_t bsf,
                                         int sh, f32x16_t (&acc)[4][2]) {
  const uint32_t la = XR_A + wave * 4096, lb = XR_B + wave * 4096;
  const uint32_t ls = wave < 4 ? wave * 1024 : XR_M * 16 + (wave - 4) * 1024;
  const int ngroups = nsteps / XR_GS;
  auto issue = [&](int j) {
    const uint32_t st = ring_lds + (uint32_t)(j & 1) * XR_STAGE;
    const int k0 = j * XR_K;
#pragma unroll
    for (int i = 0; i < 4; ++i) xr_load16(st + la + 1024 * i, src.aoff[i], src.abase + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) xr_load16(st + lb + 1024 * i, src.boff[i], src.bbase + k0);
  };
  auto issue_scales = [&](int grp) {
    const uint32_t dst = ring_lds + XR_SC + (uint32_t)(grp & 1) * XR_SCB + ls;
    if (wave < 4)
      xr_load16(dst, src.soff, src.sbase + 16 * grp);
    else
      xr_load16(dst, src.bsp + 16 * grp);
  };
  auto scales_at = [&](int j) { return j >= 0 && j % XR_GS == 0 && j / XR_GS + 1 < ngroups; };

  issue_scales(0);
  issue(0);
  for (int j = 0; j < nsteps; ++j) {
    // step j's data went out at step j - 1 (or before the loop), followed only by that
    // step's scale group (loads complete in issue order)
    if (scales_at(j - 1))
      xr_sync<1>();
    else
      xr_sync<0>();
    if (j + 1 < nsteps) issue(j + 1);
    if (scales_at(j)) issue_scales(j / XR_GS + 1);
    if constexpr (NB > 0) {
      const uint8_t* st = ring + (j & 1) * XR_STAGE;
      const uint8_t* scb = ring + XR_SC + ((j / XR_GS) & 1) * XR_SCB;
      XrScale<NB> sc4;
      xr_read_scales<NB>(sc4, scb, asf, bsf, (j % XR_GS) * (XR_K / 32), sh);
      XrFrag<NB> f;
      xr_read<NB>(f, st, aof, bof, 0);
      xr_mfma<NB, 0>(f, sc4, acc);
      xr_read<NB>(f, st, aof, bof, 1);
      xr_mfma<NB, 2>(f, sc4, acc);
      xr_pin(acc);
    }
  }
}

// MXFP8 grouped GEMM, 256 x 256 tiles, eight wavefronts (2 along M x 4 along N, two per
// SIMD), each 4 row blocks x 2 B blocks of 32 x 32.  A wavefront whose 32-row blocks
// hold no valid row skips their MFMAs, so a short tile costs MFMA time in proportion to
// its valid 32-row blocks on the busier half.
template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_mx_ring_kernel(MxArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[XR_LDS];

  // ---- tile decode (as grouped_gemm_mx_kernel, tiles of XR_M rows) ----
  const int total = g.mstart[g.S] * g.NT;
  int tile;
  if (!xcd_tile<kMxXcdChunk>(total, tile)) return;
  int lo = 0, hi = g.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mstart[mid] * g.NT <= tile) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int mtiles = g.mstart[s + 1] - g.mstart[s];
  const int local = tile - g.mstart[s] * g.NT;
  const int grp = local / (kGroupM * g.NT), rem = local % (kGroupM * g.NT);
  const int gm = min(kGroupM, mtiles - grp * kGroupM);
  const int nt = rem / gm, mt = grp * kGroupM + rem % gm;
  const int row0 = g.rowstart[s] + mt * XR_M;
  const int mrows = min(XR_M, g.rowcount[s] - mt * XR_M);
  const int n0 = nt * (MODE == 0 ? XR_N / 2 : XR_N);
  const bool is_shared = (s == g.E);
  const long long e = is_shared ? 0 : s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int KB = g.K / 32;   // scale bytes per row

  int bad = 0;
  // source row of A tile row r (rows past the segment re-read the tile's first row)
  auto a_src = [&](int r) -> long long {
    const long long jr = (long long)row0 + (r < mrows ? r : 0);
    if (MODE != 0) return jr;
    long long src = is_shared ? jr - g.Tk : (long long)(g.perm[jr] / g.k);
    if (src < 0 || src >= g.T) {
      bad = 1;
      src = 0;
    }
    return src;
  };
  // row (within expert e's matrix) of staged B row r; GEMM1 alternates 32-row blocks of
  // W1 and W3 for the same 32 features
  auto b_row = [&](int r, const uint8_t*& bank, const uint8_t*& sbank) -> long long {
    if (MODE == 0) {
      const int blk = r >> 5;
      const bool w3 = blk & 1;
      bank = w3 ? (is_shared ? g.sb1 : g.b1) : (is_shared ? g.sb0 : g.b0);
      sbank = w3 ? (is_shared ? g.sb1s : g.b1s) : (is_shared ? g.sb0s : g.b0s);
      return (long long)n0 + (blk >> 1) * 32 + (r & 31);
    }
    bank = is_shared ? g.sb0 : g.b0;
    sbank = is_shared ? g.sb0s : g.b0s;
    return (long long)n0 + r;
  };

  // ---- loader: wavefront w fills A rows and B rows 32 w .. 32 w + 31 (four loads of 8
  //      rows each; lane l -> row + l / 8, slot l % 8 <- chunk slot ^ swz(row); the B rows
  //      are one 32-row block, so one bank) and the 16-byte scale groups of A rows
  //      64 w + l (w < 4) or B rows 64 (w - 4) + l.  Every byte offset from a load's base
  //      fits 32 bits (one activation matrix, or one expert's matrix). ----
  XrSrc src;
  src.abase = g.a;
  src.sbase = g.as;
  {
    const uint8_t *bank, *sbank;
    b_row(32 * wave, bank, sbank);
    src.bbase = bank + e * g.N * (long long)g.K;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ xr_swz(r);
    src.aoff[i] = (uint32_t)(a_src(r) * g.K + 16 * chunk);
    const uint8_t *bank, *sbank;
    const long long br = b_row(r, bank, sbank);
    src.boff[i] = (uint32_t)(br * g.K + 16 * chunk);
  }
  src.soff = (uint32_t)(a_src(64 * (wave & 3) + lane) * KB);
  {
    const uint8_t *bank, *sbank;   // GEMM1: W1 scales for lanes 0..31, W3 for 32..63
    const long long br = b_row(64 * (wave & 3) + lane, bank, sbank);
    src.bsp = sbank + (e * g.N + br) * (long long)KB;
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  // ---- fragment offsets within a stage: lane reads row (block base + lane % 32),
  //      chunks lane / 32 and 2 + lane / 32 of the k range ----
  const int j32 = lane & 31, hh = lane >> 5;
  const int ra = 128 * wm + j32, rb = 64 * wn + j32;
  const uint32_t aof = XR_A + ra * XR_K + 16 * (hh ^ xr_swz(ra));
  const uint32_t bof = XR_B + rb * XR_K + 16 * (hh ^ xr_swz(rb));
  const uint32_t asf = ra * 16, bsf = XR_M * 16 + rb * 16;   // within a scale buffer
  const int sh = 8 * hh;

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8*)ring;
  const int nsteps = g.K / XR_K;
  // 32-row blocks of this wavefront that hold a valid row (uniform per wavefront)
  const int nb_act = min(4, max(0, (mrows - wm * 128 + 31) >> 5));
  switch (nb_act) {
    case 4: xr_kloop<4>(ring, ring_lds, nsteps, src, wave, aof, bof, asf, bsf, sh, acc); break;
    case 3: xr_kloop<3>(ring, ring_lds, nsteps, src, wave, aof, bof, asf, bsf, sh, acc); break;
    case 2: xr_kloop<2>(ring, ring_lds, nsteps, src, wave, aof, bof, asf, bsf, sh, acc); break;
    case 1: xr_kloop<1>(ring, ring_lds, nsteps, src, wave, aof, bof, asf, bsf, sh, acc); break;
    default: xr_kloop<0>(ring, ring_lds, nsteps, src, wave, aof, bof, asf, bsf, sh, acc); break;
  }

  // ---- epilogue through LDS: each wavefront stages its 128 x (32 or 64) outputs
  //      row-major in its own 18 KB of the (now idle) ring, then writes whole MX blocks
  //      (GEMM1) or 16-byte row chunks (GEMM2).  Accumulator element v of a lane is
  //      C[i][j], j = lane % 32, i = 8 (v / 4) + 4 (lane / 32) + v % 4; the wavefront's
  //      local row 32 mb + i is tile row 128 wm + 32 mb + i. ----
  __syncthreads();   // every wavefront is done reading the ring
  uint8_t* stg = ring + wave * XR_EPI;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb >= nb_act) break;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (MODE == 0) {
        // B blocks 0 and 1 are the W1 and W3 halves of the same 32 features
        *(float*)(stg + rl * XR_EPI_ROW + j32 * 4) = silu_f32(acc[mb][0][v]) * acc[mb][1][v];
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          *(uint16_t*)(stg + rl * XR_EPI_ROW + (32 * nb + j32) * 2) = f32_to_bf16(acc[mb][nb][v]);
      }
    }
  }
  // (a wavefront reads back only what it wrote: its LDS accesses complete in order)
  if (MODE == 0) {
    // lane l: local rows l and 64 + l, one MX block (the wavefront's 32 features) each
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int rl = 64 * q2 + lane;
      const int r = 128 * wm + rl;
      if ((rl >> 5) < nb_act && r < mrows) {
        const long long orow = (long long)row0 + r;
        const int col = n0 + 32 * wn;
        mx_store_block(stg + rl * XR_EPI_ROW, (uint8_t*)g.out + orow * g.N + col,
                       g.out_scale + orow * (g.N / 32) + col / 32);
      }
    }
  } else {
    // lane l: local row 8 q + l / 8, 16-byte chunk l % 8 of the row's 64 outputs
    const int c = lane & 7;
#pragma unroll 4
    for (int q2 = 0; q2 < 16; ++q2) {
      const int rl = 8 * q2 + (lane >> 3);
      const int r = 128 * wm + rl;
      if ((rl >> 5) < nb_act && r < mrows) {
        const u32x4_t t = *(const u32x4_t*)(stg + rl * XR_EPI_ROW + 16 * c);
        *(u32x4_t*)((uint16_t*)g.out + ((long long)row0 + r) * g.N + n0 + wn * 64 + 8 * c) = t;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// fp32 path (MOE_F32): one thread per output element, fp32 fma in ascending order.
// ---------------------------------------------------------------------------
struct F32Args {
  const float* a;
  const int32_t* perm;
  int T, k, E;
  long long Tk, rows;
  const float* b0;
  const float* b1;
  const float* sb0;
  const float* sb1;
  int K, N;
  const int* rowstart;
  const int* rowcount;
  int S;
  float* out;
  int* flag;
};

template <int MODE>
__global__ __launch_bounds__(256) void grouped_ffn_f32_kernel(F32Args g) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long j = idx / g.N;
  const int n = (int)(idx % g.N);
  if (j >= g.rows) return;
  int lo = 0, hi = g.S;   // largest s with rowstart[s] <= j
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.rowstart[mid] <= j) lo = mid; else hi = mid;
  }
  const int s = lo;
  if (j >= (long long)g.rowstart[s] + g.rowcount[s]) return;   // only with corrupt offsets
  const bool is_shared = (s == g.E);
  const long long e = is_shared ? 0 : s;
  if (MODE == 0) {
    long long tok = is_shared ? j - g.Tk : g.perm[j] / g.k;
    if (tok < 0 || tok >= g.T) {
      raise_flag(g.flag, kFlagCorrupt);
      tok = 0;
    }
    const float* xr = g.a + tok * g.K;
    const float* w1 = (is_shared ? g.sb0 : g.b0) + (e * g.N + n) * (long long)g.K;
    const float* w3 = (is_shared ? g.sb1 : g.b1) + (e * g.N + n) * (long long)g.K;
    float a = 0.0f, gg = 0.0f;
    for (int i = 0; i < g.K; ++i) {
      a = fmaf(xr[i], w1[i], a);
      gg = fmaf(xr[i], w3[i], gg);
    }
    g.out[j * g.N + n] = silu_f32(a) * gg;
  } else {
    const float* hr = g.a + j * g.K;
    const float* w2 = (is_shared ? g.sb0 : g.b0) + (e * g.N + n) * (long long)g.K;
    float o = 0.0f;
    for (int i = 0; i < g.K; ++i) o = fmaf(hr[i], w2[i], o);
    g.out[j * g.N + n] = o;
  }
}

static bool bank_ok(const moe_expert_bank* b, int dtype) {
  if (!b || !b->w1 || !b->w3 || !b->w2) return false;
  if (dtype == MOE_NVFP4)
    return b->w1_scale && b->w3_scale && b->w2_scale && b->w1_rscale && b->w3_rscale && b->w2_rscale &&
           aligned(b->w1, 16) && aligned(b->w3, 16) && aligned(b->w2, 16) && aligned(b->w1_scale, 4) &&
           aligned(b->w3_scale, 4) && aligned(b->w2_scale, 4) && aligned(b->w1_rscale, 4) &&
           aligned(b->w3_rscale, 4) && aligned(b->w2_rscale, 4);
  if (b->w1_rscale || b->w3_rscale || b->w2_rscale) return false;
  if (dtype == MOE_MXFP8) return b->w1_scale && b->w3_scale && b->w2_scale;
  if (b->w1_scale || b->w3_scale || b->w2_scale) return false;
  if (dtype == MOE_BF16)
    return aligned(b->w1, 16) && aligned(b->w3, 16) && aligned(b->w2, 16);
  return true;
}

static bool mx_bank_aligned(const moe_expert_bank* b) {
  return aligned(b->w1, 16) && aligned(b->w3, 16) && aligned(b->w2, 16) && aligned(b->w1_scale, 4) &&
         aligned(b->w3_scale, 4) && aligned(b->w2_scale, 4);
}

// Checks shared by the three FFN entry points (everything but the per-half pointers).
static moe_status check_ffn_shape(int dtype, int T, int d, int E, int k, int inter,
                                  const moe_expert_bank* routed, const moe_expert_bank* shared,
                                  const void* ws, size_t ws_bytes) {
  if (!valid_layer_dtype(dtype) || T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E ||
      k > kMaxTopK || inter < 1)
    return MOE_ERR_INVALID_ARG;
  if (!bank_ok(routed, dtype) || (shared && !bank_ok(shared, dtype))) return MOE_ERR_INVALID_ARG;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_NVFP4 && (d % 256 != 0 || inter % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16 && (d % 128 != 0 || inter % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_MXFP8 && (d % 128 != 0 || inter % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ffn_ws(T, d, E, k, inter, dtype).bytes) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

struct FfnPlan {
  int* flag;
  int* mstart;
  int* rowstart;
  int* rowcount;
  void* h;
  uint8_t* hs;
  uint8_t *xc, *xs, *hc, *hsc;   // NVFP4 quantized x and h
  float *xr, *hr;
  int S, has_shared;
  long long Tk, rows, mt_bound;
  int tm;   // rows per GEMM tile (the segment table counts tiles of this height)
  bool mx_ring;   // MXFP8 on grouped_gemm_mx_ring_kernel (both GEMMs)
};

static FfnPlan plan_of(void* ws, int T, int d, int E, int k, int inter, int dtype, bool has_shared) {
  const FfnWs L = ffn_ws(T, d, E, k, inter, dtype);
  char* w = (char*)ws;
  FfnPlan p;
  p.flag = (int*)w;
  p.mstart = (int*)(w + L.seg);
  p.rowstart = p.mstart + (E + 2);
  p.rowcount = p.rowstart + (E + 2);
  p.h = w + L.h;
  p.hs = (uint8_t*)(w + L.hs);
  p.xc = (uint8_t*)(w + L.xc);
  p.xs = (uint8_t*)(w + L.xs);
  p.xr = (float*)(w + L.xr);
  p.hc = (uint8_t*)(w + L.hc);
  p.hsc = (uint8_t*)(w + L.hsc);
  p.hr = (float*)(w + L.hr);
  p.has_shared = has_shared ? 1 : 0;
  p.S = E + p.has_shared;
  p.Tk = (long long)T * k;
  p.rows = p.Tk + (has_shared ? T : 0);
  // the ring tiles GEMM2's output by XR_N columns and loads scales 16 bytes (512 K) at a time
  p.mx_ring = MOE_MX_RING && dtype == MOE_MXFP8 && d % XR_N == 0 && d % XR_GB == 0 &&
              inter % XR_GB == 0;
  p.tm = p.mx_ring ? XR_M : dtype == MOE_MXFP8 ? 64 * MOE_MX_WM : BM;   // NVFP4: BM as bf16
  p.mt_bound = (p.Tk + (long long)E * (p.tm - 1)) / p.tm + (has_shared ? (T + p.tm - 1) / p.tm : 0);
  return p;
}

// Widest wavefront count along N (from {max_wn, ..., 2}) whose tile width
// (per_wave * wn output features) divides n.  The host checks guarantee wn = 2 divides.
static int bf16_wn(int n, int per_wave, int max_wn) {
  for (int wn = max_wn; wn > 2; wn >>= 1)
    if (n % (per_wave * wn) == 0) return wn;
  return 2;
}

template <int MODE>
static void launch_bf16(int wn, unsigned grid, hipStream_t s, const GemmArgs& g) {
#if MOE_GEMM_DMA
  if (wn == 4) {
    grouped_gemm_bf16_dma_kernel<MODE, 4><<<grid, 512, 0, s>>>(g);
    return;
  }
#endif
  switch (wn) {
#if MOE_GEMM1_WN >= 8 || MOE_GEMM2_WN >= 8
    case 8:
      grouped_gemm_bf16_kernel<MODE, kGemmDepth, kGemmNtB, 8><<<grid, 1024, 0, s>>>(g);
      break;
#endif
#if MOE_GEMM1_WN >= 4 || MOE_GEMM2_WN >= 4
    case 4:
      grouped_gemm_bf16_kernel<MODE, kGemmDepth, kGemmNtB, 4><<<grid, 512, 0, s>>>(g);
      break;
#endif
    default:
      grouped_gemm_bf16_kernel<MODE, kGemmDepth, kGemmNtB, 2><<<grid, 256, 0, s>>>(g);
  }
}

// GEMM1 half: segment table, then h = silu(x W1) * (x W3) for every dispatched row.
static moe_status run_gate_up(const void* x, const uint8_t* xs, int dtype, int T, int d, int E,
                              int k, int inter, const moe_expert_bank* routed,
                              const moe_expert_bank* shared, const int32_t* offsets,
                              const int32_t* perm, const FfnPlan& p, hipStream_t s,
                              float* pre = nullptr) {
  seg_table_kernel<<<1, 1024, 0, s>>>(offsets, E, p.Tk, T, p.has_shared, p.tm, p.mstart, p.rowstart,
                                      p.rowcount, p.flag);
  if (dtype == MOE_NVFP4) {
    moe_status st = nvfp4_quantize_rows((const uint16_t*)x, T, d, nullptr, nullptr, p.xr, (uint16_t*)p.xc, s);
    if (st != MOE_OK) return st;
    Nvfp4Gemm q{};
    q.a = (const uint16_t*)p.xc;
    q.ar = p.xr;
    q.perm = perm;
    q.T = T;
    q.k = k;
    q.E = E;
    q.b0 = (const uint8_t*)routed->w1;
    q.b1 = (const uint8_t*)routed->w3;
    q.b0s = routed->w1_scale;
    q.b1s = routed->w3_scale;
    q.b0r = routed->w1_rscale;
    q.b1r = routed->w3_rscale;
    if (shared) {
      q.sb0 = (const uint8_t*)shared->w1;
      q.sb1 = (const uint8_t*)shared->w3;
      q.sb0s = shared->w1_scale;
      q.sb1s = shared->w3_scale;
      q.sb0r = shared->w1_rscale;
      q.sb1r = shared->w3_rscale;
    }
    q.K = d;
    q.N = inter;
    q.mstart = p.mstart;
    q.rowstart = p.rowstart;
    q.rowcount = p.rowcount;
    q.S = p.S;
    q.mt_bound = p.mt_bound;
    q.out = (uint16_t*)p.h;
    q.flag = p.flag;
    return nvfp4_gemm(0, q, s);   // h (bf16) is quantized by the GEMM2 half
  }
  if (dtype == MOE_MXFP8) {
    MxArgs g{};
    g.a = (const uint8_t*)x;
    g.as = xs;
    g.perm = perm;
    g.T = T;
    g.k = k;
    g.E = E;
    g.Tk = p.Tk;
    g.b0 = (const uint8_t*)routed->w1;
    g.b1 = (const uint8_t*)routed->w3;
    g.b0s = routed->w1_scale;
    g.b1s = routed->w3_scale;
    g.sb0 = shared ? (const uint8_t*)shared->w1 : nullptr;
    g.sb1 = shared ? (const uint8_t*)shared->w3 : nullptr;
    g.sb0s = shared ? shared->w1_scale : nullptr;
    g.sb1s = shared ? shared->w3_scale : nullptr;
    g.K = d;
    g.N = inter;
    g.NT = p.mx_ring ? inter / (XR_N / 2) : inter / (16 * MOE_MX_FN * MOE_MX_WN);
    g.mstart = p.mstart;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = p.h;
    g.out_scale = p.hs;
    g.flag = p.flag;
    const long long grid = tile_grid(p.mt_bound * g.NT, p.mx_ring ? kMxXcdChunk : 0);
    if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    if (p.mx_ring)
      grouped_gemm_mx_ring_kernel<0><<<(unsigned)grid, 512, 0, s>>>(g);
    else
      grouped_gemm_mx_kernel<0, MOE_MX_WM, MOE_MX_WN, MOE_MX_FN>
          <<<(unsigned)grid, 64 * MOE_MX_WM * MOE_MX_WN, 0, s>>>(g);
  } else if (dtype == MOE_BF16) {
    GemmArgs g{};
    g.a = (const uint16_t*)x;
    g.perm = perm;
    g.T = T;
    g.k = k;
    g.E = E;
    g.Tk = p.Tk;
    g.b0 = (const uint16_t*)routed->w1;
    g.b1 = (const uint16_t*)routed->w3;
    g.sb0 = shared ? (const uint16_t*)shared->w1 : nullptr;
    g.sb1 = shared ? (const uint16_t*)shared->w3 : nullptr;
    g.K = d;
    g.N = inter;
    g.NT = inter / 64;
    g.mstart = p.mstart;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = (uint16_t*)p.h;
    g.out_pre = pre;
    g.flag = p.flag;
    const int wn = bf16_wn(inter, 32, MOE_GEMM1_WN);
    g.NT = inter / (32 * wn);
    const long long grid = tile_grid(p.mt_bound * g.NT, 0);
    if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    launch_bf16<0>(wn, (unsigned)grid, s, g);
  } else {
    F32Args g{};
    g.a = (const float*)x;
    g.perm = perm;
    g.T = T;
    g.k = k;
    g.E = E;
    g.Tk = p.Tk;
    g.rows = p.rows;
    g.b0 = (const float*)routed->w1;
    g.b1 = (const float*)routed->w3;
    g.sb0 = shared ? (const float*)shared->w1 : nullptr;
    g.sb1 = shared ? (const float*)shared->w3 : nullptr;
    g.K = d;
    g.N = inter;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = (float*)p.h;
    g.flag = p.flag;
    const long long n = p.rows * inter;
    grouped_ffn_f32_kernel<0><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(g);
  }
  return launch_status();
}

// GEMM2 half: out = h W2 for every dispatched row (h and the segment table from the
// workspace, as left by the GEMM1 half).
static moe_status run_down(int dtype, int T, int d, int E, int k, int inter,
                           const moe_expert_bank* routed, const moe_expert_bank* shared, void* out,
                           const FfnPlan& p, hipStream_t s) {
  if (dtype == MOE_NVFP4) {
    // h per row to NVFP4 (decoded values and row scales) for the second GEMM
    const moe_status st =
        nvfp4_quantize_rows((const uint16_t*)p.h, p.rows, inter, nullptr, nullptr, p.hr, (uint16_t*)p.hc, s);
    if (st != MOE_OK) return st;
    Nvfp4Gemm q{};
    q.a = (const uint16_t*)p.hc;
    q.ar = p.hr;
    q.perm = nullptr;
    q.T = T;
    q.k = k;
    q.E = E;
    q.b0 = (const uint8_t*)routed->w2;
    q.b0s = routed->w2_scale;
    q.b0r = routed->w2_rscale;
    if (shared) {
      q.sb0 = (const uint8_t*)shared->w2;
      q.sb0s = shared->w2_scale;
      q.sb0r = shared->w2_rscale;
    }
    q.K = inter;
    q.N = d;
    q.mstart = p.mstart;
    q.rowstart = p.rowstart;
    q.rowcount = p.rowcount;
    q.S = p.S;
    q.mt_bound = p.mt_bound;
    q.out = (uint16_t*)out;
    q.flag = p.flag;
    return nvfp4_gemm(1, q, s);
  }
  if (dtype == MOE_MXFP8) {
    MxArgs g{};
    g.a = (const uint8_t*)p.h;
    g.as = p.hs;
    g.perm = nullptr;
    g.T = T;
    g.k = k;
    g.E = E;
    g.Tk = p.Tk;
    g.b0 = (const uint8_t*)routed->w2;
    g.b0s = routed->w2_scale;
    g.sb0 = shared ? (const uint8_t*)shared->w2 : nullptr;
    g.sb0s = shared ? shared->w2_scale : nullptr;
    g.K = inter;
    g.N = d;
    g.mstart = p.mstart;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = out;
    g.flag = p.flag;
    // the configured tile where its width divides d, else 64-column tiles of the same
    // height (same bits: every output is the same MFMA chain)
    const bool wide = d % (32 * MOE_MX_FN * MOE_MX_WN) == 0;
    g.NT = p.mx_ring ? d / XR_N : wide ? d / (32 * MOE_MX_FN * MOE_MX_WN) : d / 64;
    const long long grid = tile_grid(p.mt_bound * g.NT, p.mx_ring ? kMxXcdChunk : 0);
    if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    if (p.mx_ring)
      grouped_gemm_mx_ring_kernel<1><<<(unsigned)grid, 512, 0, s>>>(g);
    else if (wide)
      grouped_gemm_mx_kernel<1, MOE_MX_WM, MOE_MX_WN, MOE_MX_FN>
          <<<(unsigned)grid, 64 * MOE_MX_WM * MOE_MX_WN, 0, s>>>(g);
    else
      grouped_gemm_mx_kernel<1, MOE_MX_WM, 1, 2><<<(unsigned)grid, 64 * MOE_MX_WM, 0, s>>>(g);
  } else if (dtype == MOE_BF16) {
    GemmArgs g{};
    g.a = (const uint16_t*)p.h;
    g.perm = nullptr;
    g.T = T;
    g.k = k;
    g.E = E;
    g.Tk = p.Tk;
    g.b0 = (const uint16_t*)routed->w2;
    g.sb0 = shared ? (const uint16_t*)shared->w2 : nullptr;
    g.K = inter;
    g.N = d;
    g.NT = d / 128;
    g.mstart = p.mstart;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = (uint16_t*)out;
    g.flag = p.flag;
    const int wn = bf16_wn(d, 64, MOE_GEMM2_WN);
    g.NT = d / (64 * wn);
    const long long grid = tile_grid(p.mt_bound * g.NT, 0);
    if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    launch_bf16<1>(wn, (unsigned)grid, s, g);
  } else {
    F32Args g{};
    g.a = (const float*)p.h;
    g.T = T;
    g.k = k;
    g.E = E;
    g.Tk = p.Tk;
    g.rows = p.rows;
    g.b0 = (const float*)routed->w2;
    g.sb0 = shared ? (const float*)shared->w2 : nullptr;
    g.K = inter;
    g.N = d;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = (float*)out;
    g.flag = p.flag;
    const long long n = p.rows * d;
    grouped_ffn_f32_kernel<1><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(g);
  }
  return launch_status();
}

moe_status ffn_seg_table(const int32_t* offsets, int T, int E, int k, int has_shared, int* seg, int* flag,
                         hipStream_t s) {
  seg_table_kernel<<<1, 1024, 0, s>>>(offsets, E, (long long)T * k, T, has_shared, BM, seg, seg + (E + 2),
                                      seg + 2 * (E + 2), flag);
  return launch_status();
}

moe_status ffn_recompute_pre(const void* x, int T, int d, int E, int k, int inter,
                             const moe_expert_bank* routed, const moe_expert_bank* shared,
                             const int32_t* offsets, const int32_t* perm, int* seg, float* pre,
                             int* flag, hipStream_t s) {
  const int has_shared = shared ? 1 : 0;
  const long long Tk = (long long)T * k;
  int* mstart = seg;
  int* rowstart = seg + (E + 2);
  int* rowcount = rowstart + (E + 2);
  seg_table_kernel<<<1, 1024, 0, s>>>(offsets, E, Tk, T, has_shared, BM, mstart, rowstart, rowcount,
                                      flag);
  GemmArgs g{};
  g.a = (const uint16_t*)x;
  g.perm = perm;
  g.T = T;
  g.k = k;
  g.E = E;
  g.Tk = Tk;
  g.b0 = (const uint16_t*)routed->w1;
  g.b1 = (const uint16_t*)routed->w3;
  g.sb0 = shared ? (const uint16_t*)shared->w1 : nullptr;
  g.sb1 = shared ? (const uint16_t*)shared->w3 : nullptr;
  g.K = d;
  g.N = inter;
  g.mstart = mstart;
  g.rowstart = rowstart;
  g.rowcount = rowcount;
  g.S = E + has_shared;
  g.out = nullptr;
  g.out_pre = pre;
  g.flag = flag;
  const int wn = bf16_wn(inter, 32, MOE_GEMM1_WN);
  g.NT = inter / (32 * wn);
  const long long mt_bound = (Tk + (long long)E * (BM - 1)) / BM + (has_shared ? (T + BM - 1) / BM : 0);
  const long long grid = tile_grid(mt_bound * g.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (grid == 0) return launch_status();
  launch_bf16<2>(wn, (unsigned)grid, s, g);
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_expert_ffn_gate_up(const void* x, const uint8_t* x_scale, int dtype, int T,
                                             int d, int E, int k, int inter,
                                             const moe_expert_bank* routed,
                                             const moe_expert_bank* shared, const int32_t* offsets,
                                             const int32_t* perm, void* ws, size_t ws_bytes,
                                             void* stream) {
  moe_status st = check_ffn_shape(dtype, T, d, E, k, inter, routed, shared, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((dtype == MOE_MXFP8) != (x_scale != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && !aligned(x, 16)) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_MXFP8 && (!aligned(x_scale, 4) || !mx_bank_aligned(routed) ||
                             (shared && !mx_bank_aligned(shared))))
    return MOE_ERR_INVALID_ARG;
  const FfnPlan p = plan_of(ws, T, d, E, k, inter, dtype, shared != nullptr);
  return run_gate_up(x, x_scale, dtype, T, d, E, k, inter, routed, shared, offsets, perm, p,
                     (hipStream_t)stream);
}

extern "C" moe_status moe_expert_ffn_gate_up_save(const void* x, const uint8_t* x_scale, int dtype,
                                                  int T, int d, int E, int k, int inter,
                                                  const moe_expert_bank* routed,
                                                  const moe_expert_bank* shared,
                                                  const int32_t* offsets, const int32_t* perm,
                                                  float* pre, void* ws, size_t ws_bytes,
                                                  void* stream) {
  moe_status st = check_ffn_shape(dtype, T, d, E, k, inter, routed, shared, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (dtype != MOE_BF16 || MOE_GEMM_DMA) return MOE_ERR_UNSUPPORTED;
  if (x_scale || !offsets) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm || !pre || !aligned(x, 16) || !aligned(pre, 16)) return MOE_ERR_INVALID_ARG;
  const FfnPlan p = plan_of(ws, T, d, E, k, inter, dtype, shared != nullptr);
  return run_gate_up(x, x_scale, dtype, T, d, E, k, inter, routed, shared, offsets, perm, p,
                     (hipStream_t)stream, pre);
}

extern "C" moe_status moe_expert_ffn_down(int dtype, int T, int d, int E, int k, int inter,
                                          const moe_expert_bank* routed,
                                          const moe_expert_bank* shared, void* out, void* ws,
                                          size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_shape(dtype, T, d, E, k, inter, routed, shared, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!out) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_MXFP8 && (!mx_bank_aligned(routed) || (shared && !mx_bank_aligned(shared))))
    return MOE_ERR_INVALID_ARG;
  const FfnPlan p = plan_of(ws, T, d, E, k, inter, dtype, shared != nullptr);
  return run_down(dtype, T, d, E, k, inter, routed, shared, out, p, (hipStream_t)stream);
}

extern "C" moe_status moe_expert_ffn(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                     int E, int k, int inter, const moe_expert_bank* routed,
                                     const moe_expert_bank* shared, const int32_t* offsets,
                                     const int32_t* perm, void* out, void* ws, size_t ws_bytes,
                                     void* stream) {
  moe_status st = check_ffn_shape(dtype, T, d, E, k, inter, routed, shared, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if ((dtype == MOE_MXFP8) != (x_scale != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm || !out) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && (!aligned(x, 16) || !aligned(out, 16))) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_MXFP8 && (!aligned(x_scale, 4) || !mx_bank_aligned(routed) ||
                             (shared && !mx_bank_aligned(shared))))
    return MOE_ERR_INVALID_ARG;
  const FfnPlan p = plan_of(ws, T, d, E, k, inter, dtype, shared != nullptr);
  hipStream_t s = (hipStream_t)stream;
  if ((st = run_gate_up(x, x_scale, dtype, T, d, E, k, inter, routed, shared, offsets, perm, p, s)) !=
      MOE_OK)
    return st;
  return run_down(dtype, T, d, E, k, inter, routed, shared, out, p, s);
}
