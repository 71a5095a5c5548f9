// MXFP8 grouped GEMMs of the expert FFN (Composer 2 Technical Report, section 6.1
// "Kernels": MoE weights and activations in MXFP8, E4M3 elements with one E8M0 scale per
// 32; OCP Microscaling Formats v1.0 for the encoding).  Same segment table, tile order
// and per-output reduction order rules as the bf16 grouped GEMM in ffn.hip: a tile never
// mixes experts and every output is one fixed chain of scaled MFMAs over ascending K.
#include <math.h>

#include <algorithm>

#include "moe_internal.h"
#include "mx_common.h"

namespace moe {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
#ifndef MOE_MX_XCD_CHUNK
#define MOE_MX_XCD_CHUNK 16
#endif
constexpr int kMxXcdChunk = MOE_MX_XCD_CHUNK;

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
  constexpr bool G1 = MODE != 1;             // GEMM1 operands (modes 0 and 2)
  const int n0 = nt * (G1 ? TB / 2 : TB);
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
    if (G1) {
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
    if (G1) {
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
      if (G1) {
        // One MX block = this row's 32 features, spread over the 32 lanes of a half.
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
          const int col = n0 + (wn * FN / 2 + p) * 32 + j;
          if (g.out_pre && r < mrows) {   // pre-activations for the backward pass
            g.out_pre[orow * 2 * g.N + col] = acc[mb][2 * p][v];
            g.out_pre[orow * 2 * g.N + g.N + col] = acc[mb][2 * p + 1][v];
          }
          if (MODE == 0) {
            const float hv = silu_f32(acc[mb][2 * p][v]) * acc[mb][2 * p + 1][v];
            mx_store_h(hv, r < mrows, (uint8_t*)g.out + orow * g.N + col,
                       g.out_scale + orow * (g.N / 32) + col / 32, j == 0);
          }
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
// The 256-row kernel stages its epilogue in halves of 64 local rows per wavefront
// (9 KB): wavefronts 0..6 in stage 1, wavefront 7 in a spare area after the scale
// buffers, so stage 0 and scale buffer 0 can take the next tile's first loads meanwhile.
constexpr int XR_EPH = 64 * XR_EPI_ROW;          // 9 KB
constexpr int XR_SPARE = XR_LDS;
constexpr int XR_LDS_P = XR_SPARE + 16 * 1024;   // 160 KB (its last 4 bytes: the next tile's position)
constexpr int kTileCtr = 16;                     // header ints 16 .. 23: per-XCD tile counters
static_assert(XR_LDS <= 160 * 1024 && 8 * XR_EPI <= XR_LDS, "LDS budget");
static_assert(7 * XR_EPH <= XR_STAGE && XR_EPH <= 16 * 1024 && XR_LDS_P <= 160 * 1024, "LDS budget");

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

template <int NB, int SEL, int MB>
__device__ __forceinline__ void xr_mfma(const XrFrag<NB>& f, const XrScale<NB>& sc4, f32x16_t (&acc)[MB][2]) {
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

// Scale group 0 and step 0 of a tile into scale buffer 0 and stage 0 (this wavefront's
// share), in the order the K loop's first wait expects.
__device__ __forceinline__ void xr_issue_first(uint32_t ring_lds, const XrSrc& src, int wave) {
  const uint32_t ls = wave < 4 ? wave * 1024 : XR_M * 16 + (wave - 4) * 1024;
  if (wave < 4)
    xr_load16(ring_lds + XR_SC + ls, src.soff, src.sbase);
  else
    xr_load16(ring_lds + XR_SC + ls, src.bsp);
  const uint32_t la = XR_A + wave * 4096, lb = XR_B + wave * 4096;
#pragma unroll
  for (int i = 0; i < 4; ++i) xr_load16(ring_lds + la + 1024 * i, src.aoff[i], src.abase);
#pragma unroll
  for (int i = 0; i < 4; ++i) xr_load16(ring_lds + lb + 1024 * i, src.boff[i], src.bbase);
}

// The K loop of a wavefront that multiplies NB of its 4 row blocks (NB = 0: it only
// loads and synchronises).  Step j (K bytes 128 j .. 128 j + 127) lives in stage j % 2.
// At step j: wait for its data, meet (every wavefront is then done with step j - 1, whose
// stage takes step j + 1's loads), multiply.  Scale group g (steps 4 g .. 4 g + 3) goes
// out at step 4 (g - 1), after that step's data, into buffer g % 2.
template <int NB>
__device__ __forceinline__ void xr_kloop(const uint8_t* ring, uint32_t ring_lds, int nsteps, const XrSrc& src,
                                         int wave, uint32_t aof, uint32_t bof, uint32_t asf, uint32_t bsf,
                                         int sh, f32x16_t (&acc)[4][2], int* ctr, int& qn) {
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

  // scale group 0 and step 0 went out before the call (xr_issue_first)
  for (int j = 0; j < nsteps; ++j) {
    // step j's data went out at step j - 1 (or before the loop), followed only by that
    // step's scale group (loads complete in issue order)
    if (scales_at(j - 1))
      xr_sync<1>();
    else
      xr_sync<0>();
    if (j + 1 < nsteps) issue(j + 1);
    if (scales_at(j)) issue_scales(j / XR_GS + 1);
    // the next tile's position, fetched right after step 2's loads go out, so its latency
    // overlaps theirs (the ring runs at least 4 steps; were there fewer, qn would stay
    // negative: no next tile)
    if (ctr && j == 1 && threadIdx.x == 0) qn = atomicAdd(ctr, 1);
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
      // the step's MFMAs stay ahead of the next step's wait, barrier and loads
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// A pointer the whole wavefront holds, kept in scalar registers.
__device__ __forceinline__ const uint8_t* xr_uniform(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Rows, columns and loader sources of one 256-row tile.
struct XrTile {
  int row0, mrows, n0;
  XrSrc src;
};

// Decode tile `tile` of the segment-major tile list (as grouped_gemm_mx_kernel, tiles of
// XR_M rows) and set up this thread's loader sources: wavefront w fills A rows and B rows
// 32 w .. 32 w + 31 (four loads of 8 rows each; lane l -> row + l / 8, slot l % 8 <- chunk
// slot ^ swz(row); the B rows are one 32-row block, so one bank) and the 16-byte scale
// groups of A rows 64 w + l (w < 4) or B rows 64 (w - 4) + l.  Every byte offset from a
// load's base fits 32 bits (one activation matrix, or one expert's matrix).  A tile row
// past the segment re-reads the tile's first row; a routed row whose token is out of
// range sets `bad` and reads token 0.
template <int MODE>
__device__ __forceinline__ void xr_decode(const MxArgs& g, int tile, int wave, int lane, XrTile& t, int& bad) {
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
  constexpr bool G1 = MODE != 1;   // GEMM1 operands (modes 0 and 2)
  const int n0 = nt * (G1 ? XR_N / 2 : XR_N);
  const bool is_shared = (s == g.E);
  const long long e = is_shared ? 0 : s;
  const int KB = g.K / 32;   // scale bytes per row
  t.row0 = row0;
  t.mrows = mrows;
  t.n0 = n0;

  auto a_src = [&](int r) -> long long {
    const long long jr = (long long)row0 + (r < mrows ? r : 0);
    if (!G1) return jr;
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
    if (G1) {
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
  t.src.abase = g.a;
  t.src.sbase = g.as;
  {
    const uint8_t *bank, *sbank;
    b_row(32 * wave, bank, sbank);
    t.src.bbase = xr_uniform(bank + e * g.N * (long long)g.K);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ xr_swz(r);
    t.src.aoff[i] = (uint32_t)(a_src(r) * g.K + 16 * chunk);
    const uint8_t *bank, *sbank;
    const long long br = b_row(r, bank, sbank);
    t.src.boff[i] = (uint32_t)(br * g.K + 16 * chunk);
  }
  t.src.soff = (uint32_t)(a_src(64 * (wave & 3) + lane) * KB);
  {
    const uint8_t *bank, *sbank;   // GEMM1: W1 scales for lanes 0..31, W3 for 32..63
    const long long br = b_row(64 * (wave & 3) + lane, bank, sbank);
    t.src.bsp = sbank + (e * g.N + br) * (long long)KB;
  }
}

// MXFP8 grouped GEMM, 256 x 256 tiles, eight wavefronts (2 along M x 4 along N, two per
// SIMD), each 4 row blocks x 2 B blocks of 32 x 32.  A wavefront whose 32-row blocks
// hold no valid row skips their MFMAs, so a short tile costs MFMA time in proportion to
// its valid 32-row blocks on the busier half.
// PERSIST (GEMM2, whose tiles have only I / 128 K steps, so a tile's start and epilogue
// weigh more): one workgroup per CU walks its XCD's share of the tile list (the tiles
// xcd_tile<kMxXcdChunk> deals to that XCD, in order), taking the next position from a
// per-XCD counter; a tile's scale group 0 and first K step go out before the previous
// tile's epilogue, which stages its outputs in halves through stage 1 and a spare area.
// Otherwise (GEMM1, measured 3% slower persistent) one tile per workgroup.  A tile's
// result does not depend on which workgroup computes it or when.
template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_mx_ring_kernel(MxArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[XR_LDS_P];
  constexpr bool G1 = MODE != 1;   // GEMM1 operands (modes 0 and 2)
  constexpr bool PERSIST = MODE == 1;

  const int total = g.mstart[g.S] * g.NT;
  const int xcd = blockIdx.x % kXcds;
  auto tile_of = [&](int q) { return ((q / kMxXcdChunk) * kXcds + xcd) * kMxXcdChunk + q % kMxXcdChunk; };
  // PERSIST: the XCD's next tile position, from a per-XCD counter in the workspace header
  // (cleared before the launch), read by thread 0 and handed to the workgroup through LDS
  int* const ctr = PERSIST ? g.flag + kTileCtr + xcd : nullptr;
  int* const s_q = (int*)(ring + XR_LDS_P - 4);
  const int tid = threadIdx.x, lane = tid & 63;
  int tile;
  if constexpr (PERSIST) {
    if (tid == 0) *s_q = atomicAdd(ctr, 1);
    __syncthreads();
    tile = tile_of(*s_q);
    if (tile >= total) return;
  } else {
    if (!xcd_tile<kMxXcdChunk>(total, tile)) return;
  }

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---- fragment offsets within a stage: lane reads row (block base + lane % 32),
  //      chunks lane / 32 and 2 + lane / 32 of the k range ----
  const int j32 = lane & 31, hh = lane >> 5;
  const int ra = 128 * wm + j32, rb = 64 * wn + j32;
  const uint32_t aof = XR_A + ra * XR_K + 16 * (hh ^ xr_swz(ra));
  const uint32_t bof = XR_B + rb * XR_K + 16 * (hh ^ xr_swz(rb));
  const uint32_t asf = ra * 16, bsf = XR_M * 16 + rb * 16;   // within a scale buffer
  const int sh = 8 * hh;

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8*)ring;
  const int nsteps = g.K / XR_K;
  // this wavefront's epilogue staging (64 local rows per half)
  uint8_t* stg = ring + (wave < 7 ? XR_STAGE + wave * XR_EPH : XR_SPARE);

  int bad = 0;
  XrTile cur;
  xr_decode<MODE>(g, tile, wave, lane, cur, bad);
  xr_issue_first(ring_lds, cur.src, wave);
  for (;;) {
    int qn = -1;   // stays negative (no next tile) unless the K loop fetched a position
    const int row0 = cur.row0, mrows = cur.mrows, n0 = cur.n0;

    f32x16_t acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    // 32-row blocks of this wavefront that hold a valid row (uniform per wavefront)
    const int nb_act = min(4, max(0, (mrows - wm * 128 + 31) >> 5));
    switch (nb_act) {
      case 4: xr_kloop<4>(ring, ring_lds, nsteps, cur.src, wave, aof, bof, asf, bsf, sh, acc, ctr, qn); break;
      case 3: xr_kloop<3>(ring, ring_lds, nsteps, cur.src, wave, aof, bof, asf, bsf, sh, acc, ctr, qn); break;
      case 2: xr_kloop<2>(ring, ring_lds, nsteps, cur.src, wave, aof, bof, asf, bsf, sh, acc, ctr, qn); break;
      case 1: xr_kloop<1>(ring, ring_lds, nsteps, cur.src, wave, aof, bof, asf, bsf, sh, acc, ctr, qn); break;
      default: xr_kloop<0>(ring, ring_lds, nsteps, cur.src, wave, aof, bof, asf, bsf, sh, acc, ctr, qn); break;
    }

    // ---- epilogue.  Accumulator element v of a lane is C[i][j], j = lane % 32,
    //      i = 8 (v / 4) + 4 (lane / 32) + v % 4; the wavefront's local row 32 mb + i is
    //      tile row 128 wm + 32 mb + i. ----
    // (the lane's row and column indices are re-derived per tile through an opaque copy,
    // so the compiler does not hoist the per-element addresses out of the tile loop and
    // keep them live across the K loop)
    int lane_t = lane;
    asm volatile("" : "+v"(lane_t));
    const int j32 = lane_t & 31, hh = lane_t >> 5;
    if (G1 && g.out_pre) {   // pre-activations for the backward pass, from the accumulators
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb >= nb_act) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 128 * wm + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (r < mrows) {
            const long long orow = (long long)row0 + r;
            const int col = n0 + 32 * wn + j32;
            g.out_pre[orow * 2 * g.N + col] = acc[mb][0][v];
            g.out_pre[orow * 2 * g.N + g.N + col] = acc[mb][1][v];
          }
        }
      }
    }
    if (PERSIST && tid == 0) *s_q = qn;
    __syncthreads();   // every wavefront is done reading the ring; the next position is out
    qn = PERSIST ? *s_q : -1;
    const int tn = qn >= 0 ? tile_of(qn) : total;
    const bool more = tn < total;
    XrTile nxt;
    // the next tile's first loads, into stage 0 and scale buffer 0
    auto prefetch = [&]() {
      if (more) {
        xr_decode<MODE>(g, tn, wave, lane, nxt, bad);
        xr_issue_first(ring_lds, nxt.src, wave);
      }
    };
    if (MODE != 0) prefetch();   // GEMM2: before its epilogue; pre-activations only: no epilogue
    if (MODE == 1) {
      // two halves: local rows 64 h .. 64 h + 63 of every wavefront (blocks 2 h, 2 h + 1),
      // staged in stage 1 and the spare area; a wavefront reads back only what it wrote
      // (its LDS accesses complete in order)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
          const int mb = 2 * h + m2;
          if (mb >= nb_act) break;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = 32 * m2 + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              *(uint16_t*)(stg + rl * XR_EPI_ROW + (32 * nb + j32) * 2) = f32_to_bf16(acc[mb][nb][v]);
          }
        }
        // lane l: local row 8 q + l / 8 of the half, 16-byte chunk l % 8 of its 64 outputs
        const int c = lane & 7;
#pragma unroll 4
        for (int q2 = 0; q2 < 8; ++q2) {
          const int rl = 8 * q2 + (lane >> 3);
          const int r = 128 * wm + 64 * h + rl;
          if (((64 * h + rl) >> 5) < nb_act && r < mrows) {
            const u32x4_t t = *(const u32x4_t*)(stg + rl * XR_EPI_ROW + 16 * c);
            // nontemporal: the expert outputs are read once, by the combine
            __builtin_nontemporal_store(
                t, (u32x4_t*)((uint16_t*)g.out + ((long long)row0 + r) * g.N + n0 + wn * 64 + 8 * c));
          }
        }
      }
    } else if (MODE == 0) {
      // each wavefront stages its 128 x 32 values of h in its own 18 KB of the ring, then
      // thread i requantises tile row (i + 512 q) / 4, MX block i % 4 (wavefront column
      // wn's 32 features), staged by wavefront (row / 128, i % 4); four neighbouring lanes
      // write a row's 128 code bytes and its 4 scale bytes contiguously
      uint8_t* st1 = ring + wave * XR_EPI;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb >= nb_act) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
          // B blocks 0 and 1 are the W1 and W3 halves of the same 32 features
          *(float*)(st1 + rl * XR_EPI_ROW + j32 * 4) = silu_f32(acc[mb][0][v]) * acc[mb][1][v];
        }
      }
      __syncthreads();
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int idx = tid + 512 * q2, r = idx >> 2, b = idx & 3;
        if (r < mrows) {
          const long long orow = (long long)row0 + r;
          const int col = n0 + 32 * b;
          mx_store_block(ring + ((r >> 7) * 4 + b) * XR_EPI + (r & 127) * XR_EPI_ROW,
                         (uint8_t*)g.out + orow * g.N + col, g.out_scale + orow * (g.N / 32) + col / 32);
        }
      }
      __syncthreads();   // every staging read is done (the stores may still be in flight)
      prefetch();
    }
    if (!more) break;
    tile = tn;
    cur = nxt;
    cur.row0 = __builtin_amdgcn_readfirstlane(cur.row0);
    cur.mrows = __builtin_amdgcn_readfirstlane(cur.mrows);
    cur.n0 = __builtin_amdgcn_readfirstlane(cur.n0);
    cur.src.abase = xr_uniform(cur.src.abase);
    cur.src.bbase = xr_uniform(cur.src.bbase);
    cur.src.sbase = xr_uniform(cur.src.sbase);
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);
}

// ---------------------------------------------------------------------------
// Ring kernel for short segments (few rows per expert, where the GEMMs stream the
// weights from HBM): 128 x 256 tiles over a three-stage ring, so two K steps of weight
// rows are in flight per workgroup, and half the activation rows of the 256-row tile.
// Eight wavefronts (2 along M x 4 along N), each 2 row blocks x 2 B blocks of 32 x 32;
// same fragment layout, swizzle, scale staging and per-output MFMA chain as
// grouped_gemm_mx_ring_kernel (K ascending in 64-wide scaled MFMAs from zero), hence the
// same bits for every row whatever the tile height.
// ---------------------------------------------------------------------------
constexpr int XS_M = 128;                        // tile rows
constexpr int XS_ST = 3;                         // ring stages
constexpr int XS_A = 0, XS_B = XS_M * XR_K;      // tile offsets within a stage
constexpr int XS_STAGE = (XS_M + XR_N) * XR_K;   // 48 KB
constexpr int XS_SC = XS_ST * XS_STAGE;          // two scale-group buffers after the stages
constexpr int XS_SCB = (XS_M + XR_N) * 16;       // bytes per scale-group buffer (A rows, then B)
constexpr int XS_LDS = XS_SC + 2 * XS_SCB;       // 156 KB
constexpr int XS_EPI = 64 * XR_EPI_ROW;          // epilogue staging per wavefront (9 KB)
static_assert(XS_LDS <= 160 * 1024 && 8 * XS_EPI <= XS_LDS, "LDS budget");

// The K loop of a wavefront that multiplies NB of its 2 row blocks (NB = 0: it only loads
// and synchronises).  Step j lives in stage j % 3.  At step j: wait for its data (loads
// complete in issue order), meet (every wavefront is then done with step j - 1, whose
// stage takes step j + 2's loads), multiply.  Scale group g (steps 4 g .. 4 g + 3) goes
// out at step 4 (g - 1) into buffer g % 2.  Per step a wavefront issues 2 A loads and 4 B
// loads; waves 0..3 each load the scale groups of 32 A rows, waves 4..7 of 64 B rows.
template <int NB>
__device__ __forceinline__ void xs_kloop(const uint8_t* ring, uint32_t ring_lds, int nsteps, const XrSrc& src,
                                         int wave, int lane, uint32_t aof, uint32_t bof, uint32_t asf,
                                         uint32_t bsf, int sh, f32x16_t (&acc)[2][2]) {
  const uint32_t la = XS_A + wave * 2048, lb = XS_B + wave * 4096;
  const uint32_t ls = wave < 4 ? wave * 512 : XS_M * 16 + (wave - 4) * 1024;
  const int ngroups = nsteps / XR_GS;
  auto issue = [&](int j) {
    const uint32_t st = ring_lds + (uint32_t)(j % XS_ST) * XS_STAGE;
    const int k0 = j * XR_K;
#pragma unroll
    for (int i = 0; i < 2; ++i) xr_load16(st + la + 1024 * i, src.aoff[i], src.abase + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) xr_load16(st + lb + 1024 * i, src.boff[i], src.bbase + k0);
  };
  auto issue_scales = [&](int grp) {
    const uint32_t dst = ring_lds + XS_SC + (uint32_t)(grp & 1) * XS_SCB + ls;
    if (wave < 4) {
      if (lane < 32) xr_load16(dst, src.soff, src.sbase + 16 * grp);
    } else {
      xr_load16(dst, src.bsp + 16 * grp);
    }
  };
  auto scales_at = [&](int j) { return j >= 0 && j % XR_GS == 0 && j / XR_GS + 1 < ngroups; };

  issue_scales(0);
  issue(0);
  if (nsteps > 1) issue(1);
  for (int j = 0; j < nsteps; ++j) {
    // issued after step j's loads: step j + 1's (6), and the scale group issued at step
    // j - 2 or j - 1 (at most one of them)
    const bool nxt = j + 1 < nsteps;
    const bool sc = scales_at(j - 1) || (j >= 2 && scales_at(j - 2));
    if (nxt && sc)
      xr_sync<7>();
    else if (nxt)
      xr_sync<6>();
    else if (sc)
      xr_sync<1>();
    else
      xr_sync<0>();
    if (j + 2 < nsteps) issue(j + 2);
    if (scales_at(j)) issue_scales(j / XR_GS + 1);
    if constexpr (NB > 0) {
      const uint8_t* st = ring + (j % XS_ST) * XS_STAGE;
      const uint8_t* scb = ring + XS_SC + ((j / XR_GS) & 1) * XS_SCB;
      XrScale<NB> sc4;
      xr_read_scales<NB>(sc4, scb, asf, bsf, (j % XR_GS) * (XR_K / 32), sh);
      XrFrag<NB> f;
      xr_read<NB>(f, st, aof, bof, 0);
      xr_mfma<NB, 0>(f, sc4, acc);
      xr_read<NB>(f, st, aof, bof, 1);
      xr_mfma<NB, 2>(f, sc4, acc);
      // the step's MFMAs stay ahead of the next step's wait, barrier and loads
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_mx_ring128_kernel(MxArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[XS_LDS];

  // ---- tile decode (as grouped_gemm_mx_ring_kernel, tiles of XS_M rows) ----
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
  const int row0 = g.rowstart[s] + mt * XS_M;
  const int mrows = min(XS_M, g.rowcount[s] - mt * XS_M);
  constexpr bool G1 = MODE == 0 || MODE == 2;   // GEMM1 operands (gathered x; W1 | W3)
  const int n0 = nt * (G1 ? XR_N / 2 : XR_N);
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
    if (!G1) return jr;
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
    if (G1) {
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

  // ---- loader: wavefront w fills A rows 16 w .. 16 w + 15 (two loads of 8 rows) and B
  //      rows 32 w .. 32 w + 31 (four loads; one 32-row block, so one bank); lane l ->
  //      row + l / 8, slot l % 8 <- chunk slot ^ swz(row).  Scale groups: A rows
  //      32 w + l (w < 4, lanes < 32) or B rows 64 (w - 4) + l. ----
  XrSrc src;
  src.abase = g.a;
  src.sbase = g.as;
  {
    const uint8_t *bank, *sbank;
    b_row(32 * wave, bank, sbank);
    src.bbase = bank + e * g.N * (long long)g.K;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ xr_swz(r);
    src.aoff[i] = (uint32_t)(a_src(r) * g.K + 16 * chunk);
  }
  src.aoff[2] = src.aoff[3] = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ xr_swz(r);
    const uint8_t *bank, *sbank;
    const long long br = b_row(r, bank, sbank);
    src.boff[i] = (uint32_t)(br * g.K + 16 * chunk);
  }
  src.soff = (uint32_t)(a_src(32 * (wave & 3) + (lane & 31)) * KB);
  {
    const uint8_t *bank, *sbank;   // GEMM1: W1 scales for lanes 0..31, W3 for 32..63
    const long long br = b_row(64 * (wave & 3) + lane, bank, sbank);
    src.bsp = sbank + (e * g.N + br) * (long long)KB;
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  // ---- fragment offsets within a stage ----
  const int j32 = lane & 31, hh = lane >> 5;
  const int ra = 64 * wm + j32, rb = 64 * wn + j32;
  const uint32_t aof = XS_A + ra * XR_K + 16 * (hh ^ xr_swz(ra));
  const uint32_t bof = XS_B + rb * XR_K + 16 * (hh ^ xr_swz(rb));
  const uint32_t asf = ra * 16, bsf = XS_M * 16 + rb * 16;   // within a scale buffer
  const int sh = 8 * hh;

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8*)ring;
  const int nsteps = g.K / XR_K;
  const int nb_act = min(2, max(0, (mrows - wm * 64 + 31) >> 5));
  switch (nb_act) {
    case 2: xs_kloop<2>(ring, ring_lds, nsteps, src, wave, lane, aof, bof, asf, bsf, sh, acc); break;
    case 1: xs_kloop<1>(ring, ring_lds, nsteps, src, wave, lane, aof, bof, asf, bsf, sh, acc); break;
    default: xs_kloop<0>(ring, ring_lds, nsteps, src, wave, lane, aof, bof, asf, bsf, sh, acc); break;
  }

  // ---- epilogue (as grouped_gemm_mx_ring_kernel; the wavefront's local row 32 mb + i
  //      is tile row 64 wm + 32 mb + i) ----
  if (G1 && g.out_pre) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (mb >= nb_act) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 64 * wm + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (r < mrows) {
          const long long orow = (long long)row0 + r;
          const int col = n0 + 32 * wn + j32;
          g.out_pre[orow * 2 * g.N + col] = acc[mb][0][v];
          g.out_pre[orow * 2 * g.N + g.N + col] = acc[mb][1][v];
        }
      }
    }
  }
  if (MODE == 2) return;
  if (MODE >= 3) {
    // backward data GEMMs: fp32 rows straight from the accumulators (mode 3 with the
    // SwiGLU backward at the saved pre-activations: da = dh g silu'(a), dg = dh silu(a))
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (mb >= nb_act) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 64 * wm + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (r >= mrows) continue;
        const long long jr = (long long)row0 + r;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + 64 * wn + 32 * nb + j32;
          const float c = acc[mb][nb][v];
          if (MODE == 4) {
            g.out_f[jr * g.N + col] = c;
          } else {
            const float av = g.pre_in[jr * 2 * g.N + col], gv = g.pre_in[jr * 2 * g.N + g.N + col];
            const float sg = sigmoid_f32(av);
            g.out_f[jr * 2 * g.N + col] = c * gv * (sg * (1.0f + av * (1.0f - sg)));
            g.out_f[jr * 2 * g.N + g.N + col] = c * silu_f32(av);
          }
        }
      }
    }
    return;
  }
  __syncthreads();   // every wavefront is done reading the ring
  uint8_t* stg = ring + wave * XS_EPI;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (mb >= nb_act) break;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (MODE == 0) {
        *(float*)(stg + rl * XR_EPI_ROW + j32 * 4) = silu_f32(acc[mb][0][v]) * acc[mb][1][v];
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          *(uint16_t*)(stg + rl * XR_EPI_ROW + (32 * nb + j32) * 2) = f32_to_bf16(acc[mb][nb][v]);
      }
    }
  }
  if (MODE == 0) {
    // thread i: tile row i / 4, MX block i % 4, staged by wavefront (row / 64, i % 4)
    __syncthreads();
    const int r = tid >> 2, b = tid & 3;
    if (r < mrows) {
      const long long orow = (long long)row0 + r;
      const int col = n0 + 32 * b;
      mx_store_block(ring + ((r >> 6) * 4 + b) * XS_EPI + (r & 63) * XR_EPI_ROW,
                     (uint8_t*)g.out + orow * g.N + col, g.out_scale + orow * (g.N / 32) + col / 32);
    }
  } else {
    // lane l: local row 8 q + l / 8, 16-byte chunk l % 8 of the row's 64 outputs
    const int c = lane & 7;
#pragma unroll 4
    for (int q2 = 0; q2 < 8; ++q2) {
      const int rl = 8 * q2 + (lane >> 3);
      const int r = 64 * wm + rl;
      if ((rl >> 5) < nb_act && r < mrows) {
        const u32x4_t t = *(const u32x4_t*)(stg + rl * XR_EPI_ROW + 16 * c);
        __builtin_nontemporal_store(t, (u32x4_t*)((uint16_t*)g.out + ((long long)row0 + r) * g.N + n0 + wn * 64 + 8 * c));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Both GEMMs run on the ring kernel when it tiles the shape: GEMM2's output in XR_N
// columns, and 16-byte (XR_GB-element) scale groups along both reductions.
static bool mx_ring_ok(int d, int inter) {
  return MOE_MX_RING && d % XR_N == 0 && d % XR_GB == 0 && inter % XR_GB == 0;
}

// The 128-row ring where the experts average at most 128 routed rows (the GEMMs stream
// the weights; two K steps in flight), the 256-row ring above that (MFMA-bound).
int mx_tile_rows(int d, int inter, long long Tk, int E) {
  if (!mx_ring_ok(d, inter)) return 64 * MOE_MX_WM;
  return Tk <= (long long)XS_M * E ? XS_M : XR_M;
}

__global__ void mx_ctr_clear_kernel(int* p) {
  if (threadIdx.x < kXcds) p[threadIdx.x] = 0;
}

// Workgroups of a persistent launch: the current device's CUs, rounded down to a multiple
// of the XCD count (cached per device).
static long long mx_persistent_grid() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kXcds * 32;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < kXcds)
      n = kXcds * 32;
    cus[dev] = n;
  }
  return (long long)(cus[dev] / kXcds) * kXcds;
}

moe_status mx_gemm(int mode, MxArgs g, long long mt_bound, hipStream_t s) {
  const bool g1 = mode != 1;
  const int d = g1 ? g.K : g.N, inter = g1 ? g.N : g.K;
  const bool ring = mx_ring_ok(d, inter);
  // the kernel's tile height must be the one the segment table counted
  if (ring ? (g.tm != XS_M && g.tm != XR_M) : g.tm != 64 * MOE_MX_WM) return MOE_ERR_INVALID_ARG;
  if (g1) {
    g.NT = ring ? inter / (XR_N / 2) : inter / (16 * MOE_MX_FN * MOE_MX_WN);
  } else {
    // the configured tile where its width divides d, else 64-column tiles of the same
    // height (same bits: every output is the same MFMA chain)
    const bool wide = d % (32 * MOE_MX_FN * MOE_MX_WN) == 0;
    g.NT = ring ? d / XR_N : wide ? d / (32 * MOE_MX_FN * MOE_MX_WN) : d / 64;
  }
  const long long grid = tile_grid(mt_bound * g.NT, ring ? kMxXcdChunk : 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (grid == 0) return MOE_OK;
  if (ring && g.tm == XS_M) {
    if (mode == 0)
      grouped_gemm_mx_ring128_kernel<0><<<(unsigned)grid, 512, 0, s>>>(g);
    else if (mode == 2)
      grouped_gemm_mx_ring128_kernel<2><<<(unsigned)grid, 512, 0, s>>>(g);
    else
      grouped_gemm_mx_ring128_kernel<1><<<(unsigned)grid, 512, 0, s>>>(g);
  } else if (ring) {
    if (mode == 0) {
      grouped_gemm_mx_ring_kernel<0><<<(unsigned)grid, 512, 0, s>>>(g);
    } else if (mode == 2) {
      grouped_gemm_mx_ring_kernel<2><<<(unsigned)grid, 512, 0, s>>>(g);
    } else {
      // persistent: at most one workgroup per CU (each holds 160 KB of LDS)
      const unsigned pgrid = (unsigned)std::min<long long>(grid, mx_persistent_grid());
      mx_ctr_clear_kernel<<<1, 64, 0, s>>>(g.flag + kTileCtr);
      grouped_gemm_mx_ring_kernel<1><<<pgrid, 512, 0, s>>>(g);
    }
  } else if (mode == 0) {
    grouped_gemm_mx_kernel<0, MOE_MX_WM, MOE_MX_WN, MOE_MX_FN>
        <<<(unsigned)grid, 64 * MOE_MX_WM * MOE_MX_WN, 0, s>>>(g);
  } else if (mode == 2) {
    grouped_gemm_mx_kernel<2, MOE_MX_WM, MOE_MX_WN, MOE_MX_FN>
        <<<(unsigned)grid, 64 * MOE_MX_WM * MOE_MX_WN, 0, s>>>(g);
  } else if (d % (32 * MOE_MX_FN * MOE_MX_WN) == 0) {
    grouped_gemm_mx_kernel<1, MOE_MX_WM, MOE_MX_WN, MOE_MX_FN>
        <<<(unsigned)grid, 64 * MOE_MX_WM * MOE_MX_WN, 0, s>>>(g);
  } else {
    grouped_gemm_mx_kernel<1, MOE_MX_WM, 1, 2><<<(unsigned)grid, 64 * MOE_MX_WM, 0, s>>>(g);
  }
  return MOE_OK;
}

moe_status mx_gemm_bwd_data(int mode, int d, int inter, MxArgs g, long long mt_bound, hipStream_t s) {
  if ((mode != 3 && mode != 4) || !mx_ring_ok(d, inter)) return MOE_ERR_UNSUPPORTED;
  g.NT = g.N / XR_N;
  const long long grid = tile_grid(mt_bound * g.NT, kMxXcdChunk);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (grid == 0) return MOE_OK;
  if (mode == 3)
    grouped_gemm_mx_ring128_kernel<3><<<(unsigned)grid, 512, 0, s>>>(g);
  else
    grouped_gemm_mx_ring128_kernel<4><<<(unsigned)grid, 512, 0, s>>>(g);
  return MOE_OK;
}

}  // namespace moe
