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
constexpr int BK = 64;        // reduction step
constexpr int LDSS = BK + 8;  // LDS row stride in bf16 elements (144 B: conflict-free 16-B reads)

// Widest tile (wavefronts along N) each bf16 GEMM uses where the shape divides; the
// narrower tiles give the same bits (each output is the same MFMA sequence over K).
constexpr int kGemm1Wn = 4;
constexpr int kGemm2Wn = 4;


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


// MODE 0: GEMM1 (W1 and W3, SwiGLU epilogue, 32 * WN output features per tile).
// MODE 1: GEMM2 (W2, 64 * WN output features per tile).
// MODE 2: GEMM1 without the epilogue: the fp32 pre-activations x W1 and x W3 (the
//         backward pass recomputes them; same MFMA sequence as MODE 0).
// 128 * WN threads = 2 x WN wavefronts; each wavefront owns a 64-row x 64-B-row part
// of the 128 x (64 * WN) tile as 2 x 2 MFMA 32x32x16 blocks.  In GEMM1 the staged B
// rows alternate 32-row blocks of W1 and W3 for the same features, so a wavefront's
// two column blocks are the W1 and W3 halves of 32 features.
// Rows past the segment's end are neither loaded nor multiplied: their LDS rows hold
// zeros, and a wavefront skips the MFMAs of a 32-row block that holds no valid row (a
// row of an MFMA result depends only on the same row of A, so the valid rows get the
// same bits whatever is skipped).
// Wide tiles (WN >= 4) are held to 128 registers so that 4 wavefronts fit per SIMD.
template <int MODE, int WN>
__global__ __launch_bounds__(128 * WN)
__attribute__((amdgpu_waves_per_eu(WN >= 4 ? 4 : 1)))
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

  // ---- per-thread source rows.  A tile row r >= mrows is not loaded (zeros in LDS);
  //      it only feeds output row r, which is never stored. ----
  const uint16_t* aptr[LA];
  const uint16_t* bptr[LB];
  bool alive[LA];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = lr + RSTEP * i;
    alive[i] = r < mrows;
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
  // 32-row blocks of this wavefront that hold at least one valid row (wave-uniform)
  const bool live0 = wm * 64 < mrows, live1 = wm * 64 + 32 < mrows;

  // K loop: one K-step of global loads in flight per thread; each step goes
  // registers -> LDS -> MFMA.
  u32x4_t ra[LA], rb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) ra[i] = u32x4_t{0u, 0u, 0u, 0u};
  auto gload = [&](int kofs) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      if (alive[i]) ra[i] = *(const u32x4_t*)(aptr[i] + kofs);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *(const u32x4_t*)(bptr[i] + kofs);
  };
  gload(0);
  for (int k0 = 0; k0 < g.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(u32x4_t*)&sA[(lr + RSTEP * i) * LDSS + lc] = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(u32x4_t*)&sB[(lr + RSTEP * i) * LDSS + lc] = rb[i];
    __syncthreads();
    if (k0 + BK < g.K) gload(k0 + BK);
    if (live0) {
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
        for (int nb = 0; nb < 2; ++nb)
          acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bf[nb], acc[0][nb], 0, 0, 0);
        if (live1) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bf[nb], acc[1][nb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
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
        // nontemporal: the expert outputs are read once, by the combine (GEMM2 -2%)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + wn * 64 + nb * 32 + j;
          __builtin_nontemporal_store(f32_to_bf16(acc[mb][nb][v]), &g.out[orow * g.N + col]);
        }
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
  p.tm = dtype == MOE_MXFP8 ? mx_tile_rows(d, inter, p.Tk, E) : BM;   // NVFP4: BM as bf16
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
  if (wn == 4)
    grouped_gemm_bf16_kernel<MODE, 4><<<grid, 512, 0, s>>>(g);
  else
    grouped_gemm_bf16_kernel<MODE, 2><<<grid, 256, 0, s>>>(g);
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
    q.out_pre = pre;
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
    g.mstart = p.mstart;
    g.rowstart = p.rowstart;
    g.rowcount = p.rowcount;
    g.S = p.S;
    g.out = p.h;
    g.out_scale = p.hs;
    g.out_pre = pre;
    g.flag = p.flag;
    g.tm = p.tm;
    const moe_status st = mx_gemm(0, g, p.mt_bound, s);
    if (st != MOE_OK) return st;
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
    const int wn = bf16_wn(inter, 32, kGemm1Wn);
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
    g.tm = p.tm;
    const moe_status st = mx_gemm(1, g, p.mt_bound, s);
    if (st != MOE_OK) return st;
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
    const int wn = bf16_wn(d, 64, kGemm2Wn);
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

moe_status ffn_seg_table_rows(const int32_t* offsets, int T, int E, int k, int has_shared, int tm, int* seg,
                              int* flag, hipStream_t s) {
  seg_table_kernel<<<1, 1024, 0, s>>>(offsets, E, (long long)T * k, T, has_shared, tm, seg, seg + (E + 2),
                                      seg + 2 * (E + 2), flag);
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
  const int wn = bf16_wn(inter, 32, kGemm1Wn);
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
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8 && dtype != MOE_NVFP4) return MOE_ERR_UNSUPPORTED;
  if ((dtype == MOE_MXFP8) != (x_scale != nullptr) || !offsets) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm || !pre || !aligned(x, 16) || !aligned(pre, 16)) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_MXFP8 && (!aligned(x_scale, 4) || !mx_bank_aligned(routed) ||
                             (shared && !mx_bank_aligned(shared))))
    return MOE_ERR_INVALID_ARG;
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
