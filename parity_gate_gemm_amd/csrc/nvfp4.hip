// NVFP4 expert FFN: the forward-pass format of the Composer 2 Technical Report, section
// 6.1 "Kernels": FP4 E2M1 values, one FP8 E4M3 scale per block of 16 elements and one
// FP32 scale per token (per row), quantized with IEEE division.
//
// gfx950's block-scaled MFMA takes E8M0 scales per 32 elements, which cannot carry an
// E4M3 scale's mantissa, so the GEMMs run on the decoded values E2M1 x E4M3 in fp16: the
// product has at most 6 significant bits and lies in [2^-10, 2688], so it is exact in
// fp16 (11 bits, normal from 2^-14), every MFMA product is exact, and the per-row fp32
// scales of both operands multiply the fp32 accumulator in the epilogue.
//
// Quantization of a row v (K % 16 == 0), every step one fp32 operation rounded to
// nearest even: s = amax / 2688 (2688 = 6 * 448, the largest E2M1 times the largest
// E4M3); per block S = E4M3_RNE((bamax / s) / 6), saturating at 448; per element
// E2M1_RNE(v / (S s)), ties to even, saturating at 6.  A zero row has s = 0 and zero
// codes.  Codes are packed two per byte, element 2i in the low nibble.
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// E4M3 code -> fp32 (v_cvt_pk_f32_fp8 decodes every E4M3 code exactly).
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
}

// fp32 in [0, 448] -> E4M3 code, round to nearest even (v_cvt_pk_fp8_f32).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(v, 448.0f), 0.0f, 0, false) & 0xffu;
}

// fp32 -> E2M1 code, nearest with ties to the even code, saturating at 6: the count of
// midpoints below |v| (a tie rounds down where the lower grid point has the even code,
// up where the upper one has).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
               (a > 5.0f);
  return c | (signbit(v) ? 8u : 0u);
}

// Byte B of word u: two E2M1 codes (low nibble first) as an fp16 pair (scale 1: the
// conversion applies only a power-of-two scale), times the block scale S2 = {S, S}
// (a packed fp16 product, exact).
template <int B>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t u, f16x2_t S2) {
  const f16x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 1.0f, B);
  return __builtin_bit_cast(uint32_t, f * S2);
}

// 16 fp16 values of one NVFP4 block (codes c[0..1], scale code sc) into two 16-byte rows.
__device__ __forceinline__ void fp4_decode_block(u32x2_t c, uint32_t sc, u32x4_t& lo, u32x4_t& hi) {
  const _Float16 s16 = (_Float16)e4m3_decode(sc);
  const f16x2_t S = {s16, s16};
  lo = (u32x4_t){fp4_pair<0>(c[0], S), fp4_pair<1>(c[0], S), fp4_pair<2>(c[0], S), fp4_pair<3>(c[0], S)};
  hi = (u32x4_t){fp4_pair<0>(c[1], S), fp4_pair<1>(c[1], S), fp4_pair<2>(c[1], S), fp4_pair<3>(c[1], S)};
}

// One workgroup per row of a bf16 matrix [rows][K]: codes [rows][K/2], block scales
// [rows][K/16] (either may be null), row scales [rows], and optionally the decoded
// values without the row scale, E2M1(code) * E4M3(S), exact in fp16 [rows][K].
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint16_t* __restrict__ src, int K,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ bscale,
                                                          float* __restrict__ rscale,
                                                          uint16_t* __restrict__ dec) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* in = src + row * K;
  const int nb = K / 16;
  float amax = 0.0f;
  for (int b = tid; b < nb; b += 256) {
    const u32x4_t u0 = *(const u32x4_t*)(in + 16 * b), u1 = *(const u32x4_t*)(in + 16 * b + 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(u0[q] & 0xffff))));
      amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(u0[q] >> 16))));
      amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(u1[q] & 0xffff))));
      amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(u1[q] >> 16))));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / 2688.0f : 0.0f;
  if (tid == 0) rscale[row] = s;
  for (int b = tid; b < nb; b += 256) {
    const u32x4_t u0 = *(const u32x4_t*)(in + 16 * b), u1 = *(const u32x4_t*)(in + 16 * b + 8);
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32((uint16_t)(u0[q] & 0xffff));
      v[2 * q + 1] = bf16_to_f32((uint16_t)(u0[q] >> 16));
      v[8 + 2 * q] = bf16_to_f32((uint16_t)(u1[q] & 0xffff));
      v[8 + 2 * q + 1] = bf16_to_f32((uint16_t)(u1[q] >> 16));
    }
    float bamax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) bamax = fmaxf(bamax, fabsf(v[i]));
    uint32_t sc = 0;
    float den = 0.0f;
    if (s > 0.0f) {
      sc = e4m3_encode((bamax / s) / 6.0f);
      den = e4m3_decode(sc) * s;
    }
    u32x2_t packed = {0u, 0u};
    if (den > 0.0f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) packed[i >> 3] |= e2m1_encode(v[i] / den) << (4 * (i & 7));
    }
    if (codes) *(u32x2_t*)(codes + row * (K / 2) + 8 * b) = packed;
    if (bscale) bscale[row * nb + b] = (uint8_t)sc;
    if (dec) {
      u32x4_t lo, hi;
      fp4_decode_block(packed, sc, lo, hi);
      *(u32x4_t*)(dec + row * K + 16 * b) = lo;
      *(u32x4_t*)(dec + row * K + 16 * b + 8) = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM on NVFP4 operands.  Tile 128 rows x 64 WN staged B rows, K steps of 64.
// The A rows (x per token, h per row) were quantized once and their decoded values
// (E2M1 * E4M3, exact in fp16) stored, so A stages as plain fp16; each thread stages
// one 16-element block of B (8 code bytes, one E4M3 scale byte) per pass and decodes it
// (v_cvt_scalef32_pk_f16_fp4 with scale 1, then the exact packed product with the
// block scale).  The MFMA loop and the tile order are those of the bf16 grouped GEMM; the
// row scales of A (staged per tile in LDS) and of B multiply the accumulator.
//   MODE 0: GEMM1: A = x rows gathered by perm (per-token scales), B = W1 and W3 in
//           alternating 32-row blocks; epilogue h = silu(a) g with a, g the accumulators
//           times the row scales of x and of the weight rows, rounded to bf16.
//   MODE 1: GEMM2: A = h rows (per-row scales), B = W2; out rounded to bf16.
// ---------------------------------------------------------------------------
constexpr int FP_BM = 128, FP_BK = 64, FP_LDS = FP_BK + 8;

struct Fp4Args {
  const uint16_t* a;       // decoded A rows (E2M1 * E4M3, exact fp16 bits) [rows][K]
  const float* ar;         // A row scales [rows]
  const int32_t* perm;     // MODE 0: A row of output row j is token perm[j] / k
  int T, k, E;
  long long Tk;
  const uint8_t* b0;       // MODE 0: W1 codes bank; MODE 1: W2
  const uint8_t* b1;       // MODE 0: W3
  const uint8_t* b0s;
  const uint8_t* b1s;
  const float* b0r;
  const float* b1r;
  const uint8_t* sb0;      // shared expert (may be null)
  const uint8_t* sb1;
  const uint8_t* sb0s;
  const uint8_t* sb1s;
  const float* sb0r;
  const float* sb1r;
  int K, N, NT;
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  int S;
  uint16_t* out;           // MODE 0: h [rows][N] bf16; MODE 1: out [rows][N] bf16
  int* flag;
};

__device__ __forceinline__ float fp4_silu(float a) { return a / (1.0f + expf(-a)); }

template <int MODE, int WN>
__global__ __launch_bounds__(128 * WN) __attribute__((amdgpu_waves_per_eu(WN >= 4 ? 4 : 1)))
void grouped_gemm_fp4_kernel(Fp4Args g) {
  constexpr int NTHR = 128 * WN;
  constexpr int BNW = 64 * WN;            // staged B rows
  constexpr int RPP = NTHR / 4;           // rows per pass (4 blocks of 16 per 64-wide step)
  constexpr int LA = FP_BM / RPP, LB = BNW / RPP;
  static_assert(LA >= 1 && LB >= 1, "tile");
  __shared__ __attribute__((aligned(16))) uint16_t sA[FP_BM * FP_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BNW * FP_LDS];
  __shared__ float sRs[FP_BM];            // A row scales of the tile's rows

  // ---- tile decode (as the bf16 grouped GEMM: XCD-contiguous, raster groups of 8) ----
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
  constexpr int GM = 8;
  const int grp = local / (GM * g.NT), rem = local % (GM * g.NT);
  const int gm = min(GM, mtiles - grp * GM);
  const int nt = rem / gm, mt = grp * GM + rem % gm;
  const int row0 = g.rowstart[s] + mt * FP_BM;
  const int mrows = min(FP_BM, g.rowcount[s] - mt * FP_BM);
  const int n0 = nt * (MODE == 0 ? BNW / 2 : BNW);
  const bool is_shared = (s == g.E);
  const long long e = is_shared ? 0 : s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = tid >> 2, lb = tid & 3;   // loader: rows lr + RPP i, block lb of the step
  const int K2 = g.K / 2, K16 = g.K / 16;

  // source rows (A row r >= mrows re-reads the tile's first row: it feeds no output)
  const uint16_t* arow[LA];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = lr + RPP * i;
    const long long j = (long long)row0 + (r < mrows ? r : 0);
    long long src = j;
    if (MODE == 0) {
      src = is_shared ? j - g.Tk : (long long)(g.perm[j] / g.k);
      if (src < 0 || src >= g.T) {
        bad = 1;
        src = 0;
      }
    }
    arow[i] = g.a + src * g.K + 16 * lb;
    if (lb == 0) sRs[r] = g.ar[src];
  }
  const uint8_t* bcode[LB];
  const uint8_t* bscale[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = lr + RPP * i;
    long long brow;
    const uint8_t *bank, *bsc;
    if (MODE == 0) {
      const int blk = r >> 5, within = r & 31;
      const bool w3 = blk & 1;
      bank = w3 ? (is_shared ? g.sb1 : g.b1) : (is_shared ? g.sb0 : g.b0);
      bsc = w3 ? (is_shared ? g.sb1s : g.b1s) : (is_shared ? g.sb0s : g.b0s);
      brow = (long long)n0 + (blk >> 1) * 32 + within;
    } else {
      bank = is_shared ? g.sb0 : g.b0;
      bsc = is_shared ? g.sb0s : g.b0s;
      brow = (long long)n0 + r;
    }
    bcode[i] = bank + (e * g.N + brow) * K2 + 8 * lb;
    bscale[i] = bsc + (e * g.N + brow) * K16 + lb;
  }
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  u32x4_t ra[LA][2];
  u32x2_t cb[LB];
  uint32_t sbv[LB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      ra[i][0] = *(const u32x4_t*)(arow[i] + k0);
      ra[i][1] = *(const u32x4_t*)(arow[i] + k0 + 8);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      cb[i] = *(const u32x2_t*)(bcode[i] + k0 / 2);
      sbv[i] = bscale[i][k0 / 16];
    }
  };
  gload(0);
  for (int k0 = 0; k0 < g.K; k0 += FP_BK) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      *(u32x4_t*)&sA[(lr + RPP * i) * FP_LDS + 16 * lb] = ra[i][0];
      *(u32x4_t*)&sA[(lr + RPP * i) * FP_LDS + 16 * lb + 8] = ra[i][1];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      u32x4_t l, h;
      fp4_decode_block(cb[i], sbv[i], l, h);
      *(u32x4_t*)&sB[(lr + RPP * i) * FP_LDS + 16 * lb] = l;
      *(u32x4_t*)&sB[(lr + RPP * i) * FP_LDS + 16 * lb + 8] = h;
    }
    __syncthreads();
    if (k0 + FP_BK < g.K) gload(k0 + FP_BK);
#pragma unroll
    for (int kk = 0; kk < FP_BK; kk += 16) {
      const int kc = kk + (lane >> 5) * 8;
      f16x8_t af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = __builtin_bit_cast(f16x8_t,
                                    *(const u32x4_t*)&sA[(wm * 64 + mb * 32 + (lane & 31)) * FP_LDS + kc]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bf[nb] = __builtin_bit_cast(f16x8_t,
                                    *(const u32x4_t*)&sB[(wn * 64 + nb * 32 + (lane & 31)) * FP_LDS + kc]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: accumulator element v is C[i][j], j = lane % 32,
  //      i = 8 (v / 4) + 4 (lane / 32) + v % 4; the output base of the lane's first
  //      row is formed once and rows step by a wave-uniform multiple of N ----
  const int j = lane & 31;
  const int rl = wm * 64 + 4 * (lane >> 5);
  const int c0 = n0 + wn * (MODE == 0 ? 32 : 64) + j;
  uint16_t* obase = g.out + ((long long)row0 + rl) * g.N + c0;
  float cs[2];   // weight row scales of the lane's columns
  if (MODE == 0) {
    cs[0] = (is_shared ? g.sb0r : g.b0r + e * g.N)[c0];
    cs[1] = (is_shared ? g.sb1r : g.b1r + e * g.N)[c0];
  } else {
    const float* r2 = is_shared ? g.sb0r : g.b0r + e * g.N;
    cs[0] = r2[c0];
    cs[1] = r2[c0 + 32];
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = mb * 32 + 8 * (v >> 2) + (v & 3);
      if (rl + i >= mrows) continue;
      const float as = sRs[rl + i];
      uint16_t* o = obase + (long long)i * g.N;
      if (MODE == 0) {
        const float a = acc[mb][0][v] * as * cs[0], gg = acc[mb][1][v] * as * cs[1];
        o[0] = f32_to_bf16(fp4_silu(a) * gg);
      } else {
        o[0] = f32_to_bf16(acc[mb][0][v] * as * cs[0]);
        o[32] = f32_to_bf16(acc[mb][1][v] * as * cs[1]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
moe_status nvfp4_quantize_rows(const uint16_t* src, long long rows, int K, uint8_t* codes, uint8_t* bscale,
                               float* rscale, uint16_t* dec, hipStream_t s) {
  if (rows <= 0) return MOE_OK;
  if (rows > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  nvfp4_quant_kernel<<<(unsigned)rows, 256, 0, s>>>(src, K, codes, bscale, rscale, dec);
  return launch_status();
}

moe_status nvfp4_gemm(int mode, const Nvfp4Gemm& q, hipStream_t s) {
  Fp4Args g{};
  g.a = q.a;
  g.ar = q.ar;
  g.perm = q.perm;
  g.T = q.T;
  g.k = q.k;
  g.E = q.E;
  g.Tk = (long long)q.T * q.k;
  g.b0 = q.b0;
  g.b1 = q.b1;
  g.b0s = q.b0s;
  g.b1s = q.b1s;
  g.b0r = q.b0r;
  g.b1r = q.b1r;
  g.sb0 = q.sb0;
  g.sb1 = q.sb1;
  g.sb0s = q.sb0s;
  g.sb1s = q.sb1s;
  g.sb0r = q.sb0r;
  g.sb1r = q.sb1r;
  g.K = q.K;
  g.N = q.N;
  g.mstart = q.mstart;
  g.rowstart = q.rowstart;
  g.rowcount = q.rowcount;
  g.S = q.S;
  g.out = q.out;
  g.flag = q.flag;
  constexpr int WN = 4;
  g.NT = mode == 0 ? q.N / (32 * WN) : q.N / (64 * WN);
  const long long grid = tile_grid(q.mt_bound * g.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (grid == 0) return MOE_OK;
  if (mode == 0)
    grouped_gemm_fp4_kernel<0, WN><<<(unsigned)grid, 128 * WN, 0, s>>>(g);
  else
    grouped_gemm_fp4_kernel<1, WN><<<(unsigned)grid, 128 * WN, 0, s>>>(g);
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_nvfp4_quantize(const void* src, int rows, int K, uint8_t* codes,
                                         uint8_t* block_scales, float* row_scales, void* stream) {
  if (rows < 0 || K < 16 || K % 16 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!src || !codes || !block_scales || !row_scales || !aligned(src, 16) || !aligned(codes, 8))
    return MOE_ERR_INVALID_ARG;
  return nvfp4_quantize_rows((const uint16_t*)src, rows, K, codes, block_scales, row_scales, nullptr,
                             (hipStream_t)stream);
}
