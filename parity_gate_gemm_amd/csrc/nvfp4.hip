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
// Grouped GEMM on NVFP4 operands.  The A rows (x per token, h per row) were quantized
// once and their decoded values (E2M1 * E4M3, exact in fp16) stored; B (the weights)
// stays NVFP4 and is decoded in registers right before the MFMA.
//
// Tile: 128 rows x 8 wavefronts; each wavefront owns all 128 rows and 64 B rows as
// 4 x 2 MFMA 32x32x16 blocks (128 accumulators, two wavefronts per SIMD).  GEMM1: the
// wavefront's two column blocks are W1 and W3 of the same 32 features (256 features per
// tile); GEMM2: 64 output columns (512 per tile).  K advances in steps of 64.
//
// K order inside a step: lane half hf (= lane / 32) supplies, at MFMA iteration it, the
// step's elements 32 hf + 8 it .. + 7 (for A and B alike, so the dot product is the same
// sum).  A lane's B codes for a step are then 16 contiguous bytes of its row, and its
// block scales bytes 2 hf and 2 hf + 1 of the row's 4 scale bytes of the step.
//
// The weights are K-blocked (moe_nvfp4_pack_weights): the codes of 32 rows x 64 columns
// are one contiguous 1 KB tile (32 bytes per row) and their block scales one 128-byte
// tile, so a wavefront's B for one step and one block column is one 1 KB and one
// 128-byte contiguous read.
//
// Every operand goes through a 4-stage LDS ring filled by global_load_lds (lane l writes
// its 16 or 4 bytes at base + 16 l or base + 4 l): A rows with chunk c of row r in slot
// c ^ swz(r); the B codes each lane reads, in lane order (one 1 KB block per block
// column); the B scale words likewise.  B is read only by the wavefront that loads it.
// Step i waits for its own loads (vmcnt), passes a barrier (every wavefront's loads
// landed, every wavefront done with the stage to be refilled), then issues step i + 3's
// loads and multiplies.  The row scales of A (staged in LDS) and of B multiply the fp32
// accumulators in the epilogue.
//   MODE 0: GEMM1, A = x rows gathered by perm; h = bf16(silu(a) g), a and g the W1 and
//           W3 accumulators times the row scales of x and of the weight rows.
//   MODE 1: GEMM2, A = h rows; out = bf16(accumulator times the two row scales).
// ---------------------------------------------------------------------------
constexpr int FP_BM = 128, FP_BK = 64, FP_NW = 8;
constexpr int FP_SB = FP_BM * FP_BK * 2;          // B codes: 2 KB per wavefront
constexpr int FP_SS = FP_SB + FP_NW * 2048;       // B scale words: 512 B per wavefront
constexpr int FP_STAGE = FP_SS + FP_NW * 512;     // bytes of one stage
constexpr int FP_NST = 4;                         // ring stages (loads run FP_NST - 1 steps ahead)

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
  float* out_pre;          // MODE 0 (optional): a | g [rows][2N] for the backward pass
  int* flag;
};


__device__ __forceinline__ int fp4_swz(int r) { return (r ^ (r >> 3)) & 7; }

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void fp4_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// B fragment of MFMA iteration IT: codes word IT times its block's scale (fp16 pair).
template <int IT>
__device__ __forceinline__ f16x8_t fp4_bfrag(const u32x4_t& c, f16x2_t S0, f16x2_t S1) {
  const f16x2_t S = IT < 2 ? S0 : S1;
  const uint32_t w = c[IT];
  const u32x4_t r = {fp4_pair<0>(w, S), fp4_pair<1>(w, S), fp4_pair<2>(w, S), fp4_pair<3>(w, S)};
  return __builtin_bit_cast(f16x8_t, r);
}

template <int MODE>
__global__ __launch_bounds__(64 * FP_NW) __attribute__((amdgpu_waves_per_eu(2)))
void grouped_gemm_fp4_kernel(Fp4Args g) {
  constexpr int CW = MODE == 0 ? 32 : 64;   // output columns (GEMM1: features) per wavefront
  constexpr int LA = FP_BM / (8 * FP_NW);   // 1 KB A loads per wavefront per step
  static_assert(LA * 8 * FP_NW == FP_BM, "loader shape");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[FP_NST * FP_STAGE];
  __shared__ float sRs[FP_BM];            // A row scales of the tile's rows

  // ---- tile decode (XCD-contiguous, raster groups of 8 row tiles) ----
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
  const bool is_shared = (s == g.E);
  const long long e = is_shared ? 0 : s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int c0 = nt * (FP_NW * CW) + wave * CW;   // first output column of the wavefront
  const bool active = c0 < g.N;                    // wavefront-uniform

  // ---- A source rows (a tile row r >= mrows re-reads the tile's first row: it feeds
  //      no output) ----
  auto a_src = [&](int r, int& bad) -> long long {
    const long long j = (long long)row0 + (r < mrows ? r : 0);
    if (MODE == 1) return j;
    long long src = is_shared ? j - g.Tk : (long long)(g.perm[j] / g.k);
    if (src < 0 || src >= g.T) {
      bad = 1;
      src = 0;
    }
    return src;
  };
  int bad = 0;
  const uint16_t* aptr[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = 8 * (wave * LA + i) + (lane >> 3);
    const int chunk = (lane & 7) ^ fp4_swz(r);
    aptr[i] = g.a + a_src(r, bad) * g.K + chunk * 8;
  }
  if (tid < FP_BM) sRs[tid] = g.ar[a_src(tid, bad)];
  if (bad) raise_flag(g.flag, kFlagCorrupt);

  // ---- B rows of this lane: block column nb, rows c0 (+ 32 nb) .. + 31, row l32 of
  //      the 32-row group; K-blocked tiles (1 KB of codes, 128 B of scales per step) ----
  const int K2 = g.K / 2, K16 = g.K / 16, KS = g.K / FP_BK;
  const uint8_t* bc[2];   // the lane's 16 code bytes of step 0
  const uint8_t* bs[2];   // the row's 4 scale bytes of step 0
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint8_t *bank, *bsc;
    int brow;
    if (MODE == 0) {
      bank = nb ? (is_shared ? g.sb1 : g.b1) : (is_shared ? g.sb0 : g.b0);
      bsc = nb ? (is_shared ? g.sb1s : g.b1s) : (is_shared ? g.sb0s : g.b0s);
      brow = c0;
    } else {
      bank = is_shared ? g.sb0 : g.b0;
      bsc = is_shared ? g.sb0s : g.b0s;
      brow = c0 + 32 * nb;
    }
    if (!active) brow = 0;   // loads stay in bounds; nothing is computed from them
    const long long grp = brow / 32;   // brow is a multiple of 32
    bc[nb] = bank + e * g.N * K2 + grp * KS * 1024 + 32 * l32 + 16 * hf;
    bs[nb] = bsc + e * g.N * K16 + grp * KS * 128 + 4 * l32;
  }

  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue = [&](uint8_t* st, int k0) {
#if defined(__HIP_DEVICE_COMPILE__)   // a gfx950 builtin: device pass only
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds(aptr[i] + k0, (lds_ptr)(st + (wave * LA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      __builtin_amdgcn_global_load_lds(bc[nb] + k0 * 16, (lds_ptr)(st + FP_SB + (2 * wave + nb) * 1024), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(bs[nb] + k0 * 2, (lds_ptr)(st + FP_SS + (2 * wave + nb) * 256), 4, 0,
                                       0);
    }
#endif
  };
  constexpr int kLoads = LA + 4;   // load instructions per wavefront per step

  // ---- A fragment offsets: row 32 mb + l32, chunk 4 hf + it.  swz(32 mb + l32) is
  //      swz(l32) ^ (4 mb & 7), so blocks mb and mb + 2 share the slot, 8 KB apart. ----
  uint32_t aof[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int ra = 32 * mb + l32;
#pragma unroll
    for (int it = 0; it < 4; ++it) aof[mb][it] = ra * 128 + (((4 * hf + it) ^ fp4_swz(ra)) << 4);
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // The A fragment reads are inline assembly whose results pass through a separate
  // lgkmcnt(0) wait (tied by in-out operands), so that the compiler neither waits for
  // the other stages' outstanding global->LDS loads nor uses a fragment before it lands;
  // the next iteration's reads are in flight during this iteration's MFMAs.
  auto aread = [&](uint32_t st, int it, u32x4_t* f) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %4 offset:8192\n\t"
        "ds_read_b128 %3, %5 offset:8192"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(st + aof[0][it]), "v"(st + aof[1][it]));
  };
  auto await = [&](u32x4_t* f) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]));
  };
  const uint32_t bof = FP_SB + wave * 2048 + 16 * lane, sof = FP_SS + wave * 512 + 4 * lane;
  const int sshift = 16 * hf;   // the lane's two scale bytes in the row's scale word
  // nmb: the A blocks of 32 rows that hold tile rows (1 .. 4, workgroup-uniform); the
  // MFMAs of the others (rows past the segment's end) are skipped.
  const int nmb = (mrows + 31) / 32;
  auto compute = [&](uint32_t st) {
    u32x4_t bcode[2];
    uint32_t bsw[2];
    u32x4_t fa[2][4];
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b32 %2, %5\n\t"
        "ds_read_b32 %3, %5 offset:256"
        : "=&v"(bcode[0]), "=&v"(bcode[1]), "=&v"(bsw[0]), "=&v"(bsw[1])
        : "v"(st + bof), "v"(st + sof));
    aread(st, 0, fa[0]);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bcode[0]), "+v"(bcode[1]), "+v"(bsw[0]), "+v"(bsw[1]));
    await(fa[0]);
    f16x2_t S[2][2];   // [nb][block] fp16 scale pairs
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)(bsw[nb] >> sshift), false);
      const _Float16 s0 = (_Float16)f[0], s1 = (_Float16)f[1];
      S[nb][0] = (f16x2_t){s0, s0};
      S[nb][1] = (f16x2_t){s1, s1};
    }
    // B fragments one iteration ahead; scheduling fences keep iteration it's MFMAs
    // between the issue of iteration it + 1's A reads and the wait for them, so the
    // LDS latency hides behind the MFMAs.
    auto bdecode = [&](int it, f16x8_t* fb) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (it == 0) fb[nb] = fp4_bfrag<0>(bcode[nb], S[nb][0], S[nb][1]);
        if (it == 1) fb[nb] = fp4_bfrag<1>(bcode[nb], S[nb][0], S[nb][1]);
        if (it == 2) fb[nb] = fp4_bfrag<2>(bcode[nb], S[nb][0], S[nb][1]);
        if (it == 3) fb[nb] = fp4_bfrag<3>(bcode[nb], S[nb][0], S[nb][1]);
      }
    };
    f16x8_t fb[2][2];
    bdecode(0, fb[0]);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (it + 1 < 4) aread(st, it + 1, fa[(it + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (it + 1 < 4) bdecode(it + 1, fb[(it + 1) & 1]);
      const u32x4_t* f = fa[it & 1];
      // f = {A block 0, 1, 2, 3} (blocks 2 and 3 read 8 KB past blocks 0 and 1)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb > 0 && nmb <= mb) break;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, f[mb]),
                                                               fb[it & 1][nb], acc[mb][nb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (it + 1 < 4) await(fa[(it + 1) & 1]);
    }
  };

  // ---- K loop over the ring; step i lives in stage i % FP_NST ----
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t lring = (uint32_t)(uintptr_t)(lds_u8*)ring;
  const int nsteps = g.K / FP_BK;
#pragma unroll
  for (int p = 0; p < FP_NST - 1; ++p)
    if (p < nsteps) issue(ring + p * FP_STAGE, p * FP_BK);
  int scur = 0;   // stage of step i
  for (int i = 0; i < nsteps; ++i) {
    // steps i + 1 .. i + FP_NST - 2 may keep their loads outstanding
    static_assert(FP_NST == 4, "wait counts below");
    if (i + 2 < nsteps)
      fp4_wait_vmcnt<2 * kLoads>();
    else if (i + 1 < nsteps)
      fp4_wait_vmcnt<kLoads>();
    else
      fp4_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const int snext = scur == 0 ? FP_NST - 1 : scur - 1;   // stage of step i + FP_NST - 1
    if (i + FP_NST - 1 < nsteps) issue(ring + snext * FP_STAGE, (i + FP_NST - 1) * FP_BK);
    if (active) compute(lring + scur * FP_STAGE);
    scur = scur == FP_NST - 1 ? 0 : scur + 1;
  }
  if (!active) return;

  // ---- epilogue: accumulator element v of block (mb, nb) is row 32 mb + 8 (v / 4) +
  //      4 hf + v % 4, column l32 of the block ----
  const int rl = 4 * hf;
  uint16_t* obase = g.out + ((long long)row0 + rl) * g.N + c0 + l32;
  float cs[2];   // weight row scales of the lane's columns
  if (MODE == 0) {
    cs[0] = (is_shared ? g.sb0r : g.b0r + e * g.N)[c0 + l32];
    cs[1] = (is_shared ? g.sb1r : g.b1r + e * g.N)[c0 + l32];
  } else {
    const float* r2 = is_shared ? g.sb0r : g.b0r + e * g.N;
    cs[0] = r2[c0 + l32];
    cs[1] = r2[c0 + 32 + l32];
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = mb * 32 + 8 * (v >> 2) + (v & 3);
      if (rl + i >= mrows) continue;
      const float as = sRs[rl + i];
      uint16_t* o = obase + (long long)i * g.N;
      if (MODE == 0) {
        const float a = acc[mb][0][v] * as * cs[0], gg = acc[mb][1][v] * as * cs[1];
        o[0] = f32_to_bf16(silu_f32(a) * gg);
        if (g.out_pre) {   // pre-activations for the backward pass
          float* pr = g.out_pre + ((long long)row0 + rl + i) * 2 * g.N + c0 + l32;
          pr[0] = a;
          pr[g.N] = gg;
        }
      } else {
        o[0] = f32_to_bf16(acc[mb][0][v] * as * cs[0]);
        o[32] = f32_to_bf16(acc[mb][1][v] * as * cs[1]);
      }
    }
  }
}

// h = bf16(silu(a) g) from the saved pre-activations, the GEMM1 epilogue's arithmetic.
__global__ __launch_bounds__(256) void nvfp4_h_from_pre_kernel(const float* __restrict__ pre, long long n,
                                                               int I, uint16_t* __restrict__ h) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const long long r = idx / I;
  const int c = (int)(idx % I);
  const float a = pre[r * 2 * I + c], gg = pre[r * 2 * I + I + c];
  h[idx] = f32_to_bf16(silu_f32(a) * gg);
}

// ---------------------------------------------------------------------------
// K-blocking of NVFP4 weight matrices (row-major codes [R][K/2] and block scales
// [R][K/16] -> tiles of 32 rows x 64 columns: codes [R/32][K/64][32][32 bytes],
// scales [R/32][K/64][32][4 bytes]).  One thread per 16-byte piece of the codes
// (and, for the first half of a row's tile bytes, its 4 scale bytes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nvfp4_pack_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, long long total,
                                                         int R, int K, uint8_t* __restrict__ pc,
                                                         uint8_t* __restrict__ ps) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;   // destination 16-byte piece
  if (q >= total) return;
  const int KS = K / FP_BK;
  const int half = (int)(q & 1), r = (int)((q >> 1) & 31);
  const long long tile = q >> 6;                 // (matrix, group, step) in order
  const int step = (int)(tile % KS);
  const long long mg = tile / KS;                // matrix * (R / 32) + group
  const long long row = mg * 32 + r;             // row over all matrices (R % 32 == 0)
  *(u32x4_t*)(pc + q * 16) = *(const u32x4_t*)(codes + row * (K / 2) + step * 32 + half * 16);
  if (half == 0) *(uint32_t*)(ps + tile * 128 + r * 4) = *(const uint32_t*)(scales + row * (K / 16) + step * 4);
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

moe_status nvfp4_h_from_pre(const float* pre, long long rows, int I, uint16_t* h, hipStream_t s) {
  const long long n = rows * I;
  if (n <= 0) return MOE_OK;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  nvfp4_h_from_pre_kernel<<<(unsigned)blocks, 256, 0, s>>>(pre, n, I, h);
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
  g.out_pre = q.out_pre;
  g.flag = q.flag;
  // columns per tile: 8 wavefronts x 32 features (GEMM1) or x 64 columns (GEMM2)
  const int per = FP_NW * (mode == 0 ? 32 : 64);
  if (q.N % (mode == 0 ? 32 : 64) != 0 || q.K % FP_BK != 0 || q.K < FP_BK) return MOE_ERR_UNSUPPORTED;
  g.NT = (q.N + per - 1) / per;
  const long long grid = tile_grid(q.mt_bound * g.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (grid == 0) return MOE_OK;
  if (mode == 0)
    grouped_gemm_fp4_kernel<0><<<(unsigned)grid, 64 * FP_NW, 0, s>>>(g);
  else
    grouped_gemm_fp4_kernel<1><<<(unsigned)grid, 64 * FP_NW, 0, s>>>(g);
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

extern "C" moe_status moe_nvfp4_pack_weights(const uint8_t* codes, const uint8_t* block_scales, int n, int R,
                                             int K, uint8_t* packed_codes, uint8_t* packed_scales,
                                             void* stream) {
  if (n < 0 || R < 0 || K < 0 || R % 32 != 0 || K % FP_BK != 0) return MOE_ERR_INVALID_ARG;
  if (n == 0 || R == 0 || K == 0) return MOE_OK;
  if (!codes || !block_scales || !packed_codes || !packed_scales || !aligned(codes, 16) ||
      !aligned(packed_codes, 16) || !aligned(block_scales, 4) || !aligned(packed_scales, 4))
    return MOE_ERR_INVALID_ARG;
  const long long code_bytes = (long long)n * R * (K / 2), scale_bytes = (long long)n * R * (K / 16);
  const uintptr_t c0 = (uintptr_t)codes, c1 = c0 + code_bytes, s0 = (uintptr_t)block_scales,
                  s1 = s0 + scale_bytes, p0 = (uintptr_t)packed_codes, p1 = p0 + code_bytes,
                  q0 = (uintptr_t)packed_scales, q1 = q0 + scale_bytes;
  auto overlap = [](uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; };
  if (overlap(p0, p1, c0, c1) || overlap(p0, p1, s0, s1) || overlap(q0, q1, c0, c1) || overlap(q0, q1, s0, s1) ||
      overlap(p0, p1, q0, q1))
    return MOE_ERR_INVALID_ARG;
  const long long total = code_bytes / 16;
  const long long grid = (total + 255) / 256;
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  nvfp4_pack_kernel<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(codes, block_scales, total, R, K,
                                                                     packed_codes, packed_scales);
  return launch_status();
}
