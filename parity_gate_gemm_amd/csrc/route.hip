// Routing: gate GEMM, top-k selection, softmax-renormalised weights, router replay.
//
// The gate picks the top-k experts per token (Training Data podcast page "How Cursor
// Trained Composer on Fireworks", section on floating point and MoE: 8 of 384 experts
// per layer, and a fifth-decimal difference in the hidden state can flip the choice).
// Replay overrides the choice with IDs from inference while the gate scores are still
// computed (Composer 2 Technical Report, section 6.2, paragraph on inference and
// weight sync).
//
// Because a flipped expert changes the whole path, selection here is exact: it equals
// the selection made on the correctly rounded logits.  The gate GEMM runs in fp64
// with a fixed summation order; a rigorous bound on its rounding error certifies the
// top-(k+1) ordering of almost every token, and the rare token it cannot certify
// (exact ties, near-ties) is recomputed with error-free (expansion) summation and
// rounded once.  Weights always come from the fp64 GEMM logits through one device
// function, so learned routing and replay of its own IDs give identical bits.
#include <math.h>

#include "moe_internal.h"

namespace moe {

constexpr int GT_M = 64;   // tokens per gate tile
constexpr int GT_E = 32;   // experts per gate tile
constexpr int GT_K = 64;   // reduction step staged in LDS

typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

// Raw registers of one thread's 16 consecutive activations of one token, per dtype.
template <int DT>
struct XChunk;
template <>
struct XChunk<MOE_BF16> {
  u32x4_v r[2];
  __device__ void load(const void* x, const uint8_t*, size_t row, int d, int k) {
    const u32x4_v* p = (const u32x4_v*)((const uint16_t*)x + row * d + k);
    r[0] = p[0];
    r[1] = p[1];
  }
  __device__ void zero() { r[0] = r[1] = (u32x4_v){0, 0, 0, 0}; }
  __device__ double get(int i) const {
    const uint32_t w = r[i >> 3][(i >> 1) & 3];
    return (double)bf16_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffff)));
  }
};
template <>
struct XChunk<MOE_F32> {
  f32x4_v r[4];
  __device__ void load(const void* x, const uint8_t*, size_t row, int d, int k) {
    const f32x4_v* p = (const f32x4_v*)((const float*)x + row * d + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = p[i];
  }
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (f32x4_v){0.f, 0.f, 0.f, 0.f};
  }
  __device__ double get(int i) const { return (double)r[i >> 2][i & 3]; }
};
template <>
struct XChunk<MOE_MXFP8> {
  u32x4_v r;
  double scale;
  __device__ void load(const void* x, const uint8_t* xs, size_t row, int d, int k) {
    r = *(const u32x4_v*)((const uint8_t*)x + row * d + k);
    scale = e8m0_to_f64(xs[row * (size_t)(d / 32) + k / 32]);   // 16 codes lie in one 32-block
  }
  __device__ void zero() {
    r = (u32x4_v){0, 0, 0, 0};
    scale = 0.0;
  }
  __device__ double get(int i) const {
    return e4m3_to_f64((uint8_t)(r[i >> 2] >> (8 * (i & 3)))) * scale;
  }
};

// logits[t][e] = sum_i x[t][i] * wg[i][e]  (+ bias[e]) in fp64 on the matrix cores
// (v_mfma_f64_16x16x4f64), K ascending in steps of 4; the bias is added last.  Every
// product is exact in fp64 and every addition rounds once, so the rounding error of
// each output is at most gamma_{d+1} * (sum_i |x_i w_ie| + |b_e|)
//                    <= gamma_{d+1} * (||x_t|| ||w_e|| + |b_e|).
// The workgroups of the first expert tile also write ||x_t||, those of the first
// token tile ||w_e|| (fp64 sums of squares in a fixed order).
// 256 threads = 4 wavefronts; wavefront w owns tokens 16w..16w+15 of the tile and all
// 32 experts as two 16x16 MFMA blocks.  Loads of the next K-step are in flight while
// the current one is multiplied.  Requires d % 16 == 0.
template <int DT>
__global__ __launch_bounds__(256) void gate_gemm_f64_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int T, int d,
    const float* __restrict__ wg, const float* __restrict__ bias, int E,
    double* __restrict__ logits, double* __restrict__ xnorm, double* __restrict__ wnorm) {
  __shared__ double sx[GT_M][GT_K + 1];
  __shared__ double sw[GT_K][GT_E + 1];
  __shared__ double wpart[4][GT_E];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.y * GT_M, e0 = blockIdx.x * GT_E;
  const int xm = tid >> 2, xk = (tid & 3) * 16;   // x loader: token xm, k xk..xk+15
  const int wk = tid >> 2, we = (tid & 3) * 8;    // w loader: k row wk, experts we..we+7
  const bool x_row_ok = t0 + xm < T;
  const bool need_xn = blockIdx.x == 0, need_wn = blockIdx.y == 0;

  f64x4_t acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = 0.0;
  double xsq = 0.0, wsq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wsq[j] = 0.0;

  XChunk<DT> xc;
  float wv[8];
  auto gload = [&](int k0) {
    if (x_row_ok && k0 + xk < d) xc.load(x, xs, (size_t)(t0 + xm), d, k0 + xk);
    else xc.zero();
    const int kw = k0 + wk;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + we + j;
      wv[j] = (kw < d && e < E) ? wg[(size_t)kw * E + e] : 0.0f;
    }
  };
  gload(0);
  for (int k0 = 0; k0 < d; k0 += GT_K) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double v = xc.get(i);
      sx[xm][xk + i] = v;
      if (need_xn) xsq = fma(v, v, xsq);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double v = (double)wv[j];
      sw[wk][we + j] = v;
      if (need_wn) wsq[j] = fma(v, v, wsq[j]);
    }
    __syncthreads();
    if (k0 + GT_K < d) gload(k0 + GT_K);
    // A operand: lane holds x[16*wave + lane%16][k + lane/16]; B: w[k + lane/16][16*nb + lane%16].
#pragma unroll
    for (int kk = 0; kk < GT_K; kk += 4) {
      const double a = sx[16 * wave + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const double b = sw[kk + (lane >> 4)][16 * nb + (lane & 15)];
        acc[nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // Norms: the four x-loader threads of a token hold its partial sums (k strided by
  // chunk), the 64 w-loader threads of an expert chunk hold per-k-row partials.
  if (need_xn) {
    const double s1 = xsq + __shfl_xor(xsq, 1);
    const double s2 = s1 + __shfl_xor(s1, 2);
    if ((tid & 3) == 0 && x_row_ok) xnorm[t0 + xm] = sqrt(s2);
  }
  if (need_wn) {
    // Reduce over the 16 k rows of each wavefront (lanes with equal lane%4), then
    // over the 4 wavefronts, in a fixed order.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double v = wsq[j];
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) v += __shfl_xor(v, off);
      wsq[j] = v;
    }
    if (lane < 4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) wpart[wave][we + j] = wsq[j];
    }
    __syncthreads();
    if (tid < GT_E && e0 + tid < E)
      wnorm[e0 + tid] = sqrt(((wpart[0][tid] + wpart[1][tid]) + wpart[2][tid]) + wpart[3][tid]);
  }
  // D layout of a 16x16 fp64 block: element i of a lane is row lane/16 + 4*i, column
  // lane%16 (interleaved, unlike the fp32 16x16 layouts).
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int e = e0 + 16 * nb + (lane & 15);
    if (e >= E) continue;
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * wave + (lane >> 4) + 4 * i;
      if (t >= T) continue;
      double v = acc[nb][i];
      if (bias) v = v + b;
      logits[(size_t)t * E + e] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// The same fp64 gate GEMM staged through a three-stage LDS ring that direct
// global->LDS loads fill (global_load_lds_dwordx4: lane l of a wavefront writes its 16
// bytes at base + 16 l), used whenever E % 4 == 0.  Activations stay in their stored
// format in LDS and are widened to fp64 as the MFMA operands are read; two K-steps of
// loads are in flight while a third is multiplied.
// Reduction order: for every logit, the K range is cut into S = gate_splits(d) equal
// parts; each part is a chain of v_mfma_f64_16x16x4f64 from zero over its 16-wide
// chunks in ascending order, where MFMA m (0..3) of a chunk at c sums the products at
// c + m, c + 4 + m, c + 8 + m, c + 12 + m; the parts are added in ascending order and
// the bias last.  A workgroup either runs all S parts itself or, for small batches,
// one part whose partial sum gate_finish_kernel adds in the same order: the bits do
// not depend on which.  Every sum still has at most d + 1 rounded additions, so the
// error bound of gate_gemm_f64_kernel holds.
// Stage layout: 64 activation rows of 64 elements, then 64 rows (k) of the 32 experts'
// fp32 weights (128 B).  A 16-byte chunk c of activation row r sits in slot
// c ^ (r & min(7, slots - 1)); weight chunk c of row k in slot c ^ (4 * ((k >> 2) & 1)),
// so the lanes of one LDS read phase meet distinct banks (the activation read keeps a
// 2-way conflict: 16 rows share 8 slots).
// ---------------------------------------------------------------------------
constexpr int GD_STAGES = 3;

template <int DT>
struct GateStage;   // bytes of one activation row's 64-element step
template <>
struct GateStage<MOE_BF16> { static constexpr int RB = 128; };
template <>
struct GateStage<MOE_F32> { static constexpr int RB = 256; };
template <>
struct GateStage<MOE_MXFP8> { static constexpr int RB = 64; };

// One lane's LDS reads for a 16-wide chunk of the ring gate kernel: its four
// activations (8, 16 or 4 bytes at xa) and the weights of its k rows for two 16-expert
// blocks (4 rows, 128 bytes apart, at wa0 and at wa1).  Issued from inline assembly
// with their own lgkmcnt(0) wait, so that the compiler does not tie them to the
// outstanding global->LDS loads of the other ring stages (it would wait for all of
// them); the K loop's vmcnt wait and barrier order them against those loads.
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));
#define MOE_GATE_WREADS                                                                      \
  "ds_read_b32 %1, %9\n\tds_read_b32 %2, %9 offset:128\n\tds_read_b32 %3, %9 offset:256\n\t" \
  "ds_read_b32 %4, %9 offset:384\n\tds_read_b32 %5, %10\n\tds_read_b32 %6, %10 offset:128\n\t" \
  "ds_read_b32 %7, %10 offset:256\n\tds_read_b32 %8, %10 offset:384\n\ts_waitcnt lgkmcnt(0)"
#define MOE_GATE_OUTS(X)                                                                       \
  : "=&v"(X), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), \
    "=&v"(w[6]), "=&v"(w[7])                                                                   \
  : "v"(wa0), "v"(wa1), "v"(xa)
template <int DT>
__device__ __forceinline__ void gate_lds_reads(uint32_t xa, uint32_t wa0, uint32_t wa1, uint32_t sa,
                                               u32x4_v& x, uint32_t (&w)[8]) {
  if constexpr (DT == MOE_F32) {
    asm volatile("ds_read_b128 %0, %11\n\t" MOE_GATE_WREADS MOE_GATE_OUTS(x));
  } else if constexpr (DT == MOE_BF16) {
    u32x2_v v;
    asm volatile("ds_read_b64 %0, %11\n\t" MOE_GATE_WREADS MOE_GATE_OUTS(v));
    x[0] = v[0];
    x[1] = v[1];
  } else {   // MXFP8: four E4M3 codes, and the E8M0 scale byte of their block at sa
    uint32_t v, sc;
    asm volatile(
        "ds_read_b32 %0, %12\n\tds_read_u8 %9, %13\n\t"
        "ds_read_b32 %1, %10\n\tds_read_b32 %2, %10 offset:128\n\tds_read_b32 %3, %10 offset:256\n\t"
        "ds_read_b32 %4, %10 offset:384\n\tds_read_b32 %5, %11\n\tds_read_b32 %6, %11 offset:128\n\t"
        "ds_read_b32 %7, %11 offset:256\n\tds_read_b32 %8, %11 offset:384\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]),
          "=&v"(w[6]), "=&v"(w[7]), "=&v"(sc)
        : "v"(wa0), "v"(wa1), "v"(xa), "v"(sa));
    x[0] = v;
    x[1] = sc;
  }
}
#undef MOE_GATE_OUTS
#undef MOE_GATE_WREADS

struct GateArgs {
  const uint8_t* x;        // activations (bytes)
  const uint8_t* xs;       // MXFP8 scales [T][d/32]
  int T, d, E;
  const float* wg;         // [d][E], 16-byte aligned, E % 4 == 0
  const float* bias;       // [E] or null
  int ks;                  // elements per K part (d / S)
  int spw;                 // K parts per workgroup (S, or 1 when split over gridDim.z)
  double* logits;          // [T][E] final (gridDim.z == 1)
  double* part;            // [z][T][E] partial sums (gridDim.z > 1)
  double* xnorm;           // ||x_t|| (gridDim.z == 1) or partial squares [z][T]
  double* wnorm;           // ||w_e|| (gridDim.z == 1) or partial squares [z][E]
};

template <int N>
__device__ __forceinline__ void gate_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DT>
__global__ __launch_bounds__(256) void gate_gemm_f64_ring_kernel(GateArgs g) {
  constexpr int RB = GateStage<DT>::RB;
  constexpr int EB = RB / 64;                  // bytes per activation element
  constexpr int SPR = RB / 16;                 // 16-byte slots per activation row
  constexpr int XSW = SPR < 8 ? SPR - 1 : 7;   // activation slot swizzle mask
  constexpr int RPI = 1024 / RB;               // activation rows per 1 KB load
  constexpr int NXA = GT_M / RPI / 4;          // activation loads per wavefront per step
  constexpr int NWA = 2;                       // weight loads per wavefront per step
  constexpr int XB = GT_M * RB;
  constexpr int STAGE = XB + GT_K * 128;
  constexpr int PER_STEP = NXA + NWA;
  static_assert(NXA * 4 * RPI == GT_M && GT_K * 128 == NWA * 4 * 1024, "loader shape");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.x * GT_E, t0 = blockIdx.y * GT_M, z = blockIdx.z;
  const int nss = (g.ks + GT_K - 1) / GT_K;    // steps per K part
  const int nsteps = g.spw * nss;
  const int part0 = z * g.spw;
  const size_t xrow = (size_t)g.d * EB;

  // ---- loader addresses (byte offsets without the step's K offset) ----
  size_t xo[NXA];
  int xk[NXA];   // element offset of the chunk within a step
#pragma unroll
  for (int i = 0; i < NXA; ++i) {
    const int r = (wave * NXA + i) * RPI + lane / SPR;
    const int ch = (lane % SPR) ^ (r & XSW);
    const int t = t0 + r < g.T ? t0 + r : 0;
    xo[i] = (size_t)t * xrow + (size_t)ch * 16;
    xk[i] = ch * 16 / EB;
  }
  size_t wo[NWA];
  int wr[NWA];
  bool wok[NWA];
#pragma unroll
  for (int i = 0; i < NWA; ++i) {
    const int kr = (wave * NWA + i) * 8 + lane / 8;
    const int slot = (lane % 8) ^ (((kr >> 2) & 1) << 2);
    const int e = e0 + 4 * slot;
    wok[i] = e < g.E;
    wo[i] = (size_t)kr * g.E + e;
    wr[i] = kr;
  }
  // the activation row this lane reads
  const int rr = 16 * wave + (lane & 15), j = lane >> 4;
  // MXFP8: the E8M0 scales of the tile's 64 rows over this workgroup's K range, staged
  // once in LDS (row r at sscale + r * nkb) before the ring starts
  extern __shared__ uint8_t sscale[];
  const int nkb = DT == MOE_MXFP8 ? g.spw * g.ks / 32 : 0;
  if (DT == MOE_MXFP8) {
    const int nb32 = g.d / 32, kb0 = part0 * g.ks / 32;
    for (int q = tid; q < GT_M * nkb; q += 256) {
      const int r = q / nkb, c = q % nkb;
      const int t = t0 + r < g.T ? t0 + r : 0;
      sscale[q] = g.xs[(size_t)t * nb32 + kb0 + c];
    }
    __syncthreads();
  }

  typedef __attribute__((address_space(3))) void* lds_ptr;
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  auto kbase = [&](int i) { return (part0 + i / nss) * g.ks + (i % nss) * GT_K; };
  auto issue = [&](uint8_t* st, int i) {
    const int k0 = kbase(i), loc = (i % nss) * GT_K;
#if defined(__HIP_DEVICE_COMPILE__)   // a gfx950 builtin: device pass only
#pragma unroll
    for (int q = 0; q < NXA; ++q) {
      const uint8_t* src = loc + xk[q] < g.ks ? g.x + xo[q] + (size_t)k0 * EB : g.x;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr)(st + (wave * NXA + q) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < NWA; ++q) {
      const float* src = (wok[q] && loc + wr[q] < g.ks) ? g.wg + wo[q] + (size_t)k0 * g.E : g.wg;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr)(st + XB + (wave * NWA + q) * 1024), 16, 0, 0);
    }
#endif
  };

  f64x4_t acc[2], tot[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[nb][q] = tot[nb][q] = 0.0;
  double xsq = 0.0, wsq[2] = {0.0, 0.0};
  const bool do_xn = blockIdx.x == 0, do_wn = blockIdx.y == 0 && wave == 0;

  // fragment offsets within a stage
  const int wsl = (j & 1) << 2;                // weight slot swizzle of this lane's k rows
  int wof[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int el = 16 * nb + (lane & 15);
    wof[nb] = XB + (((el >> 2) ^ wsl) << 4) + (el & 3) * 4;
  }
  auto xoff = [&](int c16) -> int {
    if (DT == MOE_BF16) return rr * RB + (((2 * c16 + (j >> 1)) ^ (rr & XSW)) << 4) + (j & 1) * 8;
    if (DT == MOE_F32) return rr * RB + (((4 * c16 + j) ^ (rr & XSW)) << 4);
    return rr * RB + ((c16 ^ (rr & XSW)) << 4) + 4 * j;
  };

  const uint32_t sbase = (uint32_t)(uintptr_t)(lds_u8*)sscale + rr * nkb;
  auto compute = [&](const uint8_t* st, int i) {
    const int loc = (i % nss) * GT_K;
#pragma unroll
    for (int c16 = 0; c16 < 4; ++c16) {
      if (loc + 16 * c16 >= g.ks) break;       // ragged last step of a part
      double a[4], b[2][4];
      const uint32_t sb = (uint32_t)(uintptr_t)(lds_u8*)st;
      const uint32_t wa = sb + (16 * c16 + 4 * j) * 128;
      u32x4_v xv;
      uint32_t w[8];
      gate_lds_reads<DT>(sb + xoff(c16), wa + wof[0], wa + wof[1],
                         sbase + ((i / nss) * g.ks + loc + 16 * c16) / 32, xv, w);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        b[0][m] = (double)__uint_as_float(w[m]);
        b[1][m] = (double)__uint_as_float(w[4 + m]);
      }
      if (DT == MOE_BF16) {
        a[0] = (double)__uint_as_float(xv[0] << 16);
        a[1] = (double)__uint_as_float(xv[0] & 0xffff0000u);
        a[2] = (double)__uint_as_float(xv[1] << 16);
        a[3] = (double)__uint_as_float(xv[1] & 0xffff0000u);
      } else if (DT == MOE_F32) {
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = (double)__uint_as_float(xv[m]);
      } else {
        const double sf = e8m0_to_f64((uint8_t)xv[1]);
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = e4m3_to_f64((uint8_t)(xv[0] >> (8 * m))) * sf;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], b[nb][m], acc[nb], 0, 0, 0);
      }
      if (do_xn) {
#pragma unroll
        for (int m = 0; m < 4; ++m) xsq = fma(a[m], a[m], xsq);
      }
      if (do_wn) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int m = 0; m < 4; ++m) wsq[nb] = fma(b[nb][m], b[nb][m], wsq[nb]);
      }
    }
    if (i % nss == nss - 1) {                  // end of a K part: add it to the total
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        tot[nb] = (i == nss - 1) ? acc[nb] : tot[nb] + acc[nb];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[nb][q] = 0.0;
      }
    }
  };

  // ---- K loop over the ring; step i lives in st[i % 3] ----
  issue(st0, 0);
  if (nsteps > 1) issue(st1, 1);
  auto kstep = [&](int i, const uint8_t* cur, uint8_t* nxt) {
    if (i + 1 < nsteps)
      gate_wait_vmcnt<PER_STEP>();
    else
      gate_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (i + 2 < nsteps) issue(nxt, i + 2);
    compute(cur, i);
  };
  for (int i = 0; i < nsteps; i += GD_STAGES) {
    kstep(i, st0, st2);
    if (i + 1 < nsteps) kstep(i + 1, st1, st0);
    if (i + 2 < nsteps) kstep(i + 2, st2, st1);
  }

  // ---- outputs.  D layout of a 16x16 fp64 block: element q of a lane is row
  //      lane/16 + 4q, column lane%16. ----
  const bool final_out = gridDim.z == 1;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int e = e0 + 16 * nb + (lane & 15);
    if (e >= g.E) continue;
    const double bb = (final_out && g.bias) ? (double)g.bias[e] : 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + 16 * wave + (lane >> 4) + 4 * q;
      if (t >= g.T) continue;
      if (final_out) {
        double v = tot[nb][q];
        if (g.bias) v = v + bb;
        g.logits[(size_t)t * g.E + e] = v;
      } else {
        g.part[((size_t)z * g.T + t) * g.E + e] = tot[nb][q];
      }
    }
  }
  if (do_xn) {
    double v = xsq + __shfl_xor(xsq, 16);
    v = v + __shfl_xor(v, 32);
    const int t = t0 + rr;
    if (j == 0 && t < g.T) {
      if (final_out) g.xnorm[t] = sqrt(v);
      else g.xnorm[(size_t)z * g.T + t] = v;
    }
  }
  if (do_wn) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      double v = wsq[nb] + __shfl_xor(wsq[nb], 16);
      v = v + __shfl_xor(v, 32);
      const int e = e0 + 16 * nb + (lane & 15);
      if (j == 0 && e < g.E) {
        if (final_out) g.wnorm[e] = sqrt(v);
        else g.wnorm[(size_t)z * g.E + e] = v;
      }
    }
  }
}

// Adds the S partial sums of a K-split gate launch in ascending order, then the bias
// (the order gate_gemm_f64_ring_kernel uses when one workgroup runs every part), and
// finishes the norms.
__global__ __launch_bounds__(256) void gate_finish_kernel(const double* __restrict__ part,
                                                          const double* __restrict__ xsq,
                                                          const double* __restrict__ wsq,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int S, double* __restrict__ logits,
                                                          double* __restrict__ xnorm,
                                                          double* __restrict__ wnorm) {
  const size_t n = (size_t)T * E;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    double v = part[i];
    for (int z = 1; z < S; ++z) v = v + part[(size_t)z * n + i];
    if (bias) v = v + (double)bias[i % E];
    logits[i] = v;
  }
  if (i < (size_t)T) {
    double v = xsq[i];
    for (int z = 1; z < S; ++z) v = v + xsq[(size_t)z * T + i];
    xnorm[i] = sqrt(v);
  }
  if (i < (size_t)E) {
    double v = wsq[i];
    for (int z = 1; z < S; ++z) v = v + wsq[(size_t)z * E + i];
    wnorm[i] = sqrt(v);
  }
}

// "a ranks before b": larger logit first, then lower expert index.
__device__ __forceinline__ bool ranks_before(double av, int ae, double bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// Smallest gap that certifies an order of two computed logits beyond their bounds;
// it also keeps the exact values more than an ulp apart, so their correctly rounded
// values cannot merge into a tie.
__device__ __forceinline__ double cert_margin(double a, double b) {
  return 0x1p-45 * (fabs(a) + fabs(b));
}

constexpr int SEL_WAVES = 4;
constexpr int SEL_NV = kMaxExperts / 64;

// One wavefront per token.  k rounds of a wave-wide arg-max over (logit desc, index
// asc) give the top-k in rank order; the token is certified when every adjacent
// pair among ranks 0..k-1, and rank k-1 against every unselected expert, stays
// ordered after widening each logit by its error bound.
__global__ __launch_bounds__(256) void select_topk_kernel(
    const double* __restrict__ logits, const double* __restrict__ xnorm,
    const double* __restrict__ wnorm, const float* __restrict__ bias, int T, int E, int k,
    double two_gamma, int32_t* __restrict__ ids, int* __restrict__ tok_flag, int* flag) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int t = blockIdx.x * SEL_WAVES + wave;
  if (t >= T) return;
  const double* row = logits + (size_t)t * E;
  const double xn = xnorm[t];
  double v[SEL_NV], bnd[SEL_NV];
  uint32_t taken = 0;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < SEL_NV; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
      finite = finite && isfinite(v[i]);
      bnd[i] = two_gamma * (xn * wnorm[e] + (bias ? fabs((double)bias[e]) : 0.0));
    } else {
      v[i] = -INFINITY;
      bnd[i] = 0.0;
      taken |= 1u << i;
    }
  }
  if (!__all(finite)) {
    // Non-finite gate output: report it and emit a valid, distinct id row.
    if (lane == 0) {
      raise_flag(flag, kFlagNonFinite);
      tok_flag[t] = 0;
    }
    for (int r = lane; r < k; r += 64) ids[(size_t)t * k + r] = r;
    return;
  }
  bool ok = true;
  double pv = 0.0, pb = 0.0;
  for (int r = 0; r < k; ++r) {
    double bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < SEL_NV; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1u) && ranks_before(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == (be & 63)) taken |= 1u << (be >> 6);
    const double bb = two_gamma * (xn * wnorm[be] + (bias ? fabs((double)bias[be]) : 0.0));
    if (lane == 0) ids[(size_t)t * k + r] = be;
    if (r > 0) ok = ok && ((pv - pb) - (bv + bb) > cert_margin(pv, bv));
    pv = bv;
    pb = bb;
  }
  if (k < E) {
    double u = -INFINITY;
#pragma unroll
    for (int i = 0; i < SEL_NV; ++i)
      if (!((taken >> i) & 1u)) u = fmax(u, v[i] + bnd[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) u = fmax(u, __shfl_xor(u, off));
    ok = ok && ((pv - pb) - u > cert_margin(pv, u));
  }
  if (lane == 0) tok_flag[t] = ok ? 0 : 1;
}

// ---------------------------------------------------------------------------
// Exact logits for uncertified tokens.  Every product x_i * w_ie is exact in fp64
// (at most 24 + 24 significant bits, no underflow for fp32/bf16/MXFP8 operands), so
// the exact sum is accumulated as a non-overlapping expansion (Shewchuk, "Adaptive
// Precision Floating-Point Arithmetic and Fast Robust Geometric Predicates", 1997:
// two-sum with zero elimination) and rounded once to nearest-even from the top
// component down, with the half-way correction that looks at the next component.
// ---------------------------------------------------------------------------
constexpr int kParts = 64;

struct Expansion {
  double p[kParts];
  int n = 0;
  bool overflow = false;

  __device__ void add(double v) {
#pragma clang fp contract(off)
    int m = 0;
    for (int j = 0; j < n; ++j) {
      double y = p[j];
      if (fabs(v) < fabs(y)) {
        const double tmp = v;
        v = y;
        y = tmp;
      }
      const double hi = v + y;
      const double lo = y - (hi - v);
      if (lo != 0.0) p[m++] = lo;
      v = hi;
    }
    if (m < kParts) {
      p[m++] = v;
    } else {
      overflow = true;
    }
    n = m;
  }

  __device__ double round_nearest() const {
#pragma clang fp contract(off)
    int i = n;
    if (i == 0) return 0.0;
    double hi = p[--i];
    double lo = 0.0;
    while (i > 0) {
      const double xx = hi;
      const double y = p[--i];
      hi = xx + y;
      const double yr = hi - xx;
      lo = y - yr;
      if (lo != 0.0) break;
    }
    if (i > 0 && ((lo < 0.0 && p[i - 1] < 0.0) || (lo > 0.0 && p[i - 1] > 0.0))) {
      const double y = lo * 2.0;
      const double xx = hi + y;
      const double yr = xx - hi;
      if (y == yr) hi = xx;
    }
    return hi;
  }
};

__global__ __launch_bounds__(256) void exact_fallback_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d,
    const float* __restrict__ wg, const float* __restrict__ bias, int E, int k,
    const int* __restrict__ tok_flag, int32_t* __restrict__ ids, int* flag) {
  const int t = blockIdx.x;
  if (t >= T || tok_flag[t] != 1) return;
  __shared__ double ex[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    Expansion acc;
    for (int i = 0; i < d; ++i) {
      const double xv = load_act_f64(x, xs, dtype, (size_t)t, d, i);
      const double wv = (double)wg[(size_t)i * E + e];
      acc.add(xv * wv);
    }
    if (bias) acc.add((double)bias[e]);
    if (acc.overflow) raise_flag(flag, kFlagCorrupt);
    ex[e] = acc.round_nearest();
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const double v = ex[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) rank += ranks_before(ex[j], j, v, e) ? 1 : 0;
    if (rank < k) ids[(size_t)t * k + rank] = e;
  }
}

// Replay plausibility filter, the tokens the fp64 bound could not decide (tok_flag 1;
// their replayed ids are valid and ids still holds the router's top-k): threads
// 0..k-1 round the replayed ids' logits exactly, thread k the router's k-th choice's;
// thread 0 then keeps column j iff fl(l_j - l_(k)) >= log_tau and refills the dropped
// columns with the router's ids in rank order that no kept column holds.
__global__ __launch_bounds__(64) void filter_exact_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d,
    const float* __restrict__ wg, const float* __restrict__ bias, int E, int k,
    const int32_t* __restrict__ ids_in, double log_tau, const int* __restrict__ tok_flag,
    int32_t* __restrict__ ids, int* flag) {
  const int t = blockIdx.x;
  if (t >= T || tok_flag[t] != 1) return;
  __shared__ double ex[kMaxTopK + 1];
  __shared__ int rid[kMaxTopK];
  const int j = threadIdx.x;
  int32_t* io = ids + (size_t)t * k;
  if (j <= k) {
    const int e = j < k ? ids_in[(size_t)t * k + j] : io[k - 1];
    Expansion acc;
    for (int i = 0; i < d; ++i) {
      const double xv = load_act_f64(x, xs, dtype, (size_t)t, d, i);
      acc.add(xv * (double)wg[(size_t)i * E + e]);
    }
    if (bias) acc.add((double)bias[e]);
    if (acc.overflow) raise_flag(flag, kFlagCorrupt);
    ex[j] = acc.round_nearest();
  }
  if (j < k) rid[j] = io[j];
  __syncthreads();
  if (j != 0) return;
  uint64_t keepm = 0;
  for (int c = 0; c < k; ++c)
    if (ex[c] - ex[k] >= log_tau) keepm |= 1ull << c;
  int next = 0;   // next router rank to try
  for (int c = 0; c < k; ++c) {
    if ((keepm >> c) & 1ull) {
      io[c] = ids_in[(size_t)t * k + c];
      continue;
    }
    for (; next < k; ++next) {   // enough remain: k - kept router ids are not held
      bool held = false;
      for (int u = 0; u < k; ++u)
        if (((keepm >> u) & 1ull) && ids_in[(size_t)t * k + u] == rid[next]) held = true;
      if (!held) break;
    }
    io[c] = rid[next < k ? next++ : 0];
  }
}

// Weights of one token: softmax over all experts restricted to the chosen ones and
// renormalised, i.e. exp(l_r - m) / sum_s exp(l_s - m) with m the largest chosen
// logit, in fp64 from the fp64 GEMM logits, sum in column order, one rounding to fp32.
// Out-of-range ids are clamped for the read (the call has already flagged them).
__device__ void restricted_softmax(const double* __restrict__ row, const int32_t* __restrict__ idr,
                                   int k, int E, float* __restrict__ wout) {
  double m = -INFINITY;
  for (int r = 0; r < k; ++r) {
    const int e = min(max(idr[r], 0), E - 1);
    m = fmax(m, row[e]);
  }
  double s = 0.0;
  for (int r = 0; r < k; ++r) {
    const int e = min(max(idr[r], 0), E - 1);
    s += exp(row[e] - m);
  }
  for (int r = 0; r < k; ++r) {
    const int e = min(max(idr[r], 0), E - 1);
    wout[r] = (float)(exp(row[e] - m) / s);
  }
}

__global__ __launch_bounds__(256) void route_weights_kernel(const double* __restrict__ logits, int T,
                                                            int E, int k, const int32_t* __restrict__ ids,
                                                            float* __restrict__ weights) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  restricted_softmax(logits + (size_t)t * E, ids + (size_t)t * k, k, E, weights + (size_t)t * k);
}

// Replay: one wavefront per token checks its logits for finiteness; lane 0 validates
// the replayed ids (range, distinct) and writes the weights.
__global__ __launch_bounds__(256) void replay_kernel(const double* __restrict__ logits, int T, int E,
                                                     int k, const int32_t* __restrict__ ids_in,
                                                     const float* __restrict__ weights_in,
                                                     float* __restrict__ weights_out, int* flag) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int t = blockIdx.x * SEL_WAVES + wave;
  if (t >= T) return;
  const double* row = logits + (size_t)t * E;
  bool finite = true;
  for (int e = lane; e < E; e += 64) finite = finite && isfinite(row[e]);
  const bool all_finite = __all(finite);
  if (lane != 0) return;
  if (!all_finite) raise_flag(flag, kFlagNonFinite);
  const int32_t* idr = ids_in + (size_t)t * k;
  int bits = 0;
  for (int r = 0; r < k; ++r) {
    const int e = idr[r];
    if (e < 0 || e >= E) bits |= kFlagBadId;
    for (int q = 0; q < r; ++q)
      if (idr[q] == e) bits |= kFlagDupId;
  }
  if (bits) raise_flag(flag, bits);
  float* wo = weights_out + (size_t)t * k;
  if (weights_in) {
    for (int r = 0; r < k; ++r) wo[r] = weights_in[(size_t)t * k + r];
  } else {
    restricted_softmax(row, idr, k, E, wo);
  }
}

static moe_status check_route_args(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                   const float* w_gate, int E, int k, const void* ws,
                                   size_t ws_bytes) {
  if (!valid_dtype(dtype) || T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E ||
      k > kMaxTopK)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !ws) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_MXFP8 && (!x_scale || d % 32 != 0)) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_MXFP8 && x_scale) return MOE_ERR_INVALID_ARG;
  if (d % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (!aligned(x, 16)) return MOE_ERR_INVALID_ARG;
  if ((long long)T * E > 0x7fffffffLL || (long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (E % 4 == 0 && !aligned(w_gate, 16)) return MOE_ERR_INVALID_ARG;
  if (!aligned(w_gate, 4)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < route_ws(T, d, E).bytes) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// gamma_n = n u / (1 - n u), u = 2^-53; doubled for safety (covers directed
// rounding inside the hardware fma and the rounding of the norms themselves).
static double two_gamma(int d) {
  const double nu = (double)(d + 1) * 0x1p-53;
  return 2.0 * nu / (1.0 - nu);
}

static moe_status launch_gate(const void* x, const uint8_t* xs, int dtype, int T, int d,
                              const float* w_gate, const float* bias, int E, char* w,
                              hipStream_t s) {
  const RouteWs L = route_ws(T, d, E);
  double* lg = (double*)(w + L.logits);
  double* xn = (double*)(w + L.xnorm);
  double* wn = (double*)(w + L.wnorm);
  if (E % 4 != 0) {   // weight rows not 16-byte granular: register-staged kernel
    dim3 grid((E + GT_E - 1) / GT_E, (T + GT_M - 1) / GT_M);
    if (dtype == MOE_BF16)
      gate_gemm_f64_kernel<MOE_BF16><<<grid, 256, 0, s>>>(x, xs, T, d, w_gate, bias, E, lg, xn, wn);
    else if (dtype == MOE_F32)
      gate_gemm_f64_kernel<MOE_F32><<<grid, 256, 0, s>>>(x, xs, T, d, w_gate, bias, E, lg, xn, wn);
    else
      gate_gemm_f64_kernel<MOE_MXFP8><<<grid, 256, 0, s>>>(x, xs, T, d, w_gate, bias, E, lg, xn, wn);
    return launch_status();
  }
  const int S = gate_splits(d);
  const bool split = gate_split_launch(T, d, E);
  GateArgs g{};
  g.x = (const uint8_t*)x;
  g.xs = xs;
  g.T = T;
  g.d = d;
  g.E = E;
  g.wg = w_gate;
  g.bias = bias;
  g.ks = d / S;
  g.spw = split ? 1 : S;
  g.logits = lg;
  g.part = (double*)(w + L.part);
  g.xnorm = split ? (double*)(w + L.xsq) : xn;
  g.wnorm = split ? (double*)(w + L.wsq) : wn;
  dim3 grid((E + GT_E - 1) / GT_E, (T + GT_M - 1) / GT_M, split ? S : 1);
  if (dtype == MOE_BF16)
    gate_gemm_f64_ring_kernel<MOE_BF16><<<grid, 256, 0, s>>>(g);
  else if (dtype == MOE_F32)
    gate_gemm_f64_ring_kernel<MOE_F32><<<grid, 256, 0, s>>>(g);
  else
    gate_gemm_f64_ring_kernel<MOE_MXFP8><<<grid, 256, (size_t)GT_M * (g.spw * g.ks / 32), s>>>(g);
  if (split) {
    const size_t n = (size_t)T * E;
    gate_finish_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        g.part, g.xnorm, g.wnorm, bias, T, E, S, lg, xn, wn);
  }
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                const float* w_gate, const float* bias, int E, int k, int32_t* ids,
                                float* weights, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_route_args(x, x_scale, dtype, T, d, w_gate, E, k, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!ids || !weights) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  int* flag = (int*)w;
  const RouteWs L = route_ws(T, d, E);
  if (gate_screened(dtype, d) && !gate_split_launch(T, d, E)) {
    if ((st = screen_route_select(x, x_scale, dtype, T, d, w_gate, bias, E, k, ids, w, s)) != MOE_OK)
      return st;
    exact_fallback_kernel<<<T, 256, 0, s>>>(x, x_scale, dtype, T, d, w_gate, bias, E, k,
                                            (const int*)(w + L.tok_flag), ids, flag);
    return screen_route_weights(x, x_scale, dtype, T, d, bias, E, k, ids, nullptr, weights, w, s);
  }
  if ((st = launch_gate(x, x_scale, dtype, T, d, w_gate, bias, E, w, s)) != MOE_OK) return st;
  select_topk_kernel<<<(T + SEL_WAVES - 1) / SEL_WAVES, 256, 0, s>>>(
      (const double*)(w + L.logits), (const double*)(w + L.xnorm), (const double*)(w + L.wnorm),
      bias, T, E, k, two_gamma(d), ids, (int*)(w + L.tok_flag), flag);
  exact_fallback_kernel<<<T, 256, 0, s>>>(x, x_scale, dtype, T, d, w_gate, bias, E, k,
                                          (const int*)(w + L.tok_flag), ids, flag);
  if (gate_screened(dtype, d)) {   // weights from the per-pair fp64 logits, as for large batches
    if ((st = chosen_ids_refine(x, x_scale, dtype, T, d, w_gate, bias, E, k, ids, w, s)) != MOE_OK)
      return st;
    return screen_route_weights(x, x_scale, dtype, T, d, bias, E, k, ids, nullptr, weights, w, s);
  }
  route_weights_kernel<<<(T + 255) / 256, 256, 0, s>>>((const double*)(w + L.logits), T, E, k, ids,
                                                       weights);
  return launch_status();
}

extern "C" moe_status moe_route_replay(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                       const float* w_gate, const float* bias, int E, int k,
                                       const int32_t* ids_in, const float* weights_in,
                                       float* weights_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_route_args(x, x_scale, dtype, T, d, w_gate, E, k, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!ids_in || !weights_out) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  if (gate_screened(dtype, d))
    return screen_replay(x, x_scale, dtype, T, d, w_gate, bias, E, k, ids_in, weights_in, weights_out,
                         w, s);
  const RouteWs L = route_ws(T, d, E);
  if ((st = launch_gate(x, x_scale, dtype, T, d, w_gate, bias, E, w, s)) != MOE_OK) return st;
  replay_kernel<<<(T + SEL_WAVES - 1) / SEL_WAVES, 256, 0, s>>>(
      (const double*)(w + L.logits), T, E, k, ids_in, weights_in, weights_out, (int*)w);
  return launch_status();
}

extern "C" moe_status moe_route_replay_filtered(const void* x, const uint8_t* x_scale, int dtype, int T,
                                                int d, const float* w_gate, const float* bias, int E,
                                                int k, const int32_t* ids_in, double log_tau,
                                                int32_t* ids_out, float* weights_out, void* ws,
                                                size_t ws_bytes, void* stream) {
  moe_status st = check_route_args(x, x_scale, dtype, T, d, w_gate, E, k, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!ids_in || !ids_out || !weights_out || isnan(log_tau)) return MOE_ERR_INVALID_ARG;
  const size_t n = (size_t)T * k;
  if (ids_in < ids_out + n && ids_out < ids_in + n) return MOE_ERR_INVALID_ARG;
  // the router's own top-k (rank order) into ids_out, its logits into the workspace
  if ((st = moe_route(x, x_scale, dtype, T, d, w_gate, bias, E, k, ids_out, weights_out, ws, ws_bytes,
                      stream)) != MOE_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  FilterArgs a{};
  a.x = x;
  a.xs = x_scale;
  a.dtype = dtype;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  a.bias = bias;
  a.ids_in = ids_in;
  a.log_tau = log_tau;
  a.tg = two_gamma(d);
  a.ids = ids_out;
  a.weights = weights_out;
  const bool screened = gate_screened(dtype, d);
  if ((st = filter_launch(a, screened, w, 0, s)) != MOE_OK) return st;
  const RouteWs L = route_ws(T, d, E);
  filter_exact_kernel<<<T, 64, 0, s>>>(x, x_scale, dtype, T, d, w_gate, bias, E, k, ids_in, log_tau,
                                       (const int*)(w + L.tok_flag), ids_out, (int*)w);
  if ((st = launch_status()) != MOE_OK) return st;
  return filter_launch(a, screened, w, 1, s);
}
