// Two-tier gate for bf16 and MXFP8 activations: a bf16 matrix-core screen with a
// rigorous error bound picks, per token, the experts that can still be among the top
// k; only those get fp64 logits, which decide the selection (with the fp64 bound, and
// the exact fallback for what that bound cannot separate) and give the weights.
//
// The gate picks the top-k experts per token (Training Data podcast page "How Cursor
// Trained Composer on Fireworks", section on floating point and MoE: 8 of 384 experts
// per layer, and a fifth-decimal difference in the hidden state can flip the choice),
// so the selection has to equal the one made on the exact logits.
//
// Screen: Wg is split exactly into three bf16 planes, w = hi + mid + lo.  For each
// chunk of the reduction (64 elements for bf16 x, one 32-element MX block for MXFP8
// x) v_mfma_f32_32x32x16_bf16 sums x * plane in fp32 from zero, and the chunk sums are
// added in fp64 (times the chunk's E8M0 scale for MXFP8).  Every product of two bf16
// values is exact in fp32; a chunk sum of m = 3 * chunk products has at most m
// rounded additions, so with u = 2^-23 (which also covers truncating adders)
//   |screen - exact| <= gamma_m(u) * (1 + 2^-6) * ||x_t|| ||w_e||
//                       + gamma_{d+1}(2^-53) * (||x_t|| ||w_e|| + |b_e|) + flush term,
// doubled for safety (the flush term covers fp32 results below 2^-126 flushed to zero).
// Every expert whose screen interval reaches the k-th largest lower bound is a
// candidate; any other expert's exact logit lies below k candidates' exact logits.
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Gate weights, transposed: wt [E][d] fp32 (for the fp64 logits) and, when `planes`
// is given, the exact three-way bf16 split planes [3][E][d] (hi, mid, lo).
// hi = RNE(w); w - hi is exact in fp32 with at most 16 significant bits, mid = RNE of
// it, and the rest has at most 8 bits, so lo holds it exactly (w below 2^-110 aside,
// whose parts can fall under bf16's subnormal grid: the flush term covers them).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_prep_kernel(const float* __restrict__ wg, int d, int E,
                                                        float* __restrict__ wt,
                                                        uint16_t* __restrict__ planes) {
  __shared__ float tile[64][65];
  const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int q = tid; q < 64 * 64; q += 256) {
    const int kr = q / 64, ec = q % 64;
    const int k = k0 + kr, e = e0 + ec;
    tile[kr][ec] = (k < d && e < E) ? wg[(size_t)k * E + e] : 0.0f;
  }
  __syncthreads();
  const size_t plane = (size_t)E * d;
  for (int q = tid; q < 64 * 64; q += 256) {
    const int er = q / 64, kc = q % 64;
    const int k = k0 + kc, e = e0 + er;
    if (k < d && e < E) {
      const float w = tile[kc][er];
      const size_t o = (size_t)e * d + k;
      wt[o] = w;
      if (planes) {
        const uint16_t hi = f32_to_bf16(w);
        const float r1 = w - bf16_to_f32(hi);
        const uint16_t mid = f32_to_bf16(r1);
        const float r2 = r1 - bf16_to_f32(mid);
        planes[o] = hi;
        planes[plane + o] = mid;
        planes[2 * plane + o] = f32_to_bf16(r2);
      }
    }
  }
}

// ||w_e||_2 in fp64, one workgroup per expert (thread-strided sums, then a fixed
// tree over the 256 threads).
__global__ __launch_bounds__(256) void gate_wnorm_kernel(const float* __restrict__ wt, int d, int E,
                                                         double* __restrict__ wnorm) {
  __shared__ double part[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const float* row = wt + (size_t)e * d;
  double acc = 0.0;
  for (int i = tid; i < d; i += 256) {
    const double v = (double)row[i];
    acc = fma(v, v, acc);
  }
  part[tid] = acc;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (tid < h) part[tid] += part[tid + h];
    __syncthreads();
  }
  if (tid == 0) wnorm[e] = sqrt(part[0]);
}

// ---------------------------------------------------------------------------
// Screen GEMM.  Workgroup tile: 128 experts x 128 tokens; 8 wavefronts, wavefront
// (we, wt) owns experts 64 we .. +63 (two 32-row A blocks, one per plane triple) and
// tokens 32 wt .. +31 (one 32-column B block).  The experts are the MFMA's rows, so a
// lane's 16 accumulator values all belong to one token (column lane % 32) and the
// token's MX scale is one value per lane.  K advances 64 per step through LDS (144-byte
// rows) with the next step's loads in registers.
// The K steps are cut into gridDim.z parts of `spart` steps (more workgroups for small
// batches; the screen needs no fixed summation order, only its bound, which holds for
// any grouping of the chunk sums).  Output: partial sums s[z][t][e] (fp64, without the
// bias); the first expert tile also writes the partial squared norms xsq[z][t].
// ---------------------------------------------------------------------------
constexpr int SC_E = 128, SC_T = 128, SC_K = 64, SC_LDS = SC_K + 8, SC_THR = 512;

template <int DT>
__global__ __launch_bounds__(SC_THR) void gate_screen_kernel(const void* __restrict__ x,
                                                             const uint8_t* __restrict__ xs, int T,
                                                             int d, int E, int spart,
                                                             const uint16_t* __restrict__ planes,
                                                             double* __restrict__ s,
                                                             double* __restrict__ xsqp) {
  constexpr int CPR = SC_K / 8;                           // 16-byte bf16 chunks per row
  constexpr int NW = 3 * SC_E * CPR / SC_THR;             // plane chunks per thread
  constexpr int NX = DT == MOE_BF16 ? SC_T * CPR / SC_THR : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sW[3][SC_E][SC_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t sX[SC_T][SC_LDS];
  __shared__ double sS[SC_T][2];                          // MXFP8: the two block scales of a step

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int we = wave >> 2, wt = wave & 3;
  // workgroup -> (expert tile bx, token tile by, K part bz).  When the (expert tile, K
  // part) slices are a multiple of the 8 XCDs, XCD b % 8 runs slices xcd, xcd + 8, ...
  // one after another with all token tiles of a slice side by side: a slice's plane rows
  // are then read from HBM once per XCD and shared through its L2.
  const int ex = (E + SC_E - 1) / SC_E, ty = (T + SC_T - 1) / SC_T;
  const int nslice = (int)(gridDim.x / ty);   // ex * parts
  int bx, by, bz;
  {
    const int b = blockIdx.x;
    if (nslice % kXcds == 0) {
      const int q = b / kXcds, p = b % kXcds + kXcds * (q / ty);
      by = q % ty;
      bx = p % ex;
      bz = p / ex;
    } else {
      bx = b % ex;
      by = (b / ex) % ty;
      bz = b / (ex * ty);
    }
  }
  const int e0 = bx * SC_E, t0 = by * SC_T;
  const size_t plane = (size_t)E * d;
  const int nb32 = d / 32;

  // loaders: plane chunk q = tid + SC_THR i is plane q / (SC_E CPR), row (q % (SC_E CPR)) / CPR,
  // k offset 8 (q % CPR); activation chunk likewise (bf16: 8 values; MXFP8: 16 codes).
  const uint16_t* wp[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int q = tid + SC_THR * i, p = q / (SC_E * CPR), r = (q % (SC_E * CPR)) / CPR, c = (q % CPR) * 8;
    const int e = e0 + r < E ? e0 + r : 0;
    wp[i] = planes + p * plane + (size_t)e * d + c;
  }
  int xr[NX], xc[NX];
  size_t xo[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int q = tid + SC_THR * i;
    xr[i] = DT == MOE_BF16 ? q / CPR : q / 4;
    xc[i] = DT == MOE_BF16 ? (q % CPR) * 8 : (q % 4) * 16;
    const int t = t0 + xr[i] < T ? t0 + xr[i] : 0;
    xo[i] = (size_t)t * d + xc[i];
  }
  const int sr = tid >> 1, sb = tid & 1;                  // MXFP8 scale loader (tid < 2 SC_T)
  const size_t so = (size_t)(t0 + sr < T ? t0 + sr : 0) * nb32 + sb;

  u32x4_t rw[NW], rx[NX];
  uint32_t rsc = 0;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NW; ++i) rw[i] = *(const u32x4_t*)(wp[i] + k0);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      if (DT == MOE_BF16) rx[i] = *(const u32x4_t*)((const uint16_t*)x + xo[i] + k0);
      else rx[i] = *(const u32x4_t*)((const uint8_t*)x + xo[i] + k0);
    }
    if (DT == MOE_MXFP8 && tid < 2 * SC_T) rsc = xs[so + k0 / 32];
  };

  f32x16_t acc32[2];
  double acc64[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc32[mb][v] = 0.0f;
      acc64[mb][v] = 0.0;
    }
  const bool do_xn = bx == 0 && we == 0;
  double xsq = 0.0, csq = 0.0;    // csq: this chunk's sum of squared (unscaled) activations
  const int trow = wt * 32 + (lane & 31);

  // fold the fp32 chunk sums (times the chunk's scale) into the fp64 accumulators
  auto fold = [&](double sc) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc64[mb][v] = fma((double)acc32[mb][v], sc, acc64[mb][v]);
        acc32[mb][v] = 0.0f;
      }
    if (do_xn) {
      xsq = fma(csq, sc * sc, xsq);
      csq = 0.0;
    }
  };

  const int st0 = bz * spart;
  const int nsteps = min(d / SC_K - st0, spart);
  gload(st0 * SC_K);
  for (int st = 0; st < nsteps; ++st) {
    // registers -> LDS
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int q = tid + SC_THR * i, p = q / (SC_E * CPR), r = (q % (SC_E * CPR)) / CPR, c = (q % CPR) * 8;
      *(u32x4_t*)&sW[p][r][c] = rw[i];
    }
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      if (DT == MOE_BF16) {
        *(u32x4_t*)&sX[xr[i]][xc[i]] = rx[i];
      } else {
        // v_cvt_pk_f32_fp8 decodes two codes exactly into fp32; every E4M3 value is a
        // bf16 value, so its upper 16 bits are the bf16 encoding (NaN stays NaN)
        u32x4_t lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)rx[i][q], false);   // bytes 0, 1
          const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)rx[i][q], true);    // bytes 2, 3
          const uint32_t w0 = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
          const uint32_t w1 = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
          if (q < 2) {
            lo[2 * q] = w0;
            lo[2 * q + 1] = w1;
          } else {
            hi[2 * q - 4] = w0;
            hi[2 * q - 3] = w1;
          }
        }
        *(u32x4_t*)&sX[xr[i]][xc[i]] = lo;
        *(u32x4_t*)&sX[xr[i]][xc[i] + 8] = hi;
      }
    }
    if (DT == MOE_MXFP8 && tid < 2 * SC_T) sS[sr][sb] = e8m0_to_f64((uint8_t)rsc);
    __syncthreads();
    if (st + 1 < nsteps) gload((st0 + st + 1) * SC_K);

#pragma unroll
    for (int kk = 0; kk < SC_K; kk += 16) {
      const int kc = kk + 8 * (lane >> 5);
      const bf16x8_t bx = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sX[trow][kc]);
      if (do_xn) {
        const u32x4_t u = __builtin_bit_cast(u32x4_t, bx);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const double v = (double)__uint_as_float((q & 1) ? (u[q >> 1] & 0xffff0000u) : (u[q >> 1] << 16));
          csq = fma(v, v, csq);
        }
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8_t aw =
              __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)&sW[p][we * 64 + mb * 32 + (lane & 31)][kc]);
          acc32[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bx, acc32[mb], 0, 0, 0);
        }
      // chunk ends: every 32 k for MXFP8 (one scale block), every 64 k for bf16
      if (DT == MOE_MXFP8 && (kk == 16 || kk == 48)) fold(sS[trow][kk >> 5]);
    }
    if (DT == MOE_BF16) fold(1.0);
    __syncthreads();
  }

  // outputs: accumulator element v is expert row 8 (v / 4) + 4 (lane / 32) + v % 4 of
  // the block, token column lane % 32
  const int t = t0 + trow;
  double* sz = s + (size_t)bz * T * E;
  if (t < T) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int e = e0 + we * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (e < E) sz[(size_t)t * E + e] = acc64[mb][v];
      }
  }
  if (do_xn) {
    const double v = xsq + __shfl_xor(xsq, 32);
    if (lane < 32 && t < T) xsqp[(size_t)bz * T + t] = v;
  }
}

// ---------------------------------------------------------------------------
// fp64 logit x_t . w_e, computed by one whole wavefront: lane l accumulates elements
// 8 l + 512 j .. +7 (j ascending) with fma, then a fixed butterfly adds the lanes.
// Every product is exact in fp64, so each term is rounded once.  The same function
// serves the learned path, router replay and the weights, so their values agree bit
// for bit.  Requires d % 8 == 0.
// ---------------------------------------------------------------------------
// The helpers are instantiated per activation type (DT: MOE_BF16 or MOE_MXFP8) so their
// unrolled loops hold no branch on it: a branch there made every load wait for the one
// before it.
template <int DT>
__device__ __forceinline__ void wave_dot_xload(const void* __restrict__ x, const uint8_t* __restrict__ xs,
                                               int t, int d, int i0, double (&xv)[8]) {
  if constexpr (DT == MOE_BF16) {
    const u32x4_t u = *(const u32x4_t*)((const uint16_t*)x + (size_t)t * d + i0);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      xv[q] = (double)__uint_as_float((q & 1) ? (u[q >> 1] & 0xffff0000u) : (u[q >> 1] << 16));
  } else {
    // v_cvt_pk_f32_fp8 decodes two OCP E4M3 codes exactly (every E4M3 value, NaN and the
    // subnormal grid included, is an fp32 value; checked against the bit-level decode for
    // all 256 codes)
    const u32x2_t u = *(const u32x2_t*)((const uint8_t*)x + (size_t)t * d + i0);
    const double sc = e8m0_to_f64(xs[(size_t)t * (d / 32) + i0 / 32]);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[w], false);   // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[w], true);    // bytes 2, 3
      xv[4 * w] = (double)lo[0] * sc;
      xv[4 * w + 1] = (double)lo[1] * sc;
      xv[4 * w + 2] = (double)hi[0] * sc;
      xv[4 * w + 3] = (double)hi[1] * sc;
    }
  }
}

template <int DT>
__device__ __forceinline__ void wave_dot_load(const void* __restrict__ x, const uint8_t* __restrict__ xs,
                                              int t, int d, const float* __restrict__ w,
                                              int i0, double (&xv)[8], float (&wv)[8]) {
  wave_dot_xload<DT>(x, xs, t, d, i0, xv);
  const float4 w0 = *(const float4*)(w + i0), w1 = *(const float4*)(w + i0 + 4);
  wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
  wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
}

template <int DT>
__device__ double wave_dot_t(const void* __restrict__ x, const uint8_t* __restrict__ xs,
                             int t, int d, const float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  double acc = 0.0;
  int i0 = 8 * lane;
  for (; i0 + 512 < d; i0 += 1024) {     // two iterations' loads issued before their fmas
    double xa[8], xb[8];
    float wa[8], wb[8];
    wave_dot_load<DT>(x, xs, t, d, w, i0, xa, wa);
    wave_dot_load<DT>(x, xs, t, d, w, i0 + 512, xb, wb);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fma(xa[q], (double)wa[q], acc);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fma(xb[q], (double)wb[q], acc);
  }
  if (i0 < d) {
    double xa[8];
    float wa[8];
    wave_dot_load<DT>(x, xs, t, d, w, i0, xa, wa);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fma(xa[q], (double)wa[q], acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  return acc;
}
__device__ __forceinline__ double wave_dot(const void* __restrict__ x, const uint8_t* __restrict__ xs,
                                           int dtype, int t, int d, const float* __restrict__ w) {
  return dtype == MOE_BF16 ? wave_dot_t<MOE_BF16>(x, xs, t, d, w) : wave_dot_t<MOE_MXFP8>(x, xs, t, d, w);
}

// ---------------------------------------------------------------------------
// Candidates, one wavefront per token: lower/upper screen bounds (bias added in
// fp64), L = k-th largest lower bound, candidates = experts whose upper bound reaches
// L, listed in ascending expert order.  tok_flag: 0 candidates listed, 1 more than
// kCandMax candidates (exact fallback), 2 non-finite screen value (flagged; ids 0..k-1).
// ---------------------------------------------------------------------------
template <int CD_NV>   // experts per lane (E <= 64 CD_NV)
__global__ __launch_bounds__(256) void screen_cand_kernel(
    const double* __restrict__ s, int nz, const double* __restrict__ xsqp, double* __restrict__ xnorm,
    const double* __restrict__ wnorm, const float* __restrict__ bias, const uint8_t* __restrict__ xs,
    int dtype, int T, int d, int E, int k, double cs, double tg, double ca,
    int32_t* __restrict__ cand, int* __restrict__ ccount, int* __restrict__ tok_flag,
    int32_t* __restrict__ ids, int* flag) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  // flush term scale: the token's largest MX block scale (1 for bf16)
  double sfac = 1.0;
  if (dtype == MOE_MXFP8) {
    int m = 0;
    for (int b = lane; b < d / 32; b += 64) m = max(m, (int)xs[(size_t)t * (d / 32) + b]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, __shfl_xor(m, off));
    sfac = ldexp(1.0, m - 127);
  }
  double xq = xsqp[t];
  for (int z = 1; z < nz; ++z) xq += xsqp[(size_t)z * T + t];
  const double xn = sqrt(xq);
  if (lane == 0) xnorm[t] = xn;
  double lo[CD_NV], up[CD_NV];
  bool finite = isfinite(xn);
#pragma unroll
  for (int i = 0; i < CD_NV; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const double b = bias ? (double)bias[e] : 0.0;
      double sv = s[(size_t)t * E + e];
      for (int z = 1; z < nz; ++z) sv += s[((size_t)z * T + t) * E + e];
      const double v = sv + b;
      const double bnd = cs * xn * wnorm[e] + tg * fabs(b) + ca * sfac;
      finite = finite && isfinite(v) && isfinite(bnd);
      lo[i] = v - bnd;
      up[i] = v + bnd;
    } else {
      lo[i] = -INFINITY;
      up[i] = -INFINITY;
    }
  }
  if (!__all(finite)) {
    if (lane == 0) {
      raise_flag(flag, kFlagNonFinite);
      tok_flag[t] = 2;
      ccount[t] = 0;
    }
    for (int r = lane; r < k; r += 64) ids[(size_t)t * k + r] = r;
    return;
  }
  // L: the k-th largest lower bound (k rounds of a wave-wide maximum, one removal each)
  uint32_t taken = 0;
  double L = -INFINITY;
  for (int r = 0; r < k; ++r) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < CD_NV; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (lo[i] > bv || (lo[i] == bv && e < bi))) {
        bv = lo[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
    L = bv;
  }
  int m = 0;
  uint64_t masks[CD_NV];
#pragma unroll
  for (int i = 0; i < CD_NV; ++i) {
    masks[i] = __ballot(lane + 64 * i < E && up[i] >= L);
    m += __popcll(masks[i]);
  }
  if (m > kCandMax) {
    if (lane == 0) {
      tok_flag[t] = 1;
      ccount[t] = 0;
    }
    return;
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < CD_NV; ++i) {
    if ((masks[i] >> lane) & 1u) {
      const int pos = base + __popcll(masks[i] & ((1ull << lane) - 1ull));
      cand[(size_t)t * kCandMax + pos] = lane + 64 * i;
    }
    base += __popcll(masks[i]);
  }
  if (lane == 0) {
    ccount[t] = m;
    tok_flag[t] = 0;
  }
}

// ---------------------------------------------------------------------------
// fp64 logits of the candidates: workgroup (expert e, 64 tokens) gathers the tokens
// whose candidate list holds e and gives each (token, slot) pair to one wavefront.
// cval[t][j] = wave_dot(x_t, w_e) + b_e.
// ---------------------------------------------------------------------------
// Candidate pairs grouped by expert, in (expert, token) order, with positions from
// counts and prefix sums only.  A workgroup owns 256 tokens, one per thread; LDS holds,
// per expert and wavefront, the 64-bit mask of the wavefront's tokens that list the
// expert (built with atomic OR, whose result does not depend on the order of the
// updates).  A pair's rank inside its workgroup is the number of set bits of earlier
// tokens; a replayed row that names an expert twice (flagged as bad ids) keeps only its
// first occurrence, whose value every later lookup finds first.
constexpr int PAIR_TOK = 256;

__device__ __forceinline__ uint32_t pair_mark(const int32_t* __restrict__ cand, int t, int m,
                                              uint64_t (*bits)[4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t me = 1ull << lane;
  uint32_t dup = 0;
  for (int j = 0; j < m; ++j) {
    const int e = cand[(size_t)t * kCandMax + j];
    if (atomicOr(&bits[e][wave], me) & me) dup |= 1u << j;
  }
  return dup;
}

// Per-workgroup pair counts: pblk[b][e] = number of tokens of workgroup b listing e.
__global__ __launch_bounds__(PAIR_TOK) void pair_count_kernel(const int32_t* __restrict__ cand,
                                                              const int* __restrict__ ccount, int T,
                                                              int E, int* __restrict__ pblk) {
  __shared__ uint64_t bits[kMaxExperts][4];
  for (int i = threadIdx.x; i < 4 * E; i += PAIR_TOK) bits[i >> 2][i & 3] = 0;
  __syncthreads();
  const int t = blockIdx.x * PAIR_TOK + threadIdx.x;
  pair_mark(cand, t, t < T ? ccount[t] : 0, bits);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PAIR_TOK)
    pblk[(size_t)blockIdx.x * E + e] = __popcll(bits[e][0]) + __popcll(bits[e][1]) +
                                       __popcll(bits[e][2]) + __popcll(bits[e][3]);
}

// pblk[b][e] -> exclusive prefix over workgroups (the workgroup's base inside expert e's
// range); cnt[E .. 2E] = exclusive prefix of the experts' totals (range starts, cnt[2E] =
// all pairs); cnt[2E+1 .. 3E+1] = exclusive prefix of the experts' chunk counts
// (ceil(total / rf_p); cnt[3E+1] = all chunks).  cnt[0 .. E) keeps the totals.
__global__ __launch_bounds__(1024) void pair_scan_kernel(int* __restrict__ pblk, int nblk,
                                                         int* __restrict__ cnt, int E, int rf_p) {
  static_assert(kMaxExperts <= 1024, "one expert per thread");
  __shared__ int wsum[2][16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int run = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nblk; b0 += 8) {   // eight loads in flight per thread
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b0 + u < nblk ? pblk[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < nblk) pblk[(size_t)(b0 + u) * E + e] = run;
        run += v[u];
      }
    }
    cnt[e] = run;
  }
  // exclusive prefixes over the experts of the totals and of the chunk counts: inclusive
  // scans within each wavefront, then of the wavefront sums
  const int tot = run, chn = e < E ? (run + rf_p - 1) / rf_p : 0;
  int a = tot, c = chn;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ua = __shfl_up(a, off), uc = __shfl_up(c, off);
    if (lane >= off) {
      a += ua;
      c += uc;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = a;
    wsum[1][wave] = c;
  }
  __syncthreads();
  int ba = 0, bc = 0;
  for (int w = 0; w < wave; ++w) {
    ba += wsum[0][w];
    bc += wsum[1][w];
  }
  if (e < E) {
    cnt[E + e] = ba + a - tot;
    cnt[2 * E + 1 + e] = bc + c - chn;
  }
  if (e == E - 1) {
    cnt[2 * E] = ba + a;
    cnt[3 * E + 1] = bc + c;
  }
}

// Each pair at: its expert's range start + the workgroup's base + its rank.
__global__ __launch_bounds__(PAIR_TOK) void pair_place_kernel(const int32_t* __restrict__ cand,
                                                              const int* __restrict__ ccount, int T,
                                                              int E, const int* __restrict__ pblk,
                                                              const int* __restrict__ cnt,
                                                              int32_t* __restrict__ pairs) {
  __shared__ uint64_t bits[kMaxExperts][4];
  for (int i = threadIdx.x; i < 4 * E; i += PAIR_TOK) bits[i >> 2][i & 3] = 0;
  __syncthreads();
  const int t = blockIdx.x * PAIR_TOK + threadIdx.x;
  const int m = t < T ? ccount[t] : 0;
  const uint32_t dup = pair_mark(cand, t, m, bits);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < m; ++j) {
    if ((dup >> j) & 1u) continue;
    const int e = cand[(size_t)t * kCandMax + j];
    int rank = __popcll(bits[e][wave] & below);
    for (int w = 0; w < wave; ++w) rank += __popcll(bits[e][w]);
    pairs[cnt[E + e] + pblk[(size_t)blockIdx.x * E + e] + rank] = t * kCandMax + j;
  }
}

// Chunks of at most RF_P pairs of one expert (8 to 64 by batch size) per workgroup,
// one wavefront per pair.  The chunk's gate column is staged in LDS when d fits and
// every pair reads it from there (wave_dot_lds), else every pair reads it from memory
// (wave_dot): which of the two computes a pair depends on d alone, never on the batch.
constexpr int RF_W = 8, RF_LDS_MAX = 16384;

// wave_dot with w in LDS: the same fma sequence (lane-strided blocks of 8, ascending,
// then the same butterfly) as wave_dot, hence the same bits; activation loads run up
// to 4 blocks ahead.
template <int DT>
__device__ double wave_dot_lds_t(const void* __restrict__ x, const uint8_t* __restrict__ xs,
                                 int t, int d, const float* w) {
  const int lane = threadIdx.x & 63;
  double acc = 0.0;
  int i0 = 8 * lane;
  for (; i0 + 3 * 512 < d; i0 += 4 * 512) {
    double xa[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) wave_dot_xload<DT>(x, xs, t, d, i0 + 512 * u, xa[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 w0 = *(const float4*)(w + i0 + 512 * u), w1 = *(const float4*)(w + i0 + 512 * u + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) acc = fma(xa[u][q], (double)wv[q], acc);
    }
  }
  for (; i0 < d; i0 += 512) {
    double xa[8];
    wave_dot_xload<DT>(x, xs, t, d, i0, xa);
    const float4 w0 = *(const float4*)(w + i0), w1 = *(const float4*)(w + i0 + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fma(xa[q], (double)wv[q], acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  return acc;
}
__device__ __forceinline__ double wave_dot_lds(const void* __restrict__ x, const uint8_t* __restrict__ xs,
                                               int dtype, int t, int d, const float* w) {
  return dtype == MOE_BF16 ? wave_dot_lds_t<MOE_BF16>(x, xs, t, d, w)
                           : wave_dot_lds_t<MOE_MXFP8>(x, xs, t, d, w);
}

__global__ __launch_bounds__(64 * RF_W) void screen_refine_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d,
    const float* __restrict__ wt, const float* __restrict__ bias, const int32_t* __restrict__ pairs,
    const int* __restrict__ cnt, int E, int RF_P, double* __restrict__ cval) {
  extern __shared__ __attribute__((aligned(16))) float wl[];   // d floats when d <= RF_LDS_MAX
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int* start = cnt + E;            // [E + 1] pair range starts
  const int* cst = cnt + 2 * E + 1;      // [E + 1] chunk starts
  const int nch = cst[E];
  const bool stage = d <= RF_LDS_MAX;
  for (int c = blockIdx.x; c < nch; c += gridDim.x) {
    int lo = 0, hi = E;                  // the expert e with cst[e] <= c < cst[e + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cst[mid] <= c) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int p0 = start[e] + (c - cst[e]) * RF_P;
    const int p1 = min(p0 + RF_P, start[e + 1]);
    if (stage) {
      __syncthreads();   // the previous chunk's readers are done
      const float* src = wt + (size_t)e * d;
      for (int i = 4 * threadIdx.x; i < d; i += 4 * 64 * RF_W) *(float4*)(wl + i) = *(const float4*)(src + i);
      __syncthreads();
    }
    const double b = bias ? (double)bias[e] : 0.0;
    for (int p = p0 + wave; p < p1; p += RF_W) {
      const int tj = pairs[p];
      const int t = tj / kCandMax;
      const double v = stage ? wave_dot_lds(x, xs, dtype, t, d, wl)
                             : wave_dot(x, xs, dtype, t, d, wt + (size_t)e * d);
      if (lane == 0) cval[tj] = bias ? v + b : v;
    }
  }
}

__device__ __forceinline__ bool sc_ranks_before(double av, int ae, double bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// ---------------------------------------------------------------------------
// Selection among the candidates, one wavefront per token: k rounds of a wave-wide
// arg-max on (fp64 logit desc, expert asc); certified when every adjacent pair of the
// top k, and rank k-1 against the best remaining candidate, stay ordered after
// widening each logit by its fp64 bound tg (||x|| ||w_e|| + |b_e|), with the relative
// margin 2^-45 that keeps the exact values more than an ulp apart.  Experts outside
// the candidate list are below k candidates by the screen bound.  Uncertified tokens
// get tok_flag 1 (exact fallback).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void screen_select_kernel(
    const int32_t* __restrict__ cand, const int* __restrict__ ccount, const double* __restrict__ cval,
    const double* __restrict__ xnorm, const double* __restrict__ wnorm,
    const float* __restrict__ bias, int T, int k, double tg, int* __restrict__ tok_flag,
    int32_t* __restrict__ ids, int* flag) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T || tok_flag[t] != 0) return;
  const int m = ccount[t];
  const bool live = lane < m;
  const int e = live ? cand[(size_t)t * kCandMax + lane] : 0x7fffffff;
  const double v = live ? cval[(size_t)t * kCandMax + lane] : -INFINITY;
  const double bnd = live ? tg * (xnorm[t] * wnorm[e] + (bias ? fabs((double)bias[e]) : 0.0)) : 0.0;
  if (!__all(!live || isfinite(v))) {
    if (lane == 0) {
      raise_flag(flag, kFlagNonFinite);
      tok_flag[t] = 2;
    }
    for (int r = lane; r < k; r += 64) ids[(size_t)t * k + r] = r;
    return;
  }
  bool taken = false, ok = true;
  double pv = 0.0, pb = 0.0;
  for (int r = 0; r < k; ++r) {
    double bv = (live && !taken) ? v : -INFINITY;
    int be = (live && !taken) ? e : 0x7fffffff;
    double bb = bnd;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      const double ob = __shfl_xor(bb, off);
      if (sc_ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
        bb = ob;
      }
    }
    if (e == be) taken = true;
    if (lane == 0) ids[(size_t)t * k + r] = be;
    if (r > 0) ok = ok && ((pv - pb) - (bv + bb) > 0x1p-45 * (fabs(pv) + fabs(bv)));
    pv = bv;
    pb = bb;
  }
  double u = (live && !taken) ? v + bnd : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) u = fmax(u, __shfl_xor(u, off));
  if (u > -INFINITY) ok = ok && ((pv - pb) - u > 0x1p-45 * (fabs(pv) + fabs(u)));
  if (lane == 0 && !ok) tok_flag[t] = 1;
}

// ---------------------------------------------------------------------------
// Weights, one wavefront per token: the fp64 logits of the k chosen experts (from the
// candidate list, or wave_dot when the token had too many candidates), then the
// restricted softmax exp(l_r - m) / sum_s exp(l_s - m) in fp64, sum in column order,
// one rounding to fp32.  With `weights_in` the caller's weights are copied instead
// (router replay); the logits are still computed and checked for finiteness.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void screen_weights_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d, int E,
    int k, const float* __restrict__ wt, const float* __restrict__ bias,
    const int32_t* __restrict__ cand, const int* __restrict__ ccount, const double* __restrict__ cval,
    const int32_t* __restrict__ ids, const float* __restrict__ weights_in,
    float* __restrict__ weights, int* flag) {
  __shared__ double lv[4][kMaxTopK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int m = ccount[t];
  for (int r = 0; r < k; ++r) {
    const int e = min(max(ids[(size_t)t * k + r], 0), E - 1);
    const bool hit = lane < m && cand[(size_t)t * kCandMax + lane] == e;
    const uint64_t hm = __ballot(hit);
    double v;
    if (hm) {
      v = cval[(size_t)t * kCandMax + (__ffsll((long long)hm) - 1)];
    } else {
      v = wave_dot(x, xs, dtype, t, d, wt + (size_t)e * d);
      if (bias) v = v + (double)bias[e];
    }
    if (lane == 0) lv[wave][r] = v;
  }
  if (lane != 0) return;
  bool finite = true;
  double mx = -INFINITY;
  for (int r = 0; r < k; ++r) {
    finite = finite && isfinite(lv[wave][r]);
    mx = fmax(mx, lv[wave][r]);
  }
  if (!finite) raise_flag(flag, kFlagNonFinite);
  float* wo = weights + (size_t)t * k;
  if (weights_in) {
    for (int r = 0; r < k; ++r) wo[r] = weights_in[(size_t)t * k + r];
    return;
  }
  double sum = 0.0;
  for (int r = 0; r < k; ++r) sum += exp(lv[wave][r] - mx);
  for (int r = 0; r < k; ++r) wo[r] = (float)(exp(lv[wave][r] - mx) / sum);
}

// fp64 logits of listed pairs without grouping them by expert (small batches): one
// wavefront per (token, slot < k).
__global__ __launch_bounds__(256) void direct_refine_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d, int k,
    const float* __restrict__ wt, const float* __restrict__ bias, const int32_t* __restrict__ cand,
    double* __restrict__ cval) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long p = (long long)blockIdx.x * 4 + wave;
  if (p >= (long long)T * k) return;
  const int t = (int)(p / k), j = (int)(p % k);
  const int e = cand[(size_t)t * kCandMax + j];
  const double v = wave_dot(x, xs, dtype, t, d, wt + (size_t)e * d);
  if (lane == 0) cval[(size_t)t * kCandMax + j] = bias ? v + (double)bias[e] : v;
}

// Router replay: the caller's ids are the candidate lists (validated: in range and
// distinct within the row, else flagged; clamped for the reads).
__global__ __launch_bounds__(256) void replay_cand_kernel(const int32_t* __restrict__ ids_in, int T,
                                                          int E, int k, int32_t* __restrict__ cand,
                                                          int* __restrict__ ccount, int* flag) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int32_t* idr = ids_in + (size_t)t * k;
  int bits = 0;
  for (int r = 0; r < k; ++r) {
    const int e = idr[r];
    if (e < 0 || e >= E) bits |= kFlagBadId;
    for (int q = 0; q < r; ++q)
      if (idr[q] == e) bits |= kFlagDupId;
    cand[(size_t)t * kCandMax + r] = min(max(e, 0), E - 1);
  }
  if (bits && flag) raise_flag(flag, bits);
  ccount[t] = k;
}

// ---------------------------------------------------------------------------
// Router replay with the plausibility filter (Composer 2 Technical Report, §6.2,
// paragraph on inference and weight sync): replayed expert e in column j stays when
// fl(l_e - l_(k)) >= ln tau on the correctly rounded logits, l_(k) being the logit of
// the router's own k-th choice; dropped columns are refilled, in column order, with
// the router's top-k ids in rank order that no kept column holds.  One wavefront per
// token, lane j < k owns column j.
// ---------------------------------------------------------------------------

// fp64 logit of (t, e) for a wave-uniform e: the value the learned path and plain
// replay use (the full fp64 gate GEMM, else the token's candidate value, else
// wave_dot + bias), so the weights below match theirs bit for bit.
__device__ __forceinline__ double filter_logit(const FilterArgs& a, int t, int e) {
  if (a.logits) return a.logits[(size_t)t * a.E + e];
  const int lane = threadIdx.x & 63;
  const bool hit = lane < a.ccount[t] && a.cand[(size_t)t * kCandMax + lane] == e;
  const uint64_t hm = __ballot(hit);
  if (hm) return a.cval[(size_t)t * kCandMax + (__ffsll((long long)hm) - 1)];
  const double v = wave_dot(a.x, a.xs, a.dtype, t, a.d, a.wt + (size_t)e * a.d);
  return a.bias ? v + (double)a.bias[e] : v;
}

// Lane j < k holds the final id f; writes the logits' softmax restricted to the row's
// ids, renormalised: max, exp(v - max) summed in column order, one division each
// (the arithmetic of the learned and replay weights).
__device__ __forceinline__ void filter_weights_row(const FilterArgs& a, int t, int f) {
  const int lane = threadIdx.x & 63;
  const bool live = lane < a.k;
  double v = 0.0;
  for (int j = 0; j < a.k; ++j) {
    const double lj = filter_logit(a, t, __shfl(f, j));
    if (lane == j) v = lj;
  }
  double mx = live ? v : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
  const double ex = exp(v - mx);
  double sum = 0.0;
  for (int j = 0; j < a.k; ++j) sum += __shfl(ex, j);
  if (!__all(!live || isfinite(v)) && lane == 0) raise_flag(a.flag, kFlagNonFinite);
  if (live) a.weights[(size_t)t * a.k + lane] = (float)(ex / sum);
}

__global__ __launch_bounds__(256) void filter_decide_kernel(FilterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const int k = a.k;
  const bool live = lane < k;
  const uint64_t kmask = (1ull << k) - 1ull;   // k <= 32
  int32_t* io = a.ids + (size_t)t * k;
  const int q = live ? a.ids_in[(size_t)t * k + lane] : -1;
  const int r = live ? io[lane] : -1;
  int bits = (live && (q < 0 || q >= a.E)) ? kFlagBadId : 0;
  for (int j = 0; j < k; ++j) {
    const int qj = __shfl(q, j);   // every lane takes part in the shuffle
    if (live && lane > j && qj == q) bits |= kFlagDupId;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) bits |= __shfl_xor(bits, off);
  if (bits) {   // rejected row: the router's own choice
    if (lane == 0) {
      raise_flag(a.flag, bits);
      a.tok_flag[t] = 0;
    }
    filter_weights_row(a, t, r);
    return;
  }
  const double lt = a.log_tau;
  uint64_t keepm;
  if (lt == -INFINITY) {
    keepm = kmask;
  } else if (lt == INFINITY) {
    keepm = 0;
  } else {
    double lq = 0.0;
    for (int j = 0; j < k; ++j) {
      const double v = filter_logit(a, t, __shfl(q, j));
      if (lane == j) lq = v;
    }
    const int ek = __shfl(r, k - 1);
    const double lk = filter_logit(a, t, ek);
    const double xn = a.xnorm[t];
    const double bk = a.tg * (xn * a.wnorm[ek] + (a.bias ? fabs((double)a.bias[ek]) : 0.0));
    bool keep = false, sure = true;
    if (live) {
      // |l~ - l| <= b for both logits (b includes the final rounding of l); the
      // relative 2^-50 covers the roundings of the difference and of the margin
      // itself, so keep / drop below hold for the exact fl(l_e - l_(k)).
      const double bq = a.tg * (xn * a.wnorm[q] + (a.bias ? fabs((double)a.bias[q]) : 0.0));
      const double dl = lq - lk;
      const double mg = bq + bk + 0x1p-50 * (fabs(lq) + fabs(lk) + fabs(lt)) + 0x1p-1000;
      if (isfinite(dl) && isfinite(mg)) {
        keep = dl - mg >= lt;
        sure = keep || dl + mg < lt;
      } else {
        raise_flag(a.flag, kFlagNonFinite);
      }
    }
    if (!__all(sure)) {
      if (lane == 0) a.tok_flag[t] = 1;
      return;
    }
    keepm = __ballot(keep) & kmask;
  }
  // refill: router ids in rank order that no kept column holds
  bool held = false;
  for (int j = 0; j < k; ++j) {
    const int qj = __shfl(q, j);
    if (((keepm >> j) & 1ull) && qj == r) held = true;
  }
  uint64_t avail = __ballot(live && !held) & kmask;
  const bool kept = (keepm >> lane) & 1ull;
  int src = 0;
  if (live && !kept) {
    const int n = __popcll(~keepm & kmask & ((1ull << lane) - 1ull));   // dropped columns before j
    for (int z = 0; z < n; ++z) avail &= avail - 1ull;
    src = __ffsll((long long)avail) - 1;
  }
  const int rv = __shfl(r, src);
  const int f = kept ? q : rv;
  if (live) io[lane] = f;
  if (lane == 0) a.tok_flag[t] = 0;
  filter_weights_row(a, t, f);
}

// Weights of the tokens the exact pass decided (their ids are final).
__global__ __launch_bounds__(256) void filter_weights_kernel(FilterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T || a.tok_flag[t] != 1) return;
  const int f = lane < a.k ? a.ids[(size_t)t * a.k + lane] : 0;
  filter_weights_row(a, t, f);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static double gamma_n(double n, double u) { return n * u / (1.0 - n * u); }

struct ScreenWs {
  double* logits;   // screen partial sums [parts][T][E]
  double* xsq;      // partial squared activation norms [parts][T]
  int* tok_flag;
  double* xnorm;
  double* wnorm;
  float* wt;
  uint16_t* planes;
  int32_t* cand;
  double* cval;
  int* ccount;
  int* pblk;        // per-workgroup pair counts, then bases [ceil(T / 256)][E]
  int* pcnt;        // totals [E], range starts [E + 1], chunk starts [E + 1]
  int32_t* pairs;   // candidate pairs t * kCandMax + j in (expert, token) order
};

static ScreenWs screen_ws_of(char* w, int T, int d, int E) {
  const RouteWs L = route_ws(T, d, E);
  ScreenWs s;
  s.logits = (double*)(w + L.screen);
  s.xsq = (double*)(w + L.sxsq);
  s.tok_flag = (int*)(w + L.tok_flag);
  s.xnorm = (double*)(w + L.xnorm);
  s.wnorm = (double*)(w + L.wnorm);
  s.wt = (float*)(w + L.wt);
  s.planes = (uint16_t*)(w + L.planes);
  s.cand = (int32_t*)(w + L.cand);
  s.cval = (double*)(w + L.cval);
  s.ccount = (int*)(w + L.ccount);
  s.pblk = (int*)(w + L.pblk);
  s.pcnt = (int*)(w + L.pcnt);
  s.pairs = (int32_t*)(w + L.pairs);
  return s;
}

// fp64 logits of every listed candidate pair (at most T * kCandMax pairs).
static moe_status refine_pairs(const void* x, const uint8_t* xs, int dtype, int T, int d, int E, int k,
                               const float* bias, const ScreenWs& S, hipStream_t s) {
  (void)k;
  if (T == 0) return MOE_OK;
  // about 8 pairs per token: aim at >= 1024 chunks
  int rf_p = 8;
  while (rf_p < 64 && (long long)rf_p * 2 * 1024 <= (long long)T * 8) rf_p *= 2;
  const int nblk = (T + PAIR_TOK - 1) / PAIR_TOK;
  pair_count_kernel<<<nblk, PAIR_TOK, 0, s>>>(S.cand, S.ccount, T, E, S.pblk);
  pair_scan_kernel<<<1, 1024, 0, s>>>(S.pblk, nblk, S.pcnt, E, rf_p);
  pair_place_kernel<<<nblk, PAIR_TOK, 0, s>>>(S.cand, S.ccount, T, E, S.pblk, S.pcnt, S.pairs);
  const long long nch_bound = ((long long)T * kCandMax + rf_p - 1) / rf_p + E;
  const size_t lds = d <= RF_LDS_MAX ? (size_t)d * sizeof(float) : 0;
  screen_refine_kernel<<<(unsigned)(nch_bound < 2048 ? nch_bound : 2048), 64 * RF_W, lds, s>>>(
      x, xs, dtype, T, d, S.wt, bias, S.pairs, S.pcnt, E, rf_p, S.cval);
  return launch_status();
}

// fp64 logits of the k listed ids per token (router replay, or the ids the fp64 gate
// chose): grouped by expert for large batches, one wavefront per pair for small ones.
static moe_status refine_ids(const void* x, const uint8_t* xs, int dtype, int T, int d, int E, int k,
                             const float* bias, const ScreenWs& S, hipStream_t s) {
  if (gate_split_launch(T, d, E)) {
    direct_refine_kernel<<<(unsigned)(((long long)T * k + 3) / 4), 256, 0, s>>>(x, xs, dtype, T, d, k, S.wt,
                                                                                bias, S.cand, S.cval);
    return launch_status();
  }
  return refine_pairs(x, xs, dtype, T, d, E, k, bias, S, s);
}

moe_status screen_route_select(const void* x, const uint8_t* xs, int dtype, int T, int d,
                               const float* w_gate, const float* bias, int E, int k, int32_t* ids,
                               char* w, hipStream_t s) {
  const ScreenWs S = screen_ws_of(w, T, d, E);
  int* flag = (int*)w;
  moe_status st;
  gate_prep_kernel<<<dim3((d + 63) / 64, (E + 63) / 64), 256, 0, s>>>(w_gate, d, E, S.wt, S.planes);
  gate_wnorm_kernel<<<E, 256, 0, s>>>(S.wt, d, E, S.wnorm);
  const int tiles = ((E + SC_E - 1) / SC_E) * ((T + SC_T - 1) / SC_T);
  const int nsteps = d / SC_K;
  const int nz = screen_parts(T, d, E);
  const int spart = (nsteps + nz - 1) / nz;
  const dim3 grid((E + SC_E - 1) / SC_E, (T + SC_T - 1) / SC_T, (nsteps + spart - 1) / spart);
  const unsigned nwg = (unsigned)tiles * grid.z;   // one-dimensional: see gate_screen_kernel
  if (dtype == MOE_BF16)
    gate_screen_kernel<MOE_BF16><<<nwg, SC_THR, 0, s>>>(x, xs, T, d, E, spart, S.planes, S.logits, S.xsq);
  else
    gate_screen_kernel<MOE_MXFP8><<<nwg, SC_THR, 0, s>>>(x, xs, T, d, E, spart, S.planes, S.logits, S.xsq);
  const int chunk = dtype == MOE_BF16 ? 64 : 32;
  const double tg = 2.0 * gamma_n(d + 1, 0x1p-53);
  const double cs = 2.0 * (gamma_n(3.0 * chunk, 0x1p-23) * (1.0 + 0x1p-6) + gamma_n(d + 1, 0x1p-53));
  const double ca = 2.0 * (4.0 * d + 64.0) * 0x1p-126;
  // the candidates add the K parts themselves (ascending part order)
  const int nzl = (int)grid.z;
#define MOE_CAND(NV)                                                                             \
  screen_cand_kernel<NV><<<(T + 3) / 4, 256, 0, s>>>(S.logits, nzl, S.xsq, S.xnorm, S.wnorm, bias, \
                                                     xs, dtype, T, d, E, k, cs, tg, ca, S.cand,     \
                                                     S.ccount, S.tok_flag, ids, flag)
  if (E <= 128) MOE_CAND(2);
  else if (E <= 256) MOE_CAND(4);
  else if (E <= 512) MOE_CAND(8);
  else MOE_CAND(16);
#undef MOE_CAND
  if ((st = refine_pairs(x, xs, dtype, T, d, E, k, bias, S, s)) != MOE_OK) return st;
  screen_select_kernel<<<(T + 3) / 4, 256, 0, s>>>(S.cand, S.ccount, S.cval, S.xnorm, S.wnorm, bias, T,
                                                   k, tg, S.tok_flag, ids, flag);
  return launch_status();
}

// The fp64 gate chose the ids (small batches): their fp64 logits for the weights.
moe_status chosen_ids_refine(const void* x, const uint8_t* xs, int dtype, int T, int d,
                             const float* w_gate, const float* bias, int E, int k, const int32_t* ids,
                             char* w, hipStream_t s) {
  const ScreenWs S = screen_ws_of(w, T, d, E);
  gate_prep_kernel<<<dim3((d + 63) / 64, (E + 63) / 64), 256, 0, s>>>(w_gate, d, E, S.wt, nullptr);
  replay_cand_kernel<<<(T + 255) / 256, 256, 0, s>>>(ids, T, E, k, S.cand, S.ccount, nullptr);
  return refine_ids(x, xs, dtype, T, d, E, k, bias, S, s);
}

moe_status screen_route_weights(const void* x, const uint8_t* xs, int dtype, int T, int d,
                                const float* bias, int E, int k, const int32_t* ids,
                                const float* weights_in, float* weights, char* w, hipStream_t s) {
  const ScreenWs S = screen_ws_of(w, T, d, E);
  screen_weights_kernel<<<(T + 3) / 4, 256, 0, s>>>(x, xs, dtype, T, d, E, k, S.wt, bias, S.cand,
                                                    S.ccount, S.cval, ids, weights_in, weights,
                                                    (int*)w);
  return launch_status();
}

moe_status screen_replay(const void* x, const uint8_t* xs, int dtype, int T, int d,
                         const float* w_gate, const float* bias, int E, int k, const int32_t* ids_in,
                         const float* weights_in, float* weights_out, char* w, hipStream_t s) {
  const ScreenWs S = screen_ws_of(w, T, d, E);
  gate_prep_kernel<<<dim3((d + 63) / 64, (E + 63) / 64), 256, 0, s>>>(w_gate, d, E, S.wt, nullptr);
  replay_cand_kernel<<<(T + 255) / 256, 256, 0, s>>>(ids_in, T, E, k, S.cand, S.ccount, (int*)w);
  moe_status st = refine_ids(x, xs, dtype, T, d, E, k, bias, S, s);
  if (st != MOE_OK) return st;
  return screen_route_weights(x, xs, dtype, T, d, bias, E, k, ids_in, weights_in, weights_out, w, s);
}

moe_status filter_launch(FilterArgs a, bool screened, char* w, int pass, hipStream_t s) {
  const RouteWs L = route_ws(a.T, a.d, a.E);
  a.xnorm = (const double*)(w + L.xnorm);
  a.wnorm = (const double*)(w + L.wnorm);
  a.tok_flag = (int*)(w + L.tok_flag);
  a.flag = (int*)w;
  if (screened) {
    const ScreenWs S = screen_ws_of(w, a.T, a.d, a.E);
    a.logits = nullptr;
    a.wt = S.wt;
    a.cand = S.cand;
    a.ccount = S.ccount;
    a.cval = S.cval;
  } else {
    a.logits = (const double*)(w + L.logits);
    a.wt = nullptr;
    a.cand = nullptr;
    a.ccount = nullptr;
    a.cval = nullptr;
  }
  const unsigned blocks = (unsigned)((a.T + 3) / 4);
  if (pass == 0)
    filter_decide_kernel<<<blocks, 256, 0, s>>>(a);
  else
    filter_weights_kernel<<<blocks, 256, 0, s>>>(a);
  return launch_status();
}

}  // namespace moe
