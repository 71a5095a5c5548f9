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
  if (t >= T || tok_flag[t] == 0) return;
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
  if (ws_bytes < route_ws(T, E).bytes) return MOE_ERR_WORKSPACE;
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
  const RouteWs L = route_ws(T, E);
  dim3 grid((E + GT_E - 1) / GT_E, (T + GT_M - 1) / GT_M);
  double* lg = (double*)(w + L.logits);
  double* xn = (double*)(w + L.xnorm);
  double* wn = (double*)(w + L.wnorm);
  if (dtype == MOE_BF16)
    gate_gemm_f64_kernel<MOE_BF16><<<grid, 256, 0, s>>>(x, xs, T, d, w_gate, bias, E, lg, xn, wn);
  else if (dtype == MOE_F32)
    gate_gemm_f64_kernel<MOE_F32><<<grid, 256, 0, s>>>(x, xs, T, d, w_gate, bias, E, lg, xn, wn);
  else
    gate_gemm_f64_kernel<MOE_MXFP8><<<grid, 256, 0, s>>>(x, xs, T, d, w_gate, bias, E, lg, xn, wn);
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
  const RouteWs L = route_ws(T, E);
  if ((st = launch_gate(x, x_scale, dtype, T, d, w_gate, bias, E, w, s)) != MOE_OK) return st;
  select_topk_kernel<<<(T + SEL_WAVES - 1) / SEL_WAVES, 256, 0, s>>>(
      (const double*)(w + L.logits), (const double*)(w + L.xnorm), (const double*)(w + L.wnorm),
      bias, T, E, k, two_gamma(d), ids, (int*)(w + L.tok_flag), flag);
  exact_fallback_kernel<<<T, 256, 0, s>>>(x, x_scale, dtype, T, d, w_gate, bias, E, k,
                                          (const int*)(w + L.tok_flag), ids, flag);
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
  const RouteWs L = route_ws(T, E);
  if ((st = launch_gate(x, x_scale, dtype, T, d, w_gate, bias, E, w, s)) != MOE_OK) return st;
  replay_kernel<<<(T + SEL_WAVES - 1) / SEL_WAVES, 256, 0, s>>>(
      (const double*)(w + L.logits), T, E, k, ids_in, weights_in, weights_out, (int*)w);
  return launch_status();
}
