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
constexpr int GT_E = 64;   // experts per gate tile
constexpr int GT_K = 16;   // reduction chunk staged in LDS

// logits[t][e] = sum_i x[t][i] * wg[i][e]  (+ bias[e]), fp64, i ascending, one fma per
// term; the bias is added last.  Rounding error of every output is at most
// gamma_{d+1} * (sum_i |x_i w_ie| + |b_e|) <= gamma_{d+1} * (||x_t|| ||w_e|| + |b_e|).
// The WGs of the first expert tile also write ||x_t||, those of the first token tile
// ||w_e|| (fp64 sums of squares over the same tiles).
__global__ __launch_bounds__(256) void gate_gemm_f64_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d,
    const float* __restrict__ wg, const float* __restrict__ bias, int E,
    double* __restrict__ logits, double* __restrict__ xnorm, double* __restrict__ wnorm) {
  __shared__ double sx[GT_K][GT_M + 1];
  __shared__ double sw[GT_K][GT_E + 1];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int t0 = blockIdx.y * GT_M, e0 = blockIdx.x * GT_E;
  const bool x_owner = (blockIdx.x == 0) && tid < GT_M;
  const bool w_owner = (blockIdx.y == 0) && tid >= 64 && tid < 64 + GT_E;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  double sq = 0.0;

  for (int k0 = 0; k0 < d; k0 += GT_K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = tid + 256 * i, m = l / GT_K, kk = l % GT_K;
      const int t = t0 + m, kx = k0 + kk;
      sx[kk][m] = (t < T && kx < d) ? load_act_f64(x, xs, dtype, (size_t)t, d, kx) : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = tid + 256 * i, kk = l / GT_E, ee = l % GT_E;
      const int e = e0 + ee, kw = k0 + kk;
      sw[kk][ee] = (e < E && kw < d) ? (double)wg[(size_t)kw * E + e] : 0.0;
    }
    __syncthreads();
    if (x_owner) {
#pragma unroll
      for (int kk = 0; kk < GT_K; ++kk) sq = fma(sx[kk][tid], sx[kk][tid], sq);
    }
    if (w_owner) {
#pragma unroll
      for (int kk = 0; kk < GT_K; ++kk) sq = fma(sw[kk][tid - 64], sw[kk][tid - 64], sq);
    }
#pragma unroll
    for (int kk = 0; kk < GT_K; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sx[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sw[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (x_owner && t0 + tid < T) xnorm[t0 + tid] = sqrt(sq);
  if (w_owner && e0 + tid - 64 < E) wnorm[e0 + tid - 64] = sqrt(sq);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e >= E) continue;
      double v = acc[i][j];
      if (bias) v = v + (double)bias[e];
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
  gate_gemm_f64_kernel<<<grid, 256, 0, s>>>(x, xs, dtype, T, d, w_gate, bias, E,
                                            (double*)(w + L.logits), (double*)(w + L.xnorm),
                                            (double*)(w + L.wnorm));
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
