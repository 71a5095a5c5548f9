// MXFP8 backward of the expert FFN (Composer 2 Technical Report, section 6.1 "Kernels":
// the MoE backward runs in MXFP8, E4M3 values with one E8M0 scale per block of 32;
// Figure 10: the layer is trained as one grouped-GEMM flow).  Every backward GEMM takes
// both operands in MXFP8 blocked along its own reduction dimension, on the block-scaled
// matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4):
//
//   data half (reductions over d or I, so every activation operand is quantised per
//   row and a token's dx does not depend on the other tokens):
//     dq   = MX_row(d_out)                       [rows][d]
//     dh   = dq  . W2t^T,  W2t[e] = MX_d(W2[e]^T)  [I][d]
//     da, dg = dh g silu'(a), dh silu(a)          (a, g: the forward's pre-activations)
//     dgq  = MX_row(da | dg)                     [rows][2I]
//     dx   = dgq . W13t^T, W13t[e] = MX_I([W1[e]^T | W3[e]^T])  [d][2I]
//   weights half (reductions over an expert's rows; operands quantised along the rows in
//   blocks of 32 from the expert's first row, stored transposed, each expert's rows
//   padded with zeros to a multiple of 128):
//     dW2[e]      = MX_rows(d_out)^T . MX_rows(hq)    (hq: the forward's MXFP8 h)
//     dW1|dW3[e]  = MX_rows(da | dg)^T . MX_rows(x)
//
// Block scales take the smallest power of two with amax / X <= 448 (no element
// saturates) and elements round to the nearest E4M3 value (ties to even), the rule of
// the forward's h.  Every output has one fixed reduction order (K ascending in 64-wide
// scaled MFMAs, no split-K, no atomics): the gradients are bitwise reproducible.
#include <math.h>

#include "moe_internal.h"
#include "mx_common.h"

namespace moe {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Padded K starts of the segments: kst[s] = sum over earlier segments of their row
// counts rounded up to 128, kst[S] = the total.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void mx_kst_kernel(const int* __restrict__ rowcount, int S,
                                                      int* __restrict__ kst) {
  __shared__ int c[kMaxExperts + 2];
  for (int s = threadIdx.x; s < S; s += blockDim.x) c[s] = (rowcount[s] + 127) / 128 * 128;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int s = 0; s < S; ++s) {
      kst[s] = run;
      run += c[s];
    }
    kst[S] = run;
  }
}

// ---------------------------------------------------------------------------
// Row quantiser: fp32 or bf16 rows [R][C] (C % 32 == 0) -> MXFP8 codes [R][C] and scales
// [R][C / 32], one 32-block per thread.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void mx_rowq_kernel(const void* __restrict__ src, long long R, int C,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int nb = C / 32;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * nb) return;
  const long long r = idx / nb;
  const int b = (int)(idx % nb);
  float v[32];
  if (BF16) {
    const u32x4_t* p = (const u32x4_t*)((const uint16_t*)src + r * C + 32 * b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t u = p[q];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[8 * q + 2 * w] = bf16_to_f32((uint16_t)(u[w] & 0xffffu));
        v[8 * q + 2 * w + 1] = bf16_to_f32((uint16_t)(u[w] >> 16));
      }
    }
  } else {
    const float4* p = (const float4*)((const float*)src + r * C + 32 * b);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 t = p[q];
      v[4 * q] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int se;
  uint32_t scode;
  mx_block_scale(amax, se, scode);
  u32x4_t w[2];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q >> 2][q & 3] = mx_pack4(ldexpf(v[4 * q], -se), ldexpf(v[4 * q + 1], -se), ldexpf(v[4 * q + 2], -se),
                                ldexpf(v[4 * q + 3], -se));
  uint8_t* out = codes + r * C + 32 * b;
  *(u32x4_t*)out = w[0];
  *(u32x4_t*)(out + 16) = w[1];
  scales[r * nb + b] = (uint8_t)scode;
}

// ---------------------------------------------------------------------------
// Column quantiser: 32-row blocks of a source matrix, quantised along the rows (one MX
// block per column) and written transposed: output row c holds the 32 codes at K offset
// kout, and one scale at kout / 32.  Sources: bf16 rows, fp32 rows, MXFP8 rows (codes and
// scales along the row), or the fp32 pre-activations a | g, from which h = silu(a) g is
// formed and quantised per row along I first (the forward's hq).
// Segment mode (kst != null): block q covers padded K positions 32 q .. 32 q + 31, in the
// segment s with kst[s] <= 32 q < kst[s + 1]; its rows are dispatched rows
// rowstart[s] + r (gathered to tokens when `gather`), rows past the segment read as zero.
// Matrix mode (kst == null): block q is rows 32 (q % (R / 32)) .. of matrix q / (R / 32),
// written to matrix s's output at K offset col0 + its first row.
// ---------------------------------------------------------------------------
enum { kColBf16 = 0, kColF32 = 1, kColMx = 2, kColPre = 3 };
struct ColqArgs {
  const void* src;
  const uint8_t* src_s;     // MXFP8 source scales, src_ld / 32 per row; NVFP4 block scales
  const float* src_r;       // NVFP4 sources: fp32 scale per source row
  long long src_ld;         // elements per source row
  long long src_mat;        // matrix mode: elements between matrices
  int gather;               // segment mode: source row of dispatched row j = its token
  const int32_t* perm;
  int k, T;
  long long Tk;
  const int* rowstart;
  const int* rowcount;
  const int* kst;
  int S, R, C;
  uint8_t* out;
  uint8_t* out_s;
  long long out_ld;         // bytes per output row (a multiple of 32)
  long long out_mat;        // matrix mode: bytes between output matrices
  int col0;
  int* flag;
};
constexpr int CQ_COLS = 256;

template <int KIND>
__global__ __launch_bounds__(256) void mx_colq_kernel(ColqArgs a) {
  __shared__ float t[32][CQ_COLS + 1];
  __shared__ long long srow[32];
  const int q = blockIdx.x;
  const int c0 = blockIdx.y * CQ_COLS;
  int s, r0;
  long long kout;
  uint8_t* obase;
  uint8_t* osbase;
  if (a.kst) {
    const int kq = 32 * q;
    if (kq >= a.kst[a.S]) return;
    int lo = 0, hi = a.S;   // kst[lo] <= kq < kst[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.kst[mid] <= kq) lo = mid; else hi = mid;
    }
    s = lo;
    r0 = kq - a.kst[s];
    kout = kq;
    obase = a.out;
    osbase = a.out_s;
  } else {
    const int per = a.R / 32;
    s = q / per;
    r0 = (q % per) * 32;
    if (s >= a.S) return;
    kout = a.col0 + r0;
    obase = a.out + s * a.out_mat;
    osbase = a.out_s + s * (a.out_mat / 32);
  }
  if (threadIdx.x < 32) {
    const int r = r0 + threadIdx.x;
    long long off = -1;
    if (a.kst) {
      if (r < a.rowcount[s]) {
        const long long j = (long long)a.rowstart[s] + r;
        long long src = j;
        if (a.gather) {
          src = j >= a.Tk ? j - a.Tk : (long long)(a.perm[j] / a.k);
          if (src < 0 || src >= a.T) {
            raise_flag(a.flag, kFlagCorrupt);
            src = 0;
          }
        }
        off = src * a.src_ld;
      }
    } else {
      off = s * a.src_mat + (long long)r * a.src_ld;
    }
    srow[threadIdx.x] = off;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 32 * CQ_COLS; i += 256) {
    const int rr = i / CQ_COLS, cc = i % CQ_COLS, c = c0 + cc;
    const long long off = srow[rr];
    float v = 0.0f;
    if (off >= 0 && c < a.C) {
      if (KIND == kColBf16) {
        v = bf16_to_f32(((const uint16_t*)a.src)[off + c]);
      } else if (KIND == kColF32) {
        v = ((const float*)a.src)[off + c];
      } else if (KIND == kColMx) {
        const uint32_t code = ((const uint8_t*)a.src)[off + c];
        const int sc = (int)a.src_s[off / 32 + c / 32];
        v = ldexpf(e4m3_to_f32(code), sc - 127);
      } else {
        const float av = ((const float*)a.src)[off + c];
        const float gv = ((const float*)a.src)[off + a.C + c];
        v = silu_f32(av) * gv;
      }
    }
    t[rr][cc] = v;
  }
  __syncthreads();
  if (KIND == kColPre) {
    // the forward's h: each row's 32-feature blocks quantised along the row
    const int rr = threadIdx.x >> 3, b = threadIdx.x & 7;
    float amax = 0.0f;
#pragma unroll 8
    for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(t[rr][32 * b + u]));
    int se;
    uint32_t scode;
    mx_block_scale(amax, se, scode);
#pragma unroll 8
    for (int u = 0; u < 32; u += 4) {
      float* p = &t[rr][32 * b + u];
      const uint32_t w = mx_pack4(ldexpf(p[0], -se), ldexpf(p[1], -se), ldexpf(p[2], -se), ldexpf(p[3], -se));
#pragma unroll
      for (int z = 0; z < 4; ++z) p[z] = ldexpf(e4m3_to_f32((w >> (8 * z)) & 0xffu), se);
    }
    __syncthreads();
  }
  const int c = c0 + threadIdx.x;
  if (c >= a.C) return;
  float amax = 0.0f;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(t[i][threadIdx.x]));
  int se;
  uint32_t scode;
  mx_block_scale(amax, se, scode);
  u32x4_t w[2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i >> 2][i & 3] = mx_pack4(ldexpf(t[4 * i][threadIdx.x], -se), ldexpf(t[4 * i + 1][threadIdx.x], -se),
                                ldexpf(t[4 * i + 2][threadIdx.x], -se), ldexpf(t[4 * i + 3][threadIdx.x], -se));
  uint8_t* o = obase + (long long)c * a.out_ld + kout;
  *(u32x4_t*)o = w[0];
  *(u32x4_t*)(o + 16) = w[1];
  osbase[(long long)c * (a.out_ld / 32) + kout / 32] = (uint8_t)scode;
}

// ---------------------------------------------------------------------------
// Column quantiser in 128-row blocks (segment mode: the dispatched-row operands; matrix
// mode: the weights), 64 columns per workgroup: whole 16-byte source chunks per load,
// and the four 32-row blocks of a column written by four neighbouring lanes as one
// 128-byte run of its output row (plus one 4-byte store of their scales).  Every 32-row
// block is quantised exactly as in mx_colq_kernel (same decode, scale rule and
// encoding), so both give the same bytes; segments start at multiples of 128 padded
// rows, so a workgroup never straddles two.
// ---------------------------------------------------------------------------
constexpr int C4_R = 128, C4_C = 64;

template <int KIND>
__global__ __launch_bounds__(256) void mx_colq4_kernel(ColqArgs a) {
  __shared__ float t[C4_R][C4_C + 1];
  __shared__ long long srow[C4_R];
  const int c0 = blockIdx.y * C4_C;
  int s, r0;
  long long kout;
  uint8_t* obase;
  uint8_t* osbase;
  if (a.kst) {   // segment mode: padded K positions kout .. kout + 127 of one segment
    const int kq = C4_R * blockIdx.x;
    if (kq >= a.kst[a.S]) return;
    int lo = 0, hi = a.S;   // kst[lo] <= kq < kst[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.kst[mid] <= kq) lo = mid; else hi = mid;
    }
    s = lo;
    r0 = kq - a.kst[s];
    kout = kq;
    obase = a.out;
    osbase = a.out_s;
  } else {       // matrix mode: rows r0 .. r0 + 127 of matrix s
    const int per = a.R / C4_R;
    s = blockIdx.x / per;
    r0 = (blockIdx.x % per) * C4_R;
    if (s >= a.S) return;
    kout = a.col0 + r0;
    obase = a.out + s * a.out_mat;
    osbase = a.out_s + s * (a.out_mat / 32);
  }
  const int tid = threadIdx.x;
  if (tid < C4_R) {
    const int r = r0 + tid;
    long long off = -1;
    if (!a.kst) {
      off = s * a.src_mat + (long long)r * a.src_ld;
    } else if (r < a.rowcount[s]) {
      const long long j = (long long)a.rowstart[s] + r;
      long long src = j;
      if (a.gather) {
        src = j >= a.Tk ? j - a.Tk : (long long)(a.perm[j] / a.k);
        if (src < 0 || src >= a.T) {
          raise_flag(a.flag, kFlagCorrupt);
          src = 0;
        }
      }
      off = src * a.src_ld;
    }
    srow[tid] = off;
  }
  __syncthreads();
  // ---- loads: chunks of EPC elements (16 bytes of the source), NI per thread, all
  //      issued before the first is decoded; a chunk outside the source (padding row,
  //      column past C) loads the source's first chunk instead and is stored as zeros ----
  constexpr int EPC = KIND == kColBf16 ? 8 : KIND == kColMx ? 16 : 4;
  constexpr int CPR = C4_C / EPC;   // chunks per row
  constexpr int NI = C4_R * CPR / 256;
  static_assert(C4_R * CPR % 256 == 0, "whole chunks per thread");
  u32x4_t qa[NI], qg[NI];   // qg: the g half of a pre-activation row (kColPre)
  int sc[NI];
  bool ok[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int i = tid + 256 * n;
    const int rr = i / CPR, c = c0 + (i % CPR) * EPC;
    const long long off = srow[rr];
    ok[n] = off >= 0 && c < a.C;
    const long long o = ok[n] ? off + c : 0;
    if (KIND == kColBf16) {
      qa[n] = *(const u32x4_t*)((const uint16_t*)a.src + o);
    } else if (KIND == kColMx) {
      qa[n] = *(const u32x4_t*)((const uint8_t*)a.src + o);
      sc[n] = (int)a.src_s[o / 32];
    } else {
      qa[n] = *(const u32x4_t*)((const float*)a.src + o);
      if (KIND == kColPre) qg[n] = *(const u32x4_t*)((const float*)a.src + o + a.C);
    }
  }
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int i = tid + 256 * n;
    const int rr = i / CPR, cc = (i % CPR) * EPC;
    float v[EPC];
    if (KIND == kColBf16) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = bf16_to_f32((uint16_t)(qa[n][u >> 1] >> (16 * (u & 1))));
    } else if (KIND == kColF32) {
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __uint_as_float(qa[n][u]);
    } else if (KIND == kColMx) {
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = ldexpf(e4m3_to_f32((qa[n][u >> 2] >> (8 * (u & 3))) & 0xffu), sc[n] - 127);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = silu_f32(__uint_as_float(qa[n][u])) * __uint_as_float(qg[n][u]);
    }
#pragma unroll
    for (int u = 0; u < EPC; ++u) t[rr][cc + u] = ok[n] ? v[u] : 0.0f;
  }
  __syncthreads();
  if (KIND == kColPre) {
    // the forward's h: each row's 32-feature blocks quantised along the row
    const int rr = tid >> 1, b = tid & 1;
    float amax = 0.0f;
#pragma unroll 8
    for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(t[rr][32 * b + u]));
    int se;
    uint32_t scode;
    mx_block_scale(amax, se, scode);
#pragma unroll 8
    for (int u = 0; u < 32; u += 4) {
      float* p = &t[rr][32 * b + u];
      const uint32_t w = mx_pack4(ldexpf(p[0], -se), ldexpf(p[1], -se), ldexpf(p[2], -se), ldexpf(p[3], -se));
#pragma unroll
      for (int z = 0; z < 4; ++z) p[z] = ldexpf(e4m3_to_f32((w >> (8 * z)) & 0xffu), se);
    }
    __syncthreads();
  }
  // ---- lane (column cl, block g): rows 32 g .. 32 g + 31 of column c0 + cl ----
  const int cl = tid >> 2, g = tid & 3, c = c0 + cl;
  float amax = 0.0f;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(t[32 * g + i][cl]));
  int se;
  uint32_t scode;
  mx_block_scale(amax, se, scode);
  u32x4_t w[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 32 * g + 4 * i;
    w[i >> 2][i & 3] = mx_pack4(ldexpf(t[r][cl], -se), ldexpf(t[r + 1][cl], -se), ldexpf(t[r + 2][cl], -se),
                                ldexpf(t[r + 3][cl], -se));
  }
  // the four scale codes of the column, gathered on its first lane
  const uint32_t s1 = __shfl_down(scode, 1), s2 = __shfl_down(scode, 2), s3 = __shfl_down(scode, 3);
  if (c >= a.C) return;
  uint8_t* o = obase + (long long)c * a.out_ld + kout + 32 * g;
  *(u32x4_t*)o = w[0];
  *(u32x4_t*)(o + 16) = w[1];
  if (g == 0)
    *(uint32_t*)(osbase + (long long)c * (a.out_ld / 32) + kout / 32) = scode | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

// ---------------------------------------------------------------------------
// Column quantiser for the operands of an NVFP4 layer (same blocks and outputs as
// mx_colq_kernel), on values held exactly in float64: an NVFP4 value E2M1 x E4M3 x row
// scale has up to 30 significant bits.
//   kColNvDec (segment mode): decoded rows E2M1 x E4M3 in fp16 [rows][C] (the forward
//             quantizer's output) times the fp32 scale of the source row, src_r[row];
//   kColNvW (matrix mode): K-blocked NVFP4 weight matrices of R rows x C columns (codes
//             [R/32][C/64][32][32 bytes], block scales [R/32][C/64][32][4 bytes]) with
//             one fp32 scale per row.
// ---------------------------------------------------------------------------
enum { kColNvDec = 4, kColNvW = 5 };

__device__ __forceinline__ double e2m1_f64(uint32_t c) {
  const double m[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double v = m[c & 7u];
  return (c & 8u) ? -v : v;
}

template <int KIND>
__global__ __launch_bounds__(256) void mx_colq_nv_kernel(ColqArgs a) {
  __shared__ double t[32][CQ_COLS + 1];
  __shared__ long long srow[32];   // source row (over all matrices in matrix mode), -1: padding
  const int q = blockIdx.x;
  const int c0 = blockIdx.y * CQ_COLS;
  int s, r0;
  long long kout;
  uint8_t* obase;
  uint8_t* osbase;
  if (a.kst) {
    const int kq = 32 * q;
    if (kq >= a.kst[a.S]) return;
    int lo = 0, hi = a.S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.kst[mid] <= kq) lo = mid; else hi = mid;
    }
    s = lo;
    r0 = kq - a.kst[s];
    kout = kq;
    obase = a.out;
    osbase = a.out_s;
  } else {
    const int per = a.R / 32;
    s = q / per;
    r0 = (q % per) * 32;
    if (s >= a.S) return;
    kout = a.col0 + r0;
    obase = a.out + s * a.out_mat;
    osbase = a.out_s + s * (a.out_mat / 32);
  }
  if (threadIdx.x < 32) {
    const int r = r0 + threadIdx.x;
    long long row = -1;
    if (a.kst) {
      if (r < a.rowcount[s]) {
        const long long j = (long long)a.rowstart[s] + r;
        row = j;
        if (a.gather) {
          row = j >= a.Tk ? j - a.Tk : (long long)(a.perm[j] / a.k);
          if (row < 0 || row >= a.T) {
            raise_flag(a.flag, kFlagCorrupt);
            row = 0;
          }
        }
      }
    } else {
      row = (long long)s * a.R + r;
    }
    srow[threadIdx.x] = row;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 32 * CQ_COLS; i += 256) {
    const int rr = i / CQ_COLS, cc = i % CQ_COLS, c = c0 + cc;
    const long long row = srow[rr];
    double v = 0.0;
    if (row >= 0 && c < a.C) {
      if (KIND == kColNvDec) {
        const uint16_t bits = ((const uint16_t*)a.src)[row * a.C + c];
        v = (double)(float)__builtin_bit_cast(_Float16, bits) * (double)a.src_r[row];
      } else {
        const long long m = row / a.R;
        const int r = (int)(row % a.R);
        const long long tile = (long long)(r / 32) * (a.C / 64) + c / 64;
        const uint8_t* codes = (const uint8_t*)a.src + m * ((long long)a.R * a.C / 2);
        const uint8_t* sc = a.src_s + m * ((long long)a.R * a.C / 16);
        const uint32_t byte = codes[tile * 1024 + (r % 32) * 32 + (c % 64) / 2];
        const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 15u);
        const uint32_t scode = sc[tile * 128 + (r % 32) * 4 + (c % 64) / 16];
        v = e2m1_f64(code) * (double)e4m3_to_f32(scode) * (double)a.src_r[row];
      }
    }
    t[rr][cc] = v;
  }
  __syncthreads();
  const int c = c0 + threadIdx.x;
  if (c >= a.C) return;
  double amax = 0.0;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(t[i][threadIdx.x]));
  int se;
  uint32_t scode;
  mx_block_scale_f64(amax, se, scode);
  u32x4_t w[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t u = 0;
#pragma unroll
    for (int z = 0; z < 4; ++z) u |= e4m3_rne_f64(ldexp(t[4 * i + z][threadIdx.x], -se)) << (8 * z);
    w[i >> 2][i & 3] = u;
  }
  uint8_t* o = obase + (long long)c * a.out_ld + kout;
  *(u32x4_t*)o = w[0];
  *(u32x4_t*)(o + 16) = w[1];
  osbase[(long long)c * (a.out_ld / 32) + kout / 32] = (uint8_t)scode;
}

// ---------------------------------------------------------------------------
// Grouped MXFP8 GEMM of the backward, C = A . B^T with both operands K-contiguous MXFP8
// rows.  Tile 128 x 128, four wavefronts (2 x 2), each 64 x 64 as 2 x 2 MFMA blocks of
// 32 x 32; K advances 128 bytes a step (registers -> LDS -> two 64-wide scaled MFMAs).
//   MB_DH: tiles over (segment, row tile, column tile) of the dispatched rows: A = dq rows,
//          B = W2t of the segment's expert [I][d]; epilogue: SwiGLU backward into da | dg.
//   MB_DX: the same tiles: A = dgq rows, B = W13t [d][2I]; epilogue: fp32 dx rows.
//   MB_DW: tiles over (segment, M tile, N tile): A, B = transposed operands [M][Kp],
//          [N][Kp] over the segment's padded K range; epilogue: the expert's fp32 weight
//          gradient (rows below `split` into dw_a, the others into dw_b).
// ---------------------------------------------------------------------------
enum { MB_DH = 0, MB_DX = 1, MB_DW = 2 };
struct MxBwdGemm {
  const uint8_t* a;
  const uint8_t* as;
  long long lda;            // bytes per A row (scales: lda / 32 per row)
  const uint8_t* b;
  const uint8_t* bs;
  long long ldb;
  long long b_e;            // MB_DH / MB_DX: bytes between the experts' B matrices
  const uint8_t* sb;        // MB_DH / MB_DX: the shared expert's B
  const uint8_t* sbs;
  int K;                    // MB_DH / MB_DX reduction length
  int M, N, MT, NT;
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  const int* kst;
  int S, E;
  const float* pre;         // MB_DH: [rows][2I]
  int I;
  float* out;               // MB_DH: da | dg [rows][2I]; MB_DX: dx rows [rows][N]
  long long ldo;
  float* dw_a;
  float* dw_b;
  float* sdw_a;
  float* sdw_b;
  int split;
  int* flag;
};
constexpr int BB_T = 128, BB_K = 128, BB_LDS = BB_K + 16, BB_THR = 256;

template <int MODE>
__global__ __launch_bounds__(BB_THR) void mx_bwd_gemm_kernel(MxBwdGemm g) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[BB_T * BB_LDS];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BB_T * BB_LDS];
  __shared__ uint32_t sAs[BB_T];
  __shared__ uint32_t sBs[BB_T];

  int s, row0 = 0, mrows = BB_T, m0 = 0, n0, K;
  long long kbase = 0;
  if (MODE == MB_DW) {
    const int per = g.MT * g.NT;
    int tile;
    if (!xcd_tile<0>(g.S * per, tile)) return;
    s = tile / per;
    const int rem = tile % per;
    m0 = (rem / g.NT) * BB_T;
    n0 = (rem % g.NT) * BB_T;
    kbase = g.kst[s];
    K = g.kst[s + 1] - g.kst[s];
  } else {
    const int total = g.mstart[g.S] * g.NT;
    int tile;
    if (!xcd_tile<0>(total, tile)) return;
    int lo = 0, hi = g.S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.mstart[mid] * g.NT <= tile) lo = mid; else hi = mid;
    }
    s = lo;
    const int mtiles = g.mstart[s + 1] - g.mstart[s];
    const int local = tile - g.mstart[s] * g.NT;
    const int grp = local / (kGroupM * g.NT), rem = local % (kGroupM * g.NT);
    const int gm = min(kGroupM, mtiles - grp * kGroupM);
    const int nt = rem / gm, mt = grp * kGroupM + rem % gm;
    row0 = g.rowstart[s] + mt * BB_T;
    mrows = min(BB_T, g.rowcount[s] - mt * BB_T);
    n0 = nt * BB_T;
    K = g.K;
  }
  const bool is_shared = (s == g.E);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = tid >> 3, lc = (tid & 7) * 16;   // loader: rows lr + 32 i, 16-byte chunk lc
  constexpr int LD = BB_T / 32;                    // rows per loader thread per operand

  // A and B row pointers (byte offsets of row starts at K = kbase)
  const uint8_t* aptr[LD];
  const uint8_t* bptr[LD];
  const uint8_t* bmat = g.b;
  const uint8_t* bsmat = g.bs;
  if (MODE != MB_DW) {
    bmat = is_shared ? g.sb : g.b + (long long)s * g.b_e;
    bsmat = is_shared ? g.sbs : g.bs + (long long)s * (g.b_e / 32);
  }
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int r = lr + 32 * i;
    long long ar;
    if (MODE == MB_DW)
      ar = m0 + r;
    else
      ar = (long long)row0 + (r < mrows ? r : 0);
    aptr[i] = g.a + ar * g.lda + kbase + lc;
    bptr[i] = bmat + (long long)(n0 + r) * g.ldb + kbase + lc;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;

  // scale words of a step: thread t < 128 stages A row t's four scale bytes, threads
  // 128 .. 255 those of B row t - 128
  const uint8_t* sptr;
  {
    const int sr = tid & (BB_T - 1);
    if (tid < BB_T) {
      const long long row = MODE == MB_DW ? (long long)(m0 + sr) : (long long)row0 + (sr < mrows ? sr : 0);
      sptr = g.as + row * (g.lda / 32) + kbase / 32;
    } else {
      sptr = bsmat + (long long)(n0 + sr) * (g.ldb / 32) + kbase / 32;
    }
  }

  u32x4_t ra[LD], rb[LD];
  uint32_t rs = 0;
  if (K > 0) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      ra[i] = *(const u32x4_t*)(aptr[i]);
      rb[i] = *(const u32x4_t*)(bptr[i]);
    }
    rs = *(const uint32_t*)sptr;
  }
  for (int k0 = 0; k0 < K; k0 += BB_K) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      *(u32x4_t*)&sA[(lr + 32 * i) * BB_LDS + lc] = ra[i];
      *(u32x4_t*)&sB[(lr + 32 * i) * BB_LDS + lc] = rb[i];
    }
    if (tid < BB_T) sAs[tid] = rs; else sBs[tid - BB_T] = rs;
    __syncthreads();
    const int kn = k0 + BB_K;
    if (kn < K) {
#pragma unroll
      for (int i = 0; i < LD; ++i) {
        ra[i] = *(const u32x4_t*)(aptr[i] + kn);
        rb[i] = *(const u32x4_t*)(bptr[i] + kn);
      }
      rs = *(const uint32_t*)(sptr + kn / 32);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kc = sub * 64 + (lane >> 5) * 16;
      const int sh = 8 * (sub * 2 + (lane >> 5));
      i32x8_t af[2], bf[2];
      int sa[2], sb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + (lane & 31);
        const u32x4_t u0 = *(const u32x4_t*)&sA[row * BB_LDS + kc];
        const u32x4_t u1 = *(const u32x4_t*)&sA[row * BB_LDS + kc + 32];
        af[mb] = (i32x8_t){(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                           (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
        sa[mb] = (int)((sAs[row] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = wn * 64 + nb * 32 + (lane & 31);
        const u32x4_t u0 = *(const u32x4_t*)&sB[row * BB_LDS + kc];
        const u32x4_t u1 = *(const u32x4_t*)&sB[row * BB_LDS + kc + 32];
        bf[nb] = (i32x8_t){(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                           (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
        sb[nb] = (int)((sBs[row] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mb], bf[nb], acc[mb][nb], 0, 0, 0,
                                                                       sa[mb], 0, sb[nb]);
    }
    __syncthreads();
  }

  // ---- epilogue.  Accumulator element v of a lane is C[i][j], j = lane % 32,
  //      i = 8 (v / 4) + 4 (lane / 32) + v % 4. ----
  const int j = lane & 31;
  float* dwa = nullptr;
  float* dwb = nullptr;
  if (MODE == MB_DW) {
    dwa = is_shared ? g.sdw_a : g.dw_a + (long long)s * g.split * g.N;
    dwb = is_shared ? g.sdw_b : g.dw_b + (long long)s * (g.M - g.split) * g.N;
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + j;
        const float c = acc[mb][nb][v];
        if (MODE == MB_DH) {
          if (r < mrows) {
            const long long jr = (long long)row0 + r;
            const float av = g.pre[jr * 2 * g.I + col], gv = g.pre[jr * 2 * g.I + g.I + col];
            const float sg = sigmoid_f32(av);
            const float da = c * gv * (sg * (1.0f + av * (1.0f - sg)));
            const float dg = c * silu_f32(av);
            g.out[jr * g.ldo + col] = da;
            g.out[jr * g.ldo + g.I + col] = dg;
          }
        } else if (MODE == MB_DX) {
          if (r < mrows) g.out[((long long)row0 + r) * g.ldo + col] = c;
        } else {
          const int m = m0 + r;
          float* dst = m < g.split ? dwa + (long long)m * g.N + col : dwb + (long long)(m - g.split) * g.N + col;
          __builtin_nontemporal_store(c, dst);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static unsigned colq_blocks_y(int C) { return (unsigned)((C + CQ_COLS - 1) / CQ_COLS); }

// mx_colq_nv_kernel in the layout of mx_colq4_kernel: 128 rows x 64 columns per
// workgroup, 16-byte loads (kColNvDec: 8 decoded fp16 values of a row; kColNvW: 32 codes
// of a row of one K-blocked 32 x 64 block, with its two E4M3 block scales), the four
// 32-row blocks of a column quantised in float64 (as mx_colq_nv_kernel) by four
// neighbouring lanes that store one 128-byte run of the output row.  Same bytes as
// mx_colq_nv_kernel.
template <int KIND>
__global__ __launch_bounds__(256) void mx_colq4_nv_kernel(ColqArgs a) {
  __shared__ double t[C4_R][C4_C + 1];
  __shared__ long long srow[C4_R];
  const int c0 = blockIdx.y * C4_C;
  int s, r0;
  long long kout;
  uint8_t* obase;
  uint8_t* osbase;
  if (a.kst) {   // segment mode
    const int kq = C4_R * blockIdx.x;
    if (kq >= a.kst[a.S]) return;
    int lo = 0, hi = a.S;   // kst[lo] <= kq < kst[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.kst[mid] <= kq) lo = mid; else hi = mid;
    }
    s = lo;
    r0 = kq - a.kst[s];
    kout = kq;
    obase = a.out;
    osbase = a.out_s;
  } else {       // matrix mode
    const int per = a.R / C4_R;
    s = blockIdx.x / per;
    r0 = (blockIdx.x % per) * C4_R;
    if (s >= a.S) return;
    kout = a.col0 + r0;
    obase = a.out + s * a.out_mat;
    osbase = a.out_s + s * (a.out_mat / 32);
  }
  const int tid = threadIdx.x;
  if (tid < C4_R) {
    const int r = r0 + tid;
    long long row = -1;
    if (!a.kst) {
      row = (long long)s * a.R + r;
    } else if (r < a.rowcount[s]) {
      const long long j = (long long)a.rowstart[s] + r;
      row = j;
      if (a.gather) {
        row = j >= a.Tk ? j - a.Tk : (long long)(a.perm[j] / a.k);
        if (row < 0 || row >= a.T) {
          raise_flag(a.flag, kFlagCorrupt);
          row = 0;
        }
      }
    }
    srow[tid] = row;
  }
  __syncthreads();
  if (KIND == kColNvDec) {
    // the thread's NI chunks loaded before the first is decoded; a chunk outside the
    // source (padding row, column past C) loads row 0's first chunk and stores zeros
    constexpr int CPR = C4_C / 8, NI = C4_R * CPR / 256;
    u32x4_t q[NI];
    float rsf[NI];
    bool ok[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int i = tid + 256 * n;
      const int c = c0 + (i % CPR) * 8;
      const long long row = srow[i / CPR];
      ok[n] = row >= 0 && c < a.C;
      const long long rw = ok[n] ? row : 0;
      q[n] = *(const u32x4_t*)((const uint16_t*)a.src + rw * a.C + (ok[n] ? c : 0));
      rsf[n] = a.src_r[rw];
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int i = tid + 256 * n;
      const int rr = i / CPR, cc = (i % CPR) * 8;
      const double rs = (double)rsf[n];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double v = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(q[n][u >> 1] >> (16 * (u & 1)))) * rs;
        t[rr][cc + u] = ok[n] ? v : 0.0;
      }
    }
  } else {
    // thread: row rr of the tile, codes of columns c0 + 32 h .. c0 + 32 h + 31
    const int rr = tid >> 1, h = tid & 1;
    const long long row = srow[rr];
    const long long m = row / a.R;
    const int r = (int)(row % a.R);
    const long long tile = (long long)(r / 32) * (a.C / 64) + c0 / 64;
    const uint8_t* codes = (const uint8_t*)a.src + m * ((long long)a.R * a.C / 2) + tile * 1024 + (r % 32) * 32 + 16 * h;
    const uint8_t* sc = a.src_s + m * ((long long)a.R * a.C / 16) + tile * 128 + (r % 32) * 4 + 2 * h;
    const u32x4_t q = *(const u32x4_t*)codes;
    const double rs = (double)a.src_r[row];
    const double s0 = (double)e4m3_to_f32(sc[0]) * rs, s1 = (double)e4m3_to_f32(sc[1]) * rs;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const uint32_t byte = (q[u >> 3] >> (8 * ((u >> 1) & 3))) & 0xffu;
      const uint32_t code = (u & 1) ? (byte >> 4) : (byte & 15u);
      t[rr][32 * h + u] = e2m1_f64(code) * (u < 16 ? s0 : s1);
    }
  }
  __syncthreads();
  const int cl = tid >> 2, g = tid & 3, c = c0 + cl;
  double amax = 0.0;
#pragma unroll 8
  for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(t[32 * g + i][cl]));
  int se;
  uint32_t scode;
  mx_block_scale_f64(amax, se, scode);
  u32x4_t w[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t u = 0;
#pragma unroll
    for (int z = 0; z < 4; ++z) u |= e4m3_rne_f64(ldexp(t[32 * g + 4 * i + z][cl], -se)) << (8 * z);
    w[i >> 2][i & 3] = u;
  }
  const uint32_t s1 = __shfl_down(scode, 1), s2 = __shfl_down(scode, 2), s3 = __shfl_down(scode, 3);
  if (c >= a.C) return;
  uint8_t* o = obase + (long long)c * a.out_ld + kout + 32 * g;
  *(u32x4_t*)o = w[0];
  *(u32x4_t*)(o + 16) = w[1];
  if (g == 0)
    *(uint32_t*)(osbase + (long long)c * (a.out_ld / 32) + kout / 32) = scode | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

template <int KIND>
static void colq_launch(const ColqArgs& a, long long nq, hipStream_t s) {
  if (nq <= 0) return;
  if constexpr (KIND == kColNvDec || KIND == kColNvW) {
    if (nq % 4 == 0 && a.C % 64 == 0 &&
        (KIND == kColNvDec ? a.kst != nullptr
                           : !a.kst && a.R % C4_R == 0 && a.col0 % C4_R == 0 && a.out_ld % C4_R == 0))
      mx_colq4_nv_kernel<KIND><<<dim3((unsigned)(nq / 4), (unsigned)(a.C / C4_C)), 256, 0, s>>>(a);
    else
      mx_colq_nv_kernel<KIND><<<dim3((unsigned)nq, colq_blocks_y(a.C)), 256, 0, s>>>(a);
  } else if (a.C % 16 == 0 && a.src_ld % 16 == 0 && nq % 4 == 0 &&
             (a.kst || (a.R % C4_R == 0 && a.col0 % C4_R == 0 && a.out_ld % C4_R == 0 && a.src_mat % 16 == 0))) {
    // 128-row workgroups: 16-byte source chunks stay aligned and inside a row, and the
    // 128-row blocks (segments padded to 128 rows; whole matrices of R rows) stay inside
    // one segment or matrix and start output runs and scale words on aligned offsets
    mx_colq4_kernel<KIND><<<dim3((unsigned)(nq / 4), (unsigned)((a.C + C4_C - 1) / C4_C)), 256, 0, s>>>(a);
  } else {
    mx_colq_kernel<KIND><<<dim3((unsigned)nq, colq_blocks_y(a.C)), 256, 0, s>>>(a);
  }
}

static void rowq_launch(const void* src, bool bf16, long long R, int C, uint8_t* codes, uint8_t* scales,
                        hipStream_t s) {
  const long long n = R * (C / 32);
  if (n <= 0) return;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (bf16)
    mx_rowq_kernel<true><<<blocks, 256, 0, s>>>(src, R, C, codes, scales);
  else
    mx_rowq_kernel<false><<<blocks, 256, 0, s>>>(src, R, C, codes, scales);
}

// Workspace of the MXFP8 backward (after the prefix the route backward shares).
struct MxBwdWs {
  size_t seg, fseg, kst, pre, dq, dqs, dadg, dgq, dgqs, dT, dTs, hT, hTs, gT, gTs, xT, xTs;
  size_t xc, xr, hb, hc, hr;   // NVFP4 layers: x and h as the forward quantized them
  size_t bytes;
  long long rows, kp;
};
static MxBwdWs mxbwd_ws(int T, int d, int E, int k, int inter, bool nv) {
  const BwdWs B = bwd_ws(T, d, E, k, inter);
  MxBwdWs w;
  w.rows = (long long)T * k + T;
  w.kp = (w.rows + (long long)(E + 1) * 127 + 127) / 128 * 128;
  w.seg = B.seg;
  w.pre = B.pre;
  size_t o = B.pre + align_up((size_t)w.rows * 2 * inter * sizeof(float), 256);
  const size_t R = (size_t)w.rows, KP = (size_t)w.kp;
  auto take = [&](size_t n) { const size_t at = o; o = align_up(o + n, 256); return at; };
  w.fseg = take((size_t)3 * (E + 2) * sizeof(int));
  w.kst = take((size_t)(E + 2) * sizeof(int));
  w.dq = take(R * d);
  w.dqs = take(R * (d / 32));
  w.dadg = take(R * 2 * inter * sizeof(float));
  w.dgq = take(R * 2 * inter);
  w.dgqs = take(R * (2 * inter / 32));
  w.dT = take((size_t)d * KP);
  w.dTs = take((size_t)d * (KP / 32));
  w.hT = take((size_t)inter * KP);
  w.hTs = take((size_t)inter * (KP / 32));
  w.gT = take((size_t)2 * inter * KP);
  w.gTs = take((size_t)2 * inter * (KP / 32));
  w.xT = take((size_t)d * KP);
  w.xTs = take((size_t)d * (KP / 32));
  w.xc = w.xr = w.hb = w.hc = w.hr = 0;
  if (nv) {
    w.xc = take((size_t)T * d * 2);
    w.xr = take((size_t)T * sizeof(float));
    w.hb = take(R * inter * 2);
    w.hc = take(R * inter * 2);
    w.hr = take(R * sizeof(float));
  }
  w.bytes = o;
  return w;
}

size_t mxfp8_backward_ws_bytes(int T, int d, int E, int k, int inter, bool nvfp4_layer) {
  return mxbwd_ws(T, d, E, k, inter, nvfp4_layer).bytes;
}

static bool tbank_ok(const moe_mxfp8_tbank* t) {
  return t && t->w2t && t->w2t_scale && t->w13t && t->w13t_scale && aligned(t->w2t, 16) &&
         aligned(t->w13t, 16) && aligned(t->w2t_scale, 4) && aligned(t->w13t_scale, 4);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_mxfp8_transpose_weights(const moe_expert_bank* bank, int n, int d, int inter,
                                                  const moe_mxfp8_tbank* out, void* stream) {
  if (!bank || !out || n < 0 || d < 1 || inter < 1) return MOE_ERR_INVALID_ARG;
  if (d % 128 != 0 || inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!bank->w1 || !bank->w3 || !bank->w2 || !bank->w1_scale || !bank->w3_scale || !bank->w2_scale ||
      bank->w1_rscale || bank->w3_rscale || bank->w2_rscale || !tbank_ok(out))
    return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  ColqArgs a{};
  a.kst = nullptr;
  a.S = n;
  // W2 [n][d][I], blocks along I -> W2t [n][I][d], blocks along d
  a.src = bank->w2;
  a.src_s = bank->w2_scale;
  a.src_ld = inter;
  a.src_mat = (long long)d * inter;
  a.R = d;
  a.C = inter;
  a.out = out->w2t;
  a.out_s = out->w2t_scale;
  a.out_ld = d;
  a.out_mat = (long long)inter * d;
  a.col0 = 0;
  colq_launch<kColMx>(a, (long long)n * (d / 32), s);
  // W1, W3 [n][I][d], blocks along d -> W13t [n][d][2I], blocks along I
  a.src_ld = d;
  a.src_mat = (long long)inter * d;
  a.R = inter;
  a.C = d;
  a.out = out->w13t;
  a.out_s = out->w13t_scale;
  a.out_ld = 2 * inter;
  a.out_mat = (long long)d * 2 * inter;
  a.src = bank->w1;
  a.src_s = bank->w1_scale;
  a.col0 = 0;
  colq_launch<kColMx>(a, (long long)n * (inter / 32), s);
  a.src = bank->w3;
  a.src_s = bank->w3_scale;
  a.col0 = inter;
  colq_launch<kColMx>(a, (long long)n * (inter / 32), s);
  return launch_status();
}

// The MXFP8 backward of the expert FFN of an MXFP8 layer (nv == false: MXFP8 x, pre
// optional) or of an NVFP4 layer (nv == true: bf16 x, pre required; x and h enter the
// weight gradients as the forward quantized them to NVFP4).
static moe_status mx_backward(bool nv,
    const void* x, const uint8_t* x_scale, int T, int d, int E, int k, int inter,
    const moe_expert_bank* routed, const moe_expert_bank* shared, const moe_mxfp8_tbank* routed_t,
    const moe_mxfp8_tbank* shared_t, const int32_t* offsets, const int32_t* perm, const float* pre,
    const void* d_out, float* dx_rows, const moe_grad_bank* routed_grads,
    const moe_grad_bank* shared_grads, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxTopK || inter < 1)
    return MOE_ERR_INVALID_ARG;
  if (d % 128 != 0 || inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (!ws || !routed || !routed_grads || !tbank_ok(routed_t)) return MOE_ERR_INVALID_ARG;
  if ((shared != nullptr) != (shared_t != nullptr) || (shared != nullptr) != (shared_grads != nullptr))
    return MOE_ERR_INVALID_ARG;
  if (shared && !tbank_ok(shared_t)) return MOE_ERR_INVALID_ARG;
  const moe_grad_bank* gbs[2] = {routed_grads, shared_grads};
  for (const moe_grad_bank* gb : gbs)
    if (gb && (!gb->dw1 || !gb->dw3 || !gb->dw2 || !aligned(gb->dw1, 16) || !aligned(gb->dw3, 16) ||
               !aligned(gb->dw2, 16)))
      return MOE_ERR_INVALID_ARG;
  const MxBwdWs L = mxbwd_ws(T, d, E, k, inter, nv);
  if (ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  int* flag = (int*)w;
  const int has_shared = shared ? 1 : 0;
  if (T == 0) {
    const long long n13 = (long long)E * inter * d;
    zero_fill(routed_grads->dw1, n13, s);
    zero_fill(routed_grads->dw3, n13, s);
    zero_fill(routed_grads->dw2, n13, s);
    if (shared) {
      zero_fill(shared_grads->dw1, (long long)inter * d, s);
      zero_fill(shared_grads->dw3, (long long)inter * d, s);
      zero_fill(shared_grads->dw2, (long long)inter * d, s);
    }
    return launch_status();
  }
  if (!x || (nv ? x_scale != nullptr : !x_scale) || (nv && !pre) || !offsets || !perm || !d_out || !dx_rows ||
      !aligned(x, 16) || !aligned(d_out, 16) || !aligned(dx_rows, 16) || (pre && !aligned(pre, 16)))
    return MOE_ERR_INVALID_ARG;
  if (!routed->w1 || !routed->w3 || !routed->w2 || !routed->w1_scale || !routed->w3_scale || !routed->w2_scale)
    return MOE_ERR_INVALID_ARG;
  const long long Tk = (long long)T * k;
  const long long rows = Tk + (shared ? T : 0);
  const int S = E + has_shared;
  float* prew = (float*)(w + L.pre);
  if (!pre && !nv) {
    // the pre-activations, recomputed with the forward's GEMM1 (same MFMA sequence)
    int* fseg = (int*)(w + L.fseg);
    const int tm = mx_tile_rows(d, inter, Tk, E);
    moe_status st = ffn_seg_table_rows(offsets, T, E, k, has_shared, tm, fseg, flag, s);
    if (st != MOE_OK) return st;
    MxArgs m{};
    m.a = (const uint8_t*)x;
    m.as = x_scale;
    m.perm = perm;
    m.T = T;
    m.k = k;
    m.E = E;
    m.Tk = Tk;
    m.b0 = (const uint8_t*)routed->w1;
    m.b1 = (const uint8_t*)routed->w3;
    m.b0s = routed->w1_scale;
    m.b1s = routed->w3_scale;
    m.sb0 = shared ? (const uint8_t*)shared->w1 : nullptr;
    m.sb1 = shared ? (const uint8_t*)shared->w3 : nullptr;
    m.sb0s = shared ? shared->w1_scale : nullptr;
    m.sb1s = shared ? shared->w3_scale : nullptr;
    m.K = d;
    m.N = inter;
    m.mstart = fseg;
    m.rowstart = fseg + (E + 2);
    m.rowcount = fseg + 2 * (E + 2);
    m.S = S;
    m.out_pre = prew;
    m.flag = flag;
    m.tm = tm;
    const long long mtb = (Tk + (long long)E * (tm - 1)) / tm + (shared ? (T + tm - 1) / tm : 0);
    if ((st = mx_gemm(2, m, mtb, s)) != MOE_OK) return st;
    pre = prew;
  }
  int* seg = (int*)(w + L.seg);
  int* kst = (int*)(w + L.kst);
  moe_status st = ffn_seg_table(offsets, T, E, k, has_shared, seg, flag, s);
  if (st != MOE_OK) return st;
  mx_kst_kernel<<<1, 1024, 0, s>>>(seg + 2 * (E + 2), S, kst);
  uint8_t* dq = (uint8_t*)(w + L.dq);
  uint8_t* dqs = (uint8_t*)(w + L.dqs);
  float* dadg = (float*)(w + L.dadg);
  uint8_t* dgq = (uint8_t*)(w + L.dgq);
  uint8_t* dgqs = (uint8_t*)(w + L.dgqs);
  const long long mt_bound = (Tk + (long long)E * (BB_T - 1)) / BB_T + (shared ? (T + BB_T - 1) / BB_T : 0);

  // ---- data half ----
  rowq_launch(d_out, true, rows, d, dq, dqs, s);
  MxBwdGemm g{};
  g.mstart = seg;
  g.rowstart = seg + (E + 2);
  g.rowcount = seg + 2 * (E + 2);
  g.kst = kst;
  g.S = S;
  g.E = E;
  g.I = inter;
  g.flag = flag;
  g.a = dq;
  g.as = dqs;
  g.lda = d;
  g.b = routed_t->w2t;
  g.bs = routed_t->w2t_scale;
  g.ldb = d;
  g.b_e = (long long)inter * d;
  g.sb = shared ? shared_t->w2t : nullptr;
  g.sbs = shared ? shared_t->w2t_scale : nullptr;
  g.K = d;
  g.NT = inter / BB_T;
  g.pre = pre;
  g.out = dadg;
  g.ldo = 2 * inter;
  // where the ring tiles the shape, both data GEMMs run on the forward's 128-row ring
  // kernel (same MFMA chains, so the same bits as mx_bwd_gemm_kernel)
  MxArgs r{};
  r.E = E;
  r.mstart = seg;
  r.rowstart = seg + (E + 2);
  r.rowcount = seg + 2 * (E + 2);
  r.S = S;
  r.flag = flag;
  r.tm = BB_T;
  r.a = dq;
  r.as = dqs;
  r.b0 = routed_t->w2t;
  r.b0s = routed_t->w2t_scale;
  r.sb0 = shared ? shared_t->w2t : nullptr;
  r.sb0s = shared ? shared_t->w2t_scale : nullptr;
  r.K = d;
  r.N = inter;
  r.pre_in = pre;
  r.out_f = dadg;
  long long grid = 0;
  moe_status rst = mx_gemm_bwd_data(3, d, inter, r, mt_bound, s);
  if (rst == MOE_ERR_UNSUPPORTED) {
    grid = tile_grid(mt_bound * g.NT, 0);
    if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    mx_bwd_gemm_kernel<MB_DH><<<(unsigned)grid, BB_THR, 0, s>>>(g);
  } else if (rst != MOE_OK) {
    return rst;
  }
  rowq_launch(dadg, false, rows, 2 * inter, dgq, dgqs, s);
  g.a = dgq;
  g.as = dgqs;
  g.lda = 2 * inter;
  g.b = routed_t->w13t;
  g.bs = routed_t->w13t_scale;
  g.ldb = 2 * inter;
  g.b_e = (long long)d * 2 * inter;
  g.sb = shared ? shared_t->w13t : nullptr;
  g.sbs = shared ? shared_t->w13t_scale : nullptr;
  g.K = 2 * inter;
  g.NT = d / BB_T;
  g.out = dx_rows;
  g.ldo = d;
  r.a = dgq;
  r.as = dgqs;
  r.b0 = routed_t->w13t;
  r.b0s = routed_t->w13t_scale;
  r.sb0 = shared ? shared_t->w13t : nullptr;
  r.sb0s = shared ? shared_t->w13t_scale : nullptr;
  r.K = 2 * inter;
  r.N = d;
  r.pre_in = nullptr;
  r.out_f = dx_rows;
  rst = mx_gemm_bwd_data(4, d, inter, r, mt_bound, s);
  if (rst == MOE_ERR_UNSUPPORTED) {
    grid = tile_grid(mt_bound * g.NT, 0);
    if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    mx_bwd_gemm_kernel<MB_DX><<<(unsigned)grid, BB_THR, 0, s>>>(g);
  } else if (rst != MOE_OK) {
    return rst;
  }

  // ---- weights half: transposed operands quantised along the rows, then the GEMMs ----
  const long long nq = L.kp / 32;
  ColqArgs c{};
  c.perm = perm;
  c.k = k;
  c.T = T;
  c.Tk = Tk;
  c.rowstart = seg + (E + 2);
  c.rowcount = seg + 2 * (E + 2);
  c.kst = kst;
  c.S = S;
  c.out_ld = L.kp;
  c.flag = flag;
  c.src = d_out;              // d_out rows -> dT [d][Kp]
  c.src_ld = d;
  c.C = d;
  c.gather = 0;
  c.out = (uint8_t*)(w + L.dT);
  c.out_s = (uint8_t*)(w + L.dTs);
  colq_launch<kColBf16>(c, nq, s);
  if (nv) {                   // the forward's NVFP4 h: bf16(silu(a) g) quantized per row
    uint16_t* hb = (uint16_t*)(w + L.hb);
    if ((st = nvfp4_h_from_pre(pre, rows, inter, hb, s)) != MOE_OK) return st;
    if ((st = nvfp4_quantize_rows(hb, rows, inter, nullptr, nullptr, (float*)(w + L.hr),
                                  (uint16_t*)(w + L.hc), s)) != MOE_OK)
      return st;
    c.src = w + L.hc;         // hq rows -> hT [I][Kp]
    c.src_r = (const float*)(w + L.hr);
    c.C = inter;
    c.out = (uint8_t*)(w + L.hT);
    c.out_s = (uint8_t*)(w + L.hTs);
    colq_launch<kColNvDec>(c, nq, s);
  } else {
    c.src = pre;              // hq rows (from a | g) -> hT [I][Kp]
    c.src_ld = 2 * inter;
    c.C = inter;
    c.out = (uint8_t*)(w + L.hT);
    c.out_s = (uint8_t*)(w + L.hTs);
    colq_launch<kColPre>(c, nq, s);
  }
  c.src = dadg;               // da | dg rows -> gT [2I][Kp]
  c.src_ld = 2 * inter;
  c.C = 2 * inter;
  c.out = (uint8_t*)(w + L.gT);
  c.out_s = (uint8_t*)(w + L.gTs);
  colq_launch<kColF32>(c, nq, s);
  c.C = d;                    // the gathered tokens' x -> xT [d][Kp]
  c.gather = 1;
  c.out = (uint8_t*)(w + L.xT);
  c.out_s = (uint8_t*)(w + L.xTs);
  if (nv) {                   // x as the forward quantized it to NVFP4 (per token)
    if ((st = nvfp4_quantize_rows((const uint16_t*)x, T, d, nullptr, nullptr, (float*)(w + L.xr),
                                  (uint16_t*)(w + L.xc), s)) != MOE_OK)
      return st;
    c.src = w + L.xc;
    c.src_r = (const float*)(w + L.xr);
    colq_launch<kColNvDec>(c, nq, s);
  } else {
    c.src = x;
    c.src_s = x_scale;
    c.src_ld = d;
    colq_launch<kColMx>(c, nq, s);
  }

  MxBwdGemm q{};
  q.kst = kst;
  q.S = S;
  q.E = E;
  q.flag = flag;
  q.lda = L.kp;
  q.ldb = L.kp;
  // dW2[e] [d][I] = dT . hT^T
  q.a = (const uint8_t*)(w + L.dT);
  q.as = (const uint8_t*)(w + L.dTs);
  q.b = (const uint8_t*)(w + L.hT);
  q.bs = (const uint8_t*)(w + L.hTs);
  q.M = d;
  q.N = inter;
  q.MT = d / BB_T;
  q.NT = inter / BB_T;
  q.split = d;
  q.dw_a = routed_grads->dw2;
  q.sdw_a = shared ? shared_grads->dw2 : nullptr;
  grid = tile_grid((long long)S * q.MT * q.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  mx_bwd_gemm_kernel<MB_DW><<<(unsigned)grid, BB_THR, 0, s>>>(q);
  // dW1[e] | dW3[e] [2I][d] = gT . xT^T
  q.a = (const uint8_t*)(w + L.gT);
  q.as = (const uint8_t*)(w + L.gTs);
  q.b = (const uint8_t*)(w + L.xT);
  q.bs = (const uint8_t*)(w + L.xTs);
  q.M = 2 * inter;
  q.N = d;
  q.MT = 2 * inter / BB_T;
  q.NT = d / BB_T;
  q.split = inter;
  q.dw_a = routed_grads->dw1;
  q.dw_b = routed_grads->dw3;
  q.sdw_a = shared ? shared_grads->dw1 : nullptr;
  q.sdw_b = shared ? shared_grads->dw3 : nullptr;
  grid = tile_grid((long long)S * q.MT * q.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  mx_bwd_gemm_kernel<MB_DW><<<(unsigned)grid, BB_THR, 0, s>>>(q);
  return launch_status();
}

extern "C" moe_status moe_expert_ffn_backward_mxfp8(
    const void* x, const uint8_t* x_scale, int T, int d, int E, int k, int inter,
    const moe_expert_bank* routed, const moe_expert_bank* shared, const moe_mxfp8_tbank* routed_t,
    const moe_mxfp8_tbank* shared_t, const int32_t* offsets, const int32_t* perm, const float* pre,
    const void* d_out, float* dx_rows, const moe_grad_bank* routed_grads,
    const moe_grad_bank* shared_grads, void* ws, size_t ws_bytes, void* stream) {
  if (routed && (routed->w1_rscale || routed->w3_rscale || routed->w2_rscale)) return MOE_ERR_INVALID_ARG;
  return mx_backward(false, x, x_scale, T, d, E, k, inter, routed, shared, routed_t, shared_t, offsets, perm,
                     pre, d_out, dx_rows, routed_grads, shared_grads, ws, ws_bytes, stream);
}

extern "C" moe_status moe_expert_ffn_backward_nvfp4(
    const void* x, int T, int d, int E, int k, int inter, const moe_expert_bank* routed,
    const moe_expert_bank* shared, const moe_mxfp8_tbank* routed_t, const moe_mxfp8_tbank* shared_t,
    const int32_t* offsets, const int32_t* perm, const float* pre, const void* d_out, float* dx_rows,
    const moe_grad_bank* routed_grads, const moe_grad_bank* shared_grads, void* ws, size_t ws_bytes,
    void* stream) {
  if (d % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (routed && (!routed->w1_rscale || !routed->w3_rscale || !routed->w2_rscale)) return MOE_ERR_INVALID_ARG;
  return mx_backward(true, x, nullptr, T, d, E, k, inter, routed, shared, routed_t, shared_t, offsets, perm, pre,
                     d_out, dx_rows, routed_grads, shared_grads, ws, ws_bytes, stream);
}

extern "C" moe_status moe_nvfp4_transpose_weights(const moe_expert_bank* bank, int n, int d, int inter,
                                                  const moe_mxfp8_tbank* out, void* stream) {
  if (!bank || !out || n < 0 || d < 1 || inter < 1) return MOE_ERR_INVALID_ARG;
  if (d % 256 != 0 || inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!bank->w1 || !bank->w3 || !bank->w2 || !bank->w1_scale || !bank->w3_scale || !bank->w2_scale ||
      !bank->w1_rscale || !bank->w3_rscale || !bank->w2_rscale || !tbank_ok(out))
    return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  ColqArgs a{};
  a.kst = nullptr;
  a.S = n;
  // W2 [n][d][I] (K-blocked along I) -> W2t [n][I][d], blocks along d
  a.src = bank->w2;
  a.src_s = bank->w2_scale;
  a.src_r = bank->w2_rscale;
  a.R = d;
  a.C = inter;
  a.out = out->w2t;
  a.out_s = out->w2t_scale;
  a.out_ld = d;
  a.out_mat = (long long)inter * d;
  a.col0 = 0;
  colq_launch<kColNvW>(a, (long long)n * (d / 32), s);
  // W1, W3 [n][I][d] (K-blocked along d) -> W13t [n][d][2I], blocks along I
  a.R = inter;
  a.C = d;
  a.out = out->w13t;
  a.out_s = out->w13t_scale;
  a.out_ld = 2 * inter;
  a.out_mat = (long long)d * 2 * inter;
  a.src = bank->w1;
  a.src_s = bank->w1_scale;
  a.src_r = bank->w1_rscale;
  a.col0 = 0;
  colq_launch<kColNvW>(a, (long long)n * (inter / 32), s);
  a.src = bank->w3;
  a.src_s = bank->w3_scale;
  a.src_r = bank->w3_rscale;
  a.col0 = inter;
  colq_launch<kColNvW>(a, (long long)n * (inter / 32), s);
  return launch_status();
}
