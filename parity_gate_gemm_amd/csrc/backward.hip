// Backward pass of the MoE layer: the chain rule of the forward (route -> dispatch ->
// grouped SwiGLU FFN -> combine) for a loss whose gradient dL/dy is given, as grouped
// GEMMs over the same expert segments as the forward (Composer 2 Technical Report,
// section 6.1 "Kernels", Figure 10: the MoE layer is trained as one grouped-GEMM flow;
// under router replay the router still computes gate scores so that gradients flow
// through them: section 6.2, paragraph on inference and weight sync).
//
//   combine:  d_out[row(t,r)] = w_tr dy_t,  d_w_tr = <dy_t, out[row(t,r)]>,
//             shared rows d_out[T k + t] = dy_t;
//   experts:  a = x W1, g = x W3 (recomputed), dh = d_out W2, da = dh g silu'(a),
//             dg = dh silu(a), dx_row = da W1^T + dg W3^T (as stored: da w1 + dg w3),
//             dW2 = d_out^T h, dW1 = da^T x, dW3 = dg^T x (per expert segment);
//   route:    dx_t = sum_r dx_row(t,r) + dx_row(shared t) + sum_r dl_tr Wg[:, e_tr],
//             dl = w (dw - <w, dw>) when the weights are the gate's renormalised
//             softmax, dWg[:, e] = sum over e's rows of dl x_t, db[e] = sum of dl.
//
// Every reduction has one fixed order: a GEMM output sweeps K in ascending 64-wide
// steps with one MFMA sequence (no split-K, no atomics), token sums run in rank order,
// so the gradients are bitwise reproducible and a token's dx does not depend on the
// rest of the batch.
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// combine backward: one workgroup per token; d_w by a per-thread fp32 FMA chain over
// the thread's 8-element chunks, a fixed butterfly per wavefront and the wavefronts'
// partial sums added in order.
// ---------------------------------------------------------------------------
template <bool kF32>
__device__ __forceinline__ void load8(const void* p, long long row, int d, int c, float (&v)[8]) {
  if (kF32) {
    const float4* q = (const float4*)((const float*)p + row * d + c);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *(const uint4*)((const uint16_t*)p + row * d + c);
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(wd[i] & 0xffff));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(wd[i] >> 16));
    }
  }
}

template <bool kF32>
__device__ __forceinline__ void store8(void* p, long long row, int d, int c, const float (&v)[8]) {
  if (kF32) {
    float4* q = (float4*)((float*)p + row * d + c);
    q[0] = make_float4(v[0], v[1], v[2], v[3]);
    q[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *(uint4*)((uint16_t*)p + row * d + c) = u;
  }
}

template <bool kF32>
__global__ __launch_bounds__(1024) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const void* __restrict__ out,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ weights, int T,
                                                          int d, int k, int has_shared,
                                                          void* __restrict__ d_out,
                                                          float* __restrict__ d_weights) {
  __shared__ float part[16];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const long long Tk = (long long)T * k;
  for (int r = 0; r < k; ++r) {
    long long j = row_of[(size_t)t * k + r];
    j = (j < 0 || j >= Tk) ? 0 : j;   // guard against corrupt input (as the forward combine)
    const float w = weights[(size_t)t * k + r];
    float acc = 0.0f;
    for (int c = tid * 8; c < d; c += blockDim.x * 8) {
      float g[8], o[8], dg[8];
      load8<kF32>(dy, t, d, c, g);
      load8<kF32>(out, j, d, c, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc = fmaf(g[i], o[i], acc);
        dg[i] = w * g[i];
      }
      store8<kF32>(d_out, j, d, c, dg);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int q = 0; q < nw; ++q) s += part[q];
      d_weights[(size_t)t * k + r] = s;
    }
    __syncthreads();
  }
  if (has_shared) {
    for (int c = tid * 8; c < d; c += blockDim.x * 8) {
      float g[8];
      load8<kF32>(dy, t, d, c, g);
      store8<kF32>(d_out, Tk + t, d, c, g);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward grouped GEMMs (bf16 operands, fp32 accumulation), one kind per launch:
//   DH   : C[n][i] = sum_j d_out[n][j] W2[e][j][i]      rows x I,  K = d   (+ SwiGLU backward)
//   DX   : C[n][j] = sum_i dadg[n][i] W13[e][i][j]     rows x d,  K = 2I  (W13 = W1 then W3)
//   DW2  : C[j][i] = sum_n d_out[n][j] h[n][i]         d x I,     K = the segment's rows
//   DW13 : C[i][j] = sum_n dadg[n][i] x[tok(n)][j]     2I x d,    K = the segment's rows
// Tiles of 128 rows x 64 NWN columns, 2 x NWN wavefronts of 64 x 64 (2 x 2 MFMA 32x32x16
// blocks), K steps of 64 through LDS.  The weight-gradient kinds use NWN = 2 (128 x 128);
// the data kinds NWN = 4 (128 x 256, two workgroups per CU) where the output width is a
// multiple of 256, else NWN = 2.  A row operand (A of DH and DX) sits in LDS rows of 64
// K-values (144-byte stride).  An operand stored with K as its row index ("K-major": the
// weight operands of DH and DX, both operands of the weight gradients) is loaded as whole
// row pieces, 4 K-rows per thread, stored to LDS as it is and read transposed (k_frag);
// K-rows past a segment's end read as zero.  The tile width changes which workgroup
// computes an output, not its MFMA sequence, so both widths give the same bits.
// ---------------------------------------------------------------------------
constexpr int GB_T = 128, GB_K = 64, GB_S = GB_K + 8;
// K-major tile of 64 NWN columns: row pitch (elements); threads per workgroup
__host__ __device__ constexpr int gb_ks(int nwn) { return 64 * nwn + 8; }
__host__ __device__ constexpr int gb_thr(int nwn) { return 128 * nwn; }
static_assert(GB_K * gb_ks(2) <= GB_T * GB_S, "the weight-gradient kinds' K-major A tile fits in sA");
enum { BK_DH = 0, BK_DX = 1, BK_DW2 = 2, BK_DW13 = 3 };

// Tuning knobs of the weight-gradient GEMMs (same results for every setting):
// nontemporal gradient stores, output-column tiles per workgroup, wavefronts per SIMD
// the register allocation must allow.
#ifndef MOE_BWD_NT_STORE
#define MOE_BWD_NT_STORE 1
#endif
#ifndef MOE_BWD_NTW
#define MOE_BWD_NTW 1
#endif
#ifndef MOE_BWD_WAVES
#define MOE_BWD_WAVES 1
#endif
constexpr int kBwdNtw = MOE_BWD_NTW;

struct BwdGemm {
  const uint16_t* x;        // activations [T][d]
  const int32_t* perm;
  int T, k, E, d, I;
  long long Tk;
  const uint16_t* w1;       // routed banks [E][I][d], [E][I][d], [E][d][I]
  const uint16_t* w3;
  const uint16_t* w2;
  const uint16_t* sw1;      // shared expert (null without one)
  const uint16_t* sw3;
  const uint16_t* sw2;
  const uint16_t* d_out;    // [rows][d]
  const float* pre;         // [rows][2I]: a, then g
  uint16_t* dadg;           // [rows][2I]: da, then dg
  uint16_t* h;              // [rows][I]
  float* dx_rows;           // [rows][d]
  float* dw1;               // routed gradients, layout of the banks
  float* dw3;
  float* dw2;
  float* sdw1;              // shared expert's gradients
  float* sdw3;
  float* sdw2;
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  int* tokrow;              // token of each dispatched row [rows]
  int S;
  int MT, NT;               // tiles along M (weight-gradient kinds) and along N
  int* flag;
};

// Weight-gradient kinds: a workgroup owns one 128-row block of the output (tile row
// m0) and kBwdNtw consecutive column tiles.

template <int KIND, int NWN>
// The weight-gradient kinds fit in 128 registers without spilling, so they run four
// wavefronts per SIMD (four workgroups per CU); the 128 x 256 data kinds are held to 128
// registers too (two workgroups of eight wavefronts per CU); the 128 x 128 data kinds
// would spill there and keep three.
__global__ __launch_bounds__(gb_thr(NWN))
__attribute__((amdgpu_waves_per_eu(KIND >= BK_DW2 || NWN == 4 ? 4 : MOE_BWD_WAVES)))
void bwd_gemm_kernel(BwdGemm g) {
  constexpr bool WGRAD = KIND >= BK_DW2;
  static_assert(NWN == 2 || (NWN == 4 && !WGRAD), "tile widths");
  constexpr int TN = 64 * NWN, KS = gb_ks(NWN), THR = gb_thr(NWN);
  constexpr int SB = GB_K * KS > GB_T * GB_S ? GB_K * KS : GB_T * GB_S;
  __shared__ __attribute__((aligned(16))) uint16_t sA[GB_T * GB_S];
  __shared__ __attribute__((aligned(16))) uint16_t sB[SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;

  // ---- tile decode ----
  int s, row0, mrows = GB_T, K, m0 = 0, n0;
  if (!WGRAD) {
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
    constexpr int GM = 8;   // row tiles per raster group (they share each weight slab)
    const int grp = local / (GM * g.NT), rem = local % (GM * g.NT);
    const int gm = min(GM, mtiles - grp * GM);
    const int nt = rem / gm, mt = grp * GM + rem % gm;
    row0 = g.rowstart[s] + mt * GB_T;
    mrows = min(GB_T, g.rowcount[s] - mt * GB_T);
    n0 = nt * TN;
    K = KIND == BK_DH ? g.d : 2 * g.I;
  } else {
    const int ntw = g.NT / kBwdNtw;   // workgroups along N (each takes kBwdNtw column tiles)
    const int per = g.MT * ntw;
    int tile;
    if (!xcd_tile<0>(g.S * per, tile)) return;
    s = tile / per;
    const int rem = tile % per;
    m0 = (rem / ntw) * GB_T;
    n0 = (rem % ntw) * kBwdNtw * GB_T;
    row0 = g.rowstart[s];
    K = g.rowcount[s];
  }
  const bool is_shared = s == g.E;
  const long long e = is_shared ? 0 : s;

  // ---- loaders ----
  // row operand (A of DH / DX): rows lr + RP i, 16-byte chunk lc of the K-step
  constexpr int RP = THR / 8, NA = GB_T / RP;
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  // K-major operands (the weights of the data kinds; both operands of the weight-gradient
  // kinds): K-rows 4 bkq .. 4 bkq + 3 of the step, columns 8 brb .. 8 brb + 7, so one load
  // instruction of a wavefront reads whole row pieces (four of 256 bytes, or two of 512).
  // The tile goes to LDS as it is (K-major, row pitch KS) and the MFMA fragments are read
  // from it with the transposing ds_read_b64_tr_b16 (k_frag).
  constexpr int CPR = TN / 8;   // 16-byte chunks per K-row of the tile
  static_assert(THR / CPR * 4 == GB_K, "four K-rows per thread");
  const int bkq = tid / CPR, brb = tid % CPR;
  const uint16_t* arow[NA];
  if (!WGRAD) {
    const uint16_t* base = KIND == BK_DH ? g.d_out : g.dadg;
    const long long ld = KIND == BK_DH ? g.d : 2LL * g.I;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = lr + RP * i;
      arow[i] = base + ((long long)row0 + (r < mrows ? r : 0)) * ld + lc;
    }
  }
  const uint16_t* w1b = is_shared ? g.sw1 : g.w1 + e * g.I * (long long)g.d;
  const uint16_t* w3b = is_shared ? g.sw3 : g.w3 + e * g.I * (long long)g.d;
  const uint16_t* w2b = is_shared ? g.sw2 : g.w2 + e * g.d * (long long)g.I;
  // K-major sources.  Weight operands (DH, DX): K-row kg of the weight matrix.  Weight-
  // gradient operands: segment row row0 + kg; rows past the segment's end re-read its
  // last row and are zeroed after the load (no branches around the loads).
  const int Klast = K > 0 ? K - 1 : 0;
  const uint16_t* a_seg = nullptr;   // wgrad A: segment row 0, this thread's columns
  int lda = 0;
  if (KIND == BK_DW2) {
    a_seg = g.d_out + (long long)row0 * g.d + m0 + 8 * brb;
    lda = g.d;
  } else if (KIND == BK_DW13) {
    a_seg = g.dadg + (long long)row0 * 2 * g.I + m0 + 8 * brb;
    lda = 2 * g.I;
  }
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  f32x16_t acc[2][2];
  u32x4_t ra[NA], ka[4], kb[4];
  auto load_ra = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = *(const u32x4_t*)(arow[i] + k0);
  };
  auto load_a_to = [&](u32x4_t(&A)[4], int k0) {
    {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kg = k0 + 4 * bkq + i;
        const u32x4_t v = *(const u32x4_t*)(a_seg + min(kg, Klast) * lda);
        A[i] = kg < K ? v : zero4;
      }
    }
  };
  auto load_a = [&](int k0) {
    if (!WGRAD) load_ra(k0);
    else load_a_to(ka, k0);
  };
  auto load_b_to = [&](u32x4_t(&B)[4], int k0, int c0) {
    if (KIND == BK_DH || KIND == BK_DX) {
      // the K-step lies in one weight matrix (I % 64 == 0)
      const uint16_t* base;
      int ldb;
      if (KIND == BK_DH) {
        base = w2b + (long long)k0 * g.I;
        ldb = g.I;
      } else {
        base = k0 < g.I ? w1b + (long long)k0 * g.d : w3b + (long long)(k0 - g.I) * g.d;
        ldb = g.d;
      }
      base += c0 + 8 * brb;
#pragma unroll
      for (int i = 0; i < 4; ++i) B[i] = *(const u32x4_t*)(base + (4 * bkq + i) * ldb);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kg = k0 + 4 * bkq + i;
        const int jr = row0 + min(kg, Klast);
        const uint16_t* p = KIND == BK_DW2 ? g.h + (long long)jr * g.I
                                           : g.x + (long long)g.tokrow[jr] * g.d;
        const u32x4_t v = *(const u32x4_t*)(p + c0 + 8 * brb);
        B[i] = kg < K ? v : zero4;
      }
    }
  };
  auto load_b = [&](int k0, int c0) { load_b_to(kb, k0, c0); };
  // a K-major tile as it is, row pitch KS (conflict-free 16-byte stores: 16 lanes write
  // 256 contiguous bytes of one row)
  auto store_k = [&](uint16_t* sX, const u32x4_t(&R)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4_t*)&sX[(4 * bkq + i) * KS + 8 * brb] = R[i];
  };
  auto store_a = [&]() {
    if (!WGRAD) {
#pragma unroll
      for (int i = 0; i < NA; ++i) *(u32x4_t*)&sA[(lr + RP * i) * GB_S + lc] = ra[i];
    } else {
      store_k(sA, ka);
    }
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  };
  // MFMA operand of 32-row (or 32-column) block cb of a K-major tile, k = kc .. kc + 7.
  // ds_read_b64_tr_b16: in each 16-lane group, lane i receives halfword i % 4 of the
  // 8-byte chunks that lanes 4 q + i / 4 (q = 0..3) address, as element q.  Lane 4 q + p
  // addresses K-row kc + q, columns c + 4 p .. c + 4 p + 3, so lane i receives column c + i
  // at K-rows kc .. kc + 3; a second read gives kc + 4 .. kc + 7.
  auto k_frag = [&](const uint16_t* sX, int cb, int kc) {
    typedef __attribute__((address_space(3))) v4i16_t lds_v4;
    const int i16 = lane & 15;
    const int c = cb + 16 * ((lane >> 4) & 1);
    const uint16_t* p0 = &sX[(kc + (i16 >> 2)) * KS + c + 4 * (i16 & 3)];
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p0));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p0 + 4 * KS));
    const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };
  // kvalid: K-values of this step that lie inside the reduction.  The weight-gradient
  // kinds stop after the last 16-row chunk holding one: the rest of the step is zero
  // padding, whose products (+0) would change no sum except a -0 into +0.
  auto mma = [&](int kvalid) {
#pragma unroll
    for (int kk = 0; kk < GB_K; kk += 16) {
      if (WGRAD && kk >= kvalid) break;
      const int kc = kk + (lane >> 5) * 8;
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (WGRAD)
          af[mb] = k_frag(sA, wm * 64 + mb * 32, kc);
        else   // row operand: row lane % 32 of the block, k = kc .. kc + 7
          af[mb] = __builtin_bit_cast(bf16x8_t,
                                      *(const u32x4_t*)&sA[(wm * 64 + mb * 32 + (lane & 31)) * GB_S + kc]);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bf[nb] = k_frag(sB, wn * 64 + nb * 32, kc);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
  };

  // ---- epilogue: accumulator element v of a lane is C[i][j], j = lane % 32,
  //      i = 8 (v / 4) + 4 (lane / 32) + v % 4 ----
  auto epilogue = [&](int c0) {
    const int j = lane & 31;
    // weight gradients: output row m0 + r, column c0 + ..., one matrix per workgroup
    // (a 128-row block lies in dW1 or in dW3 because I % 128 == 0)
    float* wbase = nullptr;
    int wld = 0;
    if (KIND == BK_DW2) {
      wbase = (is_shared ? g.sdw2 : g.dw2 + e * g.d * (long long)g.I) + (long long)m0 * g.I + c0;
      wld = g.I;
    } else if (KIND == BK_DW13) {
      float* mat = m0 < g.I ? (is_shared ? g.sdw1 : g.dw1 + e * g.I * (long long)g.d)
                            : (is_shared ? g.sdw3 : g.dw3 + e * g.I * (long long)g.d);
      wbase = mat + (long long)(m0 < g.I ? m0 : m0 - g.I) * g.d + c0;
      wld = g.d;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (!WGRAD && r >= mrows) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = c0 + wn * 64 + nb * 32 + j;
          const float c = acc[mb][nb][v];
          if (KIND == BK_DH) {
            const long long orow = (long long)row0 + r;
            const float a = g.pre[orow * 2 * g.I + col], gg = g.pre[orow * 2 * g.I + g.I + col];
            const float sg = sigmoid_f32(a), sl = silu_f32(a);   // as in the forward
            g.dadg[orow * 2 * g.I + col] = f32_to_bf16(c * gg * (sg * (1.0f + a * (1.0f - sg))));
            g.dadg[orow * 2 * g.I + g.I + col] = f32_to_bf16(c * sl);
            g.h[orow * g.I + col] = f32_to_bf16(sl * gg);
          } else if (KIND == BK_DX) {
            g.dx_rows[((long long)row0 + r) * g.d + col] = c;
          } else {
            float* dp = wbase + r * wld + (col - c0);
            if (MOE_BWD_NT_STORE) __builtin_nontemporal_store(c, dp); else *dp = c;
          }
        }
      }
    }
  };

  const int nsteps = (K + GB_K - 1) / GB_K;
  const int ntiles = WGRAD ? kBwdNtw : 1;
  for (int q = 0; q < ntiles; ++q) {
    const int c0 = n0 + q * TN;
    zero_acc();
    if (nsteps > 0) {
      load_a(0);
      load_b(0, c0);
    }
    for (int st = 0; st < nsteps; ++st) {
      store_a();
      store_k(sB, kb);
      __syncthreads();
      if (st + 1 < nsteps) {
        load_a((st + 1) * GB_K);
        load_b((st + 1) * GB_K, c0);
      }
      mma(K - st * GB_K);
      __syncthreads();
    }
    epilogue(c0);
  }
}

// tokrow[j]: the token of dispatched row j (perm[j] / k for routed rows, j - T k for the
// shared expert's); an out-of-range entry is flagged and read as token 0.
__global__ __launch_bounds__(256) void tokrow_kernel(const int32_t* __restrict__ perm, int T, int k,
                                                     long long rows, int* __restrict__ tokrow,
                                                     int* flag) {
  const long long j = (long long)blockIdx.x * 256 + threadIdx.x;
  if (j >= rows) return;
  const long long Tk = (long long)T * k;
  long long t = j < Tk ? (long long)(perm[j] / k) : j - Tk;
  if (t < 0 || t >= T) {
    raise_flag(flag, kFlagCorrupt);
    t = 0;
  }
  tokrow[j] = (int)t;
}

// Zero fill by a kernel (callers may capture these calls in a graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(float* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    p[i] = 0.0f;
}
void zero_fill(float* p, long long n, hipStream_t s) {
  if (n <= 0) return;
  const long long blocks = (n + 255) / 256;
  zero_fill_kernel<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(p, n);
}

// ---------------------------------------------------------------------------
// Route backward
// ---------------------------------------------------------------------------
// dl_tr = w_tr (dw_tr - sum_s w_ts dw_ts), the sum in column order.
__global__ __launch_bounds__(256) void route_bwd_dl_kernel(const float* __restrict__ w,
                                                           const float* __restrict__ dw, int T, int k,
                                                           float* __restrict__ dl) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float s = 0.0f;
  for (int r = 0; r < k; ++r) s = fmaf(w[(size_t)t * k + r], dw[(size_t)t * k + r], s);
  for (int r = 0; r < k; ++r) dl[(size_t)t * k + r] = w[(size_t)t * k + r] * (dw[(size_t)t * k + r] - s);
}

// wt[e][i] = wg[i][e] through 64 x 64 LDS tiles.
__global__ __launch_bounds__(256) void gate_transpose_kernel(const float* __restrict__ wg, int d, int E,
                                                             float* __restrict__ wt) {
  __shared__ float tile[64][65];
  const int i0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  for (int q = threadIdx.x; q < 64 * 64; q += 256) {
    const int ir = q / 64, ec = q % 64;
    tile[ir][ec] = (i0 + ir < d && e0 + ec < E) ? wg[(size_t)(i0 + ir) * E + e0 + ec] : 0.0f;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * 64; q += 256) {
    const int er = q / 64, ic = q % 64;
    if (i0 + ic < d && e0 + er < E) wt[(size_t)(e0 + er) * d + i0 + ic] = tile[ic][er];
  }
}

// dx_t = sum_r dx_rows[row(t,r)] (r ascending) + dx_rows[T k + t] + sum_r dl_tr wt[e_tr]
// (r ascending), fp32; one workgroup per token, 4 columns per thread.
__global__ __launch_bounds__(1024) void route_bwd_dx_kernel(
    const float* __restrict__ dx_rows, const int32_t* __restrict__ row_of, int T, int d, int k,
    int has_shared, const int32_t* __restrict__ ids, const float* __restrict__ dl,
    const float* __restrict__ wt, int E, float* __restrict__ dx) {
  __shared__ long long srow[kMaxTopK];
  __shared__ int sid[kMaxTopK];
  __shared__ float sdl[kMaxTopK];
  const int t = blockIdx.x;
  const long long Tk = (long long)T * k;
  if (threadIdx.x < k) {
    long long r = row_of[(size_t)t * k + threadIdx.x];
    srow[threadIdx.x] = (r < 0 || r >= Tk) ? 0 : r;
    if (dl) {
      const int e = ids[(size_t)t * k + threadIdx.x];
      sid[threadIdx.x] = (e < 0 || e >= E) ? 0 : e;
      sdl[threadIdx.x] = dl[(size_t)t * k + threadIdx.x];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < k; ++r) {
      const float4 v = *(const float4*)(dx_rows + srow[r] * d + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (has_shared) {
      const float4 v = *(const float4*)(dx_rows + (Tk + t) * d + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (dl) {
      for (int r = 0; r < k; ++r) {
        const float4 v = *(const float4*)(wt + (size_t)sid[r] * d + c);
        const float q = sdl[r];
        acc.x = fmaf(q, v.x, acc.x); acc.y = fmaf(q, v.y, acc.y);
        acc.z = fmaf(q, v.z, acc.z); acc.w = fmaf(q, v.w, acc.w);
      }
    }
    *(float4*)(dx + (size_t)t * d + c) = acc;
  }
}

// dWg[:, e] = sum over expert e's dispatched rows (token ascending) of dl x_t, db[e] the
// sum of those dl; workgroup (column chunk of 1024, expert e), four adjacent columns per
// thread, so a wavefront reads 256 contiguous bytes of an MXFP8 row per load (512 bf16,
// 1024 fp32) and one scale byte serves the thread's four columns.  The rows' tokens and
// dl go through LDS in chunks of 256, and a thread issues the activation loads of 16 rows
// before their multiply-adds; each sum is one chain in ascending row order.
constexpr int kWgB = 16;   // rows per batch of loads in flight
__global__ __launch_bounds__(256) void route_bwd_wgate_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ xs, int dtype, int T, int d, int k, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const float* __restrict__ dl, float* __restrict__ dwg, float* __restrict__ db, int* flag) {
  __shared__ int stok[256];
  __shared__ float sq[256];
  const int e = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;   // d % 4 == 0
  const long long Tk = (long long)T * k;
  long long lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > Tk ? Tk : lo);
  hi = hi < lo ? lo : (hi > Tk ? Tk : hi);
  const int cc = c < d ? c : 0;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float bacc = 0.0f;
  for (long long base = lo; base < hi; base += 256) {
    const int n = (int)(hi - base < 256 ? hi - base : 256);
    if ((int)threadIdx.x < n) {
      long long p = perm[base + threadIdx.x];
      if (p < 0 || p >= Tk) {
        raise_flag(flag, kFlagCorrupt);
        p = 0;
      }
      stok[threadIdx.x] = (int)(p / k);
      sq[threadIdx.x] = dl[p];
    }
    __syncthreads();
    // rows in batches of kWgB: every load of a batch is issued before its first
    // multiply-add.  A batch's rows past n re-read row n - 1 and their results are
    // discarded (selects, no branch, so the loads stay ahead of the arithmetic).
    for (int i0 = 0; i0 < n; i0 += kWgB) {
      float q[kWgB], v[kWgB][4];
      if (dtype == MOE_MXFP8) {
        // each E4M3 code decoded exactly by the hardware, times the block scale
        // 2^(s - 127) (an fp32 value for every s < 255; s = 0 gives the subnormal 2^-127,
        // s = 255 NaN, both by setting bit 22): one rounding of the exact product, the
        // value load_act_f64 gives after its conversion to fp32
        int codes[kWgB];
        uint32_t se[kWgB];
#pragma unroll
        for (int j = 0; j < kWgB; ++j) {
          const int r = min(i0 + j, n - 1);
          const size_t row = (size_t)stok[r];
          q[j] = sq[r];
          codes[j] = *(const int*)((const uint8_t*)x + row * d + cc);
          se[j] = xs[row * (size_t)(d / 32) + cc / 32];
        }
#pragma unroll
        for (int j = 0; j < kWgB; ++j) {
          const float sc = __uint_as_float((se[j] << 23) | ((uint32_t)(se[j] == 0 || se[j] == 255) << 22));
          const auto v01 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[j], false);
          const auto v23 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[j], true);
          v[j][0] = v01[0] * sc;
          v[j][1] = v01[1] * sc;
          v[j][2] = v23[0] * sc;
          v[j][3] = v23[1] * sc;
        }
      } else if (dtype == MOE_BF16) {
#pragma unroll
        for (int j = 0; j < kWgB; ++j) {
          const int r = min(i0 + j, n - 1);
          q[j] = sq[r];
          const u32x2_t u = *(const u32x2_t*)((const uint16_t*)x + (size_t)stok[r] * d + cc);
          v[j][0] = __uint_as_float(u[0] << 16);
          v[j][1] = __uint_as_float(u[0] & 0xffff0000u);
          v[j][2] = __uint_as_float(u[1] << 16);
          v[j][3] = __uint_as_float(u[1] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kWgB; ++j) {
          const int r = min(i0 + j, n - 1);
          q[j] = sq[r];
          const float4 f = *(const float4*)((const float*)x + (size_t)stok[r] * d + cc);
          v[j][0] = f.x;
          v[j][1] = f.y;
          v[j][2] = f.z;
          v[j][3] = f.w;
        }
      }
#pragma unroll
      for (int j = 0; j < kWgB; ++j) {
        const bool live = i0 + j < n;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = fmaf(q[j], v[j][t], acc[t]);
          acc[t] = live ? a : acc[t];
        }
        const float b = bacc + q[j];
        bacc = live ? b : bacc;
      }
    }
    __syncthreads();
  }
  if (c < d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dwg[(size_t)(c + j) * E + e] = acc[j];
  }
  if (db && blockIdx.x == 0 && threadIdx.x == 0) db[e] = bacc;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_backward_workspace_size(int T, int d, int E, int k, int inter, int dtype,
                                                  size_t* bytes) {
  if (!bytes || T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxTopK ||
      inter < 1 || !valid_layer_dtype(dtype))
    return MOE_ERR_INVALID_ARG;
  const size_t a = workspace_bytes(T, d, E, k, inter, dtype);
  const size_t b = dtype == MOE_MXFP8 || dtype == MOE_NVFP4
                       ? mxfp8_backward_ws_bytes(T, d, E, k, inter, dtype == MOE_NVFP4)
                       : bwd_ws(T, d, E, k, inter).bytes;
  *bytes = a > b ? a : b;
  return MOE_OK;
}

extern "C" moe_status moe_combine_backward(const void* dy, int dtype, const void* out,
                                           const int32_t* row_of, const float* weights, int T, int d,
                                           int k, int has_shared, void* d_out, float* d_weights,
                                           void* stream) {
  if (!valid_dtype(dtype) || T < 0 || d < 1 || k < 1 || k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dy || !out || !row_of || !weights || !d_out || !d_weights) return MOE_ERR_INVALID_ARG;
  if (!aligned(dy, 16) || !aligned(out, 16) || !aligned(d_out, 16)) return MOE_ERR_INVALID_ARG;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const int chunks = d / 8, passes = (chunks + 1023) / 1024;
  const int thr = ((chunks + passes - 1) / passes + 63) / 64 * 64;
  if (dtype == MOE_F32)
    combine_bwd_kernel<true><<<T, thr, 0, s>>>(dy, out, row_of, weights, T, d, k, has_shared ? 1 : 0,
                                               d_out, d_weights);
  else
    combine_bwd_kernel<false><<<T, thr, 0, s>>>(dy, out, row_of, weights, T, d, k, has_shared ? 1 : 0,
                                                d_out, d_weights);
  return launch_status();
}

static bool grads_ok(const moe_grad_bank* g) {
  return g && g->dw1 && g->dw3 && g->dw2 && aligned(g->dw1, 16) && aligned(g->dw3, 16) &&
         aligned(g->dw2, 16);
}

// Argument checks and kernel arguments shared by the three expert-backward entry points.
static moe_status bwd_setup(const void* x, const uint8_t* x_scale, int dtype, int T, int d, int E, int k,
                            int inter, const moe_expert_bank* routed, const moe_expert_bank* shared,
                            const int32_t* offsets, const int32_t* perm, const float* pre,
                            const void* d_out,
                            float* dx_rows, const moe_grad_bank* routed_grads,
                            const moe_grad_bank* shared_grads, void* ws, size_t ws_bytes, bool data,
                            bool weights, BwdGemm& g) {
  if (!valid_dtype(dtype) || T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E ||
      k > kMaxTopK || inter < 1)
    return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (x_scale) return MOE_ERR_INVALID_ARG;
  if (d % 128 != 0 || inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!ws || !routed || !routed->w1 || !routed->w3 || !routed->w2 || routed->w1_scale ||
      routed->w3_scale || routed->w2_scale)
    return MOE_ERR_INVALID_ARG;
  if (shared && (!shared->w1 || !shared->w3 || !shared->w2)) return MOE_ERR_INVALID_ARG;
  if (weights) {
    if (!grads_ok(routed_grads)) return MOE_ERR_INVALID_ARG;
    if ((shared != nullptr) != (shared_grads != nullptr)) return MOE_ERR_INVALID_ARG;
    if (shared && !grads_ok(shared_grads)) return MOE_ERR_INVALID_ARG;
  }
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  const BwdWs L = bwd_ws(T, d, E, k, inter);
  if (ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;
  if (T > 0 && (!x || !perm || !aligned(x, 16) || (data && !offsets))) return MOE_ERR_INVALID_ARG;
  if (T > 0 && data && (!d_out || !dx_rows || !aligned(d_out, 16) || !aligned(dx_rows, 16)))
    return MOE_ERR_INVALID_ARG;
  const moe_expert_bank* banks[2] = {routed, shared};
  for (const moe_expert_bank* b : banks)
    if (b && (!aligned(b->w1, 16) || !aligned(b->w3, 16) || !aligned(b->w2, 16)))
      return MOE_ERR_INVALID_ARG;
  char* w = (char*)ws;
  const int has_shared = shared ? 1 : 0;
  g = BwdGemm{};
  g.x = (const uint16_t*)x;
  g.perm = perm;
  g.T = T;
  g.k = k;
  g.E = E;
  g.d = d;
  g.I = inter;
  g.Tk = (long long)T * k;
  g.w1 = (const uint16_t*)routed->w1;
  g.w3 = (const uint16_t*)routed->w3;
  g.w2 = (const uint16_t*)routed->w2;
  g.sw1 = shared ? (const uint16_t*)shared->w1 : nullptr;
  g.sw3 = shared ? (const uint16_t*)shared->w3 : nullptr;
  g.sw2 = shared ? (const uint16_t*)shared->w2 : nullptr;
  g.d_out = (const uint16_t*)d_out;
  if (pre && !aligned(pre, 16)) return MOE_ERR_INVALID_ARG;
  g.pre = pre ? pre : (const float*)(w + L.pre);
  g.dadg = (uint16_t*)(w + L.dadg);
  g.h = (uint16_t*)(w + L.h);
  g.dx_rows = dx_rows;
  if (weights) {
    g.dw1 = routed_grads->dw1;
    g.dw3 = routed_grads->dw3;
    g.dw2 = routed_grads->dw2;
    g.sdw1 = shared ? shared_grads->dw1 : nullptr;
    g.sdw3 = shared ? shared_grads->dw3 : nullptr;
    g.sdw2 = shared ? shared_grads->dw2 : nullptr;
  }
  g.tokrow = (int*)(w + L.tokrow);
  int* seg = (int*)(w + L.seg);
  g.mstart = seg;
  g.rowstart = seg + (E + 2);
  g.rowcount = seg + 2 * (E + 2);
  g.S = E + has_shared;
  g.flag = (int*)w;
  return MOE_OK;
}

// Data half: recomputed pre-activations, dh with the SwiGLU backward, dx_rows.
static moe_status bwd_data(BwdGemm& g, const moe_expert_bank* routed, const moe_expert_bank* shared,
                           const int32_t* offsets, bool saved, hipStream_t s) {
  if (g.T == 0) return MOE_OK;
  moe_status st = saved ? ffn_seg_table(offsets, g.T, g.E, g.k, g.S > g.E, (int*)g.mstart, g.flag, s)
                        : ffn_recompute_pre(g.x, g.T, g.d, g.E, g.k, g.I, routed, shared, offsets, g.perm,
                                            (int*)g.mstart, (float*)g.pre, g.flag, s);
  if (st != MOE_OK) return st;
  const long long mt_bound =
      (g.Tk + (long long)g.E * (GB_T - 1)) / GB_T + (g.S > g.E ? (g.T + GB_T - 1) / GB_T : 0);
  // 256-column tiles where the output width allows them, else 128
  const bool wide_dh = g.I % 256 == 0, wide_dx = g.d % 256 == 0;
  g.NT = g.I / (wide_dh ? 256 : 128);
  long long grid = tile_grid(mt_bound * g.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (wide_dh) bwd_gemm_kernel<BK_DH, 4><<<(unsigned)grid, gb_thr(4), 0, s>>>(g);
  else bwd_gemm_kernel<BK_DH, 2><<<(unsigned)grid, gb_thr(2), 0, s>>>(g);
  g.NT = g.d / (wide_dx ? 256 : 128);
  grid = tile_grid(mt_bound * g.NT, 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (wide_dx) bwd_gemm_kernel<BK_DX, 4><<<(unsigned)grid, gb_thr(4), 0, s>>>(g);
  else bwd_gemm_kernel<BK_DX, 2><<<(unsigned)grid, gb_thr(2), 0, s>>>(g);
  return launch_status();
}

// Weights half: dW2, then dW1 and dW3, for every expert (and the shared one).
static moe_status bwd_weights(BwdGemm& g, hipStream_t s) {
  if (g.T == 0) {   // empty batch: every weight gradient is zero
    const long long n13 = (long long)g.E * g.I * g.d;
    zero_fill(g.dw1, n13, s);
    zero_fill(g.dw3, n13, s);
    zero_fill(g.dw2, n13, s);
    if (g.S > g.E) {
      zero_fill(g.sdw1, (long long)g.I * g.d, s);
      zero_fill(g.sdw3, (long long)g.I * g.d, s);
      zero_fill(g.sdw2, (long long)g.I * g.d, s);
    }
    return launch_status();
  }
  const long long rows = g.Tk + (g.S > g.E ? g.T : 0);
  tokrow_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(g.perm, g.T, g.k, rows, g.tokrow, g.flag);
  g.MT = g.d / GB_T;
  g.NT = g.I / GB_T;
  if (g.NT % kBwdNtw != 0 || (g.d / GB_T) % kBwdNtw != 0) return MOE_ERR_UNSUPPORTED;
  long long grid = tile_grid((long long)g.S * g.MT * (g.NT / kBwdNtw), 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  bwd_gemm_kernel<BK_DW2, 2><<<(unsigned)grid, gb_thr(2), 0, s>>>(g);
  g.MT = 2 * g.I / GB_T;
  g.NT = g.d / GB_T;
  grid = tile_grid((long long)g.S * g.MT * (g.NT / kBwdNtw), 0);
  if (grid > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  bwd_gemm_kernel<BK_DW13, 2><<<(unsigned)grid, gb_thr(2), 0, s>>>(g);
  return launch_status();
}

extern "C" moe_status moe_expert_ffn_backward(const void* x, const uint8_t* x_scale, int dtype, int T,
                                              int d, int E, int k, int inter,
                                              const moe_expert_bank* routed,
                                              const moe_expert_bank* shared, const int32_t* offsets,
                                              const int32_t* perm, const float* pre, const void* d_out,
                                              float* dx_rows, const moe_grad_bank* routed_grads,
                                              const moe_grad_bank* shared_grads, void* ws,
                                              size_t ws_bytes, void* stream) {
  BwdGemm g;
  moe_status st = bwd_setup(x, x_scale, dtype, T, d, E, k, inter, routed, shared, offsets, perm, pre,
                            d_out, dx_rows, routed_grads, shared_grads, ws, ws_bytes, true, true, g);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = bwd_data(g, routed, shared, offsets, pre != nullptr, s)) != MOE_OK) return st;
  return bwd_weights(g, s);
}

extern "C" moe_status moe_expert_ffn_backward_data(const void* x, const uint8_t* x_scale, int dtype,
                                                   int T, int d, int E, int k, int inter,
                                                   const moe_expert_bank* routed,
                                                   const moe_expert_bank* shared,
                                                   const int32_t* offsets, const int32_t* perm,
                                                   const float* pre, const void* d_out,
                                                   float* dx_rows, void* ws, size_t ws_bytes,
                                                   void* stream) {
  BwdGemm g;
  moe_status st = bwd_setup(x, x_scale, dtype, T, d, E, k, inter, routed, shared, offsets, perm, pre,
                            d_out, dx_rows, nullptr, nullptr, ws, ws_bytes, true, false, g);
  if (st != MOE_OK) return st;
  return bwd_data(g, routed, shared, offsets, pre != nullptr, (hipStream_t)stream);
}

extern "C" moe_status moe_expert_ffn_backward_weights(const void* x, int dtype, int T, int d, int E,
                                                      int k, int inter, const moe_expert_bank* routed,
                                                      const moe_expert_bank* shared,
                                                      const int32_t* perm, const void* d_out,
                                                      const moe_grad_bank* routed_grads,
                                                      const moe_grad_bank* shared_grads, void* ws,
                                                      size_t ws_bytes, void* stream) {
  BwdGemm g;
  moe_status st = bwd_setup(x, nullptr, dtype, T, d, E, k, inter, routed, shared, nullptr, perm, nullptr,
                            d_out, nullptr, routed_grads, shared_grads, ws, ws_bytes, false, true, g);
  if (st != MOE_OK) return st;
  if (T > 0 && (!d_out || !aligned(d_out, 16))) return MOE_ERR_INVALID_ARG;
  return bwd_weights(g, (hipStream_t)stream);
}

extern "C" moe_status moe_route_backward(const void* x, const uint8_t* x_scale, int dtype, int T, int d,
                                         const float* w_gate, int E, int k, const int32_t* ids,
                                         const float* weights, const float* d_weights,
                                         const int32_t* offsets, const int32_t* perm,
                                         const int32_t* row_of, const float* dx_rows, int has_shared,
                                         float* dx, float* d_w_gate, float* d_bias, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype) || T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E ||
      k > kMaxTopK)
    return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_MXFP8 && (!x_scale || d % 32 != 0)) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_MXFP8 && x_scale) return MOE_ERR_INVALID_ARG;
  if (d % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (d_bias && !d_w_gate) return MOE_ERR_INVALID_ARG;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const BwdWs L = bwd_ws(T, d, E, k, 0);   // dl and wt come before every inter-sized buffer
  if (ws_bytes < L.wt + (size_t)E * d * sizeof(float)) return MOE_ERR_WORKSPACE;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  if (T == 0) {
    if (d_w_gate) zero_fill(d_w_gate, (long long)d * E, s);
    if (d_bias) zero_fill(d_bias, E, s);
    return launch_status();
  }
  if (!x || !row_of || !dx_rows || !dx || !aligned(dx_rows, 16) || !aligned(dx, 16))
    return MOE_ERR_INVALID_ARG;
  if (d_w_gate && (!w_gate || !ids || !weights || !d_weights || !offsets || !perm ||
                   !aligned(x, 16)))
    return MOE_ERR_INVALID_ARG;
  float* dl = nullptr;
  float* wt = nullptr;
  if (d_w_gate) {
    dl = (float*)(w + L.dl);
    wt = (float*)(w + L.wt);
    route_bwd_dl_kernel<<<(T + 255) / 256, 256, 0, s>>>(weights, d_weights, T, k, dl);
    gate_transpose_kernel<<<dim3((d + 63) / 64, (E + 63) / 64), 256, 0, s>>>(w_gate, d, E, wt);
  }
  const int q4 = d / 4, passes = (q4 + 1023) / 1024;
  const int thr = ((q4 + passes - 1) / passes + 63) / 64 * 64;
  route_bwd_dx_kernel<<<T, thr, 0, s>>>(dx_rows, row_of, T, d, k, has_shared ? 1 : 0, ids, dl, wt, E, dx);
  if (d_w_gate)
    route_bwd_wgate_kernel<<<dim3((d + 1023) / 1024, E), 256, 0, s>>>(x, x_scale, dtype, T, d, k, E, offsets,
                                                                      perm, dl, d_w_gate, d_bias, (int*)w);
  return launch_status();
}
