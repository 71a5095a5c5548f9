// Internal helpers shared by the libmoe translation units: workspace layout,
// device error flags, element decoding, host-side argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <math.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// Limits and tile constants
// ---------------------------------------------------------------------------
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kDispatchTokens = 64;   // tokens per dispatch block
constexpr int kGemmBM = 128;          // rows per grouped-GEMM tile

// Device error flag bits (OR-ed into the workspace header).
constexpr int kFlagBadId = 1;
constexpr int kFlagDupId = 2;
constexpr int kFlagNonFinite = 4;
constexpr int kFlagCorrupt = 8;       // internal consistency (bad offsets/perm fed to the FFN)

constexpr size_t kHeaderBytes = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Workspace layout.  Byte 0..255: header (int flag at offset 0).  The rest is
// scratch that each call uses for its own duration only.
// ---------------------------------------------------------------------------
// K-splits of the fp64 gate sums: the reduction over d restarts every d / S
// elements and the S partial sums are added in ascending order.  S depends on d
// only, never on T, so every logit has the same summation order in every batch.
inline int gate_splits(int d) {
  if (d % 64 != 0) return 1;
  const int steps = d / 64;
  for (int s = 8; s > 1; s >>= 1)
    if (steps % s == 0 && steps / s >= 4) return s;
  return 1;
}
// Output tiles of the gate (64 tokens x 32 experts) below which the K-splits run in
// separate workgroups (partial sums in the workspace) instead of one after another.
constexpr int kGateSplitTiles = 256;
inline int gate_tiles(int T, int E) { return ((T + 63) / 64) * ((E + 31) / 32); }
inline bool gate_split_launch(int T, int d, int E) {
  return gate_splits(d) > 1 && gate_tiles(T, E) < kGateSplitTiles;
}

// Candidate experts per token kept by the bf16 screen of the gate (more go to the
// exact fallback).
constexpr int kCandMax = 32;

// K parts of the bf16 screen: enough workgroups (128 tokens x 128 experts x part) to
// fill the chip; the screen has no fixed-order requirement.
inline int screen_parts(int T, int d, int E) {
  const int tiles = ((E + 127) / 128) * ((T + 127) / 128);
  const int steps = d / 64;
  if (tiles < 1 || steps < 1) return 1;
  int nz = (512 + tiles - 1) / tiles;
  if (nz > 16) nz = 16;
  if (nz > steps / 4) nz = steps / 4;
  if (nz < 1) nz = 1;
  // a split K: as many (expert tile, K part) slices as a multiple of the 8 XCDs where the
  // limits allow (each XCD then runs whole slices, see gate_screen_kernel)
  const int et = (E + 127) / 128;
  if (nz > 1)
    for (int z = nz; z <= 16 && z <= steps / 4; ++z)
      if ((et * z) % 8 == 0 && (steps + (steps + z - 1) / z - 1) / ((steps + z - 1) / z) == z) {
        nz = z;
        break;
      }
  const int spart = (steps + nz - 1) / nz;
  return (steps + spart - 1) / spart;
}

struct RouteWs {
  size_t logits, tok_flag, xnorm, wnorm, part, xsq, wsq;   // fp64 gate GEMM path
  size_t wt, planes, cand, cval, ccount, screen, sxsq, pblk, pcnt, pairs;   // screened path
  size_t bytes;
};
inline RouteWs route_ws(int T, int d, int E) {
  RouteWs w;
  const size_t S = gate_split_launch(T, d, E) ? (size_t)gate_splits(d) : 0;
  size_t o = kHeaderBytes;
  w.logits = o;   o = align_up(o + (size_t)T * E * sizeof(double), 256);
  w.tok_flag = o; o = align_up(o + (size_t)T * sizeof(int), 256);
  w.xnorm = o;    o = align_up(o + (size_t)T * sizeof(double), 256);
  w.wnorm = o;    o = align_up(o + (size_t)E * sizeof(double), 256);
  w.part = o;     o = align_up(o + S * T * E * sizeof(double), 256);
  w.xsq = o;      o = align_up(o + S * T * sizeof(double), 256);
  w.wsq = o;      o = align_up(o + S * E * sizeof(double), 256);
  w.wt = o;       o = align_up(o + (size_t)E * d * sizeof(float), 256);
  w.planes = o;   o = align_up(o + (size_t)3 * E * d * sizeof(uint16_t), 256);
  w.cand = o;     o = align_up(o + (size_t)T * kCandMax * sizeof(int32_t), 256);
  w.cval = o;     o = align_up(o + (size_t)T * kCandMax * sizeof(double), 256);
  w.ccount = o;   o = align_up(o + (size_t)T * sizeof(int), 256);
  const size_t nz = d % 64 == 0 ? (size_t)screen_parts(T, d, E) : 1;
  w.screen = o;   o = align_up(o + nz * T * E * sizeof(double), 256);
  w.sxsq = o;     o = align_up(o + nz * T * sizeof(double), 256);
  w.pblk = o;     o = align_up(o + (size_t)((T + 255) / 256) * E * sizeof(int), 256);
  w.pcnt = o;     o = align_up(o + (size_t)(3 * E + 2) * sizeof(int), 256);
  w.pairs = o;    o = align_up(o + (size_t)T * kCandMax * sizeof(int32_t), 256);
  w.bytes = o;
  return w;
}

// bf16 and MXFP8 activations with d % 64 == 0 take their weights (and, under
// replay, everything) from per-pair fp64 logits; the ids come from the bf16 screen
// for large batches and from the fp64 gate GEMM for small ones (gate_split_launch).
// fp32 activations use the fp64 gate GEMM for ids and weights.
inline bool gate_screened(int dtype, int d) {
  return (dtype == MOE_BF16 || dtype == MOE_MXFP8) && d % 64 == 0;
}

struct DispatchWs {
  size_t hist, total, bytes;
  int nblocks;
};
inline DispatchWs dispatch_ws(int T, int E) {
  DispatchWs w;
  w.nblocks = (T + kDispatchTokens - 1) / kDispatchTokens;
  size_t o = kHeaderBytes;
  w.hist = o;  o = align_up(o + (size_t)w.nblocks * E * sizeof(int), 256);
  w.total = o; o = align_up(o + (size_t)E * sizeof(int), 256);
  w.bytes = o;
  return w;
}

inline size_t elem_bytes_h(int dtype) { return dtype == MOE_F32 ? 4 : (dtype == MOE_BF16 ? 2 : 1); }

struct FfnWs {
  size_t h, hs, seg;
  size_t xc, xs, xr, hc, hsc, hr;   // NVFP4: quantized x (codes, block scales, row scales) and h
  size_t bytes;
  long long rows;
};
// h: intermediate activations [T*k + T][inter] (fp32 / bf16 / E4M3 codes; bf16 for NVFP4);
// hs: E8M0 scales of h [T*k + T][inter/32] (MXFP8 only);
// seg table: mstart[S+1] (int), rowstart[S] (int), rowcount[S] (int), S = E + 1;
// NVFP4 only: x and h quantized per row to NVFP4, kept as their decoded values
// E2M1 * E4M3 (exact in bf16; [T][d] and [rows][inter]) and fp32 row scales.
inline FfnWs ffn_ws(int T, int d, int E, int k, int inter, int dtype) {
  FfnWs w;
  w.rows = (long long)T * k + T;
  const bool nv = dtype == MOE_NVFP4;
  size_t o = kHeaderBytes;
  w.h = o;   o = align_up(o + (size_t)w.rows * inter * (nv ? 2 : elem_bytes_h(dtype)), 256);
  w.hs = o;  o = align_up(o + (dtype == MOE_MXFP8 ? (size_t)w.rows * (inter / 32) : 0), 256);
  w.seg = o; o = align_up(o + (size_t)(3 * (E + 2)) * sizeof(int), 256);
  const size_t tn = nv ? (size_t)T : 0, rn = nv ? (size_t)w.rows : 0;
  w.xc = o;  o = align_up(o + tn * d * 2, 256);           // decoded x (bf16)
  w.xs = o;  o = align_up(o, 256);
  w.xr = o;  o = align_up(o + tn * sizeof(float), 256);
  w.hc = o;  o = align_up(o + rn * inter * 2, 256);       // decoded h (bf16)
  w.hsc = o; o = align_up(o, 256);
  w.hr = o;  o = align_up(o + rn * sizeof(float), 256);
  w.bytes = o;
  return w;
}

inline size_t workspace_bytes(int T, int d, int E, int k, int inter, int dtype) {
  size_t a = route_ws(T, d, E).bytes, b = dispatch_ws(T, E).bytes, c = ffn_ws(T, d, E, k, inter, dtype).bytes;
  size_t m = a > b ? a : b;
  return m > c ? m : c;
}

// Backward pass (bf16 layers): segment table, the token of each dispatched row,
// recomputed pre-activations a | g
// [rows][2 inter] fp32, their gradients da | dg [rows][2 inter] bf16, h [rows][inter]
// bf16, the routing-weight gradients through the gate dl [T][k] fp32, the transposed
// gate [E][d] fp32.
struct BwdWs {
  size_t seg, tokrow, pre, dadg, h, dl, wt, bytes;
  long long rows;
};
inline BwdWs bwd_ws(int T, int d, int E, int k, int inter) {
  BwdWs w;
  w.rows = (long long)T * k + T;
  size_t o = kHeaderBytes;
  w.seg = o;  o = align_up(o + (size_t)(3 * (E + 2)) * sizeof(int), 256);
  w.dl = o;   o = align_up(o + (size_t)T * k * sizeof(float), 256);
  w.wt = o;   o = align_up(o + (size_t)E * d * sizeof(float), 256);
  w.tokrow = o; o = align_up(o + (size_t)w.rows * sizeof(int), 256);
  w.pre = o;  o = align_up(o + (size_t)w.rows * 2 * inter * sizeof(float), 256);
  w.dadg = o; o = align_up(o + (size_t)w.rows * 2 * inter * sizeof(uint16_t), 256);
  w.h = o;    o = align_up(o + (size_t)w.rows * inter * sizeof(uint16_t), 256);
  w.bytes = o;
  return w;
}

inline bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16 || dt == MOE_MXFP8; }
// The expert FFN (and the workspace) also takes NVFP4 experts (with bf16 x).
inline bool valid_layer_dtype(int dt) { return valid_dtype(dt) || dt == MOE_NVFP4; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline moe_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_flag(int* ws_flag, int bits) { atomicOr(ws_flag, bits); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP FP8 E4M3 code -> exact value (as double; every E4M3 value is exact in fp32 too).
// Normal codes (exponent field e > 0) are (1 + m/8) 2^(e-7): the fp64 bit pattern is
// built directly (biased exponent e + 1016, the 3 mantissa bits at the top of the
// fraction).  Subnormal codes are m 2^-9.  Exponent 15 with mantissa 7 is NaN.
__device__ __forceinline__ double e4m3_to_f64(uint8_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  double v;
  if (e == 15u && m == 7u) v = __builtin_nan("");
  else if (e == 0u) v = (double)m * 0x1p-9;
  else v = __hiloint2double((int)(((e + 1016u) << 20) | (m << 17)), 0);
  return (c & 0x80u) ? -v : v;
}

// E8M0 scale code -> 2^(code-127) (255 is NaN); every such power is a normal double.
__device__ __forceinline__ double e8m0_to_f64(uint8_t c) {
  return c == 255 ? __builtin_nan("") : __hiloint2double((int)((uint32_t)(c + 896) << 20), 0);
}

// Exact value of element i of activation row `row` (length d) in `dtype`.
__device__ __forceinline__ double load_act_f64(const void* x, const uint8_t* xs, int dtype,
                                               size_t row, int d, int i) {
  size_t idx = row * (size_t)d + i;
  if (dtype == MOE_F32) return (double)((const float*)x)[idx];
  if (dtype == MOE_BF16) return (double)bf16_to_f32(((const uint16_t*)x)[idx]);
  return e4m3_to_f64(((const uint8_t*)x)[idx]) * e8m0_to_f64(xs[row * (size_t)(d / 32) + i / 32]);
}

// ---------------------------------------------------------------------------
// Grouped-GEMM tile order across the XCDs
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;      // MI355X: 8 XCDs, workgroups dealt round-robin

// Row tiles per raster group of the grouped GEMMs: within a group, consecutive tiles
// share a weight slab (column tile) and the group's activation rows are reused by every
// column tile.
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 8
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;

// Tile of this workgroup.  Workgroup b runs on XCD b % 8.  With CHUNK == 0, XCD x takes
// the x-th eighth of the tile list; otherwise the list is cut into chunks of CHUNK tiles
// dealt round-robin to the XCDs.  Either way an XCD runs its tiles in list order, so
// neighbouring tiles (which share weight columns or activation rows) share its L2.
// The bf16 GEMMs keep contiguous eighths (each XCD streams one contiguous run of the
// weight banks); the MXFP8 GEMMs deal chunks of 16 (measured: bf16 GEMM2 +12% with
// chunks, MXFP8 GEMMs -3 to -4%).
template <int CHUNK>
__device__ __forceinline__ bool xcd_tile(int total, int& tile) {
  const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
  if constexpr (CHUNK == 0) {
    const int per = (total + kXcds - 1) / kXcds;
    if (q >= per) return false;
    tile = xcd * per + q;
  } else {
    tile = ((q / CHUNK) * kXcds + xcd) * CHUNK + q % CHUNK;
  }
  return tile < total;
}
// Workgroups to launch for at most `bound` tiles.
inline long long tile_grid(long long bound, int chunk) {
  const long long g = chunk == 0 ? kXcds : (long long)kXcds * chunk;
  return (bound + g - 1) / g * g;
}
// sigmoid(a) = 1 / (1 + e^-a) from the hardware 2^x and reciprocal (each within about one
// ulp), two instructions instead of the library's exp and IEEE division; silu(a) = a sigmoid(a).
// Every kernel that forms silu (forward epilogues, the backward's recomputation of h and
// its derivative) uses these two, so a backward sees the same h as its forward.
__device__ __forceinline__ float sigmoid_f32(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_f32(float a) { return a * sigmoid_f32(a); }

// MXFP8 expert FFN GEMMs (mxfp8.hip) over the segment table of the FFN: GEMM1 (mode 0:
// x W1, x W3, SwiGLU, h requantised to MXFP8 per row) and GEMM2 (mode 1: h W2 -> bf16).
struct MxArgs {
  const uint8_t* a;          // GEMM1: x codes [T][d]; GEMM2: h codes [rows][I]
  const uint8_t* as;         // matching E8M0 scales [.][K/32]
  const int32_t* perm;
  int T, k, E;
  long long Tk;
  const uint8_t* b0;         // GEMM1: W1 codes; GEMM2: W2 codes
  const uint8_t* b1;         // GEMM1: W3 codes
  const uint8_t* b0s;
  const uint8_t* b1s;
  const uint8_t* sb0;        // shared expert
  const uint8_t* sb1;
  const uint8_t* sb0s;
  const uint8_t* sb1s;
  int K, N, NT;
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  int S;
  void* out;                 // GEMM1: h codes [rows][I]; GEMM2: bf16 [rows][d]
  uint8_t* out_scale;        // GEMM1: h scales [rows][I/32]
  float* out_pre;            // GEMM1 (mode 0, optional; mode 2): fp32 x W1 | x W3 [rows][2I]
  int* flag;
  int tm;                    // rows per tile (mx_tile_rows), as counted by the segment table
  const float* pre_in;       // backward dh (mode 3): the forward's x W1 | x W3 [rows][2N]
  float* out_f;              // backward: da | dg [rows][2N] (mode 3); dx rows [rows][N] (mode 4)
};
// Rows per tile of the MXFP8 GEMMs for hidden size d, intermediate size inter and Tk
// routed rows over E experts (the segment table counts tiles of this height).  Every
// row's result is the same whatever the tile height.
int mx_tile_rows(int d, int inter, long long Tk, int E);
// Launch GEMM1 (mode 0; mode 2: only the pre-activations into out_pre) or GEMM2 (mode 1);
// mt_bound bounds the segment table's row tiles.
moe_status mx_gemm(int mode, MxArgs g, long long mt_bound, hipStream_t s);
// The MXFP8 backward's data GEMMs on the 128-row ring (A: row-quantised gradient rows;
// B: the requantised weights, rows N x K per expert): mode 3 dh = dq W2t^T with the SwiGLU
// backward at pre_in into out_f (da | dg), mode 4 dx rows = dgq W13t^T into out_f.
// MOE_ERR_UNSUPPORTED where the ring does not tile d and inter (the caller then uses its
// own kernel); the segment table must count 128-row tiles.
moe_status mx_gemm_bwd_data(int mode, int d, int inter, MxArgs g, long long mt_bound, hipStream_t s);

// NVFP4 expert FFN (nvfp4.hip).
struct Nvfp4Gemm {
  const uint16_t* a;       // A decoded (E2M1 * E4M3, bf16) [rows][K], fp32 row scales
  const float* ar;
  const int32_t* perm;     // GEMM1: the A row of output row j is token perm[j] / k
  int T, k, E;
  const uint8_t* b0;       // GEMM1: W1 and W3 banks; GEMM2: W2
  const uint8_t* b1;
  const uint8_t* b0s;
  const uint8_t* b1s;
  const float* b0r;
  const float* b1r;
  const uint8_t* sb0;      // shared expert
  const uint8_t* sb1;
  const uint8_t* sb0s;
  const uint8_t* sb1s;
  const float* sb0r;
  const float* sb1r;
  int K, N;
  const int* mstart;
  const int* rowstart;
  const int* rowcount;
  int S;
  long long mt_bound;
  uint16_t* out;
  float* out_pre;          // GEMM1 (optional): fp32 a | g [rows][2N] with the row scales applied
  int* flag;
};
// h = bf16(silu(a) g) of rows of fp32 pre-activations a | g [rows][2I], with the NVFP4
// GEMM1's epilogue arithmetic (nvfp4.hip).
moe_status nvfp4_h_from_pre(const float* pre, long long rows, int I, uint16_t* h, hipStream_t s);
moe_status nvfp4_quantize_rows(const uint16_t* src, long long rows, int K, uint8_t* codes, uint8_t* bscale,
                               float* rscale, uint16_t* dec, hipStream_t s);
moe_status nvfp4_gemm(int mode, const Nvfp4Gemm& q, hipStream_t s);

// Backward-pass support from the forward FFN (ffn.hip): the segment table for 128-row
// tiles into seg (mstart [E + 2], rowstart [E + 2], rowcount [E + 2]) and the GEMM1
// pre-activations of every dispatched row, pre [rows][2 inter] fp32 (x W1, then x W3),
// with the forward's MFMA sequence (bf16 only).
// Zero fill of n floats by a kernel (backward.hip).
void zero_fill(float* p, long long n, hipStream_t s);
// Workspace bytes of the MXFP8 backward (mxfp8_bwd.hip) of an MXFP8 or an NVFP4 layer.
size_t mxfp8_backward_ws_bytes(int T, int d, int E, int k, int inter, bool nvfp4_layer);
// Segment table with tiles of tm rows (ffn_seg_table: tm = kGemmBM).
moe_status ffn_seg_table_rows(const int32_t* offsets, int T, int E, int k, int has_shared, int tm, int* seg,
                              int* flag, hipStream_t s);
moe_status ffn_seg_table(const int32_t* offsets, int T, int E, int k, int has_shared, int* seg, int* flag,
                         hipStream_t s);
moe_status ffn_recompute_pre(const void* x, int T, int d, int E, int k, int inter,
                             const moe_expert_bank* routed, const moe_expert_bank* shared,
                             const int32_t* offsets, const int32_t* perm, int* seg, float* pre,
                             int* flag, hipStream_t s);

// Screened gate (screen.hip).  screen_route_select leaves ids for every token and
// tok_flag 1 for the tokens the exact fallback must decide; screen_route_weights then
// writes the weights of the final ids.
moe_status screen_route_select(const void* x, const uint8_t* xs, int dtype, int T, int d,
                               const float* w_gate, const float* bias, int E, int k, int32_t* ids,
                               char* ws, hipStream_t s);
moe_status screen_route_weights(const void* x, const uint8_t* xs, int dtype, int T, int d,
                                const float* bias, int E, int k, const int32_t* ids,
                                const float* weights_in, float* weights, char* ws, hipStream_t s);
moe_status chosen_ids_refine(const void* x, const uint8_t* xs, int dtype, int T, int d,
                             const float* w_gate, const float* bias, int E, int k, const int32_t* ids,
                             char* ws, hipStream_t s);
moe_status screen_replay(const void* x, const uint8_t* xs, int dtype, int T, int d,
                         const float* w_gate, const float* bias, int E, int k, const int32_t* ids_in,
                         const float* weights_in, float* weights_out, char* ws, hipStream_t s);

// Replay plausibility filter, run after moe_route has left the router's ids in `ids`
// and its fp64 logits (or candidate logits) in the workspace.
struct FilterArgs {
  const void* x;
  const uint8_t* xs;
  int dtype, T, d, E, k;
  const float* bias;
  const int32_t* ids_in;
  double log_tau;
  double tg;            // relative fp64 logit bound: |l~ - l| <= tg (||x|| ||w_e|| + |b_e|)
  int32_t* ids;         // in: router top-k in rank order; out: the filtered ids
  float* weights;
  // filled by filter_launch from the workspace
  const double* logits; // fp64 gate logits [T][E] (unscreened gate), else null
  const float* wt;      // transposed gate [E][d] (screened gate)
  const int32_t* cand;
  const int* ccount;
  const double* cval;
  const double* xnorm;
  const double* wnorm;
  int* tok_flag;
  int* flag;
};
// pass 0: certified decisions, ids and weights; tokens it cannot certify get
// tok_flag 1.  pass 1: weights of those tokens once their ids are final.
moe_status filter_launch(FilterArgs a, bool screened, char* ws, int pass, hipStream_t s);

}  // namespace moe
