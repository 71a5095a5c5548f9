// Combine: each token's output is the routing-weighted sum of its k expert outputs
// (plus the shared expert's), summed in one fixed order with fp32 fused multiply-adds
// and rounded once (Composer 2 Technical Report, section 6.1 "Parallelism": the
// combine is kept in BF16; the fixed order follows the batch-invariant kernels of the
// Training Data podcast page, section on floating point and MoE).  No atomics: one
// workgroup owns one token row, so the result never depends on scheduling.
#include "moe_internal.h"

namespace moe {

template <bool kF32>
__global__ __launch_bounds__(1024) void combine_kernel(const void* __restrict__ out,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ weights, int T, int d,
                                                      int k, int has_shared, long long rows,
                                                      void* __restrict__ y) {
  __shared__ float sw[kMaxTopK];
  __shared__ long long srow[kMaxTopK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    sw[threadIdx.x] = weights[(size_t)t * k + threadIdx.x];
    long long r = row_of[(size_t)t * k + threadIdx.x];
    srow[threadIdx.x] = (r < 0 || r >= rows) ? 0 : r;   // guard against corrupt input
  }
  __syncthreads();
  const long long shared_row = (long long)T * k + t;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int r = 0; r < k; ++r) {
      const float w = sw[r];
      float o[8];
      if (kF32) {
        const float4* p = (const float4*)((const float*)out + srow[r] * d + c);
        const float4 a = p[0], b = p[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
      } else {
        const uint4 u = *(const uint4*)((const uint16_t*)out + srow[r] * d + c);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = bf16_to_f32((uint16_t)(wd[i] & 0xffff));
          o[2 * i + 1] = bf16_to_f32((uint16_t)(wd[i] >> 16));
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, o[i], acc[i]);
    }
    if (has_shared) {
      float o[8];
      if (kF32) {
        const float4* p = (const float4*)((const float*)out + shared_row * d + c);
        const float4 a = p[0], b = p[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
      } else {
        const uint4 u = *(const uint4*)((const uint16_t*)out + shared_row * d + c);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = bf16_to_f32((uint16_t)(wd[i] & 0xffff));
          o[2 * i + 1] = bf16_to_f32((uint16_t)(wd[i] >> 16));
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = acc[i] + o[i];
    }
    if (kF32) {
      float4* q = (float4*)((float*)y + (size_t)t * d + c);
      q[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      q[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      uint4 u;
      u.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      u.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      u.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
      u.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
      *(uint4*)((uint16_t*)y + (size_t)t * d + c) = u;
    }
  }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const void* out, int dtype, const int32_t* row_of,
                                  const float* weights, int T, int d, int k, int has_shared, void* y,
                                  void* stream) {
  if (!valid_dtype(dtype) || T < 0 || d < 1 || k < 1 || k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!out || !row_of || !weights || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const long long rows = (long long)T * k + (has_shared ? T : 0);
  // as few passes of 8-element chunks over the row as 1024 threads allow, with every
  // thread busy in each pass (d = 7168: 896 chunks, 896 threads, one pass; 2% faster
  // than two passes of 448 threads, same bits)
  const int chunks = d / 8, passes = (chunks + 1023) / 1024;
  const int thr = ((chunks + passes - 1) / passes + 63) / 64 * 64;
  if (dtype == MOE_F32)
    combine_kernel<true><<<T, thr, 0, s>>>(out, row_of, weights, T, d, k, has_shared ? 1 : 0, rows, y);
  else
    combine_kernel<false><<<T, thr, 0, s>>>(out, row_of, weights, T, d, k, has_shared ? 1 : 0, rows, y);
  return launch_status();
}
