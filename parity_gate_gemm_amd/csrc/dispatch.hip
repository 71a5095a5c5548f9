// Dispatch: counting sort of the (token, slot) pairs into contiguous per-expert
// segments, the input order of the grouped GEMM (Composer 2 Technical Report,
// section 6.1: Figure 10's grouped GEMM over expert groups, and the token
// dispatch/combine paragraph).  Sort key (expert ascending, token ascending, slot
// ascending).  Positions come from per-block histograms and prefix sums; integer LDS
// atomics only count, so the result is the same bits whatever the schedule.
#include <mutex>

#include "moe_internal.h"

namespace moe {

// Block b owns tokens [b*64, b*64+64): count its pairs per expert.
__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ ids, int T,
                                                            int E, int k, int* __restrict__ hist,
                                                            int* flag) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const long long p0 = (long long)blockIdx.x * kDispatchTokens * k;
  const long long p1 = min((long long)(blockIdx.x + 1) * kDispatchTokens, (long long)T) * k;
  int bad = 0;
  for (long long p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    int e = ids[p];
    if (e < 0 || e >= E) {
      bad = 1;
      e = 0;
    }
    atomicAdd(&cnt[e], 1);
  }
  if (bad) raise_flag(flag, kFlagBadId);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One block per expert: exclusive scan of its column of the histogram over the
// blocks (in place), and the expert's total.
__global__ __launch_bounds__(256) void dispatch_colscan_kernel(int* __restrict__ hist, int nb, int E,
                                                               int* __restrict__ total) {
  __shared__ int part[256];
  const int e = blockIdx.x;
  const int per = (nb + 255) / 256;
  const int b0 = threadIdx.x * per, b1 = min(b0 + per, nb);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += hist[(size_t)b * E + e];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int c = part[i];
      part[i] = run;
      run += c;
    }
    total[e] = run;
  }
  __syncthreads();
  int run = part[threadIdx.x];
  for (int b = b0; b < b1; ++b) {
    const int c = hist[(size_t)b * E + e];
    hist[(size_t)b * E + e] = run;
    run += c;
  }
}

// offsets = exclusive scan of the expert totals (one block).
__global__ __launch_bounds__(1024) void dispatch_offsets_kernel(const int* __restrict__ total, int E,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int buf[kMaxExperts];
  const int e = threadIdx.x;
  if (e < E) buf[e] = total[e];
  __syncthreads();
  // Hillis-Steele inclusive scan over at most 1024 entries.
  for (int off = 1; off < E; off <<= 1) {
    int v = 0;
    if (e < E && e >= off) v = buf[e - off];
    __syncthreads();
    if (e < E) buf[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = buf[e];
  if (e == 0) offsets[0] = 0;
}

__global__ void zero_offsets_kernel(int E, int32_t* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = 0;
}

// Each pair's sorted row = segment start + this block's prefix for the expert + the
// number of earlier pairs (in token-major order) of this block with the same expert.
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids, int T,
                                                               int E, int k, const int* __restrict__ hist,
                                                               const int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ row_of) {
  __shared__ int sid[kDispatchTokens * kMaxTopK];
  const long long p0 = (long long)blockIdx.x * kDispatchTokens * k;
  const int np = (int)(min((long long)(blockIdx.x + 1) * kDispatchTokens, (long long)T) * k - p0);
  for (int q = threadIdx.x; q < np; q += blockDim.x) {
    int e = ids[p0 + q];
    sid[q] = (e < 0 || e >= E) ? 0 : e;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < np; q += blockDim.x) {
    const int e = sid[q];
    int rank = 0;
    for (int j = 0; j < q; ++j) rank += (sid[j] == e) ? 1 : 0;
    const int pos = offsets[e] + hist[(size_t)blockIdx.x * E + e] + rank;
    perm[pos] = (int32_t)(p0 + q);
    row_of[p0 + q] = pos;
  }
}

// Writes the device error flag of one no-allocation dispatch to the caller's status.
__global__ void dispatch_status_kernel(const int* flag, int32_t* status) {
  if (threadIdx.x == 0) *status = (*flag & (kFlagBadId | kFlagDupId)) ? MOE_ERR_BAD_IDS : MOE_OK;
}

__global__ void clear_flag_kernel(int* flag) {
  if (threadIdx.x == 0) *flag = 0;
}

// The four dispatch kernels on a scratch area laid out as dispatch_ws (header flag,
// per-block histograms, expert totals).
static void dispatch_launch(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* perm,
                            int32_t* row_of, char* w, hipStream_t s) {
  const DispatchWs L = dispatch_ws(T, E);
  int* hist = (int*)(w + L.hist);
  int* total = (int*)(w + L.total);
  if (T > 0) {
    dispatch_hist_kernel<<<L.nblocks, 256, 0, s>>>(ids, T, E, k, hist, (int*)w);
    dispatch_colscan_kernel<<<E, 256, 0, s>>>(hist, L.nblocks, E, total);
    dispatch_offsets_kernel<<<1, 1024, 0, s>>>(total, E, offsets);
    dispatch_scatter_kernel<<<L.nblocks, 256, 0, s>>>(ids, T, E, k, hist, offsets, perm, row_of);
  } else {
    // Empty batch: every segment is empty.
    zero_offsets_kernel<<<1, 1024, 0, s>>>(E, offsets);
  }
}

// Scratch of moe_dispatch_noalloc: one copy per GPU, held until the process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device (hipGetSymbolAddress once per
// device; host code never passes the symbol itself).
static char* scratch_ptr(int* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = 1;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = 1;
      return nullptr;
    }
    ptrs[dev] = p;
  }
  *err = 0;
  return (char*)ptrs[dev];
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_dispatch(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                                   int32_t* perm, int32_t* row_of, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (!offsets || !ws) return MOE_ERR_INVALID_ARG;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  const DispatchWs L = dispatch_ws(T, E);
  if (ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;
  if (T > 0 && (!ids || !perm || !row_of)) return MOE_ERR_INVALID_ARG;
  dispatch_launch(ids, T, E, k, offsets, perm, row_of, (char*)ws, (hipStream_t)stream);
  return launch_status();
}

extern "C" moe_status moe_dispatch_noalloc(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                                           int32_t* perm, int32_t* row_of, int32_t* status_out,
                                           void* stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (dispatch_ws(T, E).bytes > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!ids || !perm || !row_of)) return MOE_ERR_INVALID_ARG;
  int err = 0;
  char* w = scratch_ptr(&err);
  if (err) return MOE_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  clear_flag_kernel<<<1, 64, 0, s>>>((int*)w);   // the last call's flag stays in the array
  dispatch_launch(ids, T, E, k, offsets, perm, row_of, w, s);
  if (status_out) dispatch_status_kernel<<<1, 64, 0, s>>>((const int*)w, status_out);
  return launch_status();
}
