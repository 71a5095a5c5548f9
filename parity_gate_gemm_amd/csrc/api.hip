// Library-wide entry points: workspace sizing and initialisation, the device error
// flag check, status strings.
#include "moe_internal.h"

namespace moe {

__global__ void clear_header_kernel(int* hdr, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) hdr[i] = 0;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_workspace_size(int T, int d, int E, int k, int inter, int dtype,
                                         size_t* bytes) {
  if (!bytes || T < 0 || d < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxTopK ||
      inter < 1 || !valid_layer_dtype(dtype))
    return MOE_ERR_INVALID_ARG;
  *bytes = workspace_bytes(T, d, E, k, inter, dtype);
  return MOE_OK;
}

extern "C" moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < kHeaderBytes) return MOE_ERR_INVALID_ARG;
  clear_header_kernel<<<1, 64, 0, (hipStream_t)stream>>>((int*)ws, (int)(kHeaderBytes / sizeof(int)));
  return launch_status();
}

extern "C" moe_status moe_check(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < kHeaderBytes) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  int flag = 0;
  if (hipMemcpy(&flag, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  clear_header_kernel<<<1, 64, 0, s>>>((int*)ws, 1);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  if (flag & (kFlagBadId | kFlagDupId)) return MOE_ERR_BAD_IDS;
  if (flag & kFlagNonFinite) return MOE_ERR_NONFINITE;
  if (flag & kFlagCorrupt) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_BAD_IDS: return "MOE_ERR_BAD_IDS: expert id out of range or repeated in a row";
    case MOE_ERR_NONFINITE: return "MOE_ERR_NONFINITE: non-finite gate logit";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    default: return "unknown moe_status";
  }
}
