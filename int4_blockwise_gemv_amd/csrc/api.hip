// Status codes, error text, workspace fill, layout sizes.
#include <stdarg.h>
#include <stdio.h>
#include <algorithm>

#include "vv_internal.h"

namespace vv {

static thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof g_err, "%s failed: %s", what, hipGetErrorString(e));
  return VV_ERR_HIP;
}

void clear_error() { g_err[0] = 0; }

__global__ void k_fill_zero(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail, size_t ntail) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t st, KEv ev) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  int grid = (int)std::min<size_t>(4096, (n16 + 255) / 256);
  if (grid < 1) grid = 1;
  VV_LAUNCH(k_fill_zero, dim3(grid), dim3(256), st, ev, (uint4*)p, n16, (uint8_t*)p + n16 * 16, ntail);
  return hipGetLastError();
}

// Streaming read of a buffer (a measuring stick for the HBM-bound kernels): workgroup w reads the
// 32 KiB pieces w, w + grid, ... with eight 16-byte loads per thread in flight (each load
// instruction of the workgroup covers 4 KiB contiguous) and folds them into an XOR that is stored
// only on a value practically never met, so the loads are kept and the writes cost nothing.
constexpr size_t kStreamPiece = 32768;
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, size_t npieces,
                                                     uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (size_t pc = blockIdx.x; pc < npieces; pc += gridDim.x) {
    const u32x4* b = p + pc * (kStreamPiece / 16) + threadIdx.x;
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(b + j * 256);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace vv

using namespace vv;

extern "C" {

const char* vv_status_string(int s) {
  switch (s) {
    case VV_OK: return "ok";
    case VV_ERR_NULL: return "null pointer";
    case VV_ERR_SHAPE: return "unsupported shape";
    case VV_ERR_RANGE: return "value out of range";
    case VV_ERR_DTYPE: return "unknown dtype, mode or layout";
    case VV_ERR_WORKSPACE: return "workspace missing or too small";
    case VV_ERR_UNSUPPORTED: return "unsupported combination";
    case VV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* vv_last_error(void) { return g_err; }

int vv_version(void) { return 100; }

int vv_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (ws_bytes == 0) return VV_OK;
  VV_REQUIRE(ws != nullptr, VV_ERR_NULL, "vv_workspace_init: ws is NULL");
  VV_HIP(fill_zero(ws, ws_bytes, as_stream(stream)));
  return VV_OK;
}

int vv_stream_read(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  clear_error();
  VV_REQUIRE(p && sink, VV_ERR_NULL, "vv_stream_read: NULL pointer");
  VV_REQUIRE(bytes > 0 && bytes % kStreamPiece == 0, VV_ERR_RANGE,
             "vv_stream_read: bytes = %zu is not a positive multiple of 32768", bytes);
  VV_REQUIRE((reinterpret_cast<uintptr_t>(p) & 15) == 0, VV_ERR_RANGE, "vv_stream_read: p must be 16-byte aligned");
  const size_t np = bytes / kStreamPiece;
  const int grid = (int)std::min<size_t>(np, 2048);
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, as_stream(stream), reinterpret_cast<const u32x4*>(p), np,
                     sink);
  VV_HIP(hipGetLastError());
  return VV_OK;
}

size_t vv_packed_bytes(int64_t rows, int64_t K, int layout) {
  if (rows < 1 || K < kBlock || K % kBlock) return 0;
  const int64_t nb = K / kBlock;
  if (layout == VV_LAYOUT_ROWMAJOR) return (size_t)(rows * nb * 16);
  if (layout == VV_LAYOUT_TILED) return (size_t)(cdiv(rows, kTileRows) * nb * kTileRows * 16);
  return 0;
}

size_t vv_scale_bytes(int64_t rows, int64_t K, int layout) {
  if (rows < 1 || K < kBlock || K % kBlock) return 0;
  const int64_t nb = K / kBlock;
  if (layout == VV_LAYOUT_ROWMAJOR) return (size_t)(rows * nb * 2);
  if (layout == VV_LAYOUT_TILED) return (size_t)(cdiv(rows, kTileRows) * cdiv(nb, 8) * kTileRows * 16);
  return 0;
}

}  // extern "C"
