// Packer, repacker and dequantiser for int4 block-32 symmetric weights.
//
// Ternary rule ("vibevoice-asr-bitnet-onnx" page, ternarisation paragraph): s = 1/mean(|W|),
// W' = round(clamp(W*s, -1, 1))/s; MatMulNBits note: q = w/s + 8 in {7,8,9}, block 32, the
// block scale is the ternary scale.  Here the stored scale is fp16(mean|W|) = fp16(1/s) and
// t = round(clamp(W/m, -1, 1)) is evaluated exactly as sign(W) * [|W| > m/2].
//
// mean|W| is made independent of summation order: |W| values are binned by fp32 exponent with
// 64-bit integer adds of their 24-bit significands (integer atomics commute), the bins are
// combined into one exact multi-word integer, which is rounded once to fp64.
#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kBins = 256;

// fp64 -> fp16 bits, one round-to-nearest-even step (IEEE 754 binary16, subnormals included).
__device__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return sign | 0x7e00u;   // NaN
  if (a == 0x7ff0000000000000ull) return sign | 0x7c00u;  // inf
  const int e = (int)(a >> 52);
  if (e == 0) return sign;                                // |x| < 2^-1022
  const uint64_t mant = (a & 0xfffffffffffffull) | (1ull << 52);
  const int E = e - 1008;                                 // fp16 biased exponent if normal
  const int shift = E >= 1 ? 42 : 42 + (1 - E);
  if (shift >= 64) return sign;                           // below half the smallest subnormal
  uint64_t r = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (r & 1))) ++r;
  uint64_t bits;
  if (E >= 1) {
    bits = ((uint64_t)(E - 1) << 10) + r;   // r in [1024, 2048]: a carry bumps the exponent
    if (bits >= 0x7c00u) bits = 0x7c00u;
  } else {
    bits = r;                               // subnormal (1024 = smallest normal after rounding)
  }
  return (uint16_t)(sign | bits);
}

__global__ __launch_bounds__(256) void k_abs_bins(const float* __restrict__ W, size_t n,
                                                  unsigned long long* __restrict__ bins) {
  __shared__ unsigned long long sb[kBins];
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) sb[i] = 0;
  __syncthreads();
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  auto add = [&](float v) {
    const uint32_t bits = __float_as_uint(v) & 0x7fffffffu;
    uint32_t e = bits >> 23;
    if (e > 254) e = 254;  // non-finite input: unspecified result (documented), keep in range
    const uint32_t m = (bits & 0x7fffffu) | (e ? 0x800000u : 0u);
    if (m) atomicAdd(&sb[e], (unsigned long long)m);
  };
  const size_t n4 = n / 4;
  const float4* W4 = reinterpret_cast<const float4*>(W);
  const bool aligned = (reinterpret_cast<uintptr_t>(W) & 15) == 0;
  if (aligned) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
      const float4 v = W4[i];
      add(v.x); add(v.y); add(v.z); add(v.w);
    }
    for (size_t i = n4 * 4 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) add(W[i]);
  } else {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) add(W[i]);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += blockDim.x)
    if (sb[i]) atomicAdd(&bins[i], sb[i]);
}

// bins[e] = sum of the significands (implicit bit included) of |w| with exponent field e; the
// value of one element is sig * 2^(max(e,1) - 150).  Writes m = (exact sum rounded to fp64) / n
// and fp16(m).
__global__ void k_mean_finalize(const unsigned long long* __restrict__ bins, unsigned long long n,
                                double* __restrict__ m_out, uint16_t* __restrict__ s16_out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  uint64_t limb[12];
  for (int i = 0; i < 12; ++i) limb[i] = 0;
  for (int e = 0; e < 255; ++e) {
    const uint64_t v = bins[e];
    if (!v) continue;
    const int sh = (e > 0 ? e : 1) - 1;  // integer in units of 2^-149
    const int li = sh >> 5, bi = sh & 31;
    const uint64_t lo = v << bi;
    const uint64_t hi = bi ? (v >> (64 - bi)) : 0;
    limb[li] += lo & 0xffffffffull;
    limb[li + 1] += lo >> 32;
    limb[li + 2] += hi;
  }
  for (int i = 0; i < 11; ++i) {
    limb[i + 1] += limb[i] >> 32;
    limb[i] &= 0xffffffffull;
  }
  int top = -1;
  for (int i = 11; i >= 0 && top < 0; --i)
    for (int k = 31; k >= 0; --k)
      if ((limb[i] >> k) & 1) { top = 32 * i + k; break; }
  double S = 0.0;
  if (top >= 0) {
    auto bit = [&](int k) -> uint64_t { return k < 0 ? 0 : (limb[k >> 5] >> (k & 31)) & 1; };
    if (top <= 52) {
      uint64_t v = 0;
      for (int k = top; k >= 0; --k) v = (v << 1) | bit(k);
      S = ldexp((double)v, -149);
    } else {
      uint64_t mant = 0;
      for (int k = top; k >= top - 52; --k) mant = (mant << 1) | bit(k);
      const uint64_t rnd = bit(top - 53);
      uint64_t sticky = 0;
      for (int k = top - 54; k >= 0 && !sticky; --k) sticky |= bit(k);
      int ex = top - 52;
      if (rnd && (sticky || (mant & 1))) {
        ++mant;
        if (mant == (1ull << 53)) { mant >>= 1; ++ex; }
      }
      S = ldexp((double)mant, ex - 149);
    }
  }
  const double m = n ? S / (double)n : 0.0;
  *m_out = m;
  *s16_out = f64_to_f16_rne(m);
}

// Destination placement: source row r goes to destination row
//   (r / row_group) * group_stride + row_offset + r % row_group
// (tiled layout: tile = row / 64, lane = row % 64).
struct Dst {
  int layout;
  int64_t row_group, group_stride, row_offset;
  int nb, ng;
};

__device__ __forceinline__ int64_t dst_row(const Dst& D, int64_t r) {
  return (r / D.row_group) * D.group_stride + D.row_offset + (r % D.row_group);
}

// 32 codes (low nibble of each byte of c[]) -> 4 dwords in the destination layout
__device__ __forceinline__ uint4 encode_block(const uint8_t* c, int layout) {
  uint32_t d[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t v = 0;
    if (layout == VV_LAYOUT_ROWMAJOR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v |= (uint32_t)c[8 * w + j] << (4 * j);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v |= (uint32_t)c[8 * w + 2 * i] << (4 * i);
        v |= (uint32_t)c[8 * w + 2 * i + 1] << (16 + 4 * i);
      }
    }
    d[w] = v;
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

__device__ __forceinline__ void decode_block(uint4 q, int layout, uint8_t* c) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (layout == VV_LAYOUT_ROWMAJOR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) c[8 * w + j] = (d[w] >> (4 * j)) & 15;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[8 * w + 2 * i] = (d[w] >> (4 * i)) & 15;
        c[8 * w + 2 * i + 1] = (d[w] >> (16 + 4 * i)) & 15;
      }
    }
  }
}

__device__ __forceinline__ size_t nib_index(const Dst& D, int64_t r, int b, int64_t nrows) {
  if (D.layout == VV_LAYOUT_ROWMAJOR) return (size_t)(r * D.nb + b);  // in 16-B units
  const int64_t d = dst_row(D, r);
  return (size_t)(((d / kTileRows) * D.nb + b) * kTileRows + (d % kTileRows));
}
__device__ __forceinline__ size_t scale_index(const Dst& D, int64_t r, int b) {
  if (D.layout == VV_LAYOUT_ROWMAJOR) return (size_t)(r * D.nb + b);
  const int64_t d = dst_row(D, r);
  return (size_t)((((d / kTileRows) * D.ng + b / 8) * kTileRows + (d % kTileRows)) * 8 + (b % 8));
}

// One thread per (row, block-slot).  For the tiled layout, rows run to the end of the last row
// group (padding rows get code 8 and scale 0) and block slots to ng*8 (scale padding 0).
template <int MODE>
__global__ __launch_bounds__(256) void k_quant(const float* __restrict__ W, int64_t N, int K, int64_t nrows,
                                               int nslots, Dst D, const double* __restrict__ mptr,
                                               const uint16_t* __restrict__ s16ptr,
                                               uint4* __restrict__ out, uint16_t* __restrict__ sout) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= nrows * nslots) return;
  const int64_t r = idx / nslots;
  const int b = (int)(idx % nslots);
  if (b >= D.nb) {  // scale padding of the last group (tiled only)
    sout[scale_index(D, r, b)] = 0;
    return;
  }
  uint8_t c[32];
  uint16_t sc = 0;
  if (r >= N) {
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = 8;
  } else {
    const float4* src = reinterpret_cast<const float4*>(W + r * (int64_t)K + (int64_t)b * kBlock);
    float w[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = src[j];
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
    if (MODE == VV_Q_TERNARY) {
      const double half_m = 0.5 * (*mptr);
      sc = *s16ptr;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const double a = fabs((double)w[j]);
        c[j] = a > half_m ? (w[j] > 0.f ? 9 : 7) : 8;
      }
    } else {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(w[j]));
      sc = f64_to_f16_rne((double)amax / 7.0);
      const double s = (double)h2f(sc);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (s == 0.0) { c[j] = 8; continue; }
        double q = rint((double)w[j] / s) + 8.0;
        if (!(q == q)) q = 8.0;
        q = q < 0.0 ? 0.0 : (q > 15.0 ? 15.0 : q);
        c[j] = (uint8_t)q;
      }
    }
  }
  out[nib_index(D, r, b, nrows)] = encode_block(c, D.layout);
  sout[scale_index(D, r, b)] = sc;
}

__global__ __launch_bounds__(256) void k_repack(const uint4* __restrict__ in, const uint16_t* __restrict__ sin,
                                                int64_t N, int64_t nrows, int nslots, Dst D,
                                                uint4* __restrict__ out, uint16_t* __restrict__ sout) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= nrows * nslots) return;
  const int64_t r = idx / nslots;
  const int b = (int)(idx % nslots);
  if (b >= D.nb) {
    sout[scale_index(D, r, b)] = 0;
    return;
  }
  uint8_t c[32];
  uint16_t sc = 0;
  if (r < N) {
    decode_block(in[r * D.nb + b], VV_LAYOUT_ROWMAJOR, c);
    sc = sin[r * D.nb + b];
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = 8;
  }
  out[nib_index(D, r, b, nrows)] = encode_block(c, VV_LAYOUT_TILED);
  sout[scale_index(D, r, b)] = sc;
}

__global__ __launch_bounds__(256) void k_dequant(const uint4* __restrict__ in, const uint16_t* __restrict__ sin,
                                                 int64_t N, Dst D, float* __restrict__ W) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= N * D.nb) return;
  const int64_t r = idx / D.nb;
  const int b = (int)(idx % D.nb);
  uint8_t c[32];
  decode_block(in[nib_index(D, r, b, N)], D.layout, c);
  const float s = h2f(sin[scale_index(D, r, b)]);
  float4* dst = reinterpret_cast<float4*>(W + r * (int64_t)D.nb * kBlock + (int64_t)b * kBlock);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    dst[j] = make_float4((float)((int)c[4 * j] - 8) * s, (float)((int)c[4 * j + 1] - 8) * s,
                         (float)((int)c[4 * j + 2] - 8) * s, (float)((int)c[4 * j + 3] - 8) * s);
}

int check_common(const void* W, int64_t N, int64_t K, const char* fn) {
  VV_REQUIRE(W != nullptr, VV_ERR_NULL, "%s: input pointer is NULL", fn);
  VV_REQUIRE(N >= 1, VV_ERR_RANGE, "%s: N = %lld < 1", fn, (long long)N);
  VV_REQUIRE(K >= kBlock && K % kBlock == 0, VV_ERR_SHAPE, "%s: K = %lld is not a positive multiple of 32", fn,
             (long long)K);
  VV_REQUIRE(K <= (1 << 24), VV_ERR_RANGE, "%s: K = %lld too large", fn, (long long)K);
  return VV_OK;
}

int check_place(int64_t N, int64_t row_group, int64_t group_stride, int64_t row_offset, int64_t dst_rows,
                const char* fn) {
  VV_REQUIRE(row_group >= 1 && group_stride >= row_group && row_offset >= 0, VV_ERR_RANGE,
             "%s: need row_group >= 1, group_stride >= row_group, row_offset >= 0", fn);
  VV_REQUIRE(dst_rows >= 1 && dst_rows % kTileRows == 0, VV_ERR_RANGE, "%s: dst_rows must be a positive multiple of 64",
             fn);
  const int64_t last = (cdiv(N, row_group) - 1) * group_stride + row_offset + row_group - 1;
  VV_REQUIRE(last < dst_rows, VV_ERR_RANGE, "%s: source rows reach destination row %lld >= dst_rows %lld", fn,
             (long long)last, (long long)dst_rows);
  return VV_OK;
}

int pack_impl(const float* W, int64_t N, int64_t K, int mode, Dst D, uint8_t* packed, uint16_t* scales,
              void* ws, size_t ws_bytes, hipStream_t st, const char* fn) {
  int rc = check_common(W, N, K, fn);
  if (rc) return rc;
  VV_REQUIRE(packed && scales, VV_ERR_NULL, "%s: output pointer is NULL", fn);
  VV_REQUIRE(mode == VV_Q_TERNARY || mode == VV_Q_ABSMAX, VV_ERR_DTYPE, "%s: unknown mode %d", fn, mode);
  VV_REQUIRE((reinterpret_cast<uintptr_t>(W) & 15) == 0 && (reinterpret_cast<uintptr_t>(packed) & 15) == 0,
             VV_ERR_RANGE, "%s: W and packed must be 16-byte aligned", fn);
  const size_t need = vv_pack_int4_workspace(N, K, mode);
  if (need) VV_REQUIRE(ws && ws_bytes >= need, VV_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  const int64_t nrows = D.layout == VV_LAYOUT_TILED ? cdiv(N, D.row_group) * D.row_group : N;
  const int nslots = D.layout == VV_LAYOUT_TILED ? D.ng * 8 : D.nb;
  const int64_t total = nrows * nslots;
  const int grid = (int)cdiv(total, 256);
  if (mode == VV_Q_TERNARY) {
    auto* bins = reinterpret_cast<unsigned long long*>(ws);
    auto* mptr = reinterpret_cast<double*>(static_cast<char*>(ws) + kBins * 8);
    auto* s16 = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + kBins * 8 + 8);
    VV_HIP(fill_zero(ws, kBins * 8 + 16, st));
    const size_t n = (size_t)N * (size_t)K;
    const int g = (int)std::min<int64_t>(2048, cdiv((int64_t)n, 256 * 16));
    hipLaunchKernelGGL(k_abs_bins, dim3(g < 1 ? 1 : g), dim3(256), 0, st, W, n, bins);
    VV_HIP(hipGetLastError());
    hipLaunchKernelGGL(k_mean_finalize, dim3(1), dim3(64), 0, st, bins, (unsigned long long)n, mptr, s16);
    VV_HIP(hipGetLastError());
    hipLaunchKernelGGL(k_quant<VV_Q_TERNARY>, dim3(grid), dim3(256), 0, st, W, N, (int)K, nrows, nslots, D,
                       (const double*)mptr, (const uint16_t*)s16, reinterpret_cast<uint4*>(packed), scales);
  } else {
    hipLaunchKernelGGL(k_quant<VV_Q_ABSMAX>, dim3(grid), dim3(256), 0, st, W, N, (int)K, nrows, nslots, D,
                       (const double*)nullptr, (const uint16_t*)nullptr, reinterpret_cast<uint4*>(packed), scales);
  }
  VV_HIP(hipGetLastError());
  return VV_OK;
}

}  // namespace
}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_pack_int4_workspace(int64_t N, int64_t K, int mode) {
  (void)N; (void)K;
  return mode == VV_Q_TERNARY ? 4096 : 0;
}

int vv_pack_int4(const float* W, int64_t N, int64_t K, int mode, uint8_t* packed, uint16_t* scales, void* ws,
                 size_t ws_bytes, void* stream) {
  clear_error();
  Dst D{VV_LAYOUT_ROWMAJOR, N, N, 0, (int)(K / kBlock), (int)cdiv(K / kBlock, 8)};
  return pack_impl(W, N, K, mode, D, packed, scales, ws, ws_bytes, as_stream(stream), "vv_pack_int4");
}

int vv_pack_int4_tiled(const float* W, int64_t N, int64_t K, int mode, int64_t row_group, int64_t group_stride,
                       int64_t row_offset, int64_t dst_rows, uint8_t* packed, uint16_t* scales, void* ws,
                       size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(W, N, K, "vv_pack_int4_tiled");
  if (rc) return rc;
  rc = check_place(N, row_group, group_stride, row_offset, dst_rows, "vv_pack_int4_tiled");
  if (rc) return rc;
  Dst D{VV_LAYOUT_TILED, row_group, group_stride, row_offset, (int)(K / kBlock), (int)cdiv(K / kBlock, 8)};
  return pack_impl(W, N, K, mode, D, packed, scales, ws, ws_bytes, as_stream(stream), "vv_pack_int4_tiled");
}

int vv_repack_int4_tiled(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t row_group,
                         int64_t group_stride, int64_t row_offset, int64_t dst_rows, uint8_t* tiled,
                         uint16_t* tiled_scales, void* stream) {
  clear_error();
  int rc = check_common(packed, N, K, "vv_repack_int4_tiled");
  if (rc) return rc;
  VV_REQUIRE(scales && tiled && tiled_scales, VV_ERR_NULL, "vv_repack_int4_tiled: NULL pointer");
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(tiled)) & 15) == 0,
             VV_ERR_RANGE, "vv_repack_int4_tiled: packed buffers must be 16-byte aligned");
  rc = check_place(N, row_group, group_stride, row_offset, dst_rows, "vv_repack_int4_tiled");
  if (rc) return rc;
  Dst D{VV_LAYOUT_TILED, row_group, group_stride, row_offset, (int)(K / kBlock), (int)cdiv(K / kBlock, 8)};
  const int64_t nrows = cdiv(N, row_group) * row_group;
  const int nslots = D.ng * 8;
  hipLaunchKernelGGL(k_repack, dim3((unsigned)cdiv(nrows * nslots, 256)), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const uint4*>(packed), scales, N, nrows, nslots, D,
                     reinterpret_cast<uint4*>(tiled), tiled_scales);
  VV_HIP(hipGetLastError());
  return VV_OK;
}

int vv_dequant_int4(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int layout, float* W,
                    void* stream) {
  clear_error();
  int rc = check_common(packed, N, K, "vv_dequant_int4");
  if (rc) return rc;
  VV_REQUIRE(scales && W, VV_ERR_NULL, "vv_dequant_int4: NULL pointer");
  VV_REQUIRE(layout == VV_LAYOUT_ROWMAJOR || layout == VV_LAYOUT_TILED, VV_ERR_DTYPE,
             "vv_dequant_int4: unknown layout %d", layout);
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(W)) & 15) == 0, VV_ERR_RANGE,
             "vv_dequant_int4: packed and W must be 16-byte aligned");
  Dst D{layout, kTileRows, kTileRows, 0, (int)(K / kBlock), (int)cdiv(K / kBlock, 8)};
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)cdiv(N * D.nb, 256)), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const uint4*>(packed), scales, N, D, W);
  VV_HIP(hipGetLastError());
  return VV_OK;
}

}  // extern "C"
