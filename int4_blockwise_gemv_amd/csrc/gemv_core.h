// Device arithmetic of the int4 block-32 dot product, shared by the GEMV kernels and the prefill
// GEMM (MatMulNBits block layout, "vibevoice-asr-bitnet-onnx" page, quantisation section: code
// q = t + 8 in a nibble, one fp16 scale per 32-element block).
#pragma once

#include "vv_internal.h"

namespace vv {

// A VGPR holding a constant, opaque to the optimiser: lets (d & mask) | magic become one
// v_and_or_b32 (mask in an SGPR, magic in a VGPR; the GFX9 VOP3 encoding takes no literal).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

__device__ __forceinline__ float dot8_pairs(uint32_t d, const uint32_t* x4, float acc, uint32_t m64) {
  // the fp16 magic 64.0 (0x5400) has ulp 1/16, so a code in mantissa bits 4..7 of either half
  // reads as 64 + q exactly; the even/odd codes of pair i sit in nibbles i and 4+i
  const uint32_t p01 = ((d << 4) & 0x00F000F0u) | m64;  // nibbles 0, 4: (64+e0, 64+e1)
  const uint32_t p23 = (d & 0x00F000F0u) | m64;         // nibbles 1, 5: (64+e2, 64+e3)
  const uint32_t p45 = ((d >> 4) & 0x00F000F0u) | m64;  // nibbles 2, 6: (64+e4, 64+e5)
  const uint32_t p67 = ((d >> 8) & 0x00F000F0u) | m64;  // nibbles 3, 7: (64+e6, 64+e7)
  acc = __builtin_amdgcn_fdot2(as_h2(p01), as_h2(x4[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p23), as_h2(x4[1]), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p45), as_h2(x4[2]), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p67), as_h2(x4[3]), acc, false);
  return acc;
}

// the same over activations given as two fp16 parts x = hi + lo (about 22 significant bits, so
// the activation keeps fp32 precision).  Here the code pairs are made exact first, 64 + q - 72 =
// q - 8 by one packed fp16 add (small integers, so exact): the fp32 sums then carry no offset to
// cancel.  (Accumulating 64 + q and removing 72 sum(x) per block leaves partial sums about 15
// times the block's result, and with them an fp32 rounding error of about 2e-6 of the output,
// the precision the lo part is there to keep.)  Each pair meets both parts.
__device__ __forceinline__ float dot8_exact_hl(uint32_t d, const uint32_t* xh4, const uint32_t* xl4, float acc,
                                               uint32_t m64) {
  const h2_t off = as_h2(0xD480D480u);       // (-72, -72)
  const h2_t p01 = as_h2(((d << 4) & 0x00F000F0u) | m64) + off;
  const h2_t p23 = as_h2((d & 0x00F000F0u) | m64) + off;
  const h2_t p45 = as_h2(((d >> 4) & 0x00F000F0u) | m64) + off;
  const h2_t p67 = as_h2(((d >> 8) & 0x00F000F0u) | m64) + off;
  acc = __builtin_amdgcn_fdot2(p01, as_h2(xh4[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(p23, as_h2(xh4[1]), acc, false);
  acc = __builtin_amdgcn_fdot2(p45, as_h2(xh4[2]), acc, false);
  acc = __builtin_amdgcn_fdot2(p67, as_h2(xh4[3]), acc, false);
  acc = __builtin_amdgcn_fdot2(p01, as_h2(xl4[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(p23, as_h2(xl4[1]), acc, false);
  acc = __builtin_amdgcn_fdot2(p45, as_h2(xl4[2]), acc, false);
  acc = __builtin_amdgcn_fdot2(p67, as_h2(xl4[3]), acc, false);
  return acc;
}

// four fp32 activations -> their fp16 hi parts (two pairs) and lo parts x - hi (two pairs)
__device__ __forceinline__ void split_hl4(float a, float b, float c, float d, uint2& hi, uint2& lo) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b, hc = (_Float16)c, hd = (_Float16)d;
  const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
  const _Float16 lc = (_Float16)(c - (float)hc), ld = (_Float16)(d - (float)hd);
  hi.x = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
  hi.y = (uint32_t)__builtin_bit_cast(uint16_t, hc) | ((uint32_t)__builtin_bit_cast(uint16_t, hd) << 16);
  lo.x = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
  lo.y = (uint32_t)__builtin_bit_cast(uint16_t, lc) | ((uint32_t)__builtin_bit_cast(uint16_t, ld) << 16);
}

// C for one quarter (8 elements) of a block: (64 + 8) * (x0 + ... + x7)
__device__ __forceinline__ float corr_quarter(u32x4 xv) {
  const uint32_t c72 = 0x54805480u;  // fp16 (72, 72)
  float c = __builtin_amdgcn_fdot2(as_h2(xv.x), as_h2(c72), 0.f, false);
  c = __builtin_amdgcn_fdot2(as_h2(xv.y), as_h2(c72), c, false);
  c = __builtin_amdgcn_fdot2(as_h2(xv.z), as_h2(c72), c, false);
  c = __builtin_amdgcn_fdot2(as_h2(xv.w), as_h2(c72), c, false);
  return c;
}

// scale j (compile-time 0..7) of a group of 8 fp16 scales
__device__ __forceinline__ float pick_scale(const u32x4& s, int j) {
  const uint32_t d = (j >> 1) == 0 ? s.x : (j >> 1) == 1 ? s.y : (j >> 1) == 2 ? s.z : s.w;
  return (j & 1) ? (float)__builtin_bit_cast(h2_t, d).y : (float)__builtin_bit_cast(h2_t, d).x;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---- split-K hand-off without atomics (the VALU GEMV) ---------------------------------------------
// A writer stores its partial as a 64-bit (tag, fp32 bits) word into its slot and exits; the reader
// polls the slots, adds them in a fixed order and clears them.
constexpr uint64_t kFresh = 1ull << 32;     // tag of a filled hand-off slot (cleared slots are 0)
constexpr uint32_t kSpinLimit = 1u << 22;   // polls before a wait gives up (seconds)

// Sum of the n tagged fp32 values at p[k * stride], k in order, once every tag is set; then clears
// the slots.  Polls kPollBatch slots at a time (every lane of the wave takes part in the vote):
// 10 covers the 9 writers of the 7B down projection in one round trip and still fits in the
// registers the weight stream needs (a batch of 16 costs the M <= 2 kernels two waves per SIMD).
constexpr int kPollBatch = 10;
__device__ __forceinline__ float poll_sum(uint64_t* p, int n, size_t stride, int32_t* status) {
  float s = 0.f;
  for (int k0 = 0; k0 < n; k0 += kPollBatch) {
    uint64_t v[kPollBatch];
    for (uint32_t it = 0;; ++it) {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < kPollBatch; ++k) {
        v[k] = collect_u64(p + (size_t)min(k0 + k, n - 1) * stride);
        ok = ok && (v[k] >> 32) == 1u;
      }
      if (__all(ok)) break;
      if (it >= kSpinLimit) {
        if (status) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return __builtin_nanf("");
      }
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int k = 0; k < kPollBatch; ++k)
      if (k0 + k < n) {
        s += __uint_as_float((uint32_t)v[k]);
        publish_u64(p + (size_t)(k0 + k) * stride, 0);
      }
  }
  return s;
}

// Role of this workgroup in a split-K decomposition of ntiles tiles into wpt K-chunks: XCD x =
// wg % 8 takes tiles [x tpx, (x + 1) tpx) and runs, in dispatch order, their (wpt - 1) writers
// (tile-major) and then their readers (kg = wpt - 1).  A reader waits only for writers dispatched
// before it on its own XCD.  Needs a grid of 8 tpx wpt workgroups; returns false for padding.
// bid: the workgroup's index in that grid (blockIdx.x less a multiple of 8 of leading workgroups
// with another role, so that bid % 8 is still the XCD).
__device__ __forceinline__ bool split_role(int ntiles, int wpt, int& tile, int& kg, int bid) {
  const int x = bid % kNumXcd, i = bid / kNumXcd;
  const int tpx = (ntiles + kNumXcd - 1) / kNumXcd;
  const int nwr = tpx * (wpt - 1);
  if (i < nwr) {
    tile = x * tpx + i / (wpt - 1);
    kg = i % (wpt - 1);
  } else {
    tile = x * tpx + (i - nwr);
    kg = wpt - 1;
  }
  return tile < ntiles && i < tpx * wpt;
}

// ---- matrix-core operands (v_mfma_f32_16x16x32_f16) of the tiled layout --------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// A 16-byte block load of a wave gives lane r the 32 codes of row r of a 64-row tile, as 4 dwords
// of 8 codes.  The 4 x 4 transpose of (dword, 16-lane group) below moves dword s of row 16 g + i
// to lane 16 s + i of t[g]: t[g] is then the MFMA operand "8 consecutive k of row 16 g + lane % 16,
// k-slice lane / 16" for row group g.
__device__ __forceinline__ void block_to_operands(const u32x4& v, uint32_t (&t)[4]) {
  uint32_t t0 = v.x, t1 = v.y, t2 = v.z, t3 = v.w;
  swap32(t0, t2);
  swap32(t1, t3);
  swap16(t0, t1);
  swap16(t2, t3);
  t[0] = t0; t[1] = t1; t[2] = t2; t[3] = t3;
}

// 8 codes of one dword (even elements in nibbles 0..3, odd in 4..7) -> 8 fp16 (q - 8), k order:
// the nibble goes into the mantissa of fp16 64.0 (ulp 1/16, so the value reads 64 + q) and one
// packed fp16 add subtracts 72, exactly
__device__ __forceinline__ half8 codes_to_half8(uint32_t d, uint32_t m64) {
  const h2_t off = as_h2(0xD480D480u);       // (-72, -72)
  const h2_t p0 = as_h2(((d << 4) & 0x00F000F0u) | m64) + off;
  const h2_t p1 = as_h2((d & 0x00F000F0u) | m64) + off;
  const h2_t p2 = as_h2(((d >> 4) & 0x00F000F0u) | m64) + off;
  const h2_t p3 = as_h2(((d >> 8) & 0x00F000F0u) | m64) + off;
  return half8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

}  // namespace vv
