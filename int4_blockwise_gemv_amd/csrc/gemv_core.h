// Device arithmetic of the int4 block-32 dot product, shared by the stand-alone GEMV and the
// persistent decode-step kernel (MatMulNBits block layout, "vibevoice-asr-bitnet-onnx" page,
// quantisation section: code q = t + 8 in a nibble, one fp16 scale per 32-element block).
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

}  // namespace vv
