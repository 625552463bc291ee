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

// The 8 codes of a dword as 4 exact fp16 pairs (q - 8) in element order: pair i holds the codes
// of nibbles i and 4 + i.  Nibbles 0/4 and (after one byte shift) 2/6 sit in bits 0..3 of their
// halves, where the fp16 magic 1024.0 (ulp 1) reads them as 1024 + q; nibbles 1/5 and 3/7 sit in
// bits 4..7, where 64.0 (ulp 1/16) reads them as 64 + q.  One packed fp16 add of -1032 or -72
// then leaves q - 8 exactly (small integers).  m1024, m64: the magics in VGPRs (vconst).
__device__ __forceinline__ void code_pairs_exact(uint32_t d, uint32_t m1024, uint32_t m64, h2_t (&p)[4]) {
  const h2_t o1024 = as_h2(0xE408E408u);     // (-1032, -1032)
  const h2_t o64 = as_h2(0xD480D480u);       // (-72, -72)
  const uint32_t d8 = d >> 8;
  p[0] = as_h2((d & 0x000F000Fu) | m1024) + o1024;
  p[1] = as_h2((d & 0x00F000F0u) | m64) + o64;
  p[2] = as_h2((d8 & 0x000F000Fu) | m1024) + o1024;
  p[3] = as_h2((d8 & 0x00F000F0u) | m64) + o64;
}

// ---- fp32 activations as 8-bit digits (the vector-ALU GEMVs' fp32 input) ----------------------
// A 32-element block x_0..x_31 becomes X_i = rint(x_i 2^(22 - e)), with e the exponent of the
// block's largest magnitude (|x| < 2^e), so |X_i| <= 2^22: each element keeps 22 bits relative
// to that magnitude.  X_i is written as three signed bytes, X_i = d2 2^16 + d1 2^8 + d0 (the
// bytes of X_i + 128 (1 + 2^8 + 2^16) less 128 each).  The products with the int4 codes are then
// exact integer dot products (v_dot4_i32_i8 on the unsigned codes q), and the zero point comes off
// exactly: sum_i (q_i - 8) d_ki = sum_i q_i d_ki - 8 sum_i d_ki.  Per digit level the block sum
// is at most 32 * 15 * 128 in magnitude, and the levels combine exactly in fp32 up to one final
// rounding.
//
// LDS image of one block (kDigitDwords dwords): level k = 0, 1, 2 takes dwords 8k .. 8k + 7, where
// dword 2w holds the level-k digits of elements (0, 4, 1, 5) of word w (elements 8w .. 8w + 7)
// and dword 2w + 1 those of elements (2, 6, 3, 7), the byte orders of (codes & 0x0F0F0F0F) and
// ((codes >> 4) & 0x0F0F0F0F) for a code dword with the even elements in nibbles 0..3 and the
// odd ones in nibbles 4..7; dword 24 is the scale 2^(e - 22) as fp32 (NaN when the block holds a
// NaN or an infinity), dwords 25..27 are -8 sum_i d_ki for k = 0, 1, 2.
constexpr int kDigitDwords = 28;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// sum / max over each group of 8 lanes (every lane gets its group's result)
__device__ __forceinline__ int oct_sum(int v) {
  v += dpp_i<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);   // quad_perm [2,3,0,1]
  return v + dpp_i<0x141>(v);   // row_half_mirror: pairs the two quads of each 8 lanes
}
__device__ __forceinline__ float oct_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  return fmaxf(v, dpp_f<0x141>(v));
}

// One block's LDS image from the 8 consecutive lanes that hold it: lane r = lane % 8 holds
// elements 4r .. 4r + 3 as v and writes its three level dwords; lane 0 of the 8 writes the scale
// and the zero-point terms.  Every lane of the wave takes part (the cross-lane steps are DPP).
__device__ __forceinline__ void stage_digits(float4 v, uint32_t* blk) {
  const int r = (int)(threadIdx.x & 7);
  const float a = oct_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  // fmaxf passes over NaNs: non-finite elements are counted on their own
  constexpr float kMax = 3.40282347e38f;
  const int bad = oct_sum((fabsf(v.x) <= kMax && fabsf(v.y) <= kMax && fabsf(v.z) <= kMax && fabsf(v.w) <= kMax) ? 0 : 1);
  const int e = __builtin_amdgcn_frexp_expf(a);          // a < 2^e (0 for a = 0)
  const int sh = 22 - e;
  constexpr uint32_t kOff = 128u * (1u + 256u + 65536u);  // makes the three bytes unsigned
  const uint32_t u0 = (uint32_t)((int)__builtin_rintf(__builtin_ldexpf(v.x, sh)) + (int)kOff);
  const uint32_t u1 = (uint32_t)((int)__builtin_rintf(__builtin_ldexpf(v.y, sh)) + (int)kOff);
  const uint32_t u2 = (uint32_t)((int)__builtin_rintf(__builtin_ldexpf(v.z, sh)) + (int)kOff);
  const uint32_t u3 = (uint32_t)((int)__builtin_rintf(__builtin_ldexpf(v.w, sh)) + (int)kOff);
  // level k of the 4 elements in element order, bytes less 128 (xor 0x80)
  const uint32_t p01 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);   // (u0.b0, u1.b0, u0.b1, u1.b1)
  const uint32_t p23 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);
  const uint32_t q01 = __builtin_amdgcn_perm(u1, u0, 0x06020602u);   // (u0.b2, u1.b2, ..)
  const uint32_t q23 = __builtin_amdgcn_perm(u3, u2, 0x06020602u);
  const uint32_t L[3] = {__builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u,
                         __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u,
                         __builtin_amdgcn_perm(q23, q01, 0x05040100u) ^ 0x80808080u};
  // the pair of lanes holding word r / 2: the even lane writes elements (0, 4, 1, 5) of the word,
  // the odd one (2, 6, 3, 7); perm(other, mine): bytes 4..7 are the partner's, 0..3 this lane's
  const uint32_t sel = (r & 1) ? 0x03070206u : 0x05010400u;
  int nd[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const uint32_t other = (uint32_t)dpp_i<0xB1>((int)L[k]);
    blk[8 * k + r] = __builtin_amdgcn_perm(other, L[k], sel);
    nd[k] = -8 * oct_sum(__builtin_amdgcn_sdot4((int)L[k], 0x01010101, 0, false));
  }
  if (r == 0) {
    const float scale = bad ? __builtin_nanf("") : __builtin_ldexpf(1.0f, e - 22);
    *reinterpret_cast<u32x4*>(blk + 24) = u32x4{__float_as_uint(scale), (uint32_t)nd[0], (uint32_t)nd[1], (uint32_t)nd[2]};
  }
}

// The codes of one block (4 dwords, the tiled layout's order) split for v_dot4: lo[w] = the codes
// of elements (0, 4, 1, 5) of word w as bytes, hi[w] those of (2, 6, 3, 7)
__device__ __forceinline__ void codes_to_bytes(const uint32_t (&c)[4], uint32_t (&lo)[4], uint32_t (&hi)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    lo[w] = c[w] & 0x0F0F0F0Fu;
    hi[w] = (c[w] >> 4) & 0x0F0F0F0Fu;
  }
}

// sum_i (q_i - 8) x_i over one block for this lane's row: exact integer sums per digit level,
// combined in fp32 (one rounding) and scaled by the block's power of two
__device__ __forceinline__ float block_dot_digits(const uint32_t (&lo)[4], const uint32_t (&hi)[4],
                                                  const uint32_t* blk) {
  const u32x4 cs = *reinterpret_cast<const u32x4*>(blk + 24);
  int S[3] = {(int)cs.y, (int)cs.z, (int)cs.w};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(blk + 8 * k);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(blk + 8 * k + 4);
    int t = S[k];
    t = __builtin_amdgcn_sdot4((int)lo[0], (int)a0.x, t, false);
    t = __builtin_amdgcn_sdot4((int)hi[0], (int)a0.y, t, false);
    t = __builtin_amdgcn_sdot4((int)lo[1], (int)a0.z, t, false);
    t = __builtin_amdgcn_sdot4((int)hi[1], (int)a0.w, t, false);
    t = __builtin_amdgcn_sdot4((int)lo[2], (int)a1.x, t, false);
    t = __builtin_amdgcn_sdot4((int)hi[2], (int)a1.y, t, false);
    t = __builtin_amdgcn_sdot4((int)lo[3], (int)a1.z, t, false);
    t = __builtin_amdgcn_sdot4((int)hi[3], (int)a1.w, t, false);
    S[k] = t;
  }
  const float t = fmaf((float)S[2], 65536.f, fmaf((float)S[1], 256.f, (float)S[0]));
  return t * __uint_as_float(cs.x);
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
//
// The writers of a tile and its reader run on one XCD (split_role deals each tile's workgroups to
// one XCD; workgroup i of a launch runs on XCD i % 8), which has one L2 behind all its CUs.  So a
// slot word is written only as far as that L2 (workgroup scope: the store is not written through
// to memory, which would queue it behind the weight stream), and the reader's agent-scope loads,
// which skip the CU's own L1, find it there.  A slot word is one aligned 64-bit store, so a reader
// that sees the tag sees the value.  Kernel boundaries write the L2s back, so a slot region may be
// reused by a later launch with another tile-to-XCD deal.
constexpr uint64_t kFresh = 1ull << 32;     // tag of a filled hand-off slot (cleared slots are 0)
constexpr uint32_t kSpinLimit = 1u << 22;   // polls before a wait gives up (seconds)

__device__ __forceinline__ void slot_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

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
        slot_store(p + (size_t)(k0 + k) * stride, 0);
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

// 8 codes of one dword (even elements in nibbles 0..3, odd in 4..7) -> 8 fp16 (q - 8), k order
__device__ __forceinline__ half8 codes_to_half8(uint32_t d, uint32_t m1024, uint32_t m64) {
  h2_t p[4];
  code_pairs_exact(d, m1024, m64, p);
  return half8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

}  // namespace vv
