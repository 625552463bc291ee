// int4 block-32 GEMV straight from the MatMulNBits byte order (VV_LAYOUT_ROWMAJOR): packed
// [N][K/32][16] with element 2j of a block in the low nibble of byte j and 2j+1 in the high
// nibble, fp16 scales [N][K/32] ("vibevoice-asr-bitnet-onnx" page, MatMulNBits note: block 32,
// zero point 8, one fp16 scale per block).  This is the interchange layout; the decode step reads
// the tiled layout, which vv_repack_int4_tiled produces from these bytes.
//
// Decomposition: a wave owns kRows consecutive rows and walks K in chunks of 64 blocks, lane l
// taking block 64c + l of every row (so a row's 16-byte loads are one contiguous run and its 64
// scales one 128-byte run); the lanes' partial sums of a row meet in one wave reduction at the end.
// The workgroup stages each chunk of the activations (2048 elements per batch row) in LDS.
//
// Dequantisation without a transpose: a dword of codes holds elements e0..e7 of 8 consecutive k
// in nibbles 0..7.  Masking nibbles (0, 4), (1, 5), (2, 6), (3, 7) of the dword (and of its 4- and
// 8-bit shifts) into mantissa bits 4..7 of the two halves of fp16 64.0 gives the pairs
// (64 + e0, 64 + e4), (64 + e1, 64 + e5), (64 + e2, 64 + e6), (64 + e3, 64 + e7) with one AND-OR
// each; the activations are staged in that pair order, so v_dot2_f32_f16 multiplies them exactly.
// The offset 64 and the zero point 8 come off once per block as 72 * sum(x), and the block sum is
// scaled by the block's fp16 scale in fp32, as in the tiled kernel.
#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kRmWaves = 4;             // waves per workgroup
constexpr int kRows = 4;                // rows per wave
constexpr int kChunkBlocks = 64;        // blocks per K chunk (one per lane)
constexpr int kChunk = kChunkBlocks * kBlock;   // 2048 elements

// 8 activations x0..x7 (fp16, natural order in v) -> the pair order (x0,x4) (x1,x5) (x2,x6) (x3,x7)
__device__ __forceinline__ u32x4 pair_order(const u32x4& v) {
  // v.x = (x0, x1), v.y = (x2, x3), v.z = (x4, x5), v.w = (x6, x7) as (low, high) halves
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
  return r;
}

// sum over the 8 codes of dword d times the pair-ordered activations xp, added to acc
__device__ __forceinline__ float dot8_rowmajor(uint32_t d, const u32x4& xp, float acc, uint32_t m64) {
  const uint32_t p04 = ((d << 4) & 0x00F000F0u) | m64;
  const uint32_t p15 = (d & 0x00F000F0u) | m64;
  const uint32_t p26 = ((d >> 4) & 0x00F000F0u) | m64;
  const uint32_t p37 = ((d >> 8) & 0x00F000F0u) | m64;
  acc = __builtin_amdgcn_fdot2(as_h2(p04), as_h2(xp.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p15), as_h2(xp.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p26), as_h2(xp.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p37), as_h2(xp.w), acc, false);
  return acc;
}

template <int MT>
__global__ __launch_bounds__(64 * kRmWaves) void k_gemv_rowmajor(const u32x4* __restrict__ q,
                                                                 const uint16_t* __restrict__ s,
                                                                 const uint16_t* __restrict__ bias,
                                                                 const uint16_t* __restrict__ x, int M, int N,
                                                                 int K, void* __restrict__ y, int y_f16) {
  __shared__ __align__(16) u32x4 xs[MT][kChunk / 8];
  const int nb = K / kBlock;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = wave_id();
  const int row0 = ((int)blockIdx.x * kRmWaves + w) * kRows;
  const uint32_t m64 = vconst(0x54005400u);
  float acc[kRows][MT];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

  for (int c0 = 0; c0 < nb; c0 += kChunkBlocks) {
    // this lane's block of every row of the wave (clamped in bounds; out-of-range blocks get
    // scale 0, rows past N are computed from row N - 1 and never stored)
    const int b = min(c0 + lane, nb - 1);
    const bool bok = c0 + lane < nb;
    u32x4 wv[kRows];
    uint16_t sb[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const size_t n = (size_t)min(row0 + r, N - 1);
      wv[r] = __builtin_nontemporal_load(q + n * nb + b);
      sb[r] = s[n * nb + b];
    }
    __syncthreads();   // the previous chunk's activations are no longer read
    // stage the chunk: thread t takes elements 8t..8t+7 of every batch row (zeros past K)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      for (int t = tid; t < kChunk / 8; t += 64 * kRmWaves) {
        const int e = c0 * kBlock + 8 * t;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (e < K) v = *reinterpret_cast<const u32x4*>(x + (size_t)min(m, M - 1) * K + e);
        xs[m][t] = pair_order(v);
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      u32x4 xv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) xv[k] = xs[m][lane * 4 + k];
      // 72 * (sum of the block's 32 activations): the offset 64 and the zero point 8
      float c = 0.f;
      const uint32_t c72 = 0x54805480u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c = __builtin_amdgcn_fdot2(as_h2(xv[k].x), as_h2(c72), c, false);
        c = __builtin_amdgcn_fdot2(as_h2(xv[k].y), as_h2(c72), c, false);
        c = __builtin_amdgcn_fdot2(as_h2(xv[k].z), as_h2(c72), c, false);
        c = __builtin_amdgcn_fdot2(as_h2(xv[k].w), as_h2(c72), c, false);
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        float t = -c;
        t = dot8_rowmajor(wv[r].x, xv[0], t, m64);
        t = dot8_rowmajor(wv[r].y, xv[1], t, m64);
        t = dot8_rowmajor(wv[r].z, xv[2], t, m64);
        t = dot8_rowmajor(wv[r].w, xv[3], t, m64);
        const float sc = bok ? h2f(sb[r]) : 0.f;
        acc[r][m] = fmaf(sc, t, acc[r][m]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int n = row0 + r;
    const float bv = (bias && n < N) ? h2f(bias[n]) : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_sum(acc[r][m]) + bv;
      if (lane == 0 && n < N && m < M) {
        if (y_f16) reinterpret_cast<uint16_t*>(y)[(size_t)m * N + n] = f2h(tot);
        else reinterpret_cast<float*>(y)[(size_t)m * N + n] = tot;
      }
    }
  }
}

}  // namespace

hipError_t gemv_rowmajor_launch(const uint8_t* q, const uint16_t* s, const uint16_t* bias, const uint16_t* x, int M,
                                int N, int K, void* y, int y_f16, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(N, kRmWaves * kRows)), block(64 * kRmWaves);
  const u32x4* qv = reinterpret_cast<const u32x4*>(q);
  if (M <= 1) hipLaunchKernelGGL(k_gemv_rowmajor<1>, grid, block, 0, st, qv, s, bias, x, M, N, K, y, y_f16);
  else if (M <= 2) hipLaunchKernelGGL(k_gemv_rowmajor<2>, grid, block, 0, st, qv, s, bias, x, M, N, K, y, y_f16);
  else if (M <= 4) hipLaunchKernelGGL(k_gemv_rowmajor<4>, grid, block, 0, st, qv, s, bias, x, M, N, K, y, y_f16);
  else if (M <= 8) hipLaunchKernelGGL(k_gemv_rowmajor<8>, grid, block, 0, st, qv, s, bias, x, M, N, K, y, y_f16);
  else hipLaunchKernelGGL(k_gemv_rowmajor<16>, grid, block, 0, st, qv, s, bias, x, M, N, K, y, y_f16);
  return hipGetLastError();
}

}  // namespace vv
