// int4 block-32 GEMV for a batch of up to 16 rows on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// Same operands, layout, decomposition and split-K hand-off as the VALU kernel (gemv.hip): a
// wave owns one 64-row tile and one group of 8 blocks; lane r of a 16-byte block load holds the
// 32 codes of row r.  A batch of 16 activation rows turns each block into a dense 16 x 32 x 64
// contraction, which the matrix cores take in four 16x16x32 steps (one per group of 16 weight
// rows); on the vector ALU the same work costs 16 dot products per code and would be compute
// bound.
//
// Operand B (32 k x 16 weight rows) wants lane l to hold 8 consecutive k of row l % 16, k-slice
// l / 16.  The load gives lane r all 32 k of row r, as 4 dwords of 8 codes each, so a 4 x 4
// transpose of (dword, 16-lane group) with v_permlane32_swap and v_permlane16_swap moves dword s
// of row 16 g + i to lane 16 s + i of register g.  The codes become fp16 (q - 8) exactly: the
// nibble goes into the mantissa of fp16 64.0 (ulp 1/16, so the value reads 64 + q) and one packed
// fp16 add subtracts 72.  Operand A (16 batch rows x 32 k) comes from the activation slice in LDS.
// The fp16 block scale multiplies each block's fp32 result (products and sums stay exact up to the
// fp32 accumulation), as in the ONNX MatMulNBits semantics of the pages' export.
#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kRows = 16;                    // batch rows of the contraction
constexpr int kW = 4;                        // waves per workgroup
constexpr int kBatchM = 8;                   // blocks per wave (one scale group)
constexpr int kItemK = kW * kBatchM * kBlock;
constexpr int kXPad = 8;                     // fp16 of padding per LDS row (spreads the banks)

template <int EPI>
__device__ __forceinline__ int out_row(int tile, int n) {
  return EPI == EPI_SILU ? tile * 32 + (n & 31) : tile * kTileRows + n;
}

template <int EPI>
__global__ __launch_bounds__(64 * kW) void k_gemv_mfma(GemvParams p, const uint4* __restrict__ qw,
                                                       const uint4* __restrict__ sw,
                                                       const uint16_t* __restrict__ x) {
  // the activation slice, and after the contraction the waves' partial sums, share one buffer
  __shared__ __align__(16) uint16_t lds[kRows * (kItemK + kXPad)];
  static_assert(sizeof(float) * kW * kRows * kTileRows <= sizeof(lds), "partials fit in the slice's buffer");
  uint16_t (*xs)[kItemK + kXPad] = reinterpret_cast<uint16_t (*)[kItemK + kXPad]>(lds);
  float (*red)[kRows][kTileRows] = reinterpret_cast<float (*)[kRows][kTileRows]>(lds);
  __shared__ __align__(16) u32x4 scl[kW][kTileRows];
  __shared__ unsigned s_last;
  const int W = p.wpg;                       // waves with a block group (<= kW)
  const int K = p.K;
  const int nb = K / kBlock;
  const int ng = (nb + kBatchM - 1) / kBatchM;
  const int M = p.M;
  const uint32_t nwg = (uint32_t)p.ntiles * p.wpt;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  if (L >= nwg) return;
  const int tile = L / p.wpt;
  const int kg = L % p.wpt;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int e0 = kg * W * kBatchM * kBlock;  // first K element of this workgroup

  // activation slice: 16 rows x 256 W elements as 16-byte chunks; thread t takes chunk t % 128 of
  // rows t / 128 + 2 i (addresses clamped into the operand: rows past M re-read row M - 1, chunks
  // past the slice or past K repeat an earlier one and are never used)
  const int xc = min(tid & 127, W * 32 - 1);
  const int xe = xc * 8;
  u32x4 xr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = (tid >> 7) + 2 * i;
    xr[i] = *reinterpret_cast<const u32x4*>(x + (size_t)min(m, M - 1) * K + min(e0 + xe, K - 8));
  }
  // this wave's group: scales first (block 0 needs them), then the 8 blocks.  A wave without a
  // group issues the same nine loads from the (cached) activation row and ignores them: with equal
  // load counts on both kinds of wave, the activation's LDS write waits for its own loads only.
  const bool active = w < W;
  const int grp = kg * W + w;
  const int b0 = grp * kBatchM;
  const int nblk = active ? min(max(nb - b0, 0), kBatchM) : 0;
  const u32x4* qt = active ? reinterpret_cast<const u32x4*>(qw) + (size_t)tile * nb * kTileRows + lane
                           : reinterpret_cast<const u32x4*>(x);
  const u32x4* st = active ? reinterpret_cast<const u32x4*>(sw) + ((size_t)tile * ng + min(grp, ng - 1)) * kTileRows + lane
                           : reinterpret_cast<const u32x4*>(x);
  const size_t bstep = active ? kTileRows : 0;
  const u32x4 sv = __builtin_nontemporal_load(st);
  u32x4 wv[kBatchM];
#pragma unroll
  for (int i = 0; i < kBatchM; ++i) wv[i] = __builtin_nontemporal_load(qt + (size_t)min(b0 + i, nb - 1) * bstep);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&xs[(tid >> 7) + 2 * i][xe]) = xr[i];
  __syncthreads();

  // contraction (every wave runs it, so no load is moved under a branch; blocks past the group's
  // end, and all blocks of a wave without a group, get scale 0: their operands are finite codes
  // and activations, so they add exactly 0)
  f32x4 acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    // the 8 scales of rows 16 g + lane % 16 (each lane's own row is lane): through LDS
    scl[w][lane] = sv;
    u32x4 s4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) s4[g] = scl[w][16 * g + (lane & 15)];
    const uint32_t m64 = vconst(0x54005400u), m1024 = vconst(0x64006400u);
    const uint16_t* xa = &xs[lane & 15][min(w, W - 1) * kBatchM * kBlock + 8 * (lane >> 4)];
#pragma unroll
    for (int i = 0; i < kBatchM; ++i) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(xa + i * kBlock);
      const half8 a = __builtin_bit_cast(half8, av);
      uint32_t tg[4];
      block_to_operands(wv[i], tg);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, codes_to_half8(tg[g], m1024, m64),
                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float sc = i < nblk ? pick_scale(s4[g], i) : 0.f;
        acc[g] += sc * d;
      }
    }
  }
  __syncthreads();   // every wave is done with the slice before it is reused
  // lane l of wave w holds rows m = 4 (l / 16) + r, columns n = 16 g + l % 16
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][4 * (lane >> 4) + r][16 * g + (lane & 15)] = acc[g][r];
  __syncthreads();

  // thread (wave w, lane n): column n of rows 4 w .. 4 w + 3
  const int n = lane;
  float tot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float t = 0.f;
    for (int v = 0; v < W; ++v) t += red[v][4 * w + r][n];
    tot[r] = t;
  }
  if (p.wpt > 1) {
    float* my = p.part + ((size_t)tile * p.wpt + kg) * kRows * kTileRows;
#pragma unroll
    for (int r = 0; r < 4; ++r) publish_f32(&my[(4 * w + r) * kTileRows + n], tot[r]);
    wait_published();
    __syncthreads();
    if (tid == 0) s_last = arrive(&p.cnt[tile]) == (unsigned)(p.wpt - 1);
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tot[r] = collect_sum_f32(p.part + ((size_t)tile * p.wpt * kRows + 4 * w + r) * kTileRows + n, p.wpt,
                               (size_t)kRows * kTileRows);
    if (tid == 0) reset_counter(&p.cnt[tile]);  // ready for the next launch
  }

  // epilogue: wave w owns batch rows 4 w .. 4 w + 3, lane n the tile's row n
  const int row = out_row<EPI>(tile, n);
  const bool ok = row < p.N;
  const int rc = min(row, p.N - 1);
  float rs[4] = {1.f, 1.f, 1.f, 1.f};
  if (EPI != EPI_RESID && p.rs_parts) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = min(4 * w + r, M - 1);
      const float v = n < p.rs_nparts ? p.rs_parts[(size_t)m * p.rs_nparts + n] : 0.f;
      rs[r] = 1.0f / sqrtf(wave_sum(v) * p.rs_inv_n + p.eps);
    }
  }
  if (EPI == EPI_STORE) {
    const float bias = p.bias ? h2f(p.bias[rc]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * w + r;
      const float v = tot[r] * rs[r] + bias;
      if (ok && m < M) {
        if (p.y_f16) reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + row] = f2h(v);
        else reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + row] = v;
      }
    }
  } else if (EPI == EPI_RESID) {
    const float gam = p.gamma ? h2f(p.gamma[rc]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * w + r;
      float hn = 0.f;
      if (ok && m < M) {
        const size_t i = (size_t)m * p.N + row;
        hn = p.h[i] + tot[r];
        p.h[i] = hn;
        if (p.trace) p.trace[i] = hn;
        if (p.gamma && p.g_out) {
          if (p.g_f32) reinterpret_cast<float*>(p.g_out)[i] = gam * hn;
          else reinterpret_cast<uint16_t*>(p.g_out)[i] = f2h(gam * hn);
        }
      }
      const float ss = wave_sum(hn * hn);
      if (p.sumsq_out && n == 0 && m < M) p.sumsq_out[m * p.ntiles + tile] = ss;
    }
  } else {  // EPI_SILU: lane n < 32 holds the gate row, lane n + 32 the up row of the same output
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * w + r;
      const float gt = tot[r] * rs[r];
      const float up = __shfl(tot[r], (n & 31) + 32, kWave) * rs[r];
      if (ok && n < 32 && m < M) {
        const float a = silu(gt) * up;
        if (p.act_f32) reinterpret_cast<float*>(p.act)[(size_t)m * p.N + row] = a;
        else reinterpret_cast<uint16_t*>(p.act)[(size_t)m * p.N + row] = f2h(a);
      }
    }
  }
}

}  // namespace

// the matrix-core kernel reads fp16 activations (x_f32 must be 0)
hipError_t gemv_mfma_launch(const GemvParams& p, hipStream_t st, KEv ev) {
  if (p.x_f32) return hipErrorInvalidValue;
  const uint4* q = reinterpret_cast<const uint4*>(p.q);
  const uint4* s = reinterpret_cast<const uint4*>(p.s);
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const dim3 g(p.grid), b(64 * kW);
  switch (p.epi) {
    case EPI_STORE: VV_LAUNCH((k_gemv_mfma<EPI_STORE>), g, b, st, ev, p, q, s, x); break;
    case EPI_RESID: VV_LAUNCH((k_gemv_mfma<EPI_RESID>), g, b, st, ev, p, q, s, x); break;
    default: VV_LAUNCH((k_gemv_mfma<EPI_SILU>), g, b, st, ev, p, q, s, x); break;
  }
  return hipGetLastError();
}

}  // namespace vv
