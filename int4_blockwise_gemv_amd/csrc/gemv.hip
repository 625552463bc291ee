// int4 block-32 GEMV on the tiled layout (MatMulNBits semantics with float activations).
//
// One wave owns one 64-row tile and a contiguous range of kb blocks: lane i accumulates row
// 64t+i, so every 16-byte block load of the wave is one contiguous 1 KiB line run, and the
// activation block is the same for all lanes (wave-uniform loads).
//
// In-register dequantisation: a packed dword holds 8 codes with the even elements in nibbles
// 0..3 and the odd ones in nibbles 4..7, so a shift and one AND-OR with the fp16 exponent of
// 64.0 turn nibble pair (i, 4+i) into the fp16 pair (64 + q_2i, 64 + q_2i+1), which lines up
// with the natural fp16 pair (x_2i, x_2i+1) of the activation; v_dot2_f32_f16 then multiplies
// both with exact products and fp32 accumulation.  The offset 64 and the zero point 8 are
// removed once per block by subtracting C_b = 72 * sum_j x_j, computed once per wave for its
// blocks; the block sum is scaled by the block's fp16 scale in fp32.
//
// Split-K: the kb-block ranges of a tile are spread over the 4 waves of a workgroup (reduced in
// LDS) and over `wpt` workgroups; the last workgroup to arrive at a tile (atomic counter) adds
// the partials in a fixed order and runs the epilogue, so results do not depend on timing.
#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kWavesPerWG = 4;
constexpr int kTargetWaves = 4096;

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

__device__ __forceinline__ float pick_scale(const u32x4& s, int j) {
  const uint32_t d = (j >> 1) == 0 ? s.x : (j >> 1) == 1 ? s.y : (j >> 1) == 2 ? s.z : s.w;
  return (j & 1) ? (float)__builtin_bit_cast(h2_t, d).y : (float)__builtin_bit_cast(h2_t, d).x;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Epilogue for one tile's finished row sums (called by one wave, lane = row within the tile).
template <int MT>
__device__ void epilogue(const GemvParams& p, int unit, const float (&tot)[2][MT], int lane) {
  const int M = p.M;
  if (p.epi == EPI_STORE) {
    const int n = unit * kTileRows + lane;
    const bool ok = n < p.N;
    const float bias = (ok && p.bias) ? h2f(p.bias[n]) : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      const float rs = p.rs_parts ? rstd_from_parts(p.rs_parts + m * p.rs_nparts, p.rs_nparts, p.rs_inv_n, p.eps) : 1.f;
      const float v = tot[0][m] * rs + bias;
      if (ok) {
        if (p.y_f16) reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + n] = f2h(v);
        else reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + n] = v;
      }
    }
  } else if (p.epi == EPI_RESID) {
    const int n = unit * kTileRows + lane;
    const bool ok = n < p.N;
    const float gam = (ok && p.gamma) ? h2f(p.gamma[n]) : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      float hn = 0.f;
      if (ok) {
        const size_t i = (size_t)m * p.N + n;
        hn = p.h[i] + tot[0][m];
        p.h[i] = hn;
        if (p.trace) p.trace[i] = hn;
        if (p.gamma) {
          const float gv = gam * hn;
          if (p.g_out) p.g_out[i] = f2h(gv);
          if (p.gf_out) p.gf_out[i] = gv;
        }
      }
      const float ss = wave_sum(hn * hn);
      if (p.sumsq_out && lane == 0) p.sumsq_out[m * p.ntiles + unit] = ss;
    }
  } else {  // EPI_SILU: unit j = (gate tile 2j, up tile 2j+1)
    const int n = unit * kTileRows + lane;
    const bool ok = n < p.N;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      const float rs = p.rs_parts ? rstd_from_parts(p.rs_parts + m * p.rs_nparts, p.rs_nparts, p.rs_inv_n, p.eps) : 1.f;
      const float g = tot[0][m] * rs;
      const float u = tot[1][m] * rs;
      if (ok) p.act[(size_t)m * p.N + n] = f2h(silu(g) * u);
    }
  }
}

template <int MT, int KBMAX>
__global__ __launch_bounds__(256) void k_gemv(GemvParams p, const uint4* __restrict__ qw,
                                              const uint4* __restrict__ sw, const uint16_t* __restrict__ x) {
  __shared__ float red[kWavesPerWG][MT][kTileRows];
  const int K = p.K;
  const int nb = K / kBlock;
  const int ng = (nb + 7) >> 3;
  const int M = p.M;
  const uint32_t nwg = (uint32_t)p.ntiles * p.wpt;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  if (L >= nwg) return;
  const int tile = L / p.wpt;
  const int kg = L % p.wpt;
  const int w = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const int b0 = (kg * kWavesPerWG + w) * p.kb;
  int nblk = nb - b0;
  nblk = nblk < 0 ? 0 : (nblk > p.kb ? p.kb : nblk);

  // activation quarters for the per-block correction C_b (lane 4i+q: quarter q of block b0+i)
  u32x4 xq[MT];
  {
    const int bl = lane >> 2, qd = lane & 3;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      xq[m] = u32x4{0, 0, 0, 0};
      if (m < M && bl < nblk)
        xq[m] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + (size_t)(b0 + bl) * kBlock + qd * 8);
    }
  }

  // weights and scales of this wave: all loads issued before any use
  u32x4 wv[KBMAX];
  const u32x4* qp = reinterpret_cast<const u32x4*>(qw) + ((size_t)tile * nb + b0) * kTileRows + lane;
#pragma unroll
  for (int i = 0; i < KBMAX; ++i)
    if (i < nblk) wv[i] = __builtin_nontemporal_load(qp + (size_t)i * kTileRows);
  constexpr int SG = KBMAX / 8;  // b0 is a multiple of 8: block i of the wave is scale (i/8, i%8)
  u32x4 sv[SG];
  const int g0 = b0 >> 3;
  const u32x4* sp = reinterpret_cast<const u32x4*>(sw) + ((size_t)tile * ng + g0) * kTileRows + lane;
#pragma unroll
  for (int j = 0; j < SG; ++j)
    if (8 * j < nblk) sv[j] = __builtin_nontemporal_load(sp + (size_t)j * kTileRows);
  const uint32_t m64 = vconst(0x54005400u);

  float corr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float c = corr_quarter(xq[m]);
    c += __shfl_xor(c, 1, kWave);
    c += __shfl_xor(c, 2, kWave);
    corr[m] = c;
  }

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;

#pragma unroll
  for (int i = 0; i < KBMAX; ++i) {
    if (i < nblk) {
      const int b = b0 + i;
      const float sc = pick_scale(sv[i / 8], i % 8);
      const u32x4 q4 = wv[i];
      const uint32_t d[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          const uint32_t* xb = reinterpret_cast<const uint32_t*>(x + (size_t)m * K + (size_t)b * kBlock);
          float t = -__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, corr[m]), 4 * i));
#pragma unroll
          for (int k = 0; k < 4; ++k) t = dot8_pairs(d[k], xb + 4 * k, t, m64);
          acc[m] = fmaf(sc, t, acc[m]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < M) red[w][m][lane] = acc[m];
  __syncthreads();
  if (w != 0) return;

  float tot[2][MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    tot[0][m] = 0.f;
    tot[1][m] = 0.f;
    if (m < M) tot[0][m] = ((red[0][m][lane] + red[1][m][lane]) + red[2][m][lane]) + red[3][m][lane];
  }

  if (p.wpt == 1 && p.unit_tiles == 1) {
    epilogue<MT>(p, tile, tot, lane);
    return;
  }
  // publish this workgroup's partial, then count arrivals for the unit
  float* my = p.part + ((size_t)tile * p.wpt + kg) * MT * kTileRows;
#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < M) publish_f32(&my[m * kTileRows + lane], tot[0][m]);
  wait_published();
  const int unit = tile / p.unit_tiles;
  unsigned prev = 0;
  if (lane == 0) prev = arrive(&p.cnt[unit]);
  prev = __shfl(prev, 0, kWave);
  const unsigned arrivals = (unsigned)(p.wpt * p.unit_tiles);
  if (prev != arrivals - 1) return;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u >= p.unit_tiles) continue;
    const int t = unit * p.unit_tiles + u;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      float s = 0.f;
      for (int k = 0; k < p.wpt; ++k)
        s += collect_f32(p.part + (((size_t)t * p.wpt + k) * MT + m) * kTileRows + lane);
      tot[u][m] = s;
    }
  }
  if (lane == 0) reset_counter(&p.cnt[unit]);  // ready for the next launch
  epilogue<MT>(p, unit, tot, lane);
}

int mt_of(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

struct Plan { int kb, wpt, grid; };

// Blocks per wave: 8 or 16 (ranges start on scale-group boundaries), 16 only when the matrix
// offers more than kTargetWaves waves of 8 blocks.
Plan make_plan(int M, int ntiles, int nb) {
  (void)M;
  const int kb = (int64_t)ntiles * cdiv(nb, 8) > kTargetWaves ? 16 : 8;
  const int nkc = (int)cdiv(nb, kb);
  const int wpt = (int)cdiv(nkc, kWavesPerWG);
  Plan pl;
  pl.kb = kb;
  pl.wpt = wpt;
  pl.grid = (int)(cdiv((int64_t)ntiles * wpt, kNumXcd) * kNumXcd);
  return pl;
}

template <int MT>
hipError_t launch_mt(const GemvParams& p, hipStream_t st) {
  const uint4* q = reinterpret_cast<const uint4*>(p.q);
  const uint4* s = reinterpret_cast<const uint4*>(p.s);
  if (p.kb <= 8)
    hipLaunchKernelGGL((k_gemv<MT, 8>), dim3(p.grid), dim3(256), 0, st, p, q, s, p.x);
  else
    hipLaunchKernelGGL((k_gemv<MT, 16>), dim3(p.grid), dim3(256), 0, st, p, q, s, p.x);
  return hipGetLastError();
}

}  // namespace

void gemv_plan(GemvParams& p) {
  const Plan pl = make_plan(p.M, p.ntiles, p.K / kBlock);
  p.kb = pl.kb;
  p.wpt = pl.wpt;
  p.grid = pl.grid;
}

size_t gemv_workspace_bytes(int M, int ntiles, int unit_tiles, int nb) {
  const Plan pl = make_plan(M, ntiles, nb);
  const int MT = mt_of(M);
  const size_t part = (size_t)ntiles * pl.wpt * MT * kTileRows * sizeof(float);
  const size_t cnt = (size_t)cdiv(ntiles, unit_tiles) * sizeof(unsigned);
  return align_up(part, 256) + align_up(cnt, 256);
}

void gemv_set_workspace(GemvParams& p, void* ws) {
  const Plan pl = make_plan(p.M, p.ntiles, p.K / kBlock);
  const int MT = mt_of(p.M);
  const size_t part = (size_t)p.ntiles * pl.wpt * MT * kTileRows * sizeof(float);
  p.part = reinterpret_cast<float*>(ws);
  p.cnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + align_up(part, 256));
}

hipError_t gemv_launch(const GemvParams& p, hipStream_t st) {
  switch (mt_of(p.M)) {
    case 1: return launch_mt<1>(p, st);
    case 2: return launch_mt<2>(p, st);
    case 4: return launch_mt<4>(p, st);
    case 8: return launch_mt<8>(p, st);
    default: return launch_mt<16>(p, st);
  }
}

}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_gemv_int4_workspace(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 16 || N < 1 || K < kBlock || K % kBlock) return 0;
  return gemv_workspace_bytes((int)M, (int)cdiv(N, kTileRows), 1, (int)(K / kBlock));
}

int vv_gemv_int4(const uint8_t* packed, const uint16_t* scales, const uint16_t* bias, const uint16_t* x, int64_t M,
                 int64_t N, int64_t K, void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  VV_REQUIRE(packed && scales && x && y, VV_ERR_NULL, "vv_gemv_int4: NULL pointer");
  VV_REQUIRE(M >= 1 && M <= 16, VV_ERR_RANGE, "vv_gemv_int4: M = %lld not in 1..16", (long long)M);
  VV_REQUIRE(N >= 1 && N <= (1 << 26), VV_ERR_RANGE, "vv_gemv_int4: N = %lld out of range", (long long)N);
  VV_REQUIRE(K >= kBlock && K % kBlock == 0 && K <= (1 << 22), VV_ERR_SHAPE,
             "vv_gemv_int4: K = %lld is not a positive multiple of 32 (<= 4M)", (long long)K);
  VV_REQUIRE(y_dtype == VV_F16 || y_dtype == VV_F32, VV_ERR_DTYPE, "vv_gemv_int4: unknown y dtype %d", y_dtype);
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(scales) |
               reinterpret_cast<uintptr_t>(x)) & 15) == 0,
             VV_ERR_RANGE, "vv_gemv_int4: packed, scales and x must be 16-byte aligned");
  const size_t need = vv_gemv_int4_workspace(M, N, K);
  VV_REQUIRE(ws && ws_bytes >= need, VV_ERR_WORKSPACE, "vv_gemv_int4: workspace needs %zu bytes", need);
  GemvParams p{};
  p.q = packed; p.s = scales; p.x = x;
  p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.ntiles = (int)cdiv(N, kTileRows);
  p.unit_tiles = 1;
  p.epi = EPI_STORE;
  p.bias = bias; p.y = y; p.y_f16 = y_dtype == VV_F16; p.ldy = (int)N;
  p.eps = 0.f;
  gemv_plan(p);
  gemv_set_workspace(p, ws);
  VV_HIP(gemv_launch(p, as_stream(stream)));
  return VV_OK;
}

}  // extern "C"
