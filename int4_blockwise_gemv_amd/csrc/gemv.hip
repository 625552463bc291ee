// int4 block-32 GEMV on the tiled layout (MatMulNBits semantics with float activations).
//
// Decomposition: a wave owns one 64-row tile and one group of 8 consecutive blocks (lane i
// accumulates row 64t+i, so each 16-byte block load of the wave is one contiguous 1 KiB run, and
// the group's 8 fp16 scales are one more 16-byte load); a workgroup takes `wpg` consecutive
// groups of one tile (up to 16), and a tile's groups are spread over `wpt` workgroups.  All nine
// loads of a wave are in flight at once: short waves keep the HBM busiest.
//
// Activations: before any weight load, the workgroup's slice of x (256 elements per wave, per row)
// goes to LDS with one vector load per thread; the waves then read their block's 32 values as
// LDS broadcasts.  (Scalar loads issued block by block would put one L2 latency per block on the
// path.)
//
// In-register dequantisation: a packed dword holds 8 codes with the even elements in nibbles
// 0..3 and the odd ones in nibbles 4..7, so a shift and one AND-OR with the fp16 exponent of
// 64.0 turn nibble pair (i, 4+i) into the fp16 pair (64 + q_2i, 64 + q_2i+1), which lines up
// with the natural fp16 pair (x_2i, x_2i+1) of the activation; v_dot2_f32_f16 then multiplies
// both with exact products and fp32 accumulation.  The offset 64 and the zero point 8 are
// removed once per block by subtracting C_b = 72 * sum_j x_j; the block sum is scaled by the
// block's fp16 scale in fp32.
//
// Split-K: the waves of a workgroup are reduced in LDS; with wpt > 1 the last workgroup to
// arrive at a tile adds the partials in a fixed order and runs the epilogue, so results do not
// depend on timing.  With wpt = 1 the workgroup finishes its tile directly.
#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kWavesSmallM = 4;   // most waves (groups) per workgroup for M <= 2 (wider was slower)
constexpr int kWavesLargeM = 4;   // for M > 2 (LDS holds M activation slices)
constexpr int kBatch = 8;        // blocks per load batch (one scale group)

// Operands of the epilogue, loaded by wave 0 of every workgroup before the weight stream so the
// workgroup that finishes a tile does not wait on them.
template <int MT>
struct EpiPre {
  float rs[MT];     // 1/sqrt(mean(h^2) + eps) of the input rows (or 1)
  float bias;       // bias of this lane's row (EPI_STORE)
  float gam;        // gamma of this lane's row (EPI_RESID)
  float h[MT];      // residual of this lane's row (EPI_RESID)
};

// row of lane `lane` of tile `tile` in the output vector (EPI_SILU: lanes 0-31 gate, 32-63 up
// of the same 32 rows)
__device__ __forceinline__ int out_row(const GemvParams& p, int tile, int lane) {
  return p.epi == EPI_SILU ? tile * 32 + (lane & 31) : tile * kTileRows + lane;
}

template <int MT>
__device__ __forceinline__ void epi_prefetch(const GemvParams& p, int tile, int lane, EpiPre<MT>& e,
                                             float (&rsp)[MT]) {
  const int n = out_row(p, tile, lane);
  const bool ok = n < p.N;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    rsp[m] = 0.f;
    e.h[m] = 0.f;
    if (m < p.M && p.rs_parts && lane < p.rs_nparts) rsp[m] = p.rs_parts[m * p.rs_nparts + lane];
    if (m < p.M && p.epi == EPI_RESID && ok) e.h[m] = p.h[(size_t)m * p.N + n];
  }
  e.bias = (p.epi == EPI_STORE && ok && p.bias) ? h2f(p.bias[n]) : 0.f;
  e.gam = (p.epi == EPI_RESID && ok && p.gamma) ? h2f(p.gamma[n]) : 0.f;
}

// rstd from the per-tile sums of squares (lane l holds part l; fixed reduction tree)
template <int MT>
__device__ __forceinline__ void epi_finish_rs(const GemvParams& p, EpiPre<MT>& e, const float (&rsp)[MT]) {
#pragma unroll
  for (int m = 0; m < MT; ++m) e.rs[m] = p.rs_parts ? 1.0f / sqrtf(wave_sum(rsp[m]) * p.rs_inv_n + p.eps) : 1.f;
}

// Epilogue for one tile's finished row sums (one wave, lane = row within the tile).
template <int MT>
__device__ void epilogue(const GemvParams& p, int tile, const float (&tot)[MT], const EpiPre<MT>& e, int lane) {
  const int M = p.M;
  const int n = out_row(p, tile, lane);
  const bool ok = n < p.N;
  if (p.epi == EPI_STORE) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      const float v = tot[m] * e.rs[m] + e.bias;
      if (ok) {
        if (p.y_f16) reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + n] = f2h(v);
        else reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + n] = v;
      }
    }
  } else if (p.epi == EPI_RESID) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      float hn = 0.f;
      if (ok) {
        const size_t i = (size_t)m * p.N + n;
        hn = e.h[m] + tot[m];
        p.h[i] = hn;
        if (p.trace) p.trace[i] = hn;
        if (p.gamma) {
          const float gv = e.gam * hn;
          if (p.g_out) p.g_out[i] = f2h(gv);
          if (p.gf_out) p.gf_out[i] = gv;
        }
      }
      const float ss = wave_sum(hn * hn);
      if (p.sumsq_out && lane == 0) p.sumsq_out[m * p.ntiles + tile] = ss;
    }
  } else {  // EPI_SILU: lane i < 32 holds the gate row, lane i + 32 the up row of the same output
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      const float g = tot[m] * e.rs[m];
      const float u = __shfl(tot[m], (lane & 31) + 32, kWave) * e.rs[m];
      if (ok && lane < 32) p.act[(size_t)m * p.N + n] = f2h(silu(g) * u);
    }
  }
}

template <int MT> struct WavesFor { static constexpr int value = MT <= 2 ? kWavesSmallM : kWavesLargeM; };

// WMAX waves at most; the launch uses p.wpg = blockDim.x / 64 of them (one 8-block group each)
template <int MT>
__global__ __launch_bounds__(64 * WavesFor<MT>::value) void k_gemv(GemvParams p, const uint4* __restrict__ qw,
                                                                  const uint4* __restrict__ sw,
                                                                  const uint16_t* __restrict__ x) {
  constexpr int WMAX = WavesFor<MT>::value;
  constexpr int kItemK = WMAX * kBatch * kBlock;  // K elements per workgroup at most
  __shared__ __align__(16) uint16_t xs[MT][kItemK];
  __shared__ float red[WMAX][MT][kTileRows];
  const int W = p.wpg;
  const int K = p.K;
  const int nb = K / kBlock;
  const int ng = (nb + kBatch - 1) / kBatch;
  const int M = p.M;
  const uint32_t nwg = (uint32_t)p.ntiles * p.wpt;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  if (L >= nwg) return;
  const int tile = L / p.wpt;
  const int kg = L % p.wpt;
  const int w = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const int e0 = kg * W * kBatch * kBlock;          // first K element of this workgroup
  const int ne = min(K - e0, W * kBatch * kBlock);

  // activation slice first (its loads return before the weights), 8 bytes per thread per row
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int e = 4 * (int)threadIdx.x;
    if (m < M && e < ne)
      *reinterpret_cast<uint2*>(&xs[m][e]) = *reinterpret_cast<const uint2*>(x + (size_t)m * K + e0 + e);
  }
  static_assert(kItemK <= 4 * 64 * WMAX, "one 8-byte activation load per thread covers the slice");
  // this wave's group: 8 blocks and their 8 scales
  const int grp = kg * W + w;
  const int b0 = grp * kBatch;
  const int nblk = min(max(nb - b0, 0), kBatch);
  const u32x4* qp = reinterpret_cast<const u32x4*>(qw) + ((size_t)tile * nb + b0) * kTileRows + lane;
  u32x4 wv[kBatch];
  u32x4 sv = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kBatch; ++i)
    if (i < nblk) wv[i] = __builtin_nontemporal_load(qp + (size_t)i * kTileRows);
  if (nblk > 0) sv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sw) + ((size_t)tile * ng + grp) * kTileRows + lane);

  EpiPre<MT> ep;
  float rsp[MT];
  if (w == 0) epi_prefetch<MT>(p, tile, lane, ep, rsp);
  __syncthreads();

  const uint32_t m64 = vconst(0x54005400u);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  if (nblk > 0) {
    const int xb0 = w * kBatch * kBlock;            // this wave's first element in the slice
    float corr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      u32x4 xv = u32x4{0, 0, 0, 0};
      if (m < M && lane < 4 * nblk) xv = *reinterpret_cast<const u32x4*>(&xs[m][xb0 + lane * 8]);
      corr[m] = quad_sum(corr_quarter(xv));           // lane 4i+q: quarter q of block i
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < nblk) {
        const float sc = pick_scale(sv, i);
        const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M) {
            const u32x4* xb = reinterpret_cast<const u32x4*>(&xs[m][xb0 + i * kBlock]);
            float t = -__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, corr[m]), 4 * i));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const u32x4 xv = xb[k];
              const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
              t = dot8_pairs(d[k], x4, t, m64);
            }
            acc[m] = fmaf(sc, t, acc[m]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < M) red[w][m][lane] = acc[m];
  __syncthreads();
  if (w != 0) return;
  epi_finish_rs<MT>(p, ep, rsp);

  float tot[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    tot[m] = 0.f;
    if (m < M) {
      float t = 0.f;
      for (int v = 0; v < W; ++v) t += red[v][m][lane];
      tot[m] = t;
    }
  }
  if (p.wpt == 1) {
    epilogue<MT>(p, tile, tot, ep, lane);
    return;
  }
  // publish this workgroup's partial, then count arrivals at the tile
  float* my = p.part + ((size_t)tile * p.wpt + kg) * MT * kTileRows;
#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < M) publish_f32(&my[m * kTileRows + lane], tot[m]);
  wait_published();
  unsigned prev = 0;
  if (lane == 0) prev = arrive(&p.cnt[tile]);
  prev = __shfl(prev, 0, kWave);
  if (prev != (unsigned)(p.wpt - 1)) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= M) continue;
    tot[m] = collect_sum_f32(p.part + ((size_t)tile * p.wpt * MT + m) * kTileRows + lane, p.wpt,
                             (size_t)MT * kTileRows);
  }
  if (lane == 0) reset_counter(&p.cnt[tile]);  // ready for the next launch
  epilogue<MT>(p, tile, tot, ep, lane);
}

int mt_of(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

struct Plan { int kb, wpg, wpt, grid; };

// One 8-block group (one batch: 8 weight loads + 1 scale load, all in flight at once) per wave.
// Batch <= 2: up to 16 waves (groups) per workgroup, the groups of a tile spread evenly over
// wpt = ceil(groups / 16) workgroups; a tile of <= 16 groups is one workgroup and needs no
// cross-workgroup reduction.  Larger batches: 4 waves per workgroup (LDS holds M slices).
Plan make_plan(int M, int ntiles, int nb) {
  const int ng = (int)cdiv(nb, kBatch);
  const int wmax = M <= 2 ? kWavesSmallM : kWavesLargeM;
  Plan pl;
  pl.kb = kBatch;
  pl.wpt = (int)cdiv(ng, wmax);
  pl.wpg = (int)cdiv(ng, pl.wpt);
  pl.grid = (int)(cdiv((int64_t)ntiles * pl.wpt, kNumXcd) * kNumXcd);
  return pl;
}

}  // namespace

void gemv_plan(GemvParams& p) {
  const Plan pl = make_plan(p.M, p.ntiles, p.K / kBlock);
  p.kb = pl.kb;
  p.wpg = pl.wpg;
  p.wpt = pl.wpt;
  p.grid = pl.grid;
}

size_t gemv_workspace_bytes(int M, int ntiles, int nb) {
  const Plan pl = make_plan(M, ntiles, nb);
  const int MT = mt_of(M);
  const size_t part = (size_t)ntiles * pl.wpt * MT * kTileRows * sizeof(float);
  const size_t cnt = (size_t)ntiles * sizeof(unsigned);
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
  const uint4* q = reinterpret_cast<const uint4*>(p.q);
  const uint4* s = reinterpret_cast<const uint4*>(p.s);
  switch (mt_of(p.M)) {
    case 1: hipLaunchKernelGGL(k_gemv<1>, dim3(p.grid), dim3(64 * p.wpg), 0, st, p, q, s, p.x); break;
    case 2: hipLaunchKernelGGL(k_gemv<2>, dim3(p.grid), dim3(64 * p.wpg), 0, st, p, q, s, p.x); break;
    case 4: hipLaunchKernelGGL(k_gemv<4>, dim3(p.grid), dim3(64 * p.wpg), 0, st, p, q, s, p.x); break;
    case 8: hipLaunchKernelGGL(k_gemv<8>, dim3(p.grid), dim3(64 * p.wpg), 0, st, p, q, s, p.x); break;
    default: hipLaunchKernelGGL(k_gemv<16>, dim3(p.grid), dim3(64 * p.wpg), 0, st, p, q, s, p.x); break;
  }
  return hipGetLastError();
}

}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_gemv_int4_workspace(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 16 || N < 1 || K < kBlock || K % kBlock) return 0;
  return gemv_workspace_bytes((int)M, (int)cdiv(N, kTileRows), (int)(K / kBlock));
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
  p.epi = EPI_STORE;
  p.bias = bias; p.y = y; p.y_f16 = y_dtype == VV_F16; p.ldy = (int)N;
  p.eps = 0.f;
  gemv_plan(p);
  gemv_set_workspace(p, ws);
  VV_HIP(gemv_launch(p, as_stream(stream)));
  return VV_OK;
}

}  // extern "C"
