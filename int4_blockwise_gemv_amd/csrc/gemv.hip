// int4 block-32 GEMV on the tiled layout (MatMulNBits semantics with float activations).
//
// Decomposition: a wave owns one 64-row tile and one group of 8 consecutive blocks (lane i
// accumulates row 64t+i, so each 16-byte block load of the wave is one contiguous 1 KiB run, and
// the group's 8 fp16 scales are one more 16-byte load); a workgroup takes `wpg` consecutive
// groups of one tile (up to 8), and a tile's groups are spread over `wpt` workgroups.  All nine
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
// both with exact products and fp32 accumulation.  With fp16 activations the offset 64 and the
// zero point 8 are removed once per block by subtracting C_b = 72 * sum_j x_j; with fp32
// activations (two fp16 parts, hi + lo) one packed fp16 add per pair makes the codes q - 8
// first, so that no offset cancels in the fp32 sums.  The block sum is scaled by the block's
// fp16 scale in fp32.
//
// Split-K: the waves of a workgroup are reduced in LDS; with wpt = 1 the workgroup finishes its
// tile directly.  With wpt > 1 a tile's last K-chunk workgroup (kg = wpt - 1) is its reader and
// the others are writers: a writer stores its partial with a tag into a hand-off slot and exits
// (no store wait, no atomic, so it gives its slot back at once); the reader computes its own
// chunk, polls the slots, adds them in a fixed order (then its own partial, so results do not
// depend on timing), clears them and runs the epilogue.  The tiles are dealt to the XCDs in
// contiguous blocks, and each XCD's dispatch sequence is all writers of its tiles first, then
// all readers: a reader waits only for writers dispatched before it on its own XCD (so the wait
// always ends), and by the time it is dispatched they have mostly finished.  The wait is also
// bounded: one that gives up sets the status word (when there is one) and yields NaN.
#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kWavesSmallM = 8;   // most waves (groups) per workgroup for M <= 2
constexpr int kWavesLargeM = 4;   // for M > 2 (LDS holds M activation slices)
// M <= 2 takes 8-wave workgroups only when that still leaves >= kWideMinWgs workgroups (two per
// CU): fewer workgroups per tile shorten the cross-workgroup reduction of the large GEMVs, while
// the small ones need the parallelism (7B shape: gate/up and down 8 waves, q|k|v and o 4).
constexpr int kWideMinWgs = 512;
constexpr int kBatch = 8;        // blocks per load batch (one scale group)
// Operands of the epilogue.  Every wave loads them before its weight stream, from clamped
// in-bounds addresses, so no load sits behind a branch: a conditional load whose result merges
// with a default value makes the compiler wait for it (and for every load issued before it) on
// the spot, which serialises the stream.  Values that do not apply are zeroed at use.
template <int MT>
struct EpiPre {
  float rsp[MT];    // lane l: per-tile sum of squares l of the input rows (rstd source), raw
  float rs[MT];     // 1/sqrt(mean(h^2) + eps) of the input rows (or 1), after epi_finish
  uint32_t b16;     // raw fp16 bias (EPI_STORE) or gamma (EPI_RESID) of this lane's row
  float bias;       // bias of this lane's row (EPI_STORE), after epi_finish
  float gam;        // gamma of this lane's row (EPI_RESID), after epi_finish
  float h[MT];      // residual of this lane's row (EPI_RESID)
};

// row of lane `lane` of tile `tile` in the output vector (EPI_SILU: lanes 0-31 gate, 32-63 up
// of the same 32 rows)
template <int EPI>
__device__ __forceinline__ int out_row(int tile, int lane) {
  return EPI == EPI_SILU ? tile * 32 + (lane & 31) : tile * kTileRows + lane;
}

// gemv_launch makes rs_parts, bias and gamma readable (pointing at x when absent) and records
// which are real in rs_mask / has_bias / has_gamma, so these loads need no branch; the values are
// selected and converted only in epi_finish, after the barrier, so nothing waits on them early.
template <int MT, int EPI>
__device__ __forceinline__ void epi_prefetch(const GemvParams& p, int tile, int lane, EpiPre<MT>& e) {
  const int nc = min(out_row<EPI>(tile, lane), p.N - 1);
  if (EPI != EPI_RESID) {
    const int np = max(p.rs_nparts, 1);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      e.rsp[m] = p.rs_parts[min(m, p.M - 1) * np * p.rs_mask + min(lane, np - 1) * p.rs_mask];
  }
  if (EPI == EPI_STORE) e.b16 = p.bias[nc * p.has_bias];
  if (EPI == EPI_RESID) {
#pragma unroll
    for (int m = 0; m < MT; ++m) e.h[m] = p.h[(size_t)min(m, p.M - 1) * p.N + nc];
    e.b16 = p.gamma[nc * p.has_gamma];
  }
}

template <int MT, int EPI>
__device__ __forceinline__ void epi_finish(const GemvParams& p, int tile, int lane, EpiPre<MT>& e) {
  const bool ok = out_row<EPI>(tile, lane) < p.N;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float part = (EPI != EPI_RESID && lane < p.rs_nparts) ? e.rsp[m] : 0.f;
    e.rs[m] = (EPI != EPI_RESID && p.rs_mask) ? 1.0f / sqrtf(wave_sum(part) * p.rs_inv_n + p.eps) : 1.f;
  }
  const float v = h2f((uint16_t)e.b16);
  e.bias = (EPI == EPI_STORE && p.has_bias && ok) ? v : 0.f;
  e.gam = (EPI == EPI_RESID && p.has_gamma) ? v : 0.f;
}

// Epilogue for one tile's finished row sums (one wave, lane = row within the tile).
template <int MT, int EPI>
__device__ void epilogue(const GemvParams& p, int tile, const float (&tot)[MT], const EpiPre<MT>& e, int lane) {
  const int M = p.M;
  const int n = out_row<EPI>(tile, lane);
  const bool ok = n < p.N;
  if (EPI == EPI_STORE) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      const float v = tot[m] * e.rs[m] + e.bias;
      if (ok) {
        if (p.y_f16) reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + n] = f2h(v);
        else reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + n] = v;
      }
    }
  } else if (EPI == EPI_RESID) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      float hn = 0.f;
      if (ok) {
        const size_t i = (size_t)m * p.N + n;
        hn = e.h[m] + tot[m];
        p.h[i] = hn;
        if (p.trace) p.trace[i] = hn;
        if (p.has_gamma && p.g_out) {
          const float gv = e.gam * hn;
          if (p.g_f32) reinterpret_cast<float*>(p.g_out)[i] = gv;
          else reinterpret_cast<uint16_t*>(p.g_out)[i] = f2h(gv);
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
      if (ok && lane < 32) {
        const float a = silu(g) * u;
        if (p.act_f32) reinterpret_cast<float*>(p.act)[(size_t)m * p.N + n] = a;
        else reinterpret_cast<uint16_t*>(p.act)[(size_t)m * p.N + n] = f2h(a);
      }
    }
  }
}

// WMAX waves at most (4 or 8: separate instances, so the 4-wave launches keep the register and
// LDS budget of a 256-thread workgroup); the launch uses p.wpg = blockDim.x / 64 of them (one
// 8-block group each).
// From the first load to the barrier the code is branch-free: every load address is clamped
// into the operand (a group past the end of K re-reads the last block and gets scale 0, rows
// past M re-read row M-1 and are never stored), so all loads of a wave are in flight together.
// Fused split-KV merge (the leading p.mrg_blocks workgroups of an XT launch): wave w of workgroup
// i merges item i W + w = (batch row, query head, 64-dim half) over at most 64 splits and stores
// each dim as a tagged word (tag << 32) | fp32 bits of the normalised output, at [row][head][dim].
__device__ void fused_merge(const GemvParams& p) {
  const int W = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * W + w;
  if (item >= 2 * p.mrg_nq * p.M) return;
  const int b = item / (2 * p.mrg_nq), bi = item % (2 * p.mrg_nq);
  const int h = bi >> 1, d = 64 * (bi & 1) + lane;
  const int g = p.mrg_nq / p.mrg_nkv, kvh = h / g, hh = h % g;
  const int n = attn_splits(p.mrg_pos, nullptr, b, p.mrg_cap, p.mrg_split);
  const float* rec0 = p.mrg_part + (((size_t)b * p.mrg_nkv + kvh) * p.mrg_nsplit * kAttnMaxG + hh) * kAttnRec;
  float Mw, Lw;
  const float Ow = merge_wave64(rec0, (size_t)kAttnMaxG * kAttnRec, 0, n, d, Mw, Lw);
  const uint32_t tag = p.epoch[0] * p.tag_mul + p.tag_add;
  publish_u64(p.xtag + ((size_t)b * p.mrg_nq + h) * 128 + d, ((uint64_t)tag << 32) | __float_as_uint(Ow / Lw));
}

// XF: the activations are fp32 and each 32-element block is staged as its 8-bit digit image
// (22 bits relative to the block's largest magnitude; exact integer products with the codes);
// else they are fp16 as given and meet the codes as fp16 pairs.  XT implies XF (the merged
// attention output arrives as tagged fp32 words).
template <int MT, int EPI, int WMAX, bool XT, bool XF>
__global__ __launch_bounds__(64 * WMAX) void k_gemv(GemvParams p, const uint4* __restrict__ qw,
                                                                  const uint4* __restrict__ sw,
                                                                  const void* __restrict__ xin) {
  constexpr int kItemK = WMAX * kBatch * kBlock;  // K elements per workgroup at most
  // activations in LDS: fp16 as given, or (XF) the digit image of every 32-element block
  __shared__ __align__(16) uint16_t xs[XF ? 1 : MT][XF ? 8 : kItemK];
  __shared__ __align__(16) uint32_t xd[XF ? MT : 1][XF ? kItemK / kBlock * kDigitDwords : 4];
  __shared__ float red[WMAX][MT][kTileRows];
  static_assert(!XT || (MT <= 2 && XF), "the fused merge serves batches 1 and 2 with fp32 activations");
  if constexpr (XT) {
    if ((int)blockIdx.x < p.mrg_blocks) {
      fused_merge(p);
      return;
    }
  }
  const int W = p.wpg;
  const int K = p.K;
  const int nb = K / kBlock;
  const int ng = (nb + kBatch - 1) / kBatch;
  const int M = p.M;
  int tile, kg;
  if (!split_role(p.ntiles, p.wpt, tile, kg, XT ? (int)blockIdx.x - p.mrg_blocks : (int)blockIdx.x)) return;
  const int w = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const int e0 = kg * W * kBatch * kBlock;          // first K element of this workgroup

  // activation slice first (its loads return before the weights), 4 elements per thread per row;
  // with XT it is polled after the weight loads instead (it is still being merged)
  static_assert(kItemK == 4 * 64 * WMAX, "one 4-element activation load per thread covers the slice");
  const int ec = min(e0 + 4 * (int)threadIdx.x, K - 4);
  float4 xf[MT];
  uint2 xr[MT];
  if constexpr (!XT) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const size_t off = (size_t)min(m, M - 1) * K + ec;
      if constexpr (XF) xf[m] = *reinterpret_cast<const float4*>(static_cast<const float*>(xin) + off);
      else xr[m] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(xin) + off);
    }
  }
  EpiPre<MT> ep;
  epi_prefetch<MT, EPI>(p, tile, lane, ep);

  // this wave's group: 8 blocks and their 8 scales
  const int grp = kg * W + w;
  const int b0 = grp * kBatch;
  const int nblk = min(max(nb - b0, 0), kBatch);
  const u32x4* qt = reinterpret_cast<const u32x4*>(qw) + (size_t)tile * nb * kTileRows + lane;
  // scales first: block 0 needs them, and loads complete in order
  const u32x4 sv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sw) +
                                              ((size_t)tile * ng + min(grp, ng - 1)) * kTileRows + lane);
  u32x4 wv[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) wv[i] = __builtin_nontemporal_load(qt + (size_t)min(b0 + i, nb - 1) * kTileRows);
  // keep the LDS write of the activations behind the weight loads (its wait would hold them back)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XT) {
    // the merged attention output of this step and layer: 4 tagged words per thread and row
    // (bounded wait)
    const uint32_t tag = p.epoch[0] * p.tag_mul + p.tag_add;
    uint64_t t[MT][4];
    for (uint32_t it = 0;; ++it) {
      bool ok = true;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          t[m][k] = collect_u64(p.xtag + (size_t)min(m, M - 1) * K + ec + k);
          ok = ok && (uint32_t)(t[m][k] >> 32) == tag;
        }
      if (__all(ok)) break;
      if (it >= kSpinLimit) {
        if (p.status) __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int k = 0; k < 4; ++k) t[m][k] = 0x7fc00000u;     // fp32 NaN
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xf[m] = make_float4(__uint_as_float((uint32_t)t[m][0]), __uint_as_float((uint32_t)t[m][1]),
                          __uint_as_float((uint32_t)t[m][2]), __uint_as_float((uint32_t)t[m][3]));
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if constexpr (XF)   // 8 consecutive threads hold one block
      stage_digits(xf[m], &xd[m][((int)threadIdx.x / 8) * kDigitDwords]);
    else
      *reinterpret_cast<uint2*>(&xs[m][4 * threadIdx.x]) = xr[m];
  }
  __syncthreads();

  const int xb0 = w * kBatch * kBlock;              // this wave's first element in the slice
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  if constexpr (XF) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float sc = i < nblk ? pick_scale(sv, i) : 0.f;
      const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
      uint32_t lo[4], hi[4];
      codes_to_bytes(d, lo, hi);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m] = fmaf(sc, block_dot_digits(lo, hi, &xd[m][(xb0 / kBlock + i) * kDigitDwords]), acc[m]);
    }
  } else {
    const uint32_t m64 = vconst(0x54005400u);
    float corr[MT];   // the offset correction of the fp16 pairs, lane 4i + q: quarter q of block i
#pragma unroll
    for (int m = 0; m < MT; ++m)
      corr[m] = quad_sum(corr_quarter(*reinterpret_cast<const u32x4*>(&xs[m][xb0 + min(lane, 4 * kBatch - 1) * 8])));
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float sc = i < nblk ? pick_scale(sv, i) : 0.f;
      const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
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

#pragma unroll
  for (int m = 0; m < MT; ++m) red[w][m][lane] = acc[m];
  __syncthreads();
  if (w != 0) return;
  epi_finish<MT, EPI>(p, tile, lane, ep);

  float tot[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float t = 0.f;
    for (int v = 0; v < W; ++v) t += red[v][m][lane];
    tot[m] = t;
  }
  if (p.wpt == 1) {
    epilogue<MT, EPI>(p, tile, tot, ep, lane);
    return;
  }
  // writers: tagged partial into the tile's slot kg, then done; the reader (kg = wpt - 1) adds them
  const int nw = p.wpt - 1;
  uint64_t* sl = p.slots + (size_t)tile * nw * MT * kTileRows;
  if (kg < nw) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M) slot_store(&sl[((size_t)kg * MT + m) * kTileRows + lane], kFresh | __float_as_uint(tot[m]));
    return;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= M) continue;
    tot[m] = poll_sum(sl + (size_t)m * kTileRows + lane, nw, (size_t)MT * kTileRows, p.status) + tot[m];
  }
  epilogue<MT, EPI>(p, tile, tot, ep, lane);
}

int mt_of(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// Batches of at least kGemvMfmaMinM rows go to the matrix-core kernel (gemv_mfma.hip), which
// always computes 16 rows: its partials are sized for 16.
constexpr int kMfmaMinM = kGemvMfmaMinM;
int part_rows(int M) { return M >= kMfmaMinM ? 16 : mt_of(M); }

struct Plan { int kb, wpg, wpt, grid; };

// One 8-block group (one batch: 8 weight loads + 1 scale load, all in flight at once) per wave.
// The groups of a tile are spread evenly over wpt = ceil(groups / wmax) workgroups of at most
// wmax waves (8 or 4, see kWideMinWgs; 4 for batches > 2, whose LDS holds M slices); a tile of
// <= wmax groups is one workgroup and needs no cross-workgroup reduction.
Plan make_plan(int M, int ntiles, int nb) {
  const int ng = (int)cdiv(nb, kBatch);
  const int wmax = M <= 2 && (int64_t)ntiles * cdiv(ng, kWavesSmallM) >= kWideMinWgs ? kWavesSmallM : kWavesLargeM;
  Plan pl;
  pl.kb = kBatch;
  pl.wpt = (int)cdiv(ng, wmax);
  pl.wpg = (int)cdiv(ng, pl.wpt);
  pl.grid = (int)(cdiv(ntiles, kNumXcd) * kNumXcd * pl.wpt);
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

// Workspace: hand-off slots of the VALU kernel [tile][wpt - 1][MT][64], then the partials
// [tile][wpt][16][64] and arrival counters [tile] of the matrix-core kernel.  The regions are
// separate, so one workspace serves every batch size.
namespace {
struct WsParts { size_t slots, part, cnt; };
WsParts ws_parts(int M, int ntiles, int nb) {
  const Plan pl = make_plan(M, ntiles, nb);
  const int MT = part_rows(M);
  WsParts w;
  w.slots = align_up((size_t)ntiles * (pl.wpt - 1) * MT * kTileRows * sizeof(uint64_t), 256);
  w.part = align_up((size_t)ntiles * pl.wpt * MT * kTileRows * sizeof(float), 256);
  w.cnt = align_up((size_t)ntiles * sizeof(unsigned), 256);
  return w;
}
}  // namespace

size_t gemv_workspace_bytes(int M, int ntiles, int nb) {
  const WsParts w = ws_parts(M, ntiles, nb);
  return w.slots + w.part + w.cnt;
}

void gemv_set_workspace(GemvParams& p, void* ws) {
  const WsParts w = ws_parts(p.M, p.ntiles, p.K / kBlock);
  char* c = static_cast<char*>(ws);
  p.slots = reinterpret_cast<uint64_t*>(c);
  p.part = reinterpret_cast<float*>(c + w.slots);
  p.cnt = reinterpret_cast<unsigned*>(c + w.slots + w.part);
}

namespace {
template <int EPI, bool XF>
void launch_epi(const GemvParams& p, const uint4* q, const uint4* s, hipStream_t st, KEv ev) {
  const dim3 g(p.grid + p.mrg_blocks), b(64 * p.wpg);
  const bool wide = p.wpg > kWavesLargeM;   // only batches <= 2 get 8-wave workgroups
  switch (mt_of(p.M)) {
    case 1:
      if constexpr (EPI == EPI_RESID && XF) {   // the o projection may take the fused merge
        if (p.mrg_blocks) {
          if (wide) VV_LAUNCH((k_gemv<1, EPI, kWavesSmallM, true, true>), g, b, st, ev, p, q, s, p.x);
          else VV_LAUNCH((k_gemv<1, EPI, kWavesLargeM, true, true>), g, b, st, ev, p, q, s, p.x);
          break;
        }
      }
      if (wide) VV_LAUNCH((k_gemv<1, EPI, kWavesSmallM, false, XF>), g, b, st, ev, p, q, s, p.x);
      else VV_LAUNCH((k_gemv<1, EPI, kWavesLargeM, false, XF>), g, b, st, ev, p, q, s, p.x);
      break;
    case 2:
      if constexpr (EPI == EPI_RESID && XF) {   // the o projection may take the fused merge
        if (p.mrg_blocks) {
          if (wide) VV_LAUNCH((k_gemv<2, EPI, kWavesSmallM, true, true>), g, b, st, ev, p, q, s, p.x);
          else VV_LAUNCH((k_gemv<2, EPI, kWavesLargeM, true, true>), g, b, st, ev, p, q, s, p.x);
          break;
        }
      }
      if (wide) VV_LAUNCH((k_gemv<2, EPI, kWavesSmallM, false, XF>), g, b, st, ev, p, q, s, p.x);
      else VV_LAUNCH((k_gemv<2, EPI, kWavesLargeM, false, XF>), g, b, st, ev, p, q, s, p.x);
      break;
    default: VV_LAUNCH((k_gemv<4, EPI, kWavesLargeM, false, XF>), g, b, st, ev, p, q, s, p.x); break;
  }
}

}  // namespace

hipError_t gemv_launch(const GemvParams& p0, hipStream_t st, KEv ev) {
  if (p0.M >= kMfmaMinM) return gemv_mfma_launch(p0, st, ev);
  GemvParams p = p0;
  const uint16_t* any = static_cast<const uint16_t*>(p.x);   // readable stand-in for absent operands
  p.rs_mask = p.rs_parts ? 1 : 0;
  if (!p.rs_parts) { p.rs_parts = reinterpret_cast<const float*>(any); p.rs_nparts = 0; }
  p.has_bias = p.bias ? 1 : 0;
  if (!p.bias) p.bias = any;
  p.has_gamma = p.gamma ? 1 : 0;
  if (!p.gamma) p.gamma = any;
  const uint4* q = reinterpret_cast<const uint4*>(p.q);
  const uint4* s = reinterpret_cast<const uint4*>(p.s);
  if (!p.x_f32) {   // fp16 activations: the stand-alone GEMV of the C ABI
    if (p.epi != EPI_STORE) return hipErrorInvalidValue;
    launch_epi<EPI_STORE, false>(p, q, s, st, ev);
    return hipGetLastError();
  }
  switch (p.epi) {
    case EPI_STORE: launch_epi<EPI_STORE, true>(p, q, s, st, ev); break;
    case EPI_RESID: launch_epi<EPI_RESID, true>(p, q, s, st, ev); break;
    default: launch_epi<EPI_SILU, true>(p, q, s, st, ev); break;
  }
  return hipGetLastError();
}

}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_gemv_int4_workspace(int64_t M, int64_t N, int64_t K, int layout) {
  if (M < 1 || M > 16 || N < 1 || K < kBlock || K % kBlock) return 0;
  if (layout == VV_LAYOUT_ROWMAJOR) return 256;   // the row-major kernel uses none of it
  if (layout != VV_LAYOUT_TILED) return 0;
  return gemv_workspace_bytes((int)M, (int)cdiv(N, kTileRows), (int)(K / kBlock));
}

int vv_gemv_int4(const uint8_t* packed, const uint16_t* scales, const uint16_t* bias, const uint16_t* x, int64_t M,
                 int64_t N, int64_t K, int layout, void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  VV_REQUIRE(packed && scales && x && y, VV_ERR_NULL, "vv_gemv_int4: NULL pointer");
  VV_REQUIRE(M >= 1 && M <= 16, VV_ERR_RANGE, "vv_gemv_int4: M = %lld not in 1..16", (long long)M);
  VV_REQUIRE(N >= 1 && N <= (1 << 26), VV_ERR_RANGE, "vv_gemv_int4: N = %lld out of range", (long long)N);
  VV_REQUIRE(K >= kBlock && K % kBlock == 0 && K <= (1 << 22), VV_ERR_SHAPE,
             "vv_gemv_int4: K = %lld is not a positive multiple of 32 (<= 4M)", (long long)K);
  VV_REQUIRE(layout == VV_LAYOUT_ROWMAJOR || layout == VV_LAYOUT_TILED, VV_ERR_DTYPE,
             "vv_gemv_int4: unknown layout %d", layout);
  VV_REQUIRE(y_dtype == VV_F16 || y_dtype == VV_F32, VV_ERR_DTYPE, "vv_gemv_int4: unknown y dtype %d", y_dtype);
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(x)) & 15) == 0 &&
                 (reinterpret_cast<uintptr_t>(scales) & (layout == VV_LAYOUT_TILED ? 15 : 1)) == 0,
             VV_ERR_RANGE, "vv_gemv_int4: packed and x must be 16-byte aligned (tiled scales too, row-major 2)");
  const size_t need = vv_gemv_int4_workspace(M, N, K, layout);
  VV_REQUIRE(ws && ws_bytes >= need, VV_ERR_WORKSPACE, "vv_gemv_int4: workspace needs %zu bytes", need);
  if (layout == VV_LAYOUT_ROWMAJOR) {
    VV_HIP(gemv_rowmajor_launch(packed, scales, bias, x, (int)M, (int)N, (int)K, y, y_dtype == VV_F16,
                                as_stream(stream)));
    return VV_OK;
  }
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
