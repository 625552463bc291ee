// Chained launches of the batch-1 decode step: the GEMV stages of a layer run as segments of one
// grid, so that each stage's weight stream starts while its predecessor is still finishing.
//
// The decoder_step contract ("vibevoice-asr-bitnet-onnx" page, graph contracts) on the Qwen2 layer
// of the 1.5B STATUS page (Architecture): pre-RMSNorm, q/k/v bias, GQA, SiLU-gated MLP, residual
// adds, with the int4 block-32 MatMulNBits projections of the same page.  At batch 1 a layer is
// ~140 MB of weights against a handful of dependent stages, and a kernel boundary costs about
// 2 us of idle HBM (the ramp of the next grid and the tail of the last one), so the step runs as
//   launch 0:      [prep | q|k|v of layer 0]
//   per layer l:   attention(l)   (its own launch: RoPE, KV append, split records)
//                  [merge(l) | o(l)]
//                  [gate/up(l) | down(l) | q|k|v(l+1)]   (wide models: [gate/up(l)], then
//                                                         [down(l) | q|k|v(l+1)])
//   then the lm_head + argmax.
// The layered step borrows the [down(l) | q|k|v(l+1)] launch at batch 1, with down reading plain
// inputs written before the launch.
// (One launch for all five stages of a layer is slower: the MLP's waves, dispatched with the
// merge and o, hold their places while they wait, and their first reads of the MLP input miss.)
// A segment's workgroups read their inputs once, issue their weight loads, and then wait for any
// input that was not there yet.  Earlier segments (of the same grid or an earlier launch) publish
// them as 64-bit tagged words: a 32-bit tag (the step counter times a stride, plus the layer and
// stage) and an fp32 payload (the activations keep fp32 precision; the GEMV segments stage them as
// 8-bit digit images).  A word is stored once per step with a single atomic store, so a reader
// that sees the expected tag sees the value, and no word ever needs clearing (a stale word carries
// an older tag).  Progress: a workgroup only waits for workgroups with smaller indices (earlier
// segments, and within a segment the split-K writers dispatched before their reader on the same
// XCD) or of an earlier launch, and each XCD dispatches its workgroups in increasing index, so the
// smallest unfinished workgroup always runs to completion.  Every wait is bounded: one that gives
// up sets the step's status word and continues with NaN instead of hanging.
#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kCW = kChainWaves;           // waves per workgroup
constexpr int kCT = kCW * kWave;           // threads per workgroup
constexpr int kCItemK = kCW * 8 * kBlock;  // K elements per workgroup at most (8 groups of 8 blocks)

union CLds {
  struct { uint32_t xd[kCItemK / kBlock * kDigitDwords]; float red[kCW][kWave]; } g;   // xd: digit images
  struct { float pm[kCW], pl[kCW]; float po[kCW][kWave]; } m;
};

__device__ __forceinline__ uint64_t tag_f32(uint32_t tag, float v) {
  return ((uint64_t)tag << 32) | __float_as_uint(v);
}
__device__ __forceinline__ bool has_tag(uint64_t v, uint32_t tag) { return (uint32_t)(v >> 32) == tag; }
__device__ __forceinline__ void give_up(int32_t* status) {
  __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every lane of the wave reloads its word until all carry `tag` (bounded); returns the word
__device__ __forceinline__ uint64_t wait_word(const uint64_t* p, uint64_t v, uint32_t tag, int32_t* status) {
  for (uint32_t it = 0; !__all(has_tag(v, tag)); ++it) {
    if (it >= kSpinLimit) {
      give_up(status);
      return tag_f32(tag, __builtin_nanf(""));
    }
    __builtin_amdgcn_s_sleep(2);
    v = collect_u64(p);
  }
  return v;
}

// ---- prep: embeddings -> residual stream (layer 0's input), RMSNorm_1 numerator, sum(h^2) per
// tile, the RoPE table of the new position ----------------------------------------------------
__device__ void seg_prep(const ChainParams& P, int bid, uint32_t ebase) {
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int t = bid * kCW + w;
  const uint32_t tag = ebase + P.prep_add;
  if (t < P.H / kTileRows) {
    const int n = t * kTileRows + lane;
    const float hv = h2f(P.emb[n]);
    publish_u64(P.h + n, tag_f32(tag, hv));
    if (P.trace0) P.trace0[n] = hv;
    publish_u64(P.xq + n, tag_f32(tag, h2f(P.g1[n]) * hv));
    const float ss = wave_sum(hv * hv);
    if (lane == 0) publish_u64(P.ssq + t, tag_f32(tag, ss));
  }
  if (bid == 0 && w == 0 && P.rope_on) {
    // angle pos * theta^(-2i/128) (the inverse frequency computed on the host in fp64), reduced in
    // fp64 to a fraction of a turn in [-1/2, 1/2]; cos and sin of that fraction come from the
    // hardware's turn-based v_cos_f32 / v_sin_f32 (absolute error ~1e-6 for these arguments)
    int pp = P.pos[0];
    pp = pp < 0 ? 0 : (pp >= P.cap ? P.cap - 1 : pp);
    const double turns = (double)pp * P.inv_freq[lane] * 0.15915494309189535;   // 1 / (2 pi)
    const float f = (float)(turns - rint(turns));
    P.rope[lane * 2] = __builtin_amdgcn_cosf(f);
    P.rope[lane * 2 + 1] = __builtin_amdgcn_sinf(f);
  }
}

// ---- merge of the attention's split records: one workgroup per query head; waves 0-3 take dims
// 0-63 and waves 4-7 dims 64-127, wave w & 3 splits 32 (w & 3) .. + 31 (all 32 record loads of a
// lane in flight at once); the four quarters of each half meet in LDS ---------------------------
__device__ void seg_merge(const ChainParams& P, int bid, uint32_t ebase, CLds& L) {
  const int h = bid;
  if (h >= P.nq) return;
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int half = w >> 2, qt = w & 3;
  const int g = P.nq / P.nkv, kvh = h / g, hh = h % g;
  const int n = attn_splits(P.pos, nullptr, 0, P.cap, P.split);
  const int d = 64 * half + lane;
  const float* rec0 = P.part + ((size_t)kvh * P.nsplit * kAttnMaxG + hh) * kAttnRec;
  const size_t stride = (size_t)kAttnMaxG * kAttnRec;
  const int s0 = 32 * qt;
  float v[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) v[u] = rec0[(size_t)min(s0 + u, n - 1) * stride + 4 + d];
  const int sl = min(s0 + (lane & 31), n - 1);
  const float ms = rec0[(size_t)sl * stride], ls = rec0[(size_t)sl * stride + 1];
  const bool mine = lane < 32 && s0 + lane < n;
  const float Mw = wave_max(mine ? ms : -INFINITY);
  const float e = mine ? expf(ms - Mw) : 0.f;
  const float Lw = wave_sum(mine ? e * ls : 0.f);
  float Ow = 0.f;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const float eu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), u));
    Ow = fmaf(eu, v[u], Ow);              // e_u = 0 past the quarter's last split
  }
  if (lane == 0) {
    L.m.pm[w] = Mw;
    L.m.pl[w] = Lw;
  }
  L.m.po[w][lane] = Ow;
  __syncthreads();
  if (qt != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) M = fmaxf(M, L.m.pm[w + k]);    // finite: quarter 0 holds split 0
  float O = 0.f, Ls = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float pmk = L.m.pm[w + k];
    const float f = pmk == -INFINITY ? 0.f : expf(pmk - M);   // a quarter past the sequence: 0
    O = fmaf(f, L.m.po[w + k][lane], O);
    Ls = fmaf(f, L.m.pl[w + k], Ls);
  }
  publish_u64(P.xo + (size_t)h * 128 + d, tag_f32(ebase + P.mrg_add, O / Ls));
}

// ---- one GEMV segment (batch 1): the decomposition, dequantisation and split-K hand-off of the
// layered GEMV kernel, with tagged inputs and outputs --------------------------------------------
// PLAIN (EPI_RESID only): the input and the residual are plain fp32 written before this launch
template <int EPI, bool PLAIN = false>
__device__ void seg_gemv(const ChainParams& P, const CSeg& g, int bid, uint32_t ebase, CLds& L) {
  static_assert(!PLAIN || EPI == EPI_RESID, "plain inputs: the residual segment after a kernel boundary");
  const int K = g.K, nb = K / kBlock, ng = (nb + 7) / 8, W = g.wpg;
  int tile, kg;
  if (!split_role(g.ntiles, g.wpt, tile, kg, bid)) return;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int e0 = kg * W * 8 * kBlock;
  const bool active = w < W;

  // epilogue operands, loaded before the weights (their tags are checked where they are used)
  const int n = EPI == EPI_SILU ? tile * 32 + (lane & 31) : tile * kTileRows + lane;
  const int nc = min(n, g.N - 1);
  uint64_t ssv = 0, hv = 0;
  if (EPI != EPI_RESID) ssv = peek_u64(g.ssin + min(lane, g.ss_n - 1));
  if (EPI == EPI_RESID) hv = PLAIN ? (uint64_t)__float_as_uint(g.hp[nc]) : peek_u64(P.h + nc);
  const uint32_t p16 = EPI == EPI_STORE ? g.bias[nc * g.has_bias] : EPI == EPI_RESID ? g.gamma[nc] : 0u;

  // this wave's group: 8 blocks and their 8 scales (scales first: block 0 needs them).  No load
  // sits behind a branch (a load whose result merges with a default at a join makes the compiler
  // wait for every load issued so far): a wave past the workgroup's W groups re-reads the last
  // block of the group before it, 1 KiB that its neighbour is fetching anyway, and gets scale 0.
  // The activation slice: four tagged fp32 words per thread, read once (cached) before the
  // weight loads, so that checking them waits for nothing else (vector loads complete in order,
  // and a check behind the weight loads would hold the digit staging until the whole group had
  // arrived); polled, behind the weights, only if a tag was not there yet.
  const int ec = min(e0 + 4 * tid, K - 4);
  const uint32_t xtag = ebase + g.xin_add;
  const uint64_t* xp = g.xin + ec;
  uint64_t t[4];
  if constexpr (PLAIN) {
    const float4 xv = *reinterpret_cast<const float4*>(g.xp + ec);
    t[0] = tag_f32(xtag, xv.x); t[1] = tag_f32(xtag, xv.y); t[2] = tag_f32(xtag, xv.z); t[3] = tag_f32(xtag, xv.w);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = peek_u64(xp + k);
  }

  const int grp = kg * W + min(w, W - 1);
  const int b0 = active ? grp * 8 : min(grp * 8 + 7, nb - 1);
  const int bstep = active ? 1 : 0;
  const int nblk = active ? min(max(nb - b0, 0), 8) : 0;
  const u32x4* qt = g.q + (size_t)tile * nb * kTileRows + lane;
  const u32x4 sv = __builtin_nontemporal_load(g.s + ((size_t)tile * ng + min(grp, ng - 1)) * kTileRows + lane);
  u32x4 wv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    wv[i] = __builtin_nontemporal_load(qt + (size_t)min(b0 + bstep * i, nb - 1) * kTileRows);
  __builtin_amdgcn_sched_barrier(0);

  // Poll until every tag is there, then stage the slice in LDS as the digit images of its
  // 32-element blocks.  (Waiting on a few summary words per producer instead, and reading the
  // slice once after them, measured slower: the extra round trip lands on every hop.)
  // The first check stays outside the loop: a check shared with the loop's re-reads would wait
  // as if the words had been loaded last.
  if (!__all(has_tag(t[0], xtag) && has_tag(t[1], xtag) && has_tag(t[2], xtag) && has_tag(t[3], xtag))) {
    for (uint32_t it = 0;; ++it) {
      if (it >= kSpinLimit) {
        give_up(P.status);
#pragma unroll
        for (int k = 0; k < 4; ++k) t[k] = 0x7fc00000u;   // fp32 NaN
        break;
      }
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int k = 0; k < 4; ++k) t[k] = collect_u64(xp + k);
      if (__all(has_tag(t[0], xtag) && has_tag(t[1], xtag) && has_tag(t[2], xtag) && has_tag(t[3], xtag))) break;
    }
  }
  stage_digits(make_float4(__uint_as_float((uint32_t)t[0]), __uint_as_float((uint32_t)t[1]),
                           __uint_as_float((uint32_t)t[2]), __uint_as_float((uint32_t)t[3])),
               &L.g.xd[(tid / 8) * kDigitDwords]);
  __syncthreads();

  float acc = 0.f;
  {
    const int xb0 = w * 8;                          // this wave's first block in the slice
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sc = i < nblk ? pick_scale(sv, i) : 0.f;
      const uint32_t dw[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
      uint32_t lo[4], hi[4];
      codes_to_bytes(dw, lo, hi);
      acc = fmaf(sc, block_dot_digits(lo, hi, &L.g.xd[(xb0 + i) * kDigitDwords]), acc);
    }
  }
  L.g.red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  float tot = 0.f;
  for (int v = 0; v < W; ++v) tot += L.g.red[v][lane];
  if (g.wpt > 1) {
    const int nw = g.wpt - 1;
    uint64_t* sl = g.slots + (size_t)tile * nw * kTileRows;
    if (kg < nw) {   // writer: tagged partial into the tile's slot kg, then done
      slot_store(&sl[(size_t)kg * kTileRows + lane], kFresh | __float_as_uint(tot));
      return;
    }
    tot = poll_sum(sl + lane, nw, kTileRows, P.status) + tot;
  }

  const uint32_t otag = ebase + g.out_add;
  if (EPI == EPI_STORE || EPI == EPI_SILU) {
    ssv = wait_word(g.ssin + min(lane, g.ss_n - 1), ssv, ebase + g.ss_add, P.status);
    const float part = lane < g.ss_n ? __uint_as_float((uint32_t)ssv) : 0.f;
    const float rs = 1.0f / sqrtf(wave_sum(part) * P.inv_h + P.eps);
    if (EPI == EPI_STORE) {
      const float bias = g.has_bias ? h2f((uint16_t)p16) : 0.f;
      if (n < g.N) g.y[n] = tot * rs + bias;
    } else {   // lanes 0-31: gate rows, 32-63: the same up rows
      const float gt = tot * rs;
      const float u = __shfl(tot, (lane & 31) + 32, kWave) * rs;
      if (lane < 32 && n < g.N) publish_u64(g.act + n, tag_f32(otag, silu(gt) * u));
    }
  } else {   // EPI_RESID: h += tot; the next norm's numerator and sum(h^2) of the tile
    if constexpr (!PLAIN) hv = wait_word(P.h + nc, hv, ebase + g.hin_add, P.status);
    const float hn = __uint_as_float((uint32_t)hv) + tot;
    if constexpr (PLAIN) {
      if (n < g.N) g.hp[n] = hn;
    } else {
      publish_u64(P.h + n, tag_f32(otag, hn));
    }
    if (g.trace) g.trace[n] = hn;
    const float gv = h2f((uint16_t)p16) * hn;
    if (g.gf) g.gf[n] = gv;
    const float ss = wave_sum(hn * hn);
    if (g.sumsq && lane == 0) g.sumsq[tile] = ss;
    if (g.xgout) {
      publish_u64(g.xgout + n, tag_f32(otag, gv));
      if (lane == 0) publish_u64(g.ssout + tile, tag_f32(otag, ss));
    }
  }
}

// 8 waves per SIMD (at most 64 VGPRs): the weight streams of the GEMV segments need the
// occupancy.  One instance per launch, with its segments at fixed positions (so every segment
// field is read at a constant offset): CH_FIRST prep, q|k|v; CH_MO merge, o; CH_MLP gate/up,
// down and, if nseg == 3, the next layer's q|k|v; CH_GU gate/up alone; CH_DQ down and, if
// nseg == 2, the next layer's q|k|v; CH_LDQ the same with down's input and residual plain fp32
// (the layered plan's batch-1 launch).
template <int KIND>
__global__ __launch_bounds__(kCT, 8) void k_chain(ChainParams P) {
  __shared__ CLds L;
  const uint32_t ebase = P.epoch[0] * P.tag_mul;
  int b = blockIdx.x;
  if (b < P.seg[0].blocks) {
    if constexpr (KIND == CH_FIRST) seg_prep(P, b, ebase);
    else if constexpr (KIND == CH_MO) seg_merge(P, b, ebase, L);
    else if constexpr (KIND == CH_DQ) seg_gemv<EPI_RESID>(P, P.seg[0], b, ebase, L);
    else if constexpr (KIND == CH_LDQ) seg_gemv<EPI_RESID, true>(P, P.seg[0], b, ebase, L);
    else seg_gemv<EPI_SILU>(P, P.seg[0], b, ebase, L);
    return;
  }
  if constexpr (KIND == CH_GU) return;
  b -= P.seg[0].blocks;
  if constexpr (KIND == CH_FIRST) {
    seg_gemv<EPI_STORE>(P, P.seg[1], b, ebase, L);
  } else if constexpr (KIND == CH_MO) {
    seg_gemv<EPI_RESID>(P, P.seg[1], b, ebase, L);
  } else if constexpr (KIND == CH_DQ || KIND == CH_LDQ) {
    if (P.nseg > 1) seg_gemv<EPI_STORE>(P, P.seg[1], b, ebase, L);
  } else {
    if (b < P.seg[1].blocks) {
      seg_gemv<EPI_RESID>(P, P.seg[1], b, ebase, L);
      return;
    }
    b -= P.seg[1].blocks;
    if (P.nseg > 2) seg_gemv<EPI_STORE>(P, P.seg[2], b, ebase, L);
  }
}

}  // namespace

void chain_gemv_plan(CSeg& g) {
  const int nb = g.K / kBlock;
  const int ng = (nb + 7) / 8;
  g.wpt = (ng + kCW - 1) / kCW;
  g.wpg = (ng + g.wpt - 1) / g.wpt;
  g.blocks = (int)(cdiv(g.ntiles, kNumXcd) * kNumXcd * g.wpt);
}

hipError_t chain_launch(const ChainParams& P, hipStream_t st, KEv ev) {
  int grid = 0;
  for (int i = 0; i < P.nseg; ++i) grid += P.seg[i].blocks;
  const int k0 = P.seg[0].kind, k1 = P.nseg > 1 ? P.seg[1].kind : -1;
  if (k0 == SEG_PREP && P.nseg == 2 && k1 == SEG_QKV)
    VV_LAUNCH((k_chain<CH_FIRST>), dim3(grid), dim3(kCT), st, ev, P);
  else if (k0 == SEG_MERGE && P.nseg == 2 && k1 == SEG_O)
    VV_LAUNCH((k_chain<CH_MO>), dim3(grid), dim3(kCT), st, ev, P);
  else if (k0 == SEG_GU && k1 == SEG_DOWN && (P.nseg == 2 || (P.nseg == 3 && P.seg[2].kind == SEG_QKV)))
    VV_LAUNCH((k_chain<CH_MLP>), dim3(grid), dim3(kCT), st, ev, P);
  else if (k0 == SEG_GU && P.nseg == 1)   // alone in its launch: exactly the waves of its groups
    VV_LAUNCH((k_chain<CH_GU>), dim3(grid), dim3(kWave * P.seg[0].wpg), st, ev, P);
  else if (k0 == SEG_DOWN && (P.nseg == 1 || (P.nseg == 2 && k1 == SEG_QKV)) && P.seg[0].xp)
    VV_LAUNCH((k_chain<CH_LDQ>), dim3(grid), dim3(kCT), st, ev, P);
  else if (k0 == SEG_DOWN && (P.nseg == 1 || (P.nseg == 2 && k1 == SEG_QKV)))
    VV_LAUNCH((k_chain<CH_DQ>), dim3(grid), dim3(kCT), st, ev, P);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vv
