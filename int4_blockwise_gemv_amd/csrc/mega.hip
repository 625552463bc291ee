// Single-launch decode step: every layer of one decode step in one kernel launch.
//
// The step is the decoder_step contract of the "vibevoice-asr-bitnet-onnx" page (graph
// contracts: input_embeds and position_ids in, logits and one more K/V slot out) on the Qwen2
// layer of the 1.5B STATUS page (Architecture): pre-RMSNorm, q/k/v bias, grouped-query
// attention, SiLU-gated MLP, residual adds; projections are int4 block-32 MatMulNBits with
// float activations (same page, quantisation section).
//
// Why one launch: at batch 1 a 28-layer step is ~170 dependent stages of a few MB each.  As
// separate kernels each stage pays its dispatch ramp, first-byte latency and reduction tail
// with the HBM idle meanwhile (a few µs per kernel, comparable to the streaming time).  Here the
// whole step is one grid whose workgroups are the work items, numbered in dependency order:
//   PREP                             embeddings -> residual stream, RoPE table
//   per layer:
//   Q  (tile, K-split) of the fused q|k|v GEMV: RMSNorm_1 folded in, bias added
//   A  (sequence, KV head, 64 positions) of attention: RoPE, KV append, split softmax
//   M  (sequence, query head): merge of the attention splits
//   O  (tile, K-split) of the o GEMV + residual (writes RMSNorm_2's input)
//   G  (tile, K-split) of the gate/up GEMV + SiLU(gate)*up (RMSNorm_2 folded in)
//   D  (tile, K-split) of the down GEMV + residual (writes the next layer's RMSNorm_1 input)
// A workgroup issues the loads that do not depend on activations (its weights, its K/V rows)
// first, then polls the counter of the phase it consumes, then computes and hands its result
// on.  Workgroups waiting for a phase thus keep their weights in flight, the dispatcher refills
// slots as workgroups finish, and the HBM streams through the hand-offs.
//
// Progress: an item only waits for items with smaller indices.  Workgroups are dispatched in
// increasing index within each XCD, so the smallest unfinished item is always dispatched and
// its inputs are complete: it finishes, whatever the residency.  Each wait is bounded anyway:
// a wait that gives up sets a sticky status word (and records the item, the counter value and
// the target in the three words after it) instead of hanging.
//
// Hand-offs: a K-split partial is an agent-scope store; the workgroup then counts itself in at
// its tile, and the last one adds the partials in split order (deterministic) and runs the
// epilogue; a finished tile or item counts itself in at its phase.  Activations that are read
// with plain (cacheable) loads are written exactly once per launch into per-layer buffers, so no
// cache can hold a stale copy; everything else produced inside the launch is read with
// agent-scope loads.  The counters are cleared by a fill kernel before each launch.
#include <algorithm>

#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kW = 4;               // waves per workgroup
constexpr int kThr = kW * kWave;    // threads per workgroup
constexpr int kGB = 8;              // blocks per wave (one 16-byte scale group)
constexpr int kItemK = kW * kGB * kBlock;   // K elements per GEMV item (1024)
constexpr int kD = 128;             // head_dim
constexpr int kAS = 64;             // attention positions per item (16 per wave)
constexpr int kPS = 132;            // attention record per head: m, l, pad, pad, o[128]
constexpr int kMaxG = 8;            // query heads per KV head
constexpr int kMaxL = 32;           // layers per launch (kernel-argument table)
constexpr int kMaxMT = 1;           // batch rows handled by this path
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kPad = 32;            // u32 per phase counter (own 128-byte line)

enum Phase { PH_PREP = 0, PH_Q, PH_A, PH_M, PH_O, PH_G, PH_D };


struct MLayer {
  const u32x4* qkv_q; const u32x4* qkv_s;
  const u32x4* o_q;   const u32x4* o_s;
  const u32x4* gu_q;  const u32x4* gu_s;
  const u32x4* dn_q;  const u32x4* dn_s;
  const uint16_t* bias; const uint16_t* g1; const uint16_t* g2;
};

struct MParams {
  int L, l0, l1, B, H, I, nq, nkv, g, cap, nqkv, ntH;
  float eps, inv_h, scale, theta;
  const uint16_t* emb; const int32_t* pos;
  uint16_t* kc; uint16_t* vc; size_t kv_layer;     // cache elements per layer
  const uint16_t* gf; float* trace;
  const uint16_t* g1_next;                         // RMSNorm_1 weight of layer l1 (next launch)
  int ntq, ntg;                                    // tiles of q|k|v and of gate/up (o, down: ntH)
  int nbq, nbo, nbg, nbd;                          // blocks along K
  int nsq, nso, nsg, nsd, nsa;                     // items per tile / per (sequence, KV head)
  int nQ, nA, nM, nO, nG, nD, T, total;
  // workspace
  unsigned* err; unsigned* c_prep;
  unsigned* cnt; int cpl;                          // counters, cpl per layer
  int k_cq, k_co, k_cg, k_cd, k_ca, k_dq, k_dm, k_do, k_dg, k_dd;
  float* rope; float* gfo;
  float* ssi; float* ssm; float* hin; float* h1; float* qkv; float* ap;
  float* pq; float* po; float* pg; float* pd;
  uint16_t* xq; uint16_t* xm; uint16_t* ao; uint16_t* act;   // per layer (write-once)
  size_t xq_l, xm_l, ao_l, act_l;                  // elements per layer
  MLayer lw[kMaxL];
};

struct Item { int layer, phase, j; };

// LDS of the item kinds, overlaid (a workgroup runs one item)
union Lds {
  struct { uint16_t xs[kMaxMT][kItemK]; float red[kW][kMaxMT][kWave]; } gemv;
  struct {
    float qs[kMaxG][kD]; float sc[kMaxG][kAS]; float red[kW][kMaxG][kD];
    uint16_t knew[kD], vnew[kD]; float mh[kMaxG], lh[kMaxG];
  } attn;
  struct { float ms[1024], ws[1024]; float part[2][kD]; float Ls; } merge;
};

__device__ __forceinline__ void publish_u16(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned peek(const unsigned* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Item decode(const MParams& p, int i) {
  Item it{0, PH_PREP, 0};
  if (p.l0 == 0) {
    if (i == 0) return it;
    i -= 1;
  }
  it.layer = p.l0 + i / p.T;
  int j = i % p.T;
  if (j < p.nQ) { it.phase = PH_Q; }
  else if ((j -= p.nQ) < p.nA) { it.phase = PH_A; }
  else if ((j -= p.nA) < p.nM) { it.phase = PH_M; }
  else if ((j -= p.nM) < p.nO) { it.phase = PH_O; }
  else if ((j -= p.nO) < p.nG) { it.phase = PH_G; }
  else { j -= p.nG; it.phase = PH_D; }
  it.j = j;
  return it;
}

struct GDesc { const u32x4* q; const u32x4* s; int nb, ns; };

__device__ __forceinline__ GDesc gdesc(const MParams& p, const Item& it) {
  const MLayer& w = p.lw[it.layer - p.l0];
  switch (it.phase) {
    case PH_Q: return GDesc{w.qkv_q, w.qkv_s, p.nbq, p.nsq};
    case PH_O: return GDesc{w.o_q, w.o_s, p.nbo, p.nso};
    case PH_G: return GDesc{w.gu_q, w.gu_s, p.nbg, p.nsg};
    default:   return GDesc{w.dn_q, w.dn_s, p.nbd, p.nsd};
  }
}

__device__ __forceinline__ unsigned* lcnt(const MParams& p, int l) { return p.cnt + (size_t)l * p.cpl; }

__device__ __forceinline__ int clamp_pos(const MParams& p, int P) { return P < 0 ? 0 : (P >= p.cap ? p.cap - 1 : P); }

// ---- dependency wait: thread 0 polls, the workgroup meets at a barrier ---------------------------
__device__ void poll(const MParams& p, const unsigned* c, unsigned target, int item) {
  unsigned n = 0;
  while (peek(c) < target) {
    if ((++n & 63) == 0) {
      if (peek(p.err) != 0) return;      // an earlier wait gave up: finish without waiting
      if (n > kSpinLimit) {
        // first to give up: record which wait (item, counter value, target) after the flag
        if (__hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
          publish_u32(p.err + 1, (unsigned)item);
          publish_u32(p.err + 2, peek(c));
          publish_u32(p.err + 3, target);
        }
        return;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ void wait_dep(const MParams& p, const Item& it, int item) {
  const unsigned* c = nullptr;
  unsigned target = 0;
  const int l = it.layer;
  switch (it.phase) {
    case PH_Q:
      if (l == 0) { c = p.c_prep; target = 1; }
      else if (l > p.l0) { c = lcnt(p, l - 1) + p.k_dd; target = p.ntH; }
      break;
    case PH_A: c = lcnt(p, l) + p.k_dq; target = p.ntq; break;
    case PH_M: {
      const int b = it.j / p.nq, h = it.j % p.nq;
      c = lcnt(p, l) + p.k_ca + b * p.nkv + h / p.g;
      target = p.nsa;
      break;
    }
    case PH_O: c = lcnt(p, l) + p.k_dm; target = p.B * p.nq; break;
    case PH_G: c = lcnt(p, l) + p.k_do; target = p.ntH; break;
    case PH_D: c = lcnt(p, l) + p.k_dg; target = p.ntg; break;
    default: break;
  }
  if (c == nullptr) return;
  if (threadIdx.x == 0) poll(p, c, target, item);
  __syncthreads();
}

// ---- PREP ---------------------------------------------------------------------------------------
__device__ void prep_item(const MParams& p) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint16_t* g1 = p.lw[0].g1;
  for (int b = 0; b < p.B; ++b) {
    for (int t = w; t < p.ntH; t += kW) {
      const int n = t * kTileRows + lane;
      const size_t i = (size_t)b * p.H + n;
      const float hv = h2f(p.emb[i]);
      publish_f32(p.hin + i, hv);
      publish_u16(p.xq + i, f2h(h2f(g1[n]) * hv));
      if (p.trace) p.trace[i] = hv;
      const float ss = wave_sum(hv * hv);
      if (lane == 0) publish_f32(p.ssi + (size_t)b * p.ntH + t, ss);
    }
    if (p.theta > 0.f && tid < 64) {
      const int P = clamp_pos(p, p.pos[b]);
      const double inv = pow((double)p.theta, -(double)(2 * tid) / (double)kD);
      double s, c;
      sincos((double)P * inv, &s, &c);
      publish_f32(p.rope + ((size_t)b * 64 + tid) * 2, (float)c);
      publish_f32(p.rope + ((size_t)b * 64 + tid) * 2 + 1, (float)s);
    }
  }
  wait_published();
  __syncthreads();
  if (tid == 0) arrive(p.c_prep);
}

// ---- GEMV item: (tile, K-split), wave w takes 8-block group 4 split + w ----------------------------
template <int MT>
__device__ void gemv_item(const MParams& p, const Item& it, int item, Lds& L) {
  auto& xs = L.gemv.xs;
  auto& red = L.gemv.red;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const GDesc d = gdesc(p, it);
  const int l = it.layer;
  const int tile = it.j / d.ns, sp = it.j % d.ns;
  const int K = d.nb * kBlock;
  const int e0 = sp * kItemK;

  // weights first: they do not depend on the phase this item waits for.  Every load below is
  // unconditional from a clamped (valid) address: a load behind a branch whose result merges with
  // a default makes the compiler wait for it, and for every load before it, on the spot.
  const int grp = sp * kW + w;
  const int b0 = grp * kGB;
  const int nblk = min(max(d.nb - b0, 0), kGB);
  const int ngr = (d.nb + kGB - 1) / kGB;
  const u32x4* qt = d.q + (size_t)tile * d.nb * kTileRows + lane;
  const u32x4 sv = __builtin_nontemporal_load(d.s + ((size_t)tile * ngr + min(grp, ngr - 1)) * kTileRows + lane);
  u32x4 wv[kGB];
#pragma unroll
  for (int i = 0; i < kGB; ++i) wv[i] = __builtin_nontemporal_load(qt + (size_t)min(b0 + i, d.nb - 1) * kTileRows);

  wait_dep(p, it, item);

  // activation slice into LDS, epilogue operands (loaded by every wave, used by wave 0)
  const uint16_t* x;
  switch (it.phase) {
    case PH_Q: x = p.xq + (size_t)l * p.xq_l; break;
    case PH_O: x = p.ao + (size_t)l * p.ao_l; break;
    case PH_G: x = p.xm + (size_t)l * p.xm_l; break;
    default:   x = p.act + (size_t)l * p.act_l; break;
  }
  uint2 xr[MT];
  {
    const int ec = min(e0 + 4 * tid, K - 4);
#pragma unroll
    for (int m = 0; m < MT; ++m) xr[m] = *reinterpret_cast<const uint2*>(x + (size_t)min(m, p.B - 1) * K + ec);
  }
  const MLayer& lw = p.lw[l - p.l0];
  const int n64 = tile * kTileRows + lane;
  const bool use_ss = it.phase == PH_Q || it.phase == PH_G;
  const bool use_h = it.phase == PH_O || it.phase == PH_D;
  const float* ss_src = it.phase == PH_Q ? p.ssi : p.ssm;
  const float* h_src = it.phase == PH_D ? p.h1 : p.hin;
  const int nh = min(n64, p.H - 1);
  float e_ss[MT], e_h[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mc = min(m, p.B - 1);
    e_ss[m] = collect_f32(ss_src + (size_t)mc * p.ntH + min(lane, p.ntH - 1));
    e_h[m] = collect_f32(h_src + (size_t)mc * p.H + nh);
  }
  const bool has_bias = it.phase == PH_Q && lw.bias != nullptr;
  const uint16_t* gsrc = it.phase == PH_O ? lw.g2
                       : (l + 1 == p.L ? p.gf : (l + 1 < p.l1 ? p.lw[l + 1 - p.l0].g1 : p.g1_next));
  const uint16_t b16 = (has_bias ? lw.bias : p.gf)[has_bias ? min(n64, p.nqkv - 1) : 0];
  const uint16_t g16 = gsrc[nh];
#pragma unroll
  for (int m = 0; m < MT; ++m) *reinterpret_cast<uint2*>(&xs[m][4 * tid]) = xr[m];
  __syncthreads();
  float e_b = 0.f, e_gam = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    e_ss[m] = (use_ss && lane < p.ntH && m < p.B) ? e_ss[m] : 0.f;
    e_h[m] = (use_h && m < p.B) ? e_h[m] : 0.f;
  }
  if (has_bias && n64 < p.nqkv) e_b = h2f(b16);
  if (use_h) e_gam = h2f(g16);

  // blocks past the group's end get scale 0 (their clamped codes and activations are finite)
  const uint32_t m64 = vconst(0x54005400u);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  {
    const int xb0 = w * kGB * kBlock;
    float corr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(&xs[m][xb0 + min(lane, 4 * kGB - 1) * 8]);
      corr[m] = quad_sum(corr_quarter(xv));
    }
#pragma unroll
    for (int i = 0; i < kGB; ++i) {
      const float sc = i < nblk ? pick_scale(sv, i) : 0.f;
      const uint32_t dw[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4* xb = reinterpret_cast<const u32x4*>(&xs[m][xb0 + i * kBlock]);
        float t = -__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, corr[m]), 4 * i));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4 xv = xb[k];
          const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
          t = dot8_pairs(dw[k], x4, t, m64);
        }
        acc[m] = fmaf(sc, t, acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) red[w][m][lane] = acc[m];
  __syncthreads();
  if (w != 0) return;

  float tot[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) tot[m] = ((red[0][m][lane] + red[1][m][lane]) + red[2][m][lane]) + red[3][m][lane];

  unsigned* lc = lcnt(p, l);
  if (d.ns > 1) {
    float* part;
    unsigned* tc;
    switch (it.phase) {
      case PH_Q: part = p.pq; tc = lc + p.k_cq; break;
      case PH_O: part = p.po; tc = lc + p.k_co; break;
      case PH_G: part = p.pg; tc = lc + p.k_cg; break;
      default:   part = p.pd; tc = lc + p.k_cd; break;
    }
    float* mine = part + ((size_t)tile * d.ns + sp) * MT * kWave;
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < p.B) publish_f32(mine + m * kWave + lane, tot[m]);
    wait_published();
    unsigned prev = 0;
    if (lane == 0) prev = arrive(tc + tile);
    prev = __shfl(prev, 0, kWave);
    if (prev != (unsigned)(d.ns - 1)) return;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= p.B) continue;
      tot[m] = collect_sum_f32(part + ((size_t)tile * d.ns * MT + m) * kWave + lane, d.ns, (size_t)MT * kWave);
    }
  }

  // ---- epilogue (wave 0; lane = row of the tile) ----
  float rs[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) rs[m] = 1.f;
  if (it.phase == PH_Q || it.phase == PH_G) {
#pragma unroll
    for (int m = 0; m < MT; ++m) rs[m] = 1.0f / sqrtf(wave_sum(e_ss[m]) * p.inv_h + p.eps);
  }
  unsigned* done;
  if (it.phase == PH_Q) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < p.B && n64 < p.nqkv) publish_f32(p.qkv + (size_t)m * p.nqkv + n64, tot[m] * rs[m] + e_b);
    done = lc + p.k_dq;
  } else if (it.phase == PH_O) {
    uint16_t* xm = p.xm + (size_t)l * p.xm_l;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= p.B) continue;
      const float hn = e_h[m] + tot[m];
      const size_t i = (size_t)m * p.H + n64;
      publish_f32(p.h1 + i, hn);
      publish_u16(xm + i, f2h(e_gam * hn));
      const float ss = wave_sum(hn * hn);
      if (lane == 0) publish_f32(p.ssm + (size_t)m * p.ntH + tile, ss);
    }
    done = lc + p.k_do;
  } else if (it.phase == PH_G) {  // lanes 0-31: gate rows, 32-63: the same up rows
    uint16_t* act = p.act + (size_t)l * p.act_l;
    const int n = tile * 32 + (lane & 31);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= p.B) continue;
      const float gv = tot[m] * rs[m];
      const float uv = __shfl(tot[m], (lane & 31) + 32, kWave) * rs[m];
      if (lane < 32) publish_u16(act + (size_t)m * p.I + n, f2h(silu(gv) * uv));
    }
    done = lc + p.k_dg;
  } else {
    const bool last = l + 1 == p.L;
    uint16_t* xq = p.xq + (size_t)(l + 1) * p.xq_l;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= p.B) continue;
      const float hn = e_h[m] + tot[m];
      const size_t i = (size_t)m * p.H + n64;
      publish_f32(p.hin + i, hn);
      if (last) publish_f32(p.gfo + i, e_gam * hn);
      else publish_u16(xq + i, f2h(e_gam * hn));
      if (p.trace) p.trace[(size_t)(l + 1) * p.B * p.H + i] = hn;
      const float ss = wave_sum(hn * hn);
      if (lane == 0) publish_f32(p.ssi + (size_t)m * p.ntH + tile, ss);
    }
    done = lc + p.k_dd;
  }
  wait_published();
  if (lane == 0) arrive(done);
}

// ---- attention item: (sequence, KV head, 64 positions) ----------------------------------------------
// lane = (position 4r + lane/16 of the wave's 16, dims 8 (lane%16) .. +7); the new position's
// row comes from the q|k|v output (the cache slot is written here), the others from the cache
__device__ void attn_item(const MParams& p, const Item& it, int item, Lds& L) {
  auto& qs = L.attn.qs;
  auto& sc = L.attn.sc;
  auto& red = L.attn.red;
  auto& knew = L.attn.knew;
  auto& vnew = L.attn.vnew;
  auto& mh = L.attn.mh;
  auto& lh = L.attn.lh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = it.layer;
  const int g = p.g;
  const int sa = it.j % p.nsa, bh = it.j / p.nsa;
  const int b = bh / p.nkv, kvh = bh % p.nkv;
  const int s0 = sa * kAS;
  const int P = clamp_pos(p, p.pos[b]);
  const int npos = max(0, min(s0 + kAS, P + 1) - s0);
  unsigned* ca = lcnt(p, l) + p.k_ca + bh;
  if (npos == 0) {                   // past the sequence: nothing to attend, only count
    if (tid == 0) arrive(ca);
    return;
  }
  const bool has_new = P >= s0 && P < s0 + npos;
  const int sl = lane & 15, pg = lane >> 4;
  const int jw = w * 16;

  // K/V rows first (clamped rows are masked below)
  const size_t kvbase = (size_t)l * p.kv_layer + (size_t)bh * p.cap * kD;
  u32x4 kr[4], vr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pos = min(s0 + jw + 4 * r + pg, p.cap - 1);
    kr[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.kc + kvbase + (size_t)pos * kD + 8 * sl));
    vr[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.vc + kvbase + (size_t)pos * kD + 8 * sl));
  }

  wait_dep(p, it, item);

  // q of the group (rotated) and the new k/v: thread t < 16 g rotates dims 4c..4c+3 with
  // 64+4c..64+4c+3 of head t/16 (c = t%16); the next 16 threads the new k, the 16 after them v
  const int c16 = tid & 15;
  const float* row = p.qkv + (size_t)b * p.nqkv;
  const float* src = nullptr;
  if (tid < 16 * g) src = row + (size_t)(kvh * g + (tid >> 4)) * kD;
  else if (tid < 16 * g + 16) src = row + (size_t)p.nq * kD + (size_t)kvh * kD;
  else if (tid < 16 * g + 32) src = row + (size_t)(p.nq + p.nkv) * kD + (size_t)kvh * kD;
  if (src) {
    float x1[4], x2[4], c4[4] = {1.f, 1.f, 1.f, 1.f}, s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x1[i] = collect_f32(src + 4 * c16 + i);
      x2[i] = collect_f32(src + 64 + 4 * c16 + i);
    }
    const bool rot = p.theta > 0.f && tid < 16 * g + 16;
    if (rot) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = collect_f32(p.rope + ((size_t)b * 64 + 4 * c16 + i) * 2);
        s4[i] = collect_f32(p.rope + ((size_t)b * 64 + 4 * c16 + i) * 2 + 1);
      }
    }
    float r1[4], r2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = x1[i] * c4[i] - x2[i] * s4[i];
      r2[i] = x2[i] * c4[i] + x1[i] * s4[i];
    }
    if (tid < 16 * g) {
      const int hh = tid >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qs[hh][4 * c16 + i] = r1[i];
        qs[hh][64 + 4 * c16 + i] = r2[i];
      }
    } else if (has_new) {
      uint16_t* dst = tid < 16 * g + 16 ? knew : vnew;
      uint16_t* cache = (tid < 16 * g + 16 ? p.kc : p.vc) + kvbase + (size_t)P * kD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t a = f2h(r1[i]), bb = f2h(r2[i]);
        dst[4 * c16 + i] = a;
        dst[64 + 4 * c16 + i] = bb;
        cache[4 * c16 + i] = a;
        cache[64 + 4 * c16 + i] = bb;
      }
    }
  }
  __syncthreads();
  if (has_new) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (s0 + jw + 4 * r + pg == P) {
        kr[r] = *reinterpret_cast<const u32x4*>(&knew[8 * sl]);
        vr[r] = *reinterpret_cast<const u32x4*>(&vnew[8 * sl]);
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (jw + 4 * r + pg >= npos) vr[r] = u32x4{0, 0, 0, 0};   // probability 0: keep 0 * v finite

  // scores: 16 lanes per position, reduced across the 16
#pragma unroll 1
  for (int hh = 0; hh < g; ++hh) {
    float q8[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q8[t] = qs[hh][8 * sl + t];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = row16_sum(dot8_mix(q8, kr[r], 0.f));
      const int j = jw + 4 * r + pg;
      if (sl == 0) sc[hh][j] = j < npos ? a * p.scale : -INFINITY;
    }
  }
  __syncthreads();
  for (int hh = w; hh < g; hh += kW) {
    const float v = sc[hh][lane];
    const float m = wave_max(v);
    const float e = (m == -INFINITY) ? 0.f : expf(v - m);
    const float s = wave_sum(e);
    sc[hh][lane] = e;
    if (lane == 0) { mh[hh] = m; lh[hh] = s; }
  }
  __syncthreads();
  // P.V over the wave's 16 positions (4 per lane, then across the 4 position groups)
#pragma unroll 1
  for (int hh = 0; hh < g; ++hh) {
    float acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pj = sc[hh][jw + 4 * r + pg];
      const u32x4 v = vr[r];
      acc[0] = fma_mix_lo(pj, v.x, acc[0]); acc[1] = fma_mix_hi(pj, v.x, acc[1]);
      acc[2] = fma_mix_lo(pj, v.y, acc[2]); acc[3] = fma_mix_hi(pj, v.y, acc[3]);
      acc[4] = fma_mix_lo(pj, v.z, acc[4]); acc[5] = fma_mix_hi(pj, v.z, acc[5]);
      acc[6] = fma_mix_lo(pj, v.w, acc[6]); acc[7] = fma_mix_hi(pj, v.w, acc[7]);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = rows_lanewise_sum(acc[t]);
    if (pg == 0) {
      float* dst = &red[w][hh][8 * sl];
      *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
  __syncthreads();
  float* rec = p.ap + ((size_t)bh * p.nsa + sa) * g * kPS;
  for (int i = tid; i < g * kD; i += kThr) {
    const int hh = i >> 7, dd = i & 127;
    const float o = ((red[0][hh][dd] + red[1][hh][dd]) + red[2][hh][dd]) + red[3][hh][dd];
    publish_f32(rec + (size_t)hh * kPS + 4 + dd, o);
  }
  if (tid < g) {
    publish_f32(rec + (size_t)tid * kPS, mh[tid]);
    publish_f32(rec + (size_t)tid * kPS + 1, lh[tid]);
  }
  wait_published();
  __syncthreads();
  if (tid == 0) arrive(ca);
}

// ---- merge item: (sequence, query head); thread (half, d) takes dim d of its half's splits -------
__device__ void merge_item(const MParams& p, const Item& it, int item, Lds& L) {
  constexpr int kChunk = 16;
  auto& ms_ = L.merge.ms;
  auto& ws_ = L.merge.ws;
  auto& part = L.merge.part;
  float& Ls = L.merge.Ls;
  const int tid = threadIdx.x;
  const int l = it.layer;
  const int b = it.j / p.nq, h = it.j % p.nq;
  const int kvh = h / p.g, hh = h % p.g;
  wait_dep(p, it, item);
  const int n = (clamp_pos(p, p.pos[b]) + 1 + kAS - 1) / kAS;   // splits that hold positions
  const int d = tid & 127, half = tid >> 7;
  const int per = (n + 1) >> 1;
  const int s_beg = half * per, s_end = min(n, s_beg + per);
  const size_t stride = (size_t)p.g * kPS;
  const float* base = p.ap + (size_t)(b * p.nkv + kvh) * p.nsa * stride + (size_t)hh * kPS;
  float v[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u) v[u] = s_beg + u < s_end ? collect_f32(base + (size_t)(s_beg + u) * stride + 4 + d) : 0.f;
  if (tid < 64) {
    float M = -INFINITY;
    for (int s = tid; s < n; s += 64) {
      const float m = collect_f32(base + (size_t)s * stride);
      ms_[s] = m;
      M = fmaxf(M, m);
    }
    M = wave_max(M);
    float lsum = 0.f;
    for (int s = tid; s < n; s += 64) {
      const float e = expf(ms_[s] - M);
      ws_[s] = e;
      lsum = fmaf(e, collect_f32(base + (size_t)s * stride + 1), lsum);
    }
    lsum = wave_sum(lsum);
    if (tid == 0) Ls = lsum;
  }
  __syncthreads();
  float O = 0.f;
#pragma unroll
  for (int u = 0; u < kChunk; ++u)
    if (s_beg + u < s_end) O = fmaf(ws_[s_beg + u], v[u], O);
  for (int c0 = s_beg + kChunk; c0 < s_end; c0 += kChunk) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) v[u] = c0 + u < s_end ? collect_f32(base + (size_t)(c0 + u) * stride + 4 + d) : 0.f;
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (c0 + u < s_end) O = fmaf(ws_[c0 + u], v[u], O);
  }
  part[half][d] = O;
  __syncthreads();
  if (half == 0) {
    uint16_t* ao = p.ao + (size_t)l * p.ao_l + ((size_t)b * p.nq + h) * kD;
    publish_u16(ao + d, f2h((part[0][d] + part[1][d]) / Ls));
  }
  wait_published();
  __syncthreads();
  if (tid == 0) arrive(lcnt(p, l) + p.k_dm);
}

template <int MT>
__global__ __launch_bounds__(kThr) void k_decode_flow(MParams arg) {
  // read the parameters in place from the kernel-argument segment (scalar loads): indexing the
  // per-layer table of a by-value copy would move the whole struct to scratch memory
#if defined(__HIP_DEVICE_COMPILE__)
  (void)arg;
  const MParams& p = *reinterpret_cast<const MParams*>(__builtin_amdgcn_kernarg_segment_ptr());
#else
  const MParams& p = arg;   // host pass: the body is never run there
#endif
  __shared__ __align__(16) Lds L;
  const int i = blockIdx.x;
  if (i >= p.total) return;
  const Item it = decode(p, i);
  switch (it.phase) {
    case PH_PREP: prep_item(p); break;
    case PH_A: attn_item(p, it, i, L); break;
    case PH_M: merge_item(p, it, i, L); break;
    default: gemv_item<MT>(p, it, i, L); break;
  }
}

// ---- host side -----------------------------------------------------------------------------------
struct MDims {
  int L, B, H, I, nq, nkv, g, cap, nqkv, ntH, ntq, ntg;
  int nbq, nbo, nbg, nbd, nsq, nso, nsg, nsd, nsa;
  int cpl;
};

int splits(int nb) { return (int)cdiv(cdiv(nb, kGB), kW); }

MDims mdims(const vv_model* m, int B, int cap) {
  MDims d{};
  d.L = m->n_layers; d.B = B; d.H = m->hidden; d.I = m->inter; d.nq = m->n_q; d.nkv = m->n_kv;
  d.g = m->n_q / m->n_kv; d.cap = cap;
  d.nqkv = (m->n_q + 2 * m->n_kv) * kD;
  d.ntH = d.H / kTileRows;
  d.ntq = (int)cdiv(d.nqkv, kTileRows);
  d.ntg = 2 * (d.I / kTileRows);
  d.nbq = d.H / kBlock; d.nbo = d.nq * kD / kBlock; d.nbg = d.H / kBlock; d.nbd = d.I / kBlock;
  d.nsq = splits(d.nbq); d.nso = splits(d.nbo); d.nsg = splits(d.nbg); d.nsd = splits(d.nbd);
  d.nsa = (int)cdiv(cap, kAS);
  // counters per layer: tiles of q|k|v, o, gate/up, down; (sequence, KV head); 5 phase counters
  d.cpl = (int)align_up((size_t)d.ntq + d.ntH + d.ntg + d.ntH + (size_t)B * d.nkv, kPad) + 5 * kPad;
  return d;
}

struct MLayout {
  size_t hdr, cnt, rope, gfo, ssi, ssm, hin, h1, qkv, ap, pq, po, pg, pd, xq, xm, ao, act, total;
  size_t cnt_bytes;   // prep counter + per-layer counters (cleared before each launch)
  size_t xq_l, xm_l, ao_l, act_l;
};

MLayout mlayout(const MDims& d) {
  MLayout y{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes, 256); return o; };
  const size_t B = d.B;
  y.hdr = take(128);                                   // sticky status word
  y.cnt_bytes = 128 + (size_t)d.L * d.cpl * 4;         // prep counter, then the layers'
  y.cnt = take(y.cnt_bytes);
  y.rope = take(B * 64 * 2 * 4);
  y.gfo = take(B * d.H * 4);
  y.ssi = take(B * d.ntH * 4);
  y.ssm = take(B * d.ntH * 4);
  y.hin = take(B * d.H * 4);
  y.h1 = take(B * d.H * 4);
  y.qkv = take(B * d.nqkv * 4);
  y.ap = take(B * d.nkv * (size_t)d.nsa * d.g * kPS * 4);
  y.pq = take((size_t)d.ntq * d.nsq * kMaxMT * kWave * 4);
  y.po = take((size_t)d.ntH * d.nso * kMaxMT * kWave * 4);
  y.pg = take((size_t)d.ntg * d.nsg * kMaxMT * kWave * 4);
  y.pd = take((size_t)d.ntH * d.nsd * kMaxMT * kWave * 4);
  y.xq_l = align_up(B * d.H, 128);
  y.xm_l = align_up(B * d.H, 128);
  y.ao_l = align_up(B * d.nq * kD, 128);
  y.act_l = align_up(B * d.I, 128);
  y.xq = take(y.xq_l * 2 * (d.L + 1));
  y.xm = take(y.xm_l * 2 * d.L);
  y.ao = take(y.ao_l * 2 * d.L);
  y.act = take(y.act_l * 2 * d.L);
  y.total = off;
  return y;
}

}  // namespace

bool persistent_supported(const vv_model* m, int batch) {
  return m->n_layers >= 1 && batch >= 1 && batch <= kMaxMT && m->hidden <= 64 * kTileRows &&
         m->n_q / m->n_kv <= kMaxG && m->n_q / m->n_kv >= 1;
}

size_t persistent_workspace_bytes(const vv_model* m, int batch, int cap) {
  return mlayout(mdims(m, batch, cap)).total;
}

int persistent_enqueue(const vv_model* m, const vv_state* s, char* ws, hipStream_t st, KEv ev) {
  const MDims d = mdims(m, s->batch, s->cap);
  const MLayout y = mlayout(d);
  VV_REQUIRE((int64_t)cdiv(s->cap, kAS) <= 1024, VV_ERR_RANGE,
             "single-launch decode: cap %d > 65536 positions", s->cap);
  MParams p{};
  p.L = d.L; p.B = d.B; p.H = d.H; p.I = d.I; p.nq = d.nq; p.nkv = d.nkv; p.g = d.g; p.cap = d.cap;
  p.nqkv = d.nqkv; p.ntH = d.ntH;
  p.eps = m->eps; p.inv_h = 1.0f / (float)d.H; p.scale = 1.0f / sqrtf((float)kD); p.theta = m->rope_theta;
  p.emb = s->input_embeds; p.pos = s->pos;
  p.kc = static_cast<uint16_t*>(s->k_cache); p.vc = static_cast<uint16_t*>(s->v_cache);
  p.kv_layer = (size_t)d.B * d.nkv * (size_t)d.cap * kD;
  p.gf = m->gf; p.trace = s->h_trace;
  p.ntq = d.ntq; p.ntg = d.ntg;
  p.nbq = d.nbq; p.nbo = d.nbo; p.nbg = d.nbg; p.nbd = d.nbd;
  p.nsq = d.nsq; p.nso = d.nso; p.nsg = d.nsg; p.nsd = d.nsd; p.nsa = d.nsa;
  p.nQ = d.ntq * d.nsq; p.nA = d.B * d.nkv * d.nsa; p.nM = d.B * d.nq;
  p.nO = d.ntH * d.nso; p.nG = d.ntg * d.nsg; p.nD = d.ntH * d.nsd;
  p.T = p.nQ + p.nA + p.nM + p.nO + p.nG + p.nD;
  p.err = reinterpret_cast<unsigned*>(ws + y.hdr);
  p.c_prep = reinterpret_cast<unsigned*>(ws + y.cnt);
  p.cnt = reinterpret_cast<unsigned*>(ws + y.cnt + 128);
  p.cpl = d.cpl;
  p.k_cq = 0; p.k_co = d.ntq; p.k_cg = p.k_co + d.ntH; p.k_cd = p.k_cg + d.ntg; p.k_ca = p.k_cd + d.ntH;
  const int ph0 = (int)align_up((size_t)p.k_ca + (size_t)d.B * d.nkv, kPad);
  p.k_dq = ph0; p.k_dm = ph0 + kPad; p.k_do = ph0 + 2 * kPad; p.k_dg = ph0 + 3 * kPad; p.k_dd = ph0 + 4 * kPad;
  p.rope = reinterpret_cast<float*>(ws + y.rope);
  p.gfo = reinterpret_cast<float*>(ws + y.gfo);
  p.ssi = reinterpret_cast<float*>(ws + y.ssi); p.ssm = reinterpret_cast<float*>(ws + y.ssm);
  p.hin = reinterpret_cast<float*>(ws + y.hin); p.h1 = reinterpret_cast<float*>(ws + y.h1);
  p.qkv = reinterpret_cast<float*>(ws + y.qkv); p.ap = reinterpret_cast<float*>(ws + y.ap);
  p.pq = reinterpret_cast<float*>(ws + y.pq); p.po = reinterpret_cast<float*>(ws + y.po);
  p.pg = reinterpret_cast<float*>(ws + y.pg); p.pd = reinterpret_cast<float*>(ws + y.pd);
  p.xq = reinterpret_cast<uint16_t*>(ws + y.xq); p.xm = reinterpret_cast<uint16_t*>(ws + y.xm);
  p.ao = reinterpret_cast<uint16_t*>(ws + y.ao); p.act = reinterpret_cast<uint16_t*>(ws + y.act);
  p.xq_l = y.xq_l; p.xm_l = y.xm_l; p.ao_l = y.ao_l; p.act_l = y.act_l;

  // every counter starts each step at zero (a fill kernel: capture-safe, unlike a memset node)
  VV_HIP(fill_zero(ws + y.cnt, y.cnt_bytes, st, ev.first()));
  for (int l0 = 0; l0 < d.L; l0 += kMaxL) {
    p.l0 = l0;
    p.l1 = std::min(d.L, l0 + kMaxL);
    for (int l = l0; l < p.l1; ++l) {
      const vv_layer& w = m->layers[l];
      MLayer& q = p.lw[l - l0];
      q.qkv_q = reinterpret_cast<const u32x4*>(w.qkv_q); q.qkv_s = reinterpret_cast<const u32x4*>(w.qkv_s);
      q.o_q = reinterpret_cast<const u32x4*>(w.o_q); q.o_s = reinterpret_cast<const u32x4*>(w.o_s);
      q.gu_q = reinterpret_cast<const u32x4*>(w.gu_q); q.gu_s = reinterpret_cast<const u32x4*>(w.gu_s);
      q.dn_q = reinterpret_cast<const u32x4*>(w.down_q); q.dn_s = reinterpret_cast<const u32x4*>(w.down_s);
      q.bias = w.qkv_bias; q.g1 = w.g1; q.g2 = w.g2;
    }
    // RMSNorm_1 weight of the first layer of the next launch (read by this launch's last D items)
    p.g1_next = p.l1 < d.L ? m->layers[p.l1].g1 : nullptr;
    p.total = (l0 == 0 ? 1 : 0) + (p.l1 - l0) * p.T;
    const KEv e = p.l1 == d.L ? ev.last() : KEv{};
    VV_LAUNCH(k_decode_flow<1>, dim3(p.total), dim3(kThr), st, e, p);
    VV_HIP(hipGetLastError());
  }
  return VV_OK;
}

int persistent_grid() { return 1; }

// inputs of the lm_head after the single-launch layers: gamma_f * h (fp32) and per-tile sums of h^2
void persistent_lm_inputs(const vv_model* m, const vv_state* s, char* ws, const float** gf32, const float** sumsq) {
  const MDims d = mdims(m, s->batch, s->cap);
  const MLayout y = mlayout(d);
  *gf32 = reinterpret_cast<const float*>(ws + y.gfo);
  *sumsq = reinterpret_cast<const float*>(ws + y.ssi);
}

}  // namespace vv

