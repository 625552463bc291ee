// Persistent decode step: every layer of one decode step in a single launch.
//
// The step is the decoder_step contract of the "vibevoice-asr-bitnet-onnx" page (graph
// contracts: input_embeds and position_ids in, logits and one more K/V slot out) on the Qwen2
// layer of the 1.5B STATUS page (Architecture): pre-RMSNorm, q/k/v bias, grouped-query
// attention, SiLU-gated MLP, residual adds; projections are int4 block-32 MatMulNBits with
// float activations (same page, quantisation section).
//
// Why one launch: at batch 1 a 28-layer step is ~170 dependent stages, most of them a few MB of
// weights.  As separate kernels each stage pays a launch gap, a ramp and a reduction tail, and
// the HBM idles meanwhile.  Here a grid of co-resident workgroups walks one global list of work
// items in dependency order.  Per layer the items are
//   Q  (tile, K-split) of the fused q|k|v GEMV: RMSNorm_1 folded in, bias added
//   A  (sequence, KV head, 64 positions) of attention: RoPE, KV append, split softmax
//   M  (sequence, query head, 64 dims): merge of the attention splits
//   O  (tile, K-split) of the o GEMV + residual (writes RMSNorm_2's input)
//   G  (tile, K-split) of the gate/up GEMV + SiLU(gate)*up (RMSNorm_2 folded in)
//   D  (tile, K-split) of the down GEMV + residual (writes the next layer's RMSNorm_1 input)
// and one PREP item starts the step (embeddings -> residual stream, RoPE table).  Item i belongs
// to queue i % kQueues; a workgroup serves the queue given by the order in which it started and
// claims that queue's items one at a time, in increasing order (one atomic per item, spread over
// kQueues counters).  Before a workgroup waits for an item's inputs it has already issued that
// item's weight (or K/V) loads and those of its next item, so the HBM keeps streaming through
// every hand-off.  Every wait is on an item with a smaller index; the smallest unfinished item's
// queue has a running server (the first kQueues workgroups to start are running) whose earlier
// items are finished, so the walk always makes progress, whatever the residency beyond that.
// Each wait is bounded anyway (a sticky error word instead of a hang).
//
// Roles: a workgroup is 4 compute waves and 1 control wave.  Vector loads return in order and a
// wave can only wait for all of its memory operations at once, so the compute waves, whose
// queues hold the next item's weights, never issue a load or store that someone waits on: the
// control wave polls, stages activations into LDS, publishes results and runs the epilogues.
//
// Hand-offs: a K-split partial is an agent-scope store; the workgroup then counts itself in at
// its tile, and the last one adds the partials in split order (deterministic) and runs the
// epilogue; a finished tile or item counts itself in at its phase; consumers poll the phase
// counter.  Activations that are read with plain (cacheable) loads are written exactly once per
// launch into per-layer buffers, so no cache can hold a stale copy of them; everything else
// produced inside the launch is read with agent-scope loads.  The last workgroup to leave resets
// the counters for the next launch.
#include <algorithm>
#include <mutex>

#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kW = 4;               // compute waves per workgroup
constexpr int kCtl = kW;            // wave id of the control wave
constexpr int kThr = (kW + 1) * kWave;   // threads per workgroup
constexpr int kGB = 8;              // blocks per wave task (one 16-byte scale group)
constexpr int kItemK = kW * kGB * kBlock;   // K elements per GEMV item (1024)
constexpr int kD = 128;             // head_dim
constexpr int kAS = 64;             // attention positions per item (16 per wave)
constexpr int kPS = 132;            // attention record per head: m, l, pad, pad, o[128]
constexpr int kMaxG = 8;            // query heads per KV head
constexpr int kMaxL = 32;           // layers per launch (kernel-argument table)
constexpr int kMaxMT = 1;           // batch rows handled by the persistent path
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kPad = 32;            // u32 per phase counter (own 128-byte line)
constexpr int kQueues = 32;         // item queues (item i belongs to queue i % kQueues)

enum Phase { PH_PREP = 0, PH_Q, PH_A, PH_M, PH_O, PH_G, PH_D };

// Optional timing record (built with -DVV_STATS): per workgroup, wall-clock ticks (100 MHz) spent
// polling per phase and working per phase, and per layer the tick at which each phase completed.
#ifdef VV_STATS
constexpr int kStatWords = 32;
__device__ unsigned long long g_vv_stats[4096 * 32 + 256 * 8];
#define VV_STAT(...) __VA_ARGS__
#else
#define VV_STAT(...)
#endif

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
  int nQ, nA, nM, nO, nG, nD, T, total, nwg;
  // workspace
  unsigned* err; unsigned* c_prep; unsigned* c_exit; unsigned* c_start; unsigned* c_queue;
  unsigned* cnt; int cpl;                          // counters, cpl per layer
  int k_cq, k_co, k_cg, k_cd, k_ca, k_dq, k_dm, k_do, k_dg, k_dd;
  float* rope; float* gfo;
  const u32x4* zero;                               // 1 KiB that stays zero (unused load slots)
  unsigned long long* stats;                       // VV_STATS only
  float* ssi; float* ssm; float* hin; float* h1; float* qkv; float* ap;
  float* pq; float* po; float* pg; float* pd;
  uint16_t* xq; uint16_t* xm; uint16_t* ao; uint16_t* act;   // per layer (write-once)
  size_t xq_l, xm_l, ao_l, act_l;                  // elements per layer
  MLayer lw[kMaxL];
};

struct Item { int layer, phase, j; };

struct Pay { u32x4 v[kGB]; u32x4 s; };

template <int MT>
struct Shared {
  alignas(16) uint16_t x[MT][kItemK]; // GEMV activation slice
  float red[kW][MT][kWave];           // GEMV cross-wave sums
  float qs[kMaxG][kD];                // attention: rotated q
  float sc[kMaxG][kAS];               // attention: scores / probabilities
  float ared[kW][kMaxG][kD];          // attention: per-wave P.V
  float mh[kMaxG], lh[kMaxG];
  int flag;
  int idx[2];                         // item hand-over from the control wave to the compute waves
};

__device__ __forceinline__ void publish_u16(uint16_t* p, uint16_t v) {
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

// ---- loads that do not depend on activations (weights, cached K/V) ---------------------------
// Always exactly kGB + 1 loads, issued from one straight-line block whatever the item: slots an
// item does not use read a zero-filled line of the workspace.  A fixed count lets the compiler
// wait for exactly the current item's loads (vmcnt = the next item's count) instead of draining
// the queue, which would serialise the prefetch.
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;   // global (not flat) loads

// Always exactly kGB + 1 loads from one straight-line block, each a wave-uniform base plus one
// per-lane offset; slots an item does not use read a zero-filled KiB of the workspace.  A fixed
// count lets the compiler wait for exactly the current item's loads (vmcnt = the next item's
// count) instead of draining the queue, which would serialise the prefetch.
__device__ __forceinline__ void issue(const MParams& p, int i, Pay& P, int w, int lane) {
  const char* base[kGB + 1];
  const char* z = reinterpret_cast<const char*>(p.zero);
#pragma unroll
  for (int k = 0; k <= kGB; ++k) base[k] = z;
  // per-lane offsets: GEMV lane i reads row i (16 B); K/V pass r: lane (pg, sl) reads dims 8 sl..
  // of position pos_r + pg, clamped to the last cache slot (masked out later) at the end of the
  // cache; all offsets stay inside the zero KiB for unused slots
  uint32_t off[4];
  const uint32_t lin = (uint32_t)(lane * 16);
#pragma unroll
  for (int r = 0; r < 4; ++r) off[r] = lin;
  if (i >= 0) {
    const Item it = decode(p, i);
    if (it.phase == PH_A) {
      const int sa = it.j % p.nsa, bh = it.j / p.nsa;
      const size_t row0 = (size_t)it.layer * p.kv_layer + (size_t)bh * p.cap * kD;
      const int sl = lane & 15, pg = lane >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = sa * kAS + w * 16 + 4 * r;
        if (pos < p.cap) {
          base[r] = reinterpret_cast<const char*>(p.kc + row0 + (size_t)pos * kD);
          base[4 + r] = reinterpret_cast<const char*>(p.vc + row0 + (size_t)pos * kD);
          off[r] = (uint32_t)(min(pg, p.cap - 1 - pos) * kD * 2 + sl * 16);
        }
      }
    } else if (it.phase == PH_Q || it.phase == PH_O || it.phase == PH_G || it.phase == PH_D) {
      const GDesc d = gdesc(p, it);
      const int tile = it.j / d.ns, sp = it.j % d.ns;
      const int grp = sp * kW + w;
      const int b0 = grp * kGB;
      const int nblk = min(max(d.nb - b0, 0), kGB);
      const char* qb = reinterpret_cast<const char*>(d.q + ((size_t)tile * d.nb + b0) * kTileRows);
#pragma unroll
      for (int k = 0; k < kGB; ++k)
        if (k < nblk) base[k] = qb + (size_t)k * kTileRows * 16;
      if (nblk > 0)
        base[kGB] = reinterpret_cast<const char*>(d.s + ((size_t)tile * ((d.nb + kGB - 1) / kGB) + grp) * kTileRows);
    }
  }
  // explicitly global: a flat load would also count against the LDS counter and make every LDS
  // wait drain the prefetch
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    P.v[r] = __builtin_nontemporal_load((gptr_u32x4)(uintptr_t)(base[r] + off[r]));
    P.v[4 + r] = __builtin_nontemporal_load((gptr_u32x4)(uintptr_t)(base[4 + r] + off[r]));
  }
  P.s = __builtin_nontemporal_load((gptr_u32x4)(uintptr_t)(base[kGB] + lin));
}

// ---- dependency wait ---------------------------------------------------------------------------
// The control wave polls; the workgroup meets at a barrier.  A satisfied phase stays satisfied,
// so a workgroup skips the poll for later items that need the same (or an earlier) phase.
__device__ __forceinline__ void poll(const MParams& p, const unsigned* c, unsigned target, int item) {
  unsigned n = 0;
  while (peek(c) < target) {
    if ((++n & 63) == 0) {
      if (peek(p.err) != 0) return;      // an earlier wait gave up: finish without waiting
      if (n > kSpinLimit) {
        if (__hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
          const Item it = decode(p, item);
          printf("vv persistent decode: wait gave up at item %d (layer %d, phase %d, j %d) in workgroup %d: "
                 "counter %u < %u; %u of %d workgroups started\n", item, it.layer, it.phase, it.j, (int)blockIdx.x,
                 peek(c), target, peek(p.c_start), p.nwg);
        }
        return;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Both roles call this with the same item sequence, so they agree on whether to meet.
__device__ __forceinline__ void wait_dep(const MParams& p, const Item& it, int item, int& done_key, bool ctl, int lane) {
  const unsigned* c = nullptr;
  unsigned target = 0;
  int key = -1;
  const int l = it.layer;
  switch (it.phase) {
    case PH_Q:
      if (l == 0) { c = p.c_prep; target = 1; }
      else if (l > p.l0) { c = lcnt(p, l - 1) + p.k_dd; target = p.ntH; }
      key = l * 8 + 1;
      break;
    case PH_A: c = lcnt(p, l) + p.k_dq; target = p.ntq; key = l * 8 + 2; break;
    case PH_M: {
      const int bhq = it.j >> 1;
      const int b = bhq / p.nq, h = bhq % p.nq;
      c = lcnt(p, l) + p.k_ca + b * p.nkv + h / p.g;
      target = p.nsa;
      break;
    }
    case PH_O: c = lcnt(p, l) + p.k_dm; target = 2 * p.B * p.nq; key = l * 8 + 4; break;
    case PH_G: c = lcnt(p, l) + p.k_do; target = p.ntH; key = l * 8 + 5; break;
    case PH_D: c = lcnt(p, l) + p.k_dg; target = p.ntg; key = l * 8 + 6; break;
    default: break;
  }
  if (c == nullptr || (key >= 0 && key <= done_key)) return;
  VV_STAT(const unsigned long long t0 = wall_clock64();)
  if (ctl && lane == 0) poll(p, c, target, item);
  __syncthreads();
  VV_STAT(if (ctl && lane == 0) {
    unsigned long long* st = p.stats + (size_t)blockIdx.x * kStatWords;
    st[it.phase] += wall_clock64() - t0;
    st[8 + it.phase] += 1;
  })
  if (key > done_key) done_key = key;
}

// ================================================================================================
// Control wave
// ================================================================================================
template <int MT>
__device__ void prep_ctl(const MParams& p, Shared<MT>& sh, int lane, int slot, int nn) {
  if (lane == 0) sh.idx[slot] = nn;
  __syncthreads();   // S
  const uint16_t* g1 = p.lw[0].g1;
  for (int b = 0; b < p.B; ++b) {
    for (int t = 0; t < p.ntH; ++t) {
      const int n = t * kTileRows + lane;
      const size_t i = (size_t)b * p.H + n;
      const float hv = h2f(p.emb[i]);
      publish_f32(p.hin + i, hv);
      publish_u16(p.xq + i, f2h(h2f(g1[n]) * hv));
      if (p.trace) p.trace[i] = hv;
      const float ss = wave_sum(hv * hv);
      if (lane == 0) publish_f32(p.ssi + (size_t)b * p.ntH + t, ss);
    }
    if (p.theta > 0.f) {
      int P = p.pos[b];
      P = P < 0 ? 0 : (P >= p.cap ? p.cap - 1 : P);
      const double inv = pow((double)p.theta, -(double)(2 * lane) / (double)kD);
      double s, c;
      sincos((double)P * inv, &s, &c);
      publish_f32(p.rope + ((size_t)b * 64 + lane) * 2, (float)c);
      publish_f32(p.rope + ((size_t)b * 64 + lane) * 2 + 1, (float)s);
    }
  }
  wait_published();
  if (lane == 0) arrive(p.c_prep);
  VV_STAT(if (lane == 0) p.stats[(size_t)4096 * kStatWords + 7] = wall_clock64();)
}

// GEMV: stage the activation slice in LDS | (compute) | add the waves' sums, hand off, epilogue
template <int MT>
__device__ void gemv_ctl(const MParams& p, const Item& it, Shared<MT>& sh, int lane, int slot, int nn) {
  const GDesc d = gdesc(p, it);
  const int l = it.layer;
  const int tile = it.j / d.ns, sp = it.j % d.ns;
  const int K = d.nb * kBlock;
  const int e0 = sp * kItemK;
  const int ne = min(K - e0, kItemK);
  const MLayer& lw = p.lw[l - p.l0];
  const uint16_t* x;
  switch (it.phase) {
    case PH_Q: x = p.xq + (size_t)l * p.xq_l; break;
    case PH_O: x = p.ao + (size_t)l * p.ao_l; break;
    case PH_G: x = p.xm + (size_t)l * p.xm_l; break;
    default:   x = p.act + (size_t)l * p.act_l; break;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < p.B) {
      for (int e = 8 * lane; e < ne; e += 8 * kWave)
        *reinterpret_cast<u32x4*>(&sh.x[m][e]) = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + e0 + e);
    }
  }
  // epilogue operands: RMSNorm sums, residual, bias, gamma (used if this item finishes the tile)
  const int n64 = tile * kTileRows + lane;
  float e_ss[MT], e_h[MT], e_b = 0.f, e_gam = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    e_ss[m] = 0.f;
    e_h[m] = 0.f;
    if (m < p.B) {
      if ((it.phase == PH_Q || it.phase == PH_G) && lane < p.ntH)
        e_ss[m] = collect_f32((it.phase == PH_Q ? p.ssi : p.ssm) + (size_t)m * p.ntH + lane);
      if (it.phase == PH_O) e_h[m] = collect_f32(p.hin + (size_t)m * p.H + n64);
      if (it.phase == PH_D) e_h[m] = collect_f32(p.h1 + (size_t)m * p.H + n64);
    }
  }
  if (it.phase == PH_Q && lw.bias && n64 < p.nqkv) e_b = h2f(lw.bias[n64]);
  if (it.phase == PH_O) e_gam = h2f(lw.g2[n64]);
  if (it.phase == PH_D) {
    const uint16_t* gsrc = l + 1 == p.L ? p.gf : (l + 1 < p.l1 ? p.lw[l + 1 - p.l0].g1 : p.g1_next);
    e_gam = h2f(gsrc[n64]);
  }
  if (lane == 0) sh.idx[slot] = nn;
  __syncthreads();   // B1: activations staged (and the item after next handed over)
  __syncthreads();   // B2: the compute waves' sums are in LDS

  float tot[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) tot[m] = ((sh.red[0][m][lane] + sh.red[1][m][lane]) + sh.red[2][m][lane]) + sh.red[3][m][lane];

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

  // ---- epilogue (lane = row of the tile) ----
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
  if (lane == 0) {
    const unsigned prev = arrive(done);
    VV_STAT(const unsigned want = it.phase == PH_Q ? p.ntq : it.phase == PH_G ? p.ntg : p.ntH;
            if (prev + 1 == want) p.stats[(size_t)4096 * kStatWords + (size_t)l * 8 + it.phase] = wall_clock64();)
    (void)prev;
  }
}

// attention geometry shared by both roles
struct AGeo { int sa, bh, b, kvh, s0, P, npos; bool has_new; };
__device__ __forceinline__ int clamp_pos(const MParams& p, int P) { return P < 0 ? 0 : (P >= p.cap ? p.cap - 1 : P); }
// pos01: the clamped positions of sequences 0 and 1 (read once per launch: positions are inputs)
__device__ __forceinline__ AGeo ageo(const MParams& p, const Item& it, int2 pos01) {
  AGeo a;
  a.sa = it.j % p.nsa; a.bh = it.j / p.nsa;
  a.b = a.bh / p.nkv; a.kvh = a.bh % p.nkv;
  a.s0 = a.sa * kAS;
  a.P = a.b == 0 ? pos01.x : pos01.y;
  a.npos = max(0, min(a.s0 + kAS, a.P + 1) - a.s0);
  a.has_new = a.P >= a.s0 && a.P < a.s0 + a.npos;
  return a;
}

// attention: rotated q into LDS, the new position's k/v (cache slot written) | its scores |
// (softmax, P.V of the cached positions) | record with the new position's P.V, count in.
// The compute waves never see the new position's row: their payload came from the cache before
// the row was written, so the control wave scores it and adds its P.V itself.
template <int MT>
__device__ void attn_ctl(const MParams& p, const Item& it, Shared<MT>& sh, int lane, int2 pos01, int slot, int nn) {
  const AGeo a = ageo(p, it, pos01);
  const int g = p.g;
  unsigned* ca = lcnt(p, it.layer) + p.k_ca + a.bh;
  if (a.npos == 0) {                     // beyond the sequence: nothing to attend, only count
    if (lane == 0) sh.idx[slot] = nn;
    __syncthreads();   // S
    if (lane == 0) arrive(ca);
    return;
  }
  const float* row = p.qkv + (size_t)a.b * p.nqkv;
  float c = 1.f, s = 0.f;
  if (p.theta > 0.f) {
    c = collect_f32(p.rope + ((size_t)a.b * 64 + lane) * 2);
    s = collect_f32(p.rope + ((size_t)a.b * 64 + lane) * 2 + 1);
  }
  float q1[kMaxG], q2[kMaxG];
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh) {
    q1[hh] = 0.f; q2[hh] = 0.f;
    if (hh < g) {
      const float* qh = row + (size_t)(a.kvh * g + hh) * kD;
      q1[hh] = collect_f32(qh + lane);
      q2[hh] = collect_f32(qh + lane + 64);
    }
  }
  float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
  if (a.has_new) {
    const float* kh = row + (size_t)p.nq * kD + (size_t)a.kvh * kD;
    const float* vh = row + (size_t)(p.nq + p.nkv) * kD + (size_t)a.kvh * kD;
    k1 = collect_f32(kh + lane); k2 = collect_f32(kh + lane + 64);
    v1 = collect_f32(vh + lane); v2 = collect_f32(vh + lane + 64);
  }
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh) {
    const float r1 = q1[hh] * c - q2[hh] * s, r2 = q2[hh] * c + q1[hh] * s;
    q1[hh] = r1;
    q2[hh] = r2;
    if (hh < g) {
      sh.qs[hh][lane] = r1;
      sh.qs[hh][lane + 64] = r2;
    }
  }
  // the new position: fp16 k (rotated) and v, as the cache holds them
  const uint16_t ka = f2h(k1 * c - k2 * s), kb = f2h(k2 * c + k1 * s), va = f2h(v1), vb = f2h(v2);
  if (a.has_new) {
    const size_t base = (size_t)it.layer * p.kv_layer + ((size_t)a.bh * p.cap + a.P) * kD;
    p.kc[base + lane] = ka; p.kc[base + lane + 64] = kb;
    p.vc[base + lane] = va; p.vc[base + lane + 64] = vb;
  }
  const int jP = a.P - a.s0;
  if (lane == 0) sh.idx[slot] = nn;
  __syncthreads();   // B1: q in LDS (and the item after next handed over)
  if (a.has_new) {
    const float kf1 = h2f(ka), kf2 = h2f(kb);
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      if (hh < g) {
        const float sc = wave_sum(fmaf(q1[hh], kf1, q2[hh] * kf2));
        if (lane == 0) sh.sc[hh][jP] = sc * p.scale;
      }
    }
  }
  __syncthreads();   // B2: scores
  __syncthreads();   // B3: softmax statistics (probabilities in sh.sc)
  __syncthreads();   // B4: per-wave P.V of the cached positions
  float* rec = p.ap + ((size_t)a.bh * p.nsa + a.sa) * g * kPS;
  const float vf1 = h2f(va), vf2 = h2f(vb);
  for (int i = lane; i < g * kD; i += kWave) {
    const int hh = i >> 7, dd = i & 127;
    float o = ((sh.ared[0][hh][dd] + sh.ared[1][hh][dd]) + sh.ared[2][hh][dd]) + sh.ared[3][hh][dd];
    if (a.has_new) o = fmaf(sh.sc[hh][jP], dd < 64 ? vf1 : vf2, o);
    publish_f32(rec + (size_t)hh * kPS + 4 + dd, o);
  }
  if (lane < g) {
    publish_f32(rec + (size_t)lane * kPS, sh.mh[lane]);
    publish_f32(rec + (size_t)lane * kPS + 1, sh.lh[lane]);
  }
  wait_published();
  if (lane == 0) arrive(ca);
}

// merge (sequence, query head, 64-dim half): lane s holds split s's (m, l) for the weights
// e_s = exp(m_s - M), lane d accumulates sum_s e_s o_s[d]; splits in a fixed order.
template <int MT>
__device__ void merge_ctl(const MParams& p, const Item& it, Shared<MT>& sh, int lane, int slot, int nn) {
  constexpr int kChunk = 16;
  if (lane == 0) sh.idx[slot] = nn;
  __syncthreads();   // S: hand over, then let the compute waves go on
  const int l = it.layer;
  const int half = it.j & 1, bhq = it.j >> 1;
  const int b = bhq / p.nq, h = bhq % p.nq;
  const int kvh = h / p.g, hh = h % p.g;
  int Pp = p.pos[b];
  Pp = Pp < 0 ? 0 : (Pp >= p.cap ? p.cap - 1 : Pp);
  const int nv = (Pp + 1 + kAS - 1) / kAS;     // splits that hold positions
  const size_t stride = (size_t)p.g * kPS;
  const float* base = p.ap + (size_t)(b * p.nkv + kvh) * p.nsa * stride + (size_t)hh * kPS;
  const int dd = half * 64 + lane;
  float M = -INFINITY;
  for (int s0 = 0; s0 < nv; s0 += kWave) {
    const float m = s0 + lane < nv ? collect_f32(base + (size_t)(s0 + lane) * stride) : -INFINITY;
    M = fmaxf(M, wave_max(m));
  }
  float Lsum = 0.f, O = 0.f;
  for (int s0 = 0; s0 < nv; s0 += kWave) {
    float e = 0.f, lv = 0.f;
    if (s0 + lane < nv) {
      const float* r = base + (size_t)(s0 + lane) * stride;
      const float m = collect_f32(r);
      lv = collect_f32(r + 1);
      e = expf(m - M);
    }
    Lsum += wave_sum(e * lv);
    const int ns = min(kWave, nv - s0);
    for (int c0 = 0; c0 < ns; c0 += kChunk) {
      float oo[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k)
        oo[k] = c0 + k < ns ? collect_f32(base + (size_t)(s0 + c0 + k) * stride + 4 + dd) : 0.f;
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const float ek = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), c0 + k < ns ? c0 + k : 0));
        O = fmaf(c0 + k < ns ? ek : 0.f, oo[k], O);
      }
    }
  }
  uint16_t* ao = p.ao + (size_t)l * p.ao_l + ((size_t)b * p.nq + h) * kD;
  publish_u16(ao + dd, f2h(O / Lsum));
  wait_published();
  if (lane == 0) {
    const unsigned prev = arrive(lcnt(p, l) + p.k_dm);
    VV_STAT(if (prev + 1 == (unsigned)(2 * p.B * p.nq)) p.stats[(size_t)4096 * kStatWords + (size_t)l * 8 + PH_M] = wall_clock64();)
    (void)prev;
  }
}

// Next item of queue q (claims are in increasing order within a queue), or -1.
__device__ __forceinline__ int claim(const MParams& p, int q) {
  const int pos = (int)__hip_atomic_fetch_add(p.c_queue + q * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int i = pos * kQueues + q;
  return i < p.total ? i : -1;
}

template <int MT>
__device__ void ctl_loop(const MParams& p, Shared<MT>& sh, int lane) {
  int done_key = -1;
  const int2 pos01 = make_int2(clamp_pos(p, p.pos[0]), p.B > 1 ? clamp_pos(p, p.pos[1]) : 0);
  int q = 0, cur = -1, nxt = -1;
  if (lane == 0) {
    q = (int)(arrive(p.c_start) % (unsigned)kQueues);   // start order -> queue
    cur = claim(p, q);
    nxt = cur >= 0 ? claim(p, q) : -1;
    sh.idx[0] = cur;
    sh.idx[1] = nxt;
  }
  cur = __builtin_amdgcn_readfirstlane(cur);
  nxt = __builtin_amdgcn_readfirstlane(nxt);
  __syncthreads();   // S0: the first two items
  for (int t = 0; cur >= 0; ++t) {
    // claim the item after next now; it is handed to the compute waves at this item's first barrier
    int nn = -1;
    if (lane == 0 && nxt >= 0) nn = claim(p, q);
    const Item it = decode(p, cur);
    wait_dep(p, it, cur, done_key, true, lane);
    VV_STAT(const unsigned long long tw = wall_clock64();)
    const int slot = t & 1;
    switch (it.phase) {
      case PH_PREP: prep_ctl<MT>(p, sh, lane, slot, nn); break;
      case PH_A: attn_ctl<MT>(p, it, sh, lane, pos01, slot, nn); break;
      case PH_M: merge_ctl<MT>(p, it, sh, lane, slot, nn); break;
      default: gemv_ctl<MT>(p, it, sh, lane, slot, nn); break;
    }
    VV_STAT(if (lane == 0) {
      unsigned long long* st = p.stats + (size_t)blockIdx.x * kStatWords;
      st[16 + it.phase] += wall_clock64() - tw;
      st[25] += 1;
    })
    cur = nxt;
    nxt = __builtin_amdgcn_readfirstlane(nn);
  }
}

// ================================================================================================
// Compute waves
// ================================================================================================
template <int MT>
__device__ void gemv_compute(const MParams& p, const Item& it, const Pay& P, Shared<MT>& sh, int w, int lane,
                             uint32_t m64, int slot, int& nn) {
  const GDesc d = gdesc(p, it);
  const int sp = it.j % d.ns;
  const int b0 = (sp * kW + w) * kGB;
  const int nblk = min(max(d.nb - b0, 0), kGB);
  __syncthreads();   // B1: activations staged
  nn = __builtin_amdgcn_readfirstlane(sh.idx[slot]);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  if (nblk > 0) {
    const int xb0 = w * kGB * kBlock;          // this wave's first element within the item
    float corr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      u32x4 xv = u32x4{0, 0, 0, 0};
      if (m < p.B && lane < 4 * nblk) xv = *reinterpret_cast<const u32x4*>(&sh.x[m][xb0 + lane * 8]);
      corr[m] = quad_sum(corr_quarter(xv));
    }
#pragma unroll
    for (int i = 0; i < kGB; ++i) {
      if (i < nblk) {
        const float sc = pick_scale(P.s, i);
        const uint32_t dw[4] = {P.v[i].x, P.v[i].y, P.v[i].z, P.v[i].w};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < p.B) {
            const u32x4* xs = reinterpret_cast<const u32x4*>(&sh.x[m][xb0 + i * kBlock]);
            float t = -__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, corr[m]), 4 * i));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const u32x4 xv = xs[k];
              const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
              t = dot8_pairs(dw[k], x4, t, m64);
            }
            acc[m] = fmaf(sc, t, acc[m]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) sh.red[w][m][lane] = acc[m];
  __syncthreads();   // B2
}

// a * fp16(lo or hi half of h) + c in fp32 (v_fma_mix_f32: the fp16 operand is used exactly)
__device__ __forceinline__ float fma_mix_lo(float a, uint32_t h, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(h), "v"(c));
  return d;
}
__device__ __forceinline__ float fma_mix_hi(float a, uint32_t h, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(h), "v"(c));
  return d;
}
// sum_t a[t] * fp16 element t of the 8 packed in v, from c
__device__ __forceinline__ float dot8_mix(const float* a, const u32x4& v, float c) {
  c = fma_mix_lo(a[0], v.x, c); c = fma_mix_hi(a[1], v.x, c);
  c = fma_mix_lo(a[2], v.y, c); c = fma_mix_hi(a[3], v.y, c);
  c = fma_mix_lo(a[4], v.z, c); c = fma_mix_hi(a[5], v.z, c);
  c = fma_mix_lo(a[6], v.w, c); c = fma_mix_hi(a[7], v.w, c);
  return c;
}

__device__ __forceinline__ void h8_to_f32(const u32x4& v, float* f) {
  const uint32_t d4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2_t hv = as_h2(d4[i]);
    f[2 * i] = (float)hv.x;
    f[2 * i + 1] = (float)hv.y;
  }
}

// 4 passes of 4 positions per wave: lane = (position 4r + lane/16, dims 8 (lane%16) .. +7).
// The payload is only read; the new position (stale in the payload) is left to the control wave.
template <int MT>
__device__ void attn_compute(const MParams& p, const Item& it, const Pay& P, Shared<MT>& sh, int w, int lane,
                             int2 pos01, int slot, int& nn) {
  const AGeo a = ageo(p, it, pos01);
  __syncthreads();   // B1 (S for an empty item)
  nn = __builtin_amdgcn_readfirstlane(sh.idx[slot]);
  if (a.npos == 0) return;
  const int g = p.g;
  const int sl = lane & 15, pg = lane >> 4;
  const int jP = a.has_new ? a.P - a.s0 : -1;
  // scores: 16 lanes per position, reduced across the 16 (head loop kept rolled: registers)
#pragma unroll 1
  for (int hh = 0; hh < g; ++hh) {
    float q8[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q8[t] = sh.qs[hh][8 * sl + t];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sc = dot8_mix(q8, P.v[r], 0.f);
      sc = row16_sum(sc);
      const int j = w * 16 + 4 * r + pg;
      if (sl == 0 && j != jP) sh.sc[hh][j] = j < a.npos ? sc * p.scale : -INFINITY;
    }
  }
  __syncthreads();   // B2
  // split-local softmax statistics, one wave per head
  for (int hh = w; hh < g; hh += kW) {
    const float v = sh.sc[hh][lane];
    const float m = wave_max(v);
    const float e = (m == -INFINITY) ? 0.f : expf(v - m);
    const float sum = wave_sum(e);
    sh.sc[hh][lane] = e;
    if (lane == 0) { sh.mh[hh] = m; sh.lh[hh] = sum; }
  }
  __syncthreads();   // B3
  // P.V over the wave's 16 positions
#pragma unroll 1
  for (int hh = 0; hh < g; ++hh) {
    float acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = w * 16 + 4 * r + pg;
      const float pj = j == jP ? 0.f : sh.sc[hh][j];
      const u32x4 v = P.v[4 + r];
      acc[0] = fma_mix_lo(pj, v.x, acc[0]); acc[1] = fma_mix_hi(pj, v.x, acc[1]);
      acc[2] = fma_mix_lo(pj, v.y, acc[2]); acc[3] = fma_mix_hi(pj, v.y, acc[3]);
      acc[4] = fma_mix_lo(pj, v.z, acc[4]); acc[5] = fma_mix_hi(pj, v.z, acc[5]);
      acc[6] = fma_mix_lo(pj, v.w, acc[6]); acc[7] = fma_mix_hi(pj, v.w, acc[7]);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = rows_lanewise_sum(acc[t]);
      if (pg == 0) sh.ared[w][hh][8 * sl + t] = v;
    }
  }
  __syncthreads();   // B4
}

// Marks every register of a payload as used, so its loads are complete (waited for) by the end of
// the item whatever the item used; otherwise the next issue into these registers could be preceded
// by a wait for the whole queue, including the loads of the item after.
__device__ __forceinline__ void consume(const Pay& P) {
  asm volatile("" ::"v"(P.v[0]), "v"(P.v[1]), "v"(P.v[2]), "v"(P.v[3]), "v"(P.v[4]), "v"(P.v[5]), "v"(P.v[6]),
               "v"(P.v[7]), "v"(P.s));
}

template <int MT>
__device__ __forceinline__ void compute_item(const MParams& p, int cur, int nxt, Pay& C, Pay& N, Shared<MT>& sh,
                                             int& done_key, int w, int lane, uint32_t m64, int2 pos01, int slot,
                                             int& nn) {
  const Item it = decode(p, cur);
  // the next item's loads go out before the wait (a fixed count even when there is none)
  issue(p, nxt, N, w, lane);
  wait_dep(p, it, cur, done_key, false, lane);
  switch (it.phase) {
    case PH_PREP: case PH_M:           // control wave only: just the hand-over barrier
      __syncthreads();
      nn = __builtin_amdgcn_readfirstlane(sh.idx[slot]);
      break;
    case PH_A: attn_compute<MT>(p, it, C, sh, w, lane, pos01, slot, nn); break;
    default: gemv_compute<MT>(p, it, C, sh, w, lane, m64, slot, nn); break;
  }
  consume(C);
}

template <int MT>
__device__ void compute_loop(const MParams& p, Shared<MT>& sh, int w, int lane) {
  const uint32_t m64 = vconst(0x54005400u);
  int done_key = -1;
  // the only activation-side global loads of the compute waves: before any weight is in flight
  const int2 pos01 = make_int2(clamp_pos(p, p.pos[0]), p.B > 1 ? clamp_pos(p, p.pos[1]) : 0);
  __syncthreads();   // S0
  int cur = __builtin_amdgcn_readfirstlane(sh.idx[0]), nxt = __builtin_amdgcn_readfirstlane(sh.idx[1]);
  Pay A, B;
  issue(p, cur, A, w, lane);
  for (int t = 0; cur >= 0; t += 2) {
    int nn;
    compute_item<MT>(p, cur, nxt, A, B, sh, done_key, w, lane, m64, pos01, 0, nn);
    cur = nxt;
    nxt = nn;
    if (cur < 0) break;
    compute_item<MT>(p, cur, nxt, B, A, sh, done_key, w, lane, m64, pos01, 1, nn);
    cur = nxt;
    nxt = nn;
  }
}

template <int MT>
__global__ __launch_bounds__(kThr, 4) void k_decode_persistent(MParams arg) {
  // read the parameters in place from the kernel-argument segment (scalar loads): indexing the
  // per-layer table of a by-value copy would move the whole struct to scratch memory
#if defined(__HIP_DEVICE_COMPILE__)
  (void)arg;
  const MParams& p = *reinterpret_cast<const MParams*>(__builtin_amdgcn_kernarg_segment_ptr());
#else
  const MParams& p = arg;   // host pass: the body is never run there
#endif
  __shared__ Shared<MT> sh;
  const int w = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  VV_STAT(if (w == kCtl && lane == 0) p.stats[(size_t)blockIdx.x * kStatWords + 27] = wall_clock64();)
  if (w == kCtl) ctl_loop<MT>(p, sh, lane);
  else compute_loop<MT>(p, sh, w, lane);

  // leave; the last workgroup out resets this launch's counters
  __syncthreads();
  if (w == kCtl && lane == 0) sh.flag = arrive(p.c_exit) == (unsigned)(p.nwg - 1);
  __syncthreads();
  if (sh.flag) {
    unsigned* c0 = lcnt(p, p.l0);
    const size_t n = (size_t)(p.l1 - p.l0) * p.cpl;
    for (size_t i = threadIdx.x; i < n; i += kThr) reset_counter(c0 + i);
    if (threadIdx.x == 0) {
      if (p.l0 == 0) reset_counter(p.c_prep);
      reset_counter(p.c_exit);
      reset_counter(p.c_start);
      for (int q = 0; q < kQueues; ++q) reset_counter(p.c_queue + q * 32);
    }
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
  size_t hdr, queue, zero, rope, gfo, cnt, ssi, ssm, hin, h1, qkv, ap, pq, po, pg, pd, xq, xm, ao, act, total;
  size_t xq_l, xm_l, ao_l, act_l;
};

MLayout mlayout(const MDims& d) {
  MLayout y{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes, 256); return o; };
  const size_t B = d.B;
  y.hdr = take(4 * 128);
  y.queue = take((size_t)kQueues * 128);
  y.zero = take(1024);
  y.rope = take(B * 64 * 2 * 4);
  y.gfo = take(B * d.H * 4);
  y.cnt = take((size_t)d.L * d.cpl * 4);
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

struct Occ { int nwg = 0; bool done = false; };
Occ g_occ[64];
std::mutex g_occ_mu;

// workgroups that are resident at once on the current device
int resident_workgroups(int mt) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 32) return 0;
  const int slot = dev * 2 + (mt == 1 ? 0 : 1);
  std::lock_guard<std::mutex> lk(g_occ_mu);
  if (!g_occ[slot].done) {
    int cus = 0, per = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_decode_persistent<1>, kThr, 0);
    }
    g_occ[slot].nwg = (e == hipSuccess && cus > 0 && per > 0) ? cus * std::min(per, 4) : 0;
    g_occ[slot].done = true;
  }
  return g_occ[slot].nwg;
}

}  // namespace

int persistent_grid() { return resident_workgroups(1); }

bool persistent_supported(const vv_model* m, int batch) {
  return m->n_layers >= 1 && batch >= 1 && batch <= kMaxMT && m->hidden <= 64 * kTileRows &&
         m->n_q / m->n_kv <= kMaxG;
}

size_t persistent_workspace_bytes(const vv_model* m, int batch, int cap) {
  return mlayout(mdims(m, batch, cap)).total;
}

int persistent_enqueue(const vv_model* m, const vv_state* s, char* ws, hipStream_t st, void** events, int* ev) {
  const MDims d = mdims(m, s->batch, s->cap);
  const MLayout y = mlayout(d);
  const int nwg = resident_workgroups(1);
  VV_REQUIRE(nwg > 0, VV_ERR_HIP, "persistent decode: could not size the resident grid");
  MParams p{};
  p.L = d.L; p.B = d.B; p.H = d.H; p.I = d.I; p.nq = d.nq; p.nkv = d.nkv; p.g = d.g; p.cap = d.cap;
  p.nqkv = d.nqkv; p.ntH = d.ntH;
  p.eps = m->eps; p.inv_h = 1.0f / (float)d.H; p.scale = 1.0f / sqrtf((float)kD); p.theta = m->rope_theta;
  p.emb = s->input_embeds; p.pos = s->pos; p.kc = s->k_cache; p.vc = s->v_cache;
  p.kv_layer = (size_t)d.B * d.nkv * (size_t)d.cap * kD;
  p.gf = m->gf; p.trace = s->h_trace;
  p.ntq = d.ntq; p.ntg = d.ntg;
  p.nbq = d.nbq; p.nbo = d.nbo; p.nbg = d.nbg; p.nbd = d.nbd;
  p.nsq = d.nsq; p.nso = d.nso; p.nsg = d.nsg; p.nsd = d.nsd; p.nsa = d.nsa;
  p.nQ = d.ntq * d.nsq; p.nA = d.B * d.nkv * d.nsa; p.nM = 2 * d.B * d.nq;
  p.nO = d.ntH * d.nso; p.nG = d.ntg * d.nsg; p.nD = d.ntH * d.nsd;
  p.T = p.nQ + p.nA + p.nM + p.nO + p.nG + p.nD;
  p.err = reinterpret_cast<unsigned*>(ws + y.hdr);
  p.c_prep = reinterpret_cast<unsigned*>(ws + y.hdr + 128);
  p.c_exit = reinterpret_cast<unsigned*>(ws + y.hdr + 256);
  p.c_start = reinterpret_cast<unsigned*>(ws + y.hdr + 384);
  p.c_queue = reinterpret_cast<unsigned*>(ws + y.queue);
  p.cnt = reinterpret_cast<unsigned*>(ws + y.cnt);
  p.cpl = d.cpl;
  p.k_cq = 0; p.k_co = d.ntq; p.k_cg = p.k_co + d.ntH; p.k_cd = p.k_cg + d.ntg; p.k_ca = p.k_cd + d.ntH;
  const int ph0 = (int)align_up((size_t)p.k_ca + (size_t)d.B * d.nkv, kPad);
  p.k_dq = ph0; p.k_dm = ph0 + kPad; p.k_do = ph0 + 2 * kPad; p.k_dg = ph0 + 3 * kPad; p.k_dd = ph0 + 4 * kPad;
  p.rope = reinterpret_cast<float*>(ws + y.rope);
  p.zero = reinterpret_cast<const u32x4*>(ws + y.zero);
#ifdef VV_STATS
  VV_HIP(hipGetSymbolAddress(reinterpret_cast<void**>(&p.stats), HIP_SYMBOL(g_vv_stats)));
#endif
  p.gfo = reinterpret_cast<float*>(ws + y.gfo);
  p.ssi = reinterpret_cast<float*>(ws + y.ssi); p.ssm = reinterpret_cast<float*>(ws + y.ssm);
  p.hin = reinterpret_cast<float*>(ws + y.hin); p.h1 = reinterpret_cast<float*>(ws + y.h1);
  p.qkv = reinterpret_cast<float*>(ws + y.qkv); p.ap = reinterpret_cast<float*>(ws + y.ap);
  p.pq = reinterpret_cast<float*>(ws + y.pq); p.po = reinterpret_cast<float*>(ws + y.po);
  p.pg = reinterpret_cast<float*>(ws + y.pg); p.pd = reinterpret_cast<float*>(ws + y.pd);
  p.xq = reinterpret_cast<uint16_t*>(ws + y.xq); p.xm = reinterpret_cast<uint16_t*>(ws + y.xm);
  p.ao = reinterpret_cast<uint16_t*>(ws + y.ao); p.act = reinterpret_cast<uint16_t*>(ws + y.act);
  p.xq_l = y.xq_l; p.xm_l = y.xm_l; p.ao_l = y.ao_l; p.act_l = y.act_l;
  p.nwg = nwg;

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
    if (events) VV_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(events[(*ev)++]), st));
    hipLaunchKernelGGL(k_decode_persistent<1>, dim3(nwg), dim3(kThr), 0, st, p);
    VV_HIP(hipGetLastError());
  }
  return VV_OK;
}

// inputs of the lm_head after the persistent layers: gamma_f * h (fp32) and per-tile sums of h^2
void persistent_lm_inputs(const vv_model* m, const vv_state* s, char* ws, const float** gf32, const float** sumsq) {
  const MDims d = mdims(m, s->batch, s->cap);
  const MLayout y = mlayout(d);
  *gf32 = reinterpret_cast<const float*>(ws + y.gfo);
  *sumsq = reinterpret_cast<const float*>(ws + y.ssi);
}


}  // namespace vv

#ifdef VV_STATS
extern "C" int vv_stats_copy(unsigned long long* host, size_t n, int clear) {
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(vv::g_vv_stats), n * 8) != hipSuccess) return -1;
  if (clear) {
    static unsigned long long zeros[4096 * 32 + 256 * 8];
    if (hipMemcpyToSymbol(HIP_SYMBOL(vv::g_vv_stats), zeros, sizeof(zeros)) != hipSuccess) return -1;
  }
  return 0;
}
#endif
