// Decode-step launcher and its hipGraph wrapper.
//
// decoder_step contract ("vibevoice-asr-bitnet-onnx" page, graph contracts):
//   input_embeds [B,H], position_ids [B], past K/V -> logits [B,V], present K/V (one more slot)
// on the Qwen2 layer of the 1.5B STATUS page (Architecture): pre-RMSNorm, q/k/v bias, GQA,
// SiLU-gated MLP, residual adds.  The layered plan is 1 + 5 L + 1 kernels:
//   prep (embeddings -> residual stream, RoPE table)
//   per layer: QKV GEMV (RMSNorm folded in) | attention (+RoPE, KV append) and its split merge
//              (a kernel of its own, or at batch 1 over fp16 caches the leading workgroups of the
//              o GEMV's launch) | o GEMV + residual | gate/up GEMV + SiLU*up | down GEMV + residual
//   lm_head + argmax (final RMSNorm folded in).
// At batch 1 each down GEMV shares its launch with the next layer's QKV GEMV (the chained GEMV
// segments of chain.hip: the QKV workgroups stream their weights while down finishes, then wait
// for its tagged output), so a step is 2 + 4 L + 1 launches.  The chained plan (enqueue_chain_step)
// goes further for narrow models.
// RMSNorm is folded into the GEMVs: the producer of h writes fp16(gamma * h) and per-tile sums of
// h^2; the consumer scales its row sums by rstd = 1/sqrt(mean(h^2) + eps).  Positions are read
// from device memory, so one captured graph serves every step.
#include <new>
#include <vector>

#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kHeadDim = 128;

// h = fp32(input_embeds); g = gamma * h in fp32 (g_f32) or fp16, or gf = gamma * h in fp32 when
// there are no layers; per-tile sum of h^2; optional trace; RoPE (cos, sin) of pos[b] for the 64
// pairs.
__global__ __launch_bounds__(64) void k_step_prep(const uint16_t* __restrict__ emb, int H, int ntiles,
                                                  const uint16_t* __restrict__ gamma, float* __restrict__ h,
                                                  void* __restrict__ g, int g_f32, float* __restrict__ gf,
                                                  float* __restrict__ sumsq, float* __restrict__ trace,
                                                  const int32_t* __restrict__ pos, int cap, double theta,
                                                  float* __restrict__ rope) {
  const int t = blockIdx.x % ntiles, b = blockIdx.x / ntiles;
  const int lane = threadIdx.x;
  const int n = t * 64 + lane;
  const size_t i = (size_t)b * H + n;
  const float hv = h2f(emb[i]);
  h[i] = hv;
  if (trace) trace[i] = hv;
  const float gv = h2f(gamma[n]) * hv;
  if (g) {
    if (g_f32) static_cast<float*>(g)[i] = gv;
    else static_cast<uint16_t*>(g)[i] = f2h(gv);
  }
  if (gf) gf[i] = gv;
  const float ss = wave_sum(hv * hv);
  if (lane == 0) sumsq[(size_t)b * ntiles + t] = ss;
  if (t == 0 && theta > 0.0) {
    int P = pos[b];
    P = P < 0 ? 0 : (P >= cap ? cap - 1 : P);
    const double inv = pow(theta, -(double)(2 * lane) / (double)kHeadDim);
    double s, c;
    sincos((double)P * inv, &s, &c);
    rope[((size_t)b * 64 + lane) * 2] = (float)c;
    rope[((size_t)b * 64 + lane) * 2 + 1] = (float)s;
  }
}

// Greedy feedback for closed-loop decoding (one workgroup per sequence): record the token, stop
// on a stop id, else gather the token's embedding row as the next input and advance the position.
struct StopIds { int32_t id[4]; int n; };

__global__ __launch_bounds__(256) void k_feedback(const int32_t* __restrict__ token, const uint16_t* __restrict__ table,
                                                  int V, int H, uint16_t* __restrict__ emb, int32_t* __restrict__ pos,
                                                  int cap, int32_t* __restrict__ history, int32_t* __restrict__ done,
                                                  StopIds stop) {
  __shared__ int s_adv, s_tok;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const int tok = token[b];
    int P = pos[b];
    P = P < 0 ? 0 : (P >= cap ? cap - 1 : P);
    const bool active = done == nullptr || done[b] == 0;
    bool stopped = false;
    for (int i = 0; i < stop.n; ++i) stopped |= tok == stop.id[i];
    if (active && history) history[(size_t)b * cap + P] = tok;
    if (active && stopped && done) done[b] = 1;
    const bool adv = active && !stopped && P + 1 < cap && tok >= 0 && tok < V;
    if (adv) pos[b] = P + 1;
    s_adv = adv;
    s_tok = tok;
  }
  __syncthreads();
  if (!s_adv) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(table + (size_t)s_tok * H);
  u32x4* dst = reinterpret_cast<u32x4*>(emb + (size_t)b * H);
  for (int i = threadIdx.x; i < H / 8; i += blockDim.x) dst[i] = src[i];
}

struct Layout {
  size_t status, h, g, gf, qkv, o, act, sumsq, rope, ws_qkv, ws_o, ws_gu, ws_down, ws_attn, ws_lm, otag, epoch;
  size_t th, txq, tssq, txm, tssm, txo, txd;   // tagged words of the chained path (batch 1)
  size_t total;
};

struct Dims {
  int L, H, I, nq, nkv, V, B, cap, nqkv, ntH, ntI;
};

Dims dims_of(const vv_model* m, int B, int cap) {
  Dims d;
  d.L = m->n_layers; d.H = m->hidden; d.I = m->inter; d.nq = m->n_q; d.nkv = m->n_kv; d.V = m->vocab;
  d.B = B; d.cap = cap;
  d.nqkv = (m->n_q + 2 * m->n_kv) * kHeadDim;
  d.ntH = m->hidden / kTileRows;
  d.ntI = m->inter / kTileRows;
  return d;
}

Layout layout_of(const Dims& d) {
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes, 256); return o; };
  l.status = take(sizeof(int32_t));   // sticky status word: a bounded wait that gave up sets it
  l.h = take((size_t)d.B * d.H * 4);
  l.g = take((size_t)d.B * d.H * 4);                // activations: fp32 below the matrix-core batch, else fp16
  l.gf = take((size_t)d.B * d.H * 4);
  l.qkv = take((size_t)d.B * d.nqkv * 4);
  l.o = take((size_t)d.B * d.nq * kHeadDim * 4);
  l.act = take((size_t)d.B * d.I * 4);
  l.sumsq = take((size_t)d.B * d.ntH * 4);
  l.rope = take((size_t)d.B * 64 * 2 * 4);
  l.ws_qkv = take(gemv_workspace_bytes(d.B, (int)cdiv(d.nqkv, kTileRows), d.H / kBlock));
  l.ws_o = take(gemv_workspace_bytes(d.B, d.ntH, d.nq * kHeadDim / kBlock));
  l.ws_gu = take(gemv_workspace_bytes(d.B, 2 * d.ntI, d.H / kBlock));
  l.ws_down = take(gemv_workspace_bytes(d.B, d.ntH, d.I / kBlock));
  AttnParams ap{};
  ap.B = d.B; ap.nq = d.nq; ap.nkv = d.nkv; ap.cap = d.cap;
  attn_plan(ap);
  l.ws_attn = take(attn_workspace_bytes(d.B, d.nq, d.nkv, ap.nsplit));
  l.ws_lm = take(lm_workspace_bytes(d.B, d.V, d.H));
  l.otag = take((size_t)d.B * d.nq * kHeadDim * sizeof(uint64_t));   // fused merge -> o projection
  l.epoch = take(sizeof(uint32_t));                              // step counter (tags of otag)
  l.th = take((size_t)d.H * 8);
  l.txq = take((size_t)d.H * 8);
  l.tssq = take((size_t)d.ntH * 8);
  l.txm = take((size_t)d.H * 8);
  l.tssm = take((size_t)d.ntH * 8);
  l.txo = take((size_t)d.nq * kHeadDim * 8);
  l.txd = take((size_t)d.I * 8);
  l.total = off;
  return l;
}

size_t step_bytes(const vv_model* m, int B, int cap) { return align_up(layout_of(dims_of(m, B, cap)).total, 256); }

// The chained path (three launches per layer, four for wide models) serves batch 1 over fp16
// caches with 2..128 attention splits; everything else takes the layered path (five launches per
// layer, four at batch 1).
bool chain_supported(const vv_model* m, const vv_state* s) {
  if (s->batch != 1 || s->kv_dtype == VV_F32 || m->n_layers < 1) return false;
  AttnParams a{};
  a.B = 1; a.nq = m->n_q; a.nkv = m->n_kv; a.cap = s->cap;
  attn_plan(a);
  return a.nsplit >= 2 && a.nsplit <= kChainMaxSplits;
}

// AUTO takes the chained plan where it serves the state and the model is narrow (hidden <= 2048):
// there the stages are small and the hops it saves dominate (1.5B-shaped step 935 against 1037 us
// on MI355X); at the 7B width a segment's waves cannot all be resident, and those waiting for
// their inputs hold the places that later weight streams need (1705 against 1561 us with every
// stage of a layer chained, 1648 with the three-launch plan), so the layered plan stays.
constexpr int kChainAutoMaxHidden = 2048;
// wide models: the gate/up grid is more than one round of resident workgroups on its own
bool chain_split_mlp(const vv_model* m) { return m->hidden > kChainAutoMaxHidden; }
bool use_chain(const vv_model* m, const vv_state* s) {
  if (s->path == VV_PATH_CHAINED) return true;
  return s->path == VV_PATH_AUTO && m->hidden <= kChainAutoMaxHidden && chain_supported(m, s);
}

// timed operations of one step (two events each): prep, then per layer q|k|v, attention, o,
// gate/up, down, then the lm_head (at batch 1: prep, q|k|v of layer 0, per layer attention, o,
// gate/up, [down | next q|k|v], then the lm_head); chained: prep + q|k|v of layer 0, per layer
// attention, [merge | o] and [gate/up | down | next q|k|v] (wide models: [gate/up], [down | next
// q|k|v]), then the lm_head
// The layered plan at batch 1 (fp32 activations, the chained GEMV segments' batch) runs each down
// projection together with the next layer's q|k|v in one launch: 4 launches per layer after the
// first layer's q|k|v.
bool layered_fuses_down_qkv(const vv_state* s) { return s->batch == 1; }

int step_ops(const vv_model* m, const vv_state* s) {
  if (!use_chain(m, s)) return layered_fuses_down_qkv(s) && m->n_layers > 0 ? 4 * m->n_layers + 3 : 5 * m->n_layers + 2;
  return (chain_split_mlp(m) ? 4 : 3) * m->n_layers + 2;
}

int validate(const vv_model* m, const vv_state* s, const char* fn) {
  VV_REQUIRE(m && s, VV_ERR_NULL, "%s: model or state is NULL", fn);
  VV_REQUIRE(m->n_layers >= 0 && m->n_layers <= 4096, VV_ERR_RANGE, "%s: n_layers out of range", fn);
  VV_REQUIRE(m->head_dim == kHeadDim, VV_ERR_SHAPE, "%s: head_dim %d != 128", fn, m->head_dim);
  VV_REQUIRE(m->hidden >= 64 && m->hidden % 64 == 0 && m->hidden <= 4096, VV_ERR_SHAPE,
             "%s: hidden %d must be a multiple of 64 in [64, 4096]", fn, m->hidden);
  VV_REQUIRE(m->inter >= 64 && m->inter % 64 == 0 && m->inter <= (1 << 20), VV_ERR_SHAPE,
             "%s: inter %d must be a positive multiple of 64", fn, m->inter);
  VV_REQUIRE(m->n_q >= 1 && m->n_kv >= 1 && m->n_q % m->n_kv == 0 && m->n_q / m->n_kv <= 8, VV_ERR_SHAPE,
             "%s: n_q %% n_kv must be 0 with n_q/n_kv <= 8", fn);
  VV_REQUIRE(m->vocab >= 1, VV_ERR_RANGE, "%s: vocab < 1", fn);
  VV_REQUIRE(lm_table_fits(m->vocab, m->hidden), VV_ERR_RANGE, "%s: the %d x %d lm_head exceeds %lld bytes", fn,
             m->vocab, m->hidden, (long long)kLmMaxTableBytes);
  VV_REQUIRE(m->max_batch >= 1 && m->max_batch <= 16, VV_ERR_RANGE, "%s: max_batch not in 1..16", fn);
  VV_REQUIRE(m->eps >= 0.f, VV_ERR_RANGE, "%s: eps < 0", fn);
  VV_REQUIRE(m->gf && m->lm_head, VV_ERR_NULL, "%s: gf or lm_head is NULL", fn);
  VV_REQUIRE(m->n_layers == 0 || m->layers, VV_ERR_NULL, "%s: layers is NULL", fn);
  for (int l = 0; l < m->n_layers; ++l) {
    const vv_layer& y = m->layers[l];
    VV_REQUIRE(y.qkv_q && y.qkv_s && y.o_q && y.o_s && y.gu_q && y.gu_s && y.down_q && y.down_s && y.g1 && y.g2,
               VV_ERR_NULL, "%s: layer %d has a NULL weight pointer", fn, l);
    const uintptr_t a = reinterpret_cast<uintptr_t>(y.qkv_q) | reinterpret_cast<uintptr_t>(y.qkv_s) |
                        reinterpret_cast<uintptr_t>(y.o_q) | reinterpret_cast<uintptr_t>(y.o_s) |
                        reinterpret_cast<uintptr_t>(y.gu_q) | reinterpret_cast<uintptr_t>(y.gu_s) |
                        reinterpret_cast<uintptr_t>(y.down_q) | reinterpret_cast<uintptr_t>(y.down_s);
    VV_REQUIRE((a & 15) == 0, VV_ERR_RANGE, "%s: layer %d weights must be 16-byte aligned", fn, l);
  }
  VV_REQUIRE((reinterpret_cast<uintptr_t>(m->lm_head) & 15) == 0, VV_ERR_RANGE, "%s: lm_head must be 16-byte aligned",
             fn);
  VV_REQUIRE(s->batch >= 1 && s->batch <= m->max_batch, VV_ERR_RANGE, "%s: batch %d not in 1..max_batch", fn,
             s->batch);
  VV_REQUIRE(s->cap >= 1 && s->cap <= 131072, VV_ERR_RANGE, "%s: cap %d not in 1..131072", fn, s->cap);
  VV_REQUIRE(s->input_embeds && s->pos && s->token, VV_ERR_NULL, "%s: input_embeds, pos or token is NULL", fn);
  VV_REQUIRE(m->n_layers == 0 || (s->k_cache && s->v_cache), VV_ERR_NULL, "%s: KV cache is NULL", fn);
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(s->k_cache) | reinterpret_cast<uintptr_t>(s->v_cache)) & 15) == 0,
             VV_ERR_RANGE, "%s: KV caches must be 16-byte aligned", fn);
  VV_REQUIRE(s->path == VV_PATH_AUTO || s->path == VV_PATH_LAYERED || s->path == VV_PATH_CHAINED, VV_ERR_RANGE,
             "%s: unknown path %d", fn, s->path);
  VV_REQUIRE(s->n_stop >= 0 && s->n_stop <= 4, VV_ERR_RANGE, "%s: n_stop %d not in 0..4", fn, s->n_stop);
  VV_REQUIRE(s->kv_dtype == 0 || s->kv_dtype == VV_F16 || s->kv_dtype == VV_F32, VV_ERR_DTYPE,
             "%s: kv_dtype %d is not VV_F16 or VV_F32", fn, s->kv_dtype);
  VV_REQUIRE(!s->feedback_table || (reinterpret_cast<uintptr_t>(s->feedback_table) & 15) == 0, VV_ERR_RANGE,
             "%s: feedback_table must be 16-byte aligned", fn);
  const size_t need = step_bytes(m, s->batch, s->cap);
  VV_REQUIRE(s->workspace && s->workspace_bytes >= need, VV_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn,
             need);
  VV_REQUIRE((reinterpret_cast<uintptr_t>(s->workspace) & 255) == 0, VV_ERR_RANGE,
             "%s: workspace must be 256-byte aligned", fn);
  VV_REQUIRE(s->path != VV_PATH_CHAINED || chain_supported(m, s), VV_ERR_UNSUPPORTED,
             "%s: the chained path needs batch 1, fp16 caches, >= 1 layer and 2..%d attention splits", fn,
             kChainMaxSplits);
  const int nev = 2 * step_ops(m, s);
  VV_REQUIRE(!s->events || s->n_events >= nev, VV_ERR_RANGE, "%s: events needs at least %d entries", fn, nev);
  return VV_OK;
}

int enqueue_lm(const vv_model* m, const vv_state* s, const float* gf32, const float* sumsq, char* ws_lm,
               int32_t* status, uint32_t* epoch, hipStream_t st, KEv ev) {
  LmParams p{};
  p.status = status;
  p.epoch = epoch;
  p.W = m->lm_head; p.V = m->vocab; p.H = m->hidden; p.B = s->batch;
  p.x = gf32; p.x_f16 = 0;
  p.rs_parts = sumsq; p.rs_nparts = m->hidden / kTileRows; p.rs_inv_n = 1.0f / (float)m->hidden; p.eps = m->eps;
  p.logits = s->logits; p.token = s->token;
  lm_plan(p);
  lm_set_workspace(p, ws_lm);
  VV_HIP(lm_launch(p, st, ev));
  return VV_OK;
}

// event pair i of the state's timing events (both null when timing is off)
KEv event_pair(const vv_state* s, int i) {
  if (!s->events) return KEv{};
  return KEv{reinterpret_cast<hipEvent_t>(s->events[2 * i]), reinterpret_cast<hipEvent_t>(s->events[2 * i + 1])};
}

// closed-loop feedback after the argmax (when requested)
int enqueue_feedback(const vv_model* m, const vv_state* s, hipStream_t st) {
  if (!s->feedback_table) return VV_OK;
  StopIds stop{};
  stop.n = s->n_stop;
  for (int i = 0; i < s->n_stop; ++i) stop.id[i] = s->stop_ids[i];
  hipLaunchKernelGGL(k_feedback, dim3(s->batch), dim3(256), 0, st, s->token, s->feedback_table, m->vocab, m->hidden,
                     const_cast<uint16_t*>(s->input_embeds), const_cast<int32_t*>(s->pos), s->cap, s->history, s->done,
                     stop);
  VV_HIP(hipGetLastError());
  return VV_OK;
}

// The chained path: [prep | q|k|v(0)], then per layer the attention, [merge | o] and [gate/up |
// down | q|k|v(l+1)] (wide models: [gate/up] and [down | q|k|v(l+1)]), then the lm_head.  Tags: stage st of layer l is 1 + 4 l + st (st: 0 the
// q|k|v input and residual, 1 the attention output, 2 the MLP input and residual, 3 SiLU * up),
// added to epoch * (4 (L + 1) + 1); the epoch advances at the end of every step.
int enqueue_chain_step(const vv_model* m, const vv_state* s, hipStream_t st) {
  const Dims d = dims_of(m, 1, s->cap);
  const Layout lay = layout_of(d);
  char* ws = static_cast<char*>(s->workspace);
  auto U64 = [&](size_t off) { return reinterpret_cast<uint64_t*>(ws + off); };
  float* qkv = reinterpret_cast<float*>(ws + lay.qkv);
  float* gf = reinterpret_cast<float*>(ws + lay.gf);
  float* sumsq = reinterpret_cast<float*>(ws + lay.sumsq);
  float* rope = reinterpret_cast<float*>(ws + lay.rope);
  int32_t* status = reinterpret_cast<int32_t*>(ws + lay.status);
  uint32_t* epoch = reinterpret_cast<uint32_t*>(ws + lay.epoch);
  const int L = d.L, H = d.H;
  auto tagadd = [](int l, int stage) { return (uint32_t)(1 + 4 * l + stage); };
  enum { XQ = 0, XO = 1, XM = 2, XD = 3 };

  ChainParams base{};
  base.h = U64(lay.th); base.H = H; base.eps = m->eps; base.inv_h = 1.0f / (float)H;
  base.epoch = epoch; base.tag_mul = 4u * (uint32_t)(L + 1) + 1u; base.status = status;
  base.pos = s->pos; base.cap = s->cap;

  AttnParams a{};
  a.B = 1; a.nq = d.nq; a.nkv = d.nkv; a.cap = s->cap;
  attn_plan(a);
  attn_set_workspace(a, ws + lay.ws_attn);

  auto gemv_seg = [&](int kind, const uint8_t* q, const uint16_t* sc, int N, int K, int ntiles, size_t slots) {
    CSeg g{};
    g.kind = kind;
    g.q = reinterpret_cast<const u32x4*>(q); g.s = reinterpret_cast<const u32x4*>(sc);
    g.N = N; g.K = K; g.ntiles = ntiles;
    g.slots = U64(slots);
    g.ss_n = d.ntH;
    chain_gemv_plan(g);
    return g;
  };
  auto qkv_seg = [&](int l) {
    const vv_layer& y = m->layers[l];
    CSeg g = gemv_seg(SEG_QKV, y.qkv_q, y.qkv_s, d.nqkv, H, (int)cdiv(d.nqkv, kTileRows), lay.ws_qkv);
    g.xin = U64(lay.txq); g.xin_add = tagadd(l, XQ);
    g.ssin = U64(lay.tssq); g.ss_add = tagadd(l, XQ);
    g.has_bias = y.qkv_bias != nullptr;
    g.bias = y.qkv_bias ? y.qkv_bias : y.g1;      // a readable stand-in when there is no bias
    g.y = qkv;
    return g;
  };

  int op = 0;
  {  // launch 0: prep + q|k|v of layer 0
    ChainParams P = base;
    P.prep_add = tagadd(0, XQ);
    P.emb = s->input_embeds; P.g1 = m->layers[0].g1;
    P.xq = U64(lay.txq); P.ssq = U64(lay.tssq); P.trace0 = s->h_trace;
    P.rope_on = m->rope_theta > 0.f;
    P.rope = rope;
    for (int i = 0; i < 64; ++i) P.inv_freq[i] = P.rope_on ? pow((double)m->rope_theta, -(double)(2 * i) / 128.0) : 0.0;
    CSeg pg{};
    pg.kind = SEG_PREP;
    pg.blocks = (int)(cdiv(cdiv(d.ntH, kChainWaves), kNumXcd) * kNumXcd);
    P.seg[0] = pg;
    P.seg[1] = qkv_seg(0);
    P.nseg = 2;
    VV_HIP(chain_launch(P, st, event_pair(s, op++)));
  }
  const size_t layer_kv_bytes = (size_t)d.nkv * (size_t)s->cap * kHeadDim * 2;
  const bool split_mlp = chain_split_mlp(m);
  for (int l = 0; l < L; ++l) {
    const vv_layer& y = m->layers[l];
    const bool last = l == L - 1;
    {  // attention with RoPE and KV append; its split records are merged by the next launch
      AttnParams ap = a;
      ap.skip_merge = 1;
      ap.qkv = qkv; ap.ldqkv = d.nqkv; ap.pos = s->pos; ap.rope_theta = m->rope_theta;
      ap.kc = static_cast<char*>(s->k_cache) + (size_t)l * layer_kv_bytes;
      ap.vc = static_cast<char*>(s->v_cache) + (size_t)l * layer_kv_bytes;
      ap.kv_f32 = 0;
      ap.scale = 1.0f / sqrtf((float)kHeadDim);
      ap.out = nullptr; ap.out_f16 = 1;
      VV_HIP(attn_launch_with_rope(ap, rope, st, event_pair(s, op++)));
    }
    {  // [merge | o]: the split records -> the attention output -> o + residual, the MLP's input
      ChainParams P = base;
      P.part = a.part; P.nsplit = a.nsplit; P.split = a.split; P.nq = d.nq; P.nkv = d.nkv;
      P.xo = U64(lay.txo); P.mrg_add = tagadd(l, XO);
      CSeg mg{};
      mg.kind = SEG_MERGE;
      mg.blocks = (int)(cdiv(d.nq, kNumXcd) * kNumXcd);
      P.seg[0] = mg;
      CSeg g = gemv_seg(SEG_O, y.o_q, y.o_s, H, d.nq * kHeadDim, d.ntH, lay.ws_o);
      g.xin = U64(lay.txo); g.xin_add = tagadd(l, XO);
      g.hin_add = tagadd(l, XQ); g.out_add = tagadd(l, XM);
      g.gamma = y.g2; g.xgout = U64(lay.txm); g.ssout = U64(lay.tssm);
      P.seg[1] = g;
      P.nseg = 2;
      VV_HIP(chain_launch(P, st, event_pair(s, op++)));
    }
    {  // [gate/up | down | q|k|v(l+1)], or (wide models) [gate/up] and [down | q|k|v(l+1)]
      ChainParams P = base;
      CSeg g = gemv_seg(SEG_GU, y.gu_q, y.gu_s, d.I, H, 2 * d.ntI, lay.ws_gu);   // + SiLU * up
      g.xin = U64(lay.txm); g.xin_add = tagadd(l, XM);
      g.ssin = U64(lay.tssm); g.ss_add = tagadd(l, XM);
      g.act = U64(lay.txd); g.out_add = tagadd(l, XD);
      P.seg[0] = g;
      P.nseg = 1;
      if (split_mlp) {
        VV_HIP(chain_launch(P, st, event_pair(s, op++)));
        P = base;
        P.nseg = 0;
      }
      g = gemv_seg(SEG_DOWN, y.down_q, y.down_s, H, d.I, d.ntH, lay.ws_down);   // + residual
      g.xin = U64(lay.txd); g.xin_add = tagadd(l, XD);
      g.hin_add = tagadd(l, XM); g.out_add = tagadd(l + 1, XQ);
      g.gamma = last ? m->gf : m->layers[l + 1].g1;
      if (!last) { g.xgout = U64(lay.txq); g.ssout = U64(lay.tssq); }
      else { g.gf = gf; g.sumsq = sumsq; }
      g.trace = s->h_trace ? s->h_trace + (size_t)(l + 1) * H : nullptr;
      P.seg[P.nseg++] = g;
      if (!last) P.seg[P.nseg++] = qkv_seg(l + 1);
      VV_HIP(chain_launch(P, st, event_pair(s, op++)));
    }
  }
  const int rc = enqueue_lm(m, s, gf, sumsq, ws + lay.ws_lm, status, epoch, st, event_pair(s, op++));
  if (rc) return rc;
  return enqueue_feedback(m, s, st);
}

int enqueue_step(const vv_model* m, const vv_state* s, hipStream_t st) {
  if (use_chain(m, s)) return enqueue_chain_step(m, s, st);
  const Dims d = dims_of(m, s->batch, s->cap);
  const Layout lay = layout_of(d);
  char* ws = static_cast<char*>(s->workspace);
  float* h = reinterpret_cast<float*>(ws + lay.h);
  void* g = ws + lay.g;
  float* gf = reinterpret_cast<float*>(ws + lay.gf);
  float* qkv = reinterpret_cast<float*>(ws + lay.qkv);
  void* o = ws + lay.o;
  void* act = ws + lay.act;
  // the projections' inputs: fp32 for the vector-ALU GEMV (staged as fp16 hi + lo parts, so the
  // activations keep fp32 precision), fp16 for the matrix-core GEMV of batches >= 5
  const int xf32 = s->batch < kGemvMfmaMinM;
  float* sumsq = reinterpret_cast<float*>(ws + lay.sumsq);
  float* rope = reinterpret_cast<float*>(ws + lay.rope);
  const int B = d.B, H = d.H;
  const float inv_h = 1.0f / (float)H;
  // the step's sticky status word: a bounded wait (split-K hand-off, fused merge, argmax) that
  // gives up sets it
  int32_t* status = reinterpret_cast<int32_t*>(ws + lay.status);
  int op = 0;   // timing event pair of the next operation
  VV_LAUNCH(k_step_prep, dim3(B * d.ntH), dim3(64), st, event_pair(s, op++), s->input_embeds, H, d.ntH,
            d.L > 0 ? m->layers[0].g1 : m->gf, h, d.L > 0 ? g : nullptr, xf32, d.L > 0 ? nullptr : gf, sumsq,
            s->h_trace, s->pos, s->cap, (double)m->rope_theta, rope);
  VV_HIP(hipGetLastError());

  const bool kv32 = s->kv_dtype == VV_F32;
  const size_t layer_kv_bytes = (size_t)B * d.nkv * (size_t)s->cap * kHeadDim * (kv32 ? 4 : 2);
  // batch 1: the down projection and the next layer's q|k|v share one launch (the q|k|v
  // workgroups stream their weights while down finishes, then wait for its tagged output)
  const bool fuse_dq = layered_fuses_down_qkv(s);
  ChainParams cbase{};
  cbase.H = H; cbase.eps = m->eps; cbase.inv_h = inv_h;
  cbase.epoch = reinterpret_cast<const uint32_t*>(ws + lay.epoch);
  cbase.tag_mul = 4u * (uint32_t)(d.L + 1) + 1u; cbase.status = status;
  cbase.pos = s->pos; cbase.cap = s->cap;
  cbase.h = reinterpret_cast<uint64_t*>(ws + lay.th);
  for (int l = 0; l < d.L; ++l) {
    const vv_layer& y = m->layers[l];
    if (!fuse_dq || l == 0) {  // fused q|k|v projection, RMSNorm_1 folded in, bias added
      GemvParams p{};
      p.q = y.qkv_q; p.s = y.qkv_s; p.x = g; p.x_f32 = xf32;
      p.M = B; p.N = d.nqkv; p.K = H;
      p.ntiles = (int)cdiv(d.nqkv, kTileRows);
      p.epi = EPI_STORE; p.bias = y.qkv_bias; p.y = qkv; p.y_f16 = 0; p.ldy = d.nqkv;
      p.rs_parts = sumsq; p.rs_nparts = d.ntH; p.rs_inv_n = inv_h; p.eps = m->eps;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_qkv);
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
    // batches 1 and 2 with at most 64 splits (either cache precision: the split records are fp32
    // alike): the o projection's launch also merges the attention's split records (its leading
    // workgroups), so the merge needs no launch of its own
    AttnParams a{};
    a.B = B; a.nq = d.nq; a.nkv = d.nkv; a.cap = s->cap;
    attn_plan(a);
    const bool fuse_merge = B <= 2 && a.nsplit > 1 && a.nsplit <= 64;
    {  // attention with RoPE and KV append
      attn_set_workspace(a, ws + lay.ws_attn);
      a.skip_merge = fuse_merge;
      a.qkv = qkv; a.ldqkv = d.nqkv; a.pos = s->pos; a.rope_theta = m->rope_theta;
      a.kc = static_cast<char*>(s->k_cache) + (size_t)l * layer_kv_bytes;
      a.vc = static_cast<char*>(s->v_cache) + (size_t)l * layer_kv_bytes;
      a.kv_f32 = kv32;
      a.scale = 1.0f / sqrtf((float)kHeadDim);
      a.out = o; a.out_f16 = !xf32;
      VV_HIP(attn_launch_with_rope(a, rope, st, event_pair(s, op++)));
    }
    {  // o projection + residual; writes fp16(g2 * h) and sum(h^2) for the MLP
      GemvParams p{};
      p.q = y.o_q; p.s = y.o_s; p.x = o; p.x_f32 = xf32;
      p.M = B; p.N = H; p.K = d.nq * kHeadDim;
      p.ntiles = d.ntH;
      p.epi = EPI_RESID; p.h = h; p.gamma = y.g2; p.g_out = g; p.g_f32 = xf32; p.sumsq_out = sumsq;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_o);
      if (fuse_merge) {   // one wave per (row, query head, 64-dim half), whole rounds of 8 workgroups
        p.mrg_blocks = (int)(cdiv(cdiv(2 * d.nq * B, p.wpg), 8) * 8);
        p.mrg_part = a.part; p.mrg_pos = s->pos; p.mrg_nsplit = a.nsplit; p.mrg_split = a.split;
        p.mrg_cap = s->cap; p.mrg_nq = d.nq; p.mrg_nkv = d.nkv;
        p.xtag = reinterpret_cast<uint64_t*>(ws + lay.otag);
        p.epoch = reinterpret_cast<const uint32_t*>(ws + lay.epoch);
        p.tag_mul = (uint32_t)d.L + 1; p.tag_add = (uint32_t)l + 1;
      }
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
    {  // gate/up (32 gate + 32 up rows per tile) + SiLU(gate) * up, RMSNorm_2 folded in
      GemvParams p{};
      p.q = y.gu_q; p.s = y.gu_s; p.x = g; p.x_f32 = xf32;
      p.M = B; p.N = d.I; p.K = H;
      p.ntiles = 2 * d.ntI;
      p.epi = EPI_SILU; p.act = act; p.act_f32 = xf32;
      p.rs_parts = sumsq; p.rs_nparts = d.ntH; p.rs_inv_n = inv_h; p.eps = m->eps;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_gu);
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
    if (fuse_dq) {  // [down + residual | q|k|v of the next layer]
      const bool last = l == d.L - 1;
      ChainParams P = cbase;
      CSeg dn{};
      dn.kind = SEG_DOWN;
      dn.q = reinterpret_cast<const u32x4*>(y.down_q); dn.s = reinterpret_cast<const u32x4*>(y.down_s);
      dn.N = H; dn.K = d.I; dn.ntiles = d.ntH;
      dn.slots = reinterpret_cast<uint64_t*>(ws + lay.ws_down);
      dn.ss_n = d.ntH;
      chain_gemv_plan(dn);
      dn.xp = static_cast<const float*>(act); dn.hp = h;
      dn.xin = reinterpret_cast<const uint64_t*>(ws + lay.txd);   // unused (plain input), readable
      dn.out_add = 1u + 4u * (uint32_t)(l + 1);   // the chained tags: stage 0 (q|k|v input) of layer l + 1
      dn.gamma = last ? m->gf : m->layers[l + 1].g1;
      dn.trace = s->h_trace ? s->h_trace + (size_t)(l + 1) * H : nullptr;
      if (last) {
        dn.gf = gf; dn.sumsq = sumsq;
      } else {
        dn.xgout = reinterpret_cast<uint64_t*>(ws + lay.txq);
        dn.ssout = reinterpret_cast<uint64_t*>(ws + lay.tssq);
      }
      P.seg[0] = dn;
      P.nseg = 1;
      if (!last) {
        const vv_layer& yn = m->layers[l + 1];
        CSeg qs{};
        qs.kind = SEG_QKV;
        qs.q = reinterpret_cast<const u32x4*>(yn.qkv_q); qs.s = reinterpret_cast<const u32x4*>(yn.qkv_s);
        qs.N = d.nqkv; qs.K = H; qs.ntiles = (int)cdiv(d.nqkv, kTileRows);
        qs.slots = reinterpret_cast<uint64_t*>(ws + lay.ws_qkv);
        qs.ss_n = d.ntH;
        chain_gemv_plan(qs);
        qs.xin = dn.xgout; qs.xin_add = dn.out_add;
        qs.ssin = dn.ssout; qs.ss_add = dn.out_add;
        qs.has_bias = yn.qkv_bias != nullptr;
        qs.bias = yn.qkv_bias ? yn.qkv_bias : yn.g1;   // a readable stand-in when there is no bias
        qs.y = qkv;
        P.seg[P.nseg++] = qs;
      }
      VV_HIP(chain_launch(P, st, event_pair(s, op++)));
    } else {  // down projection + residual; feeds the next layer (or the lm_head)
      const bool last = l == d.L - 1;
      GemvParams p{};
      p.q = y.down_q; p.s = y.down_s; p.x = act; p.x_f32 = xf32;
      p.M = B; p.N = H; p.K = d.I;
      p.ntiles = d.ntH;
      p.epi = EPI_RESID; p.h = h;
      p.gamma = last ? m->gf : m->layers[l + 1].g1;
      p.g_out = last ? static_cast<void*>(gf) : g;    // the lm_head takes gamma_f * h in fp32
      p.g_f32 = last ? 1 : xf32;
      p.sumsq_out = sumsq;
      p.trace = s->h_trace ? s->h_trace + (size_t)(l + 1) * B * H : nullptr;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_down);
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
  }
  // final RMSNorm folded into the lm_head; greedy argmax; closed-loop feedback
  const int rc = enqueue_lm(m, s, gf, sumsq, ws + lay.ws_lm, status, reinterpret_cast<uint32_t*>(ws + lay.epoch), st,
                            event_pair(s, op++));
  if (rc) return rc;
  return enqueue_feedback(m, s, st);
}

}  // namespace
}  // namespace vv

struct vv_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

using namespace vv;

extern "C" {

size_t vv_decode_step_workspace(const vv_model* m, int batch, int cap) {
  if (!m || batch < 1 || cap < 1 || m->hidden < 64 || m->inter < 64 || m->n_kv < 1 || m->n_q < 1 ||
      m->n_q % m->n_kv)
    return 0;
  return step_bytes(m, batch, cap);
}

int vv_decode_status(const vv_model* m, const vv_state* s, int32_t* status, void* stream) {
  clear_error();
  VV_REQUIRE(m && s && status, VV_ERR_NULL, "vv_decode_status: NULL argument");
  VV_REQUIRE(s->workspace && s->batch >= 1 && s->cap >= 1, VV_ERR_RANGE, "vv_decode_status: bad state");
  const char* pws = static_cast<const char*>(s->workspace) + layout_of(dims_of(m, s->batch, s->cap)).status;
  hipStream_t st = as_stream(stream);
  VV_HIP(hipMemcpyAsync(status, pws, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  VV_HIP(hipStreamSynchronize(st));
  return VV_OK;
}

int vv_decode_path(const vv_model* m, const vv_state* s) {
  clear_error();
  const int rc = validate(m, s, "vv_decode_path");
  if (rc) return rc;
  return use_chain(m, s) ? VV_PATH_CHAINED : VV_PATH_LAYERED;
}

int vv_decode_step(const vv_model* m, const vv_state* s, void* stream) {
  clear_error();
  const int rc = validate(m, s, "vv_decode_step");
  if (rc) return rc;
  return enqueue_step(m, s, as_stream(stream));
}

int vv_decode_graph_create(const vv_model* m, const vv_state* s, void* stream, vv_graph** out) {
  clear_error();
  VV_REQUIRE(out != nullptr, VV_ERR_NULL, "vv_decode_graph_create: out is NULL");
  *out = nullptr;
  int rc = validate(m, s, "vv_decode_graph_create");
  if (rc) return rc;
  VV_REQUIRE(s->events == nullptr, VV_ERR_UNSUPPORTED, "vv_decode_graph_create: timing events are eager-only");
  (void)stream;
  hipStream_t cs;
  VV_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    hipStreamDestroy(cs);
    return hip_fail(e, "hipStreamBeginCapture");
  }
  rc = enqueue_step(m, s, cs);
  e = hipStreamEndCapture(cs, &graph);
  hipStreamDestroy(cs);
  if (rc) {
    if (graph) hipGraphDestroy(graph);
    return rc;
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(graph);
    return hip_fail(e, "hipGraphInstantiate");
  }
  vv_graph* gph = new (std::nothrow) vv_graph{graph, exec};
  if (!gph) {
    hipGraphExecDestroy(exec);
    hipGraphDestroy(graph);
    return fail(VV_ERR_RANGE, "vv_decode_graph_create: out of host memory");
  }
  *out = gph;
  return VV_OK;
}

int vv_decode_graph_launch(vv_graph* gph, void* stream) {
  clear_error();
  VV_REQUIRE(gph != nullptr, VV_ERR_NULL, "vv_decode_graph_launch: graph is NULL");
  VV_HIP(hipGraphLaunch(gph->exec, as_stream(stream)));
  return VV_OK;
}

int vv_decode_graph_destroy(vv_graph* gph) {
  clear_error();
  if (!gph) return VV_OK;
  hipGraphExecDestroy(gph->exec);
  hipGraphDestroy(gph->graph);
  delete gph;
  return VV_OK;
}

}  // extern "C"
