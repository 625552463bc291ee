// Decode-step launcher and its hipGraph wrapper.
//
// Two implementations of the same step share the entry points: the persistent kernel of
// mega.hip (one launch for all layers, then the lm_head; batch 1) and the layered
// path below (one launch per stage; any batch up to 16).  vv_state.path picks one.
//
// decoder_step contract ("vibevoice-asr-bitnet-onnx" page, graph contracts):
//   input_embeds [B,H], position_ids [B], past K/V -> logits [B,V], present K/V (one more slot)
// on the Qwen2 layer of the 1.5B STATUS page (Architecture): pre-RMSNorm, q/k/v bias, GQA,
// SiLU-gated MLP, residual adds.  One step is 1 + 5 L + 1 kernels:
//   prep (embeddings -> residual stream, RoPE table)
//   per layer: QKV GEMV (RMSNorm folded in) | attention (+RoPE, KV append) and its split merge
//              (a kernel of its own, or at batch 1 over fp16 caches the leading workgroups of the
//              o GEMV's launch) | o GEMV + residual | gate/up GEMV + SiLU*up | down GEMV + residual
//   lm_head + argmax (final RMSNorm folded in).
// RMSNorm is folded into the GEMVs: the producer of h writes fp16(gamma * h) and per-tile sums of
// h^2; the consumer scales its row sums by rstd = 1/sqrt(mean(h^2) + eps).  Positions are read
// from device memory, so one captured graph serves every step.
#include <new>
#include <vector>

#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kHeadDim = 128;

// h = fp32(input_embeds); g = fp16(gamma * h) (or gf = gamma * h in fp32 when there are no
// layers); per-tile sum of h^2; optional trace; RoPE (cos, sin) of pos[b] for the 64 pairs; the
// step counter advances.
__global__ __launch_bounds__(64) void k_step_prep(const uint16_t* __restrict__ emb, int H, int ntiles,
                                                  const uint16_t* __restrict__ gamma, float* __restrict__ h,
                                                  uint16_t* __restrict__ g, float* __restrict__ gf,
                                                  float* __restrict__ sumsq, float* __restrict__ trace,
                                                  const int32_t* __restrict__ pos, int cap, double theta,
                                                  float* __restrict__ rope, uint32_t* __restrict__ epoch) {
  const int t = blockIdx.x % ntiles, b = blockIdx.x / ntiles;
  if (blockIdx.x == 0 && threadIdx.x == 0) epoch[0] += 1;   // a new step: fresh tags for this step's words
  const int lane = threadIdx.x;
  const int n = t * 64 + lane;
  const size_t i = (size_t)b * H + n;
  const float hv = h2f(emb[i]);
  h[i] = hv;
  if (trace) trace[i] = hv;
  const float gv = h2f(gamma[n]) * hv;
  if (g) g[i] = f2h(gv);
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
  size_t h, g, gf, qkv, o, act, sumsq, rope, ws_qkv, ws_o, ws_gu, ws_down, ws_attn, ws_lm, otag, epoch, total;
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
  l.h = take((size_t)d.B * d.H * 4);
  l.g = take((size_t)d.B * d.H * 2);
  l.gf = take((size_t)d.B * d.H * 4);
  l.qkv = take((size_t)d.B * d.nqkv * 4);
  l.o = take((size_t)d.B * d.nq * kHeadDim * 2);
  l.act = take((size_t)d.B * d.I * 2);
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
  l.otag = take((size_t)d.nq * kHeadDim * sizeof(uint64_t));   // fused merge -> o projection (batch 1)
  l.epoch = take(sizeof(uint32_t));                              // step counter (tags of otag)
  l.total = off;
  return l;
}

// bytes of the layered path's region; the persistent region follows it
size_t layered_bytes(const vv_model* m, int B, int cap) { return align_up(layout_of(dims_of(m, B, cap)).total, 256); }

size_t step_bytes(const vv_model* m, int B, int cap) {
  return layered_bytes(m, B, cap) + persistent_workspace_bytes(m, B, cap);
}

// AUTO takes the layered path: on MI355X it is the faster of the two at present (the persistent
// kernel's per-item hand-offs cost more than the launches they save); see the path notes in vv.h
bool use_persistent(const vv_model* m, const vv_state* s) {
  (void)m;
  return s->path == VV_PATH_PERSISTENT;
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
  VV_REQUIRE(s->path == VV_PATH_AUTO || s->path == VV_PATH_LAYERED || s->path == VV_PATH_PERSISTENT, VV_ERR_RANGE,
             "%s: unknown path %d", fn, s->path);
  VV_REQUIRE(s->path != VV_PATH_PERSISTENT || persistent_supported(m, s->batch), VV_ERR_UNSUPPORTED,
             "%s: the persistent path needs n_layers >= 1, batch 1, hidden <= 4096", fn);
  VV_REQUIRE(s->n_stop >= 0 && s->n_stop <= 4, VV_ERR_RANGE, "%s: n_stop %d not in 0..4", fn, s->n_stop);
  VV_REQUIRE(s->kv_dtype == 0 || s->kv_dtype == VV_F16 || s->kv_dtype == VV_F32, VV_ERR_DTYPE,
             "%s: kv_dtype %d is not VV_F16 or VV_F32", fn, s->kv_dtype);
  VV_REQUIRE(s->kv_dtype != VV_F32 || !use_persistent(m, s), VV_ERR_UNSUPPORTED,
             "%s: fp32 KV caches need the layered path", fn);
  VV_REQUIRE(!s->feedback_table || (reinterpret_cast<uintptr_t>(s->feedback_table) & 15) == 0, VV_ERR_RANGE,
             "%s: feedback_table must be 16-byte aligned", fn);
  const size_t need = step_bytes(m, s->batch, s->cap);
  VV_REQUIRE(s->workspace && s->workspace_bytes >= need, VV_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn,
             need);
  VV_REQUIRE((reinterpret_cast<uintptr_t>(s->workspace) & 255) == 0, VV_ERR_RANGE,
             "%s: workspace must be 256-byte aligned", fn);
  const int nev = use_persistent(m, s) ? 2 * 2 : 2 * (5 * m->n_layers + 2);
  VV_REQUIRE(!s->events || s->n_events >= nev, VV_ERR_RANGE, "%s: events needs at least %d entries", fn, nev);
  return VV_OK;
}

int enqueue_lm(const vv_model* m, const vv_state* s, const float* gf32, const float* sumsq, char* ws_lm,
               int32_t* status, hipStream_t st, KEv ev) {
  LmParams p{};
  p.status = status;
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

int enqueue_persistent(const vv_model* m, const vv_state* s, hipStream_t st) {
  char* ws = static_cast<char*>(s->workspace);
  char* pws = ws + layered_bytes(m, s->batch, s->cap);
  const Layout lay = layout_of(dims_of(m, s->batch, s->cap));
  int rc = persistent_enqueue(m, s, pws, st, event_pair(s, 0));
  if (rc) return rc;
  const float* gf32;
  const float* sumsq;
  persistent_lm_inputs(m, s, pws, &gf32, &sumsq);
  rc = enqueue_lm(m, s, gf32, sumsq, ws + lay.ws_lm, reinterpret_cast<int32_t*>(pws), st, event_pair(s, 1));
  if (rc) return rc;
  return enqueue_feedback(m, s, st);
}

int enqueue_step(const vv_model* m, const vv_state* s, hipStream_t st) {
  if (use_persistent(m, s)) return enqueue_persistent(m, s, st);
  const Dims d = dims_of(m, s->batch, s->cap);
  const Layout lay = layout_of(d);
  char* ws = static_cast<char*>(s->workspace);
  float* h = reinterpret_cast<float*>(ws + lay.h);
  uint16_t* g = reinterpret_cast<uint16_t*>(ws + lay.g);
  float* gf = reinterpret_cast<float*>(ws + lay.gf);
  float* qkv = reinterpret_cast<float*>(ws + lay.qkv);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + lay.o);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + lay.act);
  float* sumsq = reinterpret_cast<float*>(ws + lay.sumsq);
  float* rope = reinterpret_cast<float*>(ws + lay.rope);
  const int B = d.B, H = d.H;
  const float inv_h = 1.0f / (float)H;
  // the step's sticky status word (first word of the persistent region): a GEMV hand-off wait
  // that gives up sets it
  int32_t* status = reinterpret_cast<int32_t*>(ws + layered_bytes(m, B, s->cap));
  int op = 0;   // timing event pair of the next operation
  VV_LAUNCH(k_step_prep, dim3(B * d.ntH), dim3(64), st, event_pair(s, op++), s->input_embeds, H, d.ntH,
            d.L > 0 ? m->layers[0].g1 : m->gf, h, d.L > 0 ? g : nullptr, d.L > 0 ? nullptr : gf, sumsq,
            s->h_trace, s->pos, s->cap, (double)m->rope_theta, rope,
            reinterpret_cast<uint32_t*>(ws + lay.epoch));
  VV_HIP(hipGetLastError());

  const bool kv32 = s->kv_dtype == VV_F32;
  const size_t layer_kv_bytes = (size_t)B * d.nkv * (size_t)s->cap * kHeadDim * (kv32 ? 4 : 2);
  for (int l = 0; l < d.L; ++l) {
    const vv_layer& y = m->layers[l];
    {  // fused q|k|v projection, RMSNorm_1 folded in, bias added
      GemvParams p{};
      p.q = y.qkv_q; p.s = y.qkv_s; p.x = g;
      p.M = B; p.N = d.nqkv; p.K = H;
      p.ntiles = (int)cdiv(d.nqkv, kTileRows);
      p.epi = EPI_STORE; p.bias = y.qkv_bias; p.y = qkv; p.y_f16 = 0; p.ldy = d.nqkv;
      p.rs_parts = sumsq; p.rs_nparts = d.ntH; p.rs_inv_n = inv_h; p.eps = m->eps;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_qkv);
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
    // batch 1 over fp16 caches with at most 64 splits: the o projection's launch also merges the
    // attention's split records (its leading workgroups), so the merge needs no launch of its own
    AttnParams a{};
    a.B = B; a.nq = d.nq; a.nkv = d.nkv; a.cap = s->cap;
    attn_plan(a);
    const bool fuse_merge = B == 1 && !kv32 && a.nsplit > 1 && a.nsplit <= 64;
    {  // attention with RoPE and KV append
      attn_set_workspace(a, ws + lay.ws_attn);
      a.skip_merge = fuse_merge;
      a.qkv = qkv; a.ldqkv = d.nqkv; a.pos = s->pos; a.rope_theta = m->rope_theta;
      a.kc = static_cast<char*>(s->k_cache) + (size_t)l * layer_kv_bytes;
      a.vc = static_cast<char*>(s->v_cache) + (size_t)l * layer_kv_bytes;
      a.kv_f32 = kv32;
      a.scale = 1.0f / sqrtf((float)kHeadDim);
      a.out = o; a.out_f16 = 1;
      VV_HIP(attn_launch_with_rope(a, rope, st, event_pair(s, op++)));
    }
    {  // o projection + residual; writes fp16(g2 * h) and sum(h^2) for the MLP
      GemvParams p{};
      p.q = y.o_q; p.s = y.o_s; p.x = o;
      p.M = B; p.N = H; p.K = d.nq * kHeadDim;
      p.ntiles = d.ntH;
      p.epi = EPI_RESID; p.h = h; p.gamma = y.g2; p.g_out = g; p.sumsq_out = sumsq;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_o);
      if (fuse_merge) {   // one wave per (query head, 64-dim half), whole rounds of 8 workgroups
        p.mrg_blocks = (int)(cdiv(cdiv(2 * d.nq, p.wpg), 8) * 8);
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
      p.q = y.gu_q; p.s = y.gu_s; p.x = g;
      p.M = B; p.N = d.I; p.K = H;
      p.ntiles = 2 * d.ntI;
      p.epi = EPI_SILU; p.act = act;
      p.rs_parts = sumsq; p.rs_nparts = d.ntH; p.rs_inv_n = inv_h; p.eps = m->eps;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_gu);
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
    {  // down projection + residual; feeds the next layer (or the lm_head)
      const bool last = l == d.L - 1;
      GemvParams p{};
      p.q = y.down_q; p.s = y.down_s; p.x = act;
      p.M = B; p.N = H; p.K = d.I;
      p.ntiles = d.ntH;
      p.epi = EPI_RESID; p.h = h;
      p.gamma = last ? m->gf : m->layers[l + 1].g1;
      p.g_out = last ? nullptr : g;
      p.gf_out = last ? gf : nullptr;
      p.sumsq_out = sumsq;
      p.trace = s->h_trace ? s->h_trace + (size_t)(l + 1) * B * H : nullptr;
      gemv_plan(p);
      p.status = status;
      gemv_set_workspace(p, ws + lay.ws_down);
      VV_HIP(gemv_launch(p, st, event_pair(s, op++)));
    }
  }
  // final RMSNorm folded into the lm_head; greedy argmax; closed-loop feedback
  const int rc = enqueue_lm(m, s, gf, sumsq, ws + lay.ws_lm, status, st, event_pair(s, op++));
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
  const char* pws = static_cast<const char*>(s->workspace) + layered_bytes(m, s->batch, s->cap);
  hipStream_t st = as_stream(stream);
  VV_HIP(hipMemcpyAsync(status, pws, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  VV_HIP(hipStreamSynchronize(st));
  return VV_OK;
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
  // size the persistent grid before capturing (the occupancy query is not a stream operation)
  if (use_persistent(m, s)) VV_REQUIRE(persistent_grid() > 0, VV_ERR_HIP, "vv_decode_graph_create: no resident grid");
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
