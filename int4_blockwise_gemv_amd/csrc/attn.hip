// Split-KV grouped-query decode attention over an fp16 KV cache.
//
// GroupQueryAttention decode over a cache that stays in HBM (GPU-resident KV:
// "VibeVoice-ASR — ONNX export for Vernacula", Highlights), with fp32 scores, softmax and
// accumulation (the same page reports fp32 attention as the accuracy fix over bf16).
//
// Work unit: (sequence b, KV head, split of 64/128/256 positions).  A workgroup of 8 waves issues
// every K and V row load of its split up front (16 lanes x 16 B per row, 4 rows = 1 KiB per wave
// load) and serves all g = nq/nkv query heads of the group with them.  It writes
// (max, sum, unnormalised output) per head; a second small kernel, one workgroup per query
// head, merges the splits (online-softmax rescaling, fixed order).  The kernel boundary is the
// hand-off, so no workgroup waits on another.
//
// Decode-step flavour: q/k/v come from the fused projection output; the workgroup rotates q
// (and, for the split that holds the new position, k) with RoPE, writes fp16 k and v into the
// cache slot of the new position and attends over pos+1 positions.
#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kD = 128;           // head_dim
constexpr int kMaxG = 8;          // query heads per KV head
constexpr int kPS = 132;          // partial record: m, l, pad, pad, o[128]
constexpr int kWaves = 8;         // 512 threads per workgroup
constexpr int kThreads = kWaves * 64;

__device__ void write_out(const AttnParams& p, int b, int kvh, int g, const float (*O)[kD], const float* L, int tid) {
  for (int i = tid; i < g * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    const float o = O[hh][d] / L[hh];
    const size_t oi = ((size_t)b * p.nq + (size_t)kvh * g + hh) * kD + d;
    if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(o);
    else reinterpret_cast<float*>(p.out)[oi] = o;
  }
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

// NP passes of 4 positions per wave: split = 8 waves * 4 * NP positions
template <int NP>
__global__ __launch_bounds__(kThreads) void k_attn(AttnParams p, const float* __restrict__ rope_cs) {
  constexpr int S = kWaves * 4 * NP;
  __shared__ float qs[kMaxG][kD];
  __shared__ float sc[kMaxG][S];
  __shared__ float red[kWaves][kMaxG][kD];
  __shared__ uint16_t knew[kD], vnew[kD];
  __shared__ float mh[kMaxG], lh[kMaxG];

  const int g = p.nq / p.nkv;
  const int wg = blockIdx.x;
  const int sidx = wg % p.nsplit;
  const int bh = wg / p.nsplit;            // b * nkv + kvh
  const int b = bh / p.nkv, kvh = bh % p.nkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool step = p.qkv != nullptr;

  // ---- every global load of the workgroup is issued before any result is used ----------------
  // (K/V rows of the whole split do not depend on the sequence length: rows past it are read
  // from inside the cache and masked out below; the new position's stale row is replaced)
  const int s0 = sidx * S;
  const size_t kvbase = ((size_t)b * p.nkv + kvh) * (size_t)p.cap * kD;
  const uint16_t* Kc = p.kc + kvbase;
  const uint16_t* Vc = p.vc + kvbase;
  const int sl = lane & 15;            // dims 8*sl .. 8*sl+7
  const int pg = lane >> 4;            // position within a pass
  const int jw = w * 4 * NP;           // first local position of this wave
  u32x4 kr[NP], vr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pos = s0 + jw + 4 * i + pg;
    kr[i] = u32x4{0, 0, 0, 0};
    vr[i] = u32x4{0, 0, 0, 0};
    if (pos < p.cap) {
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kc + (size_t)pos * kD + 8 * sl));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vc + (size_t)pos * kD + 8 * sl));
    }
  }
  const int pos_raw = step ? p.pos[b] : p.lens[b];
  // q pair (j, j+64) of head hh = tid/64 (step: raw projection output + RoPE coefficients)
  const int qh_ = tid >> 6, qj = tid & 63;
  float q1 = 0.f, q2 = 0.f, rc = 1.f, rsn = 0.f, k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
  float qsa[2] = {0.f, 0.f};           // stand-alone flavour: two q values per thread
  if (step) {
    const float* row = p.qkv + (size_t)b * p.ldqkv;
    if (qh_ < g) {
      const float* qh = row + (size_t)(kvh * g + qh_) * kD;
      q1 = qh[qj];
      q2 = qh[qj + 64];
    }
    if (p.rope_theta > 0.f) {
      const float* cs = rope_cs + ((size_t)b * 64 + qj) * 2;
      rc = cs[0];
      rsn = cs[1];
    }
    if (tid < 64) {
      const float* kh = row + (size_t)p.nq * kD + (size_t)kvh * kD;
      const float* vh = row + (size_t)(p.nq + p.nkv) * kD + (size_t)kvh * kD;
      k1 = kh[qj]; k2 = kh[qj + 64]; v1 = vh[qj]; v2 = vh[qj + 64];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * kThreads;
      if (i < g * kD) {
        const size_t qi = ((size_t)b * p.nq + (size_t)kvh * g + i / kD) * kD + i % kD;
        qsa[u] = p.q_f16 ? h2f(reinterpret_cast<const uint16_t*>(p.q)[qi]) : reinterpret_cast<const float*>(p.q)[qi];
      }
    }
  }

  int len, P = -1;
  if (step) {
    P = pos_raw < 0 ? 0 : (pos_raw >= p.cap ? p.cap - 1 : pos_raw);
    len = P + 1;
  } else {
    len = pos_raw < 1 ? 1 : (pos_raw > p.cap ? p.cap : pos_raw);
  }
  const int npos = max(0, min(s0 + S, len) - s0);
  const bool has_new = P >= s0 && P < s0 + npos;

  // ---- q (and the new k, v) into LDS -----------------------------------------------------------
  if (step) {
    if (qh_ < g) {
      qs[qh_][qj] = q1 * rc - q2 * rsn;
      qs[qh_][qj + 64] = q2 * rc + q1 * rsn;
    }
    if (has_new && tid < 64) {
      const uint16_t a = f2h(k1 * rc - k2 * rsn), bb = f2h(k2 * rc + k1 * rsn), c1 = f2h(v1), c2 = f2h(v2);
      knew[qj] = a; knew[qj + 64] = bb; vnew[qj] = c1; vnew[qj + 64] = c2;
      uint16_t* kd = p.kc + kvbase + (size_t)P * kD;
      uint16_t* vd = p.vc + kvbase + (size_t)P * kD;
      kd[qj] = a; kd[qj + 64] = bb; vd[qj] = c1; vd[qj + 64] = c2;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * kThreads;
      if (i < g * kD) qs[i / kD][i % kD] = qsa[u];
    }
  }
  __syncthreads();
  if (has_new) {  // the new position reads the rows just written to LDS
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (s0 + jw + 4 * i + pg == P) {
        kr[i] = *reinterpret_cast<const u32x4*>(&knew[8 * sl]);
        vr[i] = *reinterpret_cast<const u32x4*>(&vnew[8 * sl]);
      }
  }

  // ---- scores (16 lanes per position, reduced across the 16) ----------------------------------
  float qr[kMaxG][8];
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[hh][i] = hh < g ? qs[hh][8 * sl + i] : 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = jw + 4 * i + pg;
    float kf[8];
    h8_to_f32(kr[i], kf);
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      if (hh < g) {
        float a = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) a = fmaf(qr[hh][t], kf[t], a);
        a = row16_sum(a);
        if (sl == 0) sc[hh][j] = j < npos ? a * p.scale : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- split-local softmax statistics ---------------------------------------------------------
  for (int hh = w; hh < g; hh += kWaves) {
    float m = -INFINITY;
    for (int j = lane; j < S; j += 64) m = fmaxf(m, sc[hh][j]);
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j < S; j += 64) {
      const float e = (m == -INFINITY) ? 0.f : expf(sc[hh][j] - m);
      sc[hh][j] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { mh[hh] = m; lh[hh] = l; }
  }
  __syncthreads();

  // ---- weighted sum of V ------------------------------------------------------------------------
  float acc[kMaxG][8];
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[hh][t] = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = jw + 4 * i + pg;
    float vf[8];
    h8_to_f32(vr[i], vf);
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      if (hh < g) {
        const float pj = sc[hh][j];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[hh][t] = fmaf(pj, vf[t], acc[hh][t]);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh) {
    if (hh < g) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float a = rows_lanewise_sum(acc[hh][t]);
        if (pg == 0) red[w][hh][8 * sl + t] = a;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < g * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    float o = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) o += red[v][hh][d];
    red[0][hh][d] = o;
  }
  __syncthreads();

  // ---- finish: one split writes the output; otherwise its record goes to the merge kernel -----
  if (p.nsplit == 1) {
    write_out(p, b, kvh, g, red[0], lh, tid);
    return;
  }
  float* rec = p.part + ((size_t)bh * p.nsplit + sidx) * kMaxG * kPS;
  for (int i = tid; i < g * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    rec[(size_t)hh * kPS + 4 + d] = red[0][hh][d];
  }
  if (tid < g) {
    rec[(size_t)tid * kPS + 0] = mh[tid];
    rec[(size_t)tid * kPS + 1] = lh[tid];
  }
}

// One workgroup per (sequence, query head), one thread per output dimension: combines the split
// records with the online-softmax rescaling M = max m_s, L = sum e^(m_s-M) l_s,
// o = sum e^(m_s-M) o_s / L, splits in a fixed order.  All loads are issued before any use.
__global__ __launch_bounds__(kD) void k_attn_merge(AttnParams p) {
  constexpr int kChunk = 32;           // splits whose outputs one thread holds at a time
  __shared__ float ms_[512], ls_[512], wsc[512];
  __shared__ float Ms, Ls;
  const int g = p.nq / p.nkv;
  const int bq = blockIdx.x;                 // b * nq + head
  const int b = bq / p.nq, h = bq % p.nq;
  const int kvh = h / g, hh = h % g;
  const int bh = b * p.nkv + kvh;
  const int d = threadIdx.x;
  const float* rec0 = p.part + ((size_t)bh * p.nsplit * kMaxG + hh) * kPS;
  const size_t stride = (size_t)kMaxG * kPS;
  const int n = p.nsplit;
  // issue the (m, l) loads and the first chunk of outputs together
  for (int s = d; s < n; s += kD) {
    ms_[s] = rec0[s * stride];
    ls_[s] = rec0[s * stride + 1];
  }
  float v[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u) v[u] = u < n ? rec0[u * stride + 4 + d] : 0.f;
  __syncthreads();
  if (d < 64) {
    float M = -INFINITY;
    for (int s = d; s < n; s += 64) M = fmaxf(M, ms_[s]);
    M = wave_max(M);
    float L = 0.f;
    for (int s = d; s < n; s += 64) {
      const float e = ms_[s] == -INFINITY ? 0.f : expf(ms_[s] - M);
      wsc[s] = e;
      L = fmaf(e, ls_[s], L);
    }
    L = wave_sum(L);
    if (d == 0) { Ms = M; Ls = L; }
  }
  __syncthreads();
  float O = 0.f;
#pragma unroll
  for (int u = 0; u < kChunk; ++u)
    if (u < n) O = fmaf(wsc[u], v[u], O);
  for (int s0 = kChunk; s0 < n; s0 += kChunk) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) v[u] = s0 + u < n ? rec0[(s0 + u) * stride + 4 + d] : 0.f;
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (s0 + u < n) O = fmaf(wsc[s0 + u], v[u], O);
  }
  const float o = O / Ls;
  const size_t oi = ((size_t)b * p.nq + h) * kD + d;
  if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(o);
  else reinterpret_cast<float*>(p.out)[oi] = o;
}

int pow2ceil(int64_t v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

}  // namespace

// Split size 64/128/256 positions: aims at ~192 workgroups, at most 512 splits per sequence
// (the merge kernel keeps one weight per split in LDS).
void attn_plan(AttnParams& p) {
  const int64_t work = (int64_t)p.B * p.nkv * p.cap;
  int S = pow2ceil(cdiv(work, 192));
  S = S < 64 ? 64 : (S > 256 ? 256 : S);
  p.split = S;
  p.nsplit = (int)cdiv(p.cap, S);
}

size_t attn_workspace_bytes(int B, int nq, int nkv, int nsplit) {
  (void)nq;
  return align_up((size_t)B * nkv * nsplit * kMaxG * kPS * sizeof(float), 256);
}

void attn_set_workspace(AttnParams& p, void* ws) {
  p.part = reinterpret_cast<float*>(ws);
  p.part2 = nullptr;
  p.cnt = nullptr;
}

hipError_t attn_launch_with_rope(const AttnParams& p, const float* rope_cs, hipStream_t st) {
  const int grid = p.B * p.nkv * p.nsplit;
  switch (p.split) {
    case 64: hipLaunchKernelGGL(k_attn<2>, dim3(grid), dim3(kThreads), 0, st, p, rope_cs); break;
    case 128: hipLaunchKernelGGL(k_attn<4>, dim3(grid), dim3(kThreads), 0, st, p, rope_cs); break;
    default: hipLaunchKernelGGL(k_attn<8>, dim3(grid), dim3(kThreads), 0, st, p, rope_cs); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(p.B * p.nq), dim3(kD), 0, st, p);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnParams& p, hipStream_t st) { return attn_launch_with_rope(p, nullptr, st); }

}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_gqa_decode_workspace(int B, int nq, int nkv, int cap) {
  if (B < 1 || nq < 1 || nkv < 1 || cap < 1) return 0;
  AttnParams p{};
  p.B = B; p.nq = nq; p.nkv = nkv; p.cap = cap;
  attn_plan(p);
  return attn_workspace_bytes(B, nq, nkv, p.nsplit);
}

int vv_gqa_decode(const void* q, int q_dtype, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* lens,
                  int B, int nq, int nkv, int cap, int head_dim, float softmax_scale, void* out, int out_dtype,
                  void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  VV_REQUIRE(q && k_cache && v_cache && lens && out, VV_ERR_NULL, "vv_gqa_decode: NULL pointer");
  VV_REQUIRE(head_dim == kD, VV_ERR_SHAPE, "vv_gqa_decode: head_dim %d != 128", head_dim);
  VV_REQUIRE(B >= 1 && nq >= 1 && nkv >= 1 && cap >= 1, VV_ERR_RANGE, "vv_gqa_decode: B/nq/nkv/cap must be >= 1");
  VV_REQUIRE(nq % nkv == 0 && nq / nkv <= kMaxG, VV_ERR_SHAPE,
             "vv_gqa_decode: nq %% nkv must be 0 and nq/nkv <= %d", kMaxG);
  VV_REQUIRE(q_dtype == VV_F16 || q_dtype == VV_F32, VV_ERR_DTYPE, "vv_gqa_decode: unknown q dtype");
  VV_REQUIRE(out_dtype == VV_F16 || out_dtype == VV_F32, VV_ERR_DTYPE, "vv_gqa_decode: unknown out dtype");
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15) == 0,
             VV_ERR_RANGE, "vv_gqa_decode: caches must be 16-byte aligned");
  VV_REQUIRE(cap <= 256 * 512, VV_ERR_RANGE, "vv_gqa_decode: cap %d > 131072 positions", cap);
  const size_t need = vv_gqa_decode_workspace(B, nq, nkv, cap);
  VV_REQUIRE(ws && ws_bytes >= need, VV_ERR_WORKSPACE, "vv_gqa_decode: workspace needs %zu bytes", need);
  AttnParams p{};
  p.B = B; p.nq = nq; p.nkv = nkv; p.cap = cap;
  attn_plan(p);
  attn_set_workspace(p, ws);
  p.q = q; p.q_f16 = q_dtype == VV_F16; p.lens = lens;
  p.kc = const_cast<uint16_t*>(k_cache); p.vc = const_cast<uint16_t*>(v_cache);
  p.scale = softmax_scale;
  p.out = out; p.out_f16 = out_dtype == VV_F16;
  VV_HIP(attn_launch(p, as_stream(stream)));
  return VV_OK;
}

}  // extern "C"
