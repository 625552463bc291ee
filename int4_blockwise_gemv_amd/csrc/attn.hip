// Split-KV grouped-query decode attention over an fp16 KV cache.
//
// GroupQueryAttention decode over a cache that stays in HBM (GPU-resident KV:
// "VibeVoice-ASR — ONNX export for Vernacula", Highlights), with fp32 scores, softmax and
// accumulation (the same page reports fp32 attention as the accuracy fix over bf16).
//
// Work unit: (sequence b, KV head, split of 64/128/256 positions).  A workgroup of 8 waves issues
// every K and V row load of its split up front (16 lanes x 16 B per row, 4 rows = 1 KiB per wave
// load) and serves all g = nq/nkv query heads of the group with them.  It publishes
// (max, sum, unnormalised output) per head; the last of each group of 8 splits to finish merges
// that group (online-softmax rescaling, fixed order) and the last group merger merges the group
// results, so no single workgroup reads more than 64 records.
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
constexpr int kGroup = 8;         // splits merged per first-level merge
constexpr int kMaxMerge = 64;     // partials one merge reads (kGroup, or the number of groups)

struct MergeLds {
  float m[kMaxMerge][kMaxG];
  float w[kMaxMerge][kMaxG];      // e^(m_s - M), 0 for empty partials
  float M[kMaxG], L[kMaxG];
  float O[kMaxG][kD];
};

// Merges n partial records (m, l, o) per head into (M, L, O = sum e^(m_s-M) o_s) in LDS.
__device__ void merge_parts(const float* parts, int n, int g, MergeLds& ml, int tid) {
  for (int i = tid; i < n * g; i += kThreads) {
    const int s = i / g, hh = i % g;
    ml.m[s][hh] = collect_f32(parts + ((size_t)s * kMaxG + hh) * kPS);
  }
  __syncthreads();
  if (tid < g) {
    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, ml.m[s][tid]);
    ml.M[tid] = M;
  }
  __syncthreads();
  for (int i = tid; i < n * g; i += kThreads) {
    const int s = i / g, hh = i % g;
    const float ms = ml.m[s][hh];
    ml.w[s][hh] = (ms == -INFINITY) ? 0.f : expf(ms - ml.M[hh]);
  }
  __syncthreads();
  if (tid < g) {
    float L = 0.f;
    for (int s = 0; s < n; ++s)
      if (ml.w[s][tid] != 0.f) L = fmaf(ml.w[s][tid], collect_f32(parts + ((size_t)s * kMaxG + tid) * kPS + 1), L);
    ml.L[tid] = L;
  }
  for (int i = tid; i < g * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    float O = 0.f;
    int s = 0;
    for (; s + 8 <= n; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = collect_f32(parts + ((size_t)(s + u) * kMaxG + hh) * kPS + 4 + d);
#pragma unroll
      for (int u = 0; u < 8; ++u) O = fmaf(ml.w[s + u][hh], v[u], O);
    }
    for (; s < n; ++s) O = fmaf(ml.w[s][hh], collect_f32(parts + ((size_t)s * kMaxG + hh) * kPS + 4 + d), O);
    ml.O[hh][d] = O;
  }
  __syncthreads();
}

__device__ void publish_record(float* rec, int g, const float* M, const float* L, const float (*O)[kD], int tid) {
  for (int i = tid; i < g * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    publish_f32(rec + (size_t)hh * kPS + 4 + d, O[hh][d]);
  }
  if (tid < g) {
    publish_f32(rec + (size_t)tid * kPS + 0, M[tid]);
    publish_f32(rec + (size_t)tid * kPS + 1, L[tid]);
  }
  wait_published();
}

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
  __shared__ MergeLds ml;
  __shared__ unsigned s_flag;

  const int g = p.nq / p.nkv;
  const int wg = blockIdx.x;
  const int sidx = wg % p.nsplit;
  const int bh = wg / p.nsplit;            // b * nkv + kvh
  const int b = bh / p.nkv, kvh = bh % p.nkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool step = p.qkv != nullptr;

  int len, P = -1;
  if (step) {
    P = p.pos[b];
    P = P < 0 ? 0 : (P >= p.cap ? p.cap - 1 : P);
    len = P + 1;
  } else {
    len = p.lens[b];
    len = len < 1 ? 1 : (len > p.cap ? p.cap : len);
  }
  const int s0 = sidx * S;
  const int npos = max(0, min(s0 + S, len) - s0);
  const size_t kvbase = ((size_t)b * p.nkv + kvh) * (size_t)p.cap * kD;
  const uint16_t* Kc = p.kc + kvbase;
  const uint16_t* Vc = p.vc + kvbase;

  // ---- issue every K and V row load of this wave first ----------------------------------------
  const int sl = lane & 15;            // dims 8*sl .. 8*sl+7
  const int pg = lane >> 4;            // position within a pass
  const int jw = w * 4 * NP;           // first local position of this wave
  u32x4 kr[NP], vr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = jw + 4 * i + pg;
    const int pos = s0 + j;
    kr[i] = u32x4{0, 0, 0, 0};
    vr[i] = u32x4{0, 0, 0, 0};
    if (j < npos && pos != P) {
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kc + (size_t)pos * kD + 8 * sl));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vc + (size_t)pos * kD + 8 * sl));
    }
  }

  // ---- q (and the new k, v) into LDS ---------------------------------------------------------
  if (step) {
    const float* row = p.qkv + (size_t)b * p.ldqkv;
    const float* cs = rope_cs + (size_t)b * 64 * 2;
    const bool rope = p.rope_theta > 0.f;
    for (int i = tid; i < g * 64; i += kThreads) {
      const int hh = i / 64, j = i % 64;
      const float* qh = row + (size_t)(kvh * g + hh) * kD;
      const float x1 = qh[j], x2 = qh[j + 64];
      if (rope) {
        const float c = cs[2 * j], s = cs[2 * j + 1];
        qs[hh][j] = x1 * c - x2 * s;
        qs[hh][j + 64] = x2 * c + x1 * s;
      } else {
        qs[hh][j] = x1;
        qs[hh][j + 64] = x2;
      }
    }
    if (P >= s0 && P < s0 + npos && tid < 64) {
      const float* kh = row + (size_t)p.nq * kD + (size_t)kvh * kD;
      const float* vh = row + (size_t)(p.nq + p.nkv) * kD + (size_t)kvh * kD;
      const int j = tid;
      float k1 = kh[j], k2 = kh[j + 64];
      if (rope) {
        const float c = cs[2 * j], s = cs[2 * j + 1];
        const float r1 = k1 * c - k2 * s, r2 = k2 * c + k1 * s;
        k1 = r1;
        k2 = r2;
      }
      const uint16_t a = f2h(k1), bb = f2h(k2), c1 = f2h(vh[j]), c2 = f2h(vh[j + 64]);
      knew[j] = a; knew[j + 64] = bb; vnew[j] = c1; vnew[j + 64] = c2;
      uint16_t* kd = p.kc + kvbase + (size_t)P * kD;
      uint16_t* vd = p.vc + kvbase + (size_t)P * kD;
      kd[j] = a; kd[j + 64] = bb; vd[j] = c1; vd[j + 64] = c2;
    }
  } else {
    for (int i = tid; i < g * kD; i += kThreads) {
      const int hh = i / kD, j = i % kD;
      const size_t qi = ((size_t)b * p.nq + (size_t)kvh * g + hh) * kD + j;
      qs[hh][j] = p.q_f16 ? h2f(reinterpret_cast<const uint16_t*>(p.q)[qi]) : reinterpret_cast<const float*>(p.q)[qi];
    }
  }
  __syncthreads();
  if (P >= s0 && P < s0 + npos) {  // the new position reads the rows just written to LDS
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
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        a += __shfl_xor(a, 4, 64);
        a += __shfl_xor(a, 8, 64);
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
        float a = acc[hh][t];
        a += __shfl_xor(a, 16, 64);
        a += __shfl_xor(a, 32, 64);
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

  // ---- finish: one split writes directly; otherwise two-level merge of the split records -------
  if (p.nsplit == 1) {
    write_out(p, b, kvh, g, red[0], lh, tid);
    return;
  }
  const int ngroups = (p.nsplit + kGroup - 1) / kGroup;
  const int grp = sidx / kGroup;
  const int gcount = min(kGroup, p.nsplit - grp * kGroup);
  float* part1 = p.part + (size_t)bh * p.nsplit * kMaxG * kPS;
  publish_record(part1 + (size_t)sidx * kMaxG * kPS, g, mh, lh, red[0], tid);
  __syncthreads();
  if (tid == 0) s_flag = arrive(&p.cnt[(size_t)bh * ngroups + grp]) == (unsigned)(gcount - 1);
  __syncthreads();
  if (!s_flag) return;
  merge_parts(part1 + (size_t)grp * kGroup * kMaxG * kPS, gcount, g, ml, tid);
  if (tid == 0) reset_counter(&p.cnt[(size_t)bh * ngroups + grp]);
  if (ngroups == 1) {
    write_out(p, b, kvh, g, ml.O, ml.L, tid);
    return;
  }
  float* part2 = p.part2 + (size_t)bh * ngroups * kMaxG * kPS;
  publish_record(part2 + (size_t)grp * kMaxG * kPS, g, ml.M, ml.L, ml.O, tid);
  __syncthreads();
  unsigned* cnt2 = p.cnt + (size_t)p.B * p.nkv * ngroups;
  if (tid == 0) s_flag = arrive(&cnt2[bh]) == (unsigned)(ngroups - 1);
  __syncthreads();
  if (!s_flag) return;
  merge_parts(part2, ngroups, g, ml, tid);
  if (tid == 0) reset_counter(&cnt2[bh]);
  write_out(p, b, kvh, g, ml.O, ml.L, tid);
}

int pow2ceil(int64_t v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

}  // namespace

// Split size 64/128/256 positions: aims at ~192 workgroups, at most 512 splits per sequence.
void attn_plan(AttnParams& p) {
  const int64_t work = (int64_t)p.B * p.nkv * p.cap;
  int S = pow2ceil(cdiv(work, 192));
  S = S < 64 ? 64 : (S > 256 ? 256 : S);
  p.split = S;
  p.nsplit = (int)cdiv(p.cap, S);
}

size_t attn_workspace_bytes(int B, int nq, int nkv, int nsplit) {
  (void)nq;
  const size_t ngroups = (size_t)cdiv(nsplit, kGroup);
  const size_t rec = (size_t)kMaxG * kPS * sizeof(float);
  const size_t part1 = (size_t)B * nkv * nsplit * rec;
  const size_t part2 = (size_t)B * nkv * ngroups * rec;
  const size_t cnt = (size_t)B * nkv * (ngroups + 1) * sizeof(unsigned);
  return align_up(part1, 256) + align_up(part2, 256) + align_up(cnt, 256);
}

void attn_set_workspace(AttnParams& p, void* ws) {
  const size_t ngroups = (size_t)cdiv(p.nsplit, kGroup);
  const size_t rec = (size_t)kMaxG * kPS * sizeof(float);
  const size_t part1 = (size_t)p.B * p.nkv * p.nsplit * rec;
  const size_t part2 = (size_t)p.B * p.nkv * ngroups * rec;
  char* c = static_cast<char*>(ws);
  p.part = reinterpret_cast<float*>(c);
  p.part2 = reinterpret_cast<float*>(c + align_up(part1, 256));
  p.cnt = reinterpret_cast<unsigned*>(c + align_up(part1, 256) + align_up(part2, 256));
}

hipError_t attn_launch_with_rope(const AttnParams& p, const float* rope_cs, hipStream_t st) {
  const int grid = p.B * p.nkv * p.nsplit;
  switch (p.split) {
    case 64: hipLaunchKernelGGL(k_attn<2>, dim3(grid), dim3(kThreads), 0, st, p, rope_cs); break;
    case 128: hipLaunchKernelGGL(k_attn<4>, dim3(grid), dim3(kThreads), 0, st, p, rope_cs); break;
    default: hipLaunchKernelGGL(k_attn<8>, dim3(grid), dim3(kThreads), 0, st, p, rope_cs); break;
  }
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
