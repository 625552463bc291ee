// Split-KV grouped-query decode attention over an fp16 KV cache.
//
// GroupQueryAttention decode over a cache that stays in HBM (GPU-resident KV:
// "VibeVoice-ASR — ONNX export for Vernacula", Highlights), with fp32 scores, softmax and
// accumulation (the same page reports fp32 attention as the accuracy fix over bf16).
//
// Work unit: (sequence b, KV head, split of `split` positions).  A workgroup reads each K and V
// row of its split once (16 lanes x 16 B per row, rows contiguous in HBM) and serves all
// g = nq/nkv query heads of the group with it.  It writes (max, sum, unnormalised output) per
// head; the last workgroup of a (b, KV head) to finish merges the splits in a fixed order
// (online-softmax rescaling) and writes the output.
//
// Decode-step flavour: q/k/v come from the fused projection output; the workgroup rotates q
// (and, for the split that holds the new position, k) with RoPE, writes fp16 k and v into the
// cache slot of the new position and attends over pos+1 positions.
#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kD = 128;        // head_dim
constexpr int kMaxG = 8;       // query heads per KV head
constexpr int kPartStride = 132;  // m, l, pad, pad, o[128]

__global__ __launch_bounds__(256) void k_attn(AttnParams p, const float* __restrict__ rope_cs) {
  __shared__ float qs[kMaxG][kD];
  __shared__ float sc[kMaxG][256];
  __shared__ float red[4][kMaxG][kD];
  __shared__ uint16_t knew[kD], vnew[kD];
  __shared__ float mh[kMaxG], lh[kMaxG];
  __shared__ unsigned s_last;

  const int g = p.nq / p.nkv;
  const int S = p.split;
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
  const int s1 = min(s0 + S, len);
  const int npos = s1 > s0 ? s1 - s0 : 0;

  const size_t kvbase = ((size_t)b * p.nkv + kvh) * (size_t)p.cap * kD;
  const uint16_t* Kc = p.kc + kvbase;
  const uint16_t* Vc = p.vc + kvbase;

  // ---- q (and new k, v) into LDS --------------------------------------------------------
  if (step) {
    const float* row = p.qkv + (size_t)b * p.ldqkv;
    const float* cs = rope_cs + (size_t)b * 64 * 2;
    const bool rope = p.rope_theta > 0.f;
    for (int i = tid; i < g * 64; i += 256) {
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
    if (P >= s0 && P < s1 && tid < 64) {
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
    for (int i = tid; i < g * kD; i += 256) {
      const int hh = i / kD, j = i % kD;
      const size_t qi = ((size_t)b * p.nq + (size_t)kvh * g + hh) * kD + j;
      qs[hh][j] = p.q_f16 ? h2f(reinterpret_cast<const uint16_t*>(p.q)[qi]) : reinterpret_cast<const float*>(p.q)[qi];
    }
  }
  __syncthreads();

  // ---- scores: 16 lanes per position (8 dims each), 4 positions per wave pass -------------
  const int sl = lane & 15;          // dim slice: dims 8*sl .. 8*sl+7
  const int pg = lane >> 4;          // position within the wave pass
  float qr[kMaxG][8];
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[hh][i] = hh < g ? qs[hh][8 * sl + i] : 0.f;

  for (int base = w * 4; base < S; base += 16) {
    const int j = base + pg;         // local position
    const int pos = s0 + j;
    const bool valid = j < npos;
    u32x4 kv = u32x4{0, 0, 0, 0};
    if (valid) {
      if (pos == P) kv = *reinterpret_cast<const u32x4*>(&knew[8 * sl]);
      else kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kc + (size_t)pos * kD + 8 * sl));
    }
    float kf[8];
    {
      const uint32_t d4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2_t hv = as_h2(d4[i]);
        kf[2 * i] = (float)hv.x;
        kf[2 * i + 1] = (float)hv.y;
      }
    }
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      if (hh < g) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(qr[hh][i], kf[i], a);
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        a += __shfl_xor(a, 4, 64);
        a += __shfl_xor(a, 8, 64);
        if (sl == 0 && j < S) sc[hh][j] = valid ? a * p.scale : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- split-local softmax statistics -----------------------------------------------------
  for (int hh = w; hh < g; hh += 4) {
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

  // ---- weighted sum of V --------------------------------------------------------------------
  float acc[kMaxG][8];
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[hh][i] = 0.f;
  for (int base = w * 4; base < S; base += 16) {
    const int j = base + pg;
    const int pos = s0 + j;
    if (j < npos) {
      u32x4 vv;
      if (pos == P) vv = *reinterpret_cast<const u32x4*>(&vnew[8 * sl]);
      else vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vc + (size_t)pos * kD + 8 * sl));
      float vf[8];
      const uint32_t d4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2_t hv = as_h2(d4[i]);
        vf[2 * i] = (float)hv.x;
        vf[2 * i + 1] = (float)hv.y;
      }
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh) {
        if (hh < g) {
          const float pj = sc[hh][j];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[hh][i] = fmaf(pj, vf[i], acc[hh][i]);
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh) {
    if (hh < g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = acc[hh][i];
        a += __shfl_xor(a, 16, 64);
        a += __shfl_xor(a, 32, 64);
        if (pg == 0) red[w][hh][8 * sl + i] = a;
      }
    }
  }
  __syncthreads();

  // ---- publish / finish ---------------------------------------------------------------------
  const size_t bhbase = (size_t)bh * p.nsplit;
  if (p.nsplit == 1) {
    for (int i = tid; i < g * kD; i += 256) {
      const int hh = i / kD, d = i % kD;
      const float o = (((red[0][hh][d] + red[1][hh][d]) + red[2][hh][d]) + red[3][hh][d]) / lh[hh];
      const size_t oi = ((size_t)b * p.nq + (size_t)kvh * g + hh) * kD + d;
      if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(o);
      else reinterpret_cast<float*>(p.out)[oi] = o;
    }
    return;
  }
  float* mypart = p.part + (bhbase + sidx) * kMaxG * kPartStride;
  for (int i = tid; i < g * kD; i += 256) {
    const int hh = i / kD, d = i % kD;
    mypart[hh * kPartStride + 4 + d] = ((red[0][hh][d] + red[1][hh][d]) + red[2][hh][d]) + red[3][hh][d];
  }
  if (tid < g) {
    mypart[tid * kPartStride + 0] = mh[tid];
    mypart[tid * kPartStride + 1] = lh[tid];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&p.cnt[bh], 1u) == (unsigned)(p.nsplit - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* parts = p.part + bhbase * kMaxG * kPartStride;
  for (int i = tid; i < g * kD; i += 256) {
    const int hh = i / kD, d = i % kD;
    float M = -INFINITY;
    for (int s = 0; s < p.nsplit; ++s)
      M = fmaxf(M, __builtin_nontemporal_load(parts + ((size_t)s * kMaxG + hh) * kPartStride));
    float L = 0.f, O = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
      const float* ps = parts + ((size_t)s * kMaxG + hh) * kPartStride;
      const float ms = __builtin_nontemporal_load(ps);
      if (ms == -INFINITY) continue;
      const float e = expf(ms - M);
      L = fmaf(e, __builtin_nontemporal_load(ps + 1), L);
      O = fmaf(e, __builtin_nontemporal_load(ps + 4 + d), O);
    }
    const float o = O / L;
    const size_t oi = ((size_t)b * p.nq + (size_t)kvh * g + hh) * kD + d;
    if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(o);
    else reinterpret_cast<float*>(p.out)[oi] = o;
  }
  if (tid == 0) p.cnt[bh] = 0u;
}

int pow2ceil(int64_t v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

}  // namespace

void attn_plan(AttnParams& p) {
  // aim for ~512 workgroups; splits of 32..256 positions (multiples of 16)
  const int64_t work = (int64_t)p.B * p.nkv * p.cap;
  int S = pow2ceil(cdiv(work, 512));
  S = S < 32 ? 32 : (S > 256 ? 256 : S);
  p.split = S;
  p.nsplit = (int)cdiv(p.cap, S);
}

size_t attn_workspace_bytes(int B, int nq, int nkv, int nsplit) {
  (void)nq;
  const size_t part = (size_t)B * nkv * nsplit * kMaxG * kPartStride * sizeof(float);
  const size_t cnt = (size_t)B * nkv * sizeof(unsigned);
  return align_up(part, 256) + align_up(cnt, 256);
}

void attn_set_workspace(AttnParams& p, void* ws) {
  const size_t part = (size_t)p.B * p.nkv * p.nsplit * kMaxG * kPartStride * sizeof(float);
  p.part = reinterpret_cast<float*>(ws);
  p.cnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + align_up(part, 256));
}

hipError_t attn_launch_with_rope(const AttnParams& p, const float* rope_cs, hipStream_t st) {
  const int grid = p.B * p.nkv * p.nsplit;
  hipLaunchKernelGGL(k_attn, dim3(grid), dim3(256), 0, st, p, rope_cs);
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
  VV_REQUIRE((int64_t)B * nkv * cap <= (int64_t)1 << 40, VV_ERR_RANGE, "vv_gqa_decode: cache too large");
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
