// Split-KV grouped-query decode attention over an fp16 KV cache.
//
// GroupQueryAttention decode over a cache that stays in HBM (GPU-resident KV:
// "VibeVoice-ASR — ONNX export for Vernacula", Highlights), with fp32 scores, softmax and
// accumulation (the same page reports fp32 attention as the accuracy fix over bf16).
//
// Work unit: (sequence b, KV head, split of S = 64 or 128 positions), one workgroup of 4 waves
// serving all g = nq/nkv query heads of the group.  The group's q (a few KiB) is loaded first and
// staged in LDS; then every K and V row of the split is loaded at once: 8 to 16 KiB in flight
// per wave, and B * nkv * ceil(cap / S) workgroups.  With fp16 caches the scores run on the
// matrix cores (K rows loaded straight into the MFMA operand layout, q as fp16 hi + lo parts);
// with fp32 caches 16 lanes share a position and reduce their partial dot products.  Each split
// writes (max, sum, unnormalised output) per head; a second small kernel, one workgroup per query head,
// merges the splits (online-softmax rescaling, fixed order).  The kernel boundary is the
// hand-off, so no workgroup waits on another.  Splits past the sequence exit at once.
//
// Decode-step flavour: q/k/v come from the fused projection output; the workgroup rotates q
// (and, for the split that holds the new position, k) with RoPE, writes fp16 k and v into the
// cache slot of the new position and attends over pos+1 positions.
#include <algorithm>

#include "vv_internal.h"

namespace vv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kD = 128;           // head_dim
constexpr int kMaxG = kAttnMaxG;  // query heads per KV head
constexpr int kPS = kAttnRec;     // partial record: m, l, pad, pad, o[128]
constexpr int kWaves = 4;         // 256 threads per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kMaxSplits = 1024;  // splits per sequence the merge kernel takes
constexpr int kBufWord3 = 0x00020000;  // buffer resource word 3 for raw (untyped) loads on gfx9

// Geometry of one workgroup's split.
struct Geo { int b, kvh, bh, sidx, s0, npos, P; bool has_new; };

__device__ __forceinline__ Geo geo(const AttnParams& p, int S) {
  Geo g;
  const int wg = blockIdx.x;
  g.sidx = wg % p.nsplit;
  g.bh = wg / p.nsplit;
  g.b = g.bh / p.nkv;
  g.kvh = g.bh % p.nkv;
  g.s0 = g.sidx * S;
  int len;
  g.P = -1;
  if (p.qkv) {
    const int P = p.pos[g.b];
    g.P = P < 0 ? 0 : (P >= p.cap ? p.cap - 1 : P);
    len = g.P + 1;
  } else {
    const int l = p.lens[g.b];
    len = l < 1 ? 1 : (l > p.cap ? p.cap : l);
  }
  g.npos = max(0, min(g.s0 + S, len) - g.s0);
  g.has_new = g.P >= g.s0 && g.P < g.s0 + g.npos;
  return g;
}

// K of one lane: 8 dims of one position, fp16 (one 16-byte load) or fp32 (two); V of one lane:
// 2 dims of one position, fp16 (4 bytes) or fp32 (8 bytes)
template <bool KV32> struct KvLane;
template <> struct KvLane<false> { typedef u32x4 K; typedef uint32_t V; };
template <> struct KvLane<true> { struct K { u32x4 a, b; }; typedef uint2 V; };

// q . k over the lane's 8 dims, in dim order (fp16 k read exactly by v_fma_mix_f32)
__device__ __forceinline__ float dot8_kv(const float* q, const u32x4& k, float c) { return dot8_mix(q, k, c); }
__device__ __forceinline__ float dot8_kv(const float* q, const KvLane<true>::K& k, float c) {
  const uint32_t d[8] = {k.a.x, k.a.y, k.a.z, k.a.w, k.b.x, k.b.y, k.b.z, k.b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) c = fmaf(q[i], __uint_as_float(d[i]), c);
  return c;
}
// p * v for the lane's 2 dims
__device__ __forceinline__ void pv_kv(float pj, uint32_t v, float& e, float& o) {
  e = fma_mix_lo(pj, v, e);
  o = fma_mix_hi(pj, v, o);
}
__device__ __forceinline__ void pv_kv(float pj, uint2 v, float& e, float& o) {
  e = fmaf(pj, __uint_as_float(v.x), e);
  o = fmaf(pj, __uint_as_float(v.y), o);
}

// NP passes of 4 positions per wave: split S = 4 waves * 4 * NP positions.  STEP: the decode-step
// flavour (q/k/v from the projection output, RoPE, KV append); else the stand-alone flavour.
// KV32: the cache holds fp32 K/V (the fp32-KV variant: twice the bytes, no fp16 rounding of k, v).
// PVM: P.V on the matrix cores (fp16 caches; more LDS, so the host takes it for grids that are
// resident at once anyway).
template <int NP, bool STEP, bool KV32, bool PVM>
__global__ __launch_bounds__(kThreads) void k_attn(AttnParams p, const float* __restrict__ rope_cs) {
  static_assert(!PVM || !KV32, "the matrix-core P.V reads fp16 V");
  constexpr int S = kWaves * 4 * NP;
  constexpr int kEsz = KV32 ? 4 : 2;       // bytes per cache element
  constexpr int kRow = kD * kEsz;          // bytes per cache row
  typedef typename KvLane<KV32>::K KT;
  typedef typename KvLane<KV32>::V VT;
  __shared__ __align__(16) float qs[KV32 ? kMaxG : 1][kD];   // fp32 q (fp32 caches' VALU scores)
  __shared__ __align__(16) float sc[kMaxG][S];
  __shared__ __align__(16) float red[kWaves][kMaxG][kD];      // [wave][head][dim]
  __shared__ __align__(16) uint16_t knew[KV32 ? 8 : kD], vnew[KV32 ? 8 : kD];
  __shared__ __align__(16) float knew32[KV32 ? kD : 4], vnew32[KV32 ? kD : 4];
  __shared__ float mh[kMaxG], lh[kMaxG];
  // fp16 caches: q of the group as the scores' MFMA B operand, fp16 hi + lo parts, heads g..15 zero
  __shared__ __align__(16) _Float16 qhi[KV32 ? 1 : 16][kD], qlo[KV32 ? 1 : 16][kD];
  // PVM: each wave's V transposed ([dim][position], padded rows) for the P.V MFMAs
  constexpr int kVP = 4 * NP + 4;
  __shared__ __align__(16) uint16_t vt[PVM ? kWaves : 1][PVM ? kD : 1][PVM ? kVP : 2];

  const int g = p.nq / p.nkv;
  const Geo G = geo(p, S);
  if (G.npos == 0) return;                 // past the sequence: the merge skips this split
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr bool step = STEP;

  // ---- q first (small, needed first), then every K/V row of the split; no load is behind a branch
  // step: thread t < 16 g rotates dims 4c..4c+3 with 64+4c..64+4c+3 of head t/16 (c = t%16);
  //       the next 16 threads rotate the new k, the 16 after them take the new v (the other
  //       threads read head 0 and ignore it)
  // stand-alone: thread t < 32 g takes dims 4(t%32)..+3 of head t/32
  float4 qa = make_float4(0.f, 0.f, 0.f, 0.f), qb = qa, ca = make_float4(1.f, 0.f, 1.f, 0.f), cb = ca;
  const int c16 = tid & 15;
  if (step) {
    const float* row = p.qkv + (size_t)G.b * p.ldqkv;
    const int off = tid < 16 * g ? (G.kvh * g + (tid >> 4)) * kD
                  : tid < 16 * g + 16 ? (p.nq + G.kvh) * kD
                  : tid < 16 * g + 32 ? (p.nq + p.nkv + G.kvh) * kD : 0;
    qa = *reinterpret_cast<const float4*>(row + off + 4 * c16);
    qb = *reinterpret_cast<const float4*>(row + off + 64 + 4 * c16);
    ca = *reinterpret_cast<const float4*>(rope_cs + ((size_t)G.b * 64 + 4 * c16) * 2);
    cb = *reinterpret_cast<const float4*>(rope_cs + ((size_t)G.b * 64 + 4 * c16) * 2 + 4);
  } else {
    const size_t qi = ((size_t)G.b * p.nq + (size_t)G.kvh * g + min(tid >> 5, g - 1)) * kD + 4 * (tid & 31);
    if (p.q_f16) {
      const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.q) + qi);
      const h2_t h0 = as_h2(h.x), h1 = as_h2(h.y);
      qa = make_float4((float)h0.x, (float)h0.y, (float)h1.x, (float)h1.y);
    } else {
      qa = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.q) + qi);
    }
  }
  const size_t kvbase = ((size_t)(p.kv_shared ? 0 : G.b) * p.nkv + G.kvh) * (size_t)p.cap * kD;
  const int sl = lane & 15, pg = lane >> 4;
  const int jw = w * 4 * NP;               // first local position of this wave
  // K: lane (pg, sl) holds dims 8 sl..8 sl+7 of position jw + 4 r + pg (16 lanes per position, for
  // the score reductions).  V: lane l holds dims 2 l, 2 l + 1 of every position jw + i of the wave
  // (one 256-byte row per load), so P.V needs no reduction across lanes.  Buffer loads over this
  // (sequence, KV head)'s cap rows: rows past the capacity read as zero instead of needing a clamp
  // per position, and the row offsets become immediates.
  const int kvbytes = p.cap * kRow;
  char* kbase = reinterpret_cast<char*>(p.kc) + kvbase * kEsz;
  char* vbase = reinterpret_cast<char*>(p.vc) + kvbase * kEsz;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(kbase, (short)0, kvbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(vbase, (short)0, kvbytes, kBufWord3);
  const int row0 = G.s0 + jw;              // first position of this wave
  // fp16 caches: load r = 4 nb + ks holds dims 32 ks + 8 (lane / 16) .. + 7 of position
  // jw + 16 nb + lane % 16, the A operand (16 positions x 32 dims) of the scores' MFMAs
  const int kpos = lane & 15, kdim = 8 * (lane >> 4);
  KT kr[NP];
  VT vr[4 * NP];
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    if constexpr (KV32) {
      const int off = (row0 + pg) * kRow + sl * 8 * kEsz + r * 4 * kRow;
      kr[r].a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
      kr[r].b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16, 0, 0));
    } else {
      const int off = (row0 + 16 * (r >> 2) + kpos) * kRow + (32 * (r & 3) + kdim) * kEsz;
      kr[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
    }
  }
#pragma unroll
  for (int i = 0; i < 4 * NP; ++i) {
    const int off = row0 * kRow + lane * 2 * kEsz + i * kRow;
    if constexpr (KV32) vr[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, 0));
    else vr[i] = __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, 0);
  }

  // ---- q (rotated) and the new k/v into LDS; the new position's cache slot ----------------------
  if (step) {
    // pair (j, j+64), j = 4c + i: (x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin); v is not rotated
    const bool rot = p.rope_theta > 0.f && tid < 16 * g + 16;
    const float c4[4] = {ca.x, ca.z, cb.x, cb.z}, s4[4] = {ca.y, ca.w, cb.y, cb.w};
    const float x1[4] = {qa.x, qa.y, qa.z, qa.w}, x2[4] = {qb.x, qb.y, qb.z, qb.w};
    float r1[4], r2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = rot ? x1[i] * c4[i] - x2[i] * s4[i] : x1[i];
      r2[i] = rot ? x2[i] * c4[i] + x1[i] * s4[i] : x2[i];
    }
    if (tid < 16 * g) {
      const int hh = tid >> 4;
      if constexpr (KV32) {
        *reinterpret_cast<float4*>(&qs[hh][4 * c16]) = make_float4(r1[0], r1[1], r1[2], r1[3]);
        *reinterpret_cast<float4*>(&qs[hh][64 + 4 * c16]) = make_float4(r2[0], r2[1], r2[2], r2[3]);
      }
      if constexpr (!KV32) {                 // 4 dims of hi and of lo per 8-byte store
        f16x4 h1, l1, h2, l2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h1[i] = (_Float16)r1[i];
          l1[i] = (_Float16)(r1[i] - (float)h1[i]);
          h2[i] = (_Float16)r2[i];
          l2[i] = (_Float16)(r2[i] - (float)h2[i]);
        }
        *reinterpret_cast<f16x4*>(&qhi[hh][4 * c16]) = h1;
        *reinterpret_cast<f16x4*>(&qlo[hh][4 * c16]) = l1;
        *reinterpret_cast<f16x4*>(&qhi[hh][64 + 4 * c16]) = h2;
        *reinterpret_cast<f16x4*>(&qlo[hh][64 + 4 * c16]) = l2;
      }
    } else if (G.has_new && tid < 16 * g + 32) {
      const bool isk = tid < 16 * g + 16;
      char* cb = (isk ? kbase : vbase) + (size_t)G.P * kRow;
      if constexpr (KV32) {
        float* dst = isk ? knew32 : vnew32;
        float* cache = reinterpret_cast<float*>(cb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[4 * c16 + i] = r1[i];
          dst[64 + 4 * c16 + i] = r2[i];
          cache[4 * c16 + i] = r1[i];
          cache[64 + 4 * c16 + i] = r2[i];
        }
      } else {
        uint16_t* dst = isk ? knew : vnew;
        uint16_t* cache = reinterpret_cast<uint16_t*>(cb);
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
  } else if (tid < 32 * g) {
    if constexpr (KV32) *reinterpret_cast<float4*>(&qs[tid >> 5][4 * (tid & 31)]) = qa;
    if constexpr (!KV32) {
      const float v[4] = {qa.x, qa.y, qa.z, qa.w};
      f16x4 hv, lv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[i] = (_Float16)v[i];
        lv[i] = (_Float16)(v[i] - (float)hv[i]);
      }
      *reinterpret_cast<f16x4*>(&qhi[tid >> 5][4 * (tid & 31)]) = hv;
      *reinterpret_cast<f16x4*>(&qlo[tid >> 5][4 * (tid & 31)]) = lv;
    }
  }
  if constexpr (!KV32) {                     // heads g..15 of the operand are zero (16-byte stores)
    for (int i = tid; i < (16 - g) * (kD / 8); i += kThreads) {
      *reinterpret_cast<u32x4*>(&qhi[g + i / (kD / 8)][8 * (i % (kD / 8))]) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&qlo[g + i / (kD / 8)][8 * (i % (kD / 8))]) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  if (G.has_new) {  // the new position's row was loaded from the cache before it was written
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      if constexpr (KV32) {
        if (G.s0 + jw + 4 * r + pg == G.P) {
          kr[r].a = *reinterpret_cast<const u32x4*>(&knew32[8 * sl]);
          kr[r].b = *reinterpret_cast<const u32x4*>(&knew32[8 * sl + 4]);
        }
      } else {
        if (G.s0 + jw + 16 * (r >> 2) + kpos == G.P) kr[r] = *reinterpret_cast<const u32x4*>(&knew[32 * (r & 3) + kdim]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4 * NP; ++i)
      if (G.s0 + jw + i == G.P) {
        if constexpr (KV32) vr[i] = *reinterpret_cast<const uint2*>(&vnew32[2 * lane]);
        else vr[i] = *reinterpret_cast<const uint32_t*>(&vnew[2 * lane]);
      }
  }
  // rows past the sequence get probability 0; zero their V so that whatever the cache holds there
  // (it is never part of the attention) cannot turn 0 * v into a NaN
#pragma unroll
  for (int i = 0; i < 4 * NP; ++i)
    if (jw + i >= G.npos) vr[i] = VT{};

  // ---- scores ----------------------------------------------------------------------------------
  if constexpr (!KV32) {
    // matrix cores: D (16 positions x 16 heads) = K (16 x 32 dims) . q^T (32 dims x 16 heads) over 4
    // dim steps, q as fp16 hi + lo (the fp16 K is exact, so the products keep fp32 precision);
    // lane l gets positions jw + 16 nb + 4 (l / 16) + r of head l % 16
    f16x8 bh[4], bl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bh[ks] = *reinterpret_cast<const f16x8*>(&qhi[kpos][32 * ks + kdim]);
      bl[ks] = *reinterpret_cast<const f16x8*>(&qlo[kpos][32 * ks + kdim]);
    }
#pragma unroll
    for (int nb = 0; nb < NP / 4; ++nb) {
      f32x4v acc = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 a = __builtin_bit_cast(f16x8, kr[4 * nb + ks]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl[ks], acc, 0, 0, 0);
      }
      if (kpos < g) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jw + 16 * nb + 4 * (lane >> 4) + r;
          sc[kpos][j] = j < G.npos ? acc[r] * p.scale : -INFINITY;
        }
      }
    }
  } else {
    // fp32 caches: 16 lanes per position, reduced across the 16; two heads per pass (independent
    // chains hide the LDS and cross-lane latencies when a SIMD runs a single wave)
#pragma unroll 1
    for (int h0 = 0; h0 < g; h0 += 2) {
      const int h1 = min(h0 + 1, g - 1);     // a repeated head when g is odd: computed, not stored
      float q0[8], q1[8];
      {
        const float4 a0 = *reinterpret_cast<const float4*>(&qs[h0][8 * sl]), b0 = *reinterpret_cast<const float4*>(&qs[h0][8 * sl + 4]);
        const float4 a1 = *reinterpret_cast<const float4*>(&qs[h1][8 * sl]), b1 = *reinterpret_cast<const float4*>(&qs[h1][8 * sl + 4]);
        q0[0] = a0.x; q0[1] = a0.y; q0[2] = a0.z; q0[3] = a0.w; q0[4] = b0.x; q0[5] = b0.y; q0[6] = b0.z; q0[7] = b0.w;
        q1[0] = a1.x; q1[1] = a1.y; q1[2] = a1.z; q1[3] = a1.w; q1[4] = b1.x; q1[5] = b1.y; q1[6] = b1.z; q1[7] = b1.w;
      }
#pragma unroll
      for (int r = 0; r < NP; ++r) {
        const float s0 = row16_sum(dot8_kv(q0, kr[r], 0.f));
        const float s1 = row16_sum(dot8_kv(q1, kr[r], 0.f));
        const int j = jw + 4 * r + pg;
        if (sl == 0) {
          sc[h0][j] = j < G.npos ? s0 * p.scale : -INFINITY;
          if (h0 + 1 < g) sc[h1][j] = j < G.npos ? s1 * p.scale : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // ---- split-local softmax statistics, one wave per head -----------------------------------------
#pragma unroll
  for (int it = 0; it < kMaxG / kWaves; ++it) {       // unrolled: one wave per SIMD, registers spare
    const int hh = w + it * kWaves;
    if (hh >= g) break;
    float m = -INFINITY;
#pragma unroll
    for (int j = lane; j < S; j += 64) m = fmaxf(m, sc[hh][j]);
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int j = lane; j < S; j += 64) {
      const float e = (m == -INFINITY) ? 0.f : expf(sc[hh][j] - m);
      sc[hh][j] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { mh[hh] = m; lh[hh] = l; }
  }
  __syncthreads();

  if constexpr (PVM) {
    // ---- P.V on the matrix cores: O^T (16 dims x 16 heads) += V^T (16 dims x 16 positions) .
    // P^T (16 positions x 16 heads) per 16-position block of the wave, v_mfma_f32_16x16x16f16.  V^T:
    // the lane's two dims of every position go to this wave's LDS tile transposed (a dword holds
    // one dim at two consecutive positions); P^T: the weights from sc as fp16 hi + lo (heads past
    // g zero), so the product keeps fp32 precision against the exact fp16 V.
#pragma unroll
    for (int i = 0; i < 4 * NP; i += 2) {
      const uint32_t a = vr[i], b = vr[i + 1];
      *reinterpret_cast<uint32_t*>(&vt[w][2 * lane][i]) = __builtin_amdgcn_perm(b, a, 0x05040100u);
      *reinterpret_cast<uint32_t*>(&vt[w][2 * lane + 1][i]) = __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int hq = lane & 15, kq = 4 * (lane >> 4);
    f32x4v acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NP / 4; ++kb) {
      const float4 pp = hq < g ? *reinterpret_cast<const float4*>(&sc[hq][jw + 16 * kb + kq])
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      const float pv[4] = {pp.x, pp.y, pp.z, pp.w};
      f16x4 ph, pl;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ph[u] = (_Float16)pv[u];
        pl[u] = (_Float16)(pv[u] - (float)ph[u]);
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const f16x4 va = *reinterpret_cast<const f16x4*>(&vt[w][16 * n + hq][16 * kb + kq]);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pl, acc[n], 0, 0, 0);
      }
    }
    // lane l holds dims 16 n + 4 (l / 16) + r of head l % 16
    if (hq < g) {
#pragma unroll
      for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4v*>(&red[w][hq][16 * n + kq]) = acc[n];
    }
  } else {
    // ---- P.V: lane l accumulates dims 2 l, 2 l + 1 over the wave's 4 NP positions
    // (weights read from LDS as broadcasts, four positions per read); two heads per pass
#pragma unroll
    for (int h0 = 0; h0 < kMaxG; h0 += 2) {             // unrolled: the LDS reads of later pairs overlap
      if (h0 >= g) break;
      const int h1 = min(h0 + 1, g - 1);
      float e0 = 0.f, o0 = 0.f, e1 = 0.f, o1 = 0.f;
#pragma unroll
      for (int r = 0; r < NP; ++r) {
        const float4 a0 = *reinterpret_cast<const float4*>(&sc[h0][jw + 4 * r]);
        const float4 a1 = *reinterpret_cast<const float4*>(&sc[h1][jw + 4 * r]);
        const float q0[4] = {a0.x, a0.y, a0.z, a0.w}, q1[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          pv_kv(q0[u], vr[4 * r + u], e0, o0);
          pv_kv(q1[u], vr[4 * r + u], e1, o1);
        }
      }
      *reinterpret_cast<float2*>(&red[w][h0][2 * lane]) = make_float2(e0, o0);
      if (h0 + 1 < g) *reinterpret_cast<float2*>(&red[w][h1][2 * lane]) = make_float2(e1, o1);
    }
  }
  __syncthreads();

  // ---- the split's output: final when it is the only split, else a record for the merge ----------
  const bool single = p.nsplit == 1;
  float* rec = p.part + ((size_t)G.bh * p.nsplit + G.sidx) * kMaxG * kPS;
#pragma unroll
  for (int it = 0; it < kMaxG * kD / kThreads; ++it) {
    const int i = tid + it * kThreads;
    if (i >= g * kD) break;
    const int hh = i >> 7, d = i & 127;
    float o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) o += red[ww][hh][d];
    if (single) {
      const size_t oi = ((size_t)G.b * p.nq + (size_t)G.kvh * g + hh) * kD + d;
      if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(o / lh[hh]);
      else reinterpret_cast<float*>(p.out)[oi] = o / lh[hh];
    } else {
      rec[(size_t)hh * kPS + 4 + d] = o;
    }
  }
  if (!single && tid < g) {
    rec[(size_t)tid * kPS + 0] = mh[tid];
    rec[(size_t)tid * kPS + 1] = lh[tid];
  }
}

// One workgroup per (sequence, query head, 64-dim half) of W = ceil(nsplit / 64) waves; wave w
// takes splits 64 w .. 64 w + 63.  Lane s of a wave loads the (m, l) of its split s and lane d the
// wave's 64 split values of dim d, all at once; the wave's max and weighted sum come from wave
// reductions and the split weights e_s = exp(m_s - M_w) reach every lane by readlane, so a single
// wave needs no LDS and no barrier.  With W > 1 the waves' (M_w, L_w, O_w) are combined by wave 0
// through LDS after one barrier.  o = sum_s e_s o_s / sum_s e_s l_s, splits in order within a
// wave, then the waves in order.
constexpr int kMergeWaves = kMaxSplits / 64;
__global__ __launch_bounds__(64 * kMergeWaves) void k_attn_merge(AttnParams p, int S) {
  __shared__ float pm[kMergeWaves], pl[kMergeWaves], po[kMergeWaves][64];
  const int g = p.nq / p.nkv;
  const int bq = blockIdx.x >> 1;            // b * nq + head
  const int b = bq / p.nq, h = bq % p.nq;
  const int kvh = h / g, hh = h % g;
  const int bh = b * p.nkv + kvh;
  const int n = attn_splits(p.qkv ? p.pos : nullptr, p.lens, b, p.cap, S);
  const int W = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = 64 * (blockIdx.x & 1) + lane;
  const float* rec0 = p.part + ((size_t)bh * p.nsplit * kMaxG + hh) * kPS;
  float Mw, Lw;
  const float Ow = merge_wave64(rec0, (size_t)kMaxG * kPS, 64 * w, n, d, Mw, Lw);
  const size_t oi = ((size_t)b * p.nq + h) * kD + d;
  if (W == 1) {
    if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(Ow / Lw);
    else reinterpret_cast<float*>(p.out)[oi] = Ow / Lw;
    return;
  }
  if (lane == 0) { pm[w] = Mw; pl[w] = Lw; }
  po[w][lane] = Ow;
  __syncthreads();
  if (w != 0) return;
  float M = -INFINITY;
  for (int ww = 0; ww < W; ++ww) M = fmaxf(M, pm[ww]);      // finite: wave 0 holds split 0
  float O = 0.f, L = 0.f;
  for (int ww = 0; ww < W; ++ww) {
    const float f = pm[ww] == -INFINITY ? 0.f : expf(pm[ww] - M);   // a wave past the sequence: 0
    O = fmaf(f, po[ww][lane], O);
    L = fmaf(f, pl[ww], L);
  }
  if (p.out_f16) reinterpret_cast<uint16_t*>(p.out)[oi] = f2h(O / L);
  else reinterpret_cast<float*>(p.out)[oi] = O / L;
}

}  // namespace

// Split size 64 positions, or 128 when that would give more than ~2048 workgroups or more than
// the merge's 1024 splits per sequence (so cap <= 131072 always fits).
void attn_plan(AttnParams& p) {
  const int64_t n64 = cdiv(p.cap, 64);
  const int64_t wgs64 = (int64_t)p.B * p.nkv * n64;
  p.split = wgs64 > 2048 || n64 > kMaxSplits ? 128 : 64;
  p.nsplit = (int)cdiv(p.cap, p.split);
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

hipError_t attn_launch_with_rope(const AttnParams& p, const float* rope_cs, hipStream_t st, KEv ev) {
  const int grid = p.B * p.nkv * p.nsplit;
  const KEv e1 = p.nsplit == 1 || p.skip_merge ? ev : ev.first();
  const bool step = p.qkv != nullptr;
  // the matrix-core P.V takes more LDS: only for grids resident at once with it (<= 2 per CU)
  const bool pvm = !p.kv_f32 && grid <= 2 * 256;
#define VV_ATTN_CASE(NP, KV32, PVM)                                                                      \
  if (step) VV_LAUNCH((k_attn<NP, true, KV32, PVM>), dim3(grid), dim3(kThreads), st, e1, p, rope_cs);     \
  else VV_LAUNCH((k_attn<NP, false, KV32, PVM>), dim3(grid), dim3(kThreads), st, e1, p, rope_cs);
  if (p.split == 64) {
    if (p.kv_f32) { VV_ATTN_CASE(4, true, false) } else if (pvm) { VV_ATTN_CASE(4, false, true) } else { VV_ATTN_CASE(4, false, false) }
  } else {
    if (p.kv_f32) { VV_ATTN_CASE(8, true, false) } else if (pvm) { VV_ATTN_CASE(8, false, true) } else { VV_ATTN_CASE(8, false, false) }
  }
#undef VV_ATTN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1 || p.skip_merge) return e;
  VV_LAUNCH(k_attn_merge, dim3(p.B * p.nq * 2), dim3(64 * cdiv(p.nsplit, 64)), st, ev.last(), p, p.split);
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
  VV_REQUIRE(cap <= 128 * kMaxSplits, VV_ERR_RANGE, "vv_gqa_decode: cap %d > 131072 positions", cap);
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
