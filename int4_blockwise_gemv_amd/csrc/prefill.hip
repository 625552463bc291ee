// Prefill (decoder_init) of one sequence: the S prompt embeddings at positions 0..S-1 of an empty
// cache -> the present K/V of those positions, written into the decode step's cache layout, and
// the logits and greedy token of the last position ("vibevoice-asr-bitnet-onnx" page, graph
// contracts: decoder_init runs the prompt, decoder_step then continues from its cache).  The
// layer is the decode step's Qwen2 layer (1.5B STATUS page, Architecture) applied to S rows.
//
// Per layer: RMSNorm rows -> q|k|v GEMM (+bias) -> RoPE + K/V cache write -> causal attention ->
// o GEMM (+residual) -> RMSNorm rows -> gate/up GEMM (SiLU * up) -> down GEMM (+residual); then
// the final RMSNorm of the last row and the lm_head + argmax of the decode step.
//
// The GEMMs are int4-dequant contractions on the matrix cores over the decode step's tiled weights:
// each wave of a workgroup owns one 64-row tile, all waves share the workgroup's tokens, staged in
// LDS; per 32-k block a wave turns its tile's block (1 KiB, lane = row) into the four 16-row B
// operands with the permlane transpose, scales the dequantised codes by the block's fp16 scale and
// runs v_mfma_f32_16x16x32_f16 against every 16-token group.  The causal attention is a
// matrix-core kernel with an online softmax, over fp16 caches or (as fp16 hi + lo parts) fp32 ones.
#include <algorithm>

#include "vv_internal.h"
#include "gemv_core.h"

namespace vv {
namespace {

constexpr int kHD = 128;                     // head_dim
constexpr int kPfTG = 4;                     // GEMM token groups of 16 per workgroup (64 tokens)
constexpr int kPfNW = 4;                     // GEMM waves (64-row tiles) per workgroup

struct PfGemm {
  const uint8_t* q; const uint16_t* s;       // tiled int4 weights, ntiles tiles of 64 rows
  const uint16_t* x;                         // fp16 [S][K]
  int S, K, N, ntiles;                       // N: output rows (EPI_SILU: rows of gate = of up)
  const uint16_t* bias;                      // EPI_STORE: fp16 [N] or null
  float* y; int ldy;                         // EPI_STORE: fp32 [S][ldy]
  float* h;                                  // EPI_RESID: fp32 [S][N], h += W x
  uint16_t* act;                             // EPI_SILU: fp16 [S][N]
};

// 8 codes of one dword -> 8 fp16 (q - 8) * s, in the order of the decode GEMVs' codes_to_half8: the
// exact code pairs, then one packed multiply by the block scale s2 = (s, s): exact for ternary codes
// (q - 8 in {-1, 0, 1}); for general int4 codes the product rounds once to fp16 (relative error
// <= 2^-11).
__device__ __forceinline__ half8 codes_to_half8_scaled(uint32_t d, uint32_t m1024, uint32_t m64, h2_t s2) {
  h2_t p[4];
  code_pairs_exact(d, m1024, m64, p);
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = p[i] * s2;
  return half8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

// (s, s) for the fp16 scale of block i (0..7) out of a lane's 4 scale dwords
__device__ __forceinline__ h2_t scale_pair(const u32x4& s, int i) {
  const uint32_t d = (i >> 1) == 0 ? s.x : (i >> 1) == 1 ? s.y : (i >> 1) == 2 ? s.z : s.w;
  return as_h2(__builtin_amdgcn_perm(d, d, (i & 1) ? 0x03020302u : 0x01000100u));
}

// One workgroup = NW waves x (its own 64-row tile) x the same 16 TG tokens.
template <int EPI, int TG, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_pf_gemm(PfGemm p) {   // two waves per SIMD
  constexpr int kTok = 16 * TG;              // tokens per workgroup
  constexpr int kChunks = 8 * TG;            // 1 KiB chunks per stage: 8 blocks x TG token groups
  constexpr int kPerWave = kChunks / NW;     // chunks each wave stages
  static_assert(kChunks % NW == 0, "stage chunks split evenly over the waves");
  __shared__ __align__(16) uint8_t As[2][kChunks * 1024];
  // workgroup -> (tile group, token block): XCD x takes tile groups x, x + 8, ... and runs every
  // token block of one tile group back to back, so its tiles' weights come from HBM once and
  // from the XCD's L2 after that
  const int ntb = (p.S + kTok - 1) / kTok, ntg = (p.ntiles + NW - 1) / NW;
  const int xcd = blockIdx.x & 7, seq = blockIdx.x >> 3;
  const int tb = seq % ntb, tgrp = 8 * (seq / ntb) + xcd;
  if (tgrp >= ntg) return;                   // padding of the grid to whole rounds of 8
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int tile_u = tgrp * NW + w;
  const int tile = min(tile_u, p.ntiles - 1); // a wave past the last tile recomputes it, stores nothing
  const int t0 = tb * kTok;
  const int K = p.K, nb = K / kBlock, ng = (nb + 7) / 8;
  const u32x4* qt = reinterpret_cast<const u32x4*>(p.q) + (size_t)tile * nb * kTileRows + lane;
  const u32x4* st = reinterpret_cast<const u32x4*>(p.s) + (size_t)tile * ng * kTileRows + (lane & 15);
  // A staging, operand order: 1 KiB chunk TG i + j of a stage holds block i (of 8) of token group j
  // (16 tokens), lane l's 16 B = token 16 j + l % 16, k 32 i + 8 (l / 16) .. + 7.  Wave w fills
  // chunks NW u + w.  Token rows past S are clamped (computed, not stored); blocks past K are
  // clamped (their MFMAs are skipped).
  const uint16_t* xs[kPerWave];
#pragma unroll
  for (int u = 0; u < kPerWave; ++u) {
    const int c = NW * u + w, j = c % TG;
    xs[u] = p.x + (size_t)min(t0 + 16 * j + (lane & 15), p.S - 1) * K + 8 * (lane >> 4);
  }
  auto load_stage = [&](int grp, u32x4 (&r)[kPerWave]) {
#pragma unroll
    for (int u = 0; u < kPerWave; ++u) {
      const int blk = min(grp * 8 + (NW * u + w) / TG, nb - 1);
      r[u] = *reinterpret_cast<const u32x4*>(xs[u] + (size_t)blk * kBlock);
    }
  };
  auto store_stage = [&](int buf, const u32x4 (&r)[kPerWave]) {
#pragma unroll
    for (int u = 0; u < kPerWave; ++u) *reinterpret_cast<u32x4*>(&As[buf][(NW * u + w) * 1024 + lane * 16]) = r[u];
  };
  // a group's weights: 8 blocks of the tile (lane = row), and the 8 scales of each operand row
  // 16 g + lane % 16 (the scale rows are read straight in operand order, 4 x 16 B per lane)
  auto load_w = [&](int grp, u32x4 (&wv)[8], u32x4 (&sv)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) sv[g] = st[(size_t)grp * kTileRows + 16 * g];
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = qt[(size_t)min(grp * 8 + i, nb - 1) * kTileRows];
  };

  const uint32_t m64 = vconst(0x54005400u), m1024 = vconst(0x64006400u);
  f32x4 acc[TG][4];
#pragma unroll
  for (int j = 0; j < TG; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ar[kPerWave], wv[8], s4[4];
  load_stage(0, ar);
  load_w(0, wv, s4);
  store_stage(0, ar);
  __syncthreads();
  for (int grp = 0; grp < ng; ++grp) {
    const int cur = grp & 1, nxt = min(grp + 1, ng - 1);
    // the next group's operands are in flight while this group computes (the last group reloads
    // its own, unused, so that no load sits under a branch)
    u32x4 wn[8], sn[4];
    load_stage(nxt, ar);
    load_w(nxt, wn, sn);
    const uint8_t* as = As[cur] + lane * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (grp * 8 + i >= nb) break;          // the last group of a K that is not a multiple of 256
      half8 a[TG];
#pragma unroll
      for (int j = 0; j < TG; ++j) a[j] = *reinterpret_cast<const half8*>(as + (TG * i + j) * 1024);
      uint32_t tq[4];
      block_to_operands(wv[i], tq);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const half8 bop = codes_to_half8_scaled(tq[g], m1024, m64, scale_pair(s4[g], i));
#pragma unroll
        for (int j = 0; j < TG; ++j) acc[j][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], bop, acc[j][g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = wn[i];
#pragma unroll
    for (int g = 0; g < 4; ++g) s4[g] = sn[g];
    // every wave finished reading stage buffer cur ^ 1 before the previous barrier
    store_stage(cur ^ 1, ar);
    __syncthreads();
  }
  if (tile_u >= p.ntiles) return;

  // lane l holds tokens t0 + 16 j + 4 (l / 16) + r and tile row 16 g + l % 16
#pragma unroll
  for (int j = 0; j < TG; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * j + 4 * (lane >> 4) + r;
      if (t >= p.S) continue;
      if (EPI == EPI_SILU) {                 // rows 0..31 of the tile are gate rows, 32..63 the up rows
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int n = tile * 32 + 16 * g + (lane & 15);
          if (n < p.N) p.act[(size_t)t * p.N + n] = f2h(silu(acc[j][g][r]) * acc[j][g + 2][r]);
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = tile * kTileRows + 16 * g + (lane & 15);
          if (n >= p.N) continue;
          if (EPI == EPI_STORE) p.y[(size_t)t * p.ldy + n] = acc[j][g][r] + (p.bias ? h2f(p.bias[n]) : 0.f);
          else p.h[(size_t)t * p.N + n] += acc[j][g][r];
        }
      }
    }
}

// RMSNorm of row t: out = fp16(gamma * h * rstd), rstd = 1/sqrt(mean(h^2) + eps).  With emb set
// the row is first taken from the fp16 input embeddings into h.  With outf set (the final norm of
// the last row) the result is written in fp32 instead.
__global__ __launch_bounds__(256) void k_pf_norm(const uint16_t* __restrict__ emb, float* __restrict__ h, int row0,
                                                 int H, const uint16_t* __restrict__ gamma, float eps,
                                                 uint16_t* __restrict__ out, float* __restrict__ outf) {
  __shared__ float red[4];
  const int t = row0 + blockIdx.x;
  float* hr = h + (size_t)t * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) {
    float v;
    if (emb) {
      v = h2f(emb[(size_t)t * H + i]);
      hr[i] = v;
    } else {
      v = hr[i];
    }
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float rstd = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256) {
    const float v = h2f(gamma[i]) * hr[i] * rstd;
    if (outf) outf[i] = v;
    else out[(size_t)t * H + i] = f2h(v);
  }
}

// element i of a cache, fp16 or fp32
__device__ __forceinline__ void put_kv(void* c, size_t i, float v, bool kv32) {
  if (kv32) static_cast<float*>(c)[i] = v;
  else static_cast<uint16_t*>(c)[i] = f2h(v);
}

// RoPE of token t at position t (NeoX rotate-half pairs (j, j + 64), angles in fp64 as in the
// decode step): q -> qr fp32 [S][nq][128]; k, v -> fp16 (fp32 with kv32) into the cache slot t.
__global__ __launch_bounds__(256) void k_pf_rope_kv(const float* __restrict__ qkv, int nq, int nkv, int cap,
                                                    double theta, float* __restrict__ qr, void* __restrict__ kc,
                                                    void* __restrict__ vc, int kv32) {
  __shared__ float cs[64][2];
  const int t = blockIdx.x;
  const int ld = (nq + 2 * nkv) * kHD;
  const float* row = qkv + (size_t)t * ld;
  if (threadIdx.x < 64) {
    float c = 1.f, s = 0.f;
    if (theta > 0.0) {
      const double inv = pow(theta, -(double)(2 * threadIdx.x) / (double)kHD);
      double sd, cd;
      sincos((double)t * inv, &sd, &cd);
      c = (float)cd;
      s = (float)sd;
    }
    cs[threadIdx.x][0] = c;
    cs[threadIdx.x][1] = s;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < (nq + nkv) * 64; idx += 256) {
    const int hh = idx >> 6, j = idx & 63;
    const float x1 = row[hh * kHD + j], x2 = row[hh * kHD + j + 64];
    const float c = cs[j][0], s = cs[j][1];
    const float r1 = x1 * c - x2 * s, r2 = x2 * c + x1 * s;
    if (hh < nq) {
      qr[((size_t)t * nq + hh) * kHD + j] = r1;
      qr[((size_t)t * nq + hh) * kHD + j + 64] = r2;
    } else {
      const size_t i0 = ((size_t)(hh - nq) * cap + t) * kHD;
      put_kv(kc, i0 + j, r1, kv32);
      put_kv(kc, i0 + j + 64, r2, kv32);
    }
  }
  for (int idx = threadIdx.x; idx < nkv * kHD; idx += 256) {
    const int kvh = idx / kHD, d = idx % kHD;
    put_kv(vc, ((size_t)kvh * cap + t) * kHD + d, row[(nq + nkv) * kHD + idx], kv32);
  }
}

// ---- causal attention of the prompt on the matrix cores (fp16 caches) -----------------------------
// A workgroup takes one query head and a block of 64 consecutive queries (4 waves x 16) and walks the keys
// 0 .. (its last query) in blocks of 32 with an online softmax in base 2 (q carries log2 e), fp32.
// The products are taken transposed so that every lane owns one query:
//   S^T = K Q^T: A = K (16 keys x 32 dims, the fp16 cache: exact), B = Q^T (the fp16 hi + lo parts
//     of the scaled fp32 q, so the product keeps fp32 precision) -> lane l holds query l % 16 and
//     keys 16 nb + 4 (l / 16) + r of the block;
//   O^T += V^T P^T: B = P^T straight from those registers (fp16 hi + lo of the fp32 weights); the
//     k order of this product is the lane groups' key order, so V is staged transposed with its
//     keys permuted to match (lane group g's 8 keys contiguous) -> lane l holds query l % 16 and
//     dims 16 n + 4 (l / 16) + r.
// The max, the rescale factor and the running sum are then per lane; the max is exchanged across
// the 4 lane groups with two lane shuffles.  K and V blocks are staged in double-buffered LDS,
// one barrier per block, the next block's loads in flight during the current one; a wave skips
// the blocks that lie entirely after its queries.  A workgroup takes two query blocks, the
// (nqb - 1 - x)-th and the x-th, so that every workgroup walks about the same number of keys.
constexpr int kFaQ = 64;                     // queries per workgroup
constexpr int kFaK = 32;                     // keys per block
constexpr int kFaKP = kFaK + 8;              // padded LDS rows
constexpr int kFaDP = kHD + 8;

__device__ __forceinline__ void split_hi_lo(const float* v, half8& hi, half8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)v[i];
    hi[i] = h;
    lo[i] = (_Float16)(v[i] - (float)h);
  }
}

// max and sum over the 4 lane groups (lanes l % 16 equal)
__device__ __forceinline__ float groups_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  return fmaxf(v, __shfl_xor(v, 32, kWave));
}
__device__ __forceinline__ float groups_sum(float v) {
  v += __shfl_xor(v, 16, kWave);
  return v + __shfl_xor(v, 32, kWave);
}

// fp16 hi and lo parts of 8 fp32 values, packed in k order
__device__ __forceinline__ void split8(const u32x4& a, const u32x4& b, u32x4& hi, u32x4& lo) {
  const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float f = __uint_as_float(v[i]);
    const _Float16 t = (_Float16)f;
    h[i] = __builtin_bit_cast(uint16_t, t);
    l[i] = __builtin_bit_cast(uint16_t, (_Float16)(f - (float)t));
  }
  hi = u32x4{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
  lo = u32x4{l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16};
}

// KV32: fp32 caches.  K and V are staged as fp16 hi + lo parts (Ks/Vt and Kl/Vl), and each product
// takes the three terms hi.hi, hi.lo, lo.hi (the lo.lo term is below fp32 rounding).
template <bool KV32>
__global__ __launch_bounds__(256, 2) void k_pf_flash(const float* __restrict__ qr, const void* __restrict__ kc,
                                                     const void* __restrict__ vc, int S, int nq, int nkv, int cap,
                                                     float scale, uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint16_t Ks[2][kFaK][kFaDP];       // [buffer][key][dim]
  __shared__ __align__(16) uint16_t Vt[2][kHD][kFaKP];        // [buffer][dim][permuted key]
  __shared__ __align__(16) uint16_t Kl[KV32 ? 2 : 1][KV32 ? kFaK : 1][KV32 ? kFaDP : 8];
  __shared__ __align__(16) uint16_t Vl[KV32 ? 2 : 1][KV32 ? kHD : 1][KV32 ? kFaKP : 8];
  constexpr int kEsz = KV32 ? 4 : 2;
  constexpr int kLd = KV32 ? 4 : 2;          // 16-byte loads per row chunk of 8 dims: K, V of two rows
  const int h = blockIdx.y, kvh = h / (nq / nkv);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, grp = lane >> 4;
  const char* kbase = static_cast<const char*>(kc) + (size_t)kvh * cap * kHD * kEsz;
  const char* vbase = static_cast<const char*>(vc) + (size_t)kvh * cap * kHD * kEsz;
  // staging: thread -> key pair sp (rows 2 sp, 2 sp + 1) and 8-dim chunk sc; four consecutive
  // lanes read 64 (fp32: 128) contiguous bytes of a row.  V goes to LDS transposed, as dwords
  // holding the pair's two keys of one dimension, at the permuted key position of key 2 sp.
  const int sp = lane >> 2, sc = 4 * w + (lane & 3);
  const int kp = 2 * sp;
  const int vpos = 8 * ((kp & 15) >> 2) + 4 * (kp >> 4) + (kp & 3);
  // r: K row 2 sp, K row 2 sp + 1, V row 2 sp, V row 2 sp + 1 (each 8 dims: 1 or 2 loads)
  auto load_blk = [&](int kb, u32x4 (&r)[2 * kLd]) {
    const size_t r0 = ((size_t)min(kb + kp, S - 1) * kHD + 8 * sc) * kEsz;
    const size_t r1 = ((size_t)min(kb + kp + 1, S - 1) * kHD + 8 * sc) * kEsz;
    const size_t off[4] = {r0, r1, r0, r1};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const char* base = j < 2 ? kbase : vbase;
#pragma unroll
      for (int c = 0; c < kLd / 2; ++c) r[j * (kLd / 2) + c] = *reinterpret_cast<const u32x4*>(base + off[j] + 16 * c);
    }
  };
  auto put_v = [&](uint16_t (*dst)[kFaKP], const u32x4& a4, const u32x4& b4) {
    const uint32_t a[4] = {a4.x, a4.y, a4.z, a4.w}, b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)              // (V[2 sp][d], V[2 sp + 1][d]) for d = 8 sc + i
      *reinterpret_cast<uint32_t*>(&dst[8 * sc + i][vpos]) =
          __builtin_amdgcn_perm(b[i >> 1], a[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
  };
  auto stage = [&](int buf, const u32x4 (&r)[2 * kLd]) {
    if constexpr (KV32) {
      u32x4 kh0, kl0, kh1, kl1, vh0, vl0, vh1, vl1;
      split8(r[0], r[1], kh0, kl0);
      split8(r[2], r[3], kh1, kl1);
      split8(r[4], r[5], vh0, vl0);
      split8(r[6], r[7], vh1, vl1);
      *reinterpret_cast<u32x4*>(&Ks[buf][kp][8 * sc]) = kh0;
      *reinterpret_cast<u32x4*>(&Ks[buf][kp + 1][8 * sc]) = kh1;
      *reinterpret_cast<u32x4*>(&Kl[buf][kp][8 * sc]) = kl0;
      *reinterpret_cast<u32x4*>(&Kl[buf][kp + 1][8 * sc]) = kl1;
      put_v(Vt[buf], vh0, vh1);
      put_v(Vl[buf], vl0, vl1);
    } else {
      *reinterpret_cast<u32x4*>(&Ks[buf][kp][8 * sc]) = r[0];
      *reinterpret_cast<u32x4*>(&Ks[buf][kp + 1][8 * sc]) = r[1];
      put_v(Vt[buf], r[2], r[3]);
    }
  };

  // the workgroup takes query block nqb - 1 - x and then query block x: every workgroup walks
  // about the same number of keys
  const int nqb = (S + kFaQ - 1) / kFaQ;
  for (int pass = 0; pass < 2; ++pass) {
    const int qblk = pass == 0 ? nqb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (pass == 1 && qblk >= nqb - 1 - (int)blockIdx.x) break;   // the middle block of an odd count
    const int qb = qblk * kFaQ;
    const int q0 = qb + 16 * w, q = q0 + (lane & 15);

    // B operands of q: query q, dims 32 ks + 8 (lane / 16) .. + 7, scaled, hi + lo
    half8 qh[4], ql[4];
    {
      const float* qrow = qr + ((size_t)min(q, S - 1) * nq + h) * kHD + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 a = *reinterpret_cast<const float4*>(qrow + 32 * ks);
        const float4 b = *reinterpret_cast<const float4*>(qrow + 32 * ks + 4);
        const float v[8] = {a.x * scale, a.y * scale, a.z * scale, a.w * scale,
                            b.x * scale, b.y * scale, b.z * scale, b.w * scale};
        split_hi_lo(v, qh[ks], ql[ks]);
      }
    }
    float m_i = -INFINITY, l_part = 0.f;     // running max of query q; this lane's share of its sum
    f32x4 O[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int kend = min(S, qb + kFaQ);      // keys the block's last query sees
    u32x4 kv[2 * kLd];
    load_blk(0, kv);
    stage(0, kv);                            // every wave finished the previous pass before its last barrier
    __syncthreads();
    load_blk(kFaK, kv);
    int buf = 0;
    for (int kb = 0; kb < kend; kb += kFaK, buf ^= 1) {
      if (kb <= q0 + 15) {                   // else every query of this wave is before the block
        // scores (base 2): sT[nb][r] = query q . key kb + 16 nb + 4 grp + r
        f32x4 sT[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const half8 kop = *reinterpret_cast<const half8*>(&Ks[buf][16 * nb + (lane & 15)][32 * ks + 8 * grp]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qh[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, ql[ks], acc, 0, 0, 0);
            if constexpr (KV32) {
              const half8 klo = *reinterpret_cast<const half8*>(&Kl[buf][16 * nb + (lane & 15)][32 * ks + 8 * grp]);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(klo, qh[ks], acc, 0, 0, 0);
            }
          }
          sT[nb] = acc;
        }
        if (kb + kFaK - 1 > q0 || kb + kFaK > S) {   // causal mask (and the end of the prompt)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kb + 16 * nb + 4 * grp + r;
              if (key > q || key >= S) sT[nb][r] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(sT[0][0], sT[0][1]), fmaxf(sT[0][2], sT[0][3])),
                         fmaxf(fmaxf(sT[1][0], sT[1][1]), fmaxf(sT[1][2], sT[1][3])));
        // finite: key 0 is in the first block of every query
        const float m_new = fmaxf(m_i, groups_max(mx));
        const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);   // v_exp_f32 (2^-126 and below flush to 0)
        m_i = m_new;
        l_part *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) O[n] *= alpha;
        half8 ph, pl;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = __builtin_amdgcn_exp2f(sT[nb][r] - m_new);
            l_part += pv;
            const _Float16 hi = (_Float16)pv;
            ph[4 * nb + r] = hi;
            pl[4 * nb + r] = (_Float16)(pv - (float)hi);
          }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const half8 vop = *reinterpret_cast<const half8*>(&Vt[buf][16 * n + (lane & 15)][8 * grp]);
          O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, ph, O[n], 0, 0, 0);
          O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pl, O[n], 0, 0, 0);
          if constexpr (KV32) {
            const half8 vlo = *reinterpret_cast<const half8*>(&Vl[buf][16 * n + (lane & 15)][8 * grp]);
            O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, ph, O[n], 0, 0, 0);
          }
        }
      }
      // the other buffer was last read before the previous barrier
      stage(buf ^ 1, kv);
      __syncthreads();
      load_blk(kb + 2 * kFaK, kv);           // rows clamp to the prompt: always in bounds
    }
    // O^T / l -> out[q][h][dims 16 n + 4 grp .. + 3] (fp16, 8 bytes per lane and n)
    const float inv = 1.0f / groups_sum(l_part);
    if (q < S) {
      uint16_t* orow = out + ((size_t)q * nq + h) * kHD + 4 * grp;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint32_t lo = (uint32_t)f2h(O[n][0] * inv) | ((uint32_t)f2h(O[n][1] * inv) << 16);
        const uint32_t hi = (uint32_t)f2h(O[n][2] * inv) | ((uint32_t)f2h(O[n][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * n) = make_uint2(lo, hi);
      }
    }
  }
}

struct PfDims { int L, H, I, nq, nkv, V, S, cap, nqkv; };

struct PfLayout { size_t h, x, act, qkv, qr, o, gf, lm, total; };


PfLayout pf_layout(const PfDims& d) {
  PfLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes, 256); return o; };
  const size_t S = d.S;
  // the argmax keys first: their offset does not depend on S, so a workspace that served a longer
  // prompt (whose activations sit further on) still holds cleared keys here for a shorter one
  l.lm = take(lm_workspace_bytes(1, d.V, d.H));
  l.h = take(S * d.H * 4);
  l.x = take(S * d.H * 2);
  l.act = take(S * d.I * 2);
  l.qkv = take(S * d.nqkv * 4);
  l.qr = take(S * d.nq * kHD * 4);
  l.o = take(S * d.nq * kHD * 2);
  l.gf = take((size_t)d.H * 4);
  l.total = off;
  return l;
}

PfDims pf_dims(const vv_model* m, int S, int cap) {
  PfDims d;
  d.L = m->n_layers; d.H = m->hidden; d.I = m->inter; d.nq = m->n_q; d.nkv = m->n_kv; d.V = m->vocab;
  d.S = S; d.cap = cap;
  d.nqkv = (m->n_q + 2 * m->n_kv) * kHD;
  return d;
}

// TG token groups of 16 and NW tiles (one per wave) per workgroup
template <int EPI, int TG, int NW>
hipError_t pf_gemm_launch(const PfGemm& p, hipStream_t st) {
  const int ntg = (int)cdiv(p.ntiles, NW);
  const dim3 grid((unsigned)(8 * cdiv(ntg, 8) * cdiv(p.S, 16 * TG))), block(64 * NW);
  hipLaunchKernelGGL((k_pf_gemm<EPI, TG, NW>), grid, block, 0, st, p);
  return hipGetLastError();
}
template <int EPI>
hipError_t pf_gemm(const PfGemm& p, hipStream_t st) {
  return pf_gemm_launch<EPI, kPfTG, kPfNW>(p, st);
}

}  // namespace
}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_prefill_workspace(const vv_model* m, int S, int cap) {
  if (!m || S < 1 || cap < S || m->hidden < 64 || m->inter < 64 || m->n_kv < 1 || m->n_q < 1 || m->n_q % m->n_kv)
    return 0;
  return pf_layout(pf_dims(m, S, cap)).total;
}

int vv_prefill(const vv_model* m, const uint16_t* input_embeds, int S, void* k_cache, void* v_cache, int cap,
               int kv_dtype, float* logits, int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  VV_REQUIRE(m && input_embeds && token, VV_ERR_NULL, "vv_prefill: model, input_embeds or token is NULL");
  VV_REQUIRE(m->head_dim == kHD, VV_ERR_SHAPE, "vv_prefill: head_dim %d != 128", m->head_dim);
  VV_REQUIRE(m->hidden >= 64 && m->hidden % 64 == 0 && m->hidden <= 4096, VV_ERR_SHAPE,
             "vv_prefill: hidden %d must be a multiple of 64 in [64, 4096]", m->hidden);
  VV_REQUIRE(m->inter >= 64 && m->inter % 64 == 0, VV_ERR_SHAPE, "vv_prefill: inter %d must be a multiple of 64",
             m->inter);
  VV_REQUIRE(m->n_q >= 1 && m->n_kv >= 1 && m->n_q % m->n_kv == 0 && m->n_q / m->n_kv <= 8, VV_ERR_SHAPE,
             "vv_prefill: n_q %% n_kv must be 0 with n_q/n_kv <= 8");
  VV_REQUIRE(m->n_layers >= 0 && m->n_layers <= 4096 && (m->n_layers == 0 || m->layers), VV_ERR_RANGE,
             "vv_prefill: bad layer list");
  VV_REQUIRE(m->gf && m->lm_head && m->vocab >= 1, VV_ERR_NULL, "vv_prefill: gf or lm_head is NULL");
  VV_REQUIRE(lm_table_fits(m->vocab, m->hidden), VV_ERR_RANGE, "vv_prefill: the %d x %d lm_head exceeds %lld bytes",
             m->vocab, m->hidden, (long long)kLmMaxTableBytes);
  VV_REQUIRE(S >= 1 && cap >= S && cap <= 131072, VV_ERR_RANGE, "vv_prefill: need 1 <= S <= cap <= 131072");
  VV_REQUIRE(kv_dtype == 0 || kv_dtype == VV_F16 || kv_dtype == VV_F32, VV_ERR_DTYPE,
             "vv_prefill: kv_dtype %d is not VV_F16 or VV_F32", kv_dtype);
  VV_REQUIRE(m->n_layers == 0 || (k_cache && v_cache), VV_ERR_NULL, "vv_prefill: KV cache is NULL");
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(input_embeds) | reinterpret_cast<uintptr_t>(k_cache) |
               reinterpret_cast<uintptr_t>(v_cache)) & 15) == 0,
             VV_ERR_RANGE, "vv_prefill: input_embeds and the caches must be 16-byte aligned");
  for (int l = 0; l < m->n_layers; ++l) {
    const vv_layer& y = m->layers[l];
    VV_REQUIRE(y.qkv_q && y.qkv_s && y.o_q && y.o_s && y.gu_q && y.gu_s && y.down_q && y.down_s && y.g1 && y.g2,
               VV_ERR_NULL, "vv_prefill: layer %d has a NULL weight pointer", l);
  }
  const PfDims d = pf_dims(m, S, cap);
  const PfLayout lay = pf_layout(d);
  VV_REQUIRE(ws && ws_bytes >= lay.total, VV_ERR_WORKSPACE, "vv_prefill: workspace needs %zu bytes", lay.total);
  VV_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255) == 0, VV_ERR_RANGE, "vv_prefill: workspace must be 256-byte aligned");

  hipStream_t st = as_stream(stream);
  char* w = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(w + lay.h);
  uint16_t* x = reinterpret_cast<uint16_t*>(w + lay.x);
  uint16_t* act = reinterpret_cast<uint16_t*>(w + lay.act);
  float* qkv = reinterpret_cast<float*>(w + lay.qkv);
  float* qr = reinterpret_cast<float*>(w + lay.qr);
  uint16_t* o = reinterpret_cast<uint16_t*>(w + lay.o);
  float* gf = reinterpret_cast<float*>(w + lay.gf);
  const bool kv32 = kv_dtype == VV_F32;
  const size_t layer_kv_bytes = (size_t)d.nkv * cap * kHD * (kv32 ? 4 : 2);

  if (d.L == 0) {
    hipLaunchKernelGGL(k_pf_norm, dim3(1), dim3(256), 0, st, input_embeds, h, S - 1, d.H, m->gf, m->eps,
                       (uint16_t*)nullptr, gf);
    VV_HIP(hipGetLastError());
  }
  for (int l = 0; l < d.L; ++l) {
    const vv_layer& y = m->layers[l];
    // RMSNorm_1 (the first layer also takes the embeddings into the residual stream)
    hipLaunchKernelGGL(k_pf_norm, dim3(S), dim3(256), 0, st, l == 0 ? input_embeds : nullptr, h, 0, d.H, y.g1,
                       m->eps, x, (float*)nullptr);
    VV_HIP(hipGetLastError());
    {  // q|k|v (+bias)
      PfGemm p{};
      p.q = y.qkv_q; p.s = y.qkv_s; p.x = x; p.S = S; p.K = d.H; p.N = d.nqkv;
      p.ntiles = (int)cdiv(d.nqkv, kTileRows);
      p.bias = y.qkv_bias; p.y = qkv; p.ldy = d.nqkv;
      VV_HIP(pf_gemm<EPI_STORE>(p, st));
    }
    void* kc = static_cast<char*>(k_cache) + (size_t)l * layer_kv_bytes;
    void* vc = static_cast<char*>(v_cache) + (size_t)l * layer_kv_bytes;
    hipLaunchKernelGGL(k_pf_rope_kv, dim3(S), dim3(256), 0, st, qkv, d.nq, d.nkv, cap, (double)m->rope_theta, qr,
                       kc, vc, (int)kv32);
    VV_HIP(hipGetLastError());
    {  // causal attention on the matrix cores: token t attends to 0..t
      const dim3 grid((unsigned)cdiv(cdiv(S, kFaQ), 2), d.nq);
      const float sc = (float)(1.4426950408889634 / std::sqrt((double)kHD));
      if (kv32) hipLaunchKernelGGL(k_pf_flash<true>, grid, dim3(256), 0, st, qr, kc, vc, S, d.nq, d.nkv, cap, sc, o);
      else hipLaunchKernelGGL(k_pf_flash<false>, grid, dim3(256), 0, st, qr, kc, vc, S, d.nq, d.nkv, cap, sc, o);
      VV_HIP(hipGetLastError());
    }
    {  // o (+residual)
      PfGemm p{};
      p.q = y.o_q; p.s = y.o_s; p.x = o; p.S = S; p.K = d.nq * kHD; p.N = d.H;
      p.ntiles = d.H / kTileRows;
      p.h = h;
      VV_HIP(pf_gemm<EPI_RESID>(p, st));
    }
    hipLaunchKernelGGL(k_pf_norm, dim3(S), dim3(256), 0, st, (const uint16_t*)nullptr, h, 0, d.H, y.g2, m->eps, x,
                       (float*)nullptr);
    VV_HIP(hipGetLastError());
    {  // gate/up (SiLU * up)
      PfGemm p{};
      p.q = y.gu_q; p.s = y.gu_s; p.x = x; p.S = S; p.K = d.H; p.N = d.I;
      p.ntiles = 2 * d.I / kTileRows;
      p.act = act;
      VV_HIP(pf_gemm<EPI_SILU>(p, st));
    }
    {  // down (+residual)
      PfGemm p{};
      p.q = y.down_q; p.s = y.down_s; p.x = act; p.S = S; p.K = d.I; p.N = d.H;
      p.ntiles = d.H / kTileRows;
      p.h = h;
      VV_HIP(pf_gemm<EPI_RESID>(p, st));
    }
  }
  if (d.L > 0) {  // final RMSNorm of the last row, in fp32
    hipLaunchKernelGGL(k_pf_norm, dim3(1), dim3(256), 0, st, (const uint16_t*)nullptr, h, S - 1, d.H, m->gf, m->eps,
                       (uint16_t*)nullptr, gf);
    VV_HIP(hipGetLastError());
  }
  LmParams lp{};
  lp.W = m->lm_head; lp.V = d.V; lp.H = d.H; lp.B = 1;
  lp.x = gf; lp.x_f16 = 0;
  lp.logits = logits; lp.token = token;
  lm_plan(lp);
  lm_set_workspace(lp, w + lay.lm);
  VV_HIP(lm_launch(lp, st));
  return VV_OK;
}

}  // extern "C"
