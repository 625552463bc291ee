// Internal declarations shared by the HIP sources of libvv (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/vv.h"

namespace vv {

// ---------------------------------------------------------------------------------------------
// host-side error reporting
// ---------------------------------------------------------------------------------------------
int fail(int status, const char* fmt, ...);           // records a message, returns status
int hip_fail(hipError_t e, const char* what);          // VV_ERR_HIP with the HIP error string
void clear_error();

#define VV_REQUIRE(cond, status, ...) \
  do { if (!(cond)) return ::vv::fail((status), __VA_ARGS__); } while (0)
#define VV_HIP(call) \
  do { hipError_t e_ = (call); if (e_ != hipSuccess) return ::vv::hip_fail(e_, #call); } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kBlock = 32;       // quantisation block (elements)
constexpr int kTileRows = 64;    // rows per tile of the tiled layout (= lanes of a wave)
constexpr int kWave = 64;
constexpr int kNumXcd = 8;       // MI355X: 8 XCDs, workgroups are dealt round-robin

// ---------------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------------
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Maps a workgroup id so that consecutive logical ids land on the same XCD (workgroups are
// dispatched round-robin over the XCDs).  Requires gridDim.x % kNumXcd == 0.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t wg, uint32_t nwg) {
  const uint32_t per = nwg / kNumXcd;
  return (wg % kNumXcd) * per + wg / kNumXcd;
}

__device__ __forceinline__ uint32_t wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}
__device__ __forceinline__ uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Cross-lane reductions with DPP (VALU-latency data movement, no LDS round trip).  Every lane
// of the wave must be active.  The reduction trees are fixed, so results are reproducible.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over each group of 4 lanes (every lane gets its group's sum)
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  return v;
}
// sum / max over each row of 16 lanes (every lane gets its row's result)
__device__ __forceinline__ float row16_sum(float v) {
  v = quad_sum(v);
  v += dpp_f<0x141>(v);  // row_half_mirror: pairs the two quads of each half-row
  v += dpp_f<0x140>(v);  // row_mirror: pairs the two half-rows
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
// lane-wise sum over the 4 rows of the wave (every lane l gets sum_r v[16r + l%16]) as
// (r0 + r1) + (r2 + r3) in every lane (the two partial sums commute), by two lane shuffles.  (A
// v_permlane16_swap with the same value in both operands would do it without LDS, but the
// compiler has been seen to take its two results for one.)
__device__ __forceinline__ float rows_lanewise_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}
// sum / max over the whole wave (uniform result)
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
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

// Monotone key for a float: larger float -> larger key; NaN maps below every number.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN never wins
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------------------------
// Cross-workgroup hand-off inside one kernel.  The 8 XCDs have separate L2 caches, and an
// agent-scope fence writes back and invalidates the whole L2.  Data published to another
// workgroup therefore goes through agent-scope atomic stores and loads (coherent by themselves:
// they are not served from a stale line of another XCD's L2), and the publisher waits for its
// stores to complete before the arrival counter is bumped.  No fence touches the L2.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void publish_f32(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float collect_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint64_t collect_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A first, cached read of a tagged word.  collect_u64 is the same 64-bit load with the agent-scope
// bit, which makes it skip this XCD's L2; this one may be served by a stale cached copy, but tag
// and value come from one 64-bit store, so a word that carries the expected tag is the current
// one, and any other sends the reader on to collect_u64.
__device__ __forceinline__ uint64_t peek_u64(const uint64_t* p) { return *p; }
// all of this wave's earlier memory operations have completed (s_waitcnt 0); also a compiler barrier
__device__ __forceinline__ void wait_published() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- split-KV merge of one wave ------------------------------------------------------------------
// Split records of the decode attention: per (sequence, KV head, split) and query head of the group,
// kAttnRec floats = m, l, 2 pad, o[128] (m the split's max score, l = sum e^{s-m}, o = sum e^{s-m} v).
constexpr int kAttnMaxG = 8;                 // query heads per KV head
constexpr int kAttnRec = 132;
// The wave merges splits s0 .. s0 + 63 (those below n) of one query head for dim d of this lane:
// lane s loads split s0 + s's (m, l) and every lane the 64 splits' values of its dim, all at once;
// Mw and Lw come from wave reductions and each split's weight e_s = exp(m_s - Mw) reaches every lane
// by readlane.  Returns Ow = sum_s e_s o_s[d] (splits in order), with Lw = sum_s e_s l_s; a wave with
// no split gets Mw = -inf, Lw = Ow = 0.  rec0: the head's record of split 0; stride: floats from one
// split's record to the next.
__device__ __forceinline__ float merge_wave64(const float* rec0, size_t stride, int s0, int n, int d, float& Mw,
                                              float& Lw) {
  const int lane = threadIdx.x & 63;
  const int ns = min(max(n - s0, 0), 64);
  float v[64];
#pragma unroll
  for (int u = 0; u < 64; ++u) v[u] = rec0[(size_t)min(s0 + u, n - 1) * stride + 4 + d];
  const int sl = min(s0 + lane, n - 1);
  const float ms = rec0[(size_t)sl * stride], ls = rec0[(size_t)sl * stride + 1];
  const bool mine = lane < ns;
  Mw = wave_max(mine ? ms : -INFINITY);
  const float e = mine ? expf(ms - Mw) : 0.f;
  Lw = wave_sum(e * ls);
  float Ow = 0.f;
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    const float eu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), u));
    Ow = fmaf(eu, v[u], Ow);                 // e_u = 0 past the wave's last split
  }
  return Ow;
}
// number of splits that hold positions for sequence b (the step flavour reads pos, else lens)
__device__ __forceinline__ int attn_splits(const int32_t* pos, const int32_t* lens, int b, int cap, int S) {
  int len;
  if (pos) {
    const int P = pos[b];
    len = (P < 0 ? 0 : (P >= cap ? cap - 1 : P)) + 1;
  } else {
    const int l = lens[b];
    len = l < 1 ? 1 : (l > cap ? cap : l);
  }
  return (len + S - 1) / S;
}
// sum_{k < n} p[k * stride] in k order, with the loads issued 16 at a time (a runtime-length
// loop of agent-scope loads would wait for each one before issuing the next)
__device__ __forceinline__ float collect_sum_f32(const float* p, int n, size_t stride) {
  float s = 0.f;
  for (int k0 = 0; k0 < n; k0 += 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = k0 + k < n ? collect_f32(p + (size_t)(k0 + k) * stride) : 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += v[k];
  }
  return s;
}
// arrival counter: returns the previous count (agent scope, performed coherently across XCDs)
__device__ __forceinline__ unsigned arrive(unsigned* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(unsigned* c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------------
// internal launchers used by the decode step (enqueue only; arguments already validated)
// ---------------------------------------------------------------------------------------------
enum EpiKind { EPI_STORE = 0, EPI_RESID = 1, EPI_SILU = 2 };

// Optional timing events of a launch: hipExtLaunchKernel stores the kernel's own start and end
// times in them (the dispatch timestamps, not the time the stream reaches a marker).  An
// operation of several kernels puts `start` on its first launch and `stop` on its last.
struct KEv {
  hipEvent_t start = nullptr, stop = nullptr;
  KEv first() const { return KEv{start, nullptr}; }
  KEv last() const { return KEv{nullptr, stop}; }
};
#define VV_LAUNCH(kern, grid, block, st, ev, ...)                                                     \
  do {                                                                                                \
    const ::vv::KEv vv_ev_ = (ev); /* evaluated once */                                               \
    if (vv_ev_.start || vv_ev_.stop)                                                                  \
      hipExtLaunchKernelGGL(kern, grid, block, 0, st, vv_ev_.start, vv_ev_.stop, 0, __VA_ARGS__);    \
    else                                                                                              \
      hipLaunchKernelGGL(kern, grid, block, 0, st, __VA_ARGS__);                                      \
  } while (0)

struct GemvParams {
  const uint8_t* q;          // tiled nibbles
  const uint16_t* s;         // tiled scales
  const void* x;             // [M][K]: fp32 (x_f32, the VALU kernel splits it into fp16 hi + lo) or fp16
  int x_f32;
  int M, N, K;               // N valid output rows (EPI_SILU: rows of gate = rows of up)
  int ntiles;                // tiles in the matrix
  float* part;               // workspace partials (matrix-core kernel)
  unsigned* cnt;             // workspace counters (matrix-core kernel)
  uint64_t* slots;           // workspace hand-off slots (VALU kernel): (tag << 32) | fp32 bits
  int32_t* status;           // sticky status word set when a bounded wait gives up, or null
  int kb, wpg, wpt, grid;    // decomposition (filled by gemv_plan): waves per workgroup, workgroups per tile
  int epi;
  // EPI_STORE
  const uint16_t* bias;      // fp16 [N] or null
  void* y; int y_f16; int ldy;
  // rstd source (EPI_STORE / EPI_SILU), optional
  const float* rs_parts; int rs_nparts; float rs_inv_n; float eps;
  int rs_mask, has_bias, has_gamma;   // set by gemv_launch (which points absent operands at x)
  // EPI_RESID
  float* h;                  // fp32 [M][N]
  const uint16_t* gamma;     // fp16 [N]
  void* g_out; int g_f32;    // [M][N] gamma * h, fp32 (g_f32) or fp16 (if gamma and g_out)
  float* sumsq_out;          // fp32 [M][ntiles]
  float* trace;              // fp32 [M][N] copy of h or null
  // EPI_SILU
  void* act; int act_f32;    // [M][N] SiLU(gate) * up, fp32 (act_f32) or fp16
  // fused split-KV merge (batch 1, at most 64 splits): the first mrg_blocks workgroups merge the
  // attention records into tagged activation words xtag[k] = (tag << 32) | fp32 bits, which the
  // GEMV workgroups poll instead of reading x; tag = epoch[0] * tag_mul + tag_add (the step's
  // epoch, so that no word needs clearing)
  int mrg_blocks;            // 0: no fused merge
  const float* mrg_part; const int32_t* mrg_pos; int mrg_nsplit, mrg_split, mrg_cap, mrg_nq, mrg_nkv;
  uint64_t* xtag; const uint32_t* epoch; uint32_t tag_mul, tag_add;
};

// batches of at least this many rows run on the matrix cores (fp16 activations); smaller ones on
// the vector ALU (fp32 activations as fp16 hi + lo parts, or fp16)
constexpr int kGemvMfmaMinM = 5;
void gemv_plan(GemvParams& p);                       // fills kb/wpg/wpt/grid
size_t gemv_workspace_bytes(int M, int ntiles, int nb);
void gemv_set_workspace(GemvParams& p, void* ws);    // carves part/cnt from ws
hipError_t gemv_launch(const GemvParams& p, hipStream_t st, KEv ev = {});
hipError_t gemv_mfma_launch(const GemvParams& p, hipStream_t st, KEv ev);   // 5..16 rows (gemv_launch picks it)
// the stand-alone GEMV on the MatMulNBits row-major bytes (no workspace, 1..16 rows)
hipError_t gemv_rowmajor_launch(const uint8_t* q, const uint16_t* s, const uint16_t* bias, const uint16_t* x, int M,
                                int N, int K, void* y, int y_f16, hipStream_t st);

struct AttnParams {
  int B, nq, nkv, cap, split, nsplit;
  // step flavour: q/k/v from the fused projection output (fp32 [B][ldqkv])
  const float* qkv; int ldqkv;
  const int32_t* pos;        // step: new token position; attention over pos+1 positions
  float rope_theta;
  // stand-alone flavour
  const void* q; int q_f16;
  const int32_t* lens;
  void* kc; void* vc;           // [B][nkv][cap][128] fp16 (fp32 with kv_f32), or one
                                // [nkv][cap][128] cache for all B (kv_shared)
  int kv_shared;                // 1: every sequence b reads the same cache (prefill: b = token)
  int kv_f32;                   // 1: the caches hold fp32
  float scale;
  void* out; int out_f16;       // [B][nq][128]
  float* part; float* part2; unsigned* cnt;
  int skip_merge;               // 1: the split records are merged elsewhere (a fused consumer)
};
void attn_plan(AttnParams& p);
size_t attn_workspace_bytes(int B, int nq, int nkv, int nsplit);
void attn_set_workspace(AttnParams& p, void* ws);
hipError_t attn_launch(const AttnParams& p, hipStream_t st);
// step flavour: rope_cs = [B][64][2] (cos, sin) of the new positions
hipError_t attn_launch_with_rope(const AttnParams& p, const float* rope_cs, hipStream_t st, KEv ev = {});

struct LmParams {
  const uint16_t* W; int V, H, B;
  const void* x; int x_f16;
  const float* rs_parts; int rs_nparts; float rs_inv_n; float eps;
  float* logits; int32_t* token;
  uint64_t* keys;            // workspace: one key per (batch row, workgroup)
  int32_t* status;           // sticky status word set when a bounded wait gives up, or null
  uint32_t* epoch;           // decode step counter, advanced by the argmax's last workgroup, or null
  int grid, rows_per_wg;
};
// The row-stream kernel addresses the table with 32-bit byte offsets from one buffer resource, so
// every entry point that runs the lm_head rejects a table larger than this (VV_ERR_RANGE).
constexpr int64_t kLmMaxTableBytes = 0x7fffffff;
bool lm_table_fits(int64_t V, int64_t H);
// the allocation-free lm_head's argmax keys: a file-scope device array of this size (lmhead.hip)
constexpr size_t kLmScratchBytes = 256 * 1024;
int scratch_address(void** out);   // the current device's address of that array
void lm_plan(LmParams& p);
size_t lm_workspace_bytes(int B, int V, int H);
void lm_set_workspace(LmParams& p, void* ws);
hipError_t lm_launch(const LmParams& p, hipStream_t st, KEv ev = {});

hipError_t fill_zero(void* p, size_t bytes, hipStream_t st, KEv ev = {});

// ---- chained launches of the batch-1 step (chain.hip) ------------------------------------------
// One grid runs several stages as segments (consecutive ranges of workgroups, each a multiple of 8
// so that a workgroup's index within its segment keeps its XCD).  Cross-segment data are 64-bit
// tagged words (tag << 32 | fp32 bits); a tag is epoch * tag_mul + add.
constexpr int kChainWaves = 8;        // waves per workgroup
constexpr int kChainMaxSeg = 3;
constexpr int kChainMaxSplits = 128;  // attention splits the merge segment takes
enum ChainSegKind { SEG_PREP = 0, SEG_MERGE, SEG_QKV, SEG_O, SEG_GU, SEG_DOWN };
// the launches of the chained step: [prep | q|k|v], [merge | o], [gate/up | down (| q|k|v)], or
// for wide models [gate/up] and [down (| q|k|v)]; and the layered plan's batch-1
// [down (plain inputs) | q|k|v]
enum ChainLaunch { CH_FIRST = 0, CH_MO, CH_MLP, CH_GU, CH_DQ, CH_LDQ };
struct CSeg {
  int kind, blocks;
  // GEMV segments (batch 1, tiled weights; wpt workgroups of wpg waves per tile)
  const u32x4* q; const u32x4* s;
  int N, K, ntiles, wpt, wpg;
  uint64_t* slots;                               // split-K hand-off slots [tile][wpt - 1][64]
  const uint64_t* xin; uint32_t xin_add;         // tagged inputs [K]
  const uint64_t* ssin; uint32_t ss_add; int ss_n;   // QKV, GU: tagged sum(h^2) per tile (rstd)
  uint32_t hin_add;                              // O, DOWN: tag of the residual they add to
  uint32_t out_add;                              // tag of the words this segment writes
  const uint16_t* bias; int has_bias; float* y;  // QKV: fp16 bias (readable stand-in if absent), fp32 out
  const uint16_t* gamma;                         // O, DOWN: weight of the next RMSNorm
  uint64_t* xgout; uint64_t* ssout;              // O, DOWN: tagged gamma * h [N], sum(h^2) per tile
  float* trace; float* gf; float* sumsq;         // DOWN: optional plain copies (trace, lm_head inputs)
  uint64_t* act;                                 // GU: tagged SiLU(gate) * up [N]
  // DOWN after a kernel boundary (the layered plan's [down | next q|k|v] launch): plain fp32
  // input xp [K] and residual hp [N], updated in place (no tags to wait for)
  const float* xp; float* hp;
};
struct ChainParams {
  int nseg;
  CSeg seg[kChainMaxSeg];
  uint64_t* h;                                   // tagged fp32 residual stream [H]
  int H;
  float eps, inv_h;
  const uint32_t* epoch; uint32_t tag_mul;
  int32_t* status;
  // SEG_PREP: embeddings -> h, g1 * h, sum(h^2) per tile, the RoPE table
  uint32_t prep_add;
  const uint16_t* emb; const uint16_t* g1; uint64_t* xq; uint64_t* ssq; float* trace0;
  const int32_t* pos; int cap; int rope_on; float* rope;
  double inv_freq[64];                           // theta^(-2i/128), i = 0..63 (host fp64)
  // SEG_MERGE: attention split records -> the tagged attention output [nq * 128]
  const float* part; int nsplit, split, nq, nkv;
  uint64_t* xo; uint32_t mrg_add;
};
void chain_gemv_plan(CSeg& g);                  // fills wpt / wpg / blocks from ntiles and K
hipError_t chain_launch(const ChainParams& P, hipStream_t st, KEv ev = {});

}  // namespace vv
