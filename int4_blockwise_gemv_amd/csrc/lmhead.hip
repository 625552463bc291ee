// fp16 lm_head GEMV with a fused greedy argmax.
//
// The lm_head (and the embedding table it is tied to in the 1.5B model) stays fp16, row-major
// [V][H] ("vibevoice-asr-bitnet-onnx" page: lm_head/embeddings stay fp16; embed_tokens.bin is a
// raw fp16 row-major table); decoding is greedy.  Each wave streams whole rows (lane i reads
// 16-byte chunks i, i+64, ... of a row: 1 KiB contiguous per load instruction), keeps its slice
// of the activation in registers, and reduces each row across the wave.  The largest logit is
// tracked as a 64-bit key (order-preserving float bits, then the complemented index, so ties go
// to the smallest index); each workgroup publishes its best key and the grid's last workgroup
// polls them and picks the winner (the maximum does not depend on the order).
#include <mutex>

#include "vv_internal.h"

namespace vv {
namespace {

constexpr int kRowsPerIter = 2;   // rows per pass of the two-buffer row stream
constexpr int kLmMfmaMinB = 3;          // batches from 3 rows take the matrix cores
constexpr int kMaxChunksPerLane = 8;   // H <= 8 * 64 * 8 = 4096

// key = order-preserving float bits : filled flag : (2^31 - 1 - index).  The flag (set in every
// published key, cleared slots are 0) does not change the order among published keys.
constexpr uint64_t kKeyFilled = 1ull << 31;
constexpr uint32_t kSpinLimit = 1u << 22;
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  return ((uint64_t)float_order_key(v) << 32) | kKeyFilled | (uint64_t)(0x7fffffffu - idx);
}

// Argmax over the workgroups' keys.  Every workgroup stores its keys (with the filled flag) and
// is done: no store waits and no arrival counter, so no workgroup holds its slot for a memory
// round trip after its rows (an arrival atomic per workgroup, queued behind the weight stream,
// costs ~12 us over the lm_head's ~1000 workgroups).  The last workgroup of the grid, dispatched
// after all others, polls the keys of each batch row until every one is filled, takes the
// maximum (independent of order), clears the slots for the next launch and writes the token.
// The wait is bounded: one that gives up sets the status word (when there is one) and writes
// token -1.  All threads of the workgroup call this after publishing their keys.
__device__ void argmax_finish(const LmParams& p, int B) {
  if (blockIdx.x != gridDim.x - 1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = (int)gridDim.x;
  for (int b = w; b < B; b += 4) {
    uint64_t* keys = p.keys + (size_t)b * n;
    uint64_t k = 0;
    bool gave_up = false;
    for (int i0 = 0; i0 < n; i0 += 64 * 16) {
      uint64_t v[16];
      for (uint32_t it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          v[u] = collect_u64(keys + min(i0 + lane + 64 * u, n - 1));
          ok = ok && (v[u] & kKeyFilled) != 0;
        }
        if (__all(ok)) break;
        if (it >= kSpinLimit) { gave_up = true; break; }
        __builtin_amdgcn_s_sleep(2);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        k = v[u] > k ? v[u] : k;
        if (i0 + lane + 64 * u < n) publish_u64(keys + i0 + lane + 64 * u, 0);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t x = __shfl_xor(k, o, 64);
      k = x > k ? x : k;
    }
    if (lane == 0) {
      if (gave_up && p.status) __hip_atomic_store(p.status, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      p.token[b] = gave_up ? -1 : (int32_t)(0x7fffffffu - (uint32_t)(k & 0x7fffffffu));
    }
  }
  // the decode step ends here: advance its counter, so the next step's tagged words get new tags
  // (nothing in this launch reads it; the next step's kernels run after this one)
  if (p.epoch && tid == 0) p.epoch[0] += 1;
}

template <int CPL, int BT>
__global__ __launch_bounds__(256) void k_lmhead(LmParams p, const u32x4* __restrict__ W) {
  __shared__ uint64_t best_w[4][BT];
  const int H = p.H, V = p.V;
  const int nch = H / 8;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int wg = blockIdx.x;
  const int r0 = wg * p.rows_per_wg;
  const int r1 = min(V, r0 + p.rows_per_wg);
  const int rpw = (p.rows_per_wg + 3) / 4;
  const int wr0 = r0 + w * rpw;
  const int wr1 = min(r1, wr0 + rpw);
  const int table_bytes = (int)min<int64_t>((int64_t)V * H * 2, 0x7fffffff);

  for (int bb = 0; bb < p.B; bb += BT) {
    const int nbt = min(BT, p.B - bb);
    // activation slice in registers, chunk c = lane + 64 j holding x[8c .. 8c+7] scaled by rstd
    // (so that it stays in fp16 range) and split into fp16 pairs x = hi + lo (~22 bits):
    // v_dot2_f32_f16 then multiplies both parts by the fp16 weights exactly, accumulating in fp32
    uint32_t xh[BT][CPL][4], xl[BT][CPL][4];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      float rs = 1.f;
      if (t < nbt && p.rs_parts) {  // lane l adds part l (at most 64 parts), fixed reduction tree
        const float v = lane < p.rs_nparts ? p.rs_parts[(size_t)(bb + t) * p.rs_nparts + lane] : 0.f;
        rs = 1.0f / sqrtf(wave_sum(v) * p.rs_inv_n + p.eps);
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        float xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = 0.f;
        if (t < nbt && c < nch) {
          if (p.x_f16) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.x) + (size_t)(bb + t) * H + 8 * c);
            const uint32_t d4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              xv[2 * i] = (float)as_h2(d4[i]).x;
              xv[2 * i + 1] = (float)as_h2(d4[i]).y;
            }
          } else {
            const float* xs = reinterpret_cast<const float*>(p.x) + (size_t)(bb + t) * H + 8 * c;
            const float4 a = *reinterpret_cast<const float4*>(xs);
            const float4 b = *reinterpret_cast<const float4*>(xs + 4);
            xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
            xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = xv[2 * i] * rs, x1 = xv[2 * i + 1] * rs;
          const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
          const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
          xh[t][j][i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          xl[t][j][i] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
      }
    }
    uint64_t best[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) best[t] = 0;

    // rows stream through two register buffers: the loads of the next row are in flight while
    // the current one is reduced.  No load sits behind a branch: a row past the wave's range
    // re-reads its last row, and the loads are buffer loads over the whole table, so a chunk past
    // H reads the next row's bytes (or zeros past the end of the table) against x = 0.
    if (wr0 < wr1) {
      const int row_bytes = H * 2;
      auto load_row = [&](u32x4 (&buf)[CPL], int row) {
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<u32x4*>(W), (short)0, __builtin_amdgcn_readfirstlane(table_bytes), 0x00020000);
        const int off = min(row, wr1 - 1) * row_bytes + lane * 16;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          buf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, j * 1024, 2));
      };
      // chunks past H hold the next row's weights: they are zeroed, not multiplied by x = 0, so a
      // non-finite weight of one row never reaches another row's sum (0 * NaN would).  Only the
      // last chunk of a lane can lie past H.
      const bool tail_live = lane + 64 * (CPL - 1) < nch;
      auto reduce_row = [&](const u32x4 (&buf)[CPL], int row) {
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          if (t >= nbt) continue;
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            const bool live = j + 1 < CPL || tail_live;
            const uint32_t d4[4] = {live ? buf[j].x : 0u, live ? buf[j].y : 0u, live ? buf[j].z : 0u,
                                    live ? buf[j].w : 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              a = __builtin_amdgcn_fdot2(as_h2(d4[i]), as_h2(xh[t][j][i]), a, false);
              a = __builtin_amdgcn_fdot2(as_h2(d4[i]), as_h2(xl[t][j][i]), a, false);
            }
          }
          a = wave_sum(a);
          if (row < wr1) {
            if (p.logits && lane == 0) p.logits[(size_t)(bb + t) * V + row] = a;
            const uint64_t k = make_key(a, (uint32_t)row);
            best[t] = k > best[t] ? k : best[t];
          }
        }
      };
      u32x4 wa[CPL], wb[CPL];
      load_row(wa, wr0);
      for (int r = wr0; r < wr1; r += 2) {
        load_row(wb, r + 1);
        reduce_row(wa, r);
        load_row(wa, r + 2);
        reduce_row(wb, r + 1);
      }
    }
#pragma unroll
    for (int t = 0; t < BT; ++t)
      if (lane == 0) best_w[w][t] = best[t];
    __syncthreads();
    if (tid < nbt) {
      uint64_t k = best_w[0][tid];
      for (int i = 1; i < 4; ++i) k = best_w[i][tid] > k ? best_w[i][tid] : k;
      publish_u64(&p.keys[(size_t)(bb + tid) * gridDim.x + wg], k | kKeyFilled);
    }
    __syncthreads();
  }
  argmax_finish(p, p.B);
}

// ---- batches of kLmMfmaMinB..16 rows: fp16 matrix cores ----------------------------------------
// A operand: 16 vocabulary rows x 32 k straight from the row-major table; B: the activation as two
// fp16 parts (x = hi + lo, ~22 bits), so the input keeps fp32 precision and each product is
// exact.  The k order inside a 128-element sub-chunk is permuted the same way on both operands
// (lane group s takes 32 contiguous k, one MFMA step per 8), which lets each lane load 64
// contiguous bytes of its row.  A workgroup of 4 waves owns 64 * rgw consecutive rows (wave w
// takes row groups w, w + 4, ...) and walks H in chunks of kLmKC, staging the chunk of all 16
// activation rows in LDS.
typedef _Float16 lm_half8 __attribute__((ext_vector_type(8)));
typedef float lm_f32x4 __attribute__((ext_vector_type(4)));
constexpr int kLmKC = 256;        // k per staged chunk
constexpr int kLmMaxRGW = 8;      // row groups (16 rows) per wave at most
constexpr int kLmXS = kLmKC + 8;  // padded LDS row

__global__ __launch_bounds__(256) void k_lmhead_mfma(LmParams p, const u32x4* __restrict__ W) {
  __shared__ __align__(16) uint16_t xh[16][kLmXS], xl[16][kLmXS];
  __shared__ float rs_s[16];
  __shared__ uint64_t best_w[4][16];
  const int H = p.H, V = p.V, B = p.B;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wg = blockIdx.x;
  const int rgw = p.rows_per_wg / 64;                // row groups per wave
  const int rg0 = wg * 4 * rgw;                      // first row group of the workgroup
  const int li = lane & 15, ls = lane >> 4;

  // rstd of each batch row (wave 0; lane n adds part n)
  if (w == 0) {
    for (int j = 0; j < 16; ++j) {
      float r = 1.f;
      if (p.rs_parts && j < B) {
        const float v = lane < p.rs_nparts ? p.rs_parts[(size_t)j * p.rs_nparts + lane] : 0.f;
        r = 1.0f / sqrtf(wave_sum(v) * p.rs_inv_n + p.eps);
      }
      if (lane == 0) rs_s[j] = r;
    }
  }

  lm_f32x4 acc[kLmMaxRGW];
#pragma unroll
  for (int j = 0; j < kLmMaxRGW; ++j) acc[j] = lm_f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < H; c0 += kLmKC) {
    __syncthreads();   // the previous chunk is consumed
    {  // thread t: row t / 16, elements 16 (t % 16) .. + 15 of the chunk
      const int m = tid >> 4, k = (tid & 15) * 16;
      const int mc = min(m, B - 1);
      float v[16];
      if (p.x_f16) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(p.x) + (size_t)mc * H + c0 + k;
        const u32x4 a = *reinterpret_cast<const u32x4*>(src), b = *reinterpret_cast<const u32x4*>(src + 8);
        const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) { v[2 * i] = (float)as_h2(d[i]).x; v[2 * i + 1] = (float)as_h2(d[i]).y; }
      } else {
        const float* src = reinterpret_cast<const float*>(p.x) + (size_t)mc * H + c0 + k;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 f = *reinterpret_cast<const float4*>(src + 4 * i);
          v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
      }
      uint16_t hi[16], lo[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = m < B ? v[i] : 0.f;
        const _Float16 h = (_Float16)x;
        hi[i] = __builtin_bit_cast(uint16_t, h);
        lo[i] = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)h));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4 a, b;
        a.x = hi[8 * i] | ((uint32_t)hi[8 * i + 1] << 16); a.y = hi[8 * i + 2] | ((uint32_t)hi[8 * i + 3] << 16);
        a.z = hi[8 * i + 4] | ((uint32_t)hi[8 * i + 5] << 16); a.w = hi[8 * i + 6] | ((uint32_t)hi[8 * i + 7] << 16);
        b.x = lo[8 * i] | ((uint32_t)lo[8 * i + 1] << 16); b.y = lo[8 * i + 2] | ((uint32_t)lo[8 * i + 3] << 16);
        b.z = lo[8 * i + 4] | ((uint32_t)lo[8 * i + 5] << 16); b.w = lo[8 * i + 6] | ((uint32_t)lo[8 * i + 7] << 16);
        *reinterpret_cast<u32x4*>(&xh[m][k + 8 * i]) = a;
        *reinterpret_cast<u32x4*>(&xl[m][k + 8 * i]) = b;
      }
    }
    __syncthreads();
    // B operands of this lane for the chunk: batch row li, k = 128 u + 32 ls + 8 e
    for (int j = 0; j < rgw; ++j) {
      const int row = min((rg0 + w + 4 * j) * 16 + li, V - 1);
      const u32x4* wr = W + ((size_t)row * H + c0) / 8 + 4 * ls;
      u32x4 a[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * u + e] = __builtin_nontemporal_load(wr + 16 * u + e);
      lm_f32x4 c = acc[0];
#pragma unroll
      for (int jj = 0; jj < kLmMaxRGW; ++jj) if (jj == j) c = acc[jj];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 128 * u + 32 * ls + 8 * e;
          const lm_half8 bh = __builtin_bit_cast(lm_half8, *reinterpret_cast<const u32x4*>(&xh[li][k]));
          const lm_half8 bl = __builtin_bit_cast(lm_half8, *reinterpret_cast<const u32x4*>(&xl[li][k]));
          const lm_half8 av = __builtin_bit_cast(lm_half8, a[4 * u + e]);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, c, 0, 0, 0);
        }
#pragma unroll
      for (int jj = 0; jj < kLmMaxRGW; ++jj) if (jj == j) acc[jj] = c;
    }
  }

  // lane l: rows 16 g + 4 (l / 16) + r of its row groups g, batch row l % 16
  const int b = li;
  const float rsb = rs_s[b];
  uint64_t best = 0;
#pragma unroll
  for (int j = 0; j < kLmMaxRGW; ++j) {
    if (j >= rgw) break;
    const int rbase = (rg0 + w + 4 * j) * 16 + 4 * ls;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rbase + r;
      const float v = acc[j][r] * rsb;
      if (row < V && b < B) {
        if (p.logits) p.logits[(size_t)b * V + row] = v;
        const uint64_t k = make_key(v, (uint32_t)row);
        best = k > best ? k : best;
      }
    }
  }
  // lanes b, b + 16, b + 32, b + 48 hold batch row b
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const uint64_t v = __shfl_xor(best, o, 64);
    best = v > best ? v : best;
  }
  if (lane < 16) best_w[w][lane] = best;
  __syncthreads();
  if (tid < B) {
    uint64_t k = best_w[0][tid];
    for (int i = 1; i < 4; ++i) k = best_w[i][tid] > k ? best_w[i][tid] : k;
    publish_u64(&p.keys[(size_t)tid * gridDim.x + wg], k | kKeyFilled);
  }
  argmax_finish(p, B);
}

bool lm_use_mfma(const LmParams& p) { return p.B >= kLmMfmaMinB && p.H % kLmKC == 0; }

}  // namespace

void lm_plan(LmParams& p) {
  if (lm_use_mfma(p)) {   // 64 rows per row-group layer; about 512 workgroups
    const int64_t ngroups = cdiv(p.V, 16);
    const int rgw = (int)std::min<int64_t>(kLmMaxRGW, std::max<int64_t>(1, cdiv(ngroups, 4 * 512)));
    p.rows_per_wg = 64 * rgw;
    p.grid = (int)cdiv(p.V, p.rows_per_wg);
    return;
  }
  int grid = (int)cdiv(p.V, 64);            // at least 16 rows per wave
  grid = grid > 1024 ? 1024 : (grid < 1 ? 1 : grid);
  p.rows_per_wg = (int)cdiv(p.V, grid);
  p.rows_per_wg = (int)cdiv(p.rows_per_wg, 4 * kRowsPerIter) * 4 * kRowsPerIter;
  p.grid = (int)cdiv(p.V, p.rows_per_wg);
}

// Workspace: one key per (batch row, workgroup).
bool lm_table_fits(int64_t V, int64_t H) { return V * H * 2 <= kLmMaxTableBytes; }

size_t lm_workspace_bytes(int B, int V, int H) {
  LmParams p{};
  p.B = B; p.V = V; p.H = H;
  lm_plan(p);
  return align_up((size_t)B * p.grid * sizeof(uint64_t), 256);
}

void lm_set_workspace(LmParams& p, void* ws) { p.keys = reinterpret_cast<uint64_t*>(ws); }

hipError_t lm_launch(const LmParams& p, hipStream_t st, KEv ev) {
  const int cpl = (int)cdiv(p.H / 8, 64);
  const u32x4* W = reinterpret_cast<const u32x4*>(p.W);
  if (lm_use_mfma(p)) {
    VV_LAUNCH(k_lmhead_mfma, dim3(p.grid), dim3(256), st, ev, p, W);
    return hipGetLastError();
  }
#define VV_LM_CASE(C)                                                                   \
  case C:                                                                               \
    if (p.B == 1) VV_LAUNCH((k_lmhead<C, 1>), dim3(p.grid), dim3(256), st, ev, p, W);       \
    else VV_LAUNCH((k_lmhead<C, 2>), dim3(p.grid), dim3(256), st, ev, p, W);                \
    break;
  switch (cpl) {
    VV_LM_CASE(1) VV_LM_CASE(2) VV_LM_CASE(3) VV_LM_CASE(4) VV_LM_CASE(5) VV_LM_CASE(6) VV_LM_CASE(7)
    VV_LM_CASE(8)
    default: break;
  }
#undef VV_LM_CASE
  return hipGetLastError();
}

}  // namespace vv

// ---- the allocation-free entry point's scratch ----------------------------------------------
// The argmax keys of vv_lm_head_argmax_noalloc live in this file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, once per device, and is what the kernels receive.
static __device__ __align__(256) uint64_t scratch[vv::kLmScratchBytes / sizeof(uint64_t)];

namespace vv {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int scratch_address(void** out) {
  int dev = -1;
  VV_HIP(hipGetDevice(&dev));
  VV_REQUIRE(dev >= 0 && dev < kMaxDevices, VV_ERR_RANGE, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    VV_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    VV_REQUIRE(p != nullptr, VV_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VV_OK;
}

int lm_validate(const uint16_t* W, const void* x, int x_dtype, int B, int V, int H, const int32_t* token,
                const char* fn) {
  VV_REQUIRE(W && x && token, VV_ERR_NULL, "%s: NULL pointer", fn);
  VV_REQUIRE(B >= 1 && B <= 16, VV_ERR_RANGE, "%s: B = %d not in 1..16", fn, B);
  VV_REQUIRE(V >= 1, VV_ERR_RANGE, "%s: V = %d < 1", fn, V);
  VV_REQUIRE(H >= 8 && H % 8 == 0 && H <= 8 * 64 * kMaxChunksPerLane, VV_ERR_SHAPE,
             "%s: H = %d must be a multiple of 8 in [8, 4096]", fn, H);
  VV_REQUIRE(lm_table_fits(V, H), VV_ERR_RANGE, "%s: a %d x %d fp16 table exceeds %lld bytes", fn, V, H,
             (long long)kLmMaxTableBytes);
  VV_REQUIRE(x_dtype == VV_F16 || x_dtype == VV_F32, VV_ERR_DTYPE, "%s: unknown x dtype", fn);
  VV_REQUIRE(((reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(x)) & 15) == 0, VV_ERR_RANGE,
             "%s: W and x must be 16-byte aligned", fn);
  return VV_OK;
}
}  // namespace vv

using namespace vv;

extern "C" {

size_t vv_lm_head_argmax_workspace(int B, int V, int H) {
  if (B < 1 || V < 1 || H < 8) return 0;
  return lm_workspace_bytes(B, V, H);
}

int vv_lm_head_argmax(const uint16_t* W, const void* x, int x_dtype, int B, int V, int H, float* logits,
                      int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = lm_validate(W, x, x_dtype, B, V, H, token, "vv_lm_head_argmax");
  if (rc) return rc;
  const size_t need = vv_lm_head_argmax_workspace(B, V, H);
  VV_REQUIRE(ws && ws_bytes >= need, VV_ERR_WORKSPACE, "vv_lm_head_argmax: workspace needs %zu bytes", need);
  LmParams p{};
  p.W = W; p.V = V; p.H = H; p.B = B;
  p.x = x; p.x_f16 = x_dtype == VV_F16;
  p.logits = logits; p.token = token;
  lm_plan(p);
  lm_set_workspace(p, ws);
  VV_HIP(lm_launch(p, as_stream(stream)));
  return VV_OK;
}

int vv_lm_head_argmax_noalloc(const uint16_t* W, const void* x, int x_dtype, int B, int V, int H, float* logits,
                              int32_t* token, void* stream) {
  clear_error();
  int rc = lm_validate(W, x, x_dtype, B, V, H, token, "vv_lm_head_argmax_noalloc");
  if (rc) return rc;
  const size_t need = vv_lm_head_argmax_workspace(B, V, H);
  VV_REQUIRE(need <= kLmScratchBytes, VV_ERR_RANGE,
             "vv_lm_head_argmax_noalloc: %d rows x %d vocabulary rows need %zu bytes of argmax keys, more than "
             "the %zu of its scratch (use vv_lm_head_argmax with a workspace)",
             B, V, need, kLmScratchBytes);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  // the keys this call uses start cleared (a fill kernel, not a memset: capture-safe)
  VV_HIP(fill_zero(ws, need, st));
  LmParams p{};
  p.W = W; p.V = V; p.H = H; p.B = B;
  p.x = x; p.x_f16 = x_dtype == VV_F16;
  p.logits = logits; p.token = token;
  lm_plan(p);
  lm_set_workspace(p, ws);
  VV_HIP(lm_launch(p, st));
  return VV_OK;
}

}  // extern "C"
