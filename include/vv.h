/*
 * vv.h — C ABI of the int4 block-32 decode-step library for MI355X (gfx950).
 *
 * The library implements the single-token decode step of the Qwen2 decoder that the
 * VibeVoice ONNX pages describe:
 *   - int4 block-32 symmetric projections (com.microsoft::MatMulNBits: block 32, zero point 8,
 *     q = w/s + 8, one fp16 scale per block), with the ternary export rule
 *     s = 1/mean(|W|), W' = round(clamp(W*s, -1, 1))/s
 *     ("vibevoice-asr-bitnet-onnx" model page: ternarisation paragraph and MatMulNBits note);
 *   - grouped-query attention over a device-resident fp16 KV cache
 *     (decoder_step graph contract on the same page: past K/V [28,1,kv,P,128] -> present [.., P+1, 128];
 *     GPU-resident KV: "VibeVoice-ASR — ONNX export for Vernacula", Highlights);
 *   - the fp16 lm_head GEMV and a greedy argmax (bitnet-onnx page: lm_head/embeddings stay fp16;
 *     decoding note: greedy decode).
 *
 * Conventions for every call:
 *   - All pointers named "device" are device (HBM) addresses owned by the caller; the library never
 *     allocates, frees or retains device memory, except that a vv_graph keeps raw pointers until
 *     vv_decode_graph_destroy.  fp16 tensors are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call is asynchronous on that
 *     stream; none reads device data on the host or synchronises.
 *   - Every argument is validated before anything is enqueued: a call that returns an error has
 *     launched nothing.  Device faults surface at the caller's next synchronisation.
 *   - Workspaces: calls that take `ws`/`ws_bytes` need a device buffer of at least the size their
 *     *_workspace() query returns, ZERO-FILLED before its first use (vv_workspace_init does this);
 *     every completed call leaves its counters and hand-off slots cleared again (the decode
 *     step also keeps a step counter there, whose tagged words need no clearing), so a workspace
 *     can be reused without re-initialisation by later calls of the same entry point with the same
 *     shape arguments on the same stream (vv_prefill: any prompt length S).  Before a workspace
 *     serves another entry point or other shapes, zero-fill it again.  Two calls that run
 *     concurrently must not share a workspace.
 *   - Return value: VV_OK or a negative vv_status; vv_last_error() gives a thread-local message.
 */
#ifndef VV_H
#define VV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VV_OK = 0,
  VV_ERR_NULL = -1,        /* a required pointer is NULL */
  VV_ERR_SHAPE = -2,       /* a dimension is not supported (e.g. K % 32 != 0, head_dim != 128) */
  VV_ERR_RANGE = -3,       /* a size or index is out of range (e.g. batch < 1, cap too small) */
  VV_ERR_DTYPE = -4,       /* unknown dtype / mode / layout code */
  VV_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the *_workspace() query */
  VV_ERR_UNSUPPORTED = -6, /* valid but not implemented combination */
  VV_ERR_HIP = -7          /* a HIP runtime call failed (message in vv_last_error) */
} vv_status;

/* quantisation modes of vv_pack_int4* */
enum { VV_Q_TERNARY = 0, VV_Q_ABSMAX = 1 };
/* element types */
enum { VV_F16 = 1, VV_F32 = 2 };
/* packed weight layouts */
enum { VV_LAYOUT_ROWMAJOR = 0, VV_LAYOUT_TILED = 1 };

/*
 * Packed weight layouts (N rows = output features, K columns = input features, K % 32 == 0,
 * nb = K/32 blocks per row).  The code of element k of row n is q in 0..15; its value is
 * (q - 8) * scale[n][k/32].
 *
 * VV_LAYOUT_ROWMAJOR — the MatMulNBits byte order:
 *   packed uint8 [N][nb][16]: byte j of block b holds element 32b+2j in the low nibble and
 *   32b+2j+1 in the high nibble; scales uint16 (fp16 bits) [N][nb].
 *
 * VV_LAYOUT_TILED — the device order read by the GEMV kernels.  Rows are grouped in tiles of
 *   64 (rows beyond N up to the tile boundary are padding: code 8, scale 0).  For tile t,
 *   block b, lane i (row 64t+i) the 16 bytes of the block sit at byte offset
 *   ((t*nb + b)*64 + i)*16, as four little-endian dwords; dword w holds elements 8w..8w+7 of
 *   the block with the even elements 8w, 8w+2, 8w+4, 8w+6 in nibbles 0..3 and the odd elements
 *   8w+1, 8w+3, 8w+5, 8w+7 in nibbles 4..7.  Scales: ng = ceil(nb/8) groups per row; the 8
 *   fp16 scales of blocks 8g..8g+7 of row 64t+i sit at uint16 offset ((t*ng + g)*64 + i)*8
 *   (blocks >= nb hold 0).  Total bytes: vv_packed_bytes / vv_scale_bytes.
 *   A tiled buffer may hold several matrices: the *_tiled packers place source row r at
 *   destination row (r / row_group) * group_stride + row_offset + r % row_group (tile = row/64,
 *   lane = row%64).  Plain placement is row_group = group_stride = 64, row_offset = 0.  Source
 *   rows run to the end of their last row group; rows beyond N there are padding (code 8,
 *   scale 0).
 */
size_t vv_packed_bytes(int64_t rows, int64_t K, int layout);
size_t vv_scale_bytes(int64_t rows, int64_t K, int layout);

/* ---------------------------------------------------------------------------------------------
 * Packer (bitnet-onnx page, ternarisation paragraph + MatMulNBits note).
 *
 *   W: device fp32 [N][K] row-major master weights (finite values).
 *   mode VV_Q_TERNARY: m = mean(|W|) over the whole tensor, computed as the exact sum of |W|
 *     correctly rounded to fp64, divided by N*K in fp64; t = sign(W) if |W| > m/2 else 0 (the
 *     exact value of round(clamp(W/m, -1, 1)) with ties to even); q = t + 8 in {7,8,9}; every
 *     block scale = fp16(m), one round-to-nearest-even step from fp64.  All-zero W gives q = 8,
 *     scale 0.
 *   mode VV_Q_ABSMAX (general int4): per block scale = fp16(absmax/7) (one RNE step from the
 *     fp64 quotient); q = clamp(rint(w / scale) + 8, 0, 15) with the division in fp64 and ties
 *     to even; a block whose scale is 0 gets q = 8.
 *   Output: vv_pack_int4 writes VV_LAYOUT_ROWMAJOR into packed [N*nb*16] / scales [N*nb];
 *   vv_pack_int4_tiled writes VV_LAYOUT_TILED rows into a destination of dst_rows rows
 *   (a multiple of 64) placed as the layout note says.
 *   ws: device workspace of vv_pack_int4_workspace(N, K, mode) bytes (any content; it is
 *   cleared by the call).  Errors: NULL pointers, K % 32, N < 1, unknown mode, a destination
 *   row outside [0, dst_rows), small workspace.
 * ------------------------------------------------------------------------------------------- */
size_t vv_pack_int4_workspace(int64_t N, int64_t K, int mode);
int vv_pack_int4(const float* W, int64_t N, int64_t K, int mode, uint8_t* packed, uint16_t* scales,
                 void* ws, size_t ws_bytes, void* stream);
int vv_pack_int4_tiled(const float* W, int64_t N, int64_t K, int mode, int64_t row_group,
                       int64_t group_stride, int64_t row_offset, int64_t dst_rows, uint8_t* packed,
                       uint16_t* scales, void* ws, size_t ws_bytes, void* stream);

/* Row-major (MatMulNBits) -> tiled, a pure permutation of nibbles and scales (same destination
 * placement rules as vv_pack_int4_tiled).  Lets a MatMulNBits blob from elsewhere feed the
 * GEMV kernels. */
int vv_repack_int4_tiled(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                         int64_t row_group, int64_t group_stride, int64_t row_offset,
                         int64_t dst_rows, uint8_t* tiled, uint16_t* tiled_scales, void* stream);

/* Dequantiser (bitnet-onnx page, MatMulNBits note: symmetric block-32 codes with zero point 8
 * and one fp16 scale per block, so an element's value is (q - 8) * scale; ternary codes give
 * exactly -scale, 0, +scale, the values the ternarisation paragraph says fp16 holds exactly).
 *   W[n][k] = (q - 8) * scale as fp32 (exact for both modes: a 4-bit integer times an fp16 value
 *   needs at most 15 significant bits).  `layout` says how packed/scales are stored; for
 *   VV_LAYOUT_TILED, rows 0..N-1 of tiles 0..ceil(N/64)-1 are read.  W: device fp32 [N][K].
 *   Errors: NULL pointers, K % 32, N < 1, unknown layout. */
int vv_dequant_int4(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int layout,
                    float* W, void* stream);

/* ---------------------------------------------------------------------------------------------
 * int4 GEMV (MatMulNBits with float activations; bitnet-onnx page: MatMulNBits note for the
 * weights, ternarisation paragraph: activations run in float).
 *   y[m][n] = sum_k deq(W)[n][k] * x[m][k] + bias[n], deq(W) = (q - 8) * scale.
 *   packed/scales in `layout`: VV_LAYOUT_ROWMAJOR (the MatMulNBits bytes [N][K/32][16] and fp16
 *   scales [N][K/32], e.g. vv_pack_int4's output) or VV_LAYOUT_TILED (ceil(N/64) tiles, the
 *   decode step's layout, e.g. vv_pack_int4_tiled's or vv_repack_int4_tiled's output).
 *   x: device fp16 [M][K]; bias: device fp16 [N] or NULL; y: device [M][N] of y_dtype (VV_F32
 *   or VV_F16).  M in 1..16, K % 32 == 0.  packed and x 16-byte aligned; scales 16-byte aligned
 *   (tiled) or 2-byte aligned (row-major).
 *   Accumulation is fp32 (products of fp16 x and exact small integers, block sums scaled once).
 *   ws: vv_gemv_int4_workspace(M, N, K, layout) bytes, zero-filled before first use (the
 *   row-major kernel needs no workspace but takes the query's small size for uniformity).
 *   Errors: NULL pointers, M/N out of range, K % 32, unknown layout or dtype, misalignment,
 *   small workspace.  The query returns 0 for arguments the call would reject.
 * ------------------------------------------------------------------------------------------- */
size_t vv_gemv_int4_workspace(int64_t M, int64_t N, int64_t K, int layout);
int vv_gemv_int4(const uint8_t* packed, const uint16_t* scales, const uint16_t* bias,
                 const uint16_t* x, int64_t M, int64_t N, int64_t K, int layout, void* y,
                 int y_dtype, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * GQA decode attention: the GroupQueryAttention node of each layer ("VibeVoice-1.5B — Current
 * Status", Done section: one GroupQueryAttention per layer beside its MatMulNBits projections)
 * over the KV cache of the decoder_step contract (bitnet-onnx page, graph contracts: past K/V
 * [L,1,kv,P,128] with 128-wide heads), kept on the GPU ("VibeVoice-ASR — ONNX export for
 * Vernacula", Highlights: device-resident KV instead of host round trips; fp32 attention math).
 *   q: device [B][nq][head_dim] of q_dtype (VV_F32 / VV_F16);
 *   k_cache, v_cache: device fp16 [B][nkv][cap][head_dim];
 *   lens: device int32 [B]; sequence b attends over positions [0, lens[b]) (1 <= lens[b] <= cap,
 *     not checked on the host: out-of-range lengths are clamped to [1, cap] on the device);
 *   query head h reads KV head h / (nq/nkv); softmax scale `softmax_scale` (1/sqrt(head_dim)
 *   for Qwen2); scores, softmax and the weighted sum are fp32.
 *   out: device [B][nq][head_dim] of out_dtype.  head_dim must be 128, nq % nkv == 0,
 *   nq/nkv <= 8.  ws: vv_gqa_decode_workspace(B, nq, nkv, cap) bytes, zero-filled before first use.
 * ------------------------------------------------------------------------------------------- */
size_t vv_gqa_decode_workspace(int B, int nq, int nkv, int cap);
int vv_gqa_decode(const void* q, int q_dtype, const uint16_t* k_cache, const uint16_t* v_cache,
                  const int32_t* lens, int B, int nq, int nkv, int cap, int head_dim,
                  float softmax_scale, void* out, int out_dtype, void* ws, size_t ws_bytes,
                  void* stream);

/* ---------------------------------------------------------------------------------------------
 * lm_head GEMV + greedy argmax (bitnet-onnx page: lm_head stays fp16; greedy decoding).
 *   W: device fp16 [V][H] row-major; x: device [B][H] of x_dtype (VV_F32 / VV_F16);
 *   logits: device fp32 [B][V] or NULL; token: device int32 [B] = index of the largest logit
 *   (the smallest such index on ties; NaN logits never win).  H % 8 == 0, B in 1..16.
 *   ws: vv_lm_head_argmax_workspace(B, V, H) bytes, zero-filled before first use.
 * ------------------------------------------------------------------------------------------- */
size_t vv_lm_head_argmax_workspace(int B, int V, int H);
int vv_lm_head_argmax(const uint16_t* W, const void* x, int x_dtype, int B, int V, int H,
                      float* logits, int32_t* token, void* ws, size_t ws_bytes, void* stream);

/* vv_lm_head_argmax for callers that cannot allocate device memory (code under hipGraph capture,
 * serving loops, harnesses that forbid allocation): the same kernels and results, with the argmax
 * keys in a library-held scratch array instead of a caller workspace.  The array is a 256 KiB
 * file-scope device allocation that each GPU the library runs on holds until the process ends; the
 * call itself allocates and frees nothing.  Calls needing more keys than it holds
 * (vv_lm_head_argmax_workspace(B, V, H) > 256 KiB, e.g. 16 rows over more than about a million
 * vocabulary rows) return VV_ERR_RANGE before launching anything.  Each call clears the keys it
 * uses with a fill kernel first.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (other streams, other threads) race and must not be issued. */
int vv_lm_head_argmax_noalloc(const uint16_t* W, const void* x, int x_dtype, int B, int V, int H,
                              float* logits, int32_t* token, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Decode step (bitnet-onnx page, decoder_step contract:
 *   input_embeds [B,H], position_ids [B], past K/V [L,B,nkv,P,128]
 *   -> logits [B,V], present K/V [L,B,nkv,P+1,128]),
 * on the Qwen2 layer of the 1.5B STATUS page's Architecture section (pre-RMSNorm, q/k/v bias,
 * GQA, SiLU-gated MLP, residual adds), with rotate-half RoPE (theta = rope_theta, disabled
 * when <= 0) on q and the new k.
 *
 * Per layer l and sequence b at position p = pos[b]:
 *   a = RMSNorm(h; g1), [q|k|v] = W_qkv a + b_qkv, q,k = RoPE(q,k; p),
 *   K[l][b][:,p] = fp16(k), V[l][b][:,p] = fp16(v), o = GQA(q, K[..,0..p], V[..,0..p]),
 *   h += W_o o, m = RMSNorm(h; g2), h += W_down (silu(W_gate m) * (W_up m));
 * then logits = lm_head RMSNorm(h; gf), token = argmax.
 *
 * Weights use VV_LAYOUT_TILED:
 *   qkv: one tiled matrix of nq*d + 2*nkv*d rows (q rows, then k rows, then v rows), K = H;
 *   o:   H rows, K = nq*d;
 *   gu:  gate and up rows interleaved in each tile: lanes 0-31 of tile j hold gate rows
 *        32j..32j+31 and lanes 32-63 the same up rows (pack gate with row_group 32,
 *        group_stride 64, row_offset 0 and up with row_offset 32), 2*I rows, K = H;
 *   down: H rows, K = I.
 * H and I must be multiples of 64, head_dim 128, nq % nkv == 0, nq/nkv <= 8, cap <= 131072.
 *
 * Two launch plans compute the same step (vv_state.path):
 *   VV_PATH_LAYERED  one launch per stage: 1 + 5 L + 1 kernels (plus a split merge per layer
 *                    when the cache is split, except at batches 1 and 2 with at most 64 splits, where
 *                    the o projection's launch does the merge); any batch up to
 *                    max_batch, fp16 or fp32 caches.  At batch 1 each layer's down projection
 *                    and the next layer's q|k|v share one launch (2 + 4 L + 1 kernels).
 *   VV_PATH_CHAINED  three launches per layer: the attention, one grid running the split merge
 *                    and o, and one running gate/up, down and the next layer's q|k|v, as
 *                    consecutive segments whose workgroups start their weight streams before
 *                    their inputs are ready and wait for them on tagged words (1 + 3 L + 1
 *                    kernels); above hidden 2048 gate/up runs in a launch of its own (1 + 4 L + 1
 *                    kernels); batch 1, fp16 caches, n_layers >= 1 and 2..128 attention
 *                    splits (cap 65..8192 positions), else VV_ERR_UNSUPPORTED.
 *   VV_PATH_AUTO     the chained path where it applies and hidden <= 2048 (measured faster for
 *                    the 1.5B-shaped step), else the layered one (faster at the 7B width).
 * Both are deterministic; their results agree to rounding (K-splits and merge order differ).
 * The split-K GEMV hand-offs, the merges, the chained segments and the lm_head argmax wait on
 * other workgroups of their own launch, only on workgroups with smaller indices; each wait is
 * bounded: one that gives up sets a sticky nonzero status word in the workspace instead of
 * hanging (vv_decode_status reads it; vv_workspace_init clears it).
 * ------------------------------------------------------------------------------------------- */
enum { VV_PATH_AUTO = 0, VV_PATH_LAYERED = 1, VV_PATH_CHAINED = 2 };

typedef struct vv_layer {
  const uint8_t* qkv_q;   const uint16_t* qkv_s;    /* device, tiled */
  const uint8_t* o_q;     const uint16_t* o_s;
  const uint8_t* gu_q;    const uint16_t* gu_s;
  const uint8_t* down_q;  const uint16_t* down_s;
  const uint16_t* qkv_bias;                         /* device fp16 [nq*d + 2*nkv*d] or NULL */
  const uint16_t* g1;     const uint16_t* g2;       /* device fp16 [H] RMSNorm weights */
} vv_layer;

typedef struct vv_model {
  int n_layers, hidden, inter, n_q, n_kv, head_dim, vocab;
  int max_batch;            /* largest batch a vv_state may use with this model (1..16) */
  float eps;                /* RMSNorm epsilon */
  float rope_theta;         /* RoPE base; <= 0 disables RoPE */
  const vv_layer* layers;   /* HOST array [n_layers]; copied by the calls that take it */
  const uint16_t* gf;       /* device fp16 [H] final RMSNorm weight */
  const uint16_t* lm_head;  /* device fp16 [V][H] */
} vv_model;

typedef struct vv_state {
  int batch;                       /* 1..max_batch */
  int cap;                         /* cache capacity in positions */
  const uint16_t* input_embeds;    /* device fp16 [B][H] */
  const int32_t* pos;              /* device int32 [B]; 0 <= pos[b] < cap (clamped on device) */
  void* k_cache;                   /* device [L][B][nkv][cap][head_dim], fp16 (fp32 when
                                      kv_dtype is VV_F32) */
  void* v_cache;
  float* logits;                   /* device fp32 [B][V] or NULL */
  int32_t* token;                  /* device int32 [B] */
  float* h_trace;                  /* device fp32 [L+1][B][H] residual stream before each layer
                                      and after the last, or NULL */
  void* workspace;                 /* device, vv_decode_step_workspace(model, batch, cap) bytes,
                                      zero-filled before first use */
  size_t workspace_bytes;
  void** events;                   /* optional HOST array of hipEvent_t (created with timing on)
                                      used to time the operations of an eager vv_decode_step:
                                      events 2i and 2i+1 receive the start and end times of
                                      operation i's kernels (hipExtLaunchKernel's kernel
                                      timestamps, not stream markers).  Layered: prep, then
                                      per layer qkv, attention (+ split merge), o, gate/up,
                                      down, then lm_head: 2*(5*n_layers + 2) events; at batch 1
                                      prep, qkv of layer 0, per layer attention, o, gate/up and
                                      down + the next qkv, then lm_head: 2*(4*n_layers + 3).
                                      Chained: prep + qkv of layer 0, per layer attention,
                                      merge + o and gate/up + down + the next qkv (above hidden
                                      2048: gate/up, then down + the next qkv), then lm_head:
                                      2*(3*n_layers + 2) (2*(4*n_layers + 2)) events.  NULL
                                      disables; graphs reject it. */
  int n_events;                    /* entries in events */
  int path;                        /* VV_PATH_AUTO (0), VV_PATH_LAYERED or VV_PATH_CHAINED */
  /* Closed-loop greedy decoding (optional).  With feedback_table set, each step ends with a
   * small kernel that, for every sequence not yet done, records token[b] at history[b][pos[b]]
   * and then either marks the sequence done (token[b] is one of stop_ids) or gathers
   * input_embeds[b] = feedback_table[token[b]] and advances pos[b] by one (while pos[b] + 1 <
   * cap).  The next step, or the next replay of a captured graph, then decodes the following
   * token with no host round trip ("vibevoice-asr-bitnet-onnx" page, decoding note: greedy
   * decode, the lm_head tied to the fp16 embedding table, stop tokens 151645 / 151643).
   * input_embeds and pos are then written by the step, so they must be writable device
   * buffers.  A done sequence keeps its input and position: its later steps recompute the same
   * slot and token. */
  const uint16_t* feedback_table;  /* device fp16 [vocab][hidden] or NULL (no feedback) */
  int32_t* history;                /* device int32 [B][cap] or NULL */
  int32_t* done;                   /* device int32 [B] or NULL; set to 1 by a stop token (the
                                      caller zeroes it before the first step) */
  int32_t stop_ids[4];             /* stop tokens, n_stop of them */
  int n_stop;                      /* 0..4 */
  /* KV precision: 0 or VV_F16 = fp16 caches; VV_F32 = fp32 caches (the fp32 KV + attention
   * variant that the ASR-ONNX card reports as its accuracy fix: k, v are stored unrounded, at
   * twice the cache bytes). */
  int kv_dtype;
} vv_state;

size_t vv_decode_step_workspace(const vv_model* m, int batch, int cap);
int vv_decode_step(const vv_model* m, const vv_state* s, void* stream);
/* The launch plan vv_decode_step takes for m and s: VV_PATH_LAYERED or VV_PATH_CHAINED (what
 * VV_PATH_AUTO resolves to), or the negative status vv_decode_step would return.  Host only. */
int vv_decode_path(const vv_model* m, const vv_state* s);

/* Copies the step's sticky status word to *status (host) and waits for the stream: 0 = every
 * bounded wait of every launch so far was satisfied; nonzero = a wait gave up (results of that
 * step and later ones are invalid until vv_workspace_init clears the workspace). */
int vv_decode_status(const vv_model* m, const vv_state* s, int32_t* status, void* stream);

/* hipGraph capture of one vv_decode_step: one host->GPU submission per step instead of one per
 * kernel ("VibeVoice-ASR — ONNX export for Vernacula", Highlights: per-launch overhead, about
 * 1950 launches of ~7 us each per step, was the largest share of that runtime's decode time).
 *   create: validates m and s as vv_decode_step does (events must be NULL), captures the step's
 *     launches and instantiates the graph; *out receives a library-owned handle.  The graph keeps
 *     the device pointers of m and s (weights, caches, workspace, inputs, outputs): those buffers
 *     must stay allocated and unmoved until destroy.  pos/input_embeds are read from device memory
 *     at replay, so one graph serves every step whose shapes and buffers stay the same.
 *   launch: replays the step on `stream` (asynchronous); destroy: frees the handle (NULL is a
 *     no-op).  Errors: the vv_decode_step errors at create, VV_ERR_NULL for a NULL handle at
 *     launch, VV_ERR_HIP if the runtime fails. */
typedef struct vv_graph vv_graph;
int vv_decode_graph_create(const vv_model* m, const vv_state* s, void* stream, vv_graph** out);
int vv_decode_graph_launch(vv_graph* g, void* stream);
int vv_decode_graph_destroy(vv_graph* g);

/* ---------------------------------------------------------------------------------------------
 * Prefill (bitnet-onnx page, graph contracts: decoder_init runs the prompt and returns logits and
 * the present K/V that decoder_step continues from), batch 1.
 *   input_embeds: device fp16 [S][H], the prompt's S embeddings at positions 0..S-1.
 *   k_cache/v_cache: device [L][1][nkv][cap][head_dim] (the vv_state layout with batch 1), fp16
 *     or, with kv_dtype VV_F32, fp32; positions 0..S-1 of every layer are written (k after RoPE,
 *     v), the rest untouched.
 *     A decode step with pos = S then continues the sequence.
 *   logits: device fp32 [V] of the last position, or NULL; token: device int32 [1], its greedy
 *     argmax (smallest index on ties).
 *   ws: vv_prefill_workspace(m, S, cap) bytes, 256-byte aligned (no zero-fill needed beyond the
 *     usual first-use rule).  Needs 1 <= S <= cap <= 131072 and the vv_decode_step shape rules.
 * Computes in the decode step's precisions: int4 weights x fp16 activations with fp32 sums
 * (matrix cores), fp32 residual stream, RMSNorm and softmax; causal attention over the fp16
 * cache.
 * ------------------------------------------------------------------------------------------- */
size_t vv_prefill_workspace(const vv_model* m, int S, int cap);
int vv_prefill(const vv_model* m, const uint16_t* input_embeds, int S, void* k_cache,
               void* v_cache, int cap, int kv_dtype, float* logits, int32_t* token, void* ws,
               size_t ws_bytes, void* stream);

/* Measuring stick: reads `bytes` (a positive multiple of 32768) of device memory at p (16-byte
 * aligned) once, as a pure stream of 16-byte loads from the whole chip, and stores nothing (sink:
 * a device uint32 that is written only on a value practically never met).  The time it takes is
 * the part's streaming-read ceiling, against which the decode kernels' achieved bandwidth can be
 * read next to the published 8 TB/s. */
int vv_stream_read(const void* p, size_t bytes, uint32_t* sink, void* stream);

/* Zero-fills a workspace (one fill kernel, capture-safe) */
int vv_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Diagnostics */
const char* vv_status_string(int status);
const char* vv_last_error(void);
int vv_version(void);   /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* VV_H */
