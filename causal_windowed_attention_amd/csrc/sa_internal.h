// Internal launch parameters shared by the host library (sa_host.cpp) and the
// HIP kernels (rope_kernels.hip, attention_kernels.hip). Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kMaxTemporalPairs = 320;  // F * d_t / 2 per launch (table passed by value)
constexpr int kMaxRefreshSlots = 64;    // slots re-rotated by one refresh launch
constexpr int kMaxRefreshPairs = 64;    // d_t / 2 <= D / 2 <= 64

// bf16 attention tiling (chunk_attention_bf16*): 4 waves x 32 or 64 query rows,
// 64-key tiles.
constexpr int kBf16BlockM = 128;      // variant 1: 32 query rows per wave
constexpr int kBf16BlockMWide = 256;  // variant 2: 64 query rows per wave; variant 3: 8 waves x 32
constexpr int kBf16BlockN = 64;
// fp32 attention tiling (chunk_attention_f32): 64 query rows, 32-key tiles.
constexpr int kF32BlockM = 64;
constexpr int kF32BlockN = 32;
// Key-range splits per query tile (partials are merged by attn_combine).
constexpr int kMaxKvSplits = 8;
constexpr int kMaxGroups = 8;           // chunks of one moving-buffer attend (SA_MAX_BUFFER_CHUNKS)
constexpr int kMaxSegs = 4;             // key-row ranges per chunk (SA_MAX_KEY_SEGMENTS)

// Rotate-and-store of a chunk's K (and optionally Q) plus V into the cache:
// rope_apply (Q -> scratch, K/V -> staging slot), kv_ring_append (K/V -> a slot),
// and the sink update (one launch per sink chunk).
struct RopeWriteParams {
  const void* q;        // [B, in_tokens, H, D] or null (no Q)
  const void* k;        // [B, in_tokens, H, D]
  const void* v;        // [B, in_tokens, H, D]
  void* qrot;           // [B*H][Nc][D] rotated Q scratch (when q != null)
  void* kcache;         // [B*H][n_slots*Nc][D]
  void* vtcache;        // [B*H][D][key_stride]
  const float2* h_cs;   // [Hf][d_h/2] (cos, sin) of y * theta_h,j
  const float2* w_cs;   // [Wf][d_w/2] (cos, sin) of x * theta_w,j
  int64_t k_bh_stride;  // elements
  int64_t vt_bh_stride; // elements
  int32_t key_stride;   // elements per V^T channel row
  int32_t row0;         // first cache row (key index) of the target slot
  int32_t n_tokens;     // tokens written (Nc)
  int32_t in_tokens;    // tokens per batch entry in the input tensors
  int32_t in_tok0;      // first input token of this launch
  int32_t B, H, D, Hf, Wf;
  int32_t dt, dh, dw;
  int32_t n_frames;     // frames covered by t_cs (F)
  int32_t q_rows;       // rows per (b, h) of the Q scratch
  int32_t q_row0;       // first Q scratch row written by this launch
  float q_scale;        // fp8 cache: factor on rotated Q before rounding (else unused)
  float2 t_cs[kMaxTemporalPairs];  // [frame][d_t/2]: (cos, sin) of (t0 + frame) * theta_t,j
};

// One launch of rope_apply for the n streams of a ragged batch: stream e's q, k, v go
// to its own Q scratch and staging slot (row0[e]), rotated at positions t0[e] + frame.
// The geometry is shared (the streams have equal configurations); each stream's temporal
// (cos, sin) come from theta_t in fp64 on the device.
constexpr int kMaxBatchStreams = 8;     // SA_MAX_BATCH_STREAMS
struct RopeBatchParams {
  const float2* h_cs;   // [Hf][d_h/2], as in RopeWriteParams (stream 0's copy)
  const float2* w_cs;   // [Wf][d_w/2]
  int64_t k_bh_stride;  // elements
  int64_t vt_bh_stride; // elements
  int32_t key_stride;
  int32_t n_tokens;     // Nc
  int32_t in_tokens;
  int32_t B, H, D, Hf, Wf;
  int32_t dt, dh, dw;
  int32_t n_frames;
  int32_t q_rows;
  float q_scale;
  int32_t n;            // streams
  const void* q[kMaxBatchStreams];
  const void* k[kMaxBatchStreams];
  const void* v[kMaxBatchStreams];
  void* qrot[kMaxBatchStreams];
  void* kcache[kMaxBatchStreams];
  void* vtcache[kMaxBatchStreams];
  int32_t row0[kMaxBatchStreams];
  int32_t t0[kMaxBatchStreams];     // temporal position of each stream's first frame
  double theta_t[64];               // theta^(-2j / d_t) for j < d_t / 2
};

// In-place re-rotation of the temporal pairs of whole cache slots by -Delta.
struct RefreshParams {
  void* kcache;         // [B*H][n_slots*Nc][D]
  int64_t k_bh_stride;  // elements
  int32_t BH, D, Nc, dt;
  int32_t n_slot;
  int32_t slot_row0[kMaxRefreshSlots];
  float2 cs[kMaxRefreshPairs];     // (cos, sin) of -Delta * theta_t,j
};

// Attention of one chunk over the visible key prefix [0, n_keys) of every (b, h).
struct AttnParams {
  const void* q;        // [B*H][Nc][D] rotated queries
  const void* kcache;   // [B*H][rows][D]
  const void* vtcache;  // [B*H][D][key_stride]
  void* out;            // [B][Nc][H][D]
  float* lse;           // [B][H][Nc] natural log, or null
  float* part_o;        // [splits][B*H][Nc][D] normalised partial outputs
  float* part_lse;      // [splits][B*H][Nc] partial log2-sum-exp (log2 units)
  int64_t k_bh_stride;  // elements
  int64_t vt_bh_stride; // elements
  int32_t key_stride;
  int32_t n_keys;
  int32_t Nc, B, H, D;
  int32_t variant;      // bf16 kernel: 1 (4 waves x 32 rows), 2 (4 x 64), 3 (ping-pong 8 x 32)
  int32_t q_rows_per_block;  // BlockM of the kernel variant
  int32_t q_tiles;      // ceil(Nc / BlockM)
  int32_t kv_splits;    // >= 1
  int32_t key_tiles;    // ceil(n_keys / BlockN)
  float scale_log2;     // softmax_scale * log2(e)
  int32_t qk_scale_e8m0;  // fp8: E8M0 block scale 2^-k on the Q operand (Q stored times scale_log2 * 2^k)
  int32_t sk_groups;    // > 0: stream-K schedule with this many persistent workgroups (variant 3)
  float* sk_part_o;     // [2 * sk_groups][BlockM][D] stream-K partial outputs
  float* sk_part_lse;   // [2 * sk_groups][BlockM] stream-K partial log2-sum-exp
  // Query groups of a moving-buffer attend: group g holds query rows
  // [g * group_rows, (g + 1) * group_rows) and attends to its n_seg[g] key-row
  // ranges [seg_lo, seg_hi). n_groups = 0: one group, rows [0, Nc), keys [0, n_keys).
  int32_t n_groups;
  int32_t group_rows;
  int32_t group_qtiles; // q-tiles per group (q_tiles = n_groups * group_qtiles)
  int32_t n_seg[kMaxGroups];
  int32_t seg_lo[kMaxGroups][kMaxSegs];
  int32_t seg_hi[kMaxGroups][kMaxSegs];
  // ragged = 1 (a ragged batch): group g is an independent stream with its own
  // bases below and query rows [0, group_rows); the shared fields above are unused
  int32_t ragged;
  const void* g_q[kMaxGroups];
  const void* g_kc[kMaxGroups];
  const void* g_vt[kMaxGroups];
  void* g_out[kMaxGroups];
  float* g_lse[kMaxGroups];
};

constexpr int kMaxSkGroups = 512;

// Gated delta rule (GDN) forward, chunkwise: tokens in blocks of kGdnBlock; the state scan
// runs kGdnScanRows rows of each (b, h) state per workgroup.
constexpr int kGdnBlock = 64;
constexpr int kGdnScanRows = 16;

struct GdnParams {
  const void* q;          // [B, N, H, D] bf16
  const void* k;          // [B, N, H, D] bf16
  const void* v;          // [B, N, H, D] bf16
  const float* alpha;     // [B, H, N] decay gates in (0, 1]
  const float* beta;      // [B, H, N] write strengths in [0, 1]
  const float* state_in;  // [B, H, D, D] (Dv x Dk), or null for zeros
  float* state_out;       // [B, H, D, D]; may equal state_in
  void* out;              // [B, N, H, D] bf16
  // workspace (nb = ceil(N / kGdnBlock) blocks per (b, h))
  float* g;               // [B*H][nb*64] log of the cumulative gate within each block
  void* W;                // [B*H][nb][3 * 64 * D] bf16: T diag(gam) K in three bf16 parts (scan order)
  float* Up;              // [B*H][nb][D * 64] (T V)^T (in the scan's load order)
  void* Kt;               // [B*H][nb][D * 64] bf16: K^T (in the scan's load order)
  float* U;               // [B*H][nb][D][64] pseudo-values, transposed (U^T)
  float* Sst;             // [B*H][nb][D][D] state at each block start
  int32_t B, N, H, D, nb;
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  void* out;            // [B][Nc][H][D]
  float* lse;           // or null
  int32_t Nc, B, H, D, kv_splits;
};

// dtype: 0 = fp32, 1 = bf16 (sa_dtype)
hipError_t launch_rope_apply(const RopeWriteParams& p, int dtype, hipStream_t st);
hipError_t launch_rope_apply_batch(const RopeBatchParams& p, int dtype, hipStream_t st);
hipError_t launch_kv_append(const RopeWriteParams& p, int dtype, hipStream_t st);
hipError_t launch_sink_update(const RopeWriteParams& p, int dtype, hipStream_t st);
hipError_t launch_rope_refresh(const RefreshParams& p, int dtype, hipStream_t st);
hipError_t launch_chunk_attention(const AttnParams& p, int dtype, hipStream_t st);
hipError_t launch_attn_combine(const CombineParams& p, int dtype, hipStream_t st);
hipError_t launch_attn_sk_combine(const AttnParams& p, hipStream_t st);
hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st);
hipError_t launch_mfma_probe_data(float* out, const void* ops, int blocks, int iters, hipStream_t st);
hipError_t launch_gdn_forward(const GdnParams& p, hipStream_t st);
// Bytes of the fixed device scratch of the workspace-free GDN forward, and its address on the
// device of stream st (null: the current device), looked up once per device.
constexpr size_t kGdnScratchBytes = size_t(64) << 20;
hipError_t gdn_scratch_address(hipStream_t st, void** out);
// out[0, n) = in[0, n), or zeros when in is null (n floats, a multiple of 4; in == out: nothing)
hipError_t launch_gdn_state_pass(const float* in, float* out, size_t n, hipStream_t st);

}  // namespace sa
